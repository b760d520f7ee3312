"""The host-side repacker (kie_host.cpp, HIP-free) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and checked by
tests/host/repack_check.cpp: every row lands once where the layout rules put
it, the RMSNorm gains fold as W diag(g) rounded to fp16, padding is zero,
nothing is written past a block, the rotary table and the fp16 conversions
are exact; with FP8 and FP4 weights (dense and MoE layer blocks, the LM head
and the experts) every row's codes and scale sit where the pair and four-row
unit rules put them. No GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "memory_bandwidth_bound_amd", "csrc")


@pytest.mark.timeout(300)
def test_repack_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "repack_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "kie_host.cpp"), os.path.join(ROOT, "tests", "host", "repack_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=240)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert p.stdout.strip().endswith("OK")
