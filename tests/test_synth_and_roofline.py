"""Seeded inputs are deterministic, and the byte/roofline arithmetic reproduces
the figures the pages print."""
import json
import os

import numpy as np
import pytest

import synth
from memory_bandwidth_bound_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_weights_deterministic_and_stream_independent():
    cfg = synth.get_config("tiny")
    a = synth.make_weights(cfg)
    b = synth.make_weights(cfg)
    assert synth.weights_sha256(a) == synth.weights_sha256(b)
    # tensor i does not depend on the others: a config with more layers keeps E
    c = synth.make_weights(cfg.with_(n_layers=3))
    assert np.array_equal(a[0], c[0])
    assert all(t.dtype == np.float16 for t in a)


def test_weight_statistics_and_gains():
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg)
    names = [n for n, _, _ in synth.tensor_specs(cfg)]
    Wq = W[names.index("l0.Wq")].astype(np.float64)
    assert abs(Wq.std() - 0.02) < 0.001 and abs(Wq.mean()) < 0.001
    assert np.all(W[names.index("l0.g_attn")] == 1)
    assert np.all(W[names.index("g_final")] == 1)
    g = synth.make_weights(cfg.with_(gain_sigma=0.1))[names.index("l1.g_ffn")].astype(np.float64)
    assert 0.05 < g.std() < 0.15 and abs(g.mean() - 1) < 0.03


def test_prompt_and_kv():
    cfg = synth.get_config("tiny")
    p = synth.make_prompt(cfg)
    assert p.dtype == np.int32 and p.shape == (16,) and p.min() >= 0 and p.max() < cfg.vocab
    assert np.array_equal(p, synth.make_prompt(cfg))
    c4 = synth.get_config("2b_32k").with_(n_layers=2)
    K, V = synth.make_kv_prefill(c4, 64)
    K2, _ = synth.make_kv_prefill(c4, 32)
    assert K.shape == (2, 64, 4, 128) and np.array_equal(K[:, :32], K2)
    assert abs(float(K.astype(np.float64).std()) - 1) < 0.05
    assert 0 <= synth.make_pending_token(c4) < c4.vocab


def test_config_sizes():
    c3 = synth.get_config("C3")
    n = sum(int(np.prod(s)) for _, s, k in synth.tensor_specs(c3) if k != "gain")
    assert n == 2_133_852_160      # 25 x 78,643,200 + 2 x 32768 x 2560
    # parameter count from the tensor list, independent of the byte formula
    emb_row = c3.d_model
    active = n - c3.vocab * c3.d_model + emb_row      # one embedding row is read
    assert roofline.active_weight_bytes(c3) == 2 * active
    assert roofline.active_weight_bytes(c3) == 4_099_937_280
    assert c3.max_seq == 1152 and synth.get_config("C4").max_seq == 33024


def test_quantised_active_bytes_from_tensor_list():
    """fp8: one byte per projection weight, fp4: half a byte, both plus a
    4-byte scale per projection row (the LM head's rows too) and one fp16
    embedding row; counted here from the tensor list."""
    for name, per in (("2b_fp8", 1.0), ("2b_fp4", 0.5)):
        c = synth.get_config(name)
        specs = synth.tensor_specs(c)
        mats = [(n, s) for n, s, k in specs if k != "gain" and n != "E"]
        weights = sum(int(np.prod(s)) for _, s in mats)
        rows = sum(int(s[0]) for _, s in mats)
        want = int(weights * per) + 4 * rows + 2 * c.d_model
        assert roofline.active_weight_bytes(c) == want


def test_quantised_moe_active_bytes_from_tensor_list():
    """fp8 / fp4 MoE: every non-expert projection and top_k of the n_experts
    experts per layer at one byte or half a byte a weight, plus a 4-byte scale
    per row read and one fp16 embedding row; counted from the tensor list."""
    for name, per in (("moe_fp8", 1.0), ("moe_fp4", 0.5)):
        c = synth.get_config(name)
        weights = rows = 0.0
        for n, s, k in synth.tensor_specs(c):
            if k == "gain" or n == "E":
                continue
            share = c.top_k / c.n_experts if ".e" in n else 1.0   # expert matrices: the selected share
            weights += share * int(np.prod(s))
            rows += share * int(s[0])
        want = int(round(weights * per)) + 4 * int(round(rows)) + 2 * c.d_model
        assert roofline.active_weight_bytes(c) == want
    # fp4 experts are a quarter of the fp16 bytes, so the fp4 MoE reads less
    # than a third of the fp16 MoE's bytes per token
    assert roofline.active_weight_bytes(synth.get_config("moe_fp4")) < \
        roofline.active_weight_bytes(synth.get_config("moe")) / 3


def test_bench_options_parse(root_dir):
    """--attention takes only the two modes; --tokens and the attention mode
    are accepted without touching a device (the GPU check comes later)."""
    import subprocess
    import sys
    p = subprocess.run([sys.executable, "bench.py", "--attention", "per_die"], cwd=root_dir, capture_output=True,
                       text=True, timeout=300)
    assert p.returncode == 2 and "--attention" in p.stderr
    p = subprocess.run([sys.executable, "bench.py", "--help"], cwd=root_dir, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0 and "xcd_local" in p.stdout and "--tokens" in p.stdout and "moe_fp4" in p.stdout


def test_moe_active_bytes_from_tensor_list():
    c5 = synth.get_config("C5")
    specs = synth.tensor_specs(c5)
    total = sum(int(np.prod(s)) for _, s, k in specs if k != "gain")
    per_expert = 3 * c5.ffn_dim * c5.d_model
    inactive = c5.n_layers * (c5.n_experts - c5.top_k) * per_expert
    active = total - inactive - c5.vocab * c5.d_model + c5.d_model
    assert roofline.active_weight_bytes(c5) == 2 * active == 3_059_748_864


def test_page_figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        g = json.load(f)
    lt = g["launch_tax"]
    us = roofline.launch_overhead_us(lt["layers"], lt["kernels_per_layer"], lt["launch_us_per_kernel"])
    assert us == pytest.approx(lt["overhead_us_per_token"])
    assert lt["layers"] * lt["kernels_per_layer"] == lt["launches_per_token"]
    cap = roofline.launch_bound_tok_per_s(lt["layers"], lt["kernels_per_layer"], lt["launch_us_per_kernel"])
    assert cap == pytest.approx(lt["launch_bound_tok_per_s_approx"], rel=lt["tolerance_rel"])
    tb = g["token_budget"]
    assert roofline.token_budget_us(tb["tok_per_s"]) == pytest.approx(tb["budget_us_approx"], abs=tb["tolerance_abs_us"])
    ac = g["aggregate_ceiling"]
    ceil = roofline.ceiling_tok_per_s(ac["effective_bandwidth_bytes_per_s"], ac["active_weight_bytes"])
    assert ceil == pytest.approx(ac["ceiling_tok_per_s_approx"], rel=ac["tolerance_rel"])
    frac = roofline.mbu(ac["active_weight_bytes"], ac["achieved_tok_per_s"], ac["effective_bandwidth_bytes_per_s"])
    assert frac == pytest.approx(ac["achieved_fraction_approx"], rel=ac["tolerance_rel"])
    al = g["agent_loop"]
    assert al["tokens"] / al["slow_tok_per_s"] / 60 == pytest.approx(al["slow_minutes_approx"], rel=0.05)
    lo, hi = al["fast_seconds_range"]
    assert lo <= al["tokens"] / al["fast_tok_per_s"] <= hi


def test_decode_bytes_sums_kv_per_pass():
    c3 = synth.get_config("C3")
    per = roofline.kv_bytes_per_position(c3)
    assert per == 51_200
    w = roofline.active_weight_bytes(c3)
    got = roofline.decode_bytes(c3, 128, 3)
    want = 3 * w + per * (129 + 130 + 131) + 3 * per
    assert got == want
    # the 70 % MBU target of the 2.1B decoder at 8 TB/s, about 1,355 tok/s
    mean_kv = per * (129 + 1152) / 2
    assert 0.7 * 8e12 / (w + mean_kv) == pytest.approx(1355, rel=0.002)


def test_bench_refuses_more_than_one_gpu(root_dir):
    """The benchmark measures one GPU; asking for several exits with a message
    (before touching a device)."""
    import subprocess
    import sys
    p = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root_dir, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_bench_cpu_baseline_stays_within_the_cache(root_dir):
    """The oracle sample the benchmark times never runs past the workload's
    KV capacity (the tiny decoder has 80 positions: 16 prompt + 64 decode)."""
    import sys
    sys.path.insert(0, root_dir)
    import bench
    cfg = synth.get_config("tiny")
    line = bench.cpu_baseline_decode(cfg, synth.make_weights(cfg), synth.make_prompt(cfg), target_s=30.0)
    first = cfg.prompt_len + 1
    assert line["kind"] == "oracle" and line["value"] > 0
    assert f"positions {first}..{cfg.max_seq - 1}" in line["sample"] or "passes" in line["sample"]
    n = int(line["sample"].split()[0])
    assert 1 <= n <= cfg.max_seq - first
