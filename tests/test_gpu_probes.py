"""GEMV bandwidth probe, inter-workgroup exchange probe and launch probe on the GPU.

Parity: the probe GEMV against the oracle's float64 GEMV within the fp32
accumulation bound, bit-exact on integer-valued inputs, and x = e_j returns
column j exactly."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import gemv_bound, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from memory_bandwidth_bound_amd import kie
    kie.load_library()
    return torch


def _run(torch, A, x, variant):
    from memory_bandwidth_bound_amd import kie
    At = torch.from_numpy(A).cuda()
    xt = torch.from_numpy(x).cuda()
    y, ms = kie.gemv_probe(At, xt, variant=variant)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64), ms


@pytest.mark.parametrize("variant", [0, 1])
# (5, 8192, 2): 160 units over 2048 stream waves, so each 16-unit row is summed
# from the partial sums of 16 waves
@pytest.mark.parametrize("shape", [(512, 2560, 3), (300, 1024, 2), (2560, 8192, 1), (257, 512, 2), (5, 8192, 2)])
def test_gemv_probe_matches_f64(torch_cuda, variant, shape):
    M, K, C = shape
    say(f"gemv probe variant={variant} M={M} K={K} copies={C}")
    rng = np.random.default_rng(M * K + C)
    A = (rng.standard_normal((C, M, K), dtype=np.float32) * 0.02).astype(np.float16)
    x = rng.standard_normal(K, dtype=np.float32).astype(np.float16)
    y, _ = _run(torch_cuda, A, x, variant)
    for c in range(C):
        ref = oracle.gemv_f64(A[c], x)
        assert np.all(np.abs(y[c] - ref) <= gemv_bound(A[c], x)), f"copy {c}"


@pytest.mark.parametrize("variant", [0, 1])
def test_gemv_probe_integer_exact_and_unit_vector(torch_cuda, variant):
    say(f"gemv probe integer/unit variant={variant}")
    rng = np.random.default_rng(7)
    M, K = 640, 2560
    A = rng.integers(-8, 9, size=(1, M, K)).astype(np.float16)
    x = rng.integers(-8, 9, size=K).astype(np.float16)
    y, _ = _run(torch_cuda, A, x, variant)
    assert np.array_equal(y[0], oracle.gemv_f64(A[0], x))
    A = rng.standard_normal((1, M, K)).astype(np.float16)
    for j in (0, 511, 2559):
        e = np.zeros(K, dtype=np.float16)
        e[j] = 1
        y, _ = _run(torch_cuda, A, e, variant)
        assert np.array_equal(y[0], A[0][:, j].astype(np.float64))


@pytest.mark.parametrize("si", [0, 1, 2, 3])
def test_gemv_probe_full_shapes_sampled(torch_cuda, si):
    """The probe shapes at full size, in the benchmark's launch configuration
    (rotating copies); sampled rows checked against the float64 GEMV."""
    cfg = synth.get_config("gemv")
    M, K = cfg.shapes[si]
    A, x = synth.make_probe(si, M, K)
    copies = 3
    say(f"gemv probe full shape {M}x{K} copies={copies}")
    Ac = np.stack([A] * copies)
    y, ms = _run(torch_cuda, Ac, x, 0)
    rows = np.random.default_rng(si).choice(M, size=min(M, 64), replace=False)
    ref = oracle.gemv_f64(A[rows], x)
    bnd = gemv_bound(A[rows], x)
    for c in range(copies):
        assert np.all(np.abs(y[c][rows] - ref) <= bnd)
    assert ms > 0


def test_e2m1_device_conversion_table(torch_cuda):
    """The device's fp4 conversion (v_cvt_scalef32_pk_f32_fp4 with scale 1,
    what the fp4 GEMVs use) gives every E2M1 code exactly the oracle's value,
    the low nibble of a byte first, each of the four bytes selectable: the
    layout the loader packs."""
    from memory_bandwidth_bound_amd import kie
    dev = kie.e2m1_table_probe().astype(np.float64)
    ref = oracle.e2m1_decode_table()
    for l in range(8):
        for b in range(4):
            assert dev[l, b, 0] == ref[(2 * l + b) % 16], (l, b)
            assert dev[l, b, 1] == ref[(2 * l + b + 8) % 16], (l, b)
            assert np.signbit(dev[l, b, 0]) == np.signbit(ref[(2 * l + b) % 16])


def test_e4m3_device_conversion_table(torch_cuda):
    """The device's fp8 conversion (what the fp8 GEMVs use) gives every E4M3
    code exactly the oracle's value from the format's definition (NaN codes
    NaN): the device reads OCP E4M3, bias 7."""
    from memory_bandwidth_bound_amd import kie
    dev = kie.e4m3_table_probe().astype(np.float64)
    ref = oracle.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(dev), nan)
    assert np.array_equal(dev[~nan], ref[~nan])
    assert np.array_equal(np.signbit(dev[~nan]), np.signbit(ref[~nan]))


def test_xcd_map(torch_cuda):
    """Every workgroup of the 256-workgroup grid reports an XCD id; the ids
    are 0..7 on MI355X, 32 workgroups each."""
    from memory_bandwidth_bound_amd import kie
    m = kie.xcd_map()
    counts = np.bincount(m, minlength=8)
    rr = bool(np.array_equal(m, np.arange(256) % 8))
    say(f"xcd map: workgroups per XCD {counts.tolist()}, round robin (XCD = workgroup % 8): {rr}")
    assert m.min() >= 0 and m.max() < 16
    assert counts.sum() == 256


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_barrier_probe(torch_cuda, variant):
    from memory_bandwidth_bound_amd import kie
    say(f"exchange probe variant={variant} 20000 rounds")
    us, err = kie.barrier_probe(20000, variant=variant)
    say(f"exchange variant {variant}: {us:.3f} us per round (256 workgroups), errors={err}")
    assert err == 0
    assert 0 < us < 100


def test_launch_probe(torch_cuda):
    from memory_bandwidth_bound_amd import kie
    us = kie.launch_probe(2000)
    say(f"launch probe: {us:.2f} us per empty kernel launch")
    assert us > 0


# ---- the matrix-core GEMM of the batched prefill ----------------------------------
def _gemm(torch, A, W):
    from memory_bandwidth_bound_amd import kie
    Y, ms = kie.gemm_probe(torch.from_numpy(A).cuda(), torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    return Y.cpu().numpy().astype(np.float64), ms


@pytest.mark.parametrize("shape", [(128, 3584, 2560), (1, 64, 64), (37, 100, 256), (300, 130, 1024),
                                   (64, 2560, 8192)])
def test_gemm_probe_matches_f64(torch_cuda, shape):
    """Y = A W^T against float64 within the bound of fp32 accumulation plus
    the two-term fp16 rounding of A (2^-22 relative per element)."""
    n, M, K = shape
    say(f"gemm probe n={n} M={M} K={K}")
    rng = np.random.default_rng(n * 7 + M + K)
    A = rng.standard_normal((n, K)).astype(np.float32)
    W = (rng.standard_normal((M, K)) * 0.02).astype(np.float16)
    Y, _ = _gemm(torch_cuda, A, W)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    bound = (K * 2.0 ** -23 + 2.0 ** -21) * (np.abs(A.astype(np.float64)) @ np.abs(W.astype(np.float64)).T) + 1e-30
    assert np.all(np.abs(Y - ref) <= bound)


def test_gemm_probe_integer_exact_and_unit_rows(torch_cuda):
    rng = np.random.default_rng(8)
    n, M, K = 70, 90, 512
    A = rng.integers(-8, 9, size=(n, K)).astype(np.float32)
    W = rng.integers(-8, 9, size=(M, K)).astype(np.float16)
    Y, _ = _gemm(torch_cuda, A, W)
    assert np.array_equal(Y, A.astype(np.float64) @ W.astype(np.float64).T)
    E = np.zeros((n, K), dtype=np.float32)
    E[np.arange(n), np.arange(n) % K] = 1.0                 # row p of A = e_(p mod K)
    W2 = (rng.standard_normal((M, K)) * 0.1).astype(np.float16)
    Y2, _ = _gemm(torch_cuda, E, W2)
    assert np.array_equal(Y2, W2.astype(np.float64)[:, np.arange(n) % K].T)
