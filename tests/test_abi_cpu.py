"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments and configurations before touching HIP."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import synth
from memory_bandwidth_bound_amd import kie

LIB = kie.LIB_PATH


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libkie.so not built")
    return kie.load_library()


def test_exports_every_declared_symbol(lib):
    declared = kie.header_symbols()
    assert len(declared) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert hasattr(lib, s)


def test_status_strings(lib):
    for code in range(0, -9, -1):
        s = lib.kie_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.kie_status_str(-99).decode() == "unknown status"


@pytest.mark.parametrize("name", ["tiny", "2b", "2b_32k", "moe"])
def test_workspace_bytes_cover_weights_and_cache(lib, name):
    cfg = synth.get_config(name)
    n = kie.workspace_bytes(cfg)
    from memory_bandwidth_bound_amd import roofline
    weights = 2 * sum(int(np.prod(s)) for _, s, k in synth.tensor_specs(cfg) if k != "gain")
    kv = 2 * roofline.kv_bytes_per_position(cfg) * cfg.max_seq // 2 * 2
    assert n >= weights + kv // 2
    assert n < 1.2 * (weights + kv) + (64 << 20)
    assert lib.kie_tensor_count(ctypes.byref(kie.make_config(cfg))) == len(synth.tensor_specs(cfg))


@pytest.mark.parametrize("bad", [
    dict(head_dim=96), dict(n_heads=6, n_kv_heads=4), dict(n_heads=36, n_kv_heads=4),
    dict(d_model=768), dict(ffn_dim=300), dict(max_seq=0), dict(max_seq=70000), dict(vocab=1),
    dict(n_layers=0), dict(rms_eps=0.0), dict(n_experts=4, top_k=5), dict(n_experts=4, top_k=2, d_model=256),
])
def test_invalid_configs_rejected(lib, bad):
    kc = kie.make_config(synth.get_config("tiny"))
    for k, v in bad.items():
        setattr(kc, k, v)
    assert lib.kie_workspace_bytes(ctypes.byref(kc)) == 0
    assert lib.kie_last_error(None).decode()
    h = ctypes.c_void_p()
    ptrs = (ctypes.c_void_p * 1)(1)
    rc = lib.kie_load(ctypes.byref(kc), ptrs, 1, ctypes.c_void_p(1), 1 << 40, None, ctypes.byref(h))
    assert rc == -2 and not h.value


def test_load_argument_errors_before_any_device_call(lib):
    cfg = synth.get_config("tiny")
    kc = kie.make_config(cfg)
    h = ctypes.c_void_p()
    n = lib.kie_tensor_count(ctypes.byref(kc))
    ptrs = (ctypes.c_void_p * n)(*([1] * n))
    # null workspace
    assert lib.kie_load(ctypes.byref(kc), ptrs, n, None, 1 << 30, None, ctypes.byref(h)) == -1
    # wrong tensor count
    assert lib.kie_load(ctypes.byref(kc), ptrs, n - 1, ctypes.c_void_p(1), 1 << 30, None, ctypes.byref(h)) == -1
    # a null tensor
    ptrs0 = (ctypes.c_void_p * n)(*([1] * (n - 1) + [0]))
    assert lib.kie_load(ctypes.byref(kc), ptrs0, n, ctypes.c_void_p(1), 1 << 30, None, ctypes.byref(h)) == -1
    # workspace too small
    ws = kie.workspace_bytes(cfg)
    assert lib.kie_load(ctypes.byref(kc), ptrs, n, ctypes.c_void_p(1), ws - 1, None, ctypes.byref(h)) == -4
    assert not h.value


def test_null_model_calls(lib):
    out = np.zeros(4, dtype=np.int32)
    assert lib.kie_decode(None, 4, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None) == -1
    assert lib.kie_reset(None) == -1
    assert lib.kie_rewind(None, 0, 0) == -1
    assert lib.kie_last_kernel_ms(None) == 0.0
    assert lib.kie_set_limits(None, 1, 1) == -1
    lib.kie_free(None)


def test_probe_argument_errors(lib):
    ms = ctypes.c_float()
    # K not a multiple of 512
    assert lib.kie_gemv_probe(ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), 4, 300, 1, 0, None,
                              ctypes.byref(ms)) == -1
    # K too long
    assert lib.kie_gemv_probe(ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), 4, 65536 + 512, 1, 0,
                              None, ctypes.byref(ms)) == -1
    # matrices smaller than the 4 KiB the streaming variant reads for idle batches
    assert lib.kie_gemv_probe(ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), 1, 512, 1, 0,
                              None, ctypes.byref(ms)) == -1
    # unknown variant
    assert lib.kie_gemv_probe(ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), 4, 512, 1, 2,
                              None, ctypes.byref(ms)) == -1
    assert lib.kie_gemv_probe(None, ctypes.c_void_p(1), ctypes.c_void_p(1), 4, 512, 1, 0, None, None) == -1
    err = ctypes.c_int32()
    assert lib.kie_barrier_probe(None, 1, 10, None, ctypes.byref(ms), ctypes.byref(err)) == -1
    assert lib.kie_barrier_probe(ctypes.c_void_p(1), 3, 10, None, ctypes.byref(ms), ctypes.byref(err)) == -1
    assert lib.kie_barrier_probe(ctypes.c_void_p(1), 1, 0, None, ctypes.byref(ms), ctypes.byref(err)) == -1
    assert lib.kie_launch_probe(0, None, ctypes.byref(ms)) == -1
    # the allocation-free probe checks its arguments before any device call
    assert lib.kie_barrier_probe_noalloc(3, 10, None, ctypes.byref(ms), ctypes.byref(err)) == -1
    assert lib.kie_xcd_map(None, None) == -1
    assert lib.kie_barrier_probe_noalloc(1, 0, None, ctypes.byref(ms), ctypes.byref(err)) == -1
    assert lib.kie_barrier_probe_noalloc(1, 10, None, None, ctypes.byref(err)) == -1


# ---- the Python binding checks shapes and lengths before any ctypes call ----
def test_binding_shape_order_matches_tensor_specs():
    for name in ("tiny", "2b", "moe"):
        cfg = synth.get_config(name)
        assert kie.expected_shapes(cfg) == [tuple(s) for _, s, _ in synth.tensor_specs(cfg)]


def test_binding_rejects_bad_tensors():
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg)
    kie.check_tensors(cfg, W)
    with pytest.raises(kie.KieError) as e:
        kie.check_tensors(cfg, W[:-1])
    assert e.value.code == -1
    bad = list(W)
    bad[3] = bad[3][:, :-1]                       # a truncated Wk
    with pytest.raises(kie.KieError):
        kie.check_tensors(cfg, bad)
    moe = synth.DecoderConfig(name="m", n_layers=1, d_model=512, n_heads=4, n_kv_heads=2, head_dim=128,
                              ffn_dim=1024, vocab=300, n_experts=2, top_k=1)
    Wm = [np.zeros(s, dtype=np.float16) for s in kie.expected_shapes(moe)]
    kie.check_tensors(moe, Wm)
    Wm[-4] = Wm[-4].T                             # an expert's Wd transposed: same bytes, wrong shape
    with pytest.raises(kie.KieError):
        kie.check_tensors(moe, Wm)
    bad = list(W)
    bad[5] = bad[5].astype(np.float32)            # fp32 would be read as twice the elements
    with pytest.raises(kie.KieError):
        kie.check_tensors(cfg, bad)


def test_binding_rejects_bad_kv_and_tokens():
    cfg = synth.get_config("tiny")
    K, V = synth.make_kv_prefill(cfg, n_pos=5)
    assert kie.check_kv(cfg, K, V) == 5
    assert kie.check_kv(cfg, K[:, :0], V[:, :0]) == 0
    for k, v in [(K, V[:, :4]), (K[:1], V[:1]), (K.astype(np.float32), V), (K[..., :32], V[..., :32]),
                 (K[0], V[0])]:
        with pytest.raises(kie.KieError) as e:
            kie.check_kv(cfg, k, v)
        assert e.value.code == -1
    assert kie.check_tokens([1, 2, 3], 2, "force").tolist() == [1, 2]
    assert kie.check_tokens(np.arange(4), 0, "tokens").dtype == np.int32
    for t, n in [([1, 2], 3), (np.zeros((2, 2), dtype=np.int32), 1), (np.array([0.5, 1.0]), 1)]:
        with pytest.raises(kie.KieError) as e:
            kie.check_tokens(t, n, "force")
        assert e.value.code == -1


# ---- fp8 weights ------------------------------------------------------------
def test_host_fp8_quantizer_matches_oracle(lib):
    """The library's E4M3 quantizer (what kie_load applies) against the
    oracle's, bit for bit: codes and scales, with and without a folded gain,
    an all-zero row, and values exactly halfway between codes."""
    import oracle
    rng = np.random.default_rng(30)
    W = (rng.standard_normal((40, 2560)) * 0.02).astype(np.float16)
    W[3] = 0
    W[4, :] = 0
    W[4, 0] = np.float16(448.0)                  # scale exactly 1: the rest encode as given
    t = oracle.e4m3_decode_table()
    mids = ((t[1:0x7e] + t[2:0x7f]) / 2).astype(np.float16)
    mids = mids[mids.astype(np.float64) == (t[1:0x7e] + t[2:0x7f]) / 2][:200]   # exact in fp16
    W[4, 1:1 + len(mids)] = mids
    W[5, :len(mids)] = -mids
    W[5, -1] = np.float16(-448.0)
    g = (1 + rng.standard_normal(2560) * 0.3).astype(np.float16)
    for gain in (None, g):
        q, s = kie.quantize_e4m3_rows(W, gain)
        qo, so = oracle.quantize_rows_e4m3(W, gain)
        assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
        assert np.array_equal(q, qo)


@pytest.mark.parametrize("bad", [
    dict(weight_format=3), dict(weight_format=-1),
    dict(weight_format=1, n_experts=4, top_k=2, d_model=512, ffn_dim=512),
    dict(weight_format=1, head_dim=64, d_model=512, n_heads=8, n_kv_heads=4, ffn_dim=512, vocab=1000),
    dict(weight_format=1, d_model=512, ffn_dim=512, n_heads=4, n_kv_heads=4, head_dim=128, vocab=1001),
    dict(weight_format=1),                       # the tiny decoder: d_model 256
])
def test_fp8_configs_rejected(lib, bad):
    kc = kie.make_config(synth.get_config("tiny"))
    for k, v in bad.items():
        setattr(kc, k, v)
    assert lib.kie_workspace_bytes(ctypes.byref(kc)) == 0
    assert lib.kie_last_error(None).decode()


def test_fp8_workspace_is_about_half(lib):
    a = kie.workspace_bytes(synth.get_config("2b"))
    b = kie.workspace_bytes(synth.get_config("2b_fp8"))
    assert 0.5 < b / a < 0.62          # weights halve; embedding, KV cache and buffers stay


# ---- fp4 weights ------------------------------------------------------------
def test_host_fp4_quantizer_matches_oracle(lib):
    """The library's E2M1 quantizer (what kie_load applies) against the
    oracle's, bit for bit: codes and scales, with and without a folded gain,
    an all-zero row, values exactly halfway between codes (ties to the even
    code), negatives that round to zero (code 8) and saturation."""
    import oracle
    rng = np.random.default_rng(31)
    W = (rng.standard_normal((40, 2560)) * 0.02).astype(np.float16)
    W[3] = 0
    W[4, :] = 0
    W[4, 0] = np.float16(6.0)                    # scale exactly 1: the rest encode as given
    t = oracle.e2m1_decode_table()[:8]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float16)   # 0.25 .. 5: all exact in fp16
    W[4, 1:8] = mids
    W[4, 8:15] = -mids
    W[4, 15:19] = np.float16([-0.2, 0.2, -0.0, 5.5])
    W[5, :] = np.float16(0.001)
    W[5, 0] = np.float16(-1.0)
    g = (1 + rng.standard_normal(2560) * 0.3).astype(np.float16)
    for gain in (None, g):
        q, s = kie.quantize_e2m1_rows(W, gain)
        qo, so = oracle.quantize_rows_e2m1(W, gain)
        assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
        assert np.array_equal(q, qo)
    q, _ = kie.quantize_e2m1_rows(W[4:5])
    assert q[0, 1:8].tolist() == [0, 2, 2, 4, 4, 6, 6]          # ties to the even code
    assert q[0, 15:19].tolist() == [8, 0, 8, 7]


@pytest.mark.parametrize("bad", [
    dict(weight_format=2, n_experts=6, top_k=2, d_model=512, ffn_dim=512, n_heads=4, n_kv_heads=4,
         head_dim=128),                          # MoE with experts not in fours
    dict(weight_format=2, head_dim=64, d_model=512, n_heads=8, n_kv_heads=4, ffn_dim=512, vocab=1000),
    dict(weight_format=2, d_model=512, ffn_dim=512, n_heads=4, n_kv_heads=4, head_dim=128, vocab=1002),
    dict(weight_format=2),                       # the tiny decoder: d_model 256
])
def test_fp4_configs_rejected(lib, bad):
    kc = kie.make_config(synth.get_config("tiny"))
    for k, v in bad.items():
        setattr(kc, k, v)
    assert lib.kie_workspace_bytes(ctypes.byref(kc)) == 0
    assert lib.kie_last_error(None).decode()


def test_fp4_moe_config_accepted_and_experts_quartered(lib):
    """fp4 MoE: experts in fours load, and each expert block takes a quarter
    of its fp16 bytes."""
    moe = synth.get_config("moe")
    a = kie.workspace_bytes(moe)
    b = kie.workspace_bytes(moe.with_(weight_format="fp4"))
    assert b > 0
    expert16 = (2 * moe.ffn_dim * moe.d_model + moe.d_model * moe.ffn_dim) * 2 * moe.n_experts * moe.n_layers
    assert a - b >= 0.75 * expert16 * 0.99   # at least the experts' three quarters saved


def test_fp4_workspace_is_about_a_quarter(lib):
    a = kie.workspace_bytes(synth.get_config("2b"))
    b = kie.workspace_bytes(synth.get_config("2b_fp4"))
    c = kie.workspace_bytes(synth.get_config("2b_fp4").with_(d_model=2560))   # same shape
    assert b == c
    assert 0.26 < b / a < 0.4          # weights quarter; embedding, KV cache and buffers stay
