"""Decode parity at the full workload sizes, in the benchmark's launch shape.

The ~2.1B dense decoder (25 layers, d 2560, 20/4 heads x 128, SwiGLU 8192,
vocab 32768), the same decoder over a 32768-position cache, and the top-8 of
64 experts MoE decoder (24 layers, d 2048). Each test compares device logits
with the oracle's element by element on passes after the prompt AND deep in
the context (both sides starting from the same seeded cache of 1100, 33000 or
608 positions), then checks the token ids of ONE launch of the benchmark's
request length (1024, 256 and 512 passes) against oracle results that do not
depend on the device: a teacher-forced request whose every pass the oracle
computes (dense: every logits row of the request compared element by element),
the leading passes of a request (32K context, MoE), and the properties that
hold at any size (a single launch equals the same passes split over several
launches, bit for bit; MoE experts are the exact top-k of the router logits).
The same checks run on the decoders with FP8 and FP4 weights (dense and MoE),
and the ~2.1B decoder runs once more with attention recomputed per XCD, whose
logits must equal the grid-wide mode's bit for bit.

Teacher forcing uses the seeded token stream of `synth.make_forced_tokens`:
pass i of a request is fed token i of the stream whatever pass i-1 produced.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from tests.parity import TOL, check_rows, moe_request_parity, report_worst, say

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1200)]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@functools.lru_cache(maxsize=1)
def _weights(name):
    say(f"{name}: generating weights")
    return synth.make_weights(synth.get_config(name))


def _model(cfg, W):
    from memory_bandwidth_bound_amd import kie
    say(f"{cfg.name}: loading the model")
    return kie.Model(cfg, W)


def _ids_agree(dev_ids, ref_rows, label):
    """Device ids against oracle logits rows: equal wherever the oracle's
    top-2 gap exceeds the tolerance. Returns (checked, total)."""
    checked = 0
    for i, (t, r) in enumerate(zip(dev_ids, ref_rows)):
        if oracle.top2_gap(r) > TOL:
            assert int(t) == int(np.argmax(r)), f"{label}: pass {i} token {t} != {int(np.argmax(r))}"
            checked += 1
    say(f"[{label}] ids checked {checked}/{len(dev_ids)}")
    return checked, len(dev_ids)


# ---- ~2.1B dense, 128-token prompt, 1024-pass requests -------------------------
def test_2b_prompt_and_forced_passes(torch_cuda):
    cfg = synth.get_config("2b")
    W = _weights("2b")
    P = synth.make_prompt(cfg)
    ref = oracle.Decoder(cfg, W)
    say("2b: oracle prefill and 4 greedy passes")
    first, last = ref.prefill_batched(P)
    ids, rows, _ = ref.decode(4, keep_logits=True)
    m = _model(cfg, W)
    try:
        g_first, g_logits, _ = m.prefill(P, logits=True)
        check_rows(g_logits[-1:], last[None], label="2b prefill")
        if oracle.top2_gap(last) > TOL:
            assert g_first == first
        m.rewind(len(P), first)
        _, g_rows, _ = m.decode(4, force=ids, logits=True)
        check_rows(g_rows, rows, label="2b decode")
        # deep in the context: both sides from the same seeded 1100-position cache
        K, V = synth.make_kv_prefill(cfg, n_pos=1100)
        F = synth.make_forced_tokens(cfg, 5)
        deep = oracle.Decoder(cfg, W)
        deep.set_kv(K, V, int(F[0]))
        say("2b: oracle 4 teacher-forced passes at positions 1100..1103")
        _, drows, _ = deep.decode(4, force=F[1:], keep_logits=True)
        m.set_kv(K, V, int(F[0]))
        _, g_drows, _ = m.decode(4, force=F[1:], logits=True)
        check_rows(g_drows, drows, label="2b deep")
    finally:
        m.close()


def test_2b_request_launch_teacher_forced(torch_cuda):
    cfg = synth.get_config("2b")
    n = cfg.decode_steps
    W = _weights("2b")
    P = synth.make_prompt(cfg)
    F = synth.make_forced_tokens(cfg, n + 1)
    m = _model(cfg, W)
    try:
        m.prefill(P)
        say(f"2b: one teacher-forced launch of {n} passes")
        m.rewind(len(P), int(F[0]))
        g_ids, _, _ = m.decode(n, force=F[1:])
        # the same passes split over launches of 64 with the debug buffers on
        m.rewind(len(P), int(F[0]))
        c_ids, c_rows, _ = m.decode(n, force=F[1:], logits=True)
        assert np.array_equal(g_ids, c_ids)
        assert np.array_equal(c_ids, np.argmax(c_rows, axis=1))
    finally:
        m.close()
    say(f"2b: oracle full causal forward over {len(P) + n} tokens")
    rows = oracle.Decoder(cfg, W).forward_full(list(P) + list(F[:n]))[len(P):]
    # every logits row of the request, element by element (the debug launches
    # of 64 passes, whose ids equal the single launch's bit for bit)
    check_rows(c_rows, rows, label="2b request-rows")
    del c_rows
    checked, total = _ids_agree(g_ids, rows, "2b request")
    assert checked >= total * 0.75
    report_worst("2b")


def test_2b_xcd_local_attention(torch_cuda):
    """XCD-local attention on the full decoder: passes at 129..416 attended
    positions, all heads' attention on every XCD up to 384, global head mode
    after. Every logits row equals the global mode's bit for bit and is
    compared with the oracle's full causal forward element by element."""
    cfg = synth.get_config("2b")
    n = 288
    W = _weights("2b")
    P = synth.make_prompt(cfg)
    F = synth.make_forced_tokens(cfg, n + 1)
    m = _model(cfg, W)
    try:
        m.prefill(P)
        say(f"2b: {n} teacher-forced passes, global attention then XCD-local")
        m.rewind(len(P), int(F[0]))
        _, g_rows, _ = m.decode(n, force=F[1:], logits=True)
        m.set_attention_mode("xcd_local")
        m.rewind(len(P), int(F[0]))
        x_ids, x_rows, _ = m.decode(n, force=F[1:], logits=True)
        assert np.array_equal(x_rows, g_rows), "XCD-local logits differ from the global mode's"
        del g_rows
        m.rewind(len(P), int(F[0]))
        s_ids, _, _ = m.decode(n, force=F[1:])
        assert np.array_equal(s_ids, x_ids)
    finally:
        m.close()
    say(f"2b: oracle full causal forward over {len(P) + n} tokens")
    rows = oracle.Decoder(cfg, W).forward_full(list(P) + list(F[:n]))[len(P):]
    check_rows(x_rows, rows, label="2b/xcd request-rows")
    report_worst("2b/xcd")


# ---- the same decoder with fp8 (E4M3, one scale per row) weights -------------------
def test_2b_fp8_prompt_deep_and_request(torch_cuda):
    """The ~2.1B decoder with every projection quantised to row-scaled E4M3 at
    load (the oracle quantises the fp16 weights itself, from the same
    definition): the prompt's last logits, 4 greedy passes, 4 passes from a
    seeded 1100-position cache, and one 1024-pass teacher-forced launch whose
    ids are checked against the oracle's full causal forward (every logits
    row of the same passes in debug launches element by element)."""
    cfg = synth.get_config("2b_fp8")
    n = cfg.decode_steps
    W = _weights("2b")          # the same fp16 tensors as the 2b workload
    P = synth.make_prompt(cfg)
    say("2b_fp8: oracle quantisation and prefill")
    ref = oracle.Decoder(cfg, W)
    first, last = ref.prefill_batched(P)
    ids, rows, _ = ref.decode(4, keep_logits=True)
    F = synth.make_forced_tokens(cfg, n + 1)
    m = _model(cfg, W)
    try:
        g_first, g_logits, _ = m.prefill(P, logits=True)
        check_rows(g_logits[-1:], last[None], label="2b_fp8 prefill")
        if oracle.top2_gap(last) > TOL:
            assert g_first == first
        m.rewind(len(P), first)
        _, g_rows, _ = m.decode(4, force=ids, logits=True)
        check_rows(g_rows, rows, label="2b_fp8 decode")
        K, V = synth.make_kv_prefill(cfg, n_pos=1100)
        ref.set_kv(K, V, int(F[0]))
        _, drows, _ = ref.decode(4, force=F[1:5], keep_logits=True)
        m.set_kv(K, V, int(F[0]))
        _, g_drows, _ = m.decode(4, force=F[1:5], logits=True)
        check_rows(g_drows, drows, label="2b_fp8 deep")
        del K, V
        m.reset()
        m.prefill(P)
        say(f"2b_fp8: one teacher-forced launch of {n} passes")
        m.rewind(len(P), int(F[0]))
        g_ids, _, _ = m.decode(n, force=F[1:])
        m.rewind(len(P), int(F[0]))
        c_ids, c_rows, _ = m.decode(n, force=F[1:], logits=True)
        assert np.array_equal(g_ids, c_ids)
        assert np.array_equal(c_ids, np.argmax(c_rows, axis=1))
    finally:
        m.close()
    say(f"2b_fp8: oracle full causal forward over {len(P) + n} tokens")
    rows = ref.forward_full(list(P) + list(F[:n]))[len(P):]
    check_rows(c_rows, rows, label="2b_fp8 request-rows")
    del c_rows
    checked, total = _ids_agree(g_ids, rows, "2b_fp8 request")
    assert checked >= total * 0.75
    report_worst("2b_fp8")


# ---- the same decoder with fp4 (E2M1, one scale per row) weights -------------------
def test_2b_fp4_prompt_deep_and_request(torch_cuda):
    """The ~2.1B decoder with every projection quantised to row-scaled E2M1 at
    load (the oracle quantises the fp16 weights itself): the prompt's last
    logits, 4 greedy passes, 4 passes from a seeded 1100-position cache, and
    one 1024-pass teacher-forced launch checked row by row against the
    oracle's full causal forward."""
    cfg = synth.get_config("2b_fp4")
    n = cfg.decode_steps
    W = _weights("2b")          # the same fp16 tensors as the 2b workload
    P = synth.make_prompt(cfg)
    say("2b_fp4: oracle quantisation and prefill")
    ref = oracle.Decoder(cfg, W)
    first, last = ref.prefill_batched(P)
    ids, rows, _ = ref.decode(4, keep_logits=True)
    F = synth.make_forced_tokens(cfg, n + 1)
    m = _model(cfg, W)
    try:
        g_first, g_logits, _ = m.prefill(P, logits=True)
        check_rows(g_logits[-1:], last[None], label="2b_fp4 prefill")
        if oracle.top2_gap(last) > TOL:
            assert g_first == first
        m.rewind(len(P), first)
        _, g_rows, _ = m.decode(4, force=ids, logits=True)
        check_rows(g_rows, rows, label="2b_fp4 decode")
        K, V = synth.make_kv_prefill(cfg, n_pos=1100)
        ref.set_kv(K, V, int(F[0]))
        _, drows, _ = ref.decode(4, force=F[1:5], keep_logits=True)
        m.set_kv(K, V, int(F[0]))
        _, g_drows, _ = m.decode(4, force=F[1:5], logits=True)
        check_rows(g_drows, drows, label="2b_fp4 deep")
        del K, V
        m.reset()
        m.prefill(P)
        say(f"2b_fp4: one teacher-forced launch of {n} passes")
        m.rewind(len(P), int(F[0]))
        g_ids, _, _ = m.decode(n, force=F[1:])
        m.rewind(len(P), int(F[0]))
        c_ids, c_rows, _ = m.decode(n, force=F[1:], logits=True)
        assert np.array_equal(g_ids, c_ids)
        assert np.array_equal(c_ids, np.argmax(c_rows, axis=1))
    finally:
        m.close()
    say(f"2b_fp4: oracle full causal forward over {len(P) + n} tokens")
    rows = ref.forward_full(list(P) + list(F[:n]))[len(P):]
    check_rows(c_rows, rows, label="2b_fp4 request-rows")
    del c_rows
    checked, total = _ids_agree(g_ids, rows, "2b_fp4 request")
    assert checked >= total * 0.75
    report_worst("2b_fp4")


# ---- the same decoder after a 32768-position cache, 256-pass requests -------------
def test_2b_32k_forced_passes_and_request(torch_cuda):
    cfg = synth.get_config("2b_32k")
    n = cfg.decode_steps
    W = _weights("2b")          # the same tensors as the 2b workload (same seed and shapes)
    K, V = synth.make_kv_prefill(cfg)
    pend = synth.make_pending_token(cfg)
    F = synth.make_forced_tokens(cfg, n)
    ref = oracle.Decoder(cfg, W)
    ref.set_kv(K, V, pend)
    say("2b_32k: oracle 8 teacher-forced passes over the 32768-position cache")
    _, rows, _ = ref.decode(8, force=F[:8], keep_logits=True)
    del ref
    m = _model(cfg, W)
    try:
        m.set_kv(K, V, pend)
        _, g_rows, _ = m.decode(8, force=F[:8], logits=True)
        check_rows(g_rows, rows, label="2b_32k decode")
        say(f"2b_32k: one teacher-forced launch of {n} passes")
        m.rewind(cfg.kv_prefill, pend)
        g_ids, _, _ = m.decode(n, force=F)
        _ids_agree(g_ids[:8], rows, "2b_32k request")
        say(f"2b_32k: free-running launches of {n} passes, twice")
        m.rewind(cfg.kv_prefill, pend)
        a, _, _ = m.decode(n)
        m.rewind(cfg.kv_prefill, pend)
        b, _, _ = m.decode(n)
        assert np.array_equal(a, b)
        # deep: both sides from the same seeded 33000-position cache
        del K, V
        deep_cfg = cfg.with_(kv_prefill=33000, decode_steps=cfg.max_seq - 33000)
        Kd, Vd = synth.make_kv_prefill(deep_cfg)
        ref = oracle.Decoder(cfg, W)
        ref.set_kv(Kd, Vd, int(F[0]))
        say("2b_32k: oracle 4 teacher-forced passes at positions 33000..33003")
        _, drows, _ = ref.decode(4, force=F[1:5], keep_logits=True)
        del ref
        m.set_kv(Kd, Vd, int(F[0]))
        del Kd, Vd
        _, g_drows, _ = m.decode(4, force=F[1:5], logits=True)
        check_rows(g_drows, drows, label="2b_32k deep")
    finally:
        m.close()
    report_worst("2b_32k")


# ---- top-8 of 64 experts MoE, 512-pass requests ------------------------------------
def test_moe_prompt_routing_and_forced_request(torch_cuda):
    cfg = synth.get_config("moe")
    W = _weights("moe")
    P = synth.make_prompt(cfg)
    m = _model(cfg, W)
    try:
        done, ties = moe_request_parity(m, cfg, W, P, cfg.decode_steps, 12, "moe")
    finally:
        m.close()
    assert done >= 8 + 32


def test_moe_fp8_prompt_routing_and_forced_request(torch_cuda):
    """The MoE decoder with router and experts in row-scaled E4M3 (the oracle
    quantises the fp16 experts itself): the prompt, 4 two-pass trials, 16
    passes deep in the cache and the 512-pass request, as for fp16."""
    cfg = synth.get_config("moe_fp8")
    W = _weights("moe")          # the same fp16 tensors as the moe workload
    P = synth.make_prompt(cfg)
    m = _model(cfg, W)
    try:
        done, ties = moe_request_parity(m, cfg, W, P, cfg.decode_steps, 4, "moe_fp8", deep=16)
    finally:
        m.close()
    assert done >= 8 + 16


def test_moe_fp4_prompt_routing_and_forced_request(torch_cuda):
    """The MoE decoder with router and experts in row-scaled E2M1 (the oracle
    quantises the fp16 experts itself): the prompt, 4 two-pass trials, 16
    passes deep in the cache and the 512-pass request, as for fp8."""
    cfg = synth.get_config("moe_fp4")
    W = _weights("moe")          # the same fp16 tensors as the moe workload
    P = synth.make_prompt(cfg)
    m = _model(cfg, W)
    try:
        done, ties = moe_request_parity(m, cfg, W, P, cfg.decode_steps, 4, "moe_fp4", deep=16)
    finally:
        m.close()
    assert done >= 8 + 16
