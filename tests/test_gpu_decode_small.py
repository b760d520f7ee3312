"""Decode parity on small decoders: the persistent kernel against the oracle.

Every case is teacher-forced with the oracle's own greedy tokens, so the rows
compared are the logits of the same inputs; the bar is a z-scored max error of
2e-2 and equal argmax wherever the oracle's top-2 gap exceeds 2e-2. Sizes span
several workgroup tiles and ragged splits (rows per workgroup differing by one).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import check_rows, moe_request_parity, report_worst, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


TINY = synth.get_config("tiny")
CASES = {
    "tiny": TINY,
    # folded gains: non-unit RMSNorm gains exercise the offline folding
    "tiny_gains": TINY.with_(name="tiny_gains", gain_sigma=0.2, decode_steps=24),
    # GQA 4:1 with head_dim 64, d = 512 (two units per row)
    "gqa_hd64": synth.DecoderConfig(name="gqa_hd64", n_layers=2, d_model=512, n_heads=8, n_kv_heads=2,
                                    head_dim=64, ffn_dim=1536, vocab=3000, prompt_len=12, decode_steps=20),
    # head_dim 128, one KV head shared by 4 query heads, ragged QKV split
    "mqa_hd128": synth.DecoderConfig(name="mqa_hd128", n_layers=3, d_model=512, n_heads=4, n_kv_heads=1,
                                     head_dim=128, ffn_dim=1024, vocab=5000, prompt_len=9, decode_steps=16),
    # 8 query heads per KV head (attention in two passes of 4 heads), head_dim 64
    "gqa8_hd64": synth.DecoderConfig(name="gqa8_hd64", n_layers=2, d_model=512, n_heads=8, n_kv_heads=1,
                                     head_dim=64, ffn_dim=512, vocab=2048, prompt_len=40, decode_steps=12),
    # 6 query heads per KV head, head_dim 128, one workgroup per query head
    "gqa6_hd128": synth.DecoderConfig(name="gqa6_hd128", n_layers=2, d_model=1024, n_heads=12, n_kv_heads=2,
                                      head_dim=128, ffn_dim=1024, vocab=3000, prompt_len=70, decode_steps=10),
    # 2 query heads per KV head, head_dim 64, 379..394 attended positions: each
    # query head's positions go from one work item to two chunks of at most 384
    # mid-launch, the first chunk's workgroup folding in the second's state
    "gqa2_chunks_hd64": synth.DecoderConfig(name="gqa2_chunks_hd64", n_layers=2, d_model=512, n_heads=8,
                                            n_kv_heads=4, head_dim=64, ffn_dim=1024, vocab=2048,
                                            prompt_len=378, decode_steps=16),
    # the 2.1B decoder's attention shape (20 query / 4 KV heads x 128, 5 per
    # group) at 761..776 attended positions: two chunks per query head, then
    # three from 769 on
    "gqa5_chunks_hd128": synth.DecoderConfig(name="gqa5_chunks_hd128", n_layers=2, d_model=512, n_heads=20,
                                             n_kv_heads=4, head_dim=128, ffn_dim=1024, vocab=2048,
                                             prompt_len=760, decode_steps=16),
    # 4 query heads per KV head, 1137..1168 attended positions: three chunks per
    # query head, then the launch crosses the 1152-position limit of work items
    # per query head and goes on with the split over positions (matrix cores)
    # and its combine
    "gqa4_long_hd128": synth.DecoderConfig(name="gqa4_long_hd128", n_layers=2, d_model=512, n_heads=4,
                                           n_kv_heads=1, head_dim=128, ffn_dim=1024, vocab=2048,
                                           prompt_len=1136, decode_steps=32),
    # fp8 (E4M3, one scale per row) weights with non-unit RMSNorm gains folded
    # in before quantising; rows of 512 and 1024 (the per-unit input path)
    "fp8_d512_gains": synth.DecoderConfig(name="fp8_d512_gains", n_layers=2, d_model=512, n_heads=4,
                                          n_kv_heads=2, head_dim=128, ffn_dim=1024, vocab=2000, prompt_len=12,
                                          decode_steps=16, gain_sigma=0.2, weight_format="fp8"),
    # fp8 with rows of 2048 (inputs held in registers), a 1536-wide FFN and a
    # ragged LM split (1501 row pairs over 256 workgroups)
    "fp8_d2048": synth.DecoderConfig(name="fp8_d2048", n_layers=2, d_model=2048, n_heads=16, n_kv_heads=4,
                                     head_dim=128, ffn_dim=1536, vocab=3002, prompt_len=40, decode_steps=12,
                                     weight_format="fp8"),
    # fp4 (E2M1, one scale per row) weights, rows in fours, gains folded in;
    # rows of 512 and 1024 (the per-unit input path)
    "fp4_d512_gains": synth.DecoderConfig(name="fp4_d512_gains", n_layers=2, d_model=512, n_heads=4,
                                          n_kv_heads=2, head_dim=128, ffn_dim=1024, vocab=2000, prompt_len=12,
                                          decode_steps=16, gain_sigma=0.2, weight_format="fp4"),
    # fp4 with rows of 2048 (inputs in registers), a 1536-wide FFN, residual
    # rows split 8 / 12 per workgroup, and a ragged LM split (751 fours of rows)
    "fp4_d2048": synth.DecoderConfig(name="fp4_d2048", n_layers=2, d_model=2048, n_heads=16, n_kv_heads=4,
                                     head_dim=128, ffn_dim=1536, vocab=3004, prompt_len=40, decode_steps=12,
                                     weight_format="fp4"),
    # fp4 across head mode into the split over positions (matrix cores)
    "fp4_long": synth.DecoderConfig(name="fp4_long", n_layers=2, d_model=512, n_heads=4, n_kv_heads=1,
                                    head_dim=128, ffn_dim=1024, vocab=2048, prompt_len=1140, decode_steps=20,
                                    weight_format="fp4"),
}


def _model(cfg, W):
    from memory_bandwidth_bound_amd import kie
    return kie.Model(cfg, W)


def _oracle_run(cfg, W, P, n):
    """Oracle free run: first token, n greedy tokens, logits of prefill's last
    pass and of every decode pass."""
    dec = oracle.Decoder(cfg, W)
    first, last = dec.prefill(P)
    ids, rows, _ = dec.decode(n, keep_logits=True)
    return first, last, ids, rows


@pytest.mark.parametrize("name", list(CASES))
def test_teacher_forced_parity(torch_cuda, name):
    cfg = CASES[name]
    say(f"case {name}: {cfg}")
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    n = cfg.decode_steps
    first, last, ids, rows = _oracle_run(cfg, W, P, n)
    m = _model(cfg, W)
    say(f"{name}: prefill {len(P)} tokens")
    g_first, g_logits, _ = m.prefill(P, logits=True)
    check_rows(g_logits[-1:], last[None], label=f"{name} prefill")
    if oracle.top2_gap(last) > 2e-2:
        assert g_first == first
    say(f"{name}: decode {n} teacher-forced")
    # restart from the oracle's first token so both sides feed identical inputs
    m.rewind(len(P), first)
    g_ids, g_rows, _ = m.decode(n, force=ids, logits=True)
    check_rows(g_rows, rows, label=f"{name} decode")
    assert m.state() == (len(P) + n, int(ids[-1]))
    m.close()
    report_worst(name)


def test_free_run_tokens_and_determinism(torch_cuda):
    cfg = TINY
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    first, _, ids, rows = _oracle_run(cfg, W, P, cfg.decode_steps)
    m = _model(cfg, W)
    say("tiny free run")
    g_first, _, _ = m.prefill(P)
    a, la, _ = m.decode(cfg.decode_steps, logits=True)
    # free-running tokens equal the oracle's while no near-tie has occurred
    gaps = [oracle.top2_gap(r) for r in rows]
    agree = 0
    for i in range(cfg.decode_steps):
        if a[i] != ids[i]:
            assert gaps[i] <= 2e-2, f"step {i}: token {a[i]} != {ids[i]} with gap {gaps[i]:.3e}"
            break
        agree += 1
    say(f"free run: {agree}/{cfg.decode_steps} tokens identical to the oracle")
    # bitwise determinism: the same request twice
    m.rewind(len(P), g_first)
    b, lb, _ = m.decode(cfg.decode_steps, logits=True)
    assert np.array_equal(a, b)
    assert np.array_equal(la, lb)
    m.close()


def test_continuation_equals_one_launch(torch_cuda):
    cfg = TINY
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    m = _model(cfg, W)
    say("tiny continuation")
    f, _, _ = m.prefill(P)
    whole, lw, _ = m.decode(40, logits=True)
    m.rewind(len(P), f)
    p1, l1, _ = m.decode(17, logits=True)
    p2, l2, _ = m.decode(23, logits=True)
    assert np.array_equal(np.concatenate([p1, p2]), whole)
    assert np.array_equal(np.concatenate([l1, l2]), lw)
    # one launch without debug buffers gives the same tokens
    m.rewind(len(P), f)
    fast, _, _ = m.decode(40)
    assert np.array_equal(fast, whole)
    m.close()


def test_long_context_split_attention(torch_cuda):
    """A pre-filled cache long enough that every KV head's attention is split
    over many workgroups and combined by the last one to finish."""
    cfg = synth.DecoderConfig(name="tiny_ctx", n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64,
                              ffn_dim=1024, vocab=4096, prompt_len=0, decode_steps=6, kv_prefill=3000)
    W = synth.make_weights(cfg)
    K, V = synth.make_kv_prefill(cfg)
    pend = synth.make_pending_token(cfg)
    dec = oracle.Decoder(cfg, W)
    dec.set_kv(K, V, pend)
    ids, rows, _ = dec.decode(cfg.decode_steps, keep_logits=True)
    m = _model(cfg, W)
    say("tiny_ctx: set_kv 3000 positions, decode 6")
    m.set_kv(K, V, pend)
    g_ids, g_rows, _ = m.decode(cfg.decode_steps, force=ids, logits=True)
    check_rows(g_rows, rows, label="tiny_ctx decode")
    m.close()


SPLIT_CASES = {
    # one query head per KV head, head_dim 128: attention is always split over
    # positions (matrix-core rounds of 16), here from the first position on,
    # the prompt run as decode passes
    "mha_hd128_passes": synth.DecoderConfig(name="mha_hd128_passes", n_layers=2, d_model=512, n_heads=4,
                                            n_kv_heads=4, head_dim=128, ffn_dim=1024, vocab=2048,
                                            prompt_len=7, decode_steps=40),
    # 8 query heads per KV head, head_dim 128, 1147..1160 attended positions:
    # head mode, then from 1153 on the split over positions with all eight
    # heads in one matrix-core pass
    "gqa8_split_hd128": synth.DecoderConfig(name="gqa8_split_hd128", n_layers=2, d_model=1024, n_heads=8,
                                            n_kv_heads=1, head_dim=128, ffn_dim=1024, vocab=2048,
                                            prompt_len=1146, decode_steps=14),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_split_attention_parity(torch_cuda, name):
    cfg = SPLIT_CASES[name]
    say(f"case {name}: {cfg}")
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    n = cfg.decode_steps
    first, last, ids, rows = _oracle_run(cfg, W, P, n)
    m = _model(cfg, W)
    say(f"{name}: prefill {len(P)} tokens")
    if name.endswith("_passes"):
        # every prompt pass, from the first position on, against the oracle's
        m.set_prefill_mode("passes")
        dec = oracle.Decoder(cfg, W)
        prompt_rows = np.stack([dec.step(int(t)) for t in P])
        g_first, g_logits, _ = m.prefill(P, logits=True)
        assert g_logits.shape[0] == len(P)
        check_rows(g_logits, prompt_rows, label=f"{name} prompt passes")
    else:
        g_first, g_logits, _ = m.prefill(P, logits=True)
    check_rows(g_logits[-1:], last[None], label=f"{name} prefill")
    if oracle.top2_gap(last) > 2e-2:
        assert g_first == first
    say(f"{name}: decode {n} teacher-forced")
    m.rewind(len(P), first)
    g_ids, g_rows, _ = m.decode(n, force=ids, logits=True)
    check_rows(g_rows, rows, label=f"{name} decode")
    m.close()
    report_worst(name)


def test_capacity_and_state_errors(torch_cuda):
    from memory_bandwidth_bound_amd import kie
    cfg = TINY.with_(decode_steps=4)
    W = synth.make_weights(cfg)
    m = _model(cfg, W)
    with pytest.raises(kie.KieError) as e:
        m.decode(1)
    assert e.value.code == -8          # no pending token yet
    P = synth.make_prompt(cfg)
    m.prefill(P)
    with pytest.raises(kie.KieError) as e:
        m.decode(cfg.max_seq)           # position + n > max_seq
    assert e.value.code == -3
    with pytest.raises(kie.KieError) as e:
        m.prefill(np.array([cfg.vocab], dtype=np.int32))
    assert e.value.code == -1
    m.close()


# ---- MoE -----------------------------------------------------------------------
MOE_CASES = {
    # 8 experts, top-2, head_dim 128
    "moe_e8k2": synth.DecoderConfig(name="moe_e8k2", n_layers=2, d_model=512, n_heads=4, n_kv_heads=2,
                                    head_dim=128, ffn_dim=512, vocab=3000, n_experts=8, top_k=2,
                                    prompt_len=10, decode_steps=16),
    # 64 experts, top-8 (the gathered down input is 8192 wide), head_dim 64
    "moe_e64k8": synth.DecoderConfig(name="moe_e64k8", n_layers=3, d_model=1024, n_heads=8, n_kv_heads=2,
                                     head_dim=64, ffn_dim=1024, vocab=5000, n_experts=64, top_k=8,
                                     prompt_len=8, decode_steps=12),
}


MOE_CASES.update({
    # fp8 router and experts: 8 experts, top-2, the router's 8 rows in pairs
    "moe_fp8_e8k2": synth.DecoderConfig(name="moe_fp8_e8k2", n_layers=2, d_model=512, n_heads=4, n_kv_heads=2,
                                        head_dim=128, ffn_dim=512, vocab=3000, n_experts=8, top_k=2,
                                        prompt_len=10, decode_steps=16, gain_sigma=0.2, weight_format="fp8"),
    # fp8, 64 experts, top-8: the gathered down input is 8192 wide, rows of 1024
    "moe_fp8_e64k8": synth.DecoderConfig(name="moe_fp8_e64k8", n_layers=2, d_model=1024, n_heads=8,
                                         n_kv_heads=2, head_dim=128, ffn_dim=1024, vocab=5000, n_experts=64,
                                         top_k=8, prompt_len=8, decode_steps=12, weight_format="fp8"),
    # fp4 router and experts: 8 experts, top-2, the router's 8 rows in two
    # fours, expert rows in fours, gains folded in
    "moe_fp4_e8k2": synth.DecoderConfig(name="moe_fp4_e8k2", n_layers=2, d_model=512, n_heads=4, n_kv_heads=2,
                                        head_dim=128, ffn_dim=512, vocab=3000, n_experts=8, top_k=2,
                                        prompt_len=10, decode_steps=16, gain_sigma=0.2, weight_format="fp4"),
    # fp4, 64 experts, top-8: the gathered down input is 8192 wide, rows of 1024
    "moe_fp4_e64k8": synth.DecoderConfig(name="moe_fp4_e64k8", n_layers=2, d_model=1024, n_heads=8,
                                         n_kv_heads=2, head_dim=128, ffn_dim=1024, vocab=5000, n_experts=64,
                                         top_k=8, prompt_len=8, decode_steps=12, weight_format="fp4"),
})


@pytest.mark.parametrize("name", list(MOE_CASES))
def test_moe_teacher_forced_parity(torch_cuda, name):
    cfg = MOE_CASES[name]
    say(f"case {name}: {cfg}")
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    m = _model(cfg, W)
    try:
        done, _ = moe_request_parity(m, cfg, W, P, cfg.decode_steps, 6, name)
    finally:
        m.close()
    assert done >= 8


# ---- XCD-local attention ----------------------------------------------------------
XCD_CASES = {
    # the 2.1B decoder's attention shape (20 query / 4 KV heads x 128) at 371..394
    # attended positions: 20 items per XCD up to 384, then two chunks per head
    # (40 items) no longer fit one XCD and the launch goes on in global head mode
    "xcd_gqa5_hd128": synth.DecoderConfig(name="xcd_gqa5_hd128", n_layers=2, d_model=512, n_heads=20,
                                          n_kv_heads=4, head_dim=128, ffn_dim=1024, vocab=2048,
                                          prompt_len=370, decode_steps=24),
    # 8 query heads at 379..394 positions: one chunk per head, then two (16
    # items per XCD), the first chunk's workgroup merging the second's state
    # through its own XCD's copy
    "gqa2_chunks_hd64": CASES["gqa2_chunks_hd64"],
    # 8 query heads per KV head (attention in two passes of 4 heads)
    "gqa8_hd64": CASES["gqa8_hd64"],
    # 4 query heads at 1137..1168 positions: three chunks per head (12 items
    # per XCD), then past 1152 the split over positions on the matrix cores
    # (the kernel variant with it, launched with the XCD-local flag set)
    "gqa4_long_hd128": CASES["gqa4_long_hd128"],
    # quantised weights: fp8 (16 query heads) and fp4 with folded gains
    "fp8_d2048": CASES["fp8_d2048"],
    "fp4_d512_gains": CASES["fp4_d512_gains"],
    # MoE: 8 experts, top-2
    "moe_e8k2": MOE_CASES["moe_e8k2"],
    # the most query heads the mode takes: 32, one item on every workgroup of
    # each XCD (8 query heads per KV head)
    "xcd_h32_hd128": synth.DecoderConfig(name="xcd_h32_hd128", n_layers=1, d_model=4096, n_heads=32,
                                         n_kv_heads=4, head_dim=128, ffn_dim=512, vocab=2048, prompt_len=20,
                                         decode_steps=12),
}


@pytest.mark.parametrize("name", list(XCD_CASES))
def test_xcd_local_attention_parity(torch_cuda, name):
    """XCD-local attention: every XCD computes all heads' attention for its own
    output-projection rows. Logits against the oracle's (teacher-forced), and
    bit for bit equal to the global head mode's on the same passes."""
    cfg = XCD_CASES[name]
    say(f"case {name} (xcd_local): {cfg}")
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    n = cfg.decode_steps
    first, last, ids, rows = _oracle_run(cfg, W, P, n)
    m = _model(cfg, W)
    try:
        m.prefill(P)
        m.rewind(len(P), first)
        _, glob_rows, _ = m.decode(n, force=ids, logits=True)
        m.set_attention_mode("xcd_local")
        say(f"{name}: decode {n} teacher-forced, XCD-local attention")
        m.rewind(len(P), first)
        x_ids, x_rows, _ = m.decode(n, force=ids, logits=True)
        assert np.array_equal(x_rows, glob_rows), f"{name}: XCD-local logits differ from the global mode's"
        if cfg.n_experts:
            # near ties in routing may pick other experts than the oracle: the
            # bit-identity above covers the mode, the request check the rest
            m.reset()   # the mode stays; the check starts from a model without state
            done, _ = moe_request_parity(m, cfg, W, P, n, 6, name + "/xcd")
            assert done >= 8
        else:
            check_rows(x_rows, rows, label=f"{name}/xcd decode")
        # one launch without the debug buffers: the same ids
        m.prefill(P)
        m.rewind(len(P), first)
        s_ids, _, _ = m.decode(n, force=ids)
        assert np.array_equal(s_ids, x_ids)
    finally:
        m.close()
    if not cfg.n_experts:
        report_worst(name + "/xcd")


def test_xcd_local_attention_rejected_where_it_cannot_run(torch_cuda):
    """One query head per KV head (no head mode) and more query heads than one
    XCD's 32 workgroups are configuration errors; unknown modes are argument
    errors."""
    from memory_bandwidth_bound_amd import kie
    for cfg in (TINY.with_(decode_steps=4),
                synth.DecoderConfig(name="h40", n_layers=1, d_model=2560, n_heads=40, n_kv_heads=8,
                                    head_dim=64, ffn_dim=512, vocab=512, prompt_len=4, decode_steps=4)):
        m = _model(cfg, synth.make_weights(cfg))
        try:
            with pytest.raises(kie.KieError) as e:
                m.set_attention_mode("xcd_local")
            assert e.value.code == -2
            m.set_attention_mode("global")
            assert m._lib.kie_set_attention_mode(m._h, 7) == -1
        finally:
            m.close()


# ---- degenerate inputs ----------------------------------------------------------
def test_one_token_prompt_and_empty_cache(torch_cuda):
    """A one-token prompt, and decoding from an empty cache (set_kv with no
    positions): the first pass attends only to itself."""
    cfg = TINY.with_(prompt_len=1, decode_steps=6)
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    ref = oracle.Decoder(cfg, W)
    first, last = ref.prefill(P)
    ids, rows, _ = ref.decode(cfg.decode_steps, keep_logits=True)
    m = _model(cfg, W)
    try:
        g_first, g_logits, _ = m.prefill(P, logits=True)
        check_rows(g_logits[-1:], last[None], label="one-token prefill")
        m.rewind(1, first)
        _, g_rows, _ = m.decode(cfg.decode_steps, force=ids, logits=True)
        check_rows(g_rows, rows, label="one-token prompt decode")

        K = np.zeros((cfg.n_layers, 0, cfg.n_kv_heads, cfg.head_dim), dtype=np.float16)
        pend = int(P[0])
        ref2 = oracle.Decoder(cfg, W)
        ref2.set_kv(K, K, pend)
        ids2, rows2, _ = ref2.decode(4, keep_logits=True)
        m.set_kv(K, K, pend)
        _, g_rows2, _ = m.decode(4, force=ids2, logits=True)
        check_rows(g_rows2, rows2, label="empty-cache decode")
    finally:
        m.close()


def test_empty_requests_are_rejected(torch_cuda):
    from memory_bandwidth_bound_amd import kie
    cfg = TINY.with_(decode_steps=4)
    m = _model(cfg, synth.make_weights(cfg))
    try:
        with pytest.raises(kie.KieError) as e:
            m.prefill(np.zeros(0, dtype=np.int32))
        assert e.value.code == -1
        m.prefill(synth.make_prompt(cfg))
        with pytest.raises(kie.KieError) as e:
            m.decode(0)
        assert e.value.code == -1
        assert m.state()[0] == cfg.prompt_len      # a rejected call changes nothing
    finally:
        m.close()


def test_two_token_vocabulary(torch_cuda):
    """The smallest vocabulary: two LM rows, so all but two workgroups have no
    LM rows and the device argmax reduces mostly empty entries."""
    cfg = TINY.with_(name="tiny_v2", vocab=2, decode_steps=10)
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    first, last, ids, rows = _oracle_run(cfg, W, P, cfg.decode_steps)
    m = _model(cfg, W)
    try:
        g_first, g_logits, _ = m.prefill(P, logits=True)
        check_rows(g_logits[-1:], last[None], label="vocab 2 prefill")
        m.rewind(len(P), first)
        g_ids, g_rows, _ = m.decode(cfg.decode_steps, force=ids, logits=True)
        check_rows(g_rows, rows, label="vocab 2 decode")
        assert np.array_equal(g_ids, np.argmax(g_rows, axis=1))
    finally:
        m.close()


# ---- failure handling: every wait is bounded, the kernel always exits ----------
def test_spin_limit_timeout_then_recovery(torch_cuda):
    """A device wait limit of one poll: the first wait that finds its input
    unpublished gives up, flags the failure, every other workgroup's waits
    give up too and the kernel exits normally; the call returns
    KIE_ERR_TIMEOUT. After kie_reset the model decodes exactly as before."""
    from memory_bandwidth_bound_amd import kie
    cfg = TINY.with_(decode_steps=8)
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    m = _model(cfg, W)
    try:
        first, _, _ = m.prefill(P)
        want, _, _ = m.decode(8)
        m.set_limits(spin_limit=1)
        m.rewind(len(P), first)
        say("spin limit 1: expecting KIE_ERR_TIMEOUT")
        with pytest.raises(kie.KieError) as e:
            m.decode(8)
        assert e.value.code == -7
        assert m.state()[1] == -1              # no pending token after a timeout
        m.set_limits(0, 0)
        m.reset()
        assert m.prefill(P)[0] == first
        got, _, _ = m.decode(8)
        assert np.array_equal(got, want)
    finally:
        m.close()


def test_host_watchdog_reports_overrun_then_recovery(torch_cuda):
    """A host watchdog of 1 ms around a launch of 1500 passes (about 80 ms):
    the host raises its abort word and the call returns KIE_ERR_TIMEOUT once
    the launch has ended; after kie_reset the model decodes as before."""
    from memory_bandwidth_bound_amd import kie
    cfg = TINY.with_(name="tiny_long", prompt_len=4, decode_steps=1500)
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    m = _model(cfg, W)
    try:
        first, _, _ = m.prefill(P)
        want, _, _ = m.decode(16)
        m.set_limits(watchdog_ms=1)
        m.rewind(len(P), first)
        say("watchdog 1 ms over 1500 passes: expecting KIE_ERR_TIMEOUT")
        with pytest.raises(kie.KieError) as e:
            m.decode(cfg.decode_steps)
        assert e.value.code == -7 and "watchdog" in str(e.value)
        m.set_limits(0, 0)
        m.reset()
        assert m.prefill(P)[0] == first
        got, _, _ = m.decode(16)
        assert np.array_equal(got, want)
    finally:
        m.close()


# ---- the batched (matrix-core) prefill ---------------------------------------------
@pytest.mark.parametrize("name", ["tiny_gains", "gqa5_chunks_hd128", "gqa8_hd64", "fp8_d512_gains", "fp8_d2048",
                                  "fp4_d2048", "fp4_long"])
def test_batched_prefill_rows_and_modes(torch_cuda, name):
    """Every prompt row's logits from the batched prefill against the oracle's
    full causal forward, element by element (the 760- and 1140-token prompts
    span three and five chunks of 256; fp8 and fp4 weights go through the
    GEMM converted to fp16 with their row scales on the outputs); the same
    prompt prefilled pass by pass gives the same first token wherever the gap
    decides it, and decoding after either prefill matches the oracle."""
    cfg = CASES[name]
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    say(f"{name}: oracle full forward over the {len(P)}-token prompt")
    ref = oracle.Decoder(cfg, W)
    rows = ref.forward_full(list(P))
    first = int(np.argmax(rows[-1]))
    dec = oracle.Decoder(cfg, W)
    dec.prefill_batched(P)
    ids, drows, _ = dec.decode(4, keep_logits=True)
    m = _model(cfg, W)
    try:
        g_first, g_logits, _ = m.prefill(P, logits=True)
        check_rows(g_logits, rows, label=f"{name} batched-prefill")
        if oracle.top2_gap(rows[-1]) > 2e-2:
            assert g_first == first
        m.rewind(len(P), first)
        _, g_rows, _ = m.decode(4, force=ids, logits=True)
        check_rows(g_rows, drows, label=f"{name} after-batched")
        m.set_prefill_mode("passes")
        p_first, p_logits, _ = m.prefill(P, logits=True)
        check_rows(p_logits[-1:], rows[-1:], label=f"{name} passes-prefill")
        if oracle.top2_gap(rows[-1]) > 2e-2:
            assert p_first == g_first
        m.rewind(len(P), first)
        _, p_rows, _ = m.decode(4, force=ids, logits=True)
        check_rows(p_rows, drows, label=f"{name} after-passes")
    finally:
        m.close()
