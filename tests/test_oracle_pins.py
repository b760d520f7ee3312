"""Pins for the CPU oracle: each test ties an oracle function to something other
than itself (closed forms, invariants, brute force on tiny inputs, the pages'
printed figures), chosen so that a dropped term, a wrong sign, a wrong index or
a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import (apply_rope, attention_decode, gemv_f64, greedy_argmax, rmsnorm,
                    rope_angles, silu, softmax, swiglu_ffn, topk_experts)
from synth import DecoderConfig, make_prompt, make_weights, tensor_specs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _const(name):
    with open(os.path.join(GOLDEN, "constants.json")) as f:
        return json.load(f)[name]["value"]


# ---------------------------------------------------------------- GEMV -----

def test_gemv_integer_exact():
    rng = np.random.default_rng(1)
    A = rng.integers(-8, 9, size=(37, 300)).astype(np.float16)
    x = rng.integers(-8, 9, size=300).astype(np.float16)
    want = [sum(int(A[i, k]) * int(x[k]) for k in range(300)) for i in range(37)]
    assert np.array_equal(gemv_f64(A, x), np.array(want, dtype=np.float64))


def test_gemv_unit_vector_returns_column():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((19, 33)).astype(np.float16)
    for j in (0, 7, 32):
        e = np.zeros(33, dtype=np.float16)
        e[j] = 1
        assert np.array_equal(gemv_f64(A, e), A[:, j].astype(np.float64))


def test_gemv_not_transposed():
    A = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float16)
    x = np.array([1, 0, -1], dtype=np.float16)
    assert np.array_equal(gemv_f64(A, x), np.array([-2.0, -2.0]))
    x = np.array([0, 1, 0], dtype=np.float16)
    assert np.array_equal(gemv_f64(A, x), np.array([2.0, 5.0]))


# ------------------------------------------------------------- RMSNorm -----

@pytest.mark.parametrize("c", [1e-3, 0.5, 3.0, -2.0])
def test_rmsnorm_constant_vector(c):
    eps = 1e-5
    g = np.linspace(0.5, 1.5, 16)
    x = np.full(16, c, dtype=np.float64)
    want = c / math.sqrt(c * c + eps) * g
    np.testing.assert_allclose(rmsnorm(x, g, eps), want, rtol=1e-14)


def test_rmsnorm_mean_square():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1000) * 0.01
    m = float(np.mean(x * x))
    eps = 1e-5
    y = rmsnorm(x, np.ones(1000), eps)
    np.testing.assert_allclose(np.mean(y * y), m / (m + eps), rtol=1e-12)


def test_rmsnorm_rows_independent():
    x = np.array([[1.0, 1.0], [3.0, 3.0]])
    y = rmsnorm(x, np.ones(2), 0.0)
    np.testing.assert_allclose(y, np.ones((2, 2)), rtol=1e-15)


# ---------------------------------------------------------------- RoPE -----

def test_rope_table_entries():
    cos, sin = rope_angles([0, 1], 128, 1e4)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    assert cos[1, 0] == pytest.approx(_const("cos_1"), abs=1e-16)
    assert sin[1, 0] == pytest.approx(_const("sin_1"), abs=1e-16)
    # frequency index 1 at position 1: angle theta^(-2/hd)
    ang = 1e4 ** (-2.0 / 128)
    assert cos[1, 1] == pytest.approx(math.cos(ang), abs=1e-15)
    # the last frequency is the slowest
    assert sin[1, -1] == pytest.approx(math.sin(1e4 ** (-126.0 / 128)), abs=1e-15)


def test_rope_position_zero_identity():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((3, 64))
    c, s = rope_angles([0], 64, 1e4)
    np.testing.assert_array_equal(apply_rope(v, c, s), v)


def test_rope_pairs_i_with_i_plus_half():
    hd = 8
    c, s = rope_angles([1], hd, 1e4)
    for i in range(hd // 2):
        e = np.zeros(hd)
        e[i] = 1.0
        r = apply_rope(e, c[0], s[0])
        ang = 1e4 ** (-2.0 * i / hd)
        want = np.zeros(hd)
        want[i] = math.cos(ang)
        want[i + hd // 2] = math.sin(ang)
        np.testing.assert_allclose(r, want, atol=1e-15)
        e = np.zeros(hd)
        e[i + hd // 2] = 1.0
        r = apply_rope(e, c[0], s[0])
        want = np.zeros(hd)
        want[i] = -math.sin(ang)
        want[i + hd // 2] = math.cos(ang)
        np.testing.assert_allclose(r, want, atol=1e-15)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(5)
    hd = 64
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    for m, n in [(7, 3), (100, 40), (33000, 32000)]:
        cm, sm = rope_angles([m], hd, 1e4)
        cn, sn = rope_angles([n], hd, 1e4)
        cd, sd = rope_angles([m - n], hd, 1e4)
        qm = apply_rope(q, cm[0], sm[0])
        kn = apply_rope(k, cn[0], sn[0])
        # norm of every rotated pair is preserved
        half = hd // 2
        np.testing.assert_allclose(qm[:half] ** 2 + qm[half:] ** 2,
                                   q[:half] ** 2 + q[half:] ** 2, rtol=1e-12)
        lhs = float(qm @ kn)
        rhs = float(apply_rope(q, cd[0], sd[0]) @ k)
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)


# ------------------------------------------------------ softmax / attn -----

def test_softmax_closed_form_and_invariants():
    np.testing.assert_allclose(softmax(np.array([0.0, math.log(3.0)])),
                               _const("softmax_0_ln3"), rtol=1e-15)
    rng = np.random.default_rng(6)
    s = rng.standard_normal(1000).astype(np.float32) * 5
    p = softmax(s)
    assert abs(float(p.sum()) - 1.0) < 1e-6
    np.testing.assert_allclose(softmax(s + np.float32(50.0)), p, rtol=1e-5, atol=1e-9)
    assert np.argmax(p) == np.argmax(s)


def test_attention_single_position_returns_value():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 16))
    K = rng.standard_normal((1, 2, 16))
    V = rng.standard_normal((1, 2, 16))
    o = attention_decode(q, K, V)
    np.testing.assert_array_equal(o[:2], np.broadcast_to(V[0, 0], (2, 16)))
    np.testing.assert_array_equal(o[2:], np.broadcast_to(V[0, 1], (2, 16)))


def test_attention_equal_keys_mean_of_values():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 8))
    K = np.repeat(rng.standard_normal((1, 1, 8)), 5, axis=0)
    V = rng.standard_normal((5, 1, 8))
    np.testing.assert_allclose(attention_decode(q, K, V)[0], V[:, 0].mean(axis=0), rtol=1e-12)


def test_attention_scale_and_weights():
    hd = 16
    q = np.zeros((1, hd)); q[0, 0] = 2.0
    K = np.zeros((2, 1, hd)); K[1, 0, 0] = 3.0          # scores 0 and 6/sqrt(16) = 1.5
    V = np.zeros((2, 1, hd)); V[0, 0, 1] = 1.0; V[1, 0, 2] = 1.0
    o = attention_decode(q, K, V)[0]
    w1 = 1.0 / (1.0 + math.exp(-1.5))
    assert o[2] == pytest.approx(w1, rel=1e-14)
    assert o[1] == pytest.approx(1.0 - w1, rel=1e-13)


def test_attention_gqa_head_map():
    H, Hkv, hd, c = 6, 2, 4, 3
    rng = np.random.default_rng(9)
    q = rng.standard_normal((H, hd))
    K = rng.standard_normal((c, Hkv, hd))
    V = np.zeros((c, Hkv, hd))
    V[:, 0, :] = 1.0
    V[:, 1, :] = 2.0
    o = attention_decode(q, K, V)
    np.testing.assert_allclose(o[:3], 1.0, rtol=1e-14)   # heads 0..2 -> kv head 0
    np.testing.assert_allclose(o[3:], 2.0, rtol=1e-14)   # heads 3..5 -> kv head 1


# -------------------------------------------------------------- SwiGLU -----

def test_silu_values():
    assert silu(np.float64(0.0)) == 0.0
    assert silu(np.float64(1.0)) == pytest.approx(_const("silu_at_1"), rel=1e-15)
    z = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(silu(z) - silu(-z), z, atol=1e-14)


def test_swiglu_gate_and_up_not_swapped():
    h = np.array([0.5, -1.0, 2.0])
    I = np.eye(3)
    a, b, c = 2.0, 3.0, 0.5
    out = swiglu_ffn(h, a * I, b * I, c * I)
    want = c * (a * h / (1 + np.exp(-a * h))) * (b * h)
    np.testing.assert_allclose(out, want, rtol=1e-14)
    swapped = c * (b * h / (1 + np.exp(-b * h))) * (a * h)
    assert not np.allclose(out, swapped)


# ------------------------------------------------------------- top-k -------

def test_topk_ties_to_lower_index():
    p = np.array([0.1, 0.3, 0.3, 0.05, 0.3])
    assert list(topk_experts(p, 2)) == [1, 2]
    assert list(topk_experts(np.full(64, 1 / 64), 8)) == list(range(8))
    assert list(topk_experts(np.array([0.0, 0.0, 1.0]), 1)) == [2]


def test_argmax_ties_to_lowest_index():
    assert greedy_argmax(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert greedy_argmax(np.array([-1.0, -1.0])) == 0


# ---------------------------------------------------------- the decoder ----

def _tiny(**kw):
    base = dict(name="pin", n_layers=2, d_model=16, n_heads=4, n_kv_heads=2, head_dim=4,
                ffn_dim=12, vocab=23, prompt_len=5, decode_steps=6, gain_sigma=0.2)
    base.update(kw)
    return DecoderConfig(**base)


def _brute_logits(cfg, W, tokens, kv16=True, experts=None):
    """Plain scalar loops in float64 from the written-out definition; with
    kv16 every cached key and value is rounded to fp16 as it is stored.
    MoE: experts[p][l], if given, is the expert set mixed at position p and
    layer l (with the router's probabilities) instead of the router's top-k."""
    names = [n for n, _, _ in tensor_specs(cfg)]
    T = {n: np.asarray(t, dtype=np.float64) for n, t in zip(names, W)}
    d, H, Hkv, hd = cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim

    def mv(M, v):
        return [sum(M[i][k] * v[k] for k in range(len(v))) for i in range(len(M))]

    def norm(v, g):
        ms = sum(a * a for a in v) / len(v)
        r = 1.0 / math.sqrt(ms + cfg.rms_eps)
        return [v[i] * r * g[i] for i in range(len(v))]

    def rot(vec, p):
        out = list(vec)
        half = hd // 2
        for i in range(half):
            ang = p * cfg.rope_theta ** (-2.0 * i / hd)
            a, b = vec[i], vec[i + half]
            out[i] = a * math.cos(ang) - b * math.sin(ang)
            out[i + half] = b * math.cos(ang) + a * math.sin(ang)
        return out

    def ffn(h, Wg, Wu, Wd):
        g = mv(Wg, h)
        u = mv(Wu, h)
        z = [g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(len(g))]
        return mv(Wd, z)

    cacheK = [[] for _ in range(cfg.n_layers)]
    cacheV = [[] for _ in range(cfg.n_layers)]
    result = []
    for p, tok in enumerate(tokens):
        x = list(T["E"][tok])
        for l in range(cfg.n_layers):
            h = norm(x, T[f"l{l}.g_attn"])
            q = mv(T[f"l{l}.Wq"], h)
            k = mv(T[f"l{l}.Wk"], h)
            v = mv(T[f"l{l}.Wv"], h)
            qh = [rot(q[j * hd:(j + 1) * hd], p) for j in range(H)]
            kh = [rot(k[g * hd:(g + 1) * hd], p) for g in range(Hkv)]
            vh = [v[g * hd:(g + 1) * hd] for g in range(Hkv)]
            if kv16:
                kh = [[float(np.float16(a)) for a in row] for row in kh]
                vh = [[float(np.float16(a)) for a in row] for row in vh]
            cacheK[l].append(kh)
            cacheV[l].append(vh)
            o = []
            for j in range(H):
                g = j // (H // Hkv)
                sc = [sum(qh[j][i] * cacheK[l][u][g][i] for i in range(hd)) / math.sqrt(hd)
                      for u in range(p + 1)]
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                tot = sum(ex)
                o += [sum(ex[u] / tot * cacheV[l][u][g][i] for u in range(p + 1))
                      for i in range(hd)]
            y = mv(T[f"l{l}.Wo"], o)
            x = [x[i] + y[i] for i in range(d)]
            h = norm(x, T[f"l{l}.g_ffn"])
            if cfg.n_experts:
                r = mv(T[f"l{l}.Wr"], h)
                mx = max(r)
                ex = [math.exp(a - mx) for a in r]
                pi = [a / sum(ex) for a in ex]
                order = sorted(range(cfg.n_experts), key=lambda e: (-pi[e], e))[:cfg.top_k]
                if experts is not None:
                    order = [int(e) for e in experts[p][l]]
                y = [0.0] * d
                for e in order:
                    ye = ffn(h, T[f"l{l}.e{e}.Wg"], T[f"l{l}.e{e}.Wu"], T[f"l{l}.e{e}.Wd"])
                    y = [y[i] + pi[e] * ye[i] for i in range(d)]
            else:
                y = ffn(h, T[f"l{l}.Wg"], T[f"l{l}.Wu"], T[f"l{l}.Wd"])
            x = [x[i] + y[i] for i in range(d)]
        result.append(mv(T["W_lm"], norm(x, T["g_final"])))
    return np.array(result)


@pytest.mark.parametrize("kw", [dict(), dict(n_experts=5, top_k=2, ffn_dim=6)])
def test_decoder_matches_scalar_brute_force(kw):
    cfg = _tiny(**kw)
    W = make_weights(cfg)
    toks = [3, 17, 0, 22, 9, 9, 1]
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    got = np.stack([dec.step(t) for t in toks])
    want = _brute_logits(cfg, W, toks)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    # a cache at the compute precision is the same definition without the rounding
    exact = oracle.Decoder(cfg, W, dtype=np.float64, kv_dtype=None)
    got = np.stack([exact.step(t) for t in toks])
    np.testing.assert_allclose(got, _brute_logits(cfg, W, toks, kv16=False), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("kw", [dict(), dict(n_experts=6, top_k=3, ffn_dim=6)])
def test_decoder_incremental_equals_full_causal(kw):
    cfg = _tiny(n_layers=3, vocab=50, **kw)
    W = make_weights(cfg)
    toks = [int(t) for t in np.random.default_rng(10).integers(0, cfg.vocab, 9)]
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    inc = np.stack([dec.step(t) for t in toks])
    full = oracle.Decoder(cfg, W, dtype=np.float64).forward_full(toks)
    np.testing.assert_allclose(inc, full, rtol=1e-11, atol=1e-12)


def test_batched_prefill_equals_incremental_prefill():
    cfg = _tiny(n_layers=2, vocab=40, decode_steps=4)
    W = make_weights(cfg)
    P = [int(t) for t in np.random.default_rng(15).integers(0, cfg.vocab, cfg.prompt_len)]
    a = oracle.Decoder(cfg, W, dtype=np.float64)
    b = oracle.Decoder(cfg, W, dtype=np.float64)
    fa, la = a.prefill(P)
    fb, lb = b.prefill_batched(P)
    assert fa == fb and a.pos == b.pos == len(P)
    np.testing.assert_allclose(la, lb, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(a.K, b.K, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(a.V, b.V, rtol=1e-11, atol=1e-13)
    ia, ra, _ = a.decode(3, keep_logits=True)
    ib, rb, _ = b.decode(3, keep_logits=True)
    np.testing.assert_array_equal(ia, ib)
    np.testing.assert_allclose(ra, rb, rtol=1e-10, atol=1e-12)


def test_moe_expert_overrides_follow_the_definition():
    """An overridden expert set is mixed with the router's own probabilities,
    in the incremental pass and in the full causal forward alike."""
    cfg = _tiny(n_experts=6, top_k=2, ffn_dim=6, n_layers=2, vocab=30)
    W = make_weights(cfg)
    toks = [4, 11, 29, 0, 7]
    rng = np.random.default_rng(16)
    ov = [[sorted(rng.choice(cfg.n_experts, cfg.top_k, replace=False).tolist()) for _ in range(cfg.n_layers)]
          for _ in toks]
    want = _brute_logits(cfg, W, toks, experts=ov)
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    inc = np.stack([dec.step(t, expert_override=ov[i]) for i, t in enumerate(toks)])
    np.testing.assert_allclose(inc, want, rtol=1e-10, atol=1e-12)
    full = oracle.Decoder(cfg, W, dtype=np.float64).forward_full(toks, expert_overrides=np.array(ov))
    np.testing.assert_allclose(full, want, rtol=1e-10, atol=1e-12)
    # overriding with the router's own choice changes nothing
    plain = oracle.Decoder(cfg, W, dtype=np.float64)
    rows, own = [], []
    for t in toks:
        rows.append(plain.step(t))
        own.append([e.tolist() for e in plain.last_experts])
    again = oracle.Decoder(cfg, W, dtype=np.float64).forward_full(toks, expert_overrides=np.array(own))
    np.testing.assert_allclose(again, np.stack(rows), rtol=1e-10, atol=1e-12)
    assert not np.allclose(want, np.stack(rows))   # the overrides above do change the result


def test_decoder_causal_mask_ignores_future_cache():
    cfg = _tiny(decode_steps=10)
    W = make_weights(cfg)
    a = oracle.Decoder(cfg, W, dtype=np.float64)
    b = oracle.Decoder(cfg, W, dtype=np.float64)
    for t in (1, 2, 3):
        a.step(t)
        b.step(t)
    b.K[:, 4:] = 1e3
    b.V[:, 4:] = -1e3
    np.testing.assert_array_equal(a.step(5), b.step(5))


def test_decoder_zero_layers_is_lm_head_of_normed_embedding():
    cfg = _tiny(n_layers=0)
    W = make_weights(cfg)
    names = [n for n, _, _ in tensor_specs(cfg)]
    T = dict(zip(names, W))
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    e = T["E"][7].astype(np.float64)
    g = T["g_final"].astype(np.float64)
    want = T["W_lm"].astype(np.float64) @ (e / np.sqrt(np.mean(e * e) + cfg.rms_eps) * g)
    np.testing.assert_allclose(dec.step(7), want, rtol=1e-13)


def test_moe_all_experts_selected_is_dense_mixture():
    cfg = _tiny(n_experts=3, top_k=3, ffn_dim=6, n_layers=1)
    W = make_weights(cfg)
    names = [n for n, _, _ in tensor_specs(cfg)]
    T = {n: t.astype(np.float64) for n, t in zip(names, W)}
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    h = np.random.default_rng(11).standard_normal(cfg.d_model)
    y, sel = dec._ffn(0, h, None)
    pi = softmax(T["l0.Wr"] @ h)
    want = sum(pi[e] * swiglu_ffn(h, T[f"l0.e{e}.Wg"], T[f"l0.e{e}.Wu"], T[f"l0.e{e}.Wd"])
               for e in range(3))
    np.testing.assert_allclose(y, want, rtol=1e-12)
    assert sorted(sel.tolist()) == [0, 1, 2]


def test_moe_single_expert_is_dense_swiglu():
    cfg = _tiny(n_experts=1, top_k=1, ffn_dim=6, n_layers=1)
    W = make_weights(cfg)
    names = [n for n, _, _ in tensor_specs(cfg)]
    T = {n: t.astype(np.float64) for n, t in zip(names, W)}
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    h = np.random.default_rng(12).standard_normal(cfg.d_model)
    y, _ = dec._ffn(0, h, None)
    np.testing.assert_allclose(y, swiglu_ffn(h, T["l0.e0.Wg"], T["l0.e0.Wu"], T["l0.e0.Wd"]),
                               rtol=1e-13)


def test_moe_constant_router_picks_first_experts_with_uniform_weight():
    cfg = _tiny(n_experts=16, top_k=8, ffn_dim=6, n_layers=1)
    W = make_weights(cfg)
    names = [n for n, _, _ in tensor_specs(cfg)]
    W[names.index("l0.Wr")][:] = 0
    T = {n: t.astype(np.float64) for n, t in zip(names, W)}
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    h = np.random.default_rng(13).standard_normal(cfg.d_model)
    y, sel = dec._ffn(0, h, None)
    assert sel.tolist() == list(range(8))
    want = sum(swiglu_ffn(h, T[f"l0.e{e}.Wg"], T[f"l0.e{e}.Wu"], T[f"l0.e{e}.Wd"]) / 16
               for e in range(8))
    np.testing.assert_allclose(y, want, rtol=1e-12)


def test_prefill_and_decode_semantics():
    cfg = _tiny()
    W = make_weights(cfg)
    P = make_prompt(cfg)
    a = oracle.Decoder(cfg, W)
    first, last = a.prefill(P)
    assert first == int(np.argmax(last)) and a.pos == len(P)
    ids, rows, _ = a.decode(4, keep_logits=True)
    assert [int(np.argmax(r)) for r in rows] == ids.tolist()
    # teacher forcing with the free-run tokens reproduces the free run
    b = oracle.Decoder(cfg, W)
    b.prefill(P)
    ids2, rows2, _ = b.decode(4, force=ids.tolist(), keep_logits=True)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_array_equal(rows2, rows)


def test_set_kv_then_decode_matches_manual_cache():
    cfg = _tiny(kv_prefill=6, prompt_len=0, decode_steps=3)
    W = make_weights(cfg)
    rng = np.random.default_rng(14)
    K = rng.standard_normal((cfg.n_layers, 6, cfg.n_kv_heads, cfg.head_dim)).astype(np.float16)
    V = rng.standard_normal(K.shape).astype(np.float16)
    d = oracle.Decoder(cfg, W, dtype=np.float64)
    d.set_kv(K, V, 4)
    assert d.pos == 6 and d.pending == 4
    ids, rows, _ = d.decode(2, keep_logits=True)
    assert rows.shape == (2, cfg.vocab)
    np.testing.assert_array_equal(d.K[:, :6], K.astype(np.float64))


# ------------------------------------------------------------ compare ------

def test_compare_measures():
    ref = np.array([0.0, 1.0, 2.0, 3.0, 10.0])
    sd = ref.std()
    dev = ref.copy(); dev[2] += 0.5
    assert oracle.zscore_error(dev, ref) == pytest.approx(0.5 / sd)
    assert oracle.top2_gap(ref) == pytest.approx(7.0 / sd)
    worst, must, bad, n = oracle.compare_logits(dev[None], ref[None])
    assert (must, bad, n) == (1, 0, 1)


@pytest.mark.parametrize("bad_value", [np.nan, np.inf, -np.inf])
def test_compare_non_finite_device_rows_fail(bad_value):
    """A NaN or infinite device logit is an infinite error, also in a row whose
    top-2 gap is below the tolerance (no argmax check there) and when it sits
    after a finite row."""
    ref = np.array([[0.0, 1.0, 2.0, 3.0, 10.0], [0.0, 1.0, 2.0, 5.0, 5.0001]])
    assert oracle.top2_gap(ref[1]) <= 2e-2
    for row in (0, 1):
        dev = ref.copy()
        dev[row, 1] = bad_value
        assert oracle.zscore_error(dev[row], ref[row]) == float("inf")
        worst, must, bad, n = oracle.compare_logits(dev, ref)
        assert worst == float("inf") and not worst <= 2e-2
    dev = np.full_like(ref, np.nan)
    worst, _, _, _ = oracle.compare_logits(dev, ref)
    assert worst == float("inf")
    # a shape mismatch is no pass either
    assert oracle.compare_logits(ref[:, :4], ref)[0] == float("inf")


# ---------------------------------------------------------------- fp8 -------

def test_e4m3_table_closed_form_points():
    """E4M3 (OCP): largest finite 448 = 1.75 * 2^8, smallest normal 2^-6,
    smallest subnormal 2^-9, 1.0 at exponent field 7, no infinities, NaN at
    0x7f / 0xff, a sign bit."""
    t = oracle.e4m3_decode_table()
    assert t[0x7e] == 448.0 and t[0xfe] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x39] == 1.125 and t[0x40] == 2.0 and t[0xb8] == -1.0
    assert np.isnan(t[0x7f]) and np.isnan(t[0xff]) and np.isfinite(t[np.r_[0:0x7f, 0x80:0xff]]).all()
    assert t[0] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7f]
    assert np.all(np.diff(pos) > 0)                         # codes increase with value
    assert np.array_equal(t[0x80:0xff], -pos)


def test_e4m3_encode_round_trip_ties_and_saturation():
    t = oracle.e4m3_decode_table()
    finite = np.array([c for c in range(256) if np.isfinite(t[c])])
    assert np.array_equal(oracle.e4m3_encode(t[finite]), finite.astype(np.uint8))
    pos = t[:0x7f]
    mid = (pos[:-1] + pos[1:]) / 2                          # ties: to the even code
    want = np.where(np.arange(1, 0x7f) % 2 == 0, np.arange(1, 0x7f), np.arange(0, 0x7e))
    assert np.array_equal(oracle.e4m3_encode(mid), want.astype(np.uint8))
    eps = np.diff(pos) * 1e-3
    assert np.array_equal(oracle.e4m3_encode(mid - eps), np.arange(0, 0x7e).astype(np.uint8))
    assert np.array_equal(oracle.e4m3_encode(mid + eps), np.arange(1, 0x7f).astype(np.uint8))
    assert oracle.e4m3_encode(np.array([500.0, -1e9, 448.5]))[:2].tolist() == [0x7e, 0xfe]
    v = np.sort(np.random.default_rng(20).standard_normal(5000) * 100)
    assert np.all(np.diff(t[oracle.e4m3_encode(v)]) >= 0)   # monotone


def test_e4m3_encode_matches_torch_cast():
    """A library routine: torch's float32 -> float8_e4m3fn cast (nearest, ties
    to even) on values within the finite range."""
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    rng = np.random.default_rng(21)
    v = np.concatenate([rng.standard_normal(50000) * 60, rng.standard_normal(50000) * 1e-2,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), want)


def test_quantize_rows_e4m3_properties():
    rng = np.random.default_rng(22)
    W = (rng.standard_normal((6, 1024)) * 0.02).astype(np.float16)
    W[1] = 0                                                 # an all-zero row: scale 1, codes 0
    W[2] = 0
    W[2, 7] = np.float16(-0.5)                               # one non-zero: it is -448 * s
    g = (1 + rng.standard_normal(1024) * 0.2).astype(np.float16)
    q, s = oracle.quantize_rows_e4m3(W, g)
    assert s.dtype == np.float32 and q.dtype == np.uint8
    assert s[1] == 1.0 and not q[1].any()
    assert q[2, 7] == 0xfe and (q[2, :7] == 0).all()
    v = W.astype(np.float32) * g.astype(np.float32)
    for r in (0, 3, 4, 5):
        k = int(np.argmax(np.abs(v[r])))
        assert q[r, k] & 0x7f == 0x7e                       # the row's largest magnitude maps to 448
        assert s[r] == np.float32(np.abs(v[r]).max() / np.float32(448.0))
    # dequantised within half a code spacing of the exact value (the wider of
    # the two spacings next to the chosen code: 2^-4 relative for normals)
    deq = oracle.dequantize_rows_e4m3(q, s)
    t = oracle.e4m3_decode_table()
    c = (q & 0x7f).astype(np.int64)
    up = t[np.minimum(c, 0x7d) + 1] - t[np.minimum(c, 0x7d)]
    down = t[np.maximum(c, 1)] - t[np.maximum(c, 1) - 1]
    step = np.maximum(up, down) * s[:, None]
    assert np.all(np.abs(deq - v) <= step / 2 * (1 + 1e-6))
    assert np.abs(deq - v).max() > 0                        # it is a quantisation


def test_fp8_decoder_is_the_model_on_dequantised_weights():
    """An fp8 decoder equals the written-out definition with every projection
    replaced by its row-wise E4M3 quantisation (gain of the preceding RMSNorm
    folded in; norms without gain)."""
    cfg = _tiny(d_model=16, weight_format="fp8")
    W = make_weights(cfg)
    names = [n for n, _, _ in tensor_specs(cfg)]
    T = dict(zip(names, W))
    deq = []
    for n, t in zip(names, W):
        if n.split(".")[-1].startswith("g_"):
            deq.append(np.ones(t.shape))
        elif n == "E":
            deq.append(t.astype(np.float64))
        else:
            mat = n.split(".")[-1]
            g = {"Wq": "g_attn", "Wk": "g_attn", "Wv": "g_attn", "Wg": "g_ffn", "Wu": "g_ffn"}.get(mat)
            if n == "W_lm":
                g = T["g_final"]
            elif g is not None:
                g = T[n.split(".")[0] + "." + g]
            deq.append(oracle.dequantize_rows_e4m3(*oracle.quantize_rows_e4m3(t, g)))
    toks = [3, 17, 0, 22, 9]
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    got = np.stack([dec.step(t) for t in toks])
    np.testing.assert_allclose(got, _brute_logits(cfg, deq, toks), rtol=1e-10, atol=1e-12)
    # and it is not the fp16 model
    plain = oracle.Decoder(cfg.with_(weight_format="fp16"), W, dtype=np.float64)
    assert not np.allclose(got, np.stack([plain.step(t) for t in toks]))


# ---------------------------------------------------------------- fp4 -------
def test_e2m1_table_is_the_published_value_set():
    """E2M1 (the OCP microscaling element type): magnitudes 0, 0.5, 1, 1.5, 2,
    3, 4, 6 in code order, the same with the sign bit set; every value is also
    exactly an E4M3 value (the two tables come from different definitions)."""
    t = oracle.e2m1_decode_table()
    assert t[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(t[8:], -t[:8]) and np.signbit(t[8])
    e4 = oracle.e4m3_decode_table()
    assert np.array_equal(e4[oracle.e4m3_encode(t[:8])], t[:8])
    assert oracle.E2M1_MAX == t.max() == 6.0


def test_e2m1_encode_against_brute_force_nearest():
    t = oracle.e2m1_decode_table()[:8]
    rng = np.random.default_rng(41)
    v = np.concatenate([rng.uniform(-8, 8, 4000), (t[1:] + t[:-1]) / 2, -(t[1:] + t[:-1]) / 2,
                        t, -t, [7.0, -100.0, 6.0001]]).astype(np.float32)
    got = oracle.e2m1_encode(v)
    for x, c in zip(v.astype(np.float64), got):
        a = min(abs(x), 6.0)
        d = np.abs(t - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]   # ties to the even code
        if np.signbit(x):
            want |= 8
        assert c == want, (x, c, want)
    assert np.array_equal(oracle.e2m1_encode(t), np.arange(8))   # round trip


def test_quantize_rows_e2m1_properties():
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((6, 1024)) * 0.02).astype(np.float16)
    W[1] = 0                                                 # all-zero row: scale 1, codes 0
    W[2] = 0
    W[2, 5] = np.float16(-0.25)                              # one non-zero: it is -6 * s
    g = (1 + rng.standard_normal(1024) * 0.2).astype(np.float16)
    q, s = oracle.quantize_rows_e2m1(W, g)
    assert s.dtype == np.float32 and q.dtype == np.uint8 and q.max() < 16
    assert s[1] == 1.0 and not q[1].any()
    assert q[2, 5] == 15 and (q[2, :5] == 0).all()
    v = W.astype(np.float32) * g.astype(np.float32)
    for r in (0, 3, 4, 5):
        k = int(np.argmax(np.abs(v[r])))
        assert q[r, k] & 7 == 7                              # the row's largest magnitude maps to 6
        assert s[r] == np.float32(np.abs(v[r]).max() / np.float32(6.0))
    deq = oracle.dequantize_rows_e2m1(q, s)
    t = oracle.e2m1_decode_table()
    c = (q & 7).astype(np.int64)
    up = t[np.minimum(c, 6) + 1] - t[np.minimum(c, 6)]
    down = t[np.maximum(c, 1)] - t[np.maximum(c, 1) - 1]
    step = np.maximum(up, down) * s[:, None]
    assert np.all(np.abs(deq - v) <= step / 2 * (1 + 1e-6))


def test_fp4_decoder_is_the_model_on_dequantised_weights():
    """An fp4 decoder equals the written-out definition with every projection
    replaced by its row-wise E2M1 quantisation (gain folded in)."""
    cfg = _tiny(d_model=16, weight_format="fp4")
    W = make_weights(cfg)
    names = [n for n, _, _ in tensor_specs(cfg)]
    T = dict(zip(names, W))
    deq = []
    for n, t in zip(names, W):
        if n.split(".")[-1].startswith("g_"):
            deq.append(np.ones(t.shape))
        elif n == "E":
            deq.append(t.astype(np.float64))
        else:
            mat = n.split(".")[-1]
            g = {"Wq": "g_attn", "Wk": "g_attn", "Wv": "g_attn", "Wg": "g_ffn", "Wu": "g_ffn"}.get(mat)
            if n == "W_lm":
                g = T["g_final"]
            elif g is not None:
                g = T[n.split(".")[0] + "." + g]
            deq.append(oracle.dequantize_rows_e2m1(*oracle.quantize_rows_e2m1(t, g)))
    toks = [3, 17, 0, 22, 9]
    dec = oracle.Decoder(cfg, W, dtype=np.float64)
    got = np.stack([dec.step(t) for t in toks])
    np.testing.assert_allclose(got, _brute_logits(cfg, deq, toks), rtol=1e-10, atol=1e-12)
    fp8 = oracle.Decoder(cfg.with_(weight_format="fp8"), W, dtype=np.float64)
    assert not np.allclose(got, np.stack([fp8.step(t) for t in toks]))
