"""Shared helpers for the GPU parity tests (imported by tests, not collected)."""
import sys

import numpy as np

import oracle

TOL = 2e-2   # z-scored logits error and top-2 gap threshold


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_rows(dev, ref, tol=TOL, label=""):
    """Element-wise parity of logits rows: max z-scored error <= tol and the
    argmax equal wherever the oracle's top-2 gap exceeds tol."""
    worst, must, bad, n = oracle.compare_logits(dev, ref, tol)
    say(f"[{label}] rows={n} max_zerr={worst:.3e} argmax_checked={must} argmax_bad={bad}")
    assert worst <= tol, f"{label}: z-scored logits error {worst:.3e} > {tol}"
    assert bad == 0, f"{label}: {bad} argmax mismatches above the gap threshold"
    return worst


def gemv_bound(A, x):
    """Error bound of an fp32-accumulated dot product of length K:
    |err_i| <= K * 2^-23 * sum_k |a_ik x_k| (fp16 x fp16 products are exact in fp32)."""
    K = A.shape[-1]
    return K * 2.0 ** -23 * (np.abs(A.astype(np.float64)) @ np.abs(x.astype(np.float64))) + 1e-30


ROUTE_TOL = 2e-2   # z-scored router-logit margin below which either expert is a valid choice


def routing_agrees(dev_sel, router_logits, k, tol=ROUTE_TOL, label=""):
    """Check one pass's device routing against the oracle's router logits.

    dev_sel [L][k]: experts the device chose; router_logits [L][E]: oracle.
    Every layer's choice must be a valid top-k: k distinct in-range experts,
    none of them below an unchosen one by more than tol (in units of the
    layer's logit spread). Returns True when every layer chose exactly the
    oracle's top-k set, False when some layer differs only inside a near tie;
    the layers after such a layer are not checked, since from there on the two
    sides legitimately compute from different states.
    """
    same = True
    for l, (sel, r) in enumerate(zip(dev_sel, router_logits)):
        r = np.asarray(r, dtype=np.float64)
        sel = np.asarray(sel, dtype=np.int64)
        assert sel.min() >= 0 and sel.max() < len(r), f"{label} layer {l}: expert out of range {sel}"
        assert len(set(sel.tolist())) == k, f"{label} layer {l}: repeated expert {sel}"
        rest = np.setdiff1d(np.arange(len(r)), sel)
        sd = r.std()
        if rest.size:
            worst = (r[rest].max() - r[sel].min()) / sd
            assert worst <= tol, f"{label} layer {l}: experts {sel} are not a top-{k} (margin {worst:.3e})"
        want = set(oracle.topk_experts(oracle.softmax(r), k).tolist())
        if set(sel.tolist()) != want:
            say(f"[{label}] layer {l}: near tie, device {sorted(sel.tolist())} vs oracle {sorted(want)}, "
                f"margin {worst:.2e}")
            return False
    return same


def moe_request_parity(m, cfg, W, P, n, trials, label):
    """MoE parity of one device model `m` (freshly loaded) against the oracle.

    1. The prompt: every pass's routing must be a valid top-k of the oracle's
       router logits; the last logits are compared when no pass hit a near tie.
    2. Trials from a seeded cache of len(P) positions that both sides store
       exactly: trial t feeds forced token t, then t+1 (two passes in one
       launch); logits are compared element by element up to the first near
       tie in routing.
    3. The request: n teacher-forced passes as ONE launch; the same passes
       split over debug launches must give the same ids bit for bit, each id
       must be the argmax of its own logits row and every pass's routing a
       valid top-k; the leading passes are compared with the oracle until the
       first near tie.
    Returns the number of passes compared with the oracle in steps 2 and 3.
    """
    import synth
    ref = oracle.Decoder(cfg, W)
    say(f"{label}: oracle batched prefill of {len(P)} tokens")
    first, last = ref.prefill_batched(P)
    routes = ref.full_router
    g_first, g_logits, g_exp = m.prefill(P, logits=True, experts=True)
    same = [routing_agrees(g_exp[i], [r[i] for r in routes], cfg.top_k, label=f"{label} prompt {i}")
            for i in range(len(P))]
    if all(same):
        check_rows(g_logits[-1:], last[None], label=f"{label} prefill")
        if oracle.top2_gap(last) > TOL:
            assert g_first == first
    else:
        say(f"{label}: near tie in the prompt's routing; its last logits are not compared")
    del ref
    K, V = synth.make_kv_prefill(cfg, n_pos=len(P))
    F = synth.make_forced_tokens(cfg, n + 1)
    dec = oracle.Decoder(cfg, W, cache_experts=True)
    compared = 0

    def follow(dev_rows, dev_exp, tokens, tag):
        nonlocal compared
        for i, tok in enumerate(tokens):
            row = dec.step(int(tok))
            if not routing_agrees(dev_exp[i], dec.last_router, cfg.top_k, label=f"{tag} pass {i}"):
                return
            check_rows(dev_rows[i:i + 1], row[None], label=f"{tag} pass {i}")
            compared += 1

    for t in range(trials):
        dec.set_kv(K, V, int(F[t]))
        m.set_kv(K, V, int(F[t]))
        _, rows, exp = m.decode(2, force=F[t + 1:t + 3], logits=True, experts=True)
        follow(rows, exp, F[t:t + 2], f"{label} trial {t}")
    say(f"{label}: one teacher-forced launch of {n} passes, then the same passes with debug output")
    m.set_kv(K, V, int(F[0]))
    g_ids, _, _ = m.decode(n, force=F[1:])
    m.rewind(len(P), int(F[0]))
    c_ids, c_rows, c_exp = m.decode(n, force=F[1:], logits=True, experts=True)
    assert np.array_equal(g_ids, c_ids)
    assert np.array_equal(c_ids, np.argmax(c_rows, axis=1))
    for i in range(n):
        for l in range(cfg.n_layers):
            sel = c_exp[i, l]
            assert sel.min() >= 0 and sel.max() < cfg.n_experts and len(set(sel.tolist())) == cfg.top_k
    dec.set_kv(K, V, int(F[0]))
    follow(c_rows, c_exp, F[:min(n, 16)], f"{label} request")
    say(f"{label}: {compared} passes compared with the oracle")
    return compared
