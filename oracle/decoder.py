"""CPU oracle for single-request (batch-1) greedy transformer decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
do. It shares no code with the device path; the two meet only in the seeded
inputs of the ``synth`` package.

What it computes follows the pages' statement of the problem:

* agentlenshq.com article, "The memory-bandwidth bottleneck": each generated
  token needs every active weight once; decode is batch 1.
* paper-digest.app digest, "Core Mechanics": batch-1 decode of one request,
  speed bounded by bandwidth / (active weight bytes + KV cache bytes).
* news.creeta.com monokernel article, "Inside the monokernel": RMSNorm,
  Q/K/V projections, rotary position embedding, attention over the cached
  keys and values, and on-device greedy token sampling.

The pages name the method's ingredients but not the block structure. The
plainest reading, used here and listed with every other reading in the
design notes, is a pre-norm residual decoder without biases::

    x = E[t]
    per layer:  h = rmsnorm(x) * g_attn
                q, k, v = Wq h, Wk h, Wv h;  rotate q, k by position p
                append k, v to the cache;  o = causal GQA attention
                x = x + Wo o
                h = rmsnorm(x) * g_ffn
                x = x + Wd (silu(Wg h) * Wu h)      (MoE: sum over top-k experts)
    logits = W_lm (rmsnorm(x) * g_final);  next token = argmax(logits)

Arithmetic is float32 on the fp16 weights (fp16 -> fp32 is exact) unless a
caller asks for float64; rotary angles are formed in float64.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Building blocks. Each is the plain definition, written out.
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (eps inside the root).

    Folded into the next projection on the device ("Inside the monokernel",
    RMSNorm folding); here it is a separate step.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + x.dtype.type(eps))) * g.astype(x.dtype)


def rope_angles(positions: Sequence[int] | np.ndarray, head_dim: int,
                theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of p * theta^(-2i/head_dim), i < head_dim/2, in float64.

    Rotary embedding is precomputed rather than recomputed per step on the
    device ("Inside the monokernel", RoPE precompute); the oracle forms the
    same angles directly. Shapes: [len(positions), head_dim/2].
    """
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half rotary embedding on the last axis.

    Element i is paired with element i + head_dim/2:
    (a, b) -> (a cos - b sin, b cos + a sin). ``cos``/``sin`` broadcast against
    v[..., :head_dim/2].
    """
    half = v.shape[-1] // 2
    a, b = v[..., :half], v[..., half:]
    c = cos.astype(v.dtype)
    s = sin.astype(v.dtype)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum(exp(s - max s)) over the last axis."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of one query position over c cached positions.

    q: [H, hd]; K, V: [c, Hkv, hd] (positions 0..p, the current one included).
    Query head j reads kv head j // (H / Hkv). Scores are scaled by 1/sqrt(hd).
    Returns o: [H, hd].
    """
    H, hd = q.shape
    Hkv = K.shape[1]
    group = H // Hkv
    scale = q.dtype.type(1.0 / np.sqrt(hd))
    o = np.empty_like(q)
    for j in range(H):
        g = j // group
        s = (K[:, g, :] @ q[j]) * scale
        p = softmax(s)
        o[j] = p @ V[:, g, :]
    return o


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (z.dtype.type(1.0) + np.exp(-z))


def swiglu_ffn(h: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """Wd (silu(Wg h) * (Wu h))."""
    return Wd @ (silu(Wg @ h) * (Wu @ h))


def topk_experts(probs: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest router probabilities, ties to the lower index."""
    order = np.argsort(-probs, kind="stable")
    return order[:k]


def greedy_argmax(logits: np.ndarray) -> int:
    """Greedy sampling: the index of the largest logit, ties to the lowest index."""
    return int(np.argmax(logits))


def gemv_f64(A: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = A x in float64 (the probe's reference: fp16 inputs are exact in f64)."""
    return A.astype(np.float64) @ x.astype(np.float64)


# --------------------------------------------------------------------------
# FP8 weights. The pages name FP8/FP4 quantisation as the way to fewer bytes
# per token (agentlenshq.com article, "Scaling to frontier MoE models") without
# fixing a format; the one used here is the OCP 8-bit float E4M3 with one
# scale per weight row, the scale mapping the row's largest magnitude to
# E4M3's largest finite value.
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes, from the format's
    definition: sign bit, 4 exponent bits e (bias 7), 3 mantissa bits m;
    e = 0 is subnormal, m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7); e = 15 with
    m = 7 is NaN (no infinities)."""
    codes = np.arange(256)
    e = (codes >> 3) & 15
    m = (codes & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(codes & 0x80, -mag, mag)


def _e4m3_encode_block(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    a = np.minimum(np.abs(v), table.dtype.type(E4M3_MAX))
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, 0x7e)   # first table value >= a
    lo = hi - 1
    # exact differences: a lies between two neighbouring table values
    dlo, dhi = a - table[lo], table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == 0, 0, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7f), code).astype(np.uint8)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """The E4M3 code nearest to each value (ties to the even code), saturating
    at +-448; NaN maps to 0x7f. Found among the sorted table of the 127
    non-negative finite codes, not by arithmetic on exponent and mantissa.
    float32 input is encoded in float32 (every table value and every
    difference to a neighbouring table value is exact there), in blocks."""
    v = np.asarray(v)
    if v.dtype != np.float32:
        v = v.astype(np.float64)
    table = e4m3_decode_table()[:0x7f].astype(v.dtype)   # codes 0x00..0x7e, increasing
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 18
    for i in range(0, flat.size, step):
        out[i:i + step] = _e4m3_encode_block(flat[i:i + step], table)
    return out.reshape(v.shape)


def quantize_rows_e4m3(W: np.ndarray, gain: Optional[np.ndarray] = None):
    """Row-wise E4M3 quantisation of fp16 weights W [rows][K], each column k
    first multiplied by gain[k] (an RMSNorm gain folded into the matrix).
    In float32, as specified: v = w * g (exact for fp16 operands),
    s = max|v| / 448 per row (1 for an all-zero row), q = E4M3(v / s).
    Returns (q uint8 [rows][K], s float32 [rows])."""
    v = np.asarray(W, dtype=np.float16).astype(np.float32)
    if gain is not None:
        v = v * np.asarray(gain, dtype=np.float16).astype(np.float32)[None, :]
    amax = np.max(np.abs(v), axis=1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = e4m3_encode((v / s[:, None]).astype(np.float32))
    return q, s


def dequantize_rows_e4m3(q: np.ndarray, s: np.ndarray, dtype=np.float64) -> np.ndarray:
    """q [rows][K] codes and s [rows] scales -> the weights they stand for."""
    return (e4m3_decode_table()[q] * np.asarray(s, dtype=np.float64)[:, None]).astype(dtype)


# --------------------------------------------------------------------------
# FP4 weights: the OCP 4-bit float E2M1 (the element type of the OCP
# microscaling formats) with, as for FP8 here, one fp32 scale per weight row
# mapping the row's largest magnitude to E2M1's largest value, 6.
# --------------------------------------------------------------------------

E2M1_MAX = 6.0


def e2m1_decode_table() -> np.ndarray:
    """float64 value of each of the 16 E2M1 codes, from the format's
    definition: sign bit 3, 2 exponent bits e (bias 1), 1 mantissa bit m;
    e = 0 is subnormal, m/2; otherwise (1 + m/2) * 2^(e-1). The magnitudes are
    0, 0.5, 1, 1.5, 2, 3, 4, 6; there is no infinity or NaN."""
    codes = np.arange(16)
    e = (codes >> 1) & 3
    m = (codes & 1).astype(np.float64)
    mag = np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * 2.0 ** (e - 1.0))
    return np.where(codes & 8, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """The E2M1 code nearest to each value (ties to the even code), saturating
    at +-6; the sign bit follows the input's (a negative value that rounds to
    zero gives code 8). Found among the 8 non-negative table values; every
    table value and every difference to a neighbour is exact in float32."""
    v = np.asarray(v)
    if v.dtype != np.float32:
        v = v.astype(np.float64)
    table = e2m1_decode_table()[:8].astype(v.dtype)   # codes 0..7, increasing
    a = np.minimum(np.abs(v), v.dtype.type(E2M1_MAX))
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, 7)
    lo = hi - 1
    dlo, dhi = a - table[lo], table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == 0, 0, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where(np.signbit(v), code | 8, code).astype(np.uint8)


def quantize_rows_e2m1(W: np.ndarray, gain: Optional[np.ndarray] = None):
    """Row-wise E2M1 quantisation of fp16 weights W [rows][K], each column k
    first multiplied by gain[k]. In float32: v = w * g, s = max|v| / 6 per row
    (1 for an all-zero row), q = E2M1(v / s). Returns (q uint8 codes 0..15
    [rows][K], s float32 [rows])."""
    v = np.asarray(W, dtype=np.float16).astype(np.float32)
    if gain is not None:
        v = v * np.asarray(gain, dtype=np.float16).astype(np.float32)[None, :]
    amax = np.max(np.abs(v), axis=1)
    s = np.where(amax > 0, amax / np.float32(E2M1_MAX), np.float32(1.0)).astype(np.float32)
    q = e2m1_encode((v / s[:, None]).astype(np.float32))
    return q, s


def dequantize_rows_e2m1(q: np.ndarray, s: np.ndarray, dtype=np.float64) -> np.ndarray:
    """q [rows][K] codes and s [rows] scales -> the weights they stand for."""
    return (e2m1_decode_table()[q] * np.asarray(s, dtype=np.float64)[:, None]).astype(dtype)


# --------------------------------------------------------------------------
# The decoder.
# --------------------------------------------------------------------------

class Decoder:
    """Incremental batch-1 decoder with a KV cache, plus a full causal forward.

    ``tensors`` is the canonical list from ``synth.make_weights``. State is a
    position ``pos`` and a ``pending`` token, so that ``prefill``/``decode``
    have the same meaning as the device library's calls:

    * ``prefill(prompt)`` runs one pass per prompt token at positions
      0..P-1 and returns the first generated token.
    * ``decode(n, force)`` runs exactly n passes. Pass i feeds the pending
      token at the current position and records argmax(logits) as output i;
      the next pending token is that output, or ``force[i]`` when teacher
      forcing.
    """

    def __init__(self, cfg, tensors: List[np.ndarray], dtype=np.float32,
                 cache_experts: bool = False, kv_dtype=np.float16):
        self.cfg = cfg
        self.dtype = np.dtype(dtype)
        # fp8 / fp4 weights: every projection is the row-wise E4M3 / E2M1
        # quantisation of the matrix with its preceding RMSNorm gain folded
        # in, and the norms themselves then carry no gain (the embedding
        # stays fp16)
        self.wfmt = getattr(cfg, "weight_format", "fp16")
        self.fp8 = self.wfmt in ("fp8", "fp4")   # a quantised model (either format)
        # The KV cache holds fp16 keys and values: each k, v is rounded to
        # fp16 when it is stored and read back exactly. kv_dtype=None keeps
        # the compute precision instead.
        self.kv_dtype = self.dtype if kv_dtype is None else np.dtype(kv_dtype)
        self._raw = tensors
        self._cache_experts = cache_experts
        self._conv: Dict[int, np.ndarray] = {}
        self._index = self._build_index()
        if self.fp8:
            # quantise every projection once, matrices in parallel (the
            # element-wise work releases the interpreter lock); MoE experts
            # only when they are cached anyway
            from concurrent.futures import ThreadPoolExecutor
            import os
            names = [n for n in self._index if n != "E" and not n.split(".")[-1].startswith("g_")
                     and (cache_experts or ".e" not in n)]
            with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
                list(ex.map(self.w, names))
        L, S, Hkv, hd = cfg.n_layers, cfg.max_seq, cfg.n_kv_heads, cfg.head_dim
        self.K = np.zeros((L, S, Hkv, hd), dtype=self.kv_dtype)
        self.V = np.zeros((L, S, Hkv, hd), dtype=self.kv_dtype)
        self.pos = 0
        self.pending: Optional[int] = None
        self.last_experts: List[np.ndarray] = []
        self.last_router: List[np.ndarray] = []   # MoE: router logits per layer of the last pass
        self.full_router: List[np.ndarray] = []   # MoE: per layer [T, E], of the last full forward

    # ---- weights ---------------------------------------------------------
    def _build_index(self) -> Dict[str, int]:
        from synth import tensor_specs  # shapes and order only, no arithmetic
        specs = tensor_specs(self.cfg)
        if len(specs) != len(self._raw):
            raise ValueError("tensor list does not match the configuration")
        for (name, shape, _), t in zip(specs, self._raw):
            if tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name}: shape {t.shape} != {shape}")
        return {name: i for i, (name, _, _) in enumerate(specs)}

    # the RMSNorm gain folded into each projection of a quantised model
    _FOLD = {"Wq": "g_attn", "Wk": "g_attn", "Wv": "g_attn", "Wg": "g_ffn", "Wu": "g_ffn", "Wo": None,
             "Wd": None, "Wr": "g_ffn"}

    def w(self, name: str) -> np.ndarray:
        i = self._index[name]
        hit = self._conv.get(i)
        if hit is not None:
            return hit
        if self.fp8 and name.split(".")[-1].startswith("g_"):   # gains live in the fp8 matrices
            a = np.ones(self._raw[i].shape, dtype=self.dtype)
        elif self.fp8 and name != "E":
            if name == "W_lm":
                g = self._raw[self._index["g_final"]]
            else:
                layer, mat = name.split(".")[0], name.split(".")[-1]
                gname = self._FOLD[mat]
                g = None if gname is None else self._raw[self._index[f"{layer}.{gname}"]]
            if self.wfmt == "fp4":
                q, s = quantize_rows_e2m1(self._raw[i], g)
                a = dequantize_rows_e2m1(q, s, self.dtype)
            else:
                q, s = quantize_rows_e4m3(self._raw[i], g)
                a = dequantize_rows_e4m3(q, s, self.dtype)
        else:
            a = self._raw[i].astype(self.dtype)
        if self._cache_experts or ".e" not in name:
            self._conv[i] = a
        return a

    # ---- state -----------------------------------------------------------
    def reset(self) -> None:
        self.K[:] = 0
        self.V[:] = 0
        self.pos = 0
        self.pending = None

    def set_kv(self, K: np.ndarray, V: np.ndarray, pending_token: int) -> None:
        """Store already-rotated keys and values at positions 0..n-1."""
        n = K.shape[1]
        self.K[:, :n] = K.astype(self.kv_dtype)
        self.V[:, :n] = V.astype(self.kv_dtype)
        self.K[:, n:] = 0
        self.V[:, n:] = 0
        self.pos = n
        self.pending = int(pending_token)

    def _moe_rows(self, l: int, Hn: np.ndarray, override: Optional[np.ndarray] = None) -> np.ndarray:
        """The MoE FFN of every row of Hn: row t gets sum over its top-k experts
        e of pi_te * FFN_e(h_t), with pi_t the softmax of its router logits.
        ``override`` [T, k], if given, replaces row t's top-k set (the same
        probabilities pi_t weigh it). Rows are grouped by expert so each
        expert's matrices are read once."""
        cfg = self.cfg
        logits = Hn @ self.w(f"l{l}.Wr").T                            # [T, E]
        self.full_router.append(logits)
        probs = softmax(logits)
        if override is None:
            sel = np.stack([topk_experts(p, cfg.top_k) for p in probs])   # [T, k]
        else:
            sel = np.asarray(override, dtype=np.int64).reshape(len(Hn), -1)
        Y = np.zeros_like(Hn)
        for e in range(cfg.n_experts):
            rows = np.nonzero((sel == e).any(axis=1))[0]
            if rows.size == 0:
                continue
            Hs = Hn[rows]
            G = Hs @ self.w(f"l{l}.e{e}.Wg").T
            U = Hs @ self.w(f"l{l}.e{e}.Wu").T
            Y[rows] += probs[rows, e:e + 1] * ((silu(G) * U) @ self.w(f"l{l}.e{e}.Wd").T)
        return Y

    # ---- one pass ----------------------------------------------------------
    def _ffn(self, l: int, h: np.ndarray,
             override: Optional[np.ndarray]) -> Tuple[np.ndarray, Optional[np.ndarray]]:
        cfg = self.cfg
        if not cfg.n_experts:
            return swiglu_ffn(h, self.w(f"l{l}.Wg"), self.w(f"l{l}.Wu"), self.w(f"l{l}.Wd")), None
        logits = self.w(f"l{l}.Wr") @ h
        self.last_router.append(logits)
        probs = softmax(logits)
        sel = topk_experts(probs, cfg.top_k) if override is None else np.asarray(override)
        out = np.zeros(cfg.d_model, dtype=self.dtype)
        for e in sel:
            e = int(e)
            y = swiglu_ffn(h, self.w(f"l{l}.e{e}.Wg"), self.w(f"l{l}.e{e}.Wu"),
                           self.w(f"l{l}.e{e}.Wd"))
            out = out + probs[e] * y
        return out, sel

    def step(self, token: int,
             expert_override: Optional[Sequence[Optional[Sequence[int]]]] = None) -> np.ndarray:
        """One forward pass of ``token`` at position ``pos``; returns logits."""
        cfg, dt = self.cfg, self.dtype
        p = self.pos
        if p >= cfg.max_seq:
            raise ValueError("KV cache full")
        H, Hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
        cos, sin = rope_angles([p], hd, cfg.rope_theta)
        x = self.w("E")[token].copy()
        experts = []
        self.last_router = []
        for l in range(cfg.n_layers):
            h = rmsnorm(x, self.w(f"l{l}.g_attn"), cfg.rms_eps)
            q = (self.w(f"l{l}.Wq") @ h).reshape(H, hd)
            k = (self.w(f"l{l}.Wk") @ h).reshape(Hkv, hd)
            v = (self.w(f"l{l}.Wv") @ h).reshape(Hkv, hd)
            q = apply_rope(q, cos, sin)
            k = apply_rope(k, cos, sin)
            self.K[l, p] = k
            self.V[l, p] = v
            o = attention_decode(q, self.K[l, :p + 1].astype(dt), self.V[l, :p + 1].astype(dt))
            x = x + self.w(f"l{l}.Wo") @ o.reshape(-1)
            h = rmsnorm(x, self.w(f"l{l}.g_ffn"), cfg.rms_eps)
            ov = None if expert_override is None else expert_override[l]
            y, sel = self._ffn(l, h, ov)
            if sel is not None:
                experts.append(np.asarray(sel, dtype=np.int32))
            x = x + y
        self.last_experts = experts
        self.pos = p + 1
        return self.w("W_lm") @ rmsnorm(x, self.w("g_final"), cfg.rms_eps)

    # ---- request-level calls ----------------------------------------------
    def prefill(self, prompt: Sequence[int]):
        """Passes at positions 0..P-1; returns (first token, last logits)."""
        self.reset()
        logits = None
        for t in prompt:
            logits = self.step(int(t))
        first = greedy_argmax(logits)
        self.pending = first
        return first, logits

    def prefill_batched(self, prompt: Sequence[int], expert_overrides=None):
        """Same result as ``prefill`` (up to rounding order), computed with one
        causal forward over the whole prompt; returns (first token, last logits).
        ``expert_overrides`` as in ``forward_full``."""
        self.reset()
        logits = self.forward_full(list(prompt), store_kv=True, expert_overrides=expert_overrides)[-1]
        self.pos = len(prompt)
        first = greedy_argmax(logits)
        self.pending = first
        return first, logits

    def decode(self, n: int, force: Optional[Sequence[int]] = None,
               keep_logits: bool = False, expert_overrides=None):
        """n passes; returns (ids, logits rows or None, experts per pass)."""
        if self.pending is None:
            raise ValueError("no pending token: call prefill or set_kv first")
        ids, rows, exps = [], [], []
        for i in range(n):
            ov = None if expert_overrides is None else expert_overrides[i]
            logits = self.step(self.pending, ov)
            nxt = greedy_argmax(logits)
            ids.append(nxt)
            exps.append(self.last_experts)
            if keep_logits:
                rows.append(logits)
            self.pending = int(force[i]) if force is not None else nxt
        return np.asarray(ids, dtype=np.int32), (np.stack(rows) if keep_logits else None), exps

    # ---- non-incremental reference ----------------------------------------
    def forward_full(self, tokens: Sequence[int], store_kv: bool = False,
                     expert_overrides: Optional[np.ndarray] = None) -> np.ndarray:
        """Logits at every position of ``tokens`` by a full causal recompute.

        All positions are projected at once and attention applies an explicit
        causal mask; the incremental path is checked against it. With
        ``store_kv`` the rotated keys and the values of positions 0..T-1 are
        also written to the cache (a batched prefill). MoE:
        ``expert_overrides`` [T][n_layers][top_k], if given, is the expert set
        of every (position, layer), used instead of the router's own top-k.
        """
        cfg, dt = self.cfg, self.dtype
        T = len(tokens)
        H, Hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
        group = H // Hkv
        cos, sin = rope_angles(np.arange(T), hd, cfg.rope_theta)   # [T, hd/2]
        X = self.w("E")[np.asarray(tokens)].astype(dt)              # [T, d]
        mask = np.triu(np.ones((T, T), dtype=bool), k=1)            # True above diagonal
        self.full_router = []   # MoE: router logits [T, E] per layer
        for l in range(cfg.n_layers):
            Hn = rmsnorm(X, self.w(f"l{l}.g_attn"), cfg.rms_eps)
            Q = (Hn @ self.w(f"l{l}.Wq").T).reshape(T, H, hd)
            Kf = (Hn @ self.w(f"l{l}.Wk").T).reshape(T, Hkv, hd)
            Vf = (Hn @ self.w(f"l{l}.Wv").T).reshape(T, Hkv, hd)
            Q = apply_rope(Q, cos[:, None, :], sin[:, None, :])
            Kf = apply_rope(Kf, cos[:, None, :], sin[:, None, :])
            Kf = Kf.astype(self.kv_dtype).astype(dt)   # attention reads what the cache holds
            Vf = Vf.astype(self.kv_dtype).astype(dt)
            if store_kv:
                self.K[l, :T] = Kf
                self.V[l, :T] = Vf
            O = np.empty((T, H, hd), dtype=dt)
            for j in range(H):
                g = j // group
                S = (Q[:, j, :] @ Kf[:, g, :].T) / dt.type(np.sqrt(hd))   # [T, T]
                S = np.where(mask, -np.inf, S)
                O[:, j, :] = softmax(S) @ Vf[:, g, :]
            X = X + O.reshape(T, H * hd) @ self.w(f"l{l}.Wo").T
            Hn = rmsnorm(X, self.w(f"l{l}.g_ffn"), cfg.rms_eps)
            if cfg.n_experts:
                ov = None if expert_overrides is None else np.asarray(expert_overrides)[:, l]
                Y = self._moe_rows(l, Hn, ov)
            else:
                G = Hn @ self.w(f"l{l}.Wg").T
                U = Hn @ self.w(f"l{l}.Wu").T
                Y = (silu(G) * U) @ self.w(f"l{l}.Wd").T
            X = X + Y
        return rmsnorm(X, self.w("g_final"), cfg.rms_eps) @ self.w("W_lm").T

