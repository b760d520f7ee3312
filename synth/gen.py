"""Seeded generators for decoder weights, prompts, pre-filled KV and probe inputs.

Every tensor draws from its own NumPy PCG64 stream, seeded with
``[seed, stream_id]``; the stream ids are fixed below, so a tensor's bytes do
not depend on which other tensors were generated or in what order. Normal
values are drawn in float32, scaled, then rounded to fp16 (round to nearest
even).

Stream ids: tensor i of the canonical order -> i; prompt -> 1000; pre-filled
K/V of layer l -> (2000, l, 0|1); first pending token after a pre-filled
cache -> 3000; GEMV probe shape s -> (4000 + s, 0) for the matrix and
(4000 + s, 1) for the vector; teacher-forcing token stream -> 5000.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Tuple

import numpy as np

from .configs import DecoderConfig, tensor_specs

PROMPT_STREAM = 1000
KV_STREAM = 2000
PENDING_STREAM = 3000
PROBE_STREAM = 4000
FORCE_STREAM = 5000


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_fp16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(sigma)
    return a.astype(np.float16)


def _one_tensor(cfg: DecoderConfig, tid: int, shape, kind: str) -> np.ndarray:
    rng = np.random.default_rng([cfg.seed, tid])
    if kind == "gain":
        if cfg.gain_sigma == 0.0:
            return np.ones(shape, dtype=np.float16)
        a = rng.standard_normal(shape, dtype=np.float32) * np.float32(cfg.gain_sigma)
        return (a + np.float32(1.0)).astype(np.float16)
    sigma = cfg.router_sigma if kind == "router" else cfg.weight_sigma
    return _normal_fp16(rng, shape, sigma)


def make_weights(cfg: DecoderConfig) -> List[np.ndarray]:
    """All decoder tensors, fp16, in the canonical order of ``tensor_specs``."""
    specs = tensor_specs(cfg)
    with ThreadPoolExecutor(_workers()) as ex:
        futs = [ex.submit(_one_tensor, cfg, i, shape, kind)
                for i, (_, shape, kind) in enumerate(specs)]
        return [f.result() for f in futs]


def make_prompt(cfg: DecoderConfig) -> np.ndarray:
    """prompt_len token ids, uniform over the vocabulary, int32."""
    rng = np.random.default_rng([cfg.seed, PROMPT_STREAM])
    return rng.integers(0, cfg.vocab, size=cfg.prompt_len, dtype=np.int64).astype(np.int32)


def make_pending_token(cfg: DecoderConfig) -> int:
    """The first decode input after a pre-filled KV cache (uniform over the vocab)."""
    rng = np.random.default_rng([cfg.seed, PENDING_STREAM])
    return int(rng.integers(0, cfg.vocab))


def make_forced_tokens(cfg: DecoderConfig, n: int) -> np.ndarray:
    """n token ids, uniform over the vocabulary, int32: inputs for teacher-forced
    decoding (pass i+1 is fed token i whatever pass i produced)."""
    rng = np.random.default_rng([cfg.seed, FORCE_STREAM])
    return rng.integers(0, cfg.vocab, size=n, dtype=np.int64).astype(np.int32)


def make_kv_prefill(cfg: DecoderConfig, n_pos: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Seeded N(0,1) fp16 keys and values, shape [L][n_pos][n_kv_heads][head_dim].

    They are taken as the already-rotated keys and the values stored at
    positions 0..n_pos-1. The first n positions of a longer draw equal a
    shorter draw, so a test can take a prefix.
    """
    n_pos = cfg.kv_prefill if n_pos is None else n_pos
    shape = (n_pos, cfg.n_kv_heads, cfg.head_dim)
    K = np.empty((cfg.n_layers,) + shape, dtype=np.float16)
    V = np.empty_like(K)

    def fill(l: int) -> None:
        for which, dst in ((0, K), (1, V)):
            rng = np.random.default_rng([cfg.seed, KV_STREAM, l, which])
            dst[l] = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(cfg.n_layers)))
    return K, V


def make_probe(shape_index: int, M: int, K: int, sigma: float = 0.02,
               seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """GEMV probe inputs: A fp16 [M][K] ~ N(0, sigma), x fp16 [K] ~ N(0, 1)."""
    ra = np.random.default_rng([seed, PROBE_STREAM + shape_index, 0])
    rx = np.random.default_rng([seed, PROBE_STREAM + shape_index, 1])
    return _normal_fp16(ra, (M, K), sigma), _normal_fp16(rx, (K,), 1.0)


def weights_sha256(tensors: List[np.ndarray]) -> List[str]:
    return [hashlib.sha256(np.ascontiguousarray(t).tobytes()).hexdigest() for t in tensors]
