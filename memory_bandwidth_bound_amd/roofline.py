"""Byte counts and bandwidth arithmetic for batch-1 decode.

The pages measure decode by memory-bandwidth utilisation, not FLOP
utilisation: at batch 1 every active weight byte crosses HBM once per token
and the ceiling is bandwidth / (active weight bytes + KV bytes)
(paper-digest.app digest, "Core Mechanics"; axbrief.com article, section on
removing the framework by low-level co-design). The launch-tax arithmetic is
the one on the news.creeta.com monokernel article, "Kernel-launch tax".

Pure Python: no device code, no oracle.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12      # MI355X HBM3E, published peak


def active_weight_bytes(cfg) -> int:
    """Bytes of weights read for one token.

    Every layer projection (Q, K, V, O), the FFN (MoE: the router plus the
    top_k selected experts), the LM head and one embedding row. RMSNorm gains
    are folded into the following projections, so they are not read. fp16
    weights take 2 bytes each; fp8 weights 1 byte each and fp4 weights half a
    byte each, plus one fp32 scale per row (the embedding row stays fp16).
    """
    d, q, kv, f = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim
    attn = q * d + 2 * kv * d + d * q
    if cfg.n_experts:
        ffn = cfg.n_experts * d + cfg.top_k * 3 * f * d
    else:
        ffn = 3 * f * d
    wf = getattr(cfg, "weight_format", "fp16")
    if wf in ("fp8", "fp4"):
        ffn_rows = (cfg.n_experts + cfg.top_k * (2 * f + d)) if cfg.n_experts else 2 * f + d
        rows = cfg.n_layers * (q + 2 * kv + d + ffn_rows) + cfg.vocab
        weights = cfg.n_layers * (attn + ffn) + cfg.vocab * d
        return (weights if wf == "fp8" else weights // 2) + 4 * rows + 2 * d
    params = cfg.n_layers * (attn + ffn) + cfg.vocab * d + d
    return 2 * params


def kv_bytes_per_position(cfg) -> int:
    """fp16 K and V bytes of one position over all layers."""
    return cfg.n_layers * 2 * cfg.kv_dim * 2


def kv_read_bytes(cfg, attended: int) -> int:
    """K/V bytes read by one pass that attends ``attended`` positions."""
    return kv_bytes_per_position(cfg) * attended


def decode_bytes(cfg, pos0: int, n: int) -> int:
    """Algorithmic bytes of n passes starting at position pos0.

    Pass i runs at position pos0 + i and attends pos0 + i + 1 positions; the
    K/V write of the new position is counted too.
    """
    w = active_weight_bytes(cfg)
    per_pos = kv_bytes_per_position(cfg)
    attended = n * pos0 + n * (n + 1) // 2
    return n * w + per_pos * attended + n * per_pos


def mbu(bytes_per_token: float, tok_per_s: float, peak: float = HBM_PEAK_BYTES_PER_S) -> float:
    """Memory-bandwidth utilisation: bytes/token x tokens/s / peak."""
    return bytes_per_token * tok_per_s / peak


def ceiling_tok_per_s(bandwidth: float, bytes_per_token: float) -> float:
    return bandwidth / bytes_per_token


def token_budget_us(tok_per_s: float) -> float:
    return 1e6 / tok_per_s


def launch_overhead_us(n_layers: int, kernels_per_layer: int, launch_us: float) -> float:
    return n_layers * kernels_per_layer * launch_us


def launch_bound_tok_per_s(n_layers: int, kernels_per_layer: int, launch_us: float) -> float:
    return 1e6 / launch_overhead_us(n_layers, kernels_per_layer, launch_us)


def gemv_bytes(M: int, K: int) -> int:
    """fp16 matrix + fp16 vector read, fp32 result written."""
    return 2 * M * K + 2 * K + 4 * M
