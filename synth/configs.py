"""Workload shapes for batch-1 decode and the GEMV bandwidth probe.

The decoder shapes stand in for the 2B "Laneformer" the pages benchmark
(page 4, "2B demo vs frontier scale": 25 layers, fp16, ~4 GB of active
weights, batch 1). The pages give no head counts or widths, so the widths here
are the synthetic ones this project is measured on: a tiny CPU-checkable
decoder, a ~2.1B dense decoder (also at 32K context), and a top-8 MoE decoder.
"""
from __future__ import annotations

from dataclasses import dataclass, replace, asdict
from typing import Dict, List, Tuple


@dataclass(frozen=True)
class DecoderConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    n_experts: int = 0          # 0 = dense SwiGLU FFN
    top_k: int = 0
    rms_eps: float = 1e-5
    rope_theta: float = 1e4
    prompt_len: int = 16
    decode_steps: int = 64
    kv_prefill: int = 0         # positions of seeded K/V stored before decoding
    weight_sigma: float = 0.02
    router_sigma: float = 0.1
    gain_sigma: float = 0.0     # 0 -> every RMSNorm gain is exactly 1
    seed: int = 0
    weight_format: str = "fp16"   # "fp8" / "fp4": projections held as row-scaled E4M3 / E2M1 (quantized at load)

    @property
    def max_seq(self) -> int:
        return self.kv_prefill + self.prompt_len + self.decode_steps

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_(self, **kw) -> "DecoderConfig":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


@dataclass(frozen=True)
class ProbeConfig:
    name: str
    shapes: Tuple[Tuple[int, int], ...]   # (rows M, cols K): y[M] = A[M,K] x[K]
    matrix_sigma: float = 0.02
    seed: int = 0


CONFIGS: Dict[str, object] = {
    # Tiny decoder, checkable on the CPU in seconds.
    "tiny": DecoderConfig(
        name="tiny", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
        ffn_dim=1024, vocab=4096, prompt_len=16, decode_steps=64),
    # Isolated GEMV bandwidth probe shapes.
    "gemv": ProbeConfig(
        name="gemv", shapes=((2560, 2560), (2560, 8192), (8192, 2560), (2560, 32768))),
    # ~2.1B dense decoder shaped like the pages' 2B model.
    "2b": DecoderConfig(
        name="2b", n_layers=25, d_model=2560, n_heads=20, n_kv_heads=4, head_dim=128,
        ffn_dim=8192, vocab=32768, prompt_len=128, decode_steps=1024),
    # Same decoder with 32768 seeded positions already in the KV cache.
    "2b_32k": DecoderConfig(
        name="2b_32k", n_layers=25, d_model=2560, n_heads=20, n_kv_heads=4, head_dim=128,
        ffn_dim=8192, vocab=32768, prompt_len=0, decode_steps=256, kv_prefill=32768),
    # The same ~2.1B decoder with every projection in row-scaled FP8 (E4M3).
    "2b_fp8": DecoderConfig(
        name="2b_fp8", n_layers=25, d_model=2560, n_heads=20, n_kv_heads=4, head_dim=128,
        ffn_dim=8192, vocab=32768, prompt_len=128, decode_steps=1024, weight_format="fp8"),
    # The same ~2.1B decoder with every projection in row-scaled FP4 (E2M1).
    "2b_fp4": DecoderConfig(
        name="2b_fp4", n_layers=25, d_model=2560, n_heads=20, n_kv_heads=4, head_dim=128,
        ffn_dim=8192, vocab=32768, prompt_len=128, decode_steps=1024, weight_format="fp4"),
    # The MoE decoder with router and experts in row-scaled FP8 (E4M3).
    "moe_fp8": DecoderConfig(
        name="moe_fp8", n_layers=24, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
        ffn_dim=1024, vocab=32768, n_experts=64, top_k=8, prompt_len=128,
        decode_steps=512, weight_format="fp8"),
    # The MoE decoder with router and experts in row-scaled FP4 (E2M1).
    "moe_fp4": DecoderConfig(
        name="moe_fp4", n_layers=24, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
        ffn_dim=1024, vocab=32768, n_experts=64, top_k=8, prompt_len=128,
        decode_steps=512, weight_format="fp4"),
    # Top-8 of 64 experts MoE decoder: only the selected experts are streamed.
    "moe": DecoderConfig(
        name="moe", n_layers=24, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
        ffn_dim=1024, vocab=32768, n_experts=64, top_k=8, prompt_len=128,
        decode_steps=512),
}

ALIASES = {"C1": "tiny", "C2": "gemv", "C3": "2b", "C4": "2b_32k", "C5": "moe"}


def get_config(name: str):
    return CONFIGS[ALIASES.get(name, name)]


def tensor_specs(cfg: DecoderConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Canonical tensor order: (name, shape, kind).

    kind is "w" (N(0, weight_sigma)), "router" (N(0, router_sigma)) or "gain".
    Every matrix is row-major [out][in], so a projection is y = W x.
    Order: E, then per layer [g_attn, Wq, Wk, Wv, Wo, g_ffn, FFN], g_final, W_lm,
    where FFN is (Wg, Wu, Wd) for a dense layer and (W_r, then per expert
    Wg, Wu, Wd) for a MoE layer. The index in this list is the tensor id that
    seeds the tensor's random stream.
    """
    d, q, kv, f = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim
    specs: List[Tuple[str, Tuple[int, ...], str]] = [("E", (cfg.vocab, d), "w")]
    for l in range(cfg.n_layers):
        specs += [
            (f"l{l}.g_attn", (d,), "gain"),
            (f"l{l}.Wq", (q, d), "w"),
            (f"l{l}.Wk", (kv, d), "w"),
            (f"l{l}.Wv", (kv, d), "w"),
            (f"l{l}.Wo", (d, q), "w"),
            (f"l{l}.g_ffn", (d,), "gain"),
        ]
        if cfg.n_experts:
            specs.append((f"l{l}.Wr", (cfg.n_experts, d), "router"))
            for e in range(cfg.n_experts):
                specs += [
                    (f"l{l}.e{e}.Wg", (f, d), "w"),
                    (f"l{l}.e{e}.Wu", (f, d), "w"),
                    (f"l{l}.e{e}.Wd", (d, f), "w"),
                ]
        else:
            specs += [
                (f"l{l}.Wg", (f, d), "w"),
                (f"l{l}.Wu", (f, d), "w"),
                (f"l{l}.Wd", (d, f), "w"),
            ]
    specs += [("g_final", (d,), "gain"), ("W_lm", (cfg.vocab, d), "w")]
    return specs
