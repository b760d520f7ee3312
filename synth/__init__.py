"""Seeded synthetic inputs shared, as data only, by the oracle and the HIP path.

This package draws random numbers and lays out shapes. It holds none of the
decoder's arithmetic (no norm, no projection, no attention, no sampling), so
that the oracle and the device path share nothing but their inputs.
"""
from .configs import CONFIGS, DecoderConfig, ProbeConfig, get_config, tensor_specs
from .gen import (make_weights, make_prompt, make_kv_prefill, make_pending_token,
                  make_forced_tokens, make_probe, weights_sha256)

__all__ = [
    "CONFIGS", "DecoderConfig", "ProbeConfig", "get_config", "tensor_specs",
    "make_weights", "make_prompt", "make_kv_prefill", "make_pending_token", "make_forced_tokens",
    "make_probe", "weights_sha256",
]
