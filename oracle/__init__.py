"""CPU oracle for batch-1 greedy decode and the GEMV probe.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The device library never imports,
links or runs anything here, and nothing here imports the device library.

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: closed forms, invariants, brute force on tiny inputs and the numbers
the pages print. No function here is left unpinned.
"""
from .decoder import (Decoder, rmsnorm, rope_angles, apply_rope, softmax, attention_decode,
                      silu, swiglu_ffn, topk_experts, greedy_argmax, gemv_f64, E4M3_MAX,
                      e4m3_decode_table, e4m3_encode, quantize_rows_e4m3, dequantize_rows_e4m3,
                      E2M1_MAX, e2m1_decode_table, e2m1_encode, quantize_rows_e2m1, dequantize_rows_e2m1)
from .compare import zscore_error, top2_gap, compare_logits

__all__ = [
    "Decoder", "rmsnorm", "rope_angles", "apply_rope", "softmax", "attention_decode",
    "silu", "swiglu_ffn", "topk_experts", "greedy_argmax", "gemv_f64", "E4M3_MAX",
    "e4m3_decode_table", "e4m3_encode", "quantize_rows_e4m3", "dequantize_rows_e4m3",
    "E2M1_MAX", "e2m1_decode_table", "e2m1_encode", "quantize_rows_e2m1", "dequantize_rows_e2m1",
    "zscore_error", "top2_gap", "compare_logits",
]
