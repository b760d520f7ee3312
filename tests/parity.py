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
