"""Parity measures between device logits and oracle logits (test infrastructure).

Per-row normalisation: both rows are z-scored with the oracle row's mean and
standard deviation, so the error is in units of the oracle row's spread. The
argmax must agree wherever the oracle's normalised top-2 gap exceeds the
tolerance; below it either index is an acceptable greedy choice.

A device row holding any NaN or infinity has an infinite error: it fails every
tolerance, whatever the oracle's top-2 gap.
"""
from __future__ import annotations

import numpy as np


def zscore_error(dev_row: np.ndarray, ref_row: np.ndarray) -> float:
    """max |dev - ref| / std(ref); inf when the device row is not all finite."""
    ref = ref_row.astype(np.float64)
    dev = dev_row.astype(np.float64)
    if dev.shape != ref.shape or not np.isfinite(dev).all():
        return float("inf")
    sd = ref.std()
    return float(np.max(np.abs(dev - ref)) / sd)


def top2_gap(ref_row: np.ndarray) -> float:
    """(largest - second largest) / std(ref)."""
    ref = ref_row.astype(np.float64)
    top = np.partition(ref, -2)[-2:]
    return float((top[1] - top[0]) / ref.std())


def compare_logits(dev: np.ndarray, ref: np.ndarray, tol: float = 2e-2):
    """Row-wise comparison of [n, vocab] logits.

    Returns (max z-score error, number of rows whose argmax must match,
    number of those that differ, rows checked). The error is inf when any
    device row is not finite or the two arrays differ in shape.
    """
    dev = np.atleast_2d(dev)
    ref = np.atleast_2d(ref)
    if dev.shape != ref.shape:
        return float("inf"), 0, 0, len(ref)
    worst, must, bad = 0.0, 0, 0
    for d, r in zip(dev, ref):
        e = zscore_error(d, r)
        worst = e if not e <= worst else worst   # NaN-safe: a non-finite error always wins
        if top2_gap(r) > tol:
            must += 1
            if int(np.argmax(d)) != int(np.argmax(r)):
                bad += 1
    return worst, must, bad, len(ref)
