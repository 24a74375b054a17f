"""Acceptance bound for a GPU GEMM result against the fp64 reference.

The bound is |C - Cref| <= 2e-4 * T for fp32 output and
|C - Cref| <= 2e-4 * T + 2^-8 * |Cref| for bf16 output, with
T = sum_k |a(i,k) * b(k,j)| from the oracle.  The 2^-8 term covers one
round-to-nearest-even step to bf16 (half an ulp of an 8-bit significand).
NaN positions must match exactly, and so must the positions and signs of
infinities ("B200 GEMM Optimization Ladder", section E step 11: NaN/Inf and
error thresholds are part of every level's correctness gate).

``fp32_slack`` (edge cases only, none of the standard workloads) adds
2^-24 * S, where the caller passes S = 2*|alpha|*T + |beta*c0|: the fp32
epilogue rounds twice, once for alpha*acc (at most 2^-24 |alpha*acc| <=
2^-24 |alpha| T) and once for the fused beta*c0 + that product (at most
2^-24 (|alpha| T + |beta*c0|)), each within half an fp32 ulp.  The literal
bound allows for neither when T is zero or tiny next to beta*c0.
"""
import numpy as np


def tolerance(cref, tsum, out_bf16, fp32_slack=None):
    tol = 2e-4 * tsum
    if out_bf16:
        tol = tol + 2.0 ** -8 * np.abs(cref)
    if fp32_slack is not None:
        tol = tol + 2.0 ** -24 * fp32_slack
    return tol


def check(c, cref, tsum, out_bf16, fp32_slack=None):
    """Returns (ok, worst_ratio, n_bad).  worst_ratio is max |C-Cref|/tol over
    finite entries (0/0 counts as 0); n_bad counts entries out of bound or
    with a NaN/Inf mismatch."""
    c = np.asarray(c, dtype=np.float64)
    cref = np.asarray(cref, dtype=np.float64)
    tsum = np.asarray(tsum, dtype=np.float64)
    if c.shape != cref.shape:
        raise ValueError(f"shape mismatch {c.shape} vs {cref.shape}")
    nan_bad = np.isnan(c) != np.isnan(cref)
    inf_c = np.isinf(c)
    inf_r = np.isinf(cref)
    inf_bad = (inf_c != inf_r) | (inf_c & inf_r & (np.sign(c) != np.sign(cref)))
    finite = np.isfinite(c) & np.isfinite(cref)
    tol = tolerance(cref, tsum, out_bf16, fp32_slack)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        err = np.where(finite, np.abs(c - cref), 0.0)
        ratio = np.where(err == 0.0, 0.0, err / tol)
    ratio = np.where(finite, ratio, 0.0)
    bad = nan_bad | inf_bad | (finite & (err > tol))
    worst = float(ratio.max()) if ratio.size else 0.0
    n_bad = int(bad.sum())
    return n_bad == 0, worst, n_bad
