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


def attention_tolerance(oref, pv, smax, seq_k, out_bf16):
    """Acceptance bound of an attention output o(i,d) (oracle/attention.c):

        |o - oref| <= (2^-8 + expm1(2 delta) + (2 seq_k + tiles + 8) 2^-24) pv
                      (+ 2^-8 |oref| for bf16 output)

    with pv(i,d) = sum_j p_ij |v(j,d)| and delta = 2.1e-4 * smax(i).
      - The probabilities enter the P V product rounded to bf16 (the bf16
        matrix-core operand): each off by at most half a bf16 ulp, 2^-8 of
        itself, so the product moves by at most 2^-8 pv.
      - The scores are a matrix-core product, within the GEMM contract
        2e-4 * scale * sum_d |q k| <= 2e-4 smax of the exact ones, plus a few
        fp32 roundings of the scaled score and the exponent argument (each
        2^-24 of at most smax; 1e-5 smax covers them).  Moving every logit
        of a row by at most delta moves each normalised probability by a
        factor within exp(+-2 delta), so the output by at most
        expm1(2 delta) pv.
      - The fp32 sums over the seq_k keys (of the output and of the
        normaliser, 2^-24 of the partial sum per add) and the online
        rescaling (one fp32 multiply per key tile) add (2 seq_k + tiles + 8)
        2^-24 pv, with tiles = ceil(seq_k / 16) taken as a generous count."""
    delta = 2.1e-4 * np.asarray(smax, dtype=np.float64)
    tiles = -(-seq_k // 16)
    rel = 2.0 ** -8 + np.expm1(2.0 * delta) + (2 * seq_k + tiles + 8) * 2.0 ** -24
    tol = rel[..., None] * np.asarray(pv, dtype=np.float64)
    if out_bf16:
        tol = tol + 2.0 ** -8 * np.abs(oref)
    return tol


def check_attention(o, oref, pv, smax, seq_k, out_bf16):
    """Returns (ok, worst_ratio, n_bad) for an attention output against the
    oracle (NaN positions must match, as for check)."""
    o = np.asarray(o, dtype=np.float64)
    oref = np.asarray(oref, dtype=np.float64)
    if o.shape != oref.shape:
        raise ValueError(f"shape mismatch {o.shape} vs {oref.shape}")
    tol = attention_tolerance(oref, pv, smax, seq_k, out_bf16)
    nan_bad = np.isnan(o) != np.isnan(oref)
    finite = np.isfinite(o) & np.isfinite(oref)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(finite, np.abs(o - oref), 0.0)
        ratio = np.where(err == 0.0, 0.0, err / tol)
    ratio = np.where(finite, ratio, 0.0)
    bad = nan_bad | (finite & (err > tol)) | (np.isinf(o) != np.isinf(oref))
    return int(bad.sum()) == 0, float(ratio.max()) if ratio.size else 0.0, int(bad.sum())
