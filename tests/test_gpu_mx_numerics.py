"""The block-scaled matrix-core instruction's own arithmetic, on the device,
at every MX level, against the CPU model of tests/mx_model.py and against
the oracle:
  - inputs with one nonzero group of 8 products per output: the result
    equals the model bit for bit (the group sum lies on a grid of at most 18
    bits, so the single fp32 add is exact), including groups whose range
    makes the instruction lose more than the 2e-4 * sum|ab| contract (the
    documented exception), and the model's bound covers that loss;
  - random workload-distribution inputs: within two fp32 roundings per add
    of the model;
  - NaN and Inf: an E8M0 scale of 0xFF inside K, E4M3 NaN codes, E5M2 Inf
    and NaN codes give the oracle's NaN/Inf pattern; a 0xFF byte in the
    scale padding past ceil(K/32) is never read.
("B200 TMEM Lifecycle Planner", section A1 case 2: block-scaled MMA, data
and scale factors staged separately; "B200 GEMM Optimization Ladder",
section E step 11: NaN/Inf and error thresholds in every level's gate.)"""
import sys

import numpy as np
import pytest
import torch

import matrix_core_engineering_amd as mce
import oracle
import mx_model
from matrix_core_engineering_amd.inputs import E4M3FN, E5M2, OUT_F32, make_problem
from helpers import oracle_full
from gpu_util import DeviceProblem

pytestmark = pytest.mark.gpu

MX_LEVELS = [3, 5, 6, 7, None]


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def run(p, level):
    d = DeviceProblem(p)
    st = d.run(level)
    assert st == mce.MCE_OK, mce.gemm_status_string(st)
    vals, raw, guards_ok = d.result()
    assert guards_ok, "a write landed outside the logical C"
    return vals


def e4m3(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def single_group_problem(M, N, K, seed):
    """Rows of A and columns of B nonzero only in K group 0 (k = 0..7): a
    large entry next to entries 2^-9 .. 2^8 of mixed sign, so groups span up
    to 17 binades; block-0 scales random, the rest 1."""
    rng = np.random.default_rng(seed)
    p = make_problem(M, N, K, fmt=E4M3FN, a_col_major=False, b_col_major=True, c_dtype=OUT_F32,
                     dist="uniform", lo=-1, hi=1, seed=seed, name="mx_single_group")

    def group(n):
        v = rng.uniform(-1.875, 1.875, (n, 8)) * 2.0 ** rng.integers(-9, 9, (n, 8))
        v[:, 0] = rng.choice([-1, 1], n) * rng.uniform(256, 448, n)
        v = np.clip(v, -448.0, 448.0)          # E4M3's largest finite value
        rng.permuted(v, axis=1, out=v)
        out = np.zeros((n, K), np.uint8)
        out[:, :8] = e4m3(v)
        return out

    p.A = group(M)
    p.B = group(N)
    p.SA = np.full((M, p.ld_sa), 127, np.uint8)
    p.SB = np.full((N, p.ld_sb), 127, np.uint8)
    p.SA[:, 0] = rng.integers(120, 135, M)
    p.SB[:, 0] = rng.integers(120, 135, N)
    return p


@pytest.mark.parametrize("level", MX_LEVELS)
def test_single_group_truncation_bitwise(level):
    """One nonzero group per output: the device result is the model's
    truncated group sum exactly; some entries are off the exact sum by more
    than the contract, and none by more than the model's bound."""
    M = N = 256
    K = 512
    p = single_group_problem(M, N, K, seed=31)
    announce(f"MX single-group truncation level={level}")
    vals = run(p, level)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    model, exact, _ = mx_model.entries(p.A, p.B, p.SA, p.SB, ii.ravel(), jj.ravel())
    model = model.reshape(M, N)
    exact = exact.reshape(M, N)
    bad = np.argwhere(vals != model)
    for i, j in bad[:4]:
        announce(f"  C[{i},{j}] device {vals[i, j]!r} model {model[i, j]!r}; A group codes "
                 f"{list(p.A[i, :8])} B group codes {list(p.B[j, :8])} SA {p.SA[i, 0]} SB {p.SB[j, 0]}")
    assert len(bad) == 0, f"{len(bad)} entries differ from the model"
    cref, tsum = oracle_full(p)
    assert np.array_equal(cref, exact)
    loss = np.abs(vals - cref)
    bound, t = mx_model.truncation_bound(p.A, p.B, p.SA, p.SB)
    assert np.allclose(t, tsum, rtol=1e-12)
    assert np.all(loss <= bound)
    over = np.count_nonzero(loss > 2e-4 * tsum)
    announce(f"  {over} of {M * N} entries beyond 2e-4 sum|ab| (the documented exception); "
             f"worst loss/sum|ab| {float((loss / tsum).max()):.3g}")
    assert over > 0


@pytest.mark.parametrize("level", MX_LEVELS)
def test_random_data_within_model(level):
    """The workload's value distribution (E4M3 from U[-448, 448], scale
    exponents -8..8): sampled entries within two fp32 roundings per add of
    the model, and every entry within the oracle's bound."""
    p = make_problem(512, 384, 2048, fmt=E4M3FN, a_col_major=False, b_col_major=True,
                     c_dtype=OUT_F32, dist="uniform", lo=-448.0, hi=448.0, seed=41,
                     name="mx_random_model")
    announce(f"MX random vs model level={level}")
    vals = run(p, level)
    rng = np.random.default_rng(5)
    ii = rng.integers(0, p.M, 3000)
    jj = rng.integers(0, p.N, 3000)
    model, _, fp32 = mx_model.entries(p.A, p.B, p.SA, p.SB, ii, jj)
    dev = np.abs(vals[ii, jj] - model)
    assert np.all(dev <= 2 * fp32), f"worst {float((dev / (2 * fp32)).max()):.3g} of the allowance"
    cref, tsum = oracle_full(p)
    ok, worst, bad = oracle.check(vals, cref, tsum, False)
    assert ok, f"{bad} entries out of bound (worst {worst:.3g})"


def nan_inf_problem(fmt, K, seed, ld_pad=0):
    lo, hi = (-4.0, 4.0)
    p = make_problem(256, 256, K, fmt=fmt, a_col_major=False, b_col_major=True, c_dtype=OUT_F32,
                     dist="uniform", lo=lo, hi=hi, seed=seed, scale_exp_lo=-2, scale_exp_hi=2,
                     name=f"mx_nan_inf_{fmt}")
    nblk = (K + 31) // 32
    if ld_pad:
        # scale rows padded past ceil(K/32) with the NaN byte: never read
        for name in ("SA", "SB"):
            s = getattr(p, name)
            wide = np.full((s.shape[0], nblk + ld_pad), 0xFF, np.uint8)
            wide[:, :nblk] = s[:, :nblk]
            setattr(p, name, wide)
        p.ld_sa = p.ld_sb = nblk + ld_pad
    return p


@pytest.mark.parametrize("level", MX_LEVELS)
@pytest.mark.parametrize("K", [512, 480])
def test_e4m3_nan_scale_and_codes(level, K):
    """E8M0 0xFF inside K (row 0 of SA, row 5 of SB) and E4M3 NaN codes
    (A[7, 100] = 0x7F, B[9, 200] = 0xFF) give NaN exactly where the oracle
    does; with K = 480 the scale rows carry 0xFF padding past ceil(K/32),
    which must not leak into the result."""
    # K = 480: 15 scale blocks per row, rows padded to 20 bytes (the
    # pipelined kernels read 4-byte scale words)
    p = nan_inf_problem(E4M3FN, K, seed=51, ld_pad=5 if K == 480 else 0)
    p.SA[0, 3] = 0xFF
    p.SB[5, 10] = 0xFF
    p.A[7, 100] = 0x7F
    p.B[9, 200] = 0xFF
    announce(f"E4M3 NaN scale/codes level={level} K={K} ld_sa={p.ld_sa}")
    vals = run(p, level)
    cref, tsum = oracle_full(p)
    assert np.isnan(cref).sum() == 4 * 256 - 4
    ok, worst, bad = oracle.check(vals, cref, tsum, False)
    assert ok, f"{bad} entries differ (NaN mask or bound), worst {worst:.3g}"


@pytest.mark.parametrize("level", MX_LEVELS)
def test_e5m2_inf_and_nan_codes(level):
    """E5M2 infinities and NaN: +Inf and -Inf in A rows, Inf against a zero
    (NaN), +Inf meeting -Inf in one sum (NaN), a NaN code; the device's
    NaN/Inf pattern and signs equal the oracle's, finite entries within the
    bound."""
    p = nan_inf_problem(E5M2, 512, seed=61)
    p.A[0, 5] = 0x7C          # +Inf
    p.A[1, 6] = 0xFC          # -Inf
    p.A[2, 7] = 0x7D          # NaN
    p.B[3, 8] = 0x7C          # +Inf in column 3
    p.A[4, 9] = 0x7C
    p.B[4, 9] = 0x00          # Inf * 0 in entry (4, 4)
    p.A[6, 300] = 0x7C
    p.A[6, 301] = 0xFC        # +Inf and -Inf in one row
    announce(f"E5M2 Inf/NaN level={level}")
    vals = run(p, level)
    cref, tsum = oracle_full(p)
    assert np.isinf(cref).any() and np.isnan(cref).any()
    ok, worst, bad = oracle.check(vals, cref, tsum, False)
    assert ok, f"{bad} entries differ (NaN/Inf mask, sign or bound), worst {worst:.3g}"
