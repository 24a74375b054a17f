"""Every element of every full-size standard workload against the fp64
oracle, through the default entry points that the benchmark times, and the
edge cases of large skinny shapes and misaligned operand pointers.

The oracle runs on the host cores in row blocks (about a minute of 16-core
fp64 time for all five workloads); the bound is the oracle's ``check``:
|C - Cref| <= 2e-4 * sum_k |a*b| (+ 2^-8 |Cref| for bf16 output), NaN/Inf
masks equal ("B200 GEMM Optimization Ladder", section E step 1: fix the
reference first; section E step 11: the error threshold, misaligned and
odd shapes as part of each level's gate)."""
import sys

import numpy as np
import pytest

import matrix_core_engineering_amd as mce
import oracle
from matrix_core_engineering_amd.inputs import (BF16, E4M3FN, E5M2, OUT_BF16, OUT_F32, config_problem,
                                                integer_problem, make_problem)
from helpers import oracle_full
from gpu_util import DeviceProblem, expected_bits

pytestmark = pytest.mark.gpu


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def run(p, level=None, a_off=0, b_off=0):
    d = DeviceProblem(p, a_off=a_off, b_off=b_off)
    st = d.run(level)
    assert st == mce.MCE_OK, mce.gemm_status_string(st)
    vals, raw, guards_ok = d.result()
    assert guards_ok, "a write landed outside the logical C"
    return vals, raw


def check_every_element(p, vals, block_elems=1 << 23):
    """All M x N entries against the oracle, in row blocks; returns the
    worst err/tol."""
    rows = max(1, block_elems // max(p.N, 1))
    worst = 0.0
    for r0 in range(0, p.M, rows):
        r1 = min(p.M, r0 + rows)
        cref, tsum = oracle_full(p, r0, r1)
        ok, w, bad = oracle.check(vals[r0:r1], cref, tsum, p.c_dtype == OUT_BF16)
        if not ok:
            err = np.abs(vals[r0:r1] - cref)
            i, j = np.unravel_index(np.nanargmax(np.where(np.isnan(err), np.inf, err)), err.shape)
            pytest.fail(f"rows {r0}..{r1 - 1}: {bad} entries out of bound, worst {w:.3g}; "
                        f"e.g. C[{r0 + i},{j}]={vals[r0 + i, j]!r} ref={cref[i, j]!r} "
                        f"T={tsum[i, j]!r}")
        worst = max(worst, w)
        if p.M * p.N >= 1 << 24:
            announce(f"  rows {r0}..{r1 - 1} checked, worst so far {worst:.3g}")
    return worst


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_every_element(cfg):
    """The standard workload at its full size through gemm_bf16 / gemm_mxfp8
    (the benchmark's launch configuration), every element checked."""
    p = config_problem(cfg)
    announce(f"full-matrix config {cfg}: {p.name} M={p.M} N={p.N} K={p.K}")
    vals, _ = run(p)
    worst = check_every_element(p, vals)
    announce(f"config {cfg}: worst err/tol {worst:.3g} over all {p.M * p.N} entries")


SKINNY = [(1, 8192, 8192), (8192, 1, 8192), (1, 1, 8192), (3, 8192, 4096), (8192, 5, 4096)]


@pytest.mark.parametrize("shape", SKINNY)
@pytest.mark.parametrize("fmt", [BF16, E4M3FN], ids=["bf16", "mx"])
def test_skinny_shapes_every_element(shape, fmt):
    """1 x N x K and M x 1 x K with a long K (the HBM-bound shapes): default
    level, real-valued data, every element."""
    M, N, K = shape
    kw = dict(dist="uniform", lo=-448.0, hi=448.0) if fmt == E4M3FN else dict(dist="normal")
    p = make_problem(M, N, K, fmt=fmt, a_col_major=False, b_col_major=True, c_dtype=OUT_BF16,
                     seed=M * 7 + N, name=f"skinny_{M}x{N}x{K}", **kw)
    announce(f"skinny {p.name} fmt={fmt}")
    vals, _ = run(p)
    check_every_element(p, vals)


# (M, N, K): the split-K skinny kernel's tile shapes (short side 1-32, 33-64),
# ragged long sides, the shortest K it takes (512, one chunk per wave), an
# uneven chunk split, and a K below its range (the ordinary kernels)
SKINNY_SPLIT = [(64, 8192, 8192), (8192, 64, 8192), (33, 4100, 1024), (4100, 47, 1088),
                (64, 300, 512), (17, 33, 576), (64, 64, 448)]


@pytest.mark.parametrize("level", [5, 6, None])
@pytest.mark.parametrize("shape", SKINNY_SPLIT, ids=lambda s: "x".join(map(str, s)))
def test_skinny_split_k_every_element(shape, level):
    """Short side at most 64: four waves split K and reduce through LDS.
    Integer data bitwise (fp32 out); real data with alpha/beta and bf16 out
    within the bound; every element."""
    M, N, K = shape
    q = integer_problem(M, N, K, c_dtype=OUT_F32, seed=M + 3 * N + K, name=f"skinny_int_{M}x{N}x{K}")
    announce(f"skinny split-K {q.name} level={level}")
    _, raw = run(q, level)
    cref, _ = oracle_full(q)
    assert np.array_equal(raw, expected_bits(q, cref))
    p = make_problem(M, N, K, a_col_major=False, b_col_major=True, c_dtype=OUT_BF16, alpha=0.75,
                     beta=-1.25, dist="normal", seed=M + 5 * N + K, name=f"skinny_{M}x{N}x{K}")
    vals, _ = run(p, level)
    check_every_element(p, vals)


# Short side 65-256 (fewer 128x128 tiles than CUs): 128x64 or 64x128 tiles
# across the short side, ragged edges, whole and partial K tiles.
MEDIUM = [(256, 8192, 1024), (8192, 200, 768), (100, 4100, 640), (300, 3000, 520), (65, 1000, 72)]


@pytest.mark.parametrize("level", [5, None])
@pytest.mark.parametrize("shape", MEDIUM, ids=lambda s: "x".join(map(str, s)))
def test_medium_short_side_every_element(shape, level):
    """Integer data bitwise (fp32 out); real data with alpha/beta and bf16
    out within the bound; every element."""
    M, N, K = shape
    q = integer_problem(M, N, K, c_dtype=OUT_F32, seed=M + 7 * N + K, name=f"medium_int_{M}x{N}x{K}")
    announce(f"medium {q.name} level={level}")
    _, raw = run(q, level)
    cref, _ = oracle_full(q)
    want = expected_bits(q, cref)
    assert np.array_equal(raw, want), f"{np.count_nonzero(raw != want)} entries differ"
    p = make_problem(M, N, K, a_col_major=False, b_col_major=True, c_dtype=OUT_BF16, alpha=0.75,
                     beta=-1.25, dist="normal", seed=M + 9 * N + K, name=f"medium_{M}x{N}x{K}")
    vals, _ = run(p, level)
    check_every_element(p, vals)


# 8-bit MX with a short side: the same two kernels with E4M3 / E5M2 operands,
# 128-wide K chunks and one scale word per row and chunk.  Shapes: both
# tile kernels (short side 1-32 and 33-64, M or N short), ragged long sides,
# the shortest K they take (1024: one chunk per wave of the register
# kernel), uneven chunk splits (1152 = 9 chunks, 1280 = 10), and a K below
# the range (896: the ordinary MX kernels).
SKINNY_MX = [(64, 8192, 8192), (8192, 64, 4096), (1, 4100, 2048), (33, 4100, 1024), (4100, 47, 1152),
             (17, 33, 1024), (64, 64, 1280), (32, 300, 896)]


@pytest.mark.parametrize("level", [5, None])
@pytest.mark.parametrize("fmt", [E4M3FN, E5M2], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", SKINNY_MX, ids=lambda s: "x".join(map(str, s)))
def test_skinny_mx_every_element(shape, fmt, level):
    """MX with a short side at most 64: integer data (scale exponents 0..2)
    bitwise with fp32 out; U[-448, 448] data with alpha/beta and bf16 out
    within the bound; every element."""
    M, N, K = shape
    q = integer_problem(M, N, K, fmt=fmt, c_dtype=OUT_F32, scale_exp_lo=0, scale_exp_hi=2,
                        seed=M + 3 * N + K + fmt, name=f"skinny_mx_int_{M}x{N}x{K}")
    announce(f"skinny MX {q.name} fmt={fmt} level={level}")
    _, raw = run(q, level)
    cref, _ = oracle_full(q)
    want = expected_bits(q, cref)
    assert np.array_equal(raw, want), f"{np.count_nonzero(raw != want)} entries differ"
    p = make_problem(M, N, K, fmt=fmt, a_col_major=False, b_col_major=True, c_dtype=OUT_BF16,
                     alpha=0.75, beta=-1.25, dist="uniform", lo=-448.0, hi=448.0,
                     seed=M + 5 * N + K + fmt, name=f"skinny_mx_{M}x{N}x{K}")
    vals, _ = run(p, level)
    check_every_element(p, vals)


@pytest.mark.parametrize("shape", [(1, 8192, 8192), (8192, 1, 8192), (257, 300, 1000)])
@pytest.mark.parametrize("layout", [(False, True), (False, False), (True, True)])
@pytest.mark.parametrize("offs", [(2, 0), (0, 2), (2, 6)])
def test_misaligned_operand_pointers(shape, layout, offs):
    """bf16 A and B base pointers 2 (or 6) bytes off 16-byte alignment: the
    default entry point takes the register-staged kernel; integer inputs so
    the result is bitwise, and every element is checked."""
    M, N, K = shape
    a_cm, b_cm = layout
    p = integer_problem(M, N, K, a_col_major=a_cm, b_col_major=b_cm, c_dtype=OUT_F32,
                        seed=M + N + K + offs[0], name=f"misaligned_{M}x{N}x{K}")
    announce(f"misaligned {p.name} layout={layout} offsets={offs}")
    vals, raw = run(p, a_off=offs[0], b_off=offs[1])
    cref, _ = oracle_full(p)
    want = expected_bits(p, cref)
    assert np.array_equal(raw, want), f"{np.count_nonzero(raw != want)} entries differ"


@pytest.mark.parametrize("level", [3, 5, 6])
def test_misaligned_real_valued(level):
    """Real-valued bf16 data through misaligned pointers with alpha/beta and
    a bf16 C: within the bound."""
    p = make_problem(1000, 777, 513, a_col_major=False, b_col_major=True, c_dtype=OUT_BF16,
                     alpha=0.75, beta=-1.25, dist="normal", seed=77, name="misaligned_real")
    announce(f"misaligned real-valued level={level}")
    vals, _ = run(p, level=level, a_off=2, b_off=4)
    check_every_element(p, vals)
