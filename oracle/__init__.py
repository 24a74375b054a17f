"""Plain fp64 CPU references (GEMM, attention) -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It loads ``liboracle.so`` (built by gcc from
``oracle.c`` alone) and shares nothing with the HIP library.

What it computes is the plain definition C <- alpha*op(A)*op(B) + beta*C0 with
exact fp64 decoding of bf16 / MX (E4M3FN, E5M2, E2M3, E3M2, E2M1 elements,
E8M0 scales; OCP MX v1.0) inputs and fp64 sums over k in
order (the baseline contract of "B200 GEMM Optimization Ladder", section E
step 1; block-scaled operands as in "B200 TMEM Lifecycle Planner", section A1
case 2).  ``attention`` is the plain scaled dot-product attention of
attention.c.  ``check`` and ``check_attention`` apply the acceptance bounds
to a GPU result.
"""
import ctypes
import os

import numpy as np

from .build import LIB_PATH, build_oracle

BF16 = 0
E4M3FN = 1
E5M2 = 2
E2M3 = 3
E3M2 = 4
E2M1 = 5
FORMAT_BITS = {BF16: 16, E4M3FN: 8, E5M2: 8, E2M3: 6, E3M2: 6, E2M1: 4}
OUT_F32 = 0
OUT_BF16 = 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build_oracle()
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    common = [i64, i64, i64,
              i32, vp, i64, i32, vp, i64,
              i32, vp, i64, i32, vp, i64,
              vp, i64, i32, i32, f32, f32]
    lib.oracle_gemm_rows.argtypes = common + [i64, i64, vp, vp]
    lib.oracle_gemm_rows.restype = i32
    lib.oracle_gemm_entries.argtypes = common + [i64, vp, vp, vp, vp]
    lib.oracle_gemm_entries.restype = i32
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_to_f64.restype = ctypes.c_double
    for name in ("e5m2", "e2m3", "e3m2", "e2m1"):
        f = getattr(lib, f"oracle_{name}_to_f64")
        f.argtypes = [ctypes.c_uint8]
        f.restype = ctypes.c_double
    lib.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_f64.restype = ctypes.c_double
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    lib.oracle_attention.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, f32, i32, i64, i64,
                                     vp, vp, vp]
    lib.oracle_attention.restype = i32
    _lib = lib
    return lib


def num_threads():
    return _load().oracle_num_threads()


def bf16_to_f64(code):
    return _load().oracle_bf16_to_f64(int(code))


def e4m3fn_to_f64(code):
    return _load().oracle_e4m3fn_to_f64(int(code))


def e5m2_to_f64(code):
    return _load().oracle_e5m2_to_f64(int(code))


def e2m3_to_f64(code):
    return _load().oracle_e2m3_to_f64(int(code))


def e3m2_to_f64(code):
    return _load().oracle_e3m2_to_f64(int(code))


def e2m1_to_f64(code):
    return _load().oracle_e2m1_to_f64(int(code))


def e8m0_to_f64(code):
    return _load().oracle_e8m0_to_f64(int(code))


def _arr(x, dtype):
    """Host numpy view of x (numpy array or CPU torch tensor) with the given
    storage dtype; returns (array, pointer) with the array kept alive."""
    if x is None:
        return None, None
    if hasattr(x, "detach"):
        x = x.detach().cpu().contiguous().numpy()
    x = np.ascontiguousarray(x)
    if x.dtype != dtype:
        x = x.view(dtype)
    return x, x.ctypes.data


def _args(M, N, K, fmt, A, lda, a_col_major, SA, ld_sa, B, ldb, b_col_major,
          SB, ld_sb, C0, ldc, c_col_major, c_dtype, alpha, beta):
    el = np.uint16 if fmt == BF16 else np.uint8
    a, pa = _arr(A, el)
    b, pb = _arr(B, el)
    sa, psa = _arr(SA, np.uint8)
    sb, psb = _arr(SB, np.uint8)
    c0, pc0 = _arr(C0, np.float32 if c_dtype == OUT_F32 else np.uint16)
    keep = (a, b, sa, sb, c0)
    args = [M, N, K,
            fmt, pa, lda, int(a_col_major), psa, ld_sa,
            fmt, pb, ldb, int(b_col_major), psb, ld_sb,
            pc0, ldc, int(c_col_major), int(c_dtype),
            float(alpha), float(beta)]
    return keep, args


def gemm_rows(M, N, K, A, lda, a_col_major, B, ldb, b_col_major,
              C0=None, ldc=0, c_col_major=False, c_dtype=OUT_F32,
              alpha=1.0, beta=0.0, fmt=BF16, SA=None, ld_sa=0, SB=None,
              ld_sb=0, row_begin=0, row_end=None):
    """Reference rows [row_begin, row_end) of C; returns (Cref, T) as
    float64 arrays of shape (rows, N)."""
    if row_end is None:
        row_end = M
    keep, args = _args(M, N, K, fmt, A, lda, a_col_major, SA, ld_sa, B, ldb,
                       b_col_major, SB, ld_sb, C0, ldc, c_col_major, c_dtype,
                       alpha, beta)
    rows = row_end - row_begin
    cref = np.zeros((max(rows, 0), N), dtype=np.float64)
    tsum = np.zeros((max(rows, 0), N), dtype=np.float64)
    rc = _load().oracle_gemm_rows(*args, row_begin, row_end,
                                  cref.ctypes.data, tsum.ctypes.data)
    del keep
    if rc != 0:
        raise ValueError(f"oracle_gemm_rows failed with code {rc}")
    return cref, tsum


def gemm_entries(M, N, K, A, lda, a_col_major, B, ldb, b_col_major, ii, jj,
                 C0=None, ldc=0, c_col_major=False, c_dtype=OUT_F32,
                 alpha=1.0, beta=0.0, fmt=BF16, SA=None, ld_sa=0, SB=None,
                 ld_sb=0):
    """Reference values and T at the entries (ii[t], jj[t])."""
    keep, args = _args(M, N, K, fmt, A, lda, a_col_major, SA, ld_sa, B, ldb,
                       b_col_major, SB, ld_sb, C0, ldc, c_col_major, c_dtype,
                       alpha, beta)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("ii and jj must have the same shape")
    out = np.zeros(ii.shape, dtype=np.float64)
    tsum = np.zeros(ii.shape, dtype=np.float64)
    rc = _load().oracle_gemm_entries(*args, ii.size, ii.ctypes.data,
                                     jj.ctypes.data, out.ctypes.data,
                                     tsum.ctypes.data)
    del keep
    if rc != 0:
        raise ValueError(f"oracle_gemm_entries failed with code {rc}")
    return out, tsum


def attention(batch, heads, seq_q, seq_k, dim, Q, K, V, scale, causal=False, row_begin=0,
              row_end=None):
    """Reference attention rows [row_begin, row_end) of the flattened
    batch x heads x seq_q query rows; Q, K, V hold bf16 bits (uint16, any
    shape with batch*heads*seq*dim elements in that order).  Returns (O, PV,
    SMAX): O and PV of shape (rows, dim), SMAX of shape (rows,)."""
    rows_total = batch * heads * seq_q
    if row_end is None:
        row_end = rows_total
    q, pq = _arr(Q, np.uint16)
    k, pk = _arr(K, np.uint16)
    v, pvv = _arr(V, np.uint16)
    rows = row_end - row_begin
    o = np.zeros((max(rows, 0), dim), dtype=np.float64)
    pv = np.zeros((max(rows, 0), dim), dtype=np.float64)
    smax = np.zeros(max(rows, 0), dtype=np.float64)
    rc = _load().oracle_attention(batch, heads, seq_q, seq_k, dim, pq, pk, pvv, float(scale),
                                  int(bool(causal)), row_begin, row_end, o.ctypes.data,
                                  pv.ctypes.data, smax.ctypes.data)
    del q, k, v
    if rc != 0:
        raise ValueError(f"oracle_attention failed with code {rc}")
    return o, pv, smax


from .check import check, check_attention, tolerance, attention_tolerance  # noqa: E402,F401
