"""Python binding of the gfx950 GEMM library (libmce.so).

Argument marshalling only: every entry point has the name and arguments of
the C function declared in include/mce.h and forwards to it through ctypes.
Operands may be given as torch tensors (their device pointer is passed) or as
raw integer device addresses; ``stream`` defaults to torch's current stream.
Nothing here computes any part of the GEMM, and there is no fallback: if the
shared library is missing, every call raises.
"""
import ctypes
import os

__all__ = ["gemm_bf16", "gemm_mxfp8", "gemm_bf16_level", "gemm_mxfp8_level",
           "gemm_bf16_pick_level", "gemm_mxfp8_pick_level", "gemm_mx",
           "gemm_mx_level", "gemm_mx_pick_level", "gemm_bf16_order", "gemm_mx_order",
           "attention_bf16",
           "MCE_MX_E4M3", "MCE_MX_E5M2",
           "MCE_MX_E2M3", "MCE_MX_E3M2", "MCE_MX_E2M1",
           "gemm_status_string", "MceError", "lib_path", "load",
           "EXPORTED_SYMBOLS", "MCE_OK", "MCE_EINVAL", "MCE_EUNSUPPORTED",
           "MCE_ELAUNCH", "MCE_OUT_F32", "MCE_OUT_BF16", "mce_matrix_core_loop",
           "MCE_LOOP_BF16_32X32X16", "MCE_LOOP_BF16_16X16X32", "MCE_LOOP_MXFP8_32X32X64",
           "MCE_LOOP_MXFP4_32X32X64", "MCE_LOOP_MXFP6_32X32X64"]

MCE_OK, MCE_EINVAL, MCE_EUNSUPPORTED, MCE_ELAUNCH = 0, 1, 2, 3
MCE_OUT_F32, MCE_OUT_BF16 = 0, 1
MCE_MX_E4M3, MCE_MX_E5M2, MCE_MX_E2M3, MCE_MX_E3M2, MCE_MX_E2M1 = 0, 1, 2, 3, 4
MCE_LOOP_BF16_32X32X16, MCE_LOOP_BF16_16X16X32, MCE_LOOP_MXFP8_32X32X64 = 0, 1, 2
MCE_LOOP_MXFP4_32X32X64, MCE_LOOP_MXFP6_32X32X64 = 3, 4

EXPORTED_SYMBOLS = ("gemm_bf16", "gemm_mxfp8", "gemm_bf16_level",
                    "gemm_mxfp8_level", "gemm_bf16_pick_level",
                    "gemm_mxfp8_pick_level", "gemm_mx", "gemm_mx_level",
                    "gemm_mx_pick_level", "gemm_bf16_order", "gemm_mx_order",
                    "attention_bf16", "mce_matrix_core_loop", "gemm_status_string")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib_path():
    return os.path.join(_HERE, "libmce.so")


class MceError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {gemm_status_string(status)}")


def load():
    """Loads libmce.so (built by build.py); raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python matrix_core_engineering_amd/build.py`")
    lib = ctypes.CDLL(path)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    mnk = [i64, i64, i64]
    bf16_args = mnk + [vp, i64, i32, vp, i64, i32, vp, i64, i32, i32, f32, f32, vp]
    mx_args = mnk + [vp, i64, i32, vp, i64, vp, i64, i32, vp, i64, vp, i64, i32, i32,
                     f32, f32, vp]
    lib.gemm_bf16.argtypes = bf16_args
    lib.gemm_mxfp8.argtypes = mx_args
    lib.gemm_bf16_level.argtypes = [i32] + bf16_args
    lib.gemm_mxfp8_level.argtypes = [i32] + mx_args
    pick = mnk + [vp, i64, i32, vp, i64, i32]
    lib.gemm_bf16_pick_level.argtypes = pick
    lib.gemm_mxfp8_pick_level.argtypes = pick
    lib.gemm_mx.argtypes = [i32] + mx_args
    lib.gemm_mx_level.argtypes = [i32, i32] + mx_args
    lib.gemm_mx_pick_level.argtypes = [i32] + mnk + [vp, i64, i32, vp, i64, vp, i64, i32, vp, i64]
    lib.gemm_bf16_order.argtypes = [i32, i32, i32] + bf16_args
    lib.gemm_mx_order.argtypes = [i32, i32, i32, i32] + mx_args
    lib.attention_bf16.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, i32, f32, i32, vp]
    lib.mce_matrix_core_loop.argtypes = [i32, vp, i64, vp, i32, i32, vp]
    for name in EXPORTED_SYMBOLS[:-1]:
        getattr(lib, name).restype = i32
    lib.gemm_status_string.argtypes = [i32]
    lib.gemm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(stream):
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _check(status, where, raise_on_error):
    if raise_on_error and status != MCE_OK:
        raise MceError(status, where)
    return status


def gemm_bf16(M, N, K, A, lda, a_col_major, B, ldb, b_col_major, C, ldc,
              c_col_major, c_dtype, alpha, beta, stream=None, raise_on_error=True):
    st = load().gemm_bf16(M, N, K, _ptr(A), lda, int(a_col_major), _ptr(B), ldb,
                          int(b_col_major), _ptr(C), ldc, int(c_col_major),
                          int(c_dtype), float(alpha), float(beta), _stream(stream))
    return _check(st, "gemm_bf16", raise_on_error)


def gemm_mxfp8(M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb, b_col_major,
               SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta,
               stream=None, raise_on_error=True):
    st = load().gemm_mxfp8(M, N, K, _ptr(A), lda, int(a_col_major), _ptr(SA), ld_sa,
                           _ptr(B), ldb, int(b_col_major), _ptr(SB), ld_sb, _ptr(C),
                           ldc, int(c_col_major), int(c_dtype), float(alpha),
                           float(beta), _stream(stream))
    return _check(st, "gemm_mxfp8", raise_on_error)


def gemm_bf16_level(level, M, N, K, A, lda, a_col_major, B, ldb, b_col_major,
                    C, ldc, c_col_major, c_dtype, alpha, beta, stream=None,
                    raise_on_error=True):
    st = load().gemm_bf16_level(int(level), M, N, K, _ptr(A), lda, int(a_col_major),
                                _ptr(B), ldb, int(b_col_major), _ptr(C), ldc,
                                int(c_col_major), int(c_dtype), float(alpha),
                                float(beta), _stream(stream))
    return _check(st, f"gemm_bf16_level({level})", raise_on_error)


def gemm_mxfp8_level(level, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                     b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha,
                     beta, stream=None, raise_on_error=True):
    st = load().gemm_mxfp8_level(int(level), M, N, K, _ptr(A), lda, int(a_col_major),
                                 _ptr(SA), ld_sa, _ptr(B), ldb, int(b_col_major),
                                 _ptr(SB), ld_sb, _ptr(C), ldc, int(c_col_major),
                                 int(c_dtype), float(alpha), float(beta),
                                 _stream(stream))
    return _check(st, f"gemm_mxfp8_level({level})", raise_on_error)


def gemm_bf16_pick_level(M, N, K, A, lda, a_col_major, B, ldb, b_col_major):
    return load().gemm_bf16_pick_level(M, N, K, _ptr(A), lda, int(a_col_major),
                                       _ptr(B), ldb, int(b_col_major))


def gemm_mxfp8_pick_level(M, N, K, A, lda, a_col_major, B, ldb, b_col_major):
    return load().gemm_mxfp8_pick_level(M, N, K, _ptr(A), lda, int(a_col_major),
                                        _ptr(B), ldb, int(b_col_major))


def gemm_mx(elem_format, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb, b_col_major,
            SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta, stream=None,
            raise_on_error=True):
    st = load().gemm_mx(int(elem_format), M, N, K, _ptr(A), lda, int(a_col_major), _ptr(SA),
                        ld_sa, _ptr(B), ldb, int(b_col_major), _ptr(SB), ld_sb, _ptr(C), ldc,
                        int(c_col_major), int(c_dtype), float(alpha), float(beta),
                        _stream(stream))
    return _check(st, f"gemm_mx({elem_format})", raise_on_error)


def gemm_mx_level(level, elem_format, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                  b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta,
                  stream=None, raise_on_error=True):
    st = load().gemm_mx_level(int(level), int(elem_format), M, N, K, _ptr(A), lda,
                              int(a_col_major), _ptr(SA), ld_sa, _ptr(B), ldb,
                              int(b_col_major), _ptr(SB), ld_sb, _ptr(C), ldc,
                              int(c_col_major), int(c_dtype), float(alpha), float(beta),
                              _stream(stream))
    return _check(st, f"gemm_mx_level({level}, {elem_format})", raise_on_error)


def gemm_mx_pick_level(elem_format, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                       b_col_major, SB, ld_sb):
    return load().gemm_mx_pick_level(int(elem_format), M, N, K, _ptr(A), lda,
                                     int(a_col_major), _ptr(SA), ld_sa, _ptr(B), ldb,
                                     int(b_col_major), _ptr(SB), ld_sb)


def gemm_bf16_order(level, xcd_order, group_m, M, N, K, A, lda, a_col_major, B, ldb,
                    b_col_major, C, ldc, c_col_major, c_dtype, alpha, beta, stream=None,
                    raise_on_error=True):
    st = load().gemm_bf16_order(int(level), int(xcd_order), int(group_m), M, N, K, _ptr(A), lda,
                                int(a_col_major), _ptr(B), ldb, int(b_col_major), _ptr(C), ldc,
                                int(c_col_major), int(c_dtype), float(alpha), float(beta),
                                _stream(stream))
    return _check(st, f"gemm_bf16_order({level}, {xcd_order}, {group_m})", raise_on_error)


def gemm_mx_order(level, xcd_order, group_m, elem_format, M, N, K, A, lda, a_col_major, SA,
                  ld_sa, B, ldb, b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha,
                  beta, stream=None, raise_on_error=True):
    st = load().gemm_mx_order(int(level), int(xcd_order), int(group_m), int(elem_format), M, N,
                              K, _ptr(A), lda, int(a_col_major), _ptr(SA), ld_sa, _ptr(B), ldb,
                              int(b_col_major), _ptr(SB), ld_sb, _ptr(C), ldc, int(c_col_major),
                              int(c_dtype), float(alpha), float(beta), _stream(stream))
    return _check(st, f"gemm_mx_order({level}, {xcd_order}, {group_m}, {elem_format})",
                  raise_on_error)


def attention_bf16(batch, heads, seq_q, seq_k, head_dim, Q, K, V, O, o_dtype, scale,
                   causal=False, stream=None, raise_on_error=True):
    st = load().attention_bf16(batch, heads, seq_q, seq_k, head_dim, _ptr(Q), _ptr(K), _ptr(V),
                               _ptr(O), int(o_dtype), float(scale), int(bool(causal)),
                               _stream(stream))
    return _check(st, "attention_bf16", raise_on_error)


def mce_matrix_core_loop(shape, frags, n_frag, out, blocks, iters, stream=None,
                         raise_on_error=True):
    st = load().mce_matrix_core_loop(int(shape), _ptr(frags), int(n_frag), _ptr(out),
                                     int(blocks), int(iters), _stream(stream))
    return _check(st, f"mce_matrix_core_loop({shape})", raise_on_error)


def gemm_status_string(status):
    return load().gemm_status_string(int(status)).decode()
