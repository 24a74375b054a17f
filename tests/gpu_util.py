"""Device-side glue for the GPU parity tests: upload a Problem, run one entry
point of the library through the C ABI, read C back with its guard bands."""
import numpy as np
import torch

import matrix_core_engineering_amd as mce
from matrix_core_engineering_amd.inputs import BF16, E2M1, E2M3, E3M2, E4M3FN, E5M2, OUT_BF16
from helpers import bf16_bits_to_f64, f64_to_bf16_bits

DEV = torch.device("cuda:0")
# generator format -> the library's element format code
MCE_FORMAT = {E4M3FN: mce.MCE_MX_E4M3, E5M2: mce.MCE_MX_E5M2, E2M3: mce.MCE_MX_E2M3,
              E3M2: mce.MCE_MX_E3M2, E2M1: mce.MCE_MX_E2M1}
GUARD_ROWS = 3
SENTINEL_F32 = 0x7F8ABCDE    # bit patterns no kernel writes
SENTINEL_BF16 = 0x7F8B
NAN_F32 = 0x7FC00000
NAN_BF16 = 0x7FC0


def to_dev(arr):
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    view = {1: np.uint8, 2: np.int16, 4: np.int32}[a.dtype.itemsize]
    return torch.from_numpy(a.view(view).copy()).to(DEV)


class Offset:
    """Operand bytes placed `off` bytes into a device buffer (16-byte aligned
    base), so the pointer handed to the library is misaligned by `off`."""

    def __init__(self, arr, off):
        a = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        host = np.zeros(a.size + 16 + off, np.uint8)
        host[off:off + a.size] = a
        self.buf = torch.from_numpy(host).to(DEV)
        self.off = off

    def data_ptr(self):
        return self.buf.data_ptr() + self.off


class DeviceProblem:
    """Operands on the device; C inside a buffer with GUARD_ROWS sentinel rows
    above and below, sentinel padding columns, and (when beta == 0) NaN in
    every logical element so that an element left unwritten is caught."""

    def __init__(self, p, a_off=0, b_off=0):
        self.p = p
        self.A = Offset(p.A, a_off) if a_off else to_dev(p.A)
        self.B = Offset(p.B, b_off) if b_off else to_dev(p.B)
        self.SA = to_dev(p.SA)
        self.SB = to_dev(p.SB)
        outer = p.N if p.c_col_major else p.M
        inner = p.M if p.c_col_major else p.N
        self.outer, self.inner = outer, inner
        # all bit patterns are handled as unsigned integers so NaN payloads
        # survive the copies exactly
        if p.c_dtype == OUT_BF16:
            host = np.full((outer + 2 * GUARD_ROWS, p.ldc), SENTINEL_BF16, np.uint16)
            fill = NAN_BF16
        else:
            host = np.full((outer + 2 * GUARD_ROWS, p.ldc), SENTINEL_F32, np.uint32)
            fill = NAN_F32
        body = host[GUARD_ROWS:GUARD_ROWS + outer]
        if p.beta != 0.0:
            c0 = np.ascontiguousarray(p.C0).view(host.dtype)
            body[:, :inner] = c0[:outer, :inner]
        else:
            body[:, :inner] = fill
        self.host_before = host.copy()
        self.cbuf = to_dev(host)
        elt = 2 if p.c_dtype == OUT_BF16 else 4
        self.c_ptr = self.cbuf.data_ptr() + GUARD_ROWS * p.ldc * elt

    def run(self, level=None, raise_on_error=True):
        p = self.p
        if p.fmt == BF16:
            args = (p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.B, p.ldb, p.b_col_major,
                    self.c_ptr, p.ldc, p.c_col_major, p.c_dtype, p.alpha, p.beta)
            if level is None:
                return mce.gemm_bf16(*args, raise_on_error=raise_on_error)
            return mce.gemm_bf16_level(level, *args, raise_on_error=raise_on_error)
        args = (p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.SA, p.ld_sa, self.B, p.ldb,
                p.b_col_major, self.SB, p.ld_sb, self.c_ptr, p.ldc, p.c_col_major, p.c_dtype,
                p.alpha, p.beta)
        if p.fmt == E4M3FN:
            if level is None:
                return mce.gemm_mxfp8(*args, raise_on_error=raise_on_error)
            return mce.gemm_mxfp8_level(level, *args, raise_on_error=raise_on_error)
        fmt = MCE_FORMAT[p.fmt]
        if level is None:
            return mce.gemm_mx(fmt, *args, raise_on_error=raise_on_error)
        return mce.gemm_mx_level(level, fmt, *args, raise_on_error=raise_on_error)

    def result(self):
        """(logical M x N float64 result, raw logical storage, guards intact)."""
        torch.cuda.synchronize()
        p = self.p
        host = self.cbuf.cpu().numpy()
        host = host.view(np.uint16 if p.c_dtype == OUT_BF16 else np.uint32)
        before = self.host_before
        g = GUARD_ROWS
        guards_ok = (np.array_equal(host[:g].view(np.uint8), before[:g].view(np.uint8)) and
                     np.array_equal(host[-g:].view(np.uint8), before[-g:].view(np.uint8)) and
                     np.array_equal(host[g:-g, self.inner:].view(np.uint8),
                                    before[g:-g, self.inner:].view(np.uint8)))
        body = host[g:g + self.outer, :self.inner]
        raw = body.T if p.c_col_major else body
        vals = (bf16_bits_to_f64(raw) if p.c_dtype == OUT_BF16
                else np.ascontiguousarray(raw).view(np.float32).astype(np.float64))
        return vals, np.ascontiguousarray(raw), guards_ok


def run_problem(p, level=None):
    d = DeviceProblem(p)
    st = d.run(level)
    assert st == mce.MCE_OK
    vals, raw, guards_ok = d.result()
    assert guards_ok, "a write landed outside the logical C"
    return vals, raw


def expected_bits(p, cref):
    """The exactly-representable result as the bits the kernel must write."""
    if p.c_dtype == OUT_BF16:
        return f64_to_bf16_bits(cref)
    return cref.astype(np.float32).view(np.uint32)
