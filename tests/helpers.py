"""Shared test helpers: independent decoders (torch / numpy) and glue between
``matrix_core_engineering_amd.inputs.Problem`` and the oracle."""
import numpy as np
import torch

import oracle
from matrix_core_engineering_amd.inputs import (BF16, E4M3FN, E5M2, FORMAT_BITS, MX_BLOCK, OUT_BF16,
                                                _INT_CODES, _SIGN)


def bf16_bits_to_f64(bits):
    """numpy uint16 bf16 bits -> float64 (via the binary32 bit pattern)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> bf16 bits, torch round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_decode_elements(codes, fmt):
    """Element decode by torch's own dtypes (independent of the oracle)."""
    t = torch.from_numpy(np.ascontiguousarray(codes))
    if fmt == BF16:
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    if fmt == E5M2:
        return t.view(torch.float8_e5m2).to(torch.float64).numpy()
    if fmt != E4M3FN:
        raise ValueError("torch has no decoder for the packed formats; use int_decode_elements")
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def unpack_codes(store, bits, inner):
    """(outer, bytes) packed storage -> (outer, inner) codes; element e of a
    row at bit offset bits * e, little-endian (written here independently of
    the generator's packer)."""
    store = np.ascontiguousarray(store, dtype=np.uint8)
    if bits == 8:
        return store[:, :inner]
    bitsrow = np.unpackbits(store, axis=1, bitorder="little")
    out = np.zeros((store.shape[0], inner), dtype=np.uint8)
    for b in range(bits):
        out |= (bitsrow[:, b:inner * bits:bits] << b).astype(np.uint8)
    return out


def int_decode_elements(store, fmt, inner):
    """Values of an 'int' draw in a packed format (codes of -4..4 only)."""
    codes = unpack_codes(store, FORMAT_BITS[fmt], inner)
    table = {}
    for v, c in enumerate(_INT_CODES[fmt]):
        table[c] = float(v)
        table[c | _SIGN[fmt]] = -float(v)
    vals = np.vectorize(lambda c: table.get(int(c), np.nan))(codes)
    if np.isnan(vals).any():
        raise ValueError("a code outside the integer table")
    return vals.astype(np.float64)


def decode_elements(p, store, rows, cols, col_major, inner):
    """Logical rows x cols values of an operand of problem p: torch for bf16
    and fp8, the integer code table for the packed formats."""
    if FORMAT_BITS[p.fmt] >= 8:
        return logical(torch_decode_elements(store, p.fmt), rows, cols, col_major)
    return logical(int_decode_elements(store, p.fmt, inner), rows, cols, col_major)


def torch_decode_scales(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def logical(store, rows, cols, col_major):
    """rows x cols logical view of a storage array (outer, ld)."""
    if col_major:
        return store[:cols, :rows].T
    return store[:rows, :cols]


def numpy_reference(p):
    """(alpha*A@B + beta*C0, |A|@|B|) in float64 by numpy, from torch decodes.
    Follows BLAS rules for alpha == 0 / K == 0 / beta == 0."""
    A = logical(torch_decode_elements(p.A, p.fmt), p.M, p.K, p.a_col_major)
    B = logical(torch_decode_elements(p.B, p.fmt), p.K, p.N, p.b_col_major)
    if p.fmt != BF16:
        sa = np.repeat(torch_decode_scales(p.SA), MX_BLOCK, axis=1)[:, :p.K]
        sb = np.repeat(torch_decode_scales(p.SB), MX_BLOCK, axis=1)[:, :p.K]
        A = A * sa
        B = B * sb.T
    out = np.zeros((p.M, p.N))
    tsum = np.zeros((p.M, p.N))
    if p.alpha != 0.0 and p.K > 0:
        out = p.alpha * (A @ B)
        tsum = np.abs(A) @ np.abs(B)
    if p.beta != 0.0:
        c0 = p.C0.astype(np.float64) if p.c_dtype != OUT_BF16 else bf16_bits_to_f64(p.C0)
        out = out + p.beta * logical(c0, p.M, p.N, p.c_col_major)
    return out, tsum


def fp32_epilogue_slack(p, tsum):
    """S = 2*|alpha|*T + |beta*c0| per logical C entry: the magnitudes the
    fp32 epilogue's two roundings scale with (see oracle.check)."""
    s = 2.0 * abs(p.alpha) * np.asarray(tsum, dtype=np.float64)
    if p.beta != 0.0:
        c0 = p.C0.astype(np.float64) if p.c_dtype != OUT_BF16 else bf16_bits_to_f64(p.C0)
        s = s + np.abs(p.beta * logical(c0, p.M, p.N, p.c_col_major))
    return s


def oracle_full(p, row_begin=0, row_end=None):
    return oracle.gemm_rows(row_begin=row_begin, row_end=row_end,
                            **p.oracle_kwargs())


def oracle_entries(p, ii, jj):
    return oracle.gemm_entries(ii=ii, jj=jj, **p.oracle_kwargs())
