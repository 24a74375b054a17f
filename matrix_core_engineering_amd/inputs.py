"""Seeded synthetic GEMM inputs, shared by the tests, the smoke check and the
benchmark.  This module holds no GEMM arithmetic: it only draws numbers and
stores them in the byte formats the library reads (bf16 bits, MX element
codes, E8M0 scale bytes, fp32 or bf16 C0), in storage order.  The 6- and
4-bit MX element codes are packed along K: element e of a row at bit offset
6e (4e) of the row's little-endian bit string.

Every draw uses its own ``torch.Generator`` seeded with ``seed*1000 + t``
(t: A=0, B=1, C0=2, SA=3, SB=4) and fills the operand in its *storage* order,
so a column-major B is drawn as an N x K array.  Rounding to bf16 / E4M3FN is
torch's round-to-nearest-even on the CPU.

The five standard workloads:
  1  single tile      128x128x64, A,B row-major, U[-1,1], fp32 out, a=1 b=0
  2  square           4096^3, A row, B col, N(0,1), bf16 out, a=1 b=0
  3  ragged           4093x3001x1027, A,B row, U[-1,1], fp32 out, a=.5 b=1,
                      C0 ~ U[-1,1] fp32
  4  large            8192^3, A row, B col, N(0, 0.02^2), bf16 out, a=1 b=0
  5  MX-fp8           8192^3, A row, B col (K-contiguous), E4M3FN from
                      U[-448,448], one E8M0 scale per 32 K with exponent
                      uniform over the integers -8..8, bf16 out, a=1 b=0
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BF16 = 0
E4M3FN = 1
E5M2 = 2
E2M3 = 3
E3M2 = 4
E2M1 = 5
MX_FORMATS = (E4M3FN, E5M2, E2M3, E3M2, E2M1)
FORMAT_BITS = {BF16: 16, E4M3FN: 8, E5M2: 8, E2M3: 6, E3M2: 6, E2M1: 4}
OUT_F32 = 0
OUT_BF16 = 1
MX_BLOCK = 32


@dataclass
class Problem:
    """One GEMM problem in storage form (all arrays are CPU numpy)."""
    M: int
    N: int
    K: int
    fmt: int                 # BF16 or one of MX_FORMATS (both operands)
    A: np.ndarray            # uint16 (bf16 bits) or uint8 (MX codes, packed for 6/4 bits)
    lda: int
    a_col_major: bool
    B: np.ndarray
    ldb: int
    b_col_major: bool
    C0: Optional[np.ndarray]  # float32 or uint16 (bf16 bits); None when beta==0
    ldc: int
    c_col_major: bool
    c_dtype: int             # OUT_F32 or OUT_BF16
    alpha: float
    beta: float
    SA: Optional[np.ndarray] = None   # uint8 E8M0, M x ld_sa row-major
    ld_sa: int = 0
    SB: Optional[np.ndarray] = None   # uint8 E8M0, N x ld_sb row-major
    ld_sb: int = 0
    name: str = ""
    extra: dict = field(default_factory=dict)

    def oracle_kwargs(self):
        return dict(M=self.M, N=self.N, K=self.K, A=self.A, lda=self.lda,
                    a_col_major=self.a_col_major, B=self.B, ldb=self.ldb,
                    b_col_major=self.b_col_major, C0=self.C0, ldc=self.ldc,
                    c_col_major=self.c_col_major, c_dtype=self.c_dtype,
                    alpha=self.alpha, beta=self.beta, fmt=self.fmt,
                    SA=self.SA, ld_sa=self.ld_sa, SB=self.SB, ld_sb=self.ld_sb)

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K


def _gen(seed, t):
    return torch.Generator().manual_seed(int(seed) * 1000 + t)


def _storage_shape(rows, cols, col_major, ld):
    """(outer, inner) of a rows x cols matrix stored with leading dim ld."""
    if col_major:
        return cols, ld
    return rows, ld


def to_bf16_bits(x):
    """float tensor -> uint16 numpy array of bf16 bits (RNE)."""
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn_codes(x):
    """float tensor -> uint8 numpy array of E4M3FN codes (RNE, saturating
    the draw range +-448 exactly onto the largest finite code)."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# Codes of the small integers 0..4 in the 6- and 4-bit formats (OCP MX v1.0
# element tables), and each format's sign bit and code count.
_INT_CODES = {E2M3: [0x00, 0x08, 0x10, 0x14, 0x18], E3M2: [0x00, 0x0C, 0x10, 0x12, 0x14],
              E2M1: [0x0, 0x2, 0x4, 0x5, 0x6]}
_SIGN = {E2M3: 0x20, E3M2: 0x20, E2M1: 0x8}
_NCODES = {E2M3: 64, E3M2: 64, E2M1: 16}


def pack_codes(codes, bits):
    """(outer, inner) uint8 codes -> (outer, inner * bits / 8) packed bytes,
    element e of a row at bit offset bits * e (little-endian)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    if bits == 8:
        return codes
    outer, inner = codes.shape
    if (inner * bits) % 8:
        raise ValueError("a packed row must fill whole bytes")
    out = np.zeros((outer, inner * bits // 8), dtype=np.uint8)
    for e in range(inner):
        bit = e * bits
        byte, off = bit // 8, bit % 8
        v = codes[:, e].astype(np.uint16) << off
        out[:, byte] |= (v & 0xFF).astype(np.uint8)
        if off + bits > 8:
            out[:, byte + 1] |= (v >> 8).astype(np.uint8)
    return out


def _small_codes(fmt, dist, shape, g, lo, hi):
    """6- or 4-bit codes: 'codes' draws every code with equal probability;
    'int' draws integers lo..hi (|v| <= 4) and takes their codes."""
    if dist == "codes":
        return torch.randint(0, _NCODES[fmt], shape, generator=g).numpy().astype(np.uint8)
    if dist == "int":
        if not (-4 <= lo <= hi <= 4):
            raise ValueError("integer draws of the small formats span -4..4")
        v = torch.randint(int(lo), int(hi) + 1, shape, generator=g).numpy()
        table = np.array(_INT_CODES[fmt], dtype=np.uint8)
        return np.where(v < 0, table[np.abs(v)] | _SIGN[fmt], table[np.abs(v)]).astype(np.uint8)
    raise ValueError(f"the 6- and 4-bit formats draw 'codes' or 'int', not {dist}")


def _draw(dist, shape, g, lo=-1.0, hi=1.0, std=1.0):
    if dist == "uniform":
        return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo
    if dist == "normal":
        return torch.randn(shape, generator=g, dtype=torch.float32) * std
    if dist == "int":
        return torch.randint(int(lo), int(hi) + 1, shape, generator=g).to(torch.float32)
    raise ValueError(dist)


def _operand(rows, cols, col_major, ld, fmt, dist, g, **kw):
    outer, inner = _storage_shape(rows, cols, col_major, ld)
    logical_inner = rows if col_major else cols
    if fmt in (E2M3, E3M2, E2M1):
        codes = _small_codes(fmt, dist, (outer, inner), g, kw.get("lo", -1.0), kw.get("hi", 1.0))
        # padding beyond the logical extent holds the largest code, so a
        # kernel that reads it shows up in the result
        codes[:, logical_inner:] = _NCODES[fmt] // 2 - 1
        return pack_codes(codes, FORMAT_BITS[fmt])
    if fmt == E5M2 and dist == "codes":
        codes = torch.randint(0, 256, (outer, inner), generator=g).numpy().astype(np.uint8)
        codes[(codes & 0x7C) == 0x7C] = 0x3C      # no infinities or NaN: 1.0
        codes[:, logical_inner:] = 0x7F
        return codes
    x = _draw(dist, (outer, inner), g, **kw)
    # padding columns beyond the logical extent hold NaN in bf16 and the NaN
    # code in fp8, so a kernel that reads them shows up in the result
    if inner > logical_inner:
        x[:, logical_inner:] = float("nan")
    if fmt == E5M2:
        return x.to(torch.float8_e5m2).view(torch.uint8).numpy()
    return to_bf16_bits(x) if fmt == BF16 else to_e4m3fn_codes(x)


def make_problem(M, N, K, *, fmt=BF16, a_col_major=False, b_col_major=True,
                 c_col_major=False, c_dtype=OUT_BF16, alpha=1.0, beta=0.0,
                 lda=None, ldb=None, ldc=None, dist="normal", std=1.0,
                 lo=-1.0, hi=1.0, c_dist="uniform", seed=0,
                 scale_exp_lo=-8, scale_exp_hi=8, ld_sa=None, ld_sb=None,
                 name=""):
    """Draws one problem.  dist is 'uniform' (U[lo,hi]), 'normal' (N(0,std^2))
    or 'int' (integers lo..hi).  Leading dimensions default to dense."""
    a_inner = M if a_col_major else K
    b_inner = K if b_col_major else N
    c_inner = M if c_col_major else N
    lda = a_inner if lda is None else lda
    ldb = b_inner if ldb is None else ldb
    ldc = c_inner if ldc is None else ldc
    lda, ldb, ldc = max(lda, 1), max(ldb, 1), max(ldc, 1)
    A = _operand(M, K, a_col_major, lda, fmt, dist, _gen(seed, 0), lo=lo, hi=hi, std=std)
    B = _operand(K, N, b_col_major, ldb, fmt, dist, _gen(seed, 1), lo=lo, hi=hi, std=std)
    C0 = None
    if beta != 0.0:
        outer = N if c_col_major else M
        c = _draw(c_dist, (outer, ldc), _gen(seed, 2), lo=-1.0, hi=1.0)
        C0 = c.numpy().astype(np.float32) if c_dtype == OUT_F32 else to_bf16_bits(c)
    SA = SB = None
    if fmt in MX_FORMATS:
        kb = (K + MX_BLOCK - 1) // MX_BLOCK
        ld_sa = max(kb, 1) if ld_sa is None else ld_sa
        ld_sb = max(kb, 1) if ld_sb is None else ld_sb
        SA = (torch.randint(scale_exp_lo, scale_exp_hi + 1, (M, ld_sa),
                            generator=_gen(seed, 3)) + 127).to(torch.uint8).numpy()
        SB = (torch.randint(scale_exp_lo, scale_exp_hi + 1, (N, ld_sb),
                            generator=_gen(seed, 4)) + 127).to(torch.uint8).numpy()
    else:
        ld_sa = ld_sb = 0
    return Problem(M=M, N=N, K=K, fmt=fmt, A=A, lda=lda, a_col_major=a_col_major,
                   B=B, ldb=ldb, b_col_major=b_col_major, C0=C0, ldc=ldc,
                   c_col_major=c_col_major, c_dtype=c_dtype, alpha=float(alpha),
                   beta=float(beta), SA=SA, ld_sa=ld_sa, SB=SB, ld_sb=ld_sb,
                   name=name)


# The five standard workloads, as keyword arguments of make_problem.
CONFIGS = {
    1: dict(M=128, N=128, K=64, a_col_major=False, b_col_major=False,
            c_dtype=OUT_F32, alpha=1.0, beta=0.0, dist="uniform",
            name="single_tile_128x128x64_bf16"),
    2: dict(M=4096, N=4096, K=4096, a_col_major=False, b_col_major=True,
            c_dtype=OUT_BF16, alpha=1.0, beta=0.0, dist="normal", std=1.0,
            name="square_4096_bf16"),
    3: dict(M=4093, N=3001, K=1027, a_col_major=False, b_col_major=False,
            c_dtype=OUT_F32, alpha=0.5, beta=1.0, dist="uniform",
            name="ragged_4093x3001x1027_bf16"),
    4: dict(M=8192, N=8192, K=8192, a_col_major=False, b_col_major=True,
            c_dtype=OUT_BF16, alpha=1.0, beta=0.0, dist="normal", std=0.02,
            name="large_8192_bf16"),
    5: dict(M=8192, N=8192, K=8192, fmt=E4M3FN, a_col_major=False,
            b_col_major=True, c_dtype=OUT_BF16, alpha=1.0, beta=0.0,
            dist="uniform", lo=-448.0, hi=448.0, name="mx_fp8_8192"),
}


# Skinny shapes (one short side): HBM-bound, measured against the HBM roofline.
SKINNY = {
    "skinny_1x8192x8192_bf16": dict(M=1, N=8192, K=8192),
    "skinny_64x8192x8192_bf16": dict(M=64, N=8192, K=8192),
    "skinny_8192x64x8192_bf16": dict(M=8192, N=64, K=8192),
    "skinny_256x8192x8192_bf16": dict(M=256, N=8192, K=8192),
    "skinny_64x8192x8192_mxfp8": dict(M=64, N=8192, K=8192, fmt=E4M3FN, dist="uniform",
                                      lo=-448.0, hi=448.0),
    "skinny_1x8192x8192_mxfp8": dict(M=1, N=8192, K=8192, fmt=E4M3FN, dist="uniform",
                                     lo=-448.0, hi=448.0),
}


def skinny_problem(name, seed=11):
    """A skinny workload: A row-major, B column-major (K-contiguous), bf16
    out, alpha 1, beta 0; bf16 entries N(0, 0.02^2), MX as workload 5."""
    kw = dict(a_col_major=False, b_col_major=True, c_dtype=OUT_BF16, alpha=1.0, beta=0.0,
              dist="normal", std=0.02, name=name)
    kw.update(SKINNY[name])
    return make_problem(seed=seed, **kw)


def config_problem(idx, seed=None):
    """The standard workload idx (1..5), seeded with idx unless given."""
    kw = dict(CONFIGS[idx])
    return make_problem(seed=idx if seed is None else seed, **kw)


def integer_problem(M, N, K, *, fmt=BF16, seed=0, **kw):
    """Exact-integer inputs: entries in -4..4 (and MX scale exponents 0..2),
    so every partial sum is an integer well below 2^24 and any summation
    order gives the same fp32 value."""
    kw.setdefault("dist", "int")
    kw.setdefault("lo", -4)
    kw.setdefault("hi", 4)
    if fmt == E4M3FN:
        kw.setdefault("scale_exp_lo", 0)
        kw.setdefault("scale_exp_hi", 2)
    return make_problem(M, N, K, fmt=fmt, seed=seed, **kw)


# Attention inputs: Q, K, V of batch x heads x seq x dim (dim contiguous) as
# bf16 bits, drawn N(0, std^2) in that order with generators t = 10, 11, 12.
# The standard workload: 16k tokens (4 sequences of 4096), 16 heads of 128.
ATTENTION_WORKLOADS = {
    "causal": dict(batch=4, heads=16, seq_q=4096, seq_k=4096, dim=128, causal=True),
    "full": dict(batch=4, heads=16, seq_q=4096, seq_k=4096, dim=128, causal=False),
}


def attention_inputs(batch, heads, seq_q, seq_k, dim, *, seed=0, std=1.0):
    """(Q, K, V) uint16 arrays of bf16 bits, shapes (batch, heads, seq, dim)."""
    out = []
    for t, seq in ((10, seq_q), (11, seq_k), (12, seq_k)):
        x = torch.randn(batch, heads, seq, dim, generator=_gen(seed, t)) * std
        out.append(to_bf16_bits(x))
    return tuple(out)


def attention_flops(batch, heads, seq_q, seq_k, dim, causal):
    """Matrix-product flops of attention: 4 * dim per visible (query, key)
    pair (the S and the P V products)."""
    pairs = 0
    for i in range(seq_q) if causal else ():
        pairs += min(max(i + seq_k - seq_q + 1, 0), seq_k)
    if not causal:
        pairs = seq_q * seq_k
    return 4.0 * dim * pairs * batch * heads
