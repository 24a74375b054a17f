"""CPU-side checks of the C ABI: the library loads, exports every function
that include/mce.h declares, and rejects bad arguments synchronously before
touching the device.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import matrix_core_engineering_amd as mce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mce.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(mce.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mce.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    mce.load()


def test_status_strings():
    for st in (mce.MCE_OK, mce.MCE_EINVAL, mce.MCE_EUNSUPPORTED, mce.MCE_ELAUNCH):
        s = mce.gemm_status_string(st)
        assert s.startswith("MCE_")
    assert mce.gemm_status_string(99) == "unknown mce status"


FAKE_A, FAKE_B, FAKE_C = 0x10000000, 0x20000000, 0x30000000


def bf16(M, N, K, lda, a_cm, ldb, b_cm, ldc, c_cm=0, c_dtype=0, alpha=1.0, beta=0.0,
         A=FAKE_A, B=FAKE_B, C=FAKE_C, level=None):
    if level is None:
        return mce.gemm_bf16(M, N, K, A, lda, a_cm, B, ldb, b_cm, C, ldc, c_cm, c_dtype,
                             alpha, beta, stream=0, raise_on_error=False)
    return mce.gemm_bf16_level(level, M, N, K, A, lda, a_cm, B, ldb, b_cm, C, ldc, c_cm,
                               c_dtype, alpha, beta, stream=0, raise_on_error=False)


@pytest.mark.parametrize("args", [
    dict(M=-1, N=4, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=4),         # negative size
    dict(M=4, N=4, K=4, lda=3, a_cm=0, ldb=4, b_cm=1, ldc=4),          # lda < K
    dict(M=4, N=4, K=4, lda=4, a_cm=1, ldb=3, b_cm=1, ldc=4),          # ldb < K
    dict(M=4, N=5, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=4),          # ldc < N
    dict(M=5, N=4, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=4, c_cm=1),  # ldc < M (col C)
    dict(M=4, N=4, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=4, c_dtype=7),
    dict(M=4, N=4, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=4, A=0),      # A NULL
    dict(M=4, N=4, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=4, C=0),      # C NULL
    dict(M=4, N=4, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=4, C=FAKE_A + 8),  # C overlaps A
    dict(M=1 << 16, N=4, K=1 << 15, lda=1 << 15, a_cm=0, ldb=1 << 15, b_cm=1, ldc=4),  # A >= 2 GiB
    dict(M=3, N=4, K=4, lda=1 << 62, a_cm=0, ldb=4, b_cm=1, ldc=4),    # lda overflows a span
    dict(M=3, N=4, K=4, lda=(1 << 31) + 8, a_cm=0, ldb=4, b_cm=1, ldc=4),  # lda above int32
    dict(M=3, N=4, K=4, lda=4, a_cm=0, ldb=4, b_cm=1, ldc=1 << 62),    # ldc overflows a span
    dict(M=3, N=4, K=4, lda=4, a_cm=0, ldb=1 << 40, b_cm=1, ldc=4),    # ldb above int32
])
def test_invalid_arguments_rejected_on_host(args):
    assert bf16(**args) == mce.MCE_EINVAL


def test_tile_order_knobs_validated():
    def order(xcd, gm, level=0):
        return mce.gemm_bf16_order(level, xcd, gm, 4, 4, 4, FAKE_A, 4, 0, FAKE_B, 4, 1, FAKE_C, 4,
                                   0, 0, 1.0, 0.0, stream=0, raise_on_error=False)
    assert order(2, 0) == mce.MCE_EINVAL
    assert order(-1, 0) == mce.MCE_EINVAL
    assert order(1, -1) == mce.MCE_EINVAL
    assert order(1, 0, level=8) == mce.MCE_EUNSUPPORTED
    st = mce.gemm_mx_order(0, 3, 0, mce.MCE_MX_E4M3, 4, 4, 32, FAKE_A, 32, 0, 0x40000000, 1,
                           FAKE_B, 32, 1, 0x50000000, 1, FAKE_C, 4, 0, 0, 1.0, 0.0, stream=0,
                           raise_on_error=False)
    assert st == mce.MCE_EINVAL


def test_level_out_of_range():
    assert bf16(4, 4, 4, 4, 0, 4, 1, 4, level=0) == mce.MCE_EUNSUPPORTED
    assert bf16(4, 4, 4, 4, 0, 4, 1, 4, level=8) == mce.MCE_EUNSUPPORTED


def test_mx_layouts_and_short_scale_ld():
    """8-bit MX operands may be MN-major (level 3 when K is not a multiple of
    128); packed ones may not; a scale row shorter than ceil(K/32) is
    invalid."""
    def mx(a_cm, b_cm, ld_sa=1, ld_sb=1, K=32):
        return mce.gemm_mxfp8(4, 4, K, FAKE_A, 4 if a_cm else K, a_cm, 0x40000000, ld_sa,
                              FAKE_B, K if b_cm else 4, b_cm, 0x50000000, ld_sb, FAKE_C, 4, 0,
                              0, 1.0, 0.0, stream=0, raise_on_error=False)
    assert mx(0, 1, ld_sa=1, K=64) == mce.MCE_EINVAL     # needs ceil(64/32) = 2
    assert mce.gemm_mxfp8_pick_level(64, 64, 64, FAKE_A, 64, 1, FAKE_B, 64, 0) == 3
    assert mce.gemm_mx_pick_level(mce.MCE_MX_E5M2, 64, 64, 64, FAKE_A, 64, 1, 0x40000000, 4,
                                  FAKE_B, 64, 0, 0x50000000, 4) == 3
    for fmt in (mce.MCE_MX_E2M3, mce.MCE_MX_E2M1):
        assert mce.gemm_mx_pick_level(fmt, 64, 64, 64, FAKE_A, 64, 1, 0x40000000, 4,
                                      FAKE_B, 64, 1, 0x50000000, 4) == 0
        st = mce.gemm_mx(fmt, 4, 4, 32, FAKE_A, 4, 1, 0x40000000, 1, FAKE_B, 32, 1, 0x50000000, 1,
                         FAKE_C, 4, 0, 0, 1.0, 0.0, stream=0, raise_on_error=False)
        assert st == mce.MCE_EUNSUPPORTED


def test_pick_level_reports_a_level():
    assert mce.gemm_bf16_pick_level(4096, 4096, 4096, FAKE_A, 4096, 0, FAKE_B, 4096, 1) >= 3
    # row-major B with 2-byte aligned rows: the register-staged kernel of level 6
    assert mce.gemm_bf16_pick_level(4093, 3001, 1027, FAKE_A, 1027, 0, FAKE_B, 3001, 0) == 6
    assert mce.gemm_mxfp8_pick_level(8192, 8192, 8192, FAKE_A, 8192, 0, FAKE_B, 8192, 1) >= 3
    assert mce.gemm_mxfp8_pick_level(-8, 8, 64, FAKE_A, 8, 1, FAKE_B, 64, 1) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mce, "_lib", None)
    monkeypatch.setattr(mce, "lib_path", lambda: str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        mce.load()


def mx_call(fmt, M=64, N=64, K=64, lda=None, ldb=None, A=0x1000, B=0x9000, level=None):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    args = (M, N, K, A, lda, 0, 0x20000, 2, B, ldb, 1, 0x30000, 2, 0x40000, N, 0, 0, 1.0, 0.0, 0)
    if level is None:
        return mce.load().gemm_mx(fmt, *args)
    return mce.load().gemm_mx_level(level, fmt, *args)


def test_mx_unknown_format_is_einval():
    for fmt in (-1, 5, 99):
        assert mx_call(fmt) == mce.MCE_EINVAL
        assert mce.gemm_mx_pick_level(fmt, 64, 64, 64, 0x1000, 64, 0, 0x20000, 2, 0x9000, 64, 1, 0x30000, 2) == 0


@pytest.mark.parametrize("fmt,unit", [(mce.MCE_MX_E2M3, 4), (mce.MCE_MX_E3M2, 4), (mce.MCE_MX_E2M1, 2)])
def test_mx_packed_formats_need_whole_bytes(fmt, unit):
    """K and the leading dimensions of the packed formats must fill whole
    bytes (multiples of 4 elements for 6 bits, 2 for 4 bits)."""
    assert mx_call(fmt, K=64 + unit - 1 if unit > 1 else 63, lda=68, ldb=68) == mce.MCE_EINVAL
    assert mx_call(fmt, K=64, lda=64 + 1, ldb=64) == mce.MCE_EINVAL
    assert mx_call(fmt, K=64, lda=64, ldb=64 + 1) == mce.MCE_EINVAL


def test_mx_pick_level_by_format():
    """Every format picks the pipelined level when the operands allow it,
    else level 3."""
    def pick(fmt, K=8192, lda=8192, ld_s=256, a_cm=0):
        return mce.gemm_mx_pick_level(fmt, 8192, 8192, K, 0x1000, lda, a_cm, 0x20000, ld_s, 0x9000,
                                      lda, 1, 0x30000, ld_s)
    for fmt in (mce.MCE_MX_E4M3, mce.MCE_MX_E5M2, mce.MCE_MX_E2M1, mce.MCE_MX_E2M3,
                mce.MCE_MX_E3M2):
        assert pick(fmt) == 6
    # the 6-bit formats' pipelined level needs K a multiple of 128 and lda,
    # ldb multiples of 64
    for fmt in (mce.MCE_MX_E2M3, mce.MCE_MX_E3M2):
        assert pick(fmt, K=8192 - 64, lda=8192) == 3
        assert pick(fmt, K=4096, lda=8192 - 32) == 3
        assert pick(fmt, K=4096, lda=8192 - 64) == 6
    # E2M1's pipelined level needs 16-byte scale rows and K a multiple of 512
    assert pick(mce.MCE_MX_E2M1, ld_s=260) == 3
    assert pick(mce.MCE_MX_E2M1, K=8192 - 256, lda=8192, ld_s=256) == 3
    # MN-major 8-bit operands: the transpose-load kernel when K is a multiple
    # of 128 and the leading dimensions of 16 bytes, else level 3
    assert pick(mce.MCE_MX_E5M2, a_cm=1) == 6
    assert pick(mce.MCE_MX_E4M3, a_cm=1, K=8192 - 64) == 3
    assert pick(mce.MCE_MX_E4M3, a_cm=1, lda=8192 - 8) == 3
    assert (mce.gemm_mxfp8_pick_level(8192, 8192, 8192, 0x1000, 8192, 0, 0x9000, 8192, 1) ==
            pick(mce.MCE_MX_E4M3))


@pytest.mark.parametrize("shape,frags,n_frag,out,blocks,iters", [
    (5, FAKE_A, 16, FAKE_C, 1, 1),            # unknown shape
    (-1, FAKE_A, 16, FAKE_C, 1, 1),
    (0, 0, 16, FAKE_C, 1, 1),                 # frags NULL
    (0, FAKE_A, 16, 0, 1, 1),                 # out NULL
    (0, FAKE_A, 0, FAKE_C, 1, 1),             # no fragment
    (1, FAKE_A, 16, FAKE_C, 0, 1),            # no workgroup
    (1, FAKE_A, 16, FAKE_C, 65536, 1),        # grid too large
    (2, FAKE_A, 16, FAKE_C, 1, 0),            # no iteration
    (2, FAKE_A, 16, FAKE_C, 1, (1 << 24) + 1),
])
def test_matrix_core_loop_rejects_bad_arguments(shape, frags, n_frag, out, blocks, iters):
    assert mce.mce_matrix_core_loop(shape, frags, n_frag, out, blocks, iters, stream=0,
                                    raise_on_error=False) == mce.MCE_EINVAL


def attn(B=1, H=1, S=4, T=4, D=64, Q=FAKE_A, K=FAKE_B, V=0x40000000, O=FAKE_C, o_dtype=1,
         scale=0.125, causal=0):
    return mce.attention_bf16(B, H, S, T, D, Q, K, V, O, o_dtype, scale, causal, stream=0,
                              raise_on_error=False)


@pytest.mark.parametrize("args", [
    dict(B=-1), dict(H=-1), dict(S=-1), dict(T=-1), dict(D=0),
    dict(o_dtype=5),
    dict(Q=0), dict(O=0), dict(K=0), dict(V=0),
    dict(O=FAKE_A + 64),                               # O overlaps Q
    dict(O=0x40000000 + 16),                           # O overlaps V
    dict(S=1 << 24, D=128),                            # fp32 output slice of 8 GiB
    dict(T=1 << 23, D=128),                            # K slice of 2 GiB
    dict(D=1 << 40),                                   # head_dim beyond 32 bits
    dict(B=1 << 20, H=1 << 12),                        # batch * heads above 2^31
])
def test_attention_invalid_arguments(args):
    assert attn(**args) == mce.MCE_EINVAL


def test_attention_empty_and_unsupported():
    # nothing to compute: no pointer is used, so NULL is fine
    for kw in (dict(B=0), dict(H=0), dict(S=0)):
        st = attn(Q=0, K=0, V=0, O=0, **kw)
        assert st in (mce.MCE_OK, mce.MCE_EUNSUPPORTED)
    # no key at all: Q and O are still needed, K and V are not
    assert attn(T=0, K=0, V=0, Q=0) == mce.MCE_EINVAL
    assert attn(D=96) == mce.MCE_EUNSUPPORTED
    assert attn(Q=FAKE_A + 8) == mce.MCE_EUNSUPPORTED
