// The C ABI boundary: argument validation, the BLAS special cases, the
// column-major-C transposition, level choice and the launch on the caller's
// stream.  No allocation; the only state is a per-device record of whether
// the device is a gfx950 and how many compute units it has.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/mce.h"
#include "launch.hpp"

namespace {

using mce::GemmArgs;

enum Fmt { FMT_BF16 = 0, FMT_MX = 1 };

constexpr int64_t kMaxBytes = (int64_t)1 << 31;   // 32-bit buffer offsets
constexpr int kMaxDevices = 64;
// Per device, queried once: 0 not yet known, -1 not gfx950, else its
// compute-unit count (the persistent grids' size).  Concurrent first calls
// may both query; they store the same value.
std::atomic<int> g_device_cus[kMaxDevices];

// Compute units of the current device if it is a gfx950, else 0.
int gfx950_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 0;
    int state = g_device_cus[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        state = -1;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
            std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
            state = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
        g_device_cus[dev].store(state, std::memory_order_release);
    }
    return state > 0 ? state : 0;
}

// Bytes spanned by rows x cols elements of `bits` bits with leading
// dimension ld (>= inner), saturated at kMaxBytes: every caller only
// compares the result with that limit, and saturating first keeps the
// products below int64 overflow for any 32-bit sizes.
int64_t span_bytes_bits(int64_t outer, int64_t inner, int64_t ld, int bits)
{
    if (outer == 0 || inner == 0)
        return 0;
    const int64_t max_elems = kMaxBytes * 8 / bits;
    if (outer - 1 > max_elems / ld)
        return kMaxBytes;
    const int64_t elems = (outer - 1) * ld + inner;
    return elems > max_elems ? kMaxBytes : (elems * bits + 7) / 8;
}

int64_t span_bytes(int64_t outer, int64_t inner, int64_t ld, int64_t elt)
{
    return span_bytes_bits(outer, inner, ld, (int)(8 * elt));
}

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (!a || !b || na == 0 || nb == 0)
        return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

struct Call {
    int level;   // 0 = pick
    Fmt fmt;
    int mx_fmt;  // MX: element format (MCE_MX_*)
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    int a_cm;
    const void *SA;
    int64_t ld_sa;
    const void *B;
    int64_t ldb;
    int b_cm;
    const void *SB;
    int64_t ld_sb;
    void *C;
    int64_t ldc;
    int c_cm;
    int c_dtype;
    float alpha, beta;
    hipStream_t stream;
    int xcd_order;   // 1 XCD-major tile walk (default), 0 dispatch order
    int group_m;     // tile rows per group; 0 = default
    int ncu;         // set by run(): compute units of the device
};

// Bits per element of the call's operands.
int elem_bits(const Call &c) { return c.fmt == FMT_BF16 ? 16 : mce::mx_bits(c.mx_fmt); }

// Levels 4-7 read operands with 16-byte direct loads: both operands
// K-contiguous, 16-byte aligned rows, K a whole number of 16-byte chunks;
// for MX only the 8-bit element formats have those kernels.
bool fast_eligible(const Call &c)
{
    if (c.fmt == FMT_MX && elem_bits(c) != 8)
        return false;
    int64_t elt = c.fmt == FMT_BF16 ? 2 : 1;
    int64_t per_chunk = 16 / elt;
    return c.a_cm == 0 && c.b_cm == 1 && (c.lda % per_chunk) == 0 && (c.ldb % per_chunk) == 0 &&
           (c.K % per_chunk) == 0 && ((uintptr_t)c.A % 16) == 0 && ((uintptr_t)c.B % 16) == 0;
}

// FP4 levels 5-6: K-contiguous 16-byte aligned rows (lda, ldb multiples of
// 32 elements), K a multiple of 512 and scale rows in whole, aligned
// 16-byte groups.
bool fp4_fast_eligible(const Call &c)
{
    return c.fmt == FMT_MX && c.mx_fmt == MCE_MX_E2M1 && c.a_cm == 0 && c.b_cm == 1 &&
           c.K % 512 == 0 && c.lda % 32 == 0 && c.ldb % 32 == 0 && c.ld_sa % 16 == 0 &&
           c.ld_sb % 16 == 0 && ((uintptr_t)c.A % 16) == 0 && ((uintptr_t)c.B % 16) == 0 &&
           ((uintptr_t)c.SA % 16) == 0 && ((uintptr_t)c.SB % 16) == 0;
}

// FP6 levels 5-6: K-contiguous operands, K a multiple of 128, lda and ldb
// multiples of 64 elements, 16-byte aligned A and B, 4-byte scale rows.
bool fp6_fast_eligible(const Call &c)
{
    return c.fmt == FMT_MX && (c.mx_fmt == MCE_MX_E2M3 || c.mx_fmt == MCE_MX_E3M2) && c.a_cm == 0 &&
           c.b_cm == 1 && c.K > 0 && c.K % 128 == 0 && c.lda % 64 == 0 && c.ldb % 64 == 0 &&
           c.ld_sa % 4 == 0 && c.ld_sb % 4 == 0 && ((uintptr_t)c.A % 16) == 0 &&
           ((uintptr_t)c.B % 16) == 0 && ((uintptr_t)c.SA % 4) == 0 && ((uintptr_t)c.SB % 4) == 0;
}

// 8-bit MX levels 5-6 with an MN-major operand: K a positive multiple of
// 128, 16-byte aligned operands with lda, ldb multiples of 16 bytes, 4-byte
// scale rows.
bool mx_mn_eligible(const Call &c)
{
    return c.fmt == FMT_MX && elem_bits(c) == 8 && (c.a_cm != 0 || c.b_cm == 0) && c.K > 0 &&
           c.K % 128 == 0 && c.lda % 16 == 0 && c.ldb % 16 == 0 && c.ld_sa % 4 == 0 &&
           c.ld_sb % 4 == 0 && ((uintptr_t)c.A % 16) == 0 && ((uintptr_t)c.B % 16) == 0 &&
           ((uintptr_t)c.SA % 4) == 0 && ((uintptr_t)c.SB % 4) == 0;
}

bool mx_scales_eligible(const Call &c)
{
    // the pipelined MX kernels read four scale bytes per 32-bit load
    return (c.ld_sa % 4) == 0 && (c.ld_sb % 4) == 0 && ((uintptr_t)c.SA % 4) == 0 &&
           ((uintptr_t)c.SB % 4) == 0;
}

// Level 9 (eight consumer waves on the early-release ring): whole K tiles,
// at least two (bf16: K a multiple of 64; MX: 8-bit elements and whole
// scale groups, K a multiple of 512 with 16-byte aligned scale rows).
bool level9_eligible(const Call &c)
{
    if (!fast_eligible(c))
        return false;
    if (c.fmt == FMT_BF16)
        return c.K > 64 && c.K % 64 == 0;
    return elem_bits(c) == 8 && c.K % 512 == 0 && c.ld_sa % 16 == 0 && c.ld_sb % 16 == 0 &&
           ((uintptr_t)c.SA % 16) == 0 && ((uintptr_t)c.SB % 16) == 0;
}

constexpr int kBestBf16Level = 6;     // the persistent pipelined kernel
constexpr int kBestMxLevel = 6;

int pick_level(const Call &c)
{
    // bf16, level 9 (eight waves, two per SIMD, on one staged ring) when
    // it accepts the problem and either the problem has no more 256x256
    // tiles than compute units (the second wave per SIMD hides the ring's
    // prologue and epilogue that one tile per workgroup leaves exposed: 4-6%
    // faster than level 6 at 4096^3) or C is whole 256x256 bf16 tiles with
    // beta = 0 and 16-byte aligned rows (the 16x16x32 kernel with the staged
    // epilogue: 1.2-1.4% faster than level 6 at 8192^3 in interleaved
    // same-run rounds); level 6 otherwise
    const bool whole16 = c.c_dtype == MCE_OUT_BF16 && c.beta == 0.0f && c.M % 256 == 0 &&
                         c.N % 256 == 0 && c.ldc % 8 == 0 && ((uintptr_t)c.C % 16) == 0;
    if (c.fmt == FMT_BF16 && level9_eligible(c) && c.ncu > 0 && c.M > 256 && c.N > 256 &&
        (whole16 || ((c.M + 255) / 256) * ((c.N + 255) / 256) <= c.ncu))
        return 9;
    if (c.fmt == FMT_BF16)   // levels 5-6 take any bf16 problem
        return kBestBf16Level;
    if (kBestMxLevel >= 5 && fast_eligible(c) && mx_scales_eligible(c))
        return kBestMxLevel;
    if (fp4_fast_eligible(c) || fp6_fast_eligible(c) || mx_mn_eligible(c))
        return kBestMxLevel;
    return 3;
}

// Whether `level` can run this (already normalised) problem.
bool level_accepts(const Call &c, int level)
{
    if (c.fmt == FMT_BF16) {
        switch (level) {
        case 1: return c.M <= 128 && c.N <= 128 && c.K <= 64;
        case 2: return c.M <= 128 && c.N <= 128;
        case 3: case 5: case 6: return true;
        case 4: case 7: return fast_eligible(c);
        case 9: return level9_eligible(c);
        default: return false;   // level 8: no gfx950 counterpart (include/mce.h)
        }
    }
    switch (level) {
    case 3: return true;
    case 5: case 6:
        return (fast_eligible(c) && mx_scales_eligible(c)) || fp4_fast_eligible(c) ||
               fp6_fast_eligible(c) || mx_mn_eligible(c);
    case 7: return fast_eligible(c) && mx_scales_eligible(c);   // 8-bit formats
    case 9: return level9_eligible(c);
    default: return false;
    }
}

int validate(const Call &c)
{
    if (c.M < 0 || c.N < 0 || c.K < 0)
        return MCE_EINVAL;
    if (c.M > INT32_MAX / 2 || c.N > INT32_MAX / 2 || c.K > INT32_MAX / 2)
        return MCE_EINVAL;
    if (c.c_dtype != MCE_OUT_F32 && c.c_dtype != MCE_OUT_BF16)
        return MCE_EINVAL;
    if (c.fmt == FMT_MX && (c.mx_fmt < MCE_MX_E4M3 || c.mx_fmt > MCE_MX_E2M1))
        return MCE_EINVAL;
    const int bits = elem_bits(c);
    // MN-major MX operands: 8-bit formats only (the packed ones are packed along K)
    if (c.fmt == FMT_MX && bits != 8 && !(c.a_cm == 0 && c.b_cm == 1))
        return MCE_EUNSUPPORTED;
    // packed 6- and 4-bit rows: every row and the K extent fill whole bytes
    const int64_t per_byte_group = bits == 6 ? 4 : bits == 4 ? 2 : 1;
    if (c.K % per_byte_group || c.lda % per_byte_group || c.ldb % per_byte_group)
        return MCE_EINVAL;
    // leading dimensions reach the kernels as 32-bit integers; bounding them
    // here also keeps the span arithmetic below far from int64 overflow
    if (c.lda > INT32_MAX || c.ldb > INT32_MAX || c.ldc > INT32_MAX ||
        (c.fmt == FMT_MX && (c.ld_sa > INT32_MAX || c.ld_sb > INT32_MAX)))
        return MCE_EINVAL;
    if (c.xcd_order != 0 && c.xcd_order != 1)
        return MCE_EINVAL;
    if (c.group_m < 0)
        return MCE_EINVAL;
    const int64_t celt = c.c_dtype == MCE_OUT_F32 ? 4 : 2;
    // leading dimensions: at least the contiguous extent, and at least 1
    auto ld_ok = [](int64_t ld, int64_t extent) { return ld >= 1 && ld >= extent; };
    if (!ld_ok(c.lda, c.a_cm ? c.M : c.K) || !ld_ok(c.ldb, c.b_cm ? c.K : c.N) ||
        !ld_ok(c.ldc, c.c_cm ? c.M : c.N))
        return MCE_EINVAL;
    const int64_t nblk = (c.K + 31) / 32;
    if (c.fmt == FMT_MX && (!ld_ok(c.ld_sa, nblk) || !ld_ok(c.ld_sb, nblk)))
        return MCE_EINVAL;
    if (c.M == 0 || c.N == 0)
        return MCE_OK;
    const bool reads_ab = c.alpha != 0.0f && c.K > 0;
    if (!c.C)
        return MCE_EINVAL;
    const int64_t nc = c.c_cm ? span_bytes(c.N, c.M, c.ldc, celt) : span_bytes(c.M, c.N, c.ldc, celt);
    if (nc >= kMaxBytes)
        return MCE_EINVAL;
    if (!reads_ab)
        return MCE_OK;
    if (!c.A || !c.B)
        return MCE_EINVAL;
    const int64_t na = c.a_cm ? span_bytes_bits(c.K, c.M, c.lda, bits) : span_bytes_bits(c.M, c.K, c.lda, bits);
    const int64_t nb = c.b_cm ? span_bytes_bits(c.N, c.K, c.ldb, bits) : span_bytes_bits(c.K, c.N, c.ldb, bits);
    if (na >= kMaxBytes || nb >= kMaxBytes)
        return MCE_EINVAL;
    if (overlaps(c.C, nc, c.A, na) || overlaps(c.C, nc, c.B, nb))
        return MCE_EINVAL;
    if (c.fmt == FMT_MX) {
        if (!c.SA || !c.SB)
            return MCE_EINVAL;
        const int64_t nsa = span_bytes(c.M, nblk, c.ld_sa, 1);
        const int64_t nsb = span_bytes(c.N, nblk, c.ld_sb, 1);
        if (nsa >= kMaxBytes || nsb >= kMaxBytes)
            return MCE_EINVAL;
        if (overlaps(c.C, nc, c.SA, nsa) || overlaps(c.C, nc, c.SB, nsb))
            return MCE_EINVAL;
    }
    return MCE_OK;
}

// A column-major C is the row-major C^T = B^T A^T: swap the operands (and
// their scales), swap M and N, and flip both operand layout flags.
Call normalise(Call c)
{
    if (!c.c_cm)
        return c;
    Call t = c;
    t.M = c.N;
    t.N = c.M;
    t.A = c.B;
    t.lda = c.ldb;
    t.a_cm = !c.b_cm;
    t.SA = c.SB;
    t.ld_sa = c.ld_sb;
    t.B = c.A;
    t.ldb = c.lda;
    t.b_cm = !c.a_cm;
    t.SB = c.SA;
    t.ld_sb = c.ld_sa;
    t.c_cm = 0;
    return t;
}

GemmArgs kernel_args(const Call &c)
{
    GemmArgs p;
    p.M = (int)c.M;
    p.N = (int)c.N;
    p.K = (int)c.K;
    p.A = c.A;
    p.lda = (int)c.lda;
    p.a_cm = c.a_cm;
    p.B = c.B;
    p.ldb = (int)c.ldb;
    p.b_cm = c.b_cm;
    p.SA = (const uint8_t *)c.SA;
    p.ld_sa = (int)c.ld_sa;
    p.SB = (const uint8_t *)c.SB;
    p.ld_sb = (int)c.ld_sb;
    p.C = c.C;
    p.ldc = (int)c.ldc;
    p.c_dtype = c.c_dtype;
    p.alpha = c.alpha;
    p.beta = c.beta;
    p.mx_fmt = c.mx_fmt;
    p.ncu = c.ncu;
    p.xcd_order = c.xcd_order;
    p.group_m = c.group_m;
    return p;
}

int run(const Call &in)
{
    int st = validate(in);
    if (st != MCE_OK)
        return st;
    const int ncu = gfx950_cus();
    if (ncu == 0)
        return MCE_EUNSUPPORTED;
    Call c = normalise(in);
    c.ncu = ncu;
    if (in.level != 0 && !level_accepts(c, in.level))
        return MCE_EUNSUPPORTED;
    if (c.M == 0 || c.N == 0)
        return MCE_OK;
    GemmArgs p = kernel_args(c);
    hipError_t err;
    if (c.alpha == 0.0f || c.K == 0) {
        err = mce::launch_scale_c(p, c.stream);
    } else {
        int level = in.level != 0 ? in.level : pick_level(c);
        if (c.fmt == FMT_BF16)
            err = level <= 3 ? mce::launch_simple_bf16(level, p, c.stream)
                  : fast_eligible(c) || level == 4 || level == 7 || level == 9
                      ? mce::launch_fast_bf16(level, p, c.stream)
                      : mce::launch_general_bf16(level, p, c.stream);
        else
            err = level <= 3 ? mce::launch_simple_mx(p, c.stream) : mce::launch_fast_mx(level, p, c.stream);
        if (err == hipErrorInvalidValue && level >= 4)
            return MCE_EUNSUPPORTED;
    }
    return err == hipSuccess ? MCE_OK : MCE_ELAUNCH;
}

Call make_call(int level, Fmt fmt, int mx_fmt, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
               int a_cm, const void *SA, int64_t ld_sa, const void *B, int64_t ldb, int b_cm,
               const void *SB, int64_t ld_sb, void *C, int64_t ldc, int c_cm, int c_dtype,
               float alpha, float beta, void *stream)
{
    Call c;
    c.level = level;
    c.fmt = fmt;
    c.mx_fmt = mx_fmt;
    c.M = M;
    c.N = N;
    c.K = K;
    c.A = A;
    c.lda = lda;
    c.a_cm = a_cm ? 1 : 0;
    c.SA = SA;
    c.ld_sa = ld_sa;
    c.B = B;
    c.ldb = ldb;
    c.b_cm = b_cm ? 1 : 0;
    c.SB = SB;
    c.ld_sb = ld_sb;
    c.C = C;
    c.ldc = ldc;
    c.c_cm = c_cm ? 1 : 0;
    c.c_dtype = c_dtype;
    c.alpha = alpha;
    c.beta = beta;
    c.stream = (hipStream_t)stream;
    c.xcd_order = 1;
    c.group_m = 0;
    c.ncu = 0;
    return c;
}

} // namespace

extern "C" {

int gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_col_major,
              const void *B, int64_t ldb, int b_col_major, void *C, int64_t ldc, int c_col_major,
              int c_dtype, float alpha, float beta, void *stream)
{
    return run(make_call(0, FMT_BF16, 0, M, N, K, A, lda, a_col_major, nullptr, 0, B, ldb,
                         b_col_major, nullptr, 0, C, ldc, c_col_major, c_dtype, alpha, beta,
                         stream));
}

int gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_col_major,
               const void *SA, int64_t ld_sa, const void *B, int64_t ldb, int b_col_major,
               const void *SB, int64_t ld_sb, void *C, int64_t ldc, int c_col_major, int c_dtype,
               float alpha, float beta, void *stream)
{
    return run(make_call(0, FMT_MX, MCE_MX_E4M3, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                         b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta,
                         stream));
}

int gemm_bf16_level(int level, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                    int a_col_major, const void *B, int64_t ldb, int b_col_major, void *C,
                    int64_t ldc, int c_col_major, int c_dtype, float alpha, float beta,
                    void *stream)
{
    if (level < 1 || level > 9)
        return MCE_EUNSUPPORTED;
    return run(make_call(level, FMT_BF16, 0, M, N, K, A, lda, a_col_major, nullptr, 0, B, ldb,
                         b_col_major, nullptr, 0, C, ldc, c_col_major, c_dtype, alpha, beta,
                         stream));
}

int gemm_mxfp8_level(int level, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                     int a_col_major, const void *SA, int64_t ld_sa, const void *B, int64_t ldb,
                     int b_col_major, const void *SB, int64_t ld_sb, void *C, int64_t ldc,
                     int c_col_major, int c_dtype, float alpha, float beta, void *stream)
{
    if (level < 1 || level > 9)
        return MCE_EUNSUPPORTED;
    return run(make_call(level, FMT_MX, MCE_MX_E4M3, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                         b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta,
                         stream));
}

int gemm_bf16_pick_level(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                         int a_col_major, const void *B, int64_t ldb, int b_col_major)
{
    // as for a row-major bf16 C with ldc = N, beta = 0 and a 16-byte
    // aligned base (the C pointer itself is not needed to pick)
    Call c = make_call(0, FMT_BF16, 0, M, N, K, A, lda, a_col_major, nullptr, 0, B, ldb, b_col_major,
                       nullptr, 0, nullptr, N > 0 ? N : 1, 0, MCE_OUT_BF16, 1.0f, 0.0f, nullptr);
    if (M < 0 || N < 0 || K < 0)
        return 0;
    c.ncu = gfx950_cus();
    return pick_level(c);
}

int gemm_mxfp8_pick_level(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                          int a_col_major, const void *B, int64_t ldb, int b_col_major)
{
    Call c = make_call(0, FMT_MX, MCE_MX_E4M3, M, N, K, A, lda, a_col_major, nullptr, 4, B, ldb, b_col_major,
                       nullptr, 4, nullptr, 1, 0, MCE_OUT_F32, 1.0f, 0.0f, nullptr);
    if (M < 0 || N < 0 || K < 0)
        return 0;
    return pick_level(c);
}

int gemm_mx(int elem_format, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
            int a_col_major, const void *SA, int64_t ld_sa, const void *B, int64_t ldb,
            int b_col_major, const void *SB, int64_t ld_sb, void *C, int64_t ldc, int c_col_major,
            int c_dtype, float alpha, float beta, void *stream)
{
    return run(make_call(0, FMT_MX, elem_format, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                         b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta, stream));
}

int gemm_mx_level(int level, int elem_format, int64_t M, int64_t N, int64_t K, const void *A,
                  int64_t lda, int a_col_major, const void *SA, int64_t ld_sa, const void *B,
                  int64_t ldb, int b_col_major, const void *SB, int64_t ld_sb, void *C, int64_t ldc,
                  int c_col_major, int c_dtype, float alpha, float beta, void *stream)
{
    if (level < 1 || level > 9)
        return MCE_EUNSUPPORTED;
    return run(make_call(level, FMT_MX, elem_format, M, N, K, A, lda, a_col_major, SA, ld_sa, B,
                         ldb, b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta,
                         stream));
}

int gemm_bf16_order(int level, int xcd_order, int group_m, int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda, int a_col_major, const void *B, int64_t ldb,
                    int b_col_major, void *C, int64_t ldc, int c_col_major, int c_dtype,
                    float alpha, float beta, void *stream)
{
    if (level < 0 || level > 9)
        return MCE_EUNSUPPORTED;
    Call c = make_call(level, FMT_BF16, 0, M, N, K, A, lda, a_col_major, nullptr, 0, B, ldb,
                       b_col_major, nullptr, 0, C, ldc, c_col_major, c_dtype, alpha, beta, stream);
    c.xcd_order = xcd_order;
    c.group_m = group_m;
    return run(c);
}

int gemm_mx_order(int level, int xcd_order, int group_m, int elem_format, int64_t M, int64_t N,
                  int64_t K, const void *A, int64_t lda, int a_col_major, const void *SA,
                  int64_t ld_sa, const void *B, int64_t ldb, int b_col_major, const void *SB,
                  int64_t ld_sb, void *C, int64_t ldc, int c_col_major, int c_dtype, float alpha,
                  float beta, void *stream)
{
    if (level < 0 || level > 9)
        return MCE_EUNSUPPORTED;
    Call c = make_call(level, FMT_MX, elem_format, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                       b_col_major, SB, ld_sb, C, ldc, c_col_major, c_dtype, alpha, beta, stream);
    c.xcd_order = xcd_order;
    c.group_m = group_m;
    return run(c);
}

int gemm_mx_pick_level(int elem_format, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                       int a_col_major, const void *SA, int64_t ld_sa, const void *B, int64_t ldb,
                       int b_col_major, const void *SB, int64_t ld_sb)
{
    Call c = make_call(0, FMT_MX, elem_format, M, N, K, A, lda, a_col_major, SA, ld_sa, B, ldb,
                       b_col_major, SB, ld_sb, nullptr, 1, 0, MCE_OUT_F32, 1.0f, 0.0f, nullptr);
    if (M < 0 || N < 0 || K < 0 || elem_format < MCE_MX_E4M3 || elem_format > MCE_MX_E2M1)
        return 0;
    if (mce::mx_bits(elem_format) != 8 && (a_col_major != 0 || b_col_major != 1))
        return 0;   // the packed formats are packed along K
    return pick_level(c);
}

int mce_matrix_core_loop(int shape, const void *frags, int64_t n_frag, float *out, int blocks,
                         int iters, void *stream)
{
    if (shape < MCE_LOOP_BF16_32X32X16 || shape > MCE_LOOP_MXFP6_32X32X64 || !frags || !out ||
        n_frag < 1 || n_frag > INT32_MAX || blocks < 1 || blocks > 65535 || iters < 1 ||
        iters > (1 << 24))
        return MCE_EINVAL;
    if (gfx950_cus() == 0)
        return MCE_EUNSUPPORTED;
    return mce::launch_matrix_core_loop(shape, frags, (int)n_frag, out, blocks, iters,
                                        (hipStream_t)stream) == hipSuccess
               ? MCE_OK
               : MCE_ELAUNCH;
}

int attention_bf16(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                   const void *Q, const void *K, const void *V, void *O, int o_dtype, float scale,
                   int causal, void *stream)
{
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || head_dim < 1)
        return MCE_EINVAL;
    if (o_dtype != MCE_OUT_F32 && o_dtype != MCE_OUT_BF16)
        return MCE_EINVAL;
    if (batch > INT32_MAX || heads > INT32_MAX || seq_q > INT32_MAX || seq_k > INT32_MAX ||
        head_dim > INT32_MAX)
        return MCE_EINVAL;
    // each (batch, head) slice is addressed with 32-bit buffer offsets (the
    // fp32 output slice included)
    if (seq_q > (kMaxBytes - 1) / 4 / head_dim || seq_k > (kMaxBytes - 1) / 2 / head_dim)
        return MCE_EINVAL;
    const int64_t bh = batch * heads;   // both below 2^31: no overflow
    if (bh > INT32_MAX || bh * ((seq_q + 127) / 128) > INT32_MAX)
        return MCE_EINVAL;
    if (bh == 0 || seq_q == 0)
        return gfx950_cus() == 0 ? MCE_EUNSUPPORTED : MCE_OK;
    if (!Q || !O || (seq_k > 0 && (!K || !V)))
        return MCE_EINVAL;
    const int64_t nq = bh * seq_q * head_dim, nk = bh * seq_k * head_dim;
    const int64_t no = nq * (o_dtype == MCE_OUT_F32 ? 4 : 2);
    if (overlaps(O, no, Q, nq * 2) || overlaps(O, no, K, nk * 2) || overlaps(O, no, V, nk * 2))
        return MCE_EINVAL;
    const int ncu = gfx950_cus();
    if (ncu == 0)
        return MCE_EUNSUPPORTED;
    if (head_dim != 64 && head_dim != 128)
        return MCE_EUNSUPPORTED;
    // 16-byte vector loads of every operand row; 8- or 16-byte output stores
    if ((uintptr_t)Q % 16 || (uintptr_t)K % 16 || (uintptr_t)V % 16 ||
        (uintptr_t)O % (o_dtype == MCE_OUT_F32 ? 16 : 8))
        return MCE_EUNSUPPORTED;
    mce::AttnArgs a;
    a.batch = (int)batch;
    a.heads = (int)heads;
    a.seq_q = (int)seq_q;
    a.seq_k = (int)seq_k;
    a.dim = (int)head_dim;
    a.Q = (const uint16_t *)Q;
    a.K = (const uint16_t *)K;
    a.V = (const uint16_t *)V;
    a.O = O;
    a.scale_log2 = scale * 1.44269504088896340736f;
    a.causal = causal ? 1 : 0;
    a.o_dtype = o_dtype;
    return mce::launch_attention(a, (hipStream_t)stream) == hipSuccess ? MCE_OK : MCE_ELAUNCH;
}

const char *gemm_status_string(int status)
{
    switch (status) {
    case MCE_OK: return "MCE_OK: success";
    case MCE_EINVAL: return "MCE_EINVAL: invalid argument";
    case MCE_EUNSUPPORTED: return "MCE_EUNSUPPORTED: device, level or layout not supported";
    case MCE_ELAUNCH: return "MCE_ELAUNCH: kernel launch failed";
    default: return "unknown mce status";
    }
}

} // extern "C"
