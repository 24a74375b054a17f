// Device building blocks shared by every GEMM level: argument block, matrix
// core (MFMA) wrappers with their register maps, buffer resources for
// bounds-checked loads, and the fp32 -> bf16 epilogue conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.hpp"

namespace mce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

enum { OUT_F32 = 0, OUT_BF16 = 1 };

// One GEMM call after host-side normalisation: C is always row-major here
// (a column-major C is turned into the transposed problem on the host).
struct GemmArgs {
    int M, N, K;
    const void *A;
    int lda;
    int a_cm;           // A column-major (M contiguous)
    const void *B;
    int ldb;
    int b_cm;           // B column-major (K contiguous)
    const uint8_t *SA;  // MX only: M x ld_sa E8M0 bytes
    int ld_sa;
    const uint8_t *SB;  // MX only: N x ld_sb E8M0 bytes
    int ld_sb;
    void *C;
    int ldc;
    int c_dtype;
    float alpha, beta;
    int mx_fmt;         // MX only: element format code of both operands (MX_E4M3 ...)
    int ncu;            // compute units of the device (persistent grid size)
    int xcd_order;      // tile walk: 1 XCD-major workgroup slots (default), 0 dispatch order
    int group_m;        // tile rows per group of the grouped order; 0 = default (8)
};


// ---------------------------------------------------------------- MFMA maps
//
// v_mfma_f32_32x32x16_bf16, D(32x32) += A(32x16) * B(16x32), one wave:
//   A operand: lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]   (8 bf16)
//   B operand: lane l holds B[8*(l/32) .. +7][l % 32]           (8 bf16)
//   D: lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32]
// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands (format code 0), with
// h = l/32:
//   A operand: lane l holds A[l % 32][k] in two 16-byte halves:
//              bytes 0..15  <- k = 16h      .. 16h + 15
//              bytes 16..31 <- k = 32 + 16h .. 32 + 16h + 15
//   B operand: the same split along k, column l % 32.
//   scale: block 0 (k 0..31) takes the E8M0 byte of lane l % 32, block 1
//          (k 32..63) that of lane 32 + l % 32, each picked from the lane's
//          32-bit scale register by op_sel.  D map as above.
//   E5M2 (format 1) uses the same map.  The 6- and 4-bit formats (2-4) hold
//   one whole 32-K block per lane: lane l holds k = 32h .. 32h + 31 of row
//   (column) l % 32 packed at 6 or 4 bits per element from bit 0 of the
//   first register (24 or 16 bytes), the rest of the 8 registers unused.
//   The instruction sums each group of 8 consecutive products in fixed
//   point, truncated 13 bits below the group's largest exponent sum, and
//   adds the group sums in fp32 (measured; exact for small-integer data).
// These maps are pinned on the device by exact-integer and closed-form
// tests.

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

__device__ __forceinline__ floatx16 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const floatx16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Block-scaled FMT x FMT -> fp32 (FMT: an MX_* element format code).  OPSEL
// picks the scale byte of sa/sb.
template <int FMT, int OPSEL>
__device__ __forceinline__ floatx16 mfma_mx(const intx8 &a, const intx8 &b, const floatx16 &c, int sa,
                                            int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, OPSEL, sa, OPSEL, sb);
}

template <int OPSEL>
__device__ __forceinline__ floatx16 mfma_mxfp8(const intx8 &a, const intx8 &b, const floatx16 &c,
                                               int sa, int sb)
{
    return mfma_mx<MX_E4M3, OPSEL>(a, b, c, sa, sb);
}

__device__ __forceinline__ floatx16 zero16()
{
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        z[i] = 0.0f;
    return z;
}

// ------------------------------------------------------------ conversions

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v)
{
    __bf16 h = (__bf16)v;   // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// --------------------------------------------------------- buffer loads
//
// A raw buffer resource: loads at byte offsets >= num_records return zero
// and touch no memory.  Masked lanes are given OOB_OFFSET.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// ------------------------------------------------------------ epilogue
//
// out = alpha * acc + beta * c0 in fp32, c0 read only when beta != 0.
__device__ __forceinline__ void store_c(const GemmArgs &p, int row, int col, float acc)
{
    size_t idx = (size_t)row * p.ldc + col;
    float v = p.alpha * acc;
    if (p.c_dtype == OUT_F32) {
        float *c = (float *)p.C;
        if (p.beta != 0.0f)
            v = __builtin_fmaf(p.beta, c[idx], v);
        c[idx] = v;
    } else {
        uint16_t *c = (uint16_t *)p.C;
        if (p.beta != 0.0f)
            v = __builtin_fmaf(p.beta, bf16_to_f32(c[idx]), v);
        c[idx] = f32_to_bf16_rne(v);
    }
}

} // namespace mce
