// The matrix-core ceiling: the rate the chip sustains when it does nothing
// but matrix-core instructions.  The pages ask to stop tuning near the
// practical roofline ("B200 GEMM Optimization Ladder", section E step 11);
// on MI355X the practical roofline of a dense contraction is set by the
// socket's power limit, not by the published 2.4 GHz peak, and depends on the
// instruction shape and the operand values.  This kernel measures it: one
// workgroup of four waves per CU (one wave per SIMD, as in the GEMM kernels),
// each wave holding the accumulators of one 128x128 tile and repeating that
// tile's instruction sequence on operand fragments loaded once from memory.
// No LDS, no other memory traffic inside the loop.
#include <hip/hip_runtime.h>

#include "../../include/mce.h"
#include "common.hpp"
#include "launch.hpp"

namespace mce {
namespace {

// Per iteration and wave 2^21 flops for every shape:
//   32x32x16 bf16: 4 k-steps x 4x4 blocks = 64 instructions of 32768 flops
//   16x16x32 bf16: 2 k-steps x 8x8 blocks = 128 instructions of 16384 flops
//   32x32x64 MX E4M3, E2M3 or E2M1: 1 k-step x 4x4 blocks = 16
//   instructions of 131072 flops (E2M3 operands: the first six of the eight
//   registers, E2M1 the first four)
// Sixteen operand fragments per lane (eight A, eight B); consecutive
// instructions take different fragments, as in the GEMM's inner loop.
template <int SHAPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void matrix_core_loop(const void *__restrict__ frags, int n_frag, float *__restrict__ out, int iters)
{
    const int gid = blockIdx.x * 256 + threadIdx.x;
    float s = 0.0f;
    if constexpr (SHAPE == MCE_LOOP_MXFP8_32X32X64 || SHAPE == MCE_LOOP_MXFP4_32X32X64 ||
                  SHAPE == MCE_LOOP_MXFP6_32X32X64) {
        constexpr int FMT = SHAPE == MCE_LOOP_MXFP8_32X32X64   ? MX_E4M3
                            : SHAPE == MCE_LOOP_MXFP6_32X32X64 ? MX_E2M3
                                                               : MX_E2M1;
        intx8 f[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            f[i] = ((const intx8 *)frags)[(gid * 16 + i) % n_frag];
        floatx16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = zero16();
        const int sc = 0x7F7F7F7F;   // E8M0 127: every block scaled by 1
        // (fragment indices are compile-time constants: an index that depends
        // on the loop counter would move the fragments out of registers)
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = mfma_mx<FMT, 0>(f[8 + ((i + 2 * j) & 7)], f[(2 * i + j) & 7], acc[i][j], sc, sc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s += acc[i][j][r];
    } else if constexpr (SHAPE == MCE_LOOP_BF16_32X32X16) {
        bf16x8 f[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            f[i] = ((const bf16x8 *)frags)[(gid * 16 + i) % n_frag];
        floatx16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = zero16();
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = mfma_bf16(f[(ks & 1) * 8 + 4 + j], f[(ks & 1) * 8 + i], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s += acc[i][j][r];
    } else {
        bf16x8 f[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            f[i] = ((const bf16x8 *)frags)[(gid * 16 + i) % n_frag];
        floatx4 acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            f[8 + ((j + ks) & 7)], f[(i + ks) & 7], acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s += acc[i][j][r];
    }
    out[gid] = s;
}

} // namespace

hipError_t launch_matrix_core_loop(int shape, const void *frags, int n_frag, float *out, int blocks,
                                   int iters, hipStream_t s)
{
    switch (shape) {
    case MCE_LOOP_BF16_32X32X16:
        hipLaunchKernelGGL((matrix_core_loop<MCE_LOOP_BF16_32X32X16>), dim3(blocks), dim3(256), 0, s,
                           frags, n_frag, out, iters);
        break;
    case MCE_LOOP_BF16_16X16X32:
        hipLaunchKernelGGL((matrix_core_loop<MCE_LOOP_BF16_16X16X32>), dim3(blocks), dim3(256), 0, s,
                           frags, n_frag, out, iters);
        break;
    case MCE_LOOP_MXFP8_32X32X64:
        hipLaunchKernelGGL((matrix_core_loop<MCE_LOOP_MXFP8_32X32X64>), dim3(blocks), dim3(256), 0, s,
                           frags, n_frag, out, iters);
        break;
    case MCE_LOOP_MXFP4_32X32X64:
        hipLaunchKernelGGL((matrix_core_loop<MCE_LOOP_MXFP4_32X32X64>), dim3(blocks), dim3(256), 0, s,
                           frags, n_frag, out, iters);
        break;
    case MCE_LOOP_MXFP6_32X32X64:
        hipLaunchKernelGGL((matrix_core_loop<MCE_LOOP_MXFP6_32X32X64>), dim3(blocks), dim3(256), 0, s,
                           frags, n_frag, out, iters);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace mce
