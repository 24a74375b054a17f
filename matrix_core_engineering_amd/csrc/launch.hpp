// Host-side launchers of every kernel family; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace mce {

// Levels 1-3 (bf16): generic synchronous copies; level selects the grid.
hipError_t launch_simple_bf16(int level, const GemmArgs &p, hipStream_t s);
// Level 3 (MX, any element format): generic synchronous copies, K-contiguous
// operands.
hipError_t launch_simple_mx(const GemmArgs &p, hipStream_t s);
// C <- beta * C (alpha == 0 or K == 0).
hipError_t launch_scale_c(const GemmArgs &p, hipStream_t s);

// Levels 4-7 (bf16): direct global->LDS loads of K-contiguous operands.
// Returns hipErrorInvalidValue if the level has no kernel.
hipError_t launch_fast_bf16(int level, const GemmArgs &p, hipStream_t s);
// Levels 5-7 (MX E4M3 and E5M2; p.mx_fmt) and 5-6 (E2M1, E2M3, E3M2):
// direct loads, as for bf16; dispatches to the per-format launchers below.
hipError_t launch_fast_mx(int level, const GemmArgs &p, hipStream_t s);
hipError_t launch_fast_e4m3(int level, const GemmArgs &p, hipStream_t s);
hipError_t launch_fast_e5m2(int level, const GemmArgs &p, hipStream_t s);
hipError_t launch_fast_fp4(int level, const GemmArgs &p, hipStream_t s);
hipError_t launch_fast_fp6(int level, const GemmArgs &p, hipStream_t s);
// 8-bit MX levels 5-6 with an MN-major operand (A column-major or B
// row-major), through the LDS transpose loads.
hipError_t launch_fast_mx_mn(int level, const GemmArgs &p, hipStream_t s);
// bf16 levels 5-6 when M or N is at most 64 (K-contiguous operands, K a
// multiple of 64 and at least 512): 32-wide tiles along the long side, the
// eight waves of a workgroup splitting K.
bool skinny_eligible(const GemmArgs &p);
hipError_t launch_skinny_bf16(const GemmArgs &p, hipStream_t s);
// 8-bit MX (E4M3 / E5M2) operands, K-contiguous, with a short side
bool skinny_mx_eligible(const GemmArgs &p);
hipError_t launch_skinny_mx(const GemmArgs &p, hipStream_t s);
// Levels 5-6 (bf16) for operands the direct-load kernels cannot take: any
// layout, alignment and K, through registers.
hipError_t launch_general_bf16(int level, const GemmArgs &p, hipStream_t s);

// Fused attention forward (bf16 Q, K, V of batch x heads x seq x dim, dim
// contiguous; O the same shape as Q).  scale_log2 = scale * log2(e).
struct AttnArgs {
    int batch, heads, seq_q, seq_k, dim;
    const uint16_t *Q, *K, *V;
    void *O;
    float scale_log2;
    int causal, o_dtype;
};
// Returns hipErrorInvalidValue for a head dimension other than 64 or 128.
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);

// The matrix-core ceiling loop (shape: MCE_LOOP_*); returns
// hipErrorInvalidValue for an unknown shape.
hipError_t launch_matrix_core_loop(int shape, const void *frags, int n_frag, float *out, int blocks,
                                   int iters, hipStream_t s);

} // namespace mce
