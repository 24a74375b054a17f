// Shared epilogue of the pipelined kernels.
#pragma once

#include "common.hpp"

namespace mce {

typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// Epilogue of one workgroup tile: out = alpha*acc + beta*C0, written straight
// from the accumulators (C^T layout: lane l owns row l % 32 and four groups
// of four consecutive columns per 32x32 block).  Interior tiles take the
// branch-free vector path (one uniform test per tile) with 8- or 16-byte
// accesses at any element alignment (gfx950 global memory accepts them);
// edge tiles mask per element.
// Epilogue variants, chosen on the host per call: EPI_BF16_WHOLE when C is
// bf16, beta == 0, M and N are whole tiles and C rows are 8-byte aligned
// (one branch-free path); EPI_BF16_LDS (gemm_early) the same with 16-byte
// aligned rows, staged through LDS for whole-line stores; EPI_F32_LDS
// (gemm_early) fp32 C of whole tiles with 16-byte aligned rows, any beta,
// staged likewise, and EPI_BF16B_LDS the same for bf16 C with beta != 0
// (8-byte aligned rows); EPI_ANY otherwise.  Keeping the choice out of the
// kernel's run-time branches lets the compiler move accumulators to stores
// one block at a time.
enum { EPI_ANY = 0, EPI_BF16_WHOLE = 1, EPI_BF16_LDS = 2, EPI_F32_LDS = 3, EPI_BF16B_LDS = 4 };

template <int EPI, class G, int BM, int BN>
__device__ __forceinline__ void store_tile(const GemmArgs &p, floatx16 (&acc)[G::TI][G::TJ],
                                           int m_tile, int n_tile, int wm, int wn, int h, int l32)
{
    const int mbase = m_tile + wm * G::WM + l32;
    const int nbase = n_tile + wn * G::WN + 4 * h;
    const bool full = m_tile + BM <= p.M && n_tile + BN <= p.N;
    if (EPI == EPI_BF16_WHOLE) {
        // the common case: one row pointer per 32-row block, columns as
        // immediate offsets, no C read
#pragma unroll
        for (int i = 0; i < G::TI; ++i) {
            uint16_t *row = (uint16_t *)p.C + (size_t)(mbase + i * 32) * p.ldc + nbase;
#pragma unroll
            for (int j = 0; j < G::TJ; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx16 &a = acc[i][j];
                    *(u16x4 *)(row + j * 32 + q * 8) =
                        u16x4{f32_to_bf16_rne(p.alpha * a[4 * q]), f32_to_bf16_rne(p.alpha * a[4 * q + 1]),
                              f32_to_bf16_rne(p.alpha * a[4 * q + 2]), f32_to_bf16_rne(p.alpha * a[4 * q + 3])};
                }
                // one 32x32 block at a time: keeps the scheduler from pulling
                // every accumulator into VGPRs at once
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else if (full && p.c_dtype == OUT_BF16 && p.beta == 0.0f) {
#pragma unroll
        for (int i = 0; i < G::TI; ++i) {
            uint16_t *row = (uint16_t *)p.C + (size_t)(mbase + i * 32) * p.ldc + nbase;
#pragma unroll
            for (int j = 0; j < G::TJ; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx16 &a = acc[i][j];
                    const u16x4 v = {f32_to_bf16_rne(p.alpha * a[4 * q]), f32_to_bf16_rne(p.alpha * a[4 * q + 1]),
                                     f32_to_bf16_rne(p.alpha * a[4 * q + 2]),
                                     f32_to_bf16_rne(p.alpha * a[4 * q + 3])};
                    __builtin_memcpy(row + j * 32 + q * 8, &v, 8);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else if (full && p.c_dtype == OUT_F32) {
#pragma unroll
        for (int i = 0; i < G::TI; ++i) {
            float *row = (float *)p.C + (size_t)(mbase + i * 32) * p.ldc + nbase;
#pragma unroll
            for (int j = 0; j < G::TJ; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx16 &a = acc[i][j];
                    floatx4 v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                    v *= p.alpha;
                    float *dst = row + j * 32 + q * 8;
                    if (p.beta != 0.0f) {
                        floatx4 c0;
                        __builtin_memcpy(&c0, dst, 16);
                        v += p.beta * c0;
                    }
                    __builtin_memcpy(dst, &v, 16);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else if (full) {
        // bf16 output with beta != 0
#pragma unroll
        for (int i = 0; i < G::TI; ++i) {
            uint16_t *row = (uint16_t *)p.C + (size_t)(mbase + i * 32) * p.ldc + nbase;
#pragma unroll
            for (int j = 0; j < G::TJ; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx16 &a = acc[i][j];
                    uint16_t *dst = row + j * 32 + q * 8;
                    u16x4 c0, o;
                    __builtin_memcpy(&c0, dst, 8);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = f32_to_bf16_rne(__builtin_fmaf(p.beta, bf16_to_f32(c0[e]), p.alpha * a[4 * q + e]));
                    __builtin_memcpy(dst, &o, 8);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // edge tile: each lane's groups of four columns that lie inside C
        // take the vector path, the one that crosses the N edge goes per
        // element; either way with store_c's operations, so an element's
        // value does not depend on which path stored it
#pragma unroll
        for (int i = 0; i < G::TI; ++i)
#pragma unroll
            for (int j = 0; j < G::TJ; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = mbase + i * 32;
                    const int n = nbase + j * 32 + q * 8;
                    const floatx16 &a = acc[i][j];
                    if (m < p.M && n + 4 <= p.N) {
                        const size_t idx = (size_t)m * p.ldc + n;
                        if (p.c_dtype == OUT_F32) {
                            float *dst = (float *)p.C + idx;
                            floatx4 v = {p.alpha * a[4 * q], p.alpha * a[4 * q + 1], p.alpha * a[4 * q + 2],
                                         p.alpha * a[4 * q + 3]};
                            if (p.beta != 0.0f) {
                                floatx4 c0;
                                __builtin_memcpy(&c0, dst, 16);
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    v[e] = __builtin_fmaf(p.beta, c0[e], v[e]);
                            }
                            __builtin_memcpy(dst, &v, 16);
                        } else {
                            uint16_t *dst = (uint16_t *)p.C + idx;
                            u16x4 c0, o;
                            if (p.beta != 0.0f)
                                __builtin_memcpy(&c0, dst, 8);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float v = p.alpha * a[4 * q + e];
                                if (p.beta != 0.0f)
                                    v = __builtin_fmaf(p.beta, bf16_to_f32(c0[e]), v);
                                o[e] = f32_to_bf16_rne(v);
                            }
                            __builtin_memcpy(dst, &o, 8);
                        }
                    } else if (m < p.M) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N)
                                store_c(p, m, n + e, a[4 * q + e]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    }
}

} // namespace mce

namespace mce {

// Epilogue staged through LDS for any C (fp32 or bf16, any beta, leading
// dimension or edge): each wave converts 32 rows of its tile at a time
// (alpha * acc, fp32) into its own buffer, reads them back so that each
// lane holds a 16-byte piece of a row, and then reads C (beta != 0),
// combines and stores by those pieces.  A store instruction then covers 256
// contiguous bytes of each of four rows (fp32) instead of 32 bytes of each
// of 32 rows.  LDS cycles (measured on gfx950): a 16-byte write serves 8
// lanes, and the 272-byte pitch puts 8 consecutive rows in 8 different
// 16-byte slots of a 128-byte window; a 16-byte read serves the 16 lanes of
// quad group parity((lane >> 2) & 7) of a 32-lane half, so each such group
// reads one whole row.  The caller's LDS must be free (no other wave may
// still read it) and is free again when every wave has returned.
constexpr int EPI_F32_PITCH = 272;
constexpr int EPI_F32_WAVE_BYTES = 32 * EPI_F32_PITCH;

// out = v + beta * C0 for one element whose alpha * acc is v
__device__ __forceinline__ void store_c_scaled(const GemmArgs &p, int row, int col, float v)
{
    const size_t idx = (size_t)row * p.ldc + col;
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

template <class G>
__device__ __forceinline__ void store_tile_staged(const GemmArgs &p, floatx16 (&acc)[G::TI][G::TJ],
                                                  int m_tile, int n_tile, int wm, int wn, int lane,
                                                  char *buf)
{
    static_assert(G::WN == 64, "rows of 64 fp32 = 256 bytes");
    const int h = lane >> 5, l32 = lane & 31;
    // read-back position: the 16 lanes of one read cycle share a row
    const int qh = (lane >> 2) & 7;
    const int rrow = 2 * (lane >> 5) + (__builtin_popcount(qh) & 1);
    const int rpiece = 4 * (qh >> 1) + (lane & 3);
    const int n0 = n_tile + wn * G::WN + rpiece * 4;
#pragma unroll
    for (int i = 0; i < G::TI; ++i) {
        // lane (l32, h) holds row l32, columns 32j + 8q + 4h .. +3
#pragma unroll
        for (int j = 0; j < G::TJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const floatx16 &a = acc[i][j];
                floatx4 v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                v *= p.alpha;
                *(floatx4 *)(buf + l32 * EPI_F32_PITCH + (j * 32 + q * 8 + h * 4) * 4) = v;
            }
        __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): this wave's writes landed
        const int m0 = m_tile + wm * G::WM + i * 32;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int row = s * 4 + rrow;
            const int m = m0 + row;
            floatx4 v = *(const floatx4 *)(buf + row * EPI_F32_PITCH + rpiece * 16);
            if (m < p.M && n0 + 4 <= p.N) {
                if (p.c_dtype == OUT_F32) {
                    float *dst = (float *)p.C + (size_t)m * p.ldc + n0;
                    if (p.beta != 0.0f) {
                        floatx4 c0;
                        __builtin_memcpy(&c0, dst, 16);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = __builtin_fmaf(p.beta, c0[e], v[e]);
                    }
                    __builtin_memcpy(dst, &v, 16);
                } else {
                    uint16_t *dst = (uint16_t *)p.C + (size_t)m * p.ldc + n0;
                    u16x4 o;
                    if (p.beta != 0.0f) {
                        u16x4 c0;
                        __builtin_memcpy(&c0, dst, 8);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[e] = f32_to_bf16_rne(__builtin_fmaf(p.beta, bf16_to_f32(c0[e]), v[e]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[e] = f32_to_bf16_rne(v[e]);
                    }
                    __builtin_memcpy(dst, &o, 8);
                }
            } else if (m < p.M) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n0 + e < p.N)
                        store_c_scaled(p, m, n0 + e, v[e]);
            }
        }
        // the next round's writes may not overtake these reads
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_sched_barrier(0);
    }
}

} // namespace mce
