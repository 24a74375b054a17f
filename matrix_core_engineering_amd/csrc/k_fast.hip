// Levels 4-6 of the GEMM ladder for bf16 ("B200 GEMM Optimization Ladder",
// section E steps 5-7), for K-contiguous operands (A row-major, B
// column-major) with 16-byte aligned rows.
//
//   level 4: operands move HBM/L2 -> LDS with direct loads
//            (buffer_load_dwordx4 ... lds: no VGPR staging, bounds-checked by
//            the buffer resource) into XOR-swizzled LDS rows; one stage, so
//            each K tile is loaded, waited for and then consumed.
//   level 5: a ring of STAGES LDS stages with ready/free hand-offs: the
//            loads of K tile kt+STAGES-1 are in flight while tile kt is
//            consumed (prologue fills STAGES-1 stages, steady state, drain).
//   level 6: a persistent grid of one workgroup per CU walks its tiles in an
//            XCD-aware grouped order; the ring runs across tile boundaries,
//            so the next tile's first loads overlap this tile's last K tile
//            and its epilogue.
//
// Workgroup: 256 threads = 4 waves in 2x2; each wave owns (BM/2) x (BN/2) of
// the output as 32x32 matrix-core blocks held in AGPR/VGPR accumulators.
// The matrix-core instruction is fed B as its first operand and A as its
// second, so each lane's 16 accumulators are C^T: lane l holds row
// m = l % 32 and four groups of four consecutive columns, which the
// epilogue writes as 8-byte (bf16) or 16-byte (fp32) vectors.
//
// The ring protocol (one barrier per K tile, no mbarrier on gfx950):
//   ready[s]: each wave waits for its own direct loads into stage s
//             (s_waitcnt vmcnt), then s_barrier: every wave's share landed.
//   free[s]:  each wave finishes its LDS reads of stage s (lgkmcnt(0))
//             before that same barrier; only after it are new loads issued
//             into the stage consumed one K tile earlier.
// ("B200 TMA Pipeline Designer", section E steps 4-7: per-stage ready/free
// protocol, initial phases, prologue / steady state / drain.)
#include "common.hpp"
#include "launch.hpp"
#include "sched.hpp"

namespace mce {
namespace {

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4] = 7, lgkmcnt[11:8] = 15: no wait on those).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) only.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that is also a compiler memory barrier, without the
// vmcnt(0) that a full __syncthreads() fence would add.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Waits until at most `n` K tiles' worth of this wave's direct loads are in
// flight (n in 0..2); loads complete in issue order.
template <int LOADS>
__device__ __forceinline__ void wait_loads_after(int n)
{
    if (n <= 0)
        wait_vmcnt<0>();
    else if (n == 1)
        wait_vmcnt<LOADS>();
    else
        wait_vmcnt<2 * LOADS>();
}

template <int BM, int BN, int STAGES, bool PERSIST>
struct FastBf16 {
    static constexpr int BK = 64;                 // bf16 per LDS row = 128 B = 8 chunks
    static constexpr int ROWB = 128;
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int TI = WM / 32, TJ = WN / 32;
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int NA = BM * 8 / 64 / 4;    // direct loads per wave per K tile (A)
    static constexpr int NB = BN * 8 / 64 / 4;
    static constexpr int LOADS = NA + NB;
    static_assert(STAGES >= 1 && STAGES <= 3, "ring depth");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(STAGES < 3 || 2 * LOADS < 64, "vmcnt range");
    static_assert(NA % 2 == 0 && NB % 2 == 0, "swizzle parity argument needs even load counts");
};

template <int BM, int BN, int STAGES, bool PERSIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fast_bf16(GemmArgs p, int group_m)
{
    using F = FastBf16<BM, BN, STAGES, PERSIST>;
    __shared__ __attribute__((aligned(1024))) char smem[F::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = (p.K + F::BK - 1) / F::BK;
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = xcd_major(wg, nwg);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;
    const int total = my_tiles * nk;

    const uint32_t a_bytes = (uint32_t)(((size_t)(p.M - 1) * p.lda + p.K) * 2);
    const uint32_t b_bytes = (uint32_t)(((size_t)(p.N - 1) * p.ldb + p.K) * 2);
    const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(p.A, a_bytes);
    const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(p.B, b_bytes);

    // Direct-load geometry.  Load t of this wave fills 1024 contiguous LDS
    // bytes = 8 rows; lane l writes row (wave*N + t)*8 + l/8 at physical
    // chunk l%8 and therefore fetches logical chunk (l%8) ^ swz8(row).  For
    // these rows swz8(row) = (l/8) ^ (t & 1) (the row's low three bits are
    // l/8 and bit 3 is the parity of wave*N + t, N even), so only two chunk
    // indices occur per lane.
    const int lrow = lane >> 3;
    const int chunk0 = (lane & 7) ^ lrow;          // even t
    int ld_m0 = 0, ld_n0 = 0;                      // tile being loaded

    auto setup_loads = [&](int tile_id) {
        int tm, tn;
        grouped_tile(tile_id, tiles_m, tiles_n, group_m, tm, tn);
        ld_m0 = __builtin_amdgcn_readfirstlane(tm * BM);
        ld_n0 = __builtin_amdgcn_readfirstlane(tn * BN);
    };

    auto issue = [&](int kt, int stage) {
        const int k0 = kt * F::BK;
        char *base = smem + stage * F::STAGE_BYTES;
#pragma unroll
        for (int t = 0; t < F::NA; ++t) {
            const int row = ld_m0 + (wave * F::NA + t) * 8 + lrow;
            const int kc = k0 + 8 * (chunk0 ^ (t & 1));
            const bool ok = row < p.M && kc < p.K;
            const uint32_t voff = ok ? (uint32_t)(row * p.lda + kc) * 2u : OOB_OFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (lds_ptr_t)(base + (wave * F::NA + t) * 1024), 16, voff, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < F::NB; ++t) {
            const int row = ld_n0 + (wave * F::NB + t) * 8 + lrow;
            const int kc = k0 + 8 * (chunk0 ^ (t & 1));
            const bool ok = row < p.N && kc < p.K;
            const uint32_t voff = ok ? (uint32_t)(row * p.ldb + kc) * 2u : OOB_OFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (lds_ptr_t)(base + F::A_BYTES + (wave * F::NB + t) * 1024), 16, voff, 0,
                0, 0);
        }
    };

    floatx16 acc[F::TI][F::TJ];
    const int swz_lane = swz8(l32);   // rows read by a lane differ by multiples of 32

    auto compute = [&](int stage) {
        const char *As = smem + stage * F::STAGE_BYTES;
        const char *Bs = As + F::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < F::BK / 16; ++ks) {
            const int chunk = ((2 * ks + h) ^ swz_lane) * 16;
            bf16x8 fa[F::TI], fb[F::TJ];
#pragma unroll
            for (int i = 0; i < F::TI; ++i)
                fa[i] = *(const bf16x8 *)(As + (wm * F::WM + i * 32 + l32) * F::ROWB + chunk);
#pragma unroll
            for (int j = 0; j < F::TJ; ++j)
                fb[j] = *(const bf16x8 *)(Bs + (wn * F::WN + j * 32 + l32) * F::ROWB + chunk);
#pragma unroll
            for (int i = 0; i < F::TI; ++i)
#pragma unroll
                for (int j = 0; j < F::TJ; ++j)
                    acc[i][j] = mfma_bf16(fb[j], fa[i], acc[i][j]);
        }
    };

    const bool vec_c = (p.ldc % 4) == 0 &&
                       ((uintptr_t)p.C % (p.c_dtype == OUT_F32 ? 16 : 8)) == 0;

    auto epilogue = [&](int tile_id) {
        int tm, tn;
        grouped_tile(tile_id, tiles_m, tiles_n, group_m, tm, tn);
        const int mbase = tm * BM + wm * F::WM + l32;
        const int nbase = tn * BN + wn * F::WN + 4 * h;
#pragma unroll
        for (int i = 0; i < F::TI; ++i) {
            const int m = mbase + i * 32;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int j = 0; j < F::TJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = nbase + j * 32 + q * 8;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = p.alpha * acc[i][j][4 * q + e];
                    const size_t idx = (size_t)m * p.ldc + n;
                    if (vec_c && n + 3 < p.N) {
                        if (p.c_dtype == OUT_F32) {
                            floatx4 *dst = (floatx4 *)((float *)p.C + idx);
                            if (p.beta != 0.0f) {
                                floatx4 c0 = *dst;
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    v[e] = __builtin_fmaf(p.beta, c0[e], v[e]);
                            }
                            *dst = floatx4{v[0], v[1], v[2], v[3]};
                        } else {
                            u16x4 *dst = (u16x4 *)((uint16_t *)p.C + idx);
                            if (p.beta != 0.0f) {
                                u16x4 c0 = *dst;
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    v[e] = __builtin_fmaf(p.beta, bf16_to_f32(c0[e]), v[e]);
                            }
                            *dst = u16x4{f32_to_bf16_rne(v[0]), f32_to_bf16_rne(v[1]),
                                         f32_to_bf16_rne(v[2]), f32_to_bf16_rne(v[3])};
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N)
                                store_c(p, m, n + e, acc[i][j][4 * q + e]);
                    }
                }
        }
    };

    // ------------------------------------------------------------ K loop
    // Global K-tile index g runs over all tiles of this workgroup: tile
    // g / nk, K tile g % nk, stage g % STAGES.
    auto tile_of = [&](int r) { return PERSIST ? persistent_tile_id(wg, nwg, r) : first; };

    if constexpr (STAGES == 1) {
        for (int g = 0; g < total; ++g) {
            const int kt = g % nk;
            wait_lgkm0();
            barrier();                       // free: every wave finished reading
            if (kt == 0)
                setup_loads(tile_of(g / nk));
            issue(kt, 0);
            wait_vmcnt<0>();
            barrier();                       // ready: every wave's loads landed
            if (kt == 0) {
#pragma unroll
                for (int i = 0; i < F::TI; ++i)
#pragma unroll
                    for (int j = 0; j < F::TJ; ++j)
                        acc[i][j] = zero16();
            }
            compute(0);
            if (kt == nk - 1)
                epilogue(tile_of(g / nk));
        }
    } else {
        // prologue: fill STAGES-1 stages
#pragma unroll
        for (int g = 0; g < STAGES - 1; ++g) {
            if (g < total) {
                if (g % nk == 0)
                    setup_loads(tile_of(g / nk));
                issue(g % nk, g % STAGES);
            }
        }
        for (int g = 0; g < total; ++g) {
            const int kt = g % nk;
            const int after = total - 1 - g;       // K tiles issued after g, capped below
            if (kt == 0)
                wait_vmcnt<0>();                   // also drains the last epilogue's stores
            else
                wait_loads_after<F::LOADS>(after < STAGES - 2 ? after : STAGES - 2);
            wait_lgkm0();
            barrier();                             // ready[g % S], free[(g-1) % S]
            const int gi = g + STAGES - 1;
            if (gi < total) {
                if (gi % nk == 0)
                    setup_loads(tile_of(gi / nk));
                issue(gi % nk, gi % STAGES);
            }
            if (kt == 0) {
#pragma unroll
                for (int i = 0; i < F::TI; ++i)
#pragma unroll
                    for (int j = 0; j < F::TJ; ++j)
                        acc[i][j] = zero16();
            }
            compute(g % STAGES);
            if (kt == nk - 1)
                epilogue(tile_of(g / nk));
        }
    }
}

int g_num_cus = 0;

int num_cus()
{
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            g_num_cus = n;
        else
            g_num_cus = 256;
    }
    return g_num_cus;
}

template <int BM, int BN, int STAGES, bool PERSIST>
hipError_t launch(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    int grid = ntiles;
    if (PERSIST)
        grid = ntiles < num_cus() ? ntiles : num_cus();
    hipLaunchKernelGGL((gemm_fast_bf16<BM, BN, STAGES, PERSIST>), dim3(grid), dim3(256), 0, s, p,
                       group_m);
    return hipGetLastError();
}

} // namespace

hipError_t launch_fast_bf16(int level, const GemmArgs &p, hipStream_t s)
{
    // 256x256 tiles when they give every CU work, 128x128 otherwise
    const bool big = (long)((p.M + 255) / 256) * ((p.N + 255) / 256) >= num_cus();
    switch (level) {
    case 4: return big ? launch<256, 256, 1, false>(p, s) : launch<128, 128, 1, false>(p, s);
    case 5: return big ? launch<256, 256, 2, false>(p, s) : launch<128, 128, 3, false>(p, s);
    case 6: return big ? launch<256, 256, 2, true>(p, s) : launch<128, 128, 3, true>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fast_mxfp8(int, const GemmArgs &, hipStream_t) { return hipErrorInvalidValue; }

} // namespace mce
