// Levels 4-6 of the GEMM ladder ("B200 GEMM Optimization Ladder", section E
// steps 5-7) for K-contiguous operands (A row-major, B column-major) with
// 16-byte aligned rows, in bf16 and in MX block-scaled fp8.
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
// One K tile is 128 bytes of K per operand row: 64 bf16 or 128 E4M3 values,
// i.e. eight 16-byte chunks per LDS row in both formats.  For MX operands
// the E8M0 scales of the tile's four 32-element blocks (one 32-bit word per
// row) travel with the stage, loaded by the same direct-load path, and are
// kept apart from the operand rows ("B200 TMEM Lifecycle Planner", section
// A1 case 2 and section B: scale layout distinct from the accumulator's).
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

struct Bf16Op {
    static constexpr bool MX = false;
    static constexpr int ELT = 2;     // bytes per element
    static constexpr int BK = 64;     // K elements per K tile (128 bytes)
};
struct Mxfp8Op {
    static constexpr bool MX = true;
    static constexpr int ELT = 1;
    static constexpr int BK = 128;
};

template <class Op, int BM, int BN, int STAGES>
struct Geometry {
    static constexpr int ROWB = 128;              // bytes per LDS operand row
    static constexpr int EPC = 16 / Op::ELT;      // K elements per 16-byte chunk
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int TI = WM / 32, TJ = WN / 32;
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    static constexpr int SA_BYTES = Op::MX ? BM * 4 : 0;   // one scale word per row
    static constexpr int SB_BYTES = Op::MX ? BN * 4 : 0;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int NA = BM * 8 / 64 / 4;    // operand direct loads per wave per K tile
    static constexpr int NB = BN * 8 / 64 / 4;
    static constexpr int NSA = Op::MX ? BM / 64 / 4 : 0;   // scale direct loads per wave
    static constexpr int NSB = Op::MX ? BN / 64 / 4 : 0;
    static constexpr int LOADS = NA + NB + NSA + NSB;
    static_assert(STAGES >= 1 && STAGES <= 3, "ring depth");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(STAGES < 3 || 2 * LOADS < 64, "vmcnt range");
    static_assert(NA % 2 == 0 && NB % 2 == 0, "swizzle parity argument needs even load counts");
    static_assert(!Op::MX || (NSA == 1 && NSB == 1), "MX scale staging assumes 256-row tiles");
};

template <class Op, int BM, int BN, int STAGES, bool PERSIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fast(GemmArgs p, int group_m)
{
    using G = Geometry<Op, BM, BN, STAGES>;
    __shared__ __attribute__((aligned(1024))) char smem[G::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = (p.K + Op::BK - 1) / Op::BK;
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = xcd_major(wg, nwg);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;
    const int total = my_tiles * nk;

    const __amdgpu_buffer_rsrc_t rsrc_a =
        make_rsrc(p.A, (uint32_t)(((size_t)(p.M - 1) * p.lda + p.K) * Op::ELT));
    const __amdgpu_buffer_rsrc_t rsrc_b =
        make_rsrc(p.B, (uint32_t)(((size_t)(p.N - 1) * p.ldb + p.K) * Op::ELT));
    const int nblk = (p.K + 31) / 32;   // MX scale blocks per row
    __amdgpu_buffer_rsrc_t rsrc_sa = rsrc_a, rsrc_sb = rsrc_b;
    if constexpr (Op::MX) {
        // scale words are 4-byte aligned (ld % 4 == 0, base % 4 == 0): the last
        // row's final word may extend past ceil(K/32) but not past its word
        const int nblk4 = (nblk + 3) & ~3;
        rsrc_sa = make_rsrc(p.SA, (uint32_t)((size_t)(p.M - 1) * p.ld_sa + nblk4));
        rsrc_sb = make_rsrc(p.SB, (uint32_t)((size_t)(p.N - 1) * p.ld_sb + nblk4));
    }

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
        const int k0 = kt * Op::BK;
        char *base = smem + stage * G::STAGE_BYTES;
#pragma unroll
        for (int t = 0; t < G::NA; ++t) {
            const int row = ld_m0 + (wave * G::NA + t) * 8 + lrow;
            const int kc = k0 + G::EPC * (chunk0 ^ (t & 1));
            const bool ok = row < p.M && kc < p.K;
            const uint32_t voff = ok ? (uint32_t)(row * p.lda + kc) * Op::ELT : OOB_OFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (lds_ptr_t)(base + (wave * G::NA + t) * 1024), 16, voff, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < G::NB; ++t) {
            const int row = ld_n0 + (wave * G::NB + t) * 8 + lrow;
            const int kc = k0 + G::EPC * (chunk0 ^ (t & 1));
            const bool ok = row < p.N && kc < p.K;
            const uint32_t voff = ok ? (uint32_t)(row * p.ldb + kc) * Op::ELT : OOB_OFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (lds_ptr_t)(base + G::A_BYTES + (wave * G::NB + t) * 1024), 16, voff, 0,
                0, 0);
        }
        if constexpr (Op::MX) {
            // one 4-byte word = scale blocks kb0..kb0+3 of one row; lane l of
            // wave w fills row 64w + l of the stage's scale table
            const int kb0 = k0 / 32;
            const int ra = ld_m0 + wave * 64 + lane, rb = ld_n0 + wave * 64 + lane;
            const uint32_t va = ra < p.M ? (uint32_t)(ra * p.ld_sa + kb0) : OOB_OFFSET;
            const uint32_t vb = rb < p.N ? (uint32_t)(rb * p.ld_sb + kb0) : OOB_OFFSET;
            char *sbase = base + G::A_BYTES + G::B_BYTES;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_sa, (lds_ptr_t)(sbase + wave * 256), 4,
                                                     va, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_sb, (lds_ptr_t)(sbase + G::SA_BYTES + wave * 256), 4, vb, 0, 0, 0);
        }
    };

    floatx16 acc[G::TI][G::TJ];
    const int swz_lane = swz8(l32);   // rows read by a lane differ by multiples of 32

    auto compute = [&](int stage, int kt) {
        const char *As = smem + stage * G::STAGE_BYTES;
        const char *Bs = As + G::A_BYTES;
        if constexpr (!Op::MX) {
#pragma unroll
            for (int ks = 0; ks < Op::BK / 16; ++ks) {
                const int chunk = ((2 * ks + h) ^ swz_lane) * 16;
                bf16x8 fa[G::TI], fb[G::TJ];
#pragma unroll
                for (int i = 0; i < G::TI; ++i)
                    fa[i] = *(const bf16x8 *)(As + (wm * G::WM + i * 32 + l32) * G::ROWB + chunk);
#pragma unroll
                for (int j = 0; j < G::TJ; ++j)
                    fb[j] = *(const bf16x8 *)(Bs + (wn * G::WN + j * 32 + l32) * G::ROWB + chunk);
#pragma unroll
                for (int i = 0; i < G::TI; ++i)
#pragma unroll
                    for (int j = 0; j < G::TJ; ++j)
                        acc[i][j] = mfma_bf16(fb[j], fa[i], acc[i][j]);
            }
        } else {
            // Scale words of this K tile: byte b = block kb0 + b.  Blocks at or
            // past ceil(K/32) hold zero data; their byte is forced to 127 (x1)
            // so a stray NaN scale there cannot poison the sum.  Lanes of the
            // upper half-wave supply the odd block of each instruction, so
            // their word is shifted down one byte; op_sel then picks byte 2*ks.
            const int left = nblk - kt * 4;
            uint32_t keep = 0xFFFFFFFFu, force = 0;
            if (left < 4) {
                keep = left <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * left));
                force = 0x7F7F7F7Fu & ~keep;
            }
            const uint32_t *SAs = (const uint32_t *)(Bs + G::B_BYTES);
            const uint32_t *SBs = SAs + BM;
            int sa[G::TI], sb[G::TJ];
#pragma unroll
            for (int i = 0; i < G::TI; ++i)
                sa[i] = (int)(((SAs[wm * G::WM + i * 32 + l32] & keep) | force) >> (8 * h));
#pragma unroll
            for (int j = 0; j < G::TJ; ++j)
                sb[j] = (int)(((SBs[wn * G::WN + j * 32 + l32] & keep) | force) >> (8 * h));
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                // lane (l32, h) holds k = 64ks + 16h + 0..15 and 64ks + 32 + 16h + 0..15
                const int c_lo = ((4 * ks + h) ^ swz_lane) * 16;
                const int c_hi = ((4 * ks + 2 + h) ^ swz_lane) * 16;
                intx8 fa[G::TI], fb[G::TJ];
#pragma unroll
                for (int i = 0; i < G::TI; ++i) {
                    const char *row = As + (wm * G::WM + i * 32 + l32) * G::ROWB;
                    intx4 lo = *(const intx4 *)(row + c_lo), hi = *(const intx4 *)(row + c_hi);
                    fa[i] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int j = 0; j < G::TJ; ++j) {
                    const char *row = Bs + (wn * G::WN + j * 32 + l32) * G::ROWB;
                    intx4 lo = *(const intx4 *)(row + c_lo), hi = *(const intx4 *)(row + c_hi);
                    fb[j] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int i = 0; i < G::TI; ++i)
#pragma unroll
                    for (int j = 0; j < G::TJ; ++j) {
                        if (ks == 0)
                            acc[i][j] = mfma_mxfp8<0>(fb[j], fa[i], acc[i][j], sb[j], sa[i]);
                        else
                            acc[i][j] = mfma_mxfp8<2>(fb[j], fa[i], acc[i][j], sb[j], sa[i]);
                    }
            }
        }
    };

    const bool vec_c = (p.ldc % 4) == 0 &&
                       ((uintptr_t)p.C % (p.c_dtype == OUT_F32 ? 16 : 8)) == 0;

    // Epilogue: out = alpha*acc + beta*C0, written straight from the
    // accumulators.  Interior tiles with vector-aligned C take the branch-free
    // vector path (one uniform test per tile); edge tiles mask per element.
    auto epilogue = [&](int tile_id) {
        int tm, tn;
        grouped_tile(tile_id, tiles_m, tiles_n, group_m, tm, tn);
        const int m_tile = tm * BM, n_tile = tn * BN;
        const int mbase = m_tile + wm * G::WM + l32;
        const int nbase = n_tile + wn * G::WN + 4 * h;
        const bool full = vec_c && m_tile + BM <= p.M && n_tile + BN <= p.N;
        if (full) {
#pragma unroll
            for (int i = 0; i < G::TI; ++i)
#pragma unroll
                for (int j = 0; j < G::TJ; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const size_t idx = (size_t)(mbase + i * 32) * p.ldc + nbase + j * 32 + q * 8;
                        floatx4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                        v *= p.alpha;
                        if (p.c_dtype == OUT_F32) {
                            floatx4 *dst = (floatx4 *)((float *)p.C + idx);
                            if (p.beta != 0.0f)
                                v += p.beta * *dst;
                            *dst = v;
                        } else {
                            u16x4 *dst = (u16x4 *)((uint16_t *)p.C + idx);
                            if (p.beta != 0.0f) {
                                u16x4 c0 = *dst;
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    v[e] += p.beta * bf16_to_f32(c0[e]);
                            }
                            *dst = u16x4{f32_to_bf16_rne(v[0]), f32_to_bf16_rne(v[1]),
                                         f32_to_bf16_rne(v[2]), f32_to_bf16_rne(v[3])};
                        }
                    }
        } else {
#pragma unroll
            for (int i = 0; i < G::TI; ++i)
#pragma unroll
                for (int j = 0; j < G::TJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = mbase + i * 32;
                        const int n = nbase + j * 32 + (r >> 2) * 8 + (r & 3);
                        if (m < p.M && n < p.N)
                            store_c(p, m, n, acc[i][j][r]);
                    }
        }
    };

    // ------------------------------------------------------------ K loop
    // g counts K tiles over all tiles of this workgroup; the stage of K tile
    // g is g % STAGES.  The load side runs STAGES-1 K tiles ahead, possibly
    // into the next tile.
    auto tile_of = [&](int r) { return PERSIST ? persistent_tile_id(wg, nwg, r) : first; };
    int ld_r = 0, ld_kt = 0, ld_stage = 0, ld_left = total;   // next K tile to load
    auto issue_next = [&]() {
        if (ld_left <= 0)
            return;
        if (ld_kt == 0)
            setup_loads(tile_of(ld_r));
        issue(ld_kt, ld_stage);
        --ld_left;
        ld_stage = ld_stage + 1 == STAGES ? 0 : ld_stage + 1;
        if (++ld_kt == nk) {
            ld_kt = 0;
            ++ld_r;
        }
    };

    if constexpr (STAGES > 1) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            issue_next();
    }
    int g = 0, stage = 0;
    for (int r = 0; r < my_tiles; ++r) {
#pragma unroll
        for (int i = 0; i < G::TI; ++i)
#pragma unroll
            for (int j = 0; j < G::TJ; ++j)
                acc[i][j] = zero16();
        for (int kt = 0; kt < nk; ++kt, ++g) {
            if constexpr (STAGES == 1) {
                wait_lgkm0();
                barrier();                         // free: every wave finished reading
                issue_next();
                wait_vmcnt<0>();
                barrier();                         // ready: every wave's loads landed
            } else {
                const int after = total - 1 - g;   // K tiles issued after g (capped)
                if (kt == 0)
                    wait_vmcnt<0>();               // also drains the last epilogue's stores
                else
                    wait_loads_after<G::LOADS>(after < STAGES - 2 ? after : STAGES - 2);
                wait_lgkm0();
                barrier();                         // ready[stage], free[stage - 1]
                issue_next();
            }
            compute(stage, kt);
            stage = stage + 1 == STAGES ? 0 : stage + 1;
        }
        epilogue(tile_of(r));
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

template <class Op, int BM, int BN, int STAGES, bool PERSIST>
hipError_t launch(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    int grid = ntiles;
    if (PERSIST)
        grid = ntiles < num_cus() ? ntiles : num_cus();
    hipLaunchKernelGGL((gemm_fast<Op, BM, BN, STAGES, PERSIST>), dim3(grid), dim3(256), 0, s, p,
                       group_m);
    return hipGetLastError();
}

bool big_tiles(const GemmArgs &p)
{
    return (long)((p.M + 255) / 256) * ((p.N + 255) / 256) >= num_cus();
}

} // namespace

hipError_t launch_fast_bf16(int level, const GemmArgs &p, hipStream_t s)
{
    // 256x256 tiles when they give every CU work, 128x128 otherwise
    const bool big = big_tiles(p);
    switch (level) {
    case 4:
        return big ? launch<Bf16Op, 256, 256, 1, false>(p, s) : launch<Bf16Op, 128, 128, 1, false>(p, s);
    case 5:
        return big ? launch<Bf16Op, 256, 256, 2, false>(p, s) : launch<Bf16Op, 128, 128, 3, false>(p, s);
    case 6:
        return big ? launch<Bf16Op, 256, 256, 2, true>(p, s) : launch<Bf16Op, 128, 128, 3, true>(p, s);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_fast_mxfp8(int level, const GemmArgs &p, hipStream_t s)
{
    switch (level) {
    case 5: return launch<Mxfp8Op, 256, 256, 2, false>(p, s);
    case 6: return launch<Mxfp8Op, 256, 256, 2, true>(p, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mce
