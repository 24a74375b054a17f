// Kernel templates of levels 4-7 of the GEMM ladder (the launchers for each
// operand format are instantiated in k_fast_*.hip, one translation unit per
// format so that they compile in parallel).
//
// Levels 4-6 of the GEMM ladder ("B200 GEMM Optimization Ladder", section E
// steps 5-7) for K-contiguous operands (A row-major, B column-major) with
// 16-byte aligned rows, in bf16 and in MX block-scaled fp8.
//
//   level 4: operands move HBM/L2 -> LDS with direct loads
//            (buffer_load_dwordx4 ... lds: no VGPR staging, bounds-checked by
//            the buffer resource) into XOR-swizzled LDS rows; one stage, so
//            each K tile is loaded, waited for and then consumed.
//   level 5: a ring of LDS stages with ready/free hand-offs: the loads of
//            later K tiles are in flight while tile kt is consumed (prologue
//            fills the ring, steady state, drain).  The tuned form for
//            256x256 tiles is gemm_early below; gemm_fast covers the rest.
//   level 6: a persistent grid of one workgroup per CU walks its tiles in an
//            XCD-aware grouped order; the ring runs across tile boundaries,
//            so the next tile's first loads overlap this tile's last K tile
//            and its epilogue.
//
// One K tile is 128 bytes of K per operand row: 64 bf16 or 128 E4M3 values,
// i.e. eight 16-byte chunks per LDS row in both formats (level 7 uses
// 64-byte rows).  For MX operands
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
// epilogue writes as 8-byte (bf16) or 16-byte (fp32) vectors.  Whole bf16
// 256x256 tiles instead run the 16x16x32 instruction (Bf16Ring64S16: 16x16
// blocks, four accumulators per lane and block, row l % 16, columns
// 4(l/16) .. +3), which sustains more flops per clock at the chip's power
// limit.
//
// The ring protocol (one barrier per K tile, no mbarrier on gfx950):
//   ready[s]: each wave waits for its own direct loads into stage s
//             (s_waitcnt vmcnt), then s_barrier: every wave's share landed.
//   free[s]:  each wave finishes its LDS reads of stage s (lgkmcnt(0))
//             before that same barrier; only after it are new loads issued
//             into the stage consumed one K tile earlier.
// ("B200 TMA Pipeline Designer", section E steps 4-7: per-stage ready/free
// protocol, initial phases, prologue / steady state / drain.)
#pragma once

#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "ring_plan.hpp"
#include "sched.hpp"

#include <type_traits>

namespace mce {
namespace {

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4] = 7, lgkmcnt[11:8] = 15: no wait on those).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The lane index (0..63) computed where it is written: a volatile asm
// statement the compiler neither hoists nor merges with an earlier copy.
__device__ __forceinline__ int lane_id_here()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
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
    static constexpr int FMT = MX_E4M3;   // element format (instruction format code)
    static constexpr int ELT = 1;
    static constexpr int BK = 128;
};
struct E5m2Op : Mxfp8Op {
    static constexpr int FMT = MX_E5M2;
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

// Whole bf16 tiles through LDS: each wave converts two 32x32 blocks at a
// time (32 rows x 64 columns = 32 rows of 128 bytes; RR = 16: half of the
// rows per round, for kernels with less LDS to spare) into its own LDS
// buffer, then reads them back so that eight consecutive lanes hold one
// row's 128 bytes, and stores 16 bytes per lane: every store instruction
// writes eight whole 128-byte lines of C instead of 32 rows x 16 bytes.
// The buffer's row pitch is 144 bytes, so the 64 lanes' 8-byte writes of a
// block fill every bank exactly twice.  Stores count in vmcnt like loads;
// the next ready wait drains them.
constexpr int EPI_PITCH = 144;                           // bytes per staged row
template <int RR> constexpr int epi_wave_bytes() { return RR * EPI_PITCH; }

template <class G, int BM, int BN, int RR>
__device__ __forceinline__ void store_tile_lds(const GemmArgs &p, floatx16 (&acc)[G::TI][G::TJ],
                                               int m_tile, int n_tile, int wm, int wn, int lane,
                                               char *buf, bool full)
{
    static_assert(G::TJ % 2 == 0, "blocks staged in pairs");
    static_assert(RR == 8 || RR == 16 || RR == 32, "rows per round");
    const int h = lane >> 5, l32 = lane & 31;
    const int rrow = lane >> 3, rchunk = lane & 7;       // read-back position
#pragma unroll
    for (int i = 0; i < G::TI; ++i)
#pragma unroll
        for (int jp = 0; jp < G::TJ / 2; ++jp)
#pragma unroll
            for (int half = 0; half < 32 / RR; ++half) {
            // lane (l32, h) holds row l32, columns 8q + 4h .. +3 of each block
            if (RR == 32 || l32 / RR == half) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const floatx16 &a = acc[i][2 * jp + jj];
                        *(u16x4 *)(buf + (l32 % RR) * EPI_PITCH + jj * 64 + q * 16 + h * 8) =
                            u16x4{f32_to_bf16_rne(p.alpha * a[4 * q]), f32_to_bf16_rne(p.alpha * a[4 * q + 1]),
                                  f32_to_bf16_rne(p.alpha * a[4 * q + 2]),
                                  f32_to_bf16_rne(p.alpha * a[4 * q + 3])};
                    }
            }
            wait_lgkm0();
            const int mr = m_tile + wm * G::WM + i * 32 + half * RR;     // the round's first row
            const int nc = n_tile + wn * G::WN + jp * 64 + rchunk * 8;   // this lane's first column
            uint16_t *c0 = (uint16_t *)p.C + (size_t)mr * p.ldc + nc;
            if (full) {
#pragma unroll
                for (int s = 0; s < RR / 8; ++s) {
                    const int row = s * 8 + rrow;
                    const intx4 v = *(const intx4 *)(buf + row * EPI_PITCH + rchunk * 16);
                    *(intx4 *)(c0 + (size_t)row * p.ldc) = v;
                }
            } else {
                // a tile crossing the M or N edge: rows past M are skipped,
                // a piece crossing N is stored per element
#pragma unroll
                for (int s = 0; s < RR / 8; ++s) {
                    const int row = s * 8 + rrow;
                    const intx4 v = *(const intx4 *)(buf + row * EPI_PITCH + rchunk * 16);
                    if (mr + row < p.M) {
                        uint16_t *dst = c0 + (size_t)row * p.ldc;
                        if (nc + 8 <= p.N) {
                            *(intx4 *)dst = v;
                        } else {
                            const u16x8 e8 = __builtin_bit_cast(u16x8, v);
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                if (nc + e < p.N)
                                    dst[e] = e8[e];
                        }
                    }
                }
            }
            // the next round's writes may not overtake these reads
            wait_lgkm0();
            __builtin_amdgcn_sched_barrier(0);
        }
}

// Whole fp32 tiles through the same buffers: a block (32 rows x 32 columns
// = 32 rows of 128 bytes) per round, RR rows at a time.  Lane (l32, h)
// writes its four 16-byte pieces of row l32 (columns 8q + 4h .. +3) at the
// 144-byte pitch (eight consecutive rows fall in eight distinct 16-byte
// slots, so the writes are conflict-free); the read-back and the stores are
// those above, with C read at the same 16-byte pieces when beta != 0.  The
// arithmetic is the register path's (alpha * acc, then + beta * C0), so the
// results are bitwise those of EPI_ANY.  BF16B: bf16 C with beta != 0, the
// fp32 alpha * acc staged the same way, then each lane's four elements
// combined with C0 and rounded as the register path does, 8-byte pieces.
template <class G, int BM, int BN, int RR, bool BF16B = false>
__device__ __forceinline__ void store_tile_lds_f32(const GemmArgs &p, floatx16 (&acc)[G::TI][G::TJ],
                                                   int m_tile, int n_tile, int wm, int wn, int lane,
                                                   char *buf, bool full)
{
    static_assert(RR == 8 || RR == 16 || RR == 32, "rows per round");
    const int h = lane >> 5, l32 = lane & 31;
    const int rrow = lane >> 3, rchunk = lane & 7;       // read-back position
#pragma unroll
    for (int i = 0; i < G::TI; ++i)
#pragma unroll
        for (int j = 0; j < G::TJ; ++j)
#pragma unroll
            for (int half = 0; half < 32 / RR; ++half) {
            if (RR == 32 || l32 / RR == half) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx16 &a = acc[i][j];
                    floatx4 v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                    v *= p.alpha;
                    *(floatx4 *)(buf + (l32 % RR) * EPI_PITCH + q * 32 + h * 16) = v;
                }
            }
            wait_lgkm0();
            const int mr = m_tile + wm * G::WM + i * 32 + half * RR;     // the round's first row
            const int nc = n_tile + wn * G::WN + j * 32 + rchunk * 4;    // this lane's first column
            const size_t e0 = (size_t)mr * p.ldc + nc;
#pragma unroll
            for (int s = 0; s < RR / 8; ++s) {
                const int row = s * 8 + rrow;
                floatx4 v = *(const floatx4 *)(buf + row * EPI_PITCH + rchunk * 16);
                const bool in = full || (mr + row < p.M && nc + 4 <= p.N);
                if (in) {
                    if constexpr (BF16B) {
                        u16x4 *dst = (u16x4 *)((uint16_t *)p.C + e0 + (size_t)row * p.ldc);
                        const u16x4 c = *dst;
                        u16x4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[e] = f32_to_bf16_rne(__builtin_fmaf(p.beta, bf16_to_f32(c[e]), v[e]));
                        *dst = o;
                    } else {
                        floatx4 *dst = (floatx4 *)((float *)p.C + e0 + (size_t)row * p.ldc);
                        if (p.beta != 0.0f) {
                            const floatx4 c = *dst;
                            v += p.beta * c;
                        }
                        *dst = v;
                    }
                } else if (mr + row < p.M) {
                    // a piece crossing the N edge, per element, the same
                    // operations (store_c: alpha * acc, then fma with C0)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (nc + e >= p.N)
                            continue;
                        const size_t idx = e0 + (size_t)row * p.ldc + e;
                        if constexpr (BF16B) {
                            uint16_t *c = (uint16_t *)p.C;
                            c[idx] = f32_to_bf16_rne(__builtin_fmaf(p.beta, bf16_to_f32(c[idx]), v[e]));
                        } else {
                            float *c = (float *)p.C;
                            c[idx] = p.beta != 0.0f ? __builtin_fmaf(p.beta, c[idx], v[e]) : v[e];
                        }
                    }
                }
            }
            // the next round's writes may not overtake these reads
            wait_lgkm0();
            __builtin_amdgcn_sched_barrier(0);
        }
}

// The same for 16x16 blocks (the 16x16x32 format): with the B operand fed
// first, lane l holds row l % 16 and columns 4(l/16) .. +3 of each block.
// Per block row and group of four blocks (16 rows x 64 columns), every lane
// writes its four 8-byte pieces into the wave's buffer, then eight
// consecutive lanes read back one row's 128 bytes and store 16 bytes each.
template <class G, int TI, int TJ>
__device__ __forceinline__ void store_tile_lds16(const GemmArgs &p, floatx4 (&acc)[TI][TJ], int m_tile,
                                                 int n_tile, int wm, int wn, int lane, char *buf)
{
    static_assert(TJ % 4 == 0, "blocks staged in fours");
    const int l16 = lane & 15, q = lane >> 4;
    const int rrow = lane >> 3, rchunk = lane & 7;       // read-back position
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int jq = 0; jq < TJ / 4; ++jq) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const floatx4 &a = acc[i][4 * jq + jj];
                *(u16x4 *)(buf + l16 * EPI_PITCH + jj * 32 + q * 8) =
                    u16x4{f32_to_bf16_rne(p.alpha * a[0]), f32_to_bf16_rne(p.alpha * a[1]),
                          f32_to_bf16_rne(p.alpha * a[2]), f32_to_bf16_rne(p.alpha * a[3])};
            }
            wait_lgkm0();
            uint16_t *c0 = (uint16_t *)p.C + (size_t)(m_tile + wm * G::WM + i * 16) * p.ldc + n_tile +
                           wn * G::WN + jq * 64 + rchunk * 8;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int row = s * 8 + rrow;
                const intx4 v = *(const intx4 *)(buf + row * EPI_PITCH + rchunk * 16);
                *(intx4 *)(c0 + (size_t)row * p.ldc) = v;
            }
            // the next round's writes may not overtake these reads
            wait_lgkm0();
            __builtin_amdgcn_sched_barrier(0);
        }
}

// Rows per round of an LDS-staged epilogue that fits beside `lds` bytes of
// ring for four waves (0: none fits).
constexpr int staged_rr(int lds)
{
    return lds + 4 * epi_wave_bytes<32>() <= 160 * 1024   ? 32
           : lds + 4 * epi_wave_bytes<16>() <= 160 * 1024 ? 16
           : lds + 4 * epi_wave_bytes<8>() <= 160 * 1024  ? 8
                                                            : 0;
}

template <class Op, int BM, int BN, int STAGES, bool PERSIST, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fast(GemmArgs p, int group_m)
{
    using G = Geometry<Op, BM, BN, STAGES>;
    // the LDS-staged epilogues' buffers (one per wave) follow the ring
    constexpr bool STAGED = EPI == EPI_BF16_LDS || EPI == EPI_F32_LDS || EPI == EPI_BF16B_LDS;
    constexpr int ERR = staged_rr(G::LDS_BYTES);
    static_assert(!STAGED || ERR > 0, "LDS budget of the staged epilogue");
    constexpr int EPI_BYTES = STAGED ? 4 * epi_wave_bytes<(ERR > 0 ? ERR : 8)>() : 0;
    __shared__ __attribute__((aligned(1024))) char smem[G::LDS_BYTES + EPI_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = (p.K + Op::BK - 1) / Op::BK;
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = wg_slot(wg, nwg, p.xcd_order);
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
                            acc[i][j] = mfma_mx<Op::FMT, 0>(fb[j], fa[i], acc[i][j], sb[j], sa[i]);
                        else
                            acc[i][j] = mfma_mx<Op::FMT, 2>(fb[j], fa[i], acc[i][j], sb[j], sa[i]);
                    }
            }
        }
    };

    auto epilogue = [&](int tile_id) {
        int tm, tn;
        grouped_tile(tile_id, tiles_m, tiles_n, group_m, tm, tn);
        if constexpr (STAGED) {
            constexpr int RR = ERR > 0 ? ERR : 8;
            const bool full = (tm + 1) * BM <= p.M && (tn + 1) * BN <= p.N;
            char *ebuf = smem + G::LDS_BYTES + wave * epi_wave_bytes<RR>();
            if constexpr (EPI == EPI_BF16_LDS)
                store_tile_lds<G, BM, BN, RR>(p, acc, tm * BM, tn * BN, wm, wn, lane_id_here(), ebuf, full);
            else
                store_tile_lds_f32<G, BM, BN, RR, EPI == EPI_BF16B_LDS>(p, acc, tm * BM, tn * BN, wm, wn,
                                                                       lane_id_here(), ebuf, full);
        } else {
            store_tile<EPI, G, BM, BN>(p, acc, tm * BM, tn * BN, wm, wn, h, l32);
        }
    };

    // ------------------------------------------------------------ K loop
    // g counts K tiles over all tiles of this workgroup; the stage of K tile
    // g is g % STAGES.  The load side runs STAGES-1 K tiles ahead, possibly
    // into the next tile.
    auto tile_of = [&](int r) { return PERSIST ? persistent_tile_id(wg, nwg, r, p.xcd_order) : first; };
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

// ---------------------------------------------------------------------------
// Pieces shared by the pipelined kernels below: scheduling-group masks for
// fixing the interleave of matrix-core instructions with LDS reads and
// direct loads inside a barrier-free region, the K-tile formats, and the
// stage geometry.  Every load address is a branch-free select of per-tile
// offsets computed once per tile (row bounds folded in), with K in the
// scalar offset.
constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100;

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order:
// a loop whose trip index is a compile-time constant in the body.
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// 64-byte LDS rows (the role-specialised kernel)
struct Bf16Ring {                     // 64-byte rows
    static constexpr bool MX = false, SG = false;
    static constexpr int ELT = 2;
    static constexpr int BK = 32;     // K elements per K tile
    static constexpr int NKS = 2;     // 32x32x16 k-steps per K tile
};
struct Mxfp8Ring {                    // 64-byte rows
    static constexpr bool MX = true, SG = false;
    static constexpr int FMT = MX_E4M3;
    static constexpr int ELT = 1;
    static constexpr int BK = 64;
    static constexpr int NKS = 1;     // one 32x32x64 k-step per K tile
};
struct E5m2Ring : Mxfp8Ring {         // E5M2: the E4M3 layout with format code 1
    static constexpr int FMT = MX_E5M2;
};

// Waits until at most n K tiles' loads (n <= 3) of LOADS direct loads each
// are still in flight.
template <int LOADS>
__device__ __forceinline__ void wait_tiles_after(int n)
{
    if (n <= 0)
        wait_vmcnt<0>();
    else if (n == 1)
        wait_vmcnt<LOADS>();
    else if (n == 2)
        wait_vmcnt<2 * LOADS>();
    else
        wait_vmcnt<3 * LOADS>();
}

// ---------------------------------------------------------------------------
// Levels 5 and 6, early release: a two-stage ring of K tiles with 128-byte
// LDS rows (64 bf16 or 128 E4M3 values per row), so every direct load moves
// whole 128-byte lines; on MI355X a direct load of 64-byte row segments
// delivers about half the bytes per clock of one of 128-byte rows.  With
// only two stages the next-but-one K tile can be loaded only once the stage
// is released, so each wave reads the whole K tile's fragments into
// registers during its first matrix-core instructions and releases the
// stage early.  Two barriers per K tile g (stage s = g % 2):
//   phase A  the first AM matrix-core instructions; the rest of the K
//            tile's fragments read;
//   barrier 1 (free):  every wave's reads of stage s are in registers;
//   phase X  the next XM instructions; the loads of K tile g+2 into stage
//            s begin;
//   barrier 2 (ready): each wave waited for its loads of K tile g+1;
//   phase Y  the last matrix-core instructions of K tile g; K tile g+1's
//            first fragments (and MX scales) read; the remaining loads.
// The loads of a K tile spread over phases X and Y of one iteration and have
// until barrier 2 of the next to land.  Needs at least two K tiles and K a
// multiple of the K tile.
// The formats, the stage geometry and the step tables of prologue and K-tile
// iteration are in ring_plan.hpp, which the host model of the ring protocol
// (tests/ring_model.cpp) replays.
template <class Op, int BM, int BN, bool PERSIST, int EPI>
__global__ __launch_bounds__(64 * Op::WAVES) __attribute__((amdgpu_waves_per_eu(Op::WAVES / 4, Op::WAVES / 4)))
void gemm_early(GemmArgs p, int group_m)
{
    using P = EarlyPlan<Op, BM, BN>;
    using G = typename P::G;
    constexpr int NKS = P::NKS;
    constexpr bool S16 = P::S16;
    constexpr int BLK = P::BLK, TI = P::TI, TJ = P::TJ, NM = P::NM, RPF = P::RPF;
    constexpr int BPK = P::BPK, GK = P::GK, UNR = P::UNR, SW = P::SW, FRAG_READS = P::FRAG_READS;
    constexpr int AM = P::AM, XM = P::XM, YM = P::YM;
    constexpr int LX = P::LX, LY = P::LY, LA = P::LA, YA = P::YA, YK = P::YK;
    static_assert(!S16 || EPI == EPI_BF16_LDS, "16x16 blocks: whole bf16 tiles staged through LDS");
    // LDS: the two stages, then (scale groups) two buffers of 16 bytes per
    // A and B row, then (staged epilogue) one buffer per wave
    constexpr int SG_BYTES = P::SG_BYTES;
    constexpr int WAVES = P::WAVES;
    // rows per round of the LDS-staged epilogue: what the LDS left over holds
    constexpr int EPI_RR = WAVES == 8 ? (Op::SG ? 8 : 16) : (Op::SG || S16 ? 16 : 32);
    constexpr int EPI_BYTES =
        EPI == EPI_BF16_LDS || EPI == EPI_F32_LDS || EPI == EPI_BF16B_LDS ? WAVES * epi_wave_bytes<EPI_RR>() : 0;
    static_assert(G::LDS_BYTES + SG_BYTES + EPI_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[G::LDS_BYTES + SG_BYTES + EPI_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = (p.K + Op::BK - 1) / Op::BK;            // >= 2 (host guarantees)
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = wg_slot(wg, nwg, p.xcd_order);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;

    const int nblk = (p.K * Op::EPU + 31) / 32;            // MX scale blocks per row

    auto tile_of = [&](int r) { return PERSIST ? persistent_tile_id(wg, nwg, r, p.xcd_order) : first; };

    // Direct-load addressing.  Each tile gets its own buffer resources (A
    // and B rows of the tile, MX scale rows) whose record count ends at the
    // tile's last valid row, so rows past M or N read as zeros; a lane's
    // offset inside the tile (row and chunk) is fixed for the whole kernel,
    // and K moves in the scalar offset.  No address arithmetic per load.
    // Load t of this wave fills 1 KiB = 8 rows of 128 bytes: lane l writes
    // row (wave*N + t)*8 + l/8 at physical chunk l%8; swz8(row) = (l/8) ^
    // (t&1) (bit 3 of the row is the parity of wave*N + t, N even).
    const int lrow = lane >> 3;
    // (16x16x32 format: swz8h(row) = swz8h(lrow), the same for every load)
    const int kc_even = ((lane & 7) ^ (S16 ? swz8h(lrow) : lrow)) * G::EPC;
    const int kc_odd = ((lane & 7) ^ (S16 ? swz8h(lrow) : lrow ^ 1)) * G::EPC;
    uint32_t va[G::NA], vb[G::NB];
#pragma unroll
    for (int t = 0; t < G::NA; ++t)
        va[t] = (uint32_t)(((wave * G::NA + t) * G::RPL + lrow) * p.lda + ((t & 1) ? kc_odd : kc_even)) *
                Op::ELT;
#pragma unroll
    for (int t = 0; t < G::NB; ++t)
        vb[t] = (uint32_t)(((wave * G::NB + t) * G::RPL + lrow) * p.ldb + ((t & 1) ? kc_odd : kc_even)) *
                Op::ELT;
    // scale rows: with eight waves, waves 0-3 load the A rows' scale words
    // and waves 4-7 the B rows'
    const int srow = (WAVES == 8 ? (wave & 3) : wave) * 64 + lane;
    const uint32_t vsa = (uint32_t)(srow * p.ld_sa);
    const uint32_t vsb = (uint32_t)(srow * p.ld_sb);

    // Base and record count of the r-th tile's resources (A rows, B rows,
    // MX scale rows); past the last tile every record count is zero (loads
    // fetch nothing and write zeros).
    struct TileSpan {
        const char *a, *b, *sa, *sb;
        uint32_t na, nb, nsa, nsb;
    };
    auto tile_span = [&](int r) {
        TileSpan t{(const char *)p.A, (const char *)p.B, (const char *)p.SA, (const char *)p.SB,
                   0, 0, 0, 0};
        if (r < my_tiles) {
            int tm, tn;
            grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
            const int m0 = tm * BM, n0 = tn * BN;
            const int ra = p.M - m0 < BM ? p.M - m0 : BM, rb = p.N - n0 < BN ? p.N - n0 : BN;
            t.a += (size_t)m0 * p.lda * Op::ELT;
            t.b += (size_t)n0 * p.ldb * Op::ELT;
            t.na = (uint32_t)(((size_t)(ra - 1) * p.lda + p.K) * Op::ELT);
            t.nb = (uint32_t)(((size_t)(rb - 1) * p.ldb + p.K) * Op::ELT);
            if constexpr (Op::MX) {
                // scale rows are 4-byte aligned: the last row's final word
                // may pass ceil(K/32) but stays inside its aligned word
                const int nblk4 = (nblk + 3) & ~3;
                t.sa += (size_t)m0 * p.ld_sa;
                t.sb += (size_t)n0 * p.ld_sb;
                t.nsa = (uint32_t)((ra - 1) * p.ld_sa + nblk4);
                t.nsb = (uint32_t)((rb - 1) * p.ld_sb + nblk4);
            }
        }
        return t;
    };
    TileSpan cur = tile_span(0), nxt = tile_span(1);

    // Direct loads number u in [LO, HI) of K tile kt of the current (next)
    // tile into `stage`: u < NA the A rows, then the B rows, then (MX) the
    // A and B scale words.  Past the workgroup's last tile, `next` selects
    // the zero-record resources.
    // (resources and offsets go through named locals: a resource-building
    // call or an element of a template-sized array captured by the lambda,
    // passed straight to the builtin, makes the host pass drop the kernel's
    // launch stub without a diagnostic)
    auto issue = [&](int lo, int hi, bool next, int kt, int stage) {
        const int soff = kt * Op::BK * Op::ELT;
        char *base = smem + stage * G::STAGE_BYTES;
        const TileSpan &t = next ? nxt : cur;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(t.a, t.na), rb = make_rsrc(t.b, t.nb);
        char *sbase = base + G::A_BYTES + G::B_BYTES;
#pragma unroll
        for (int u = lo; u < hi; ++u) {
            if (u < G::NA) {
                const uint32_t voff = va[u];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (lds_ptr_t)(base + (wave * G::NA + u) * 1024), 16, voff, soff, 0, 0);
            } else if (u < G::NA + G::NB) {
                const int v = u - G::NA;
                const uint32_t voff = vb[v];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (lds_ptr_t)(base + G::A_BYTES + (wave * G::NB + v) * 1024), 16, voff, soff,
                    0, 0);
            } else if (u == G::NA + G::NB) {
                // the K tile's aligned scale word of each row (4 blocks)
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(t.sa, t.nsa);
                const uint32_t voff = vsa;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sbase + wave * 256), 4, voff,
                                                         kt * BPK, 0, 0);
            } else {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(t.sb, t.nsb);
                const uint32_t voff = vsb;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sbase + G::SA_BYTES + wave * 256),
                                                         4, voff, kt * BPK, 0, 0);
            }
        }
    };

    typedef typename std::conditional<Op::MX, intx8, bf16x8>::type Frag;
    Frag fa[NKS][TI], fb[NKS][TJ];   // one register set per k-step of a K tile
    // MX scale words: two sets, one for the K tile being consumed and one
    // being read for the next.  With the K loop unrolled by an even number
    // of K tiles the sets alternate by unrolled copy; otherwise the next set
    // is copied into the current one at the end of each K tile.
    int sc_a[2][TI][SW], sc_b[2][TJ][SW];
    // rows a lane reads differ by multiples of 32 (16x16x32 format: 16, with
    // the swizzle swz8h): the swizzle is lane-constant
    const int lr = S16 ? (lane & 15) : l32;               // row inside a block
    const int swz_lane = S16 ? swz8h(lr) : swz8(l32);

    // fragment i (A) or j (B) of k-step ks from `stage`
    auto frag = [&](const char *rowp, int ks) -> Frag {
        if constexpr (S16) {
            // lane l: k = 32ks + 8(l/16) .. +7
            return *(const bf16x8 *)(rowp + ((4 * ks + (lane >> 4)) ^ swz_lane) * 16);
        } else if constexpr (!Op::MX) {
            return *(const bf16x8 *)(rowp + ((2 * ks + h) ^ swz_lane) * 16);
        } else if constexpr (Op::FP4) {
            // lane (l32, h): block 2ks + h = elements 64ks + 32h .. +31; the
            // instruction reads four registers, the rest stay undefined
            const intx4 v = *(const intx4 *)(rowp + ((2 * ks + h) ^ swz_lane) * 16);
            return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
        } else {
            // lane (l32, h): k = 64ks + 16h .. +15 and 64ks + 32 + 16h .. +15
            intx4 lo = *(const intx4 *)(rowp + ((4 * ks + h) ^ swz_lane) * 16);
            intx4 hi = *(const intx4 *)(rowp + ((4 * ks + 2 + h) ^ swz_lane) * 16);
            return intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    auto read_a = [&](int ks, int stage, int i) {
        fa[ks][i] = frag(smem + stage * G::STAGE_BYTES + (wm * G::WM + i * BLK + lr) * G::ROWB, ks);
    };
    auto read_b = [&](int ks, int stage, int j) {
        fb[ks][j] = frag(smem + stage * G::STAGE_BYTES + G::A_BYTES +
                             (wn * G::WN + j * BLK + lr) * G::ROWB, ks);
    };

    // MX: each lane's scale word of K tile kt (blocks 4kt .. 4kt+3 of its
    // row), blocks at or past ceil(K/32) forced to 127 (x1: they hold zero
    // data), shifted one byte down for the upper half-wave, which supplies
    // the odd block of each instruction; op_sel then picks byte 2*ks.  With
    // scale groups the word is word (gk % 4) of the row's 16 bytes in group
    // buffer (gk / 4) % 2, gk counting K tiles over the workgroup's tiles,
    // and every block is valid (K is a multiple of 512).
    auto read_scales = [&](int stage, int kt, int gk, int set) {
        auto &sn_a = sc_a[set];
        auto &sn_b = sc_b[set];
        if constexpr (Op::MX && Op::SG && Op::FP4) {
            // two words (8 blocks) of group buffer (gk / 2) % 2 at word 2 (gk % 2)
            const uint2 *SAs = (const uint2 *)(smem + G::LDS_BYTES + ((gk >> 1) & 1) * (BM + BN) * 16) + (gk & 1);
            const uint2 *SBs = SAs + BM * 2;
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const uint2 w = SAs[(wm * G::WM + i * 32 + l32) * 2];
                sn_a[i][0] = (int)(w.x >> (8 * h));
                sn_a[i][SW - 1] = (int)(w.y >> (8 * h));
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const uint2 w = SBs[(wn * G::WN + j * 32 + l32) * 2];
                sn_b[j][0] = (int)(w.x >> (8 * h));
                sn_b[j][SW - 1] = (int)(w.y >> (8 * h));
            }
        } else if constexpr (Op::MX && Op::SG) {
            const uint32_t *SAs =
                (const uint32_t *)(smem + G::LDS_BYTES + ((gk >> 2) & 1) * (BM + BN) * 16) + (gk & 3);
            const uint32_t *SBs = SAs + BM * 4;
#pragma unroll
            for (int i = 0; i < TI; ++i)
                sn_a[i][0] = (int)(SAs[(wm * G::WM + i * 32 + l32) * 4] >> (8 * h));
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                sn_b[j][0] = (int)(SBs[(wn * G::WN + j * 32 + l32) * 4] >> (8 * h));
        } else if constexpr (Op::MX) {
            const uint32_t *SAs =
                (const uint32_t *)(smem + stage * G::STAGE_BYTES + G::A_BYTES + G::B_BYTES);
            const uint32_t *SBs = SAs + BM;
            const int left = nblk - kt * 4;
            uint32_t keep = 0xFFFFFFFFu, force = 0;
            if (left < 4) {
                keep = left <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * left));
                force = 0x7F7F7F7Fu & ~keep;
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
                sn_a[i][0] = (int)(((SAs[wm * G::WM + i * 32 + l32] & keep) | force) >> (8 * h));
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                sn_b[j][0] = (int)(((SBs[wn * G::WN + j * 32 + l32] & keep) | force) >> (8 * h));
        }
    };

    // Scale groups: the 16 bytes (four K tiles) of each A and B row of the
    // group starting at K tile kt of the current (next) tile, into group
    // buffer buf; one load per wave and operand, lane l = row wave*64 + l.
    // (The K loop issues them from the first of its GK unrolled K tiles: a
    // run-time branch in the loop would let the compiler move matrix-core
    // instructions past the barriers.)
    auto issue_group = [&](bool next, int kt, int buf) {
        if constexpr (Op::SG) {
            const TileSpan &t = next ? nxt : cur;
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(t.sa, t.nsa);
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(t.sb, t.nsb);
            char *gb = smem + G::LDS_BYTES + buf * (BM + BN) * 16;
            const int soff = kt * BPK;
            if constexpr (WAVES == 4) {
                char *da = gb + wave * 1024, *db = gb + BM * 16 + wave * 1024;
                const uint32_t voa = vsa, vob = vsb;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)da, 16, voa, soff, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)db, 16, vob, soff, 0, 0);
            } else {
                // one operand per wave: a uniform select, no branch
                const bool bside = wave >= 4;
                const __amdgpu_buffer_rsrc_t rs = bside ? rb : ra;
                char *dst = gb + (bside ? BM * 16 : 0) + (wave & 3) * 1024;
                const uint32_t vo = bside ? vsb : vsa;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, vo, soff, 0, 0);
            }
        }
    };

    typename std::conditional<S16, floatx4, floatx16>::type acc[TI][TJ];
    // matrix-core instructions q in [LO, HI) of the K tile, q = ks*NM + i*TJ + j
    auto mfmas = [&](int lo, int hi, int set) {
#pragma unroll
        for (int q = lo; q < hi; ++q) {
            const int ks = q / NM, i = (q % NM) / TJ, j = q % TJ;
            // MX: k-step ks takes blocks 2ks, 2ks+1 of the K tile: byte
            // 2 (ks % 2) of scale word ks / 2 (the upper half-wave's words
            // are shifted one byte down, so it supplies block 2ks + 1)
            if constexpr (S16)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
            else if constexpr (!Op::MX)
                acc[i][j] = mfma_bf16(fb[ks][j], fa[ks][i], acc[i][j]);
            else if (ks % 2 == 0)
                acc[i][j] = mfma_mx<Op::FMT, 0>(fb[ks][j], fa[ks][i], acc[i][j], sc_b[set][j][ks / 2],
                                                sc_a[set][i][ks / 2]);
            else
                acc[i][j] = mfma_mx<Op::FMT, 2>(fb[ks][j], fa[ks][i], acc[i][j], sc_b[set][j][ks / 2],
                                                sc_a[set][i][ks / 2]);
        }
    };

    // a K tile's fragment reads in two parts: the head (phase Y of the
    // previous K tile: k-steps 0 .. YK-1 whole, then k-step YK's B fragments
    // and first YA A fragments) and the tail (phase A: the rest)
    auto read_head = [&](int stage) {
#pragma unroll
        for (int ks = 0; ks < YK; ++ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
                read_a(ks, stage, i);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                read_b(ks, stage, j);
        }
#pragma unroll
        for (int i = 0; i < YA; ++i)
            read_a(YK, stage, i);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            read_b(YK, stage, j);
    };
    auto read_tail = [&](int stage) {
#pragma unroll
        for (int i = YA; i < TI; ++i)
            read_a(YK, stage, i);
#pragma unroll
        for (int ks = YK + 1; ks < NKS; ++ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
                read_a(ks, stage, i);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                read_b(ks, stage, j);
        }
    };

    // One step of the ring (ring_plan.hpp) in iteration g: kt is K tile g's
    // index inside its tile (-1 in the prologue), stage = g % 2, gg = g with
    // its low bits known at compile time, cur / nxs the scale-word register
    // sets of K tiles g and g+1.  Direct loads of K tile g + ktile past the
    // tile's last K tile take the next tile's resources (past the
    // workgroup's last tile the zero-record ones).
    auto step = [&](auto ST, auto U, int kt, int stage, int gg, int set_cur, int set_nxt) {
        constexpr int st = decltype(ST)::value;
        constexpr int u = decltype(U)::value;
        constexpr LoadStep ls = load_step<P>(st);
        if constexpr (ls.ktile > 0) {
            const int kl = kt + ls.ktile;
            const bool lnext = kl >= nk;
            issue(ls.lo, ls.hi, lnext, lnext ? kl - nk : kl, (stage + ls.ktile) & 1);
        } else if constexpr (st == RS_READ_TAIL) {
            read_tail(stage);
        } else if constexpr (st == RS_READ_HEAD) {
            read_head(stage ^ 1);
        } else if constexpr (st == RS_READ_SCALES) {
            read_scales(stage ^ 1, kt + 1 < nk ? kt + 1 : 0, gg + 1, set_nxt);
        } else if constexpr (st == RS_MFMA_A) {
            // the first AM instructions, with the K tile's tail reads and the
            // pending loads spread over them
            mfmas(0, AM, set_cur);
            constexpr int R = (TI - YA) * RPF + FRAG_READS * (NKS - 1 - YK);
            constexpr int PER = (R + AM - 1) / AM;
#pragma unroll
            for (int x = 0; x < AM; ++x) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (x * PER < R)
                    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, PER, 0);
                if (loads_after(x, AM, LA))
                    __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
            }
        } else if constexpr (st == RS_MFMA_X) {
            mfmas(AM, AM + XM, set_cur);
#pragma unroll
            for (int x = 0; x < XM; ++x) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (loads_after(x, XM, LX))
                    __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
            }
        } else if constexpr (st == RS_MFMA_Y) {
            mfmas(AM + XM, NKS * NM, set_cur);
            constexpr int R = YK * FRAG_READS + (YA + TJ) * RPF + (Op::MX ? TI + TJ : 0);
            constexpr int PER = (R + YM - 1) / YM;
#pragma unroll
            for (int x = 0; x < YM; ++x) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (x * PER < R)
                    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, PER, 0);
                if (loads_after(x, YM, LY))
                    __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
            }
        } else if constexpr (st == RS_WAIT_LGKM) {
            // the waits and barriers are fences for the scheduler too: no
            // matrix-core instruction may drift across them
            __builtin_amdgcn_sched_barrier(0);
            wait_lgkm0();
        } else if constexpr (st == RS_WAIT_VM || st == RS_WAIT_VM_PRO) {
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<vm_wait<P>(st)>();
        } else if constexpr (st == RS_BARRIER) {
            barrier();
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (st == RS_ISSUE_GROUP0) {
            issue_group(false, 0, group_buffer(0));
        } else if constexpr (st == RS_ISSUE_GROUP) {
            if constexpr (Op::SG && u == 0) {
                // at a group's first K tile: the next group's scale words
                // into the other group buffer (the host model checks that its
                // last reads precede a barrier before this issue and that the
                // loads land before their first reader)
                const bool gnext = kt + GK >= nk;
                issue_group(gnext, gnext ? 0 : kt + GK, group_buffer(gg / GK + 1));
            }
        }
    };

    // ---------------------------------------------------------- prologue
    static_for<kEarlyPrologueSteps>([&](auto S) {
        step(std::integral_constant<int, kEarlyPrologue[decltype(S)::value]>{},
             std::integral_constant<int, 0>{}, -1, 1, -1, 0, 0);
    });

    int g = 0;
    for (int r = 0; r < my_tiles; ++r) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = {};
        // With scale groups the K loop is unrolled by a group (GK K tiles;
        // the host takes this path only when the K tiles come in whole
        // groups), so the group load sits in the first copy at compile time:
        // no branch in the loop and no placeholder loads in the others.
        for (int kt0 = 0; kt0 < nk; kt0 += UNR) {
            static_for<UNR>([&](auto U) {
                constexpr int u = decltype(U)::value;
                // scale-word sets of this K tile and of the next
                constexpr int set_c = UNR % 2 == 0 ? (u & 1) : 0, set_n = UNR % 2 == 0 ? ((u + 1) & 1) : 1;
                const int kt = kt0 + u;
                // g equals u modulo UNR (tiles hold whole loop trips): written
                // so that the compiler sees the low bits of the K-tile count,
                // and with them the stage and the scale word, as constants
                const int gg = (g & ~(UNR - 1)) | u;
                const int stage = gg & 1;
                static_for<kEarlyLoopSteps>([&](auto S) {
                    step(std::integral_constant<int, kEarlyLoop[decltype(S)::value]>{}, U, kt, stage,
                         gg, set_c, set_n);
                });
                if constexpr (Op::MX && UNR % 2 != 0) {
#pragma unroll
                    for (int w = 0; w < SW; ++w) {
#pragma unroll
                        for (int i = 0; i < TI; ++i)
                            sc_a[0][i][w] = sc_a[1][i][w];
#pragma unroll
                        for (int j = 0; j < TJ; ++j)
                            sc_b[0][j][w] = sc_b[1][j][w];
                    }
                }
                ++g;
            });
        }
        int tm, tn;
        grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
        // The LDS-staged epilogues' per-lane addresses are derived from the
        // lane index computed afresh here (a volatile asm the compiler cannot
        // move), so they are formed after the K loop instead of being hoisted
        // above the tile loop and held in registers (spilled) across it.
        // This removes the one-tile kernels' spills at no cost; the
        // persistent 16x16x32 kernel keeps its 3-10 spilled dwords per tile
        // (outside the K loop): with the fresh index its K loop schedules
        // 1.2% slower (interleaved A/B at 8192^3, every round).
        const int lane_e = S16 && PERSIST ? lane : lane_id_here();
        if constexpr (S16)
            store_tile_lds16<G, TI, TJ>(p, acc, tm * BM, tn * BN, wm, wn, lane_e,
                                        smem + G::LDS_BYTES + SG_BYTES + wave * epi_wave_bytes<EPI_RR>());
        else if constexpr (EPI == EPI_BF16_LDS)
            store_tile_lds<G, BM, BN, EPI_RR>(p, acc, tm * BM, tn * BN, wm, wn, lane_e,
                                              smem + G::LDS_BYTES + SG_BYTES + wave * epi_wave_bytes<EPI_RR>(),
                                              (tm + 1) * BM <= p.M && (tn + 1) * BN <= p.N);
        else if constexpr (EPI == EPI_F32_LDS || EPI == EPI_BF16B_LDS)
            store_tile_lds_f32<G, BM, BN, EPI_RR, EPI == EPI_BF16B_LDS>(
                p, acc, tm * BM, tn * BN, wm, wn, lane_e,
                smem + G::LDS_BYTES + SG_BYTES + wave * epi_wave_bytes<EPI_RR>(),
                (tm + 1) * BM <= p.M && (tn + 1) * BN <= p.N);
        else
            store_tile<EPI, G, BM, BN>(p, acc, tm * BM, tn * BN, wm, wn, h, l32);
        // the load side moves one tile ahead
        cur = nxt;
        nxt = tile_span(r + 2);
    }
    wait_vmcnt<0>();   // no direct load still writing LDS when the waves end
}

// ---------------------------------------------------------------------------
// Level 7: role-specialised waves ("B200 GEMM Optimization Ladder", section
// E step 8: producer / matrix-core / writeback roles and their hand-offs).
//
// Eight waves, two per SIMD, in two groups of four.  Each wave owns a 128x64
// slice of the 256x256 tile (128 accumulator registers, so two waves fit a
// SIMD's register file).  A wave alternates two roles, and the groups are
// one role apart, so on every SIMD one wave feeds the matrix core while the
// other moves data:
//   memory role:  read the whole K tile's fragments from LDS into registers,
//                 issue this wave's share of the direct loads of K tile
//                 g+S-1, write back the previous tile's result when a tile
//                 ends, and wait for its own loads of K tile g+1;
//   compute role: the K tile's matrix-core instructions, back to back, on
//                 fragments already in registers (raised issue priority).
// Every role boundary is a workgroup barrier.  The four hand-offs:
//   load -> compute (ready): a K tile's loads are waited for by each issuing
//       wave in its memory role one K tile ahead, before a barrier that
//       precedes every read of that tile;
//   compute -> load (free): a stage is reloaded only in the memory role after
//       both groups have read it (two barriers later);
//   compute -> writeback: the accumulators are stored in the memory role
//       after the tile's last compute role;
//   writeback -> compute: the accumulators are zeroed after the stores are
//       issued, before the next compute role.
// The ring: S = 4 stages of 32-wide bf16 (64-wide fp8) K tiles, 64-byte LDS
// rows with the swz4 swizzle.  Needs at least four K tiles.
struct PP {
    static constexpr int BM = 256, BN = 256, S = 4;
    static constexpr int WM = 128, WN = 64;        // wave tile
    static constexpr int TI = WM / 32, TJ = WN / 32;
    static constexpr int ROWB = 64, RPL = 16;
    static constexpr int NA = BM / RPL / 8, NB = BN / RPL / 8;   // loads per wave per K tile
};

template <class Op, bool PERSIST, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pingpong(GemmArgs p, int group_m)
{
    constexpr int BM = PP::BM, BN = PP::BN, S = PP::S;
    constexpr int TI = PP::TI, TJ = PP::TJ;
    constexpr int EPC = 16 / Op::ELT;
    constexpr int A_BYTES = BM * PP::ROWB, B_BYTES = BN * PP::ROWB;
    constexpr int SA_BYTES = Op::MX ? BM * 4 : 0, SB_BYTES = Op::MX ? BN * 4 : 0;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    constexpr int LOADS = PP::NA + PP::NB + (Op::MX ? 1 : 0);    // per wave per K tile
    constexpr int KS = Op::MX ? 1 : 2;                           // k-steps per K tile
    static_assert(S * STAGE_BYTES <= 160 * 1024, "LDS budget");
    static_assert((S - 2) * LOADS < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2, pos = wave & 3;                   // SIMD = pos
    const int wm = pos >> 1, wn = (pos & 1) * 2 + grp;
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = (p.K + Op::BK - 1) / Op::BK;                  // >= S (host guarantees)
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = wg_slot(wg, nwg, p.xcd_order);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;
    const int total = my_tiles * nk;

    const __amdgpu_buffer_rsrc_t rsrc_a =
        make_rsrc(p.A, (uint32_t)(((size_t)(p.M - 1) * p.lda + p.K) * Op::ELT));
    const __amdgpu_buffer_rsrc_t rsrc_b =
        make_rsrc(p.B, (uint32_t)(((size_t)(p.N - 1) * p.ldb + p.K) * Op::ELT));
    const int nblk = (p.K + 31) / 32;
    __amdgpu_buffer_rsrc_t rsrc_s = rsrc_a;       // this wave's scale operand (MX)
    int s_rows = 0, s_ld = 0;
    if constexpr (Op::MX) {
        const int nblk4 = (nblk + 3) & ~3;
        // waves 0-3 stage A's scale words, waves 4-7 B's
        rsrc_s = grp == 0 ? make_rsrc(p.SA, (uint32_t)((size_t)(p.M - 1) * p.ld_sa + nblk4))
                          : make_rsrc(p.SB, (uint32_t)((size_t)(p.N - 1) * p.ld_sb + nblk4));
        s_rows = grp == 0 ? p.M : p.N;
        s_ld = grp == 0 ? p.ld_sa : p.ld_sb;
    }

    auto tile_of = [&](int r) { return PERSIST ? persistent_tile_id(wg, nwg, r, p.xcd_order) : first; };

    // Direct-load geometry: this wave's loads t = 0..N-1 fill LDS rows
    // (wave*N + t)*16 .. +15; lane l writes row +l/4 at physical chunk l%4 and
    // fetches logical chunk (l%4) ^ swz4(l/4).
    const int lrow = lane >> 2;
    const int kc_lane = ((lane & 3) ^ swz4(lrow)) * EPC;
    uint32_t a_cur[PP::NA], a_nxt[PP::NA], b_cur[PP::NB], b_nxt[PP::NB];
    uint32_t s_cur = OOB_OFFSET, s_nxt = OOB_OFFSET;
    auto bases = [&](int r, uint32_t (&ab)[PP::NA], uint32_t (&bb)[PP::NB], uint32_t &sb) {
        int m0 = p.M, n0 = p.N;
        if (r < my_tiles) {
            int tm, tn;
            grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
            m0 = tm * BM;
            n0 = tn * BN;
        }
#pragma unroll
        for (int t = 0; t < PP::NA; ++t) {
            const int row = m0 + (wave * PP::NA + t) * PP::RPL + lrow;
            ab[t] = row < p.M ? (uint32_t)(row * p.lda + kc_lane) * Op::ELT : OOB_OFFSET;
        }
#pragma unroll
        for (int t = 0; t < PP::NB; ++t) {
            const int row = n0 + (wave * PP::NB + t) * PP::RPL + lrow;
            bb[t] = row < p.N ? (uint32_t)(row * p.ldb + kc_lane) * Op::ELT : OOB_OFFSET;
        }
        if constexpr (Op::MX) {
            const int row = (grp == 0 ? m0 : n0) + pos * 64 + lane;
            sb = row < s_rows ? (uint32_t)(row * s_ld) : OOB_OFFSET;
        }
    };

    // This wave's direct loads of K tile kt (current or next tile) into
    // `stage`; `on` false turns every lane out of range (LDS still written).
    auto issue = [&](bool next, int kt, int stage, bool on) {
        const int k0 = kt * Op::BK;
        const bool ok = on && k0 + kc_lane < p.K;
        const int soff = k0 * Op::ELT;
        char *base = smem + stage * STAGE_BYTES;
#pragma unroll
        for (int t = 0; t < PP::NA; ++t) {
            const uint32_t voff = ok ? (next ? a_nxt[t] : a_cur[t]) : OOB_OFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (lds_ptr_t)(base + (wave * PP::NA + t) * 1024), 16, voff, soff, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < PP::NB; ++t) {
            const uint32_t voff = ok ? (next ? b_nxt[t] : b_cur[t]) : OOB_OFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (lds_ptr_t)(base + A_BYTES + (wave * PP::NB + t) * 1024), 16, voff, soff,
                0, 0);
        }
        if constexpr (Op::MX) {
            // aligned scale word with blocks 2kt, 2kt+1 of rows pos*64 + lane
            char *sbase = base + A_BYTES + B_BYTES + grp * SA_BYTES + pos * 256;
            const uint32_t v = on ? (next ? s_nxt : s_cur) : OOB_OFFSET;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_s, (lds_ptr_t)sbase, 4, v,
                                                     (2 * kt) & ~3, 0, 0);
        }
    };

    typedef typename std::conditional<Op::MX, intx8, bf16x8>::type Frag;
    Frag fa[KS][TI], fb[KS][TJ];
    int sc_a[TI], sc_b[TJ];
    const int swz_lane = swz4(l32 & 15);

    auto read_tile = [&](int stage, int kt) {
        const char *As = smem + stage * STAGE_BYTES;
        const char *Bs = As + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (!Op::MX) {
                const int chunk = ((2 * ks + h) ^ swz_lane) * 16;
#pragma unroll
                for (int i = 0; i < TI; ++i)
                    fa[ks][i] = *(const bf16x8 *)(As + (wm * PP::WM + i * 32 + l32) * PP::ROWB + chunk);
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    fb[ks][j] = *(const bf16x8 *)(Bs + (wn * PP::WN + j * 32 + l32) * PP::ROWB + chunk);
            } else {
                const int c_lo = (h ^ swz_lane) * 16, c_hi = ((2 + h) ^ swz_lane) * 16;
#pragma unroll
                for (int i = 0; i < TI; ++i) {
                    const char *row = As + (wm * PP::WM + i * 32 + l32) * PP::ROWB;
                    intx4 lo = *(const intx4 *)(row + c_lo), hi = *(const intx4 *)(row + c_hi);
                    fa[ks][i] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const char *row = Bs + (wn * PP::WN + j * 32 + l32) * PP::ROWB;
                    intx4 lo = *(const intx4 *)(row + c_lo), hi = *(const intx4 *)(row + c_hi);
                    fb[ks][j] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            }
        }
        if constexpr (Op::MX) {
            const uint32_t *SAs = (const uint32_t *)(Bs + B_BYTES);
            const uint32_t *SBs = SAs + BM;
            const bool past = 2 * kt + h >= nblk;
            const int shift = 8 * (2 * (kt & 1) + h);
#pragma unroll
            for (int i = 0; i < TI; ++i)
                sc_a[i] = past ? 127 : (int)((SAs[wm * PP::WM + i * 32 + l32] >> shift) & 0xFF);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                sc_b[j] = past ? 127 : (int)((SBs[wn * PP::WN + j * 32 + l32] >> shift) & 0xFF);
        }
    };

    floatx16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            acc[i][j] = zero16();

    auto writeback = [&](int r) {
        int tm, tn;
        grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
        store_tile<EPI, PP, BM, BN>(p, acc, tm * BM, tn * BN, wm, wn, h, l32);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = zero16();
    };

    // ---------------------------------------------------------- prologue
    bases(0, a_cur, b_cur, s_cur);
    bases(1, a_nxt, b_nxt, s_nxt);
#pragma unroll
    for (int q = 0; q < S - 1; ++q)
        issue(false, q, q, true);                   // nk >= S: all of tile 0
    wait_vmcnt<(S - 2) * LOADS>();                  // this wave's share of K tile 0
    barrier();
    if (grp == 1)
        barrier();                                  // group 1 starts one role later

    int stage = 0, g = 0;
    for (int r = 0; r < my_tiles; ++r) {
        for (int kt = 0; kt < nk; ++kt, ++g) {
            // ------------------------------------------------- memory role
            read_tile(stage, kt);
            {
                const int kl = kt + S - 1;
                const bool nxt = kl >= nk;
                issue(nxt, nxt ? kl - nk : kl, stage == 0 ? S - 1 : stage - 1, g + S - 1 < total);
            }
            if (kt == 0 && r > 0)
                writeback(r - 1);
            wait_lgkm0();
            {
                // own loads of K tile g+1 landed (g+2 .. g+S-1 may be in flight)
                const int after = total - 2 - g;
                wait_tiles_after<LOADS>(after < S - 2 ? after : S - 2);
            }
            barrier();
            // ------------------------------------------------ compute role
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j) {
                        if constexpr (!Op::MX)
                            acc[i][j] = mfma_bf16(fb[ks][j], fa[ks][i], acc[i][j]);
                        else
                            acc[i][j] = mfma_mx<Op::FMT, 0>(fb[ks][j], fa[ks][i], acc[i][j], sc_b[j], sc_a[i]);
                    }
            __builtin_amdgcn_s_setprio(0);
            barrier();
            stage = stage + 1 == S ? 0 : stage + 1;
        }
#pragma unroll
        for (int t = 0; t < PP::NA; ++t)
            a_cur[t] = a_nxt[t];
#pragma unroll
        for (int t = 0; t < PP::NB; ++t)
            b_cur[t] = b_nxt[t];
        s_cur = s_nxt;
        bases(r + 2, a_nxt, b_nxt, s_nxt);
    }
    if (my_tiles > 0)
        writeback(my_tiles - 1);
    if (grp == 0)
        barrier();                                  // group 0 ends one role later
    wait_vmcnt<0>();
}

bool whole_bf16(const GemmArgs &p, int bm, int bn)
{
    return p.c_dtype == OUT_BF16 && p.beta == 0.0f && p.M % bm == 0 && p.N % bn == 0 &&
           p.ldc % 4 == 0 && ((uintptr_t)p.C % 8) == 0;
}

// The early-release ring's LDS-staged epilogues (edge tiles masked per row
// and per piece inside them): bf16 C with beta == 0 and 16-byte aligned
// rows; fp32 C with 16-byte aligned rows (any beta); bf16 C with beta != 0
// and 8-byte aligned rows.
bool staged_bf16(const GemmArgs &p)
{
    return p.c_dtype == OUT_BF16 && p.beta == 0.0f && p.ldc % 8 == 0 && ((uintptr_t)p.C % 16) == 0;
}
bool staged_f32(const GemmArgs &p)
{
    return p.c_dtype == OUT_F32 && p.ldc % 4 == 0 && ((uintptr_t)p.C % 16) == 0;
}
bool staged_bf16_beta(const GemmArgs &p)
{
    return p.c_dtype == OUT_BF16 && p.beta != 0.0f && p.ldc % 4 == 0 && ((uintptr_t)p.C % 8) == 0;
}

template <class Op, int BM, int BN, int STAGES, bool PERSIST>
hipError_t launch(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = group_rows(tiles_m, p.group_m);
    int grid = ntiles;
    if (PERSIST)
        grid = ntiles < p.ncu ? ntiles : p.ncu;
    // the staged epilogues where their buffers fit (bf16 pairs blocks, so
    // it needs an even number of 32-column blocks per wave); fp32 with a
    // beta term stays on the register path, which measured faster here:
    // it has every C load of the tile in flight at once, while the staged
    // path waits for C once per round
    using G = Geometry<Op, BM, BN, STAGES>;
    constexpr bool fits = staged_rr(G::LDS_BYTES) > 0;
    if (fits && G::TJ % 2 == 0 && staged_bf16(p))
        hipLaunchKernelGGL((gemm_fast<Op, BM, BN, STAGES, PERSIST, (fits && G::TJ % 2 == 0 ? EPI_BF16_LDS : EPI_ANY)>),
                           dim3(grid), dim3(256), 0, s, p, group_m);
    else if (whole_bf16(p, BM, BN))
        hipLaunchKernelGGL((gemm_fast<Op, BM, BN, STAGES, PERSIST, EPI_BF16_WHOLE>), dim3(grid),
                           dim3(256), 0, s, p, group_m);
    else if (fits && staged_f32(p) && p.beta == 0.0f)
        hipLaunchKernelGGL((gemm_fast<Op, BM, BN, STAGES, PERSIST, (fits ? EPI_F32_LDS : EPI_ANY)>), dim3(grid),
                           dim3(256), 0, s, p, group_m);
    else if (fits && staged_bf16_beta(p))
        hipLaunchKernelGGL((gemm_fast<Op, BM, BN, STAGES, PERSIST, (fits ? EPI_BF16B_LDS : EPI_ANY)>), dim3(grid),
                           dim3(256), 0, s, p, group_m);
    else
        hipLaunchKernelGGL((gemm_fast<Op, BM, BN, STAGES, PERSIST, EPI_ANY>), dim3(grid), dim3(256),
                           0, s, p, group_m);
    return hipGetLastError();
}

template <class Op, int BM, int BN, bool PERSIST>
hipError_t launch_early(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = group_rows(tiles_m, p.group_m);
    // with no more tiles than CUs a persistent grid is the one-tile grid:
    // run the simpler kernel
    if (PERSIST && ntiles <= p.ncu)
        return launch_early<Op, BM, BN, false>(p, s);
    int grid = ntiles;
    if (PERSIST)
        grid = ntiles < p.ncu ? ntiles : p.ncu;
    if (staged_bf16(p))
        hipLaunchKernelGGL((gemm_early<Op, BM, BN, PERSIST, EPI_BF16_LDS>), dim3(grid), dim3(64 * Op::WAVES), 0,
                           s, p, group_m);
    else if (whole_bf16(p, BM, BN))
        hipLaunchKernelGGL((gemm_early<Op, BM, BN, PERSIST, EPI_BF16_WHOLE>), dim3(grid), dim3(64 * Op::WAVES), 0,
                           s, p, group_m);
    else if (staged_f32(p))
        hipLaunchKernelGGL((gemm_early<Op, BM, BN, PERSIST, EPI_F32_LDS>), dim3(grid), dim3(64 * Op::WAVES), 0,
                           s, p, group_m);
    else if (staged_bf16_beta(p))
        hipLaunchKernelGGL((gemm_early<Op, BM, BN, PERSIST, EPI_BF16B_LDS>), dim3(grid), dim3(64 * Op::WAVES), 0,
                           s, p, group_m);
    else
        hipLaunchKernelGGL((gemm_early<Op, BM, BN, PERSIST, EPI_ANY>), dim3(grid), dim3(64 * Op::WAVES), 0, s, p,
                           group_m);
    return hipGetLastError();
}

// bf16 levels 5-6 (and 9) on 256x256 tiles: whole bf16 tiles that take the
// LDS-staged epilogue run the 16x16x32 format (more flops per clock at the
// power limit), everything else the 32x32x16 one.  Ring / RingS16: the
// formats of the two instruction shapes (four waves, or eight for level 9).
template <class Ring, class RingS16, bool PERSIST>
hipError_t launch_early_bf16(const GemmArgs &p, hipStream_t s)
{
    if (!whole_bf16(p, 256, 256) || p.ldc % 8 != 0 || (uintptr_t)p.C % 16 != 0)
        return launch_early<Ring, 256, 256, PERSIST>(p, s);
    const int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = group_rows(tiles_m, p.group_m);
    if (PERSIST && ntiles <= p.ncu)
        return launch_early_bf16<Ring, RingS16, false>(p, s);
    const int grid = PERSIST ? (ntiles < p.ncu ? ntiles : p.ncu) : ntiles;
    hipLaunchKernelGGL((gemm_early<RingS16, 256, 256, PERSIST, EPI_BF16_LDS>), dim3(grid),
                       dim3(64 * RingS16::WAVES), 0, s, p, group_m);
    return hipGetLastError();
}

template <class Op, bool PERSIST>
hipError_t launch_pingpong(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + PP::BM - 1) / PP::BM, tiles_n = (p.N + PP::BN - 1) / PP::BN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = group_rows(tiles_m, p.group_m);
    int grid = ntiles;
    if (PERSIST)
        grid = ntiles < p.ncu ? ntiles : p.ncu;
    if (whole_bf16(p, PP::BM, PP::BN))
        hipLaunchKernelGGL((gemm_pingpong<Op, PERSIST, EPI_BF16_WHOLE>), dim3(grid), dim3(512), 0, s, p,
                           group_m);
    else
        hipLaunchKernelGGL((gemm_pingpong<Op, PERSIST, EPI_ANY>), dim3(grid), dim3(512), 0, s, p,
                           group_m);
    return hipGetLastError();
}

bool big_tiles(const GemmArgs &p)
{
    return (long)((p.M + 255) / 256) * ((p.N + 255) / 256) >= p.ncu;
}

// Levels 5-7 and 9 for one 8-bit element format: Op (the older ring), Ring
// (64-byte rows, level 7), Ring128 / Ring128G (gemm_early without / with
// scale groups), Ring128GW8 (level 9: eight consumer waves, scale groups).
template <class Op, class Ring, class Ring128, class Ring128G, class Ring128GW8>
hipError_t launch_fast_mx8(int level, const GemmArgs &p, hipStream_t s)
{
    const bool ring_ok = p.K > Ring128::BK && p.K % Ring128::BK == 0;   // whole K tiles
    // whole groups of 16 scale blocks, 16-byte aligned scale rows
    const bool groups = p.K % 512 == 0 && p.ld_sa % 16 == 0 && p.ld_sb % 16 == 0 &&
                        (uintptr_t)p.SA % 16 == 0 && (uintptr_t)p.SB % 16 == 0;
    switch (level) {
    case 5:
        if (skinny_mx_eligible(p))
            return launch_skinny_mx(p, s);
        if (ring_ok && groups)
            return launch_early<Ring128G, 256, 256, false>(p, s);
        return ring_ok ? launch_early<Ring128, 256, 256, false>(p, s) : launch<Op, 256, 256, 2, false>(p, s);
    case 6:
        if (skinny_mx_eligible(p))
            return launch_skinny_mx(p, s);
        if (ring_ok && groups)
            return launch_early<Ring128G, 256, 256, true>(p, s);
        return ring_ok ? launch_early<Ring128, 256, 256, true>(p, s) : launch<Op, 256, 256, 2, true>(p, s);
    case 7:
        return p.K > 3 * Ring::BK ? launch_pingpong<Ring, true>(p, s) : launch<Op, 256, 256, 2, true>(p, s);
    case 9:
        if (ring_ok && groups)
            return launch_early<Ring128GW8, 256, 256, true>(p, s);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

} // namespace
} // namespace mce
