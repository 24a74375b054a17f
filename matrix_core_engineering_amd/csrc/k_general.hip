// Levels 5 and 6 of the GEMM ladder ("B200 GEMM Optimization Ladder",
// section E steps 6-7) for bf16 operands the direct-load kernels cannot
// take: either operand MN-major (A column-major or B row-major), rows that
// are not 16-byte aligned, or K not a whole number of 16-byte chunks.
//
// The operands travel through registers: each lane loads 16-byte chunks of
// a 128-row operand tile per K tile (gfx950 global loads accept any
// alignment, so a 2-byte-aligned row costs no extra instructions), then
// writes them to LDS with 16-byte writes.  A K-contiguous chunk is eight
// consecutive K of one row, kept in K-major, XOR-swizzled rows that the
// matrix-core fragment reads expect; an MN-major chunk is eight consecutive
// rows at one K, kept as loaded (256-byte K rows), and the fragment reads
// transpose it with ds_read_b64_tr_b16 ("B200 TMA Pipeline Designer",
// section B: the layout the reader expects is produced by the writer; on
// gfx950 the transposing side is the LDS read).
//
// Ring: two LDS stages of 64-byte rows (K tile 32).  K tile kt+1 is loaded
// into registers before K tile kt's matrix-core work and written to the
// other stage after it; one barrier per K tile hands both stages over.  (A
// second register set, loading two K tiles ahead, measured no faster and
// pushes the persistent kernel into spills.)  The LDS (34 KiB: the
// epilogue's four wave buffers reuse the ring) and the 168-register cap let
// three workgroups share a CU.  Level 6 walks the tiles of a persistent grid
// in the XCD-aware grouped order.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "mn_layout.hpp"
#include "sched.hpp"

namespace mce {
namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 *lds_v4i16_t;

constexpr int GBM = 128, GBN = 128;

// Element e of the result is v[e + s] for e + s < 8, else zero (s >= 0);
// selects, not branches, since s varies across lanes.
__device__ __forceinline__ u16x8 shift_down(const u16x8 &v, int s)
{
    const uint64_t lo = __builtin_bit_cast(uint64_t, u16x4{v[0], v[1], v[2], v[3]});
    const uint64_t hi = __builtin_bit_cast(uint64_t, u16x4{v[4], v[5], v[6], v[7]});
    const int b = min(16 * s, 128);
    const uint64_t lo_hi = b == 0 ? lo : b >= 64 ? 0 : lo >> b;
    const uint64_t hi_lo = b == 0 ? 0 : b >= 64 ? (b >= 128 ? 0 : hi >> (b - 64)) : hi << (64 - b);
    const uint64_t nhi = b >= 64 ? 0 : hi >> b;
    const u16x4 l4 = __builtin_bit_cast(u16x4, lo_hi | hi_lo), h4 = __builtin_bit_cast(u16x4, nhi);
    return u16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
}

template <int BK>
struct GenTile {
    static_assert(BK == 32, "K tile: 64-byte rows, a K pair per lane for MN-major operands");
    static constexpr int ROWB = BK * 2;                  // bytes per LDS row
    static constexpr int CPR = BK / 8;                   // 16-byte chunks per row
    static constexpr int CH = BK / 16;                   // chunks per lane and operand
    static constexpr int OP_BYTES = GBM * ROWB;          // one operand tile
    static constexpr int STAGE_BYTES = 2 * OP_BYTES;     // A + B
    static constexpr int RING = 2 * STAGE_BYTES;
    static constexpr int SMEM = RING > 4 * EPI_F32_WAVE_BYTES ? RING : 4 * EPI_F32_WAVE_BYTES;
    static __device__ __forceinline__ int swz(int row) { return swz4q(row); }
};

// Wave tile 64 x 64 of a 2 x 2 wave grid (the epilogue's view).
struct GenGeom {
    static constexpr int WM = 64, WN = 64, TI = 2, TJ = 2;
};

// One 128-row x BK operand tile through CH 16-byte chunks per lane.
// KC: element (r, k) at base[r * ld + k] (K-contiguous); otherwise at
// base[k * ld + r] (MN-major).  rows: the operand's extent (M or N).
// KC chunk j of lane tid: row idx / CPR, K (idx % CPR) * 8 with
// idx = j * 256 + tid.  MN chunk j: rows 8 mn_c(tid) .. +7 at K
// mn_k(tid) + j: eight consecutive lanes read 128 contiguous bytes of one K
// row and write eight chunks of one 256-byte LDS K row.
template <bool KC, int BK>
struct Stager {
    using T = GenTile<BK>;
    typedef u16x8 Regs[T::CH];             // one K tile's chunks of this lane
    const uint16_t *ptr[KC ? T::CH : 1];   // this tile's chunk addresses at K = 0
    int roff;                              // MN-major: first row of this lane's chunks in the tile
    int shift;                             // MN-major: rows that start was moved back by

    static __device__ __forceinline__ int mn_c(int tid) { return (tid & 7) | ((tid >> 7) << 3); }
    static __device__ __forceinline__ int mn_k(int tid) { return 2 * ((tid >> 3) & 15); }

    // Per tile.  Rows past the edge are never read: a KC row there is
    // clamped to the last row (its products only reach C rows or columns
    // that are never stored), and an MN-major chunk that would cross the
    // edge is fetched ending at it and shifted back into place when it is
    // written; LDS rows past the edge keep whatever they hold, which also
    // reaches only C entries that are never stored.  The MN-major clamp
    // needs eight valid rows in the tile (else every chunk that crosses the
    // edge is loaded per element).
    __device__ __forceinline__ void prep(const uint16_t *base, int ld, int rows, int r0, int tid)
    {
        if (KC) {
#pragma unroll
            for (int j = 0; j < T::CH; ++j) {
                const int idx = j * 256 + tid;
                ptr[KC ? j : 0] = base + (size_t)min(r0 + idx / T::CPR, rows - 1) * ld + (idx % T::CPR) * 8;
            }
            roff = 0;
            shift = 0;
        } else {
            // clamp only while the tile holds eight valid rows
            const int r = rows - r0 >= 8 ? min(r0 + mn_c(tid) * 8, rows - 8) : r0 + mn_c(tid) * 8;
            ptr[0] = base + (size_t)mn_k(tid) * ld + r;
            roff = r - r0;
            shift = r0 + mn_c(tid) * 8 - r;
        }
    }

    // a whole K tile: no masks
    __device__ __forceinline__ void load_fast(Regs &v, int ld, int k0) const
    {
#pragma unroll
        for (int j = 0; j < T::CH; ++j) {
            const uint16_t *src = KC ? ptr[KC ? j : 0] + k0 : ptr[0] + (size_t)(k0 + j) * ld;
            __builtin_memcpy(&v[j], src, 16);
        }
    }

    // any K tile (after prep): chunks that cross the M, N or K edge are
    // loaded per element, into the LDS rows the store expects
    __device__ __forceinline__ void load(Regs &v, const uint16_t *base, int ld, int rows, int K,
                                         int r0, int k0, int tid) const
    {
#pragma unroll
        for (int j = 0; j < T::CH; ++j) {
            const int idx = j * 256 + tid;
            const int r = KC ? r0 + idx / T::CPR : r0 + roff;
            const int k = KC ? k0 + (idx % T::CPR) * 8 : k0 + mn_k(tid) + j;
            const bool whole = KC ? (r < rows && k + 8 <= K) : (k < K && r + 8 <= rows);
            if (whole) {
                const uint16_t *src = KC ? base + (size_t)r * ld + k : base + (size_t)k * ld + r;
                __builtin_memcpy(&v[j], src, 16);
            } else {
                u16x8 t;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int rr = KC ? r : r + e, kk = KC ? k + e : k;
                    t[e] = (rr < rows && kk < K) ? base[(size_t)(KC ? rr : kk) * ld + (KC ? kk : rr)]
                                                 : (uint16_t)0;
                }
                v[j] = t;
            }
        }
    }

    // edge: the tile crosses the M or N edge (MN chunks may need shifting)
    __device__ __forceinline__ void store(const Regs &v, char *lds, bool edge, int tid) const
    {
        if (KC) {
#pragma unroll
            for (int j = 0; j < T::CH; ++j) {
                const int idx = j * 256 + tid;
                const int row = idx / T::CPR, c = idx % T::CPR;
                *(u16x8 *)(lds + row * T::ROWB + ((c ^ T::swz(row)) * 16)) = v[j];
            }
        } else {
            const int c = mn_c(tid);
#pragma unroll
            for (int j = 0; j < T::CH; ++j) {
                const int k = mn_k(tid) + j;
                *(u16x8 *)(lds + k * 256 + ((c ^ mn_swz16(k)) * 16)) = edge ? shift_down(v[j], shift) : v[j];
            }
        }
    }
};

template <bool A_KC, bool B_KC, bool PERSIST, int BK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void gemm_general(GemmArgs p, int group_m)
{
    using T = GenTile<BK>;
    __shared__ __attribute__((aligned(1024))) char smem[T::SMEM];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    // per fragment row block (wm*64 + i*32, wn*64 + j*32): a K-contiguous
    // operand's 16-byte read offset at k-step 0 (logical chunk h; k-step
    // ks is the offset ^ 32 ks), or an MN-major operand's transposing-read
    // offset (this lane supplies K row 8h + (lane % 16) / 4 and rows
    // 16 ((lane / 16) % 2) + 4 (lane % 4) .. +3 of the block; the second
    // read is 4 K rows on and k-step 1 16 on, at the same swizzle)
    auto frag_off = [&](bool kc, int rb) {
        if (kc) {
            const int row = rb + l32;
            return row * T::ROWB + ((h ^ T::swz(row)) * 16);
        }
        const int kr = 8 * h + ((lane & 15) >> 2);
        const int n = rb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        return kr * 256 + (((n >> 3) ^ mn_swz16(kr)) * 16) + (n & 7) * 2;
    };
    int off_a[2], off_b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        off_a[i] = frag_off(A_KC, wm * 64 + i * 32);
        off_b[i] = T::OP_BYTES + frag_off(B_KC, wn * 64 + i * 32);
    }
    auto frag = [&](bool kc, const char *S, int o, int ks) -> bf16x8 {
        if (kc)
            return *(const bf16x8 *)(S + (o ^ (32 * ks)));
        const char *p0 = S + o + 4096 * ks;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)p0);
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(p0 + 1024));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    const int tiles_m = (p.M + GBM - 1) / GBM, tiles_n = (p.N + GBN - 1) / GBN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = (p.K + BK - 1) / BK;
    const int nf = p.K / BK;   // K tiles wholly inside K
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = wg_slot(wg, nwg, p.xcd_order);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;
    const uint16_t *A = (const uint16_t *)p.A, *B = (const uint16_t *)p.B;

    Stager<A_KC, BK> sa;
    Stager<B_KC, BK> sb;
    typename Stager<A_KC, BK>::Regs va;
    typename Stager<B_KC, BK>::Regs vb;
    floatx16 acc[2][2];

    auto compute = [&](int stage) {
        const char *S = smem + stage * T::STAGE_BYTES;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[i] = frag(A_KC, S, off_a[i], ks);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = frag(B_KC, S, off_b[j], ks);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma_bf16(fb[j], fa[i], acc[i][j]);
        }
    };

    for (int r = 0; r < my_tiles; ++r) {
        int tm, tn;
        grouped_tile(PERSIST ? persistent_tile_id(wg, nwg, r, p.xcd_order) : first, tiles_m, tiles_n, group_m, tm,
                     tn);
        const int m0 = tm * GBM, n0 = tn * GBN;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = zero16();
        sa.prep(A, p.lda, p.M, m0, tid);
        sb.prep(B, p.ldb, p.N, n0, tid);
        // The masked loads run only for the K tile with a tail (or for an
        // MN-major operand whose tile holds fewer than eight valid rows),
        // behind a uniform branch; every other K tile takes the steady loops
        // below, whose whole-chunk loads have no branch between them, so each
        // wait before an LDS write counts exactly the loads it must.
        const bool a_in = A_KC || p.M - m0 >= 8, b_in = B_KC || p.N - n0 >= 8;
        const bool steady = a_in && b_in;
        auto load = [&](int kt) {
            const int k0 = kt * BK;
            if (k0 + BK <= p.K && a_in)
                sa.load_fast(va, p.lda, k0);
            else
                sa.load(va, A, p.lda, p.M, p.K, m0, k0, tid);
            if (k0 + BK <= p.K && b_in)
                sb.load_fast(vb, p.ldb, k0);
            else
                sb.load(vb, B, p.ldb, p.N, p.K, n0, k0, tid);
        };
        auto load_fast = [&](int kt) {
            sa.load_fast(va, p.lda, kt * BK);
            sb.load_fast(vb, p.ldb, kt * BK);
        };
        const bool a_edge = m0 + GBM > p.M, b_edge = n0 + GBN > p.N;
        auto store = [&](int stage) {
            sa.store(va, smem + stage * T::STAGE_BYTES, a_edge, tid);
            sb.store(vb, smem + stage * T::STAGE_BYTES + T::OP_BYTES, b_edge, tid);
        };

        // K tile kt+1 travels in registers under K tile kt's work and is
        // written to the other stage, which the last barrier released
        int kt = 0;
        if (steady && nf >= 2) {
            load_fast(0);
            store(0);
            __syncthreads();
            for (; kt + 1 < nf; ++kt) {
                load_fast(kt + 1);
                compute(kt & 1);
                store((kt + 1) & 1);
                __syncthreads();
            }
        } else {
            load(0);
            store(0);
            __syncthreads();
        }
        for (; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more)
                load(kt + 1);
            compute(kt & 1);
            if (more)
                store((kt + 1) & 1);
            __syncthreads();   // stage kt+1 written by every wave; stage kt read by every wave
        }
        // the last barrier released the ring: the epilogue stages C through
        // it, 256 contiguous bytes of a row per 16 lanes
        store_tile_staged<GenGeom>(p, acc, m0, n0, wm, wn, lane, smem + wave * EPI_F32_WAVE_BYTES);
        if (PERSIST)
            __syncthreads();   // every wave's buffer read before the next prologue writes
    }
}

template <bool A_KC, bool B_KC, bool PERSIST, int BK>
hipError_t launch_g(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + GBM - 1) / GBM, tiles_n = (p.N + GBN - 1) / GBN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = group_rows(tiles_m, p.group_m);
    int grid = ntiles;
    if (PERSIST) {
        // three workgroups fit a CU (34 KiB of LDS, the kernel is held to 168
        // registers per lane): the persistent grid keeps all of them busy
        if (ntiles > 3 * p.ncu)
            grid = 3 * p.ncu;
    }
    hipLaunchKernelGGL((gemm_general<A_KC, B_KC, PERSIST, BK>), dim3(grid), dim3(256), 0, s, p, group_m);
    return hipGetLastError();
}

template <bool PERSIST, int BK>
hipError_t launch_g_layout(const GemmArgs &p, hipStream_t s)
{
    const bool akc = !p.a_cm, bkc = p.b_cm;
    if (akc && bkc)
        return launch_g<true, true, PERSIST, BK>(p, s);
    if (akc)
        return launch_g<true, false, PERSIST, BK>(p, s);
    if (bkc)
        return launch_g<false, true, PERSIST, BK>(p, s);
    return launch_g<false, false, PERSIST, BK>(p, s);
}

} // namespace

hipError_t launch_general_bf16(int level, const GemmArgs &p, hipStream_t s)
{
    switch (level) {
    case 5: return launch_g_layout<false, 32>(p, s);
    case 6: {
        // while the tiles fit the three workgroups per CU at once, the
        // persistent grid is the one-tile grid (whose kernel needs fewer
        // registers)
        const long ntiles = (long)((p.M + GBM - 1) / GBM) * ((p.N + GBN - 1) / GBN);
        if (ntiles <= 3L * p.ncu)
            return launch_g_layout<false, 32>(p, s);
        return launch_g_layout<true, 32>(p, s);
    }
    default: return hipErrorInvalidValue;
    }
}

} // namespace mce
