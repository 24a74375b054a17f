// Levels 5 and 6 of the GEMM ladder ("B200 GEMM Optimization Ladder",
// section E steps 6-7) for bf16 operands the direct-load kernels cannot
// take: either operand MN-major (A column-major or B row-major), rows that
// are not 16-byte aligned, or K not a whole number of 16-byte chunks.
//
// The operands travel through registers: each lane loads two 16-byte
// chunks of a 128 x 32 operand tile per K tile (gfx950 global loads accept
// any alignment, so a 2-byte-aligned row costs no extra instructions; only
// chunks that cross the M, N or K edge fall back to masked element loads),
// then writes them to LDS in the K-major, XOR-swizzled 64-byte rows that
// the matrix-core fragment reads expect.  A K-contiguous chunk is eight
// consecutive K of one row (one 16-byte LDS write); for an MN-major operand
// a lane loads the same eight rows at two adjacent K and writes them
// transposed as eight 4-byte (k, k+1) pairs ("B200 TMA Pipeline Designer",
// section B: the layout the reader expects is produced by the writer).
//
// Ring: two LDS stages; the loads of K tile kt+1 are in registers while
// tile kt is consumed, written to the other stage after the matrix-core
// work, and one barrier per K tile hands both stages over.  (A second
// register set, loading two K tiles ahead, measured slower: the registers
// cost a workgroup per CU.)  Level 6 walks
// the tiles of a persistent grid in the XCD-aware grouped order.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "sched.hpp"

namespace mce {
namespace {

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int GBM = 128, GBN = 128, GBK = 32;
constexpr int GROWB = GBK * 2;                 // 64-byte LDS rows: 4 chunks of 8 K
constexpr int GOP_BYTES = GBM * GROWB;         // one operand tile, 8 KiB
constexpr int GSTAGE = 2 * GOP_BYTES;          // A + B
// the ring's two stages, reused by the four waves' epilogue buffers
constexpr int GSMEM = 2 * GSTAGE > 4 * EPI_F32_WAVE_BYTES ? 2 * GSTAGE : 4 * EPI_F32_WAVE_BYTES;

// Wave tile 64 x 64 of a 2 x 2 wave grid (the epilogue's view).
struct GenGeom {
    static constexpr int WM = 64, WN = 64, TI = 2, TJ = 2;
};

// One 128-row x 32-K operand tile through two 16-byte chunks per lane.
// KC: element (r, k) at base[r * ld + k] (K-contiguous); otherwise at
// base[k * ld + r] (MN-major).  rows: the operand's extent (M or N).
template <bool KC>
struct Stager {
    u16x8 v[2];

    __device__ __forceinline__ void load(const uint16_t *base, int ld, int rows, int K, int r0,
                                         int k0, int tid)
    {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int idx = j * 256 + tid;
            // KC: chunk = 8 K of one row; MN: chunk j = 8 rows at K 2*(tid/16)
            // + j (the 16 lanes of a K read 256 contiguous bytes)
            const int r = KC ? r0 + idx / 4 : r0 + (tid % 16) * 8;
            const int k = KC ? k0 + (idx % 4) * 8 : k0 + 2 * (tid / 16) + j;
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

    __device__ __forceinline__ void store(char *lds, int tid) const
    {
        if (KC) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int idx = j * 256 + tid;
                const int row = idx / 4, c = idx % 4;
                *(u16x8 *)(lds + row * GROWB + ((c ^ swz4g(row)) * 16)) = v[j];
            }
        } else {
            const int kk = 2 * (tid / 16), c = tid % 16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = c * 8 + e;
                const uint32_t pair = (uint32_t)v[0][e] | ((uint32_t)v[1][e] << 16);
                *(uint32_t *)(lds + row * GROWB + (((kk >> 3) ^ swz4g(row)) * 16) + (kk & 7) * 2) = pair;
            }
        }
    }
};

template <bool A_KC, bool B_KC, bool PERSIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void gemm_general(GemmArgs p, int group_m)
{
    __shared__ __attribute__((aligned(1024))) char smem[GSMEM];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    // rows a lane reads differ by multiples of 32: the swizzle is lane-constant
    const int swz_lane = swz4g(l32);

    const int tiles_m = (p.M + GBM - 1) / GBM, tiles_n = (p.N + GBN - 1) / GBN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = (p.K + GBK - 1) / GBK;
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = xcd_major(wg, nwg);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;
    const uint16_t *A = (const uint16_t *)p.A, *B = (const uint16_t *)p.B;

    Stager<A_KC> sa;
    Stager<B_KC> sb;
    floatx16 acc[2][2];
    for (int r = 0; r < my_tiles; ++r) {
        int tm, tn;
        grouped_tile(PERSIST ? persistent_tile_id(wg, nwg, r) : first, tiles_m, tiles_n, group_m, tm,
                     tn);
        const int m0 = tm * GBM, n0 = tn * GBN;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = zero16();
        // prologue: K tile 0 into stage 0
        sa.load(A, p.lda, p.M, p.K, m0, 0, tid);
        sb.load(B, p.ldb, p.N, p.K, n0, 0, tid);
        sa.store(smem, tid);
        sb.store(smem + GOP_BYTES, tid);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) {   // K tile kt+1 travels in registers under this tile's work
                sa.load(A, p.lda, p.M, p.K, m0, (kt + 1) * GBK, tid);
                sb.load(B, p.ldb, p.N, p.K, n0, (kt + 1) * GBK, tid);
            }
            const char *As = smem + (kt & 1) * GSTAGE, *Bs = As + GOP_BYTES;
#pragma unroll
            for (int ks = 0; ks < GBK / 16; ++ks) {
                const int chunk = ((2 * ks + h) ^ swz_lane) * 16;
                bf16x8 fa[2], fb[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    fa[i] = *(const bf16x8 *)(As + (wm * 64 + i * 32 + l32) * GROWB + chunk);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    fb[j] = *(const bf16x8 *)(Bs + (wn * 64 + j * 32 + l32) * GROWB + chunk);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = mfma_bf16(fb[j], fa[i], acc[i][j]);
            }
            if (more) {   // the other stage was released by the last barrier
                char *nxt = smem + ((kt + 1) & 1) * GSTAGE;
                sa.store(nxt, tid);
                sb.store(nxt + GOP_BYTES, tid);
            }
            __syncthreads();   // stage kt+1 written by every wave; stage kt read by every wave
        }
        // the last barrier released both stages: the epilogue stages C
        // through them, 256 contiguous bytes of a row per 16 lanes
        store_tile_staged<GenGeom>(p, acc, m0, n0, wm, wn, lane, smem + wave * EPI_F32_WAVE_BYTES);
        if (PERSIST)
            __syncthreads();   // every wave's buffer read before the next prologue writes
    }
}

template <bool A_KC, bool B_KC, bool PERSIST>
hipError_t launch_g(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + GBM - 1) / GBM, tiles_n = (p.N + GBN - 1) / GBN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    int grid = ntiles;
    if (PERSIST) {
        // three workgroups fit a CU (34 KiB of LDS, the kernel is held to 168
        // registers per lane): the persistent grid keeps all of them busy
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            ncu > 0 && ntiles > 3 * ncu)
            grid = 3 * ncu;
    }
    hipLaunchKernelGGL((gemm_general<A_KC, B_KC, PERSIST>), dim3(grid), dim3(256), 0, s, p, group_m);
    return hipGetLastError();
}

template <bool PERSIST>
hipError_t launch_g_layout(const GemmArgs &p, hipStream_t s)
{
    const bool akc = !p.a_cm, bkc = p.b_cm;
    if (akc && bkc)
        return launch_g<true, true, PERSIST>(p, s);
    if (akc)
        return launch_g<true, false, PERSIST>(p, s);
    if (bkc)
        return launch_g<false, true, PERSIST>(p, s);
    return launch_g<false, false, PERSIST>(p, s);
}

} // namespace

hipError_t launch_general_bf16(int level, const GemmArgs &p, hipStream_t s)
{
    switch (level) {
    case 5: return launch_g_layout<false>(p, s);
    case 6: {
        // while the tiles fit the three workgroups per CU at once, the
        // persistent grid is the one-tile grid (whose kernel needs fewer
        // registers and so keeps three workgroups per CU)
        const long ntiles = (long)((p.M + GBM - 1) / GBM) * ((p.N + GBN - 1) / GBN);
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            ntiles <= 3L * ncu)
            return launch_g_layout<false>(p, s);
        return launch_g_layout<true>(p, s);
    }
    default: return hipErrorInvalidValue;
    }
}

} // namespace mce
