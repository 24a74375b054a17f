// Levels 1-3 of the GEMM ladder ("B200 GEMM Optimization Ladder", section E
// steps 2-4): a 128x128 output tile per workgroup, operands copied
// synchronously global -> VGPR -> LDS element by element (any layout, any
// alignment, bounds-checked), then read from LDS into matrix-core fragments.
//
//   level 1: one workgroup, one K tile (K <= 64)        -- single tile
//   level 2: one workgroup, loop over K tiles + tail    -- K loop
//   level 3: a grid of workgroups over M and N          -- spatial tiling
//
// The same kernel body serves the three levels; the host restricts the
// problem and the grid for levels 1 and 2.  A block-scaled MX variant (level
// 3 only, any MX element format) uses the same structure with K tiles of 64
// elements.
//
// Workgroup: 256 threads = 4 waves in a 2x2 arrangement, each wave owning a
// 64x64 sub-tile = 2x2 blocks of the 32x32 matrix-core instruction.
#include "common.hpp"
#include "launch.hpp"

namespace mce {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_ROW = BK + 8;   // bf16 elements per LDS row (144 B): pads banks

// Copies the BM x BK tile of a (row0.., k0..) into lds[m][k] (K-major),
// zero-filling every element outside the logical matrix.
__device__ __forceinline__ void load_tile_bf16(const uint16_t *g, int ld, int col_major, int rows,
                                               int K, int row0, int k0, uint16_t *lds)
{
    const int tid = threadIdx.x;
#pragma unroll 4
    for (int e = 0; e < (BM * BK) / 256; ++e) {
        int idx = tid + 256 * e;
        // walk the contiguous direction fastest so the global reads coalesce
        int r, k;
        if (col_major) {
            r = idx % BM;
            k = idx / BM;
        } else {
            r = idx / BK;
            k = idx % BK;
        }
        int gr = row0 + r, gk = k0 + k;
        uint16_t v = 0;
        if (gr < rows && gk < K)
            v = col_major ? g[(size_t)gk * ld + gr] : g[(size_t)gr * ld + gk];
        lds[r * LDS_ROW + k] = v;
    }
}

template <bool KLOOP>
__global__ __launch_bounds__(256) void gemm_simple_bf16(GemmArgs p)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_ROW];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_ROW];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (p.N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
    const uint16_t *A = (const uint16_t *)p.A;
    const uint16_t *B = (const uint16_t *)p.B;

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = zero16();

    const int ktiles = KLOOP ? (p.K + BK - 1) / BK : 1;
    for (int kt = 0; kt < ktiles; ++kt) {
        const int k0 = kt * BK;
        // A: rows are m (M x K).  B is stored in LDS as Bs[n][k]: its
        // "rows" are n, and a column-major B is K-contiguous per n.
        load_tile_bf16(A, p.lda, p.a_cm, p.M, p.K, m0, k0, As);
        load_tile_bf16(B, p.ldb, !p.b_cm, p.N, p.K, n0, k0, Bs);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 fa[2], fb[2];
            const int kk = ks * 16 + 8 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int r = wm * 64 + i * 32 + (lane & 31);
                fa[i] = *(const bf16x8 *)&As[r * LDS_ROW + kk];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int c = wn * 64 + j * 32 + (lane & 31);
                fb[j] = *(const bf16x8 *)&Bs[c * LDS_ROW + kk];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int row = m0 + wm * 64 + i * 32 + acc_row(r, lane);
                int col = n0 + wn * 64 + j * 32 + acc_col(lane);
                if (row < p.M && col < p.N)
                    store_c(p, row, col, acc[i][j][r]);
            }
}

// ---------------------------------------------------------------- MX
//
// K tile of 64 elements = two 32-element scale blocks = one 32x32x64
// block-scaled instruction per (i, j) per K tile.  The packed formats are
// K-contiguous, the 8-bit ones either layout; a K tile of a row is
// 64 * bits / 8 bytes (64, 48 or 32),
// copied byte by byte into an LDS row of that length plus 16 bytes of
// padding.  Bytes past K are zero (for the packed formats K fills whole
// bytes, so no element past K shares a byte with one inside).
constexpr int MX_BK = 64;

template <int FMT>
struct MxTile {
    static constexpr int BYTES = MX_BK * mx_bits(FMT) / 8;   // K-tile bytes per row
    static constexpr int ROW = BYTES + 16;                   // LDS row pitch
};

// One operand's K tile into LDS rows (one row per M or N index, K along
// the row).  KC: byte b of row r at g[r * ld_bytes + b]; otherwise (an
// MN-major 8-bit operand, ld in elements = bytes) element (r, k) at
// g[k * ld_bytes + r], consecutive threads taking consecutive rows.
template <int FMT>
__device__ __forceinline__ void load_tile_mx(const uint8_t *g, int64_t ld_bytes, bool kc, int rows,
                                             int64_t k_bytes, int row0, int64_t kb0, uint8_t *lds)
{
    using T = MxTile<FMT>;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < BM * T::BYTES; idx += 256) {
        const int r = kc ? idx / T::BYTES : idx % BM, b = kc ? idx % T::BYTES : idx / BM;
        const int gr = row0 + r;
        const int64_t gb = kb0 + b;
        uint8_t v = 0;
        if (gr < rows && gb < k_bytes)
            v = kc ? g[(size_t)gr * ld_bytes + gb] : g[(size_t)gb * ld_bytes + gr];
        lds[r * T::ROW + b] = v;
    }
}

// The scale of (row, block kb) for lane use; rows/blocks outside the
// matrix get 127 (x1): their data bytes are zero.
__device__ __forceinline__ int scale_byte(const uint8_t *s, int ld, int rows, int nblk, int row, int kb)
{
    if (row < rows && kb < nblk)
        return s[(size_t)row * ld + kb];
    return 127;
}

// A lane's fragment of one row of the K tile (see the map in common.hpp):
// 8-bit formats two 16-byte halves (k 16h.. and 32+16h..), the packed
// formats the whole block h (k 32h .. 32h + 31) from its first bit.
template <int FMT>
__device__ __forceinline__ intx8 mx_fragment(const uint8_t *row, int h)
{
    if constexpr (mx_bits(FMT) == 8) {
        const intx4 lo = *(const intx4 *)(row + 16 * h), hi = *(const intx4 *)(row + 32 + 16 * h);
        return intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else if constexpr (mx_bits(FMT) == 6) {
        const int *w = (const int *)(row + 24 * h);   // 8-byte aligned: rows are 64-byte pitched
        return intx8{w[0], w[1], w[2], w[3], w[4], w[5], 0, 0};
    } else {
        const intx4 v = *(const intx4 *)(row + 16 * h);
        return intx8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void gemm_simple_mx(GemmArgs p)
{
    using T = MxTile<FMT>;
    __shared__ __attribute__((aligned(16))) uint8_t As[BM * T::ROW];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * T::ROW];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (p.N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
    const uint8_t *A = (const uint8_t *)p.A;
    const uint8_t *B = (const uint8_t *)p.B;
    const int nblk = (p.K + 31) / 32;
    constexpr int BITS = mx_bits(FMT);
    const int64_t lda_b = (int64_t)p.lda * BITS / 8, ldb_b = (int64_t)p.ldb * BITS / 8;
    const int64_t k_bytes = (int64_t)p.K * BITS / 8;

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = zero16();

    const int ktiles = (p.K + MX_BK - 1) / MX_BK;
    for (int kt = 0; kt < ktiles; ++kt) {
        const int64_t kb0 = (int64_t)kt * T::BYTES;
        load_tile_mx<FMT>(A, lda_b, !p.a_cm, p.M, k_bytes, m0, kb0, As);
        load_tile_mx<FMT>(B, ldb_b, p.b_cm, p.N, k_bytes, n0, kb0, Bs);
        __syncthreads();
        const int kb = kt * (MX_BK / 32) + (lane >> 5);
        intx8 fa[2], fb[2];
        int sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int r = wm * 64 + i * 32 + (lane & 31);
            fa[i] = mx_fragment<FMT>(&As[r * T::ROW], lane >> 5);
            sa[i] = scale_byte(p.SA, p.ld_sa, p.M, nblk, m0 + r, kb);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int c = wn * 64 + j * 32 + (lane & 31);
            fb[j] = mx_fragment<FMT>(&Bs[c * T::ROW], lane >> 5);
            sb[j] = scale_byte(p.SB, p.ld_sb, p.N, nblk, n0 + c, kb);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = mfma_mx<FMT, 0>(fa[i], fb[j], acc[i][j], sa[i], sb[j]);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int row = m0 + wm * 64 + i * 32 + acc_row(r, lane);
                int col = n0 + wn * 64 + j * 32 + acc_col(lane);
                if (row < p.M && col < p.N)
                    store_c(p, row, col, acc[i][j][r]);
            }
}

// C <- beta * C (alpha == 0 or K == 0): A and B are not read.
__global__ __launch_bounds__(256) void scale_c(GemmArgs p)
{
    int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= p.N)
        return;
    for (int row = blockIdx.y; row < p.M; row += gridDim.y) {
        size_t idx = (size_t)row * p.ldc + col;
        if (p.c_dtype == OUT_F32) {
            float *c = (float *)p.C;
            c[idx] = p.beta == 0.0f ? 0.0f : p.beta * c[idx];
        } else {
            uint16_t *c = (uint16_t *)p.C;
            c[idx] = p.beta == 0.0f ? (uint16_t)0 : f32_to_bf16_rne(p.beta * bf16_to_f32(c[idx]));
        }
    }
}

} // namespace

hipError_t launch_simple_bf16(int level, const GemmArgs &p, hipStream_t s)
{
    dim3 block(256);
    if (level == 1) {
        hipLaunchKernelGGL(gemm_simple_bf16<false>, dim3(1, 1), block, 0, s, p);
    } else if (level == 2) {
        hipLaunchKernelGGL(gemm_simple_bf16<true>, dim3(1, 1), block, 0, s, p);
    } else {
        dim3 grid(((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM));
        hipLaunchKernelGGL(gemm_simple_bf16<true>, grid, block, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_simple_mx(const GemmArgs &p, hipStream_t s)
{
    dim3 grid(((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM));
    switch (p.mx_fmt) {
    case MX_E4M3: hipLaunchKernelGGL(gemm_simple_mx<MX_E4M3>, grid, dim3(256), 0, s, p); break;
    case MX_E5M2: hipLaunchKernelGGL(gemm_simple_mx<MX_E5M2>, grid, dim3(256), 0, s, p); break;
    case MX_E2M3: hipLaunchKernelGGL(gemm_simple_mx<MX_E2M3>, grid, dim3(256), 0, s, p); break;
    case MX_E3M2: hipLaunchKernelGGL(gemm_simple_mx<MX_E3M2>, grid, dim3(256), 0, s, p); break;
    case MX_E2M1: hipLaunchKernelGGL(gemm_simple_mx<MX_E2M1>, grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_scale_c(const GemmArgs &p, hipStream_t s)
{
    dim3 grid((p.N + 255) / 256, p.M < 4096 ? p.M : 4096);
    hipLaunchKernelGGL(scale_c, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

} // namespace mce
