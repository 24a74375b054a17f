// GEMM with one short side (M or N at most 64): the operand along the long
// side is streamed from HBM once, so the roofline is HBM bandwidth ("B200
// GEMM Optimization Ladder", section B: skinny shapes are bound by
// bandwidth, not by the matrix cores; section A1 levels 4-6: staged loads on
// a multi-stage ring).  Both kernels take bf16 operands (FMT = SK_BF16) or
// 8-bit MX operands (E4M3 / E5M2 with one E8M0 scale per 32 K: "B200 TMEM
// Lifecycle Planner", section A1 case 2).  Either way a K chunk is 128 bytes
// of every row (64 bf16 or 128 8-bit elements), read as four 16-byte pieces
// per lane: for bf16 the A and B fragments of four 32x32x16 k-steps, for MX
// those of two 32x32x64 k-steps (pieces 2ks and 2ks + 1 are the two halves
// of k-step ks), plus one 32-bit word of four scale bytes per row.
//
// Short side at most 32 (gemm_skinny): a workgroup computes a tile of C
// holding all of the short side (NB = 1 block of 32; the kernel also takes
// NB = 2) and 32 rows or columns of the long side, so a 1 x 8192 x 8192
// problem has 256 workgroups.  (Short side 33-64: gemm_skinny_lds below.)  Each of its eight waves (two per SIMD)
// owns one 32 x 32 block: with two blocks, waves 0-3 take the first and
// 4-7 the second.  The G = 8 / NB waves of a block split K by whole
// K chunks, interleaved (wave g takes chunks g, g + G, ...: side by side
// the group reads contiguous pieces of every row), the whole sequence
// rotated by a workgroup-dependent offset so that workgroups running side by
// side read different offsets of their 2^n-byte-strided rows.  A wave loads
// its fragments straight into registers in the matrix-core layout (lane l:
// row l % 32, 16 bytes at 16 (l / 32) of each 32-byte piece of the chunk);
// the four pieces of a chunk are issued back to back, so each row's 128
// bytes reach the L2 together.  D chunks are in flight per wave in a
// register ring;
// chunks past the wave's range read through zero-record resources (no
// memory touched, zeros that add nothing), so the loop has no branch.  At
// the end the other waves of a block pass their partial accumulators
// through LDS and its first wave sums them in wave order and stores the
// block.  No memory beyond the operands and C is used.
#include "kernels_fast.hpp"

namespace mce {
namespace {

struct SkinnyGeom {
    static constexpr int TI = 1, TJ = 1, WM = 32, WN = 32;   // one 32x32 block per wave
};

constexpr int SK_BF16 = -1;                          // FMT of bf16 operands
constexpr int SK_CHUNK = 128;                        // bytes of a row per K chunk
constexpr int SK_WAVES = 8;

template <int FMT>
struct SkOp {
    static constexpr bool MX = FMT != SK_BF16;
    static constexpr int ELT = MX ? 1 : 2;           // bytes per element
    static constexpr int BK = SK_CHUNK / ELT;        // K elements per chunk
};

// One chunk's products of a 32 x 32 block from its four 16-byte pieces per
// operand (pieces j: bytes 32j + 16h .. +15 of the chunk) and, for MX, the
// rows' scale words (lane l: row l % 32's word shifted down a byte for
// l >= 32, so op_sel 2ks picks block 2ks for k 0..31 of k-step ks and block
// 2ks + 1 for k 32..63).
template <int FMT>
__device__ __forceinline__ void chunk_mma(floatx16 &acc, const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], int sa,
                                          int sb)
{
    if constexpr (FMT == SK_BF16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = mfma_bf16(fb[ks], fa[ks], acc);
    } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const intx4 al = __builtin_bit_cast(intx4, fa[2 * ks]), ah = __builtin_bit_cast(intx4, fa[2 * ks + 1]);
            const intx4 bl = __builtin_bit_cast(intx4, fb[2 * ks]), bh = __builtin_bit_cast(intx4, fb[2 * ks + 1]);
            const intx8 a8 = {al[0], al[1], al[2], al[3], ah[0], ah[1], ah[2], ah[3]};
            const intx8 b8 = {bl[0], bl[1], bl[2], bl[3], bh[0], bh[1], bh[2], bh[3]};
            if (ks == 0)
                acc = mfma_mx<FMT, 0>(b8, a8, acc, sb, sa);
            else
                acc = mfma_mx<FMT, 2>(b8, a8, acc, sb, sa);
        }
    }
}

template <int FMT, int NB, bool MSHORT, int D, int EPI>
__global__ __launch_bounds__(64 * SK_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_skinny(GemmArgs p)
{
    using Op = SkOp<FMT>;
    constexpr int BM = MSHORT ? 32 * NB : 32, BN = MSHORT ? 32 : 32 * NB;
    constexpr int G = SK_WAVES / NB;                 // waves per block
    constexpr int LOADS = Op::MX ? 10 : 8;           // loads per chunk and lane
    static_assert((D - 1) * LOADS < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) float red[NB * (G - 1) * 16 * 64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int blk = wave / G, kw = wave % G;
    const int bi = MSHORT ? blk : 0, bj = MSHORT ? 0 : blk;

    const int tiles_n = (p.N + BN - 1) / BN;
    const int slot = xcd_major(blockIdx.x, gridDim.x);
    const int m0 = (slot / tiles_n) * BM + 32 * bi, n0 = (slot % tiles_n) * BN + 32 * bj;
    const int ra = p.M - m0 < 32 ? p.M - m0 : 32, rb = p.N - n0 < 32 ? p.N - n0 : 32;

    const int nch = p.K / Op::BK;
    const int n = (nch - kw + G - 1) / G;            // chunks kw, kw + G, ...
    const int rot = (int)(((unsigned)slot * 41u) % (unsigned)nch);

    // the block's rows as buffer resources ending at the last valid row's K
    // (rows past M or N read as zeros; a block entirely past them reads
    // nothing), and zero-record twins for the chunks past the wave's range;
    // the K offset goes in the scalar offset
    const char *pa = (const char *)p.A + (size_t)(ra > 0 ? m0 : 0) * p.lda * Op::ELT;
    const char *pb = (const char *)p.B + (size_t)(rb > 0 ? n0 : 0) * p.ldb * Op::ELT;
    const uint32_t na = ra > 0 ? (uint32_t)(((size_t)(ra - 1) * p.lda + p.K) * Op::ELT) : 0u;
    const uint32_t nb = rb > 0 ? (uint32_t)(((size_t)(rb - 1) * p.ldb + p.K) * Op::ELT) : 0u;
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(pa, na), rsb = make_rsrc(pb, nb);
    const __amdgpu_buffer_rsrc_t rsa0 = make_rsrc(pa, 0u), rsb0 = make_rsrc(pb, 0u);
    const uint32_t va = (uint32_t)(l32 * p.lda * Op::ELT + 16 * h), vb = (uint32_t)(l32 * p.ldb * Op::ELT + 16 * h);
    // MX: the scale rows likewise (K / 32 bytes per row)
    const uint8_t *psa = Op::MX ? p.SA + (size_t)(ra > 0 ? m0 : 0) * p.ld_sa : nullptr;
    const uint8_t *psb = Op::MX ? p.SB + (size_t)(rb > 0 ? n0 : 0) * p.ld_sb : nullptr;
    const __amdgpu_buffer_rsrc_t rssa = make_rsrc(psa, Op::MX && ra > 0 ? (uint32_t)((ra - 1) * p.ld_sa + p.K / 32) : 0u);
    const __amdgpu_buffer_rsrc_t rssb = make_rsrc(psb, Op::MX && rb > 0 ? (uint32_t)((rb - 1) * p.ld_sb + p.K / 32) : 0u);
    const __amdgpu_buffer_rsrc_t rssa0 = make_rsrc(psa, 0u), rssb0 = make_rsrc(psb, 0u);
    const uint32_t vsa = (uint32_t)(l32 * p.ld_sa), vsb = (uint32_t)(l32 * p.ld_sb);

    bf16x8 fa[D][4], fb[D][4];                       // the register ring: D chunks
    int sa[D], sb[D];                                // MX: the chunk's scale words
    auto load = [&](int c, int d) {
        const bool live = c < n;
        const __amdgpu_buffer_rsrc_t ta = live ? rsa : rsa0, tb = live ? rsb : rsb0;
        int idx = kw + G * c + rot;
        idx = idx >= nch ? idx - nch : idx;
        const int soff = idx * SK_CHUNK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            fa[d][j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ta, va, soff + j * 32, 0));
            fb[d][j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(tb, vb, soff + j * 32, 0));
        }
        if constexpr (Op::MX) {
            sa[d] = (int)__builtin_amdgcn_raw_buffer_load_b32(live ? rssa : rssa0, vsa, idx * 4, 0);
            sb[d] = (int)__builtin_amdgcn_raw_buffer_load_b32(live ? rssb : rssb0, vsb, idx * 4, 0);
        } else {
            sa[d] = sb[d] = 0;
        }
    };

    floatx16 acc[1][1];
    acc[0][0] = zero16();
#pragma unroll
    for (int d = 0; d < D; ++d)
        load(d, d);
    for (int c = 0; c < n; c += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            // chunk c + d has landed; the D - 1 newer chunks may be in flight
            wait_vmcnt<(D - 1) * LOADS>();
            const int ssa = (int)((uint32_t)sa[d] >> (8 * h)), ssb = (int)((uint32_t)sb[d] >> (8 * h));
            chunk_mma<FMT>(acc[0][0], fa[d], fb[d], ssa, ssb);
            load(c + d + D, d);
        }
    }
    wait_vmcnt<0>();

    // reduce each block's G partial accumulators (wave order) into its
    // first wave, which stores the block
    if (kw > 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            red[((blk * (G - 1) + kw - 1) * 16 + r) * 64 + lane] = acc[0][0][r];
    }
    __syncthreads();
    if (kw == 0) {
        for (int w = 0; w < G - 1; ++w)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[0][0][r] += red[((blk * (G - 1) + w) * 16 + r) * 64 + lane];
        if (ra > 0 && rb > 0)
            store_tile<EPI, SkinnyGeom, 32, 32>(p, acc, m0, n0, 0, 0, h, l32);
    }
}

// Short side 33-64: a workgroup tile of (32 TI) x (32 TJ) (TI or TJ = 2),
// four waves splitting K into contiguous ranges of whole chunks, each with
// its own S-stage LDS ring filled by 1 KiB direct loads (eight 128-byte rows
// per load, swz8 chunk swizzle) and no barrier; for MX one more direct load
// per operand brings the 64 rows' scale words of the chunk (rows past the
// tile or the matrix read as zeros).  The short operand's rows, read by every
// workgroup, arrive as whole rows of a chunk instead of the register path's
// 32-byte row segments, which measured faster here.
template <int TI_, int TJ_>
struct SkinnyLdsGeom {
    static constexpr int TI = TI_, TJ = TJ_;
    static constexpr int WM = 32 * TI_, WN = 32 * TJ_;   // wave 0 stores the whole tile
};

template <int FMT, int TI, int TJ, int S, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_skinny_lds(GemmArgs p)
{
    using G = SkinnyLdsGeom<TI, TJ>;
    using Op = SkOp<FMT>;
    constexpr int BM = 32 * TI, BN = 32 * TJ;
    constexpr int NLA = BM / 8, NLB = BN / 8;
    constexpr int LOADS = NLA + NLB + (Op::MX ? 2 : 0);
    constexpr int SC = Op::MX ? 2 * 64 * 4 : 0;      // the A and B scale words of a chunk (64 rows each)
    constexpr int STAGE = (BM + BN) * SK_CHUNK + SC;
    constexpr int RING = S * STAGE;
    constexpr int RED = 3 * TI * TJ * 16 * 64 * 4;
    constexpr int LDS = 4 * RING > RED ? 4 * RING : RED;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(S >= 2 && (S - 2) * LOADS < 64, "ring depth");
    __shared__ __attribute__((aligned(1024))) char smem[LDS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_n = (p.N + BN - 1) / BN;
    const int slot = xcd_major(blockIdx.x, gridDim.x);
    const int m0 = (slot / tiles_n) * BM, n0 = (slot % tiles_n) * BN;
    const int ra = p.M - m0 < BM ? p.M - m0 : BM, rb = p.N - n0 < BN ? p.N - n0 : BN;

    // this wave's K chunks [c0, c0 + n)
    const int nch = p.K / Op::BK;
    const int c0 = nch * wave / 4, n = nch * (wave + 1) / 4 - c0;

    const __amdgpu_buffer_rsrc_t rsa = make_rsrc((const char *)p.A + (size_t)m0 * p.lda * Op::ELT,
                                                 (uint32_t)(((size_t)(ra - 1) * p.lda + p.K) * Op::ELT));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc((const char *)p.B + (size_t)n0 * p.ldb * Op::ELT,
                                                 (uint32_t)(((size_t)(rb - 1) * p.ldb + p.K) * Op::ELT));
    const uint8_t *psa = Op::MX ? p.SA + (size_t)m0 * p.ld_sa : nullptr;
    const uint8_t *psb = Op::MX ? p.SB + (size_t)n0 * p.ld_sb : nullptr;
    const __amdgpu_buffer_rsrc_t rssa = make_rsrc(psa, Op::MX ? (uint32_t)((ra - 1) * p.ld_sa + p.K / 32) : 0u);
    const __amdgpu_buffer_rsrc_t rssb = make_rsrc(psb, Op::MX ? (uint32_t)((rb - 1) * p.ld_sb + p.K / 32) : 0u);
    const int lrow = lane >> 3;
    char *ring = smem + wave * RING;

    // load t of a stage: rows 8t .. 8t + 7, lane l row 8t + l / 8 at
    // physical chunk l % 8, fetching logical chunk (l % 8) ^ swz8(row); MX:
    // lane l fetches the scale word of row l
    auto issue = [&](int c, int stage) {
        char *base = ring + stage * STAGE;
        const int soff = (c0 + c) * SK_CHUNK;
#pragma unroll
        for (int t = 0; t < NLA; ++t) {
            const int row = 8 * t + lrow;
            const uint32_t voff = (uint32_t)(row * p.lda * Op::ELT + (((lane & 7) ^ swz8(row)) * 16));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(base + t * 1024), 16, voff, soff, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NLB; ++t) {
            const int row = 8 * t + lrow;
            const uint32_t voff = (uint32_t)(row * p.ldb * Op::ELT + (((lane & 7) ^ swz8(row)) * 16));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(base + BM * SK_CHUNK + t * 1024), 16, voff,
                                                     soff, 0, 0);
        }
        if constexpr (Op::MX) {
            char *sbase = base + (BM + BN) * SK_CHUNK;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rssa, (lds_ptr_t)sbase, 4, (uint32_t)(lane * p.ld_sa),
                                                     (c0 + c) * 4, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rssb, (lds_ptr_t)(sbase + 256), 4, (uint32_t)(lane * p.ld_sb),
                                                     (c0 + c) * 4, 0, 0);
        }
    };

    floatx16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            acc[i][j] = zero16();

    const int swz = swz8(l32);
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (st < n)
            issue(st, st);
    int stage = 0;
    for (int c = 0; c < n; ++c) {
        // chunk c has landed: at most the S - 2 newer chunks' loads remain
        const int newer = n - 1 - c < S - 2 ? n - 1 - c : S - 2;
        if (newer >= S - 2)
            wait_vmcnt<(S - 2) * LOADS>();
        else if (newer == 1)
            wait_vmcnt<LOADS>();
        else
            wait_vmcnt<0>();
        // the stage read in the previous chunk (its reads are done: the
        // matrix-core instructions consumed them) takes chunk c + S - 1
        if (c + S - 1 < n)
            issue(c + S - 1, stage == 0 ? S - 1 : stage - 1);
        const char *base = ring + stage * STAGE;
        bf16x8 fa[TI][4], fb[TJ][4];
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
                fa[i][j4] = *(const bf16x8 *)(base + (i * 32 + l32) * SK_CHUNK + (((2 * j4 + h) ^ swz) << 4));
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                fb[j][j4] = *(const bf16x8 *)(base + (BM + j * 32 + l32) * SK_CHUNK + (((2 * j4 + h) ^ swz) << 4));
        }
        int sa[TI], sb[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i)
            sa[i] = Op::MX ? (int)(*(const uint32_t *)(base + (BM + BN) * SK_CHUNK + (i * 32 + l32) * 4) >> (8 * h)) : 0;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            sb[j] = Op::MX ? (int)(*(const uint32_t *)(base + (BM + BN) * SK_CHUNK + 256 + (j * 32 + l32) * 4) >> (8 * h))
                           : 0;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                chunk_mma<FMT>(acc[i][j], fa[i], fb[j], sa[i], sb[j]);
        stage = stage == S - 1 ? 0 : stage + 1;
    }

    // reduce the four waves' partial tiles (wave order 0 + 1 + 2 + 3)
    wait_lgkm0();
    __syncthreads();
    float *red = (float *)smem;
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    red[(((wave - 1) * TI * TJ + i * TJ + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] += red[((w * TI * TJ + i * TJ + j) * 16 + r) * 64 + lane];
        store_tile<EPI, G, BM, BN>(p, acc, m0, n0, 0, 0, h, l32);
    }
}

template <int FMT, int TI, int TJ, int S>
hipError_t launch_skinny_lds(const GemmArgs &p, hipStream_t s)
{
    constexpr int BM = 32 * TI, BN = 32 * TJ;
    const long grid = (long)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    if (whole_bf16(p, BM, BN))
        hipLaunchKernelGGL((gemm_skinny_lds<FMT, TI, TJ, S, EPI_BF16_WHOLE>), dim3((unsigned)grid), dim3(256), 0, s,
                           p);
    else
        hipLaunchKernelGGL((gemm_skinny_lds<FMT, TI, TJ, S, EPI_ANY>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int FMT, int NB, bool MSHORT, int D>
hipError_t launch_skinny_t(const GemmArgs &p, hipStream_t s)
{
    constexpr int BM = MSHORT ? 32 * NB : 32, BN = MSHORT ? 32 : 32 * NB;
    const long grid = (long)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    if (whole_bf16(p, BM, BN))
        hipLaunchKernelGGL((gemm_skinny<FMT, NB, MSHORT, D, EPI_BF16_WHOLE>), dim3((unsigned)grid),
                           dim3(64 * SK_WAVES), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_skinny<FMT, NB, MSHORT, D, EPI_ANY>), dim3((unsigned)grid), dim3(64 * SK_WAVES), 0,
                           s, p);
    return hipGetLastError();
}

// the short side (the smaller one when both are short) takes the blocks:
// at most 32 the register-ring kernel, 33-64 the LDS-ring kernel
template <int FMT>
hipError_t launch_skinny_fmt(const GemmArgs &p, hipStream_t s)
{
    const bool mshort = p.M <= 64 && (p.N > 64 || p.M <= p.N);
    const int shortside = mshort ? p.M : p.N;
    if (shortside <= 32)
        return mshort ? launch_skinny_t<FMT, 1, true, 4>(p, s) : launch_skinny_t<FMT, 1, false, 4>(p, s);
    return mshort ? launch_skinny_lds<FMT, 2, 1, 3>(p, s) : launch_skinny_lds<FMT, 1, 2, 3>(p, s);
}

} // namespace

bool skinny_eligible(const GemmArgs &p)
{
    return (p.M <= 64 || p.N <= 64) && p.K >= SK_WAVES * SkOp<SK_BF16>::BK && p.K % SkOp<SK_BF16>::BK == 0 &&
           p.a_cm == 0 && p.b_cm == 1 && p.lda % 8 == 0 && p.ldb % 8 == 0 && (uintptr_t)p.A % 16 == 0 &&
           (uintptr_t)p.B % 16 == 0;
}

hipError_t launch_skinny_bf16(const GemmArgs &p, hipStream_t s)
{
    if (!skinny_eligible(p))
        return hipErrorInvalidValue;
    return launch_skinny_fmt<SK_BF16>(p, s);
}

bool skinny_mx_eligible(const GemmArgs &p)
{
    return (p.mx_fmt == MX_E4M3 || p.mx_fmt == MX_E5M2) && (p.M <= 64 || p.N <= 64) &&
           p.K >= SK_WAVES * SkOp<MX_E4M3>::BK && p.K % SkOp<MX_E4M3>::BK == 0 && p.a_cm == 0 && p.b_cm == 1 &&
           p.lda % 16 == 0 && p.ldb % 16 == 0 && (uintptr_t)p.A % 16 == 0 && (uintptr_t)p.B % 16 == 0 &&
           p.ld_sa % 4 == 0 && p.ld_sb % 4 == 0 && (uintptr_t)p.SA % 4 == 0 && (uintptr_t)p.SB % 4 == 0;
}

hipError_t launch_skinny_mx(const GemmArgs &p, hipStream_t s)
{
    if (!skinny_mx_eligible(p))
        return hipErrorInvalidValue;
    return p.mx_fmt == MX_E4M3 ? launch_skinny_fmt<MX_E4M3>(p, s) : launch_skinny_fmt<MX_E5M2>(p, s);
}

} // namespace mce
