// MX FP6 (E2M3, E3M2) levels 5-6: a three-stage direct-load pipeline for
// the block-scaled instruction's 6-bit formats ("B200 TMEM Lifecycle
// Planner", section A1 case 2: the block-scaled MMA with per-block scale
// factors staged beside the operands; "B200 GEMM Optimization Ladder",
// section A1 levels 4-6: staged loads, a multi-stage pipeline, a persistent
// grid).
//
// The 6-bit elements are packed along K (four per three bytes).  Lane l of
// v_mfma_scale_f32_32x32x64_f8f6f4 holds the 32 elements k = 32h .. 32h+31
// (h = l / 32) of row l % 32, element e at bit 6e: 24 contiguous bytes of
// the row, at byte 48 ks + 24 h of a 64-element k-step.  A K tile is 128
// elements, 96 bytes per row, two k-steps; operand rows sit in LDS at a
// 96-byte pitch, filled by 16-byte direct loads (1 KiB per load, rows
// straddling loads), and a fragment is three 8-byte reads (the 24 bytes are
// 8-byte but not 16-byte aligned for the upper half-wave).
//
// Bank conflicts: an 8-byte read serves 32 lanes per cycle over 64 banks,
// and the 32 lanes of a half-wave read rows r .. r+31 at one offset.  At a
// 96-byte pitch rows r, r+8, r+16, r+24 start on the same bank; swapping
// the 16-byte chunks of each pair (0,1), (2,3), (4,5) in rows with bit 3
// set moves r+8 and r+24 off them.  Rows r and r+16 still share banks: with
// 16-byte direct-load granularity every lane's piece has the same parity of
// 8-byte slot, so 32 lanes reach only 32 of the 64 banks' 8-byte pairs and
// two-way is the floor.
//
// Scales: one aligned 4-byte word per row and K tile (its four 32-element
// blocks); the upper half-wave takes the word shifted one byte down so
// op_sel 2 ks selects block 2 ks + h.  With K a multiple of 512 and 16-byte
// aligned scale rows they arrive in groups: the 16 bytes of each row for
// four K tiles, one 16-byte direct load per lane and 64 rows, double-buffered
// beside the three stages (a 4-byte load per lane and row for every K tile
// spends as many cache-line requests on 256 bytes as a 1 KiB operand load;
// measured, those loads alone took a fifth of the kernel's time).
// Otherwise each stage carries its K tile's words, staged by 4-byte direct
// loads and read at a 4-byte pitch (conflict-free).
//
// Pipeline: three stages, one barrier per K tile, placed between the K
// tile's two k-steps (see the main loop): fragment reads overlap matrix-core
// work on both sides of it, and three K tiles of loads are in flight.
#include "kernels_fast.hpp"

#include <type_traits>

namespace mce {
namespace {

struct Fp6Geom {
    static constexpr int WM = 128, WN = 128;   // wave tile
    static constexpr int TI = 4, TJ = 4;       // 32x32 blocks per wave tile
};

constexpr int FP6_BM = 256, FP6_BN = 256;
constexpr int FP6_BK = 128;                    // K elements per K tile
constexpr int FP6_ROWB = FP6_BK * 6 / 8;       // 96 bytes per LDS operand row
constexpr int FP6_S = 3;                       // stages
constexpr int FP6_A_BYTES = FP6_BM * FP6_ROWB, FP6_B_BYTES = FP6_BN * FP6_ROWB;
constexpr int FP6_NL = FP6_A_BYTES / 1024 / 4;   // 6 operand loads per wave, operand and K tile
static_assert(FP6_A_BYTES % 4096 == 0, "whole 1 KiB loads per wave");

// Stage layout: operands, then (without scale groups) the K tile's scale
// words; with scale groups two group buffers of 16 bytes per row follow the
// stages.
template <bool SG>
struct Fp6Ring {
    static constexpr int STAGE = FP6_A_BYTES + FP6_B_BYTES + (SG ? 0 : (FP6_BM + FP6_BN) * 4);
    static constexpr int GROUP = (FP6_BM + FP6_BN) * 16;
    static constexpr int LDS = FP6_S * STAGE + (SG ? 2 * GROUP : 0);
    static constexpr int LOADS = 2 * FP6_NL + (SG ? 0 : 2);   // loads per wave and K tile
    static constexpr int GLOADS = SG ? 2 : 0;                 // loads per wave and scale group
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(2 * LOADS + 2 * GLOADS < 64, "vmcnt range");
};

typedef int intx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int fp6_swz(int row) { return (row >> 3) & 1; }

template <int FMT, bool SG, bool PERSIST, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp6(GemmArgs p, int group_m)
{
    using G = Fp6Geom;
    using R = Fp6Ring<SG>;
    constexpr int BM = FP6_BM, BN = FP6_BN, ROWB = FP6_ROWB, NL = FP6_NL;
    constexpr int TI = G::TI, TJ = G::TJ;
    constexpr int FP6_STAGE = R::STAGE, FP6_LOADS = R::LOADS;
    __shared__ __attribute__((aligned(1024))) char smem[R::LDS];
    char *const groups = smem + FP6_S * FP6_STAGE;   // scale groups: 2 x R::GROUP

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = p.K / FP6_BK;                   // >= 1 (host guarantees)
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = wg_slot(wg, nwg, p.xcd_order);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;
    auto tile_of = [&](int r) { return PERSIST ? persistent_tile_id(wg, nwg, r, p.xcd_order) : first; };

    // bytes per operand row in memory (lda, ldb multiples of 64 elements:
    // 48-byte multiples, so every 16-byte chunk is aligned)
    const int lda_b = p.lda / 4 * 3, ldb_b = p.ldb / 4 * 3;
    const int krow_b = p.K / 4 * 3;                // bytes of K per row

    // Direct-load addressing: load t of this wave fills LDS bytes
    // 1024 (wave NL + t) + 16 lane of the operand's stage area, i.e. row
    // q / 96 at physical chunk (q % 96) / 16, which holds logical chunk
    // physical ^ fp6_swz(row) of the row's K tile.
    uint32_t vo_a[NL], vo_b[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
        const int q = (wave * NL + t) * 1024 + lane * 16;
        const int row = q / ROWB;
        const int lc = ((q % ROWB) >> 4) ^ fp6_swz(row);
        vo_a[t] = (uint32_t)(row * lda_b + lc * 16);
        vo_b[t] = (uint32_t)(row * ldb_b + lc * 16);
    }
    const int srow = wave * 64 + lane;             // scale row this lane loads
    const uint32_t vs_a = (uint32_t)(srow * p.ld_sa), vs_b = (uint32_t)(srow * p.ld_sb);

    // the r-th tile's operand and scale rows as buffer resources whose
    // record count ends at the tile's last valid row (rows past M or N read
    // as zeros); past the workgroup's last tile every count is zero
    struct Span {
        const char *a, *b, *sa, *sb;
        uint32_t na, nb, nsa, nsb;
    };
    auto span = [&](int r) {
        Span t{(const char *)p.A, (const char *)p.B, (const char *)p.SA, (const char *)p.SB, 0, 0, 0, 0};
        if (r < my_tiles) {
            int tm, tn;
            grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
            const int m0 = tm * BM, n0 = tn * BN;
            const int ra = p.M - m0 < BM ? p.M - m0 : BM, rb = p.N - n0 < BN ? p.N - n0 : BN;
            t.a += (size_t)m0 * lda_b;
            t.b += (size_t)n0 * ldb_b;
            t.sa += (size_t)m0 * p.ld_sa;
            t.sb += (size_t)n0 * p.ld_sb;
            t.na = (uint32_t)((size_t)(ra - 1) * lda_b + krow_b);
            t.nb = (uint32_t)((size_t)(rb - 1) * ldb_b + krow_b);
            t.nsa = (uint32_t)((ra - 1) * p.ld_sa + p.K / 32);
            t.nsb = (uint32_t)((rb - 1) * p.ld_sb + p.K / 32);
        }
        return t;
    };

    // K tile kt of tile span t into `stage`.  Past the last K tile the
    // record counts are zero: the loads fetch nothing (and write zeros that
    // nothing reads), so every K tile issues the same loads and waits the
    // same counts, and the loop body has no branch for the compiler to move
    // matrix-core work across.
    auto issue = [&](const Span &t, int kt, int stage) {
        char *base = smem + stage * FP6_STAGE;
        const int soff = kt * ROWB;
        const bool live = kt < nk;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(t.a, live ? t.na : 0u), rb = make_rsrc(t.b, live ? t.nb : 0u);
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const uint32_t voff = vo_a[u];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + (wave * NL + u) * 1024), 16, voff,
                                                     soff, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const uint32_t voff = vo_b[u];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_ptr_t)(base + FP6_A_BYTES + (wave * NL + u) * 1024), 16, voff, soff, 0, 0);
        }
        if constexpr (!SG) {
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(t.sa, live ? t.nsa : 0u),
                                         rsb = make_rsrc(t.sb, live ? t.nsb : 0u);
            char *sbase = base + FP6_A_BYTES + FP6_B_BYTES;
            const uint32_t voa = vs_a, vob = vs_b;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(sbase + wave * 256), 4, voa, kt * 4, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(sbase + BM * 4 + wave * 256), 4, vob,
                                                     kt * 4, 0, 0);
        }
    };
    // Scale group gi (K tiles 4 gi .. 4 gi + 3) of tile span t into group
    // buffer gi % 2: lane l brings the 16 bytes of row 64 wave + l.  Past the
    // last group the record counts are zero (zeros land in a buffer nothing
    // reads again).
    auto issue_group = [&](const Span &t, int gi) {
        if constexpr (SG) {
            char *gb = groups + (gi & 1) * R::GROUP;
            const bool live = 4 * gi < nk;
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(t.sa, live ? t.nsa : 0u),
                                         rsb = make_rsrc(t.sb, live ? t.nsb : 0u);
            const uint32_t voa = vs_a, vob = vs_b;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(gb + wave * 1024), 16, voa, gi * 16, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(gb + BM * 16 + wave * 1024), 16, vob,
                                                     gi * 16, 0, 0);
        }
    };

    // fragment of k-step ks from the row at `rowp`: bytes 48 ks + 24 h ..
    // +23 as three 8-byte pieces; the instruction reads six registers
    const int swz = fp6_swz(l32);                  // rows a lane reads differ by multiples of 32
    auto frag = [&](const char *rowp, int ks) -> intx8 {
        intx2 pc[3];
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int byte = 48 * ks + 24 * h + 8 * m;
            pc[m] = *(const intx2 *)(rowp + (((byte >> 4) ^ swz) << 4) + (byte & 8));
        }
        const intx4 lo = __builtin_shufflevector(pc[0], pc[1], 0, 1, 2, 3);
        const intx4 hi = __builtin_shufflevector(pc[2], pc[2], 0, 1, -1, -1);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, -1, -1);
    };

    floatx16 acc[TI][TJ];
    auto read_ks = [&](int stage, int ks, intx8 (&fa)[TI], intx8 (&fb)[TJ]) {
        const char *base = smem + stage * FP6_STAGE;
#pragma unroll
        for (int i = 0; i < TI; ++i)
            fa[i] = frag(base + (wm * G::WM + i * 32 + l32) * ROWB, ks);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            fb[j] = frag(base + FP6_A_BYTES + (wn * G::WN + j * 32 + l32) * ROWB, ks);
    };
    // the scale words of K tile kt (in `stage`, or word kt % 4 of the rows'
    // 16 bytes in group buffer (kt / 4) % 2)
    auto read_sc = [&](int stage, int kt, int (&sa)[TI], int (&sb)[TJ]) {
        constexpr int PITCH = SG ? 4 : 1;          // words per row
        const uint32_t *sw = SG ? (const uint32_t *)(groups + ((kt >> 2) & 1) * R::GROUP) + (kt & 3)
                                : (const uint32_t *)(smem + stage * FP6_STAGE + FP6_A_BYTES + FP6_B_BYTES);
#pragma unroll
        for (int i = 0; i < TI; ++i)
            sa[i] = (int)(sw[(wm * G::WM + i * 32 + l32) * PITCH] >> (8 * h));
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            sb[j] = (int)(sw[(BM + wn * G::WN + j * 32 + l32) * PITCH] >> (8 * h));
    };
    // k-step ks of the K tile; B first, so lane l holds row l % 32 of each
    // C block and columns 8q + 4h .. +3 (the layout the epilogue stores)
    auto mma = [&](auto ks_tag, const intx8 (&fa)[TI], const intx8 (&fb)[TJ], const int (&sa)[TI],
                   const int (&sb)[TJ]) {
        constexpr int KS = decltype(ks_tag)::value;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = mfma_mx<FMT, 2 * KS>(fb[j], fa[i], acc[i][j], sb[j], sa[i]);
    };

    // Per K tile kt (stage s = kt % 3): k-step 1's fragments are read while
    // k-step 0 runs; then the wait for tile kt + 1's loads and the barrier,
    // after which no wave reads stage s (its reads are done) and tile kt + 3
    // goes into it (and, with scale groups, at the first K tile of group gi
    // group gi + 1 into the other group buffer, whose last reads, of K tile
    // 4 gi - 1, came before the previous barrier); then tile kt + 1's k-step
    // 0 fragments are read while k-step 1 of tile kt runs.  Three K tiles of
    // loads are in flight ahead of the one consumed.  The scheduling groups
    // interleave the fragment reads and loads with the matrix-core
    // instructions.
    intx8 f0a[TI], f0b[TJ], f1a[TI], f1b[TJ];
    int sa_c[TI], sb_c[TJ], sa_n[TI], sb_n[TJ];
    // loads issued after tile kt + 1's (the wait before K tile kt's
    // barrier): tile kt + 2's, and a group after tile kt + 3's (at kt - 1)
    // or tile kt + 2's (at kt - 2) when either of those K tiles began one
    auto k_tile = [&](const Span &t, const int kt, int &stage, auto q_c) {
        constexpr int Q = decltype(q_c)::value;    // kt % 4 (scale groups), else 0
        read_ks(stage, 1, f1a, f1b);
        mma(std::integral_constant<int, 0>{}, f0a, f0b, sa_c, sb_c);
#pragma unroll
        for (int u = 0; u < 12; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // an LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // a matrix-core instruction
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        // (matrix-core instructions touch no memory, so the barrier alone
        // would not keep them on their side of it)
        __builtin_amdgcn_sched_barrier(0);
        constexpr int AFTER = FP6_LOADS + ((SG && (Q == 1 || Q == 2)) ? R::GLOADS : 0);
        wait_vmcnt<AFTER>();
        wait_lgkm0();
        barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(t, kt + 3, stage);
        if constexpr (SG && Q == 0)
            issue_group(t, kt / 4 + 1);
        const int nstage = stage == 2 ? 0 : stage + 1;
        read_ks(nstage, 0, f0a, f0b);        // past the last K tile: unused
        read_sc(nstage, kt + 1, sa_n, sb_n);
        mma(std::integral_constant<int, 1>{}, f1a, f1b, sa_c, sb_c);
#pragma unroll
        for (int u = 0; u < 14; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);   // a direct load
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
#pragma unroll
        for (int i = 0; i < TI; ++i)
            sa_c[i] = sa_n[i];
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            sb_c[j] = sb_n[j];
        stage = nstage;
    };

    Span cur = span(0);
    for (int r = 0; r < my_tiles; ++r) {
        int tm, tn;
        grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
        // every wave is done reading the previous tile's stages and groups
        if (r > 0)
            barrier();
        issue_group(cur, 0);
        issue(cur, 0, 0);
        issue(cur, 1, 1);
        issue(cur, 2, 2);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = zero16();
        wait_vmcnt<2 * FP6_LOADS>();
        barrier();
        read_ks(0, 0, f0a, f0b);
        read_sc(0, 0, sa_c, sb_c);
        int stage = 0;
        if constexpr (SG) {
            // nk is a multiple of 4
            for (int kt = 0; kt < nk; kt += 4) {
                k_tile(cur, kt, stage, std::integral_constant<int, 0>{});
                k_tile(cur, kt + 1, stage, std::integral_constant<int, 1>{});
                k_tile(cur, kt + 2, stage, std::integral_constant<int, 2>{});
                k_tile(cur, kt + 3, stage, std::integral_constant<int, 3>{});
            }
        } else {
            for (int kt = 0; kt < nk; ++kt)
                k_tile(cur, kt, stage, std::integral_constant<int, 0>{});
        }
        store_tile<EPI, G, BM, BN>(p, acc, tm * BM, tn * BN, wm, wn, h, l32);
        cur = span(r + 1);
    }
    wait_vmcnt<0>();
}

template <int FMT, bool SG, bool PERSIST>
hipError_t launch_fp6(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + FP6_BM - 1) / FP6_BM, tiles_n = (p.N + FP6_BN - 1) / FP6_BN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = group_rows(tiles_m, p.group_m);
    if (PERSIST && ntiles <= p.ncu)
        return launch_fp6<FMT, SG, false>(p, s);
    const int grid = PERSIST ? (ntiles < p.ncu ? ntiles : p.ncu) : ntiles;
    if (whole_bf16(p, FP6_BM, FP6_BN))
        hipLaunchKernelGGL((gemm_fp6<FMT, SG, PERSIST, EPI_BF16_WHOLE>), dim3(grid), dim3(256), 0, s, p, group_m);
    else
        hipLaunchKernelGGL((gemm_fp6<FMT, SG, PERSIST, EPI_ANY>), dim3(grid), dim3(256), 0, s, p, group_m);
    return hipGetLastError();
}

// scale groups when K is a multiple of 512 and the scale rows are 16-byte
// aligned
template <int FMT>
hipError_t launch_fp6_fmt(bool persist, const GemmArgs &p, hipStream_t s)
{
    const bool sg = p.K % 512 == 0 && p.ld_sa % 16 == 0 && p.ld_sb % 16 == 0 && (uintptr_t)p.SA % 16 == 0 &&
                    (uintptr_t)p.SB % 16 == 0;
    if (sg)
        return persist ? launch_fp6<FMT, true, true>(p, s) : launch_fp6<FMT, true, false>(p, s);
    return persist ? launch_fp6<FMT, false, true>(p, s) : launch_fp6<FMT, false, false>(p, s);
}

} // namespace

// FP6 levels 5-6: K-contiguous operands with K a multiple of 128, lda and
// ldb multiples of 64 elements (48-byte row pitch multiples), 16-byte
// aligned A and B, 4-byte aligned scale rows.
hipError_t launch_fast_fp6(int level, const GemmArgs &p, hipStream_t s)
{
    if (p.K <= 0 || p.K % FP6_BK != 0 || p.lda % 64 != 0 || p.ldb % 64 != 0 || p.ld_sa % 4 != 0 ||
        p.ld_sb % 4 != 0 || (uintptr_t)p.A % 16 != 0 || (uintptr_t)p.B % 16 != 0 ||
        (uintptr_t)p.SA % 4 != 0 || (uintptr_t)p.SB % 4 != 0)
        return hipErrorInvalidValue;
    if (level != 5 && level != 6)
        return hipErrorInvalidValue;
    const bool persist = level == 6;
    if (p.mx_fmt == MX_E2M3)
        return launch_fp6_fmt<MX_E2M3>(persist, p, s);
    if (p.mx_fmt == MX_E3M2)
        return launch_fp6_fmt<MX_E3M2>(persist, p, s);
    return hipErrorInvalidValue;
}

} // namespace mce
