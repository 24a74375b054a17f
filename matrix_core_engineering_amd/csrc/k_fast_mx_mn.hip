// MX 8-bit (E4M3, E5M2) levels 5-6 with an MN-major operand (A column-major
// or B row-major): a direct-load pipeline whose MN-major tiles are read
// through the LDS transpose loads ("B200 TMEM Lifecycle Planner", section A1
// case 2: the block-scaled MMA; "B200 GEMM Optimization Ladder", section A1
// levels 4-6 and section E steps 4-7: staged loads, a multi-stage ring, a
// persistent grid).
//
// Operand fragments of v_mfma_scale_f32_32x32x64_f8f6f4 (8-bit): lane l
// (h = l / 32) holds row l % 32 of its 32-row block at k = 16h .. 16h + 15
// (registers 0-3) and 32 + 16h .. 32 + 16h + 15 (registers 4-7) of the
// 64-element k-step.
//
// K-contiguous operand: LDS rows of 128 bytes (the K tile of one row), the
// 16-byte chunks XOR-swizzled by swz8(row); a fragment is two 16-byte reads.
//
// MN-major operand: the K tile is staged as it lies in memory, 128 k-rows of
// the tile's 256 rows (256 bytes each), chunk c of k-row r at physical chunk
// c ^ mn_swz(r).  ds_read_b64_tr_b8 transposes bytes inside each 16-lane
// group: output lane i, byte b is byte i % 8 of the 8 bytes addressed by
// input lane 2b + i / 8 (measured on the device).  With input lane L of a
// group addressing k-row k0 + L / 2 at row offset m0 + 8 (L % 2), output lane
// i receives row m0 + i at k0 .. k0 + 7: a quarter of its fragment.  Four
// such reads (k0 = 16h, 16h + 8, 32 + 16h, 40 + 16h) fill the eight
// registers; lane groups 0-3 take rows m0 = 0, 16, 0, 16 of the block and h =
// 0, 0, 1, 1.  Each read touches eight consecutive k-rows and one chunk
// (both halves) per group; the swizzle puts the eight rows on eight
// distinct chunks of one parity, groups 0 and 1 (2 and 3) on opposite
// parities, so 32 lanes cover all 64 banks once.
//
// Pipeline: two stages; the barrier of each K tile sits between its two
// k-steps (as in the FP6 kernel), so a stage is free half a K tile early and
// two K tiles of loads are in flight.
#include "kernels_fast.hpp"
#include "mn_layout.hpp"

#include <type_traits>

namespace mce {
namespace {

struct MnGeom {
    static constexpr int WM = 128, WN = 128;
    static constexpr int TI = 4, TJ = 4;
};

constexpr int MN_BM = 256, MN_BN = 256;
constexpr int MN_BK = 128;                          // K elements (bytes) per K tile
constexpr int MN_OP_BYTES = 256 * MN_BK;            // one operand's K tile: 32 KiB either way
constexpr int MN_S = 2;
constexpr int MN_NL = MN_OP_BYTES / 1024 / 4;       // 8 direct loads per wave, operand and K tile

// Stage layout: the two operands' K tiles, then (without scale groups) the
// K tile's scale words; with scale groups (16 bytes per row for four K
// tiles, K a multiple of 512 and 16-byte aligned scale rows) two group
// buffers follow the stages.
template <bool SG>
struct MnRing {
    static constexpr int STAGE = 2 * MN_OP_BYTES + (SG ? 0 : (MN_BM + MN_BN) * 4);
    static constexpr int GROUP = (MN_BM + MN_BN) * 16;
    static constexpr int LDS = MN_S * STAGE + (SG ? 2 * GROUP : 0);
    static constexpr int LOADS = 2 * MN_NL + (SG ? 0 : 2);   // loads per wave and K tile
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(LOADS + 2 < 64, "vmcnt range");
};

typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 *lds_v2_t;

template <int FMT, bool A_MN, bool B_MN, bool SG, bool PERSIST, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_mn(GemmArgs p, int group_m)
{
    using G = MnGeom;
    using R = MnRing<SG>;
    constexpr int BM = MN_BM, BN = MN_BN, NL = MN_NL, TI = G::TI, TJ = G::TJ;
    constexpr int MN_STAGE = R::STAGE, MN_LOADS = R::LOADS;
    // (the LDS-staged epilogue of bf16 C with beta = 0: one buffer per wave
    // after the ring, of 32, 16 or 8 rows, whatever the ring leaves.  fp32
    // C, staged a block per round through buffers this small, measured
    // slower than the register path here and is not launched.)
    constexpr bool STAGED = EPI == EPI_BF16_LDS;
    constexpr int ERR = R::LDS + 4 * epi_wave_bytes<32>() <= 160 * 1024   ? 32
                        : R::LDS + 4 * epi_wave_bytes<16>() <= 160 * 1024 ? 16
                                                                          : 8;
    constexpr int EPI_BYTES = STAGED ? 4 * epi_wave_bytes<ERR>() : 0;
    static_assert(R::LDS + EPI_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[R::LDS + EPI_BYTES];
    char *const groups = smem + MN_S * MN_STAGE;   // scale groups: 2 x R::GROUP

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = p.K / MN_BK;                      // >= 1 (host guarantees)
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int first = wg_slot(wg, nwg, p.xcd_order);
    const int my_tiles = PERSIST ? (first < ntiles ? (ntiles - 1 - first) / nwg + 1 : 0) : 1;
    auto tile_of = [&](int r) { return PERSIST ? persistent_tile_id(wg, nwg, r, p.xcd_order) : first; };

    // Direct-load lane offsets, fixed for the kernel.  K-contiguous: load t
    // of this wave fills rows 8 (wave NL + t) .. +7, lane l row + l / 8 at
    // physical chunk l % 8 = logical ^ swz8(row); offset row * ld + 16
    // logical (the K tile moves in the scalar offset).  MN-major: load t
    // fills k-rows 4 (wave NL + t) .. +3, lane l k-row + l / 16 at physical
    // chunk l % 16 = logical ^ mn_swz(k-row); offset k-row * ld + 16
    // logical (the K tile moves in the resource base).
    auto lane_offset = [&](bool mn, int t, int ld) -> uint32_t {
        const int g = wave * NL + t;
        if (mn) {
            const int kr = 4 * g + (lane >> 4);
            return (uint32_t)(kr * ld + (((lane & 15) ^ mn_swz(kr)) << 4));
        }
        const int row = 8 * g + (lane >> 3);
        return (uint32_t)(row * ld + (((lane & 7) ^ swz8(row)) << 4));
    };
    uint32_t vo_a[NL], vo_b[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
        vo_a[t] = lane_offset(A_MN, t, p.lda);
        vo_b[t] = lane_offset(B_MN, t, p.ldb);
    }
    const int srow = wave * 64 + lane;
    const uint32_t vs_a = (uint32_t)(srow * p.ld_sa), vs_b = (uint32_t)(srow * p.ld_sb);

    // Tile spans: operand and scale bases and record counts.  K-contiguous:
    // rows of the tile, the count ending at its last valid row's K.
    // MN-major: the tile's first row in every k-row; a K tile's resource
    // starts at its k-row, and the count ends with the 16-byte chunk that
    // holds k-row K - 1's last valid row (the range check zeroes a whole
    // dword that reaches past the count, so ending at the row itself would
    // zero the last valid bytes; the rest of that aligned chunk cannot be on
    // another page).  k-rows past K read as zeros; rows past M or N inside a
    // k-row feed only rows and columns of C that are never stored.
    struct Span {
        const char *a, *b, *sa, *sb;
        int64_t na, nb;      // K-contiguous: record count; MN-major: bytes from the base to the end
        uint32_t nsa, nsb;
    };
    auto span = [&](int r) {
        Span t{(const char *)p.A, (const char *)p.B, (const char *)p.SA, (const char *)p.SB, 0, 0, 0, 0};
        if (r < my_tiles) {
            int tm, tn;
            grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
            const int m0 = tm * BM, n0 = tn * BN;
            const int ra = p.M - m0 < BM ? p.M - m0 : BM, rb = p.N - n0 < BN ? p.N - n0 : BN;
            if (A_MN) {
                t.a += m0;
                t.na = (int64_t)(p.K - 1) * p.lda + ((ra + 15) & ~15);
            } else {
                t.a += (size_t)m0 * p.lda;
                t.na = (int64_t)(ra - 1) * p.lda + p.K;
            }
            if (B_MN) {
                t.b += n0;
                t.nb = (int64_t)(p.K - 1) * p.ldb + ((rb + 15) & ~15);
            } else {
                t.b += (size_t)n0 * p.ldb;
                t.nb = (int64_t)(rb - 1) * p.ldb + p.K;
            }
            t.sa += (size_t)m0 * p.ld_sa;
            t.sb += (size_t)n0 * p.ld_sb;
            t.nsa = (uint32_t)((ra - 1) * p.ld_sa + p.K / 32);
            t.nsb = (uint32_t)((rb - 1) * p.ld_sb + p.K / 32);
        }
        return t;
    };

    // K tile kt of span t into `stage`; past the last K tile every record
    // count is zero (nothing fetched), so every K tile issues the same loads
    auto issue = [&](const Span &t, int kt, int stage) {
        char *base = smem + stage * MN_STAGE;
        const bool live = kt < nk;
        const int64_t kmn_a = (int64_t)kt * MN_BK * p.lda, kmn_b = (int64_t)kt * MN_BK * p.ldb;
        const __amdgpu_buffer_rsrc_t ra =
            A_MN ? make_rsrc(t.a + kmn_a, live ? (uint32_t)(t.na - kmn_a) : 0u)
                 : make_rsrc(t.a, live ? (uint32_t)t.na : 0u);
        const __amdgpu_buffer_rsrc_t rb =
            B_MN ? make_rsrc(t.b + kmn_b, live ? (uint32_t)(t.nb - kmn_b) : 0u)
                 : make_rsrc(t.b, live ? (uint32_t)t.nb : 0u);
        const int soff_a = A_MN ? 0 : kt * MN_BK, soff_b = B_MN ? 0 : kt * MN_BK;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const uint32_t voff = vo_a[u];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + (wave * NL + u) * 1024), 16, voff,
                                                     soff_a, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const uint32_t voff = vo_b[u];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_ptr_t)(base + MN_OP_BYTES + (wave * NL + u) * 1024), 16, voff, soff_b, 0, 0);
        }
        if constexpr (!SG) {
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(t.sa, live ? t.nsa : 0u),
                                         rsb = make_rsrc(t.sb, live ? t.nsb : 0u);
            char *sbase = base + 2 * MN_OP_BYTES;
            const uint32_t voa = vs_a, vob = vs_b;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(sbase + wave * 256), 4, voa, kt * 4, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(sbase + BM * 4 + wave * 256), 4, vob,
                                                     kt * 4, 0, 0);
        }
    };
    // Scale group gi (K tiles 4 gi .. 4 gi + 3) of span t into group buffer
    // gi % 2: lane l brings the 16 bytes of row 64 wave + l.
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

    // Fragment of k-step ks for the 32-row block starting at row `rb` of
    // the operand area `op`.
    const int swz_k = swz8(l32);                     // K-contiguous rows rb + l32, rb % 32 == 0
    const int tl = lane & 15, tg = lane >> 4;        // transpose reads: lane in group, group
    const int th = tg >> 1, ts = tg & 1;
    const int tkr = tl >> 1;                         // k-row inside the read's eight
    const int tsw = mn_swz(tkr);                     // the read's k-rows are 8-aligned
    auto frag = [&](bool mn, const char *op, int rb, int ks) -> intx8 {
        if (!mn) {
            const char *rowp = op + (rb + l32) * MN_BK;
            const intx4 lo = *(const intx4 *)(rowp + (((4 * ks + h) ^ swz_k) << 4));
            const intx4 hi = *(const intx4 *)(rowp + (((4 * ks + 2 + h) ^ swz_k) << 4));
            return intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        const int pchunk = ((rb >> 4) + ts) ^ tsw;
        intx2 q[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int kr = 64 * ks + 16 * th + 8 * (c & 1) + 32 * (c >> 1) + tkr;
            q[c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_v2_t)(op + kr * 256 + (pchunk << 4) + 8 * (tl & 1)));
        }
        return intx8{q[0].x, q[0].y, q[1].x, q[1].y, q[2].x, q[2].y, q[3].x, q[3].y};
    };

    floatx16 acc[TI][TJ];
    auto read_ks = [&](int stage, int ks, intx8 (&fa)[TI], intx8 (&fb)[TJ]) {
        const char *base = smem + stage * MN_STAGE;
#pragma unroll
        for (int i = 0; i < TI; ++i)
            fa[i] = frag(A_MN, base, wm * G::WM + i * 32, ks);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            fb[j] = frag(B_MN, base + MN_OP_BYTES, wn * G::WN + j * 32, ks);
    };
    // the scale words of K tile kt (in `stage`, or word kt % 4 of the rows'
    // 16 bytes in group buffer (kt / 4) % 2)
    auto read_sc = [&](int stage, int kt, int (&sa)[TI], int (&sb)[TJ]) {
        constexpr int PITCH = SG ? 4 : 1;          // words per row
        const uint32_t *sw = SG ? (const uint32_t *)(groups + ((kt >> 2) & 1) * R::GROUP) + (kt & 3)
                                : (const uint32_t *)(smem + stage * MN_STAGE + 2 * MN_OP_BYTES);
#pragma unroll
        for (int i = 0; i < TI; ++i)
            sa[i] = (int)(sw[(wm * G::WM + i * 32 + l32) * PITCH] >> (8 * h));
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            sb[j] = (int)(sw[(BM + wn * G::WN + j * 32 + l32) * PITCH] >> (8 * h));
    };
    // k-step ks: blocks 2ks (lanes 0-31) and 2ks + 1 (lanes 32-63) of the
    // K tile's scale word, byte 2ks after the upper half's one-byte shift;
    // B first, so lane l holds row l % 32 of each C block (the epilogue's
    // layout)
    auto mma = [&](auto ks_tag, const intx8 (&fa)[TI], const intx8 (&fb)[TJ], const int (&sa)[TI],
                   const int (&sb)[TJ]) {
        constexpr int KS = decltype(ks_tag)::value;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = mfma_mx<FMT, 2 * KS>(fb[j], fa[i], acc[i][j], sb[j], sa[i]);
    };

    intx8 f0a[TI], f0b[TJ], f1a[TI], f1b[TJ];
    int sa_c[TI], sb_c[TJ], sa_n[TI], sb_n[TJ];
    Span cur = span(0);
    for (int r = 0; r < my_tiles; ++r) {
        int tm, tn;
        grouped_tile(tile_of(r), tiles_m, tiles_n, group_m, tm, tn);
        if (r > 0)
            barrier();                               // the previous tile's stages and groups are free
        issue_group(cur, 0);
        issue(cur, 0, 0);
        issue(cur, 1, 1);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = zero16();
        wait_vmcnt<MN_LOADS>();
        barrier();
        read_ks(0, 0, f0a, f0b);
        read_sc(0, 0, sa_c, sb_c);
        int stage = 0;
        for (int kt = 0; kt < nk; ++kt) {
            read_ks(stage, 1, f1a, f1b);
            mma(std::integral_constant<int, 0>{}, f0a, f0b, sa_c, sb_c);
            // (matrix-core instructions touch no memory: keep them on their
            // side of the barrier)
            __builtin_amdgcn_sched_barrier(0);
            // tile kt + 1's loads have landed (none newer are in flight:
            // tile kt + 2 is issued below)
            wait_vmcnt<0>();
            wait_lgkm0();
            barrier();
            __builtin_amdgcn_sched_barrier(0);
            issue(cur, kt + 2, stage);
            // at a group's first K tile the next group into the other group
            // buffer, whose last reads (of K tile kt - 1) came before the
            // previous barrier; the next K tile's wait covers it
            if (SG && (kt & 3) == 0)
                issue_group(cur, kt / 4 + 1);
            const int nstage = stage ^ 1;
            read_ks(nstage, 0, f0a, f0b);            // past the last K tile: unused
            read_sc(nstage, kt + 1, sa_n, sb_n);
            mma(std::integral_constant<int, 1>{}, f1a, f1b, sa_c, sb_c);
#pragma unroll
            for (int i = 0; i < TI; ++i)
                sa_c[i] = sa_n[i];
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                sb_c[j] = sb_n[j];
            stage = nstage;
        }
        {
            const bool full = (tm + 1) * BM <= p.M && (tn + 1) * BN <= p.N;
            char *ebuf = smem + R::LDS + wave * epi_wave_bytes<ERR>();
            if constexpr (EPI == EPI_BF16_LDS)
                store_tile_lds<G, BM, BN, ERR>(p, acc, tm * BM, tn * BN, wm, wn, lane_id_here(), ebuf, full);
            else
                store_tile<EPI, G, BM, BN>(p, acc, tm * BM, tn * BN, wm, wn, h, l32);
        }
        cur = span(r + 1);
    }
    wait_vmcnt<0>();
}

template <int FMT, bool A_MN, bool B_MN, bool SG, bool PERSIST>
hipError_t launch_mn(const GemmArgs &p, hipStream_t s)
{
    const int tiles_m = (p.M + MN_BM - 1) / MN_BM, tiles_n = (p.N + MN_BN - 1) / MN_BN;
    const int ntiles = tiles_m * tiles_n;
    const int group_m = group_rows(tiles_m, p.group_m);
    if (PERSIST && ntiles <= p.ncu)
        return launch_mn<FMT, A_MN, B_MN, SG, false>(p, s);
    const int grid = PERSIST ? (ntiles < p.ncu ? ntiles : p.ncu) : ntiles;
    if (staged_bf16(p))
        hipLaunchKernelGGL((gemm_mx_mn<FMT, A_MN, B_MN, SG, PERSIST, EPI_BF16_LDS>), dim3(grid), dim3(256), 0,
                           s, p, group_m);
    else if (whole_bf16(p, MN_BM, MN_BN))
        hipLaunchKernelGGL((gemm_mx_mn<FMT, A_MN, B_MN, SG, PERSIST, EPI_BF16_WHOLE>), dim3(grid), dim3(256), 0,
                           s, p, group_m);
    else
        hipLaunchKernelGGL((gemm_mx_mn<FMT, A_MN, B_MN, SG, PERSIST, EPI_ANY>), dim3(grid), dim3(256), 0, s, p,
                           group_m);
    return hipGetLastError();
}

// scale groups when K is a multiple of 512 and the scale rows are 16-byte
// aligned
template <int FMT, bool A_MN, bool B_MN, bool PERSIST>
hipError_t launch_mn_sg(const GemmArgs &p, hipStream_t s)
{
    const bool sg = p.K % 512 == 0 && p.ld_sa % 16 == 0 && p.ld_sb % 16 == 0 && (uintptr_t)p.SA % 16 == 0 &&
                    (uintptr_t)p.SB % 16 == 0;
    return sg ? launch_mn<FMT, A_MN, B_MN, true, PERSIST>(p, s) : launch_mn<FMT, A_MN, B_MN, false, PERSIST>(p, s);
}

template <int FMT, bool PERSIST>
hipError_t launch_mn_layouts(const GemmArgs &p, hipStream_t s)
{
    const bool a_mn = p.a_cm != 0, b_mn = p.b_cm == 0;
    if (a_mn && b_mn)
        return launch_mn_sg<FMT, true, true, PERSIST>(p, s);
    if (a_mn)
        return launch_mn_sg<FMT, true, false, PERSIST>(p, s);
    if (b_mn)
        return launch_mn_sg<FMT, false, true, PERSIST>(p, s);
    return hipErrorInvalidValue;                     // both K-contiguous: the early-release ring
}

} // namespace

// 8-bit MX levels 5-6 with at least one MN-major operand: K a positive
// multiple of 128, 16-byte aligned operand bases and leading dimensions
// multiple of 16 bytes, 4-byte aligned scale rows.
hipError_t launch_fast_mx_mn(int level, const GemmArgs &p, hipStream_t s)
{
    if (p.K <= 0 || p.K % MN_BK != 0 || p.lda % 16 != 0 || p.ldb % 16 != 0 || p.ld_sa % 4 != 0 ||
        p.ld_sb % 4 != 0 || (uintptr_t)p.A % 16 != 0 || (uintptr_t)p.B % 16 != 0 ||
        (uintptr_t)p.SA % 4 != 0 || (uintptr_t)p.SB % 4 != 0 || (level != 5 && level != 6))
        return hipErrorInvalidValue;
    const bool persist = level == 6;
    if (p.mx_fmt == MX_E4M3)
        return persist ? launch_mn_layouts<MX_E4M3, true>(p, s) : launch_mn_layouts<MX_E4M3, false>(p, s);
    if (p.mx_fmt == MX_E5M2)
        return persist ? launch_mn_layouts<MX_E5M2, true>(p, s) : launch_mn_layouts<MX_E5M2, false>(p, s);
    return hipErrorInvalidValue;
}

} // namespace mce
