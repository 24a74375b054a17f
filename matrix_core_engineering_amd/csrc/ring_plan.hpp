// The early-release stage ring of gemm_early (levels 5 and 6) as data: the
// K-tile formats, the stage geometry, and the order of every step of the
// prologue and of one K-tile iteration, with each step's K tile, load range
// and wait count.  The kernel executes these tables step by step at compile
// time; tests/ring_model.cpp replays the same tables for four waves on the
// host and checks every ready and free edge of the ring ("B200 TMA Pipeline
// Designer", section E step 8: each stage's ready and free have a unique
// producer and consumer, checked before the kernel runs; section B: consuming
// right after a load is issued, or reusing a buffer before the readers are
// done, are the failure modes).  Pure constants: compiles on the host.
#pragma once

#include "formats.hpp"

namespace mce {

// ---------------------------------------------------------------- formats
//
// A K tile is 128 bytes of every A and B row (one LDS row).  Per format: AM
// matrix-core instructions in phase A (the K tile's fragment reads spread
// over them: four waves read LDS at about 108 B/clk per CU; AM need not be a
// whole k-step: the stage is free once every fragment is in registers); XM
// in phase X; LX and LY of a K tile's direct loads issued in phases X and Y
// (the address unit takes about one 1 KiB direct load per 21 clocks per CU,
// so the loads need phases X and Y to be long enough), the rest in the next
// phase A; the next K tile's first YK k-steps of fragments read whole in
// phase Y (into the registers of k-steps whose instructions all precede
// phase Y), then k-step YK's B fragments and its first YA A fragments, the
// rest in the next phase A (the instruction order needs A fragment i only
// from the (TJ*i)-th instruction on).
struct Bf16Ring64 {                   // 128-byte rows
    static constexpr int WAVES = 4;   // one wave per SIMD, 128x128 per wave
    static constexpr bool MX = false, SG = false, FP4 = false;
    static constexpr int EPU = 1;     // elements per K unit (FP4: two per byte)
    static constexpr int ELT = 2;
    static constexpr int BK = 64;
    static constexpr int NKS = 4;
    static constexpr int AM = 16, XM = 40, LX = 16, LY = 0, YA = 2, YK = 0;
    static constexpr bool S16 = false;
};
// bf16 on the 16x16x32 instruction, which sustains 4-7% more flops than
// 32x32x16 at the chip's power limit (measured with the ceiling loop): each
// wave's 128x128 tile is 8x8 blocks of 16x16, a K tile two k-steps of 32 K
// (128 instructions of 16 clocks, the same 32 fragment reads per K tile).
// A fragment is 16 rows x 32 K: lane l reads row l % 16 at logical chunk
// 4ks + l / 16 of its 128-byte row; the swizzle swz8h keeps both 16-lane
// read groups of every fragment read conflict-free.  Whole bf16 tiles with
// the LDS-staged epilogue only.
struct Bf16Ring64S16 : Bf16Ring64 {
    static constexpr bool S16 = true;
    static constexpr int NKS = 2;
    static constexpr int AM = 32, XM = 88, LX = 16, LY = 0, YA = 2, YK = 0;
};
struct Mxfp8Ring128 {                 // 128-byte rows
    static constexpr int WAVES = 4;
    static constexpr bool MX = true, SG = false, FP4 = false, S16 = false;
    static constexpr int EPU = 1;
    static constexpr int FMT = MX_E4M3;
    static constexpr int ELT = 1;
    static constexpr int BK = 128;
    static constexpr int NKS = 2;
    static constexpr int AM = 16, XM = 12, LX = 12, LY = 4, YA = 2, YK = 0;
};
// MX with K a multiple of 512 (whole groups of 16 scale blocks): the scale
// words of four K tiles travel together, 16 bytes per row, in a separate
// double-buffered area.  A 4-byte load per row and K tile touches as many
// cache lines as a 16-byte one, and 64 rows' worth per instruction doubled
// the K tile's line requests.
struct Mxfp8Ring128G : Mxfp8Ring128 {
    static constexpr bool SG = true;
    static constexpr int AM = 12, XM = 16, LX = 14, LY = 2, YA = 1, YK = 0;
};
// E5M2 elements have E4M3's byte layout and fragment map: the same kernels
// with the instruction's format code 1.
struct E5m2Ring128 : Mxfp8Ring128 {
    static constexpr int FMT = MX_E5M2;
};
struct E5m2Ring128G : Mxfp8Ring128G {
    static constexpr int FMT = MX_E5M2;
};
// FP4 (E2M1), two elements per byte.  The kernel runs in byte units (the
// host passes K, lda and ldb halved), so the loads are those of E4M3: a K
// tile is 128 bytes of a row = 256 elements = 8 scale blocks.  A lane's
// fragment of a k-step (64 elements, 32 bytes of the row) is the 16 bytes of
// its block, logical chunk 2ks + h, as for bf16; four k-steps per K tile;
// two scale words per row and K tile, a scale group (16 bytes per row)
// covers two K tiles.
struct Fp4Ring128G {
    static constexpr int WAVES = 4;
    static constexpr bool MX = true, SG = true, FP4 = true, S16 = false;
    static constexpr int EPU = 2;
    static constexpr int FMT = MX_E2M1;
    static constexpr int ELT = 1;
    static constexpr int BK = 128;    // K units (bytes) per K tile
    static constexpr int NKS = 4;
    static constexpr int AM = 16, XM = 40, LX = 16, LY = 0, YA = 2, YK = 0;
};

// Level 9: several consumers of one staged ring ("B200 GEMM Optimization
// Ladder", section A1 level 9 and section E step 10: more consumer groups
// sharing one staged operand so each staged byte feeds more matrix-core
// work).  Eight waves, two per SIMD, in two groups of four; each wave owns
// 128x64 of the 256x256 tile (128 accumulator registers, so two waves fit a
// SIMD's register file), and both groups consume every stage: each A row of
// a stage feeds four waves, each B row two.  A K tile carries half the
// matrix-core instructions per wave, so the phases are half as long; the
// other wave on the SIMD fills the gaps of each one's LDS reads and waits.
// Eight direct loads per wave and K tile.  MX formats with scale groups only
// (waves 0-3 load the A rows' scale words, waves 4-7 the B rows').
struct Bf16Ring64W8 : Bf16Ring64 {
    static constexpr int WAVES = 8;
    static constexpr int AM = 8, XM = 20, LX = 8, LY = 0, YA = 2, YK = 0;
};
// (phase split: AM 16 / XM 40 measured fastest of AM 12-24, XM 32-44, LX 6-8
// at 8192^3, within 1% of level 6 there and 1-3% faster at 4096^3)
struct Bf16Ring64S16W8 : Bf16Ring64S16 {
    static constexpr int WAVES = 8;
    static constexpr int AM = 16, XM = 40, LX = 8, LY = 0, YA = 2, YK = 0;
};
struct Mxfp8Ring128GW8 : Mxfp8Ring128G {
    static constexpr int WAVES = 8;
    static constexpr int AM = 6, XM = 8, LX = 7, LY = 1, YA = 1, YK = 0;
};
struct E5m2Ring128GW8 : Mxfp8Ring128GW8 {
    static constexpr int FMT = MX_E5M2;
};

// ---------------------------------------------------------------- geometry

template <class Op, int BM, int BN, int S>
struct RingGeometry {
    static constexpr int WAVES = Op::WAVES;                // 4 (2x2) or 8 (2x4)
    static constexpr int WAVES_N = WAVES / 2;
    static constexpr int ROWB = Op::BK * Op::ELT;          // 64 or 128 bytes per LDS row
    static constexpr int CH = ROWB / 16;                   // 16-byte chunks per row
    static constexpr int RPL = 1024 / ROWB;                // rows per direct load
    static constexpr int EPC = 16 / Op::ELT;               // K elements per chunk
    static constexpr int WM = BM / 2, WN = BN / WAVES_N;
    static constexpr int TI = WM / 32, TJ = WN / 32;
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    // one aligned 4-byte scale word per row (the four blocks containing the K
    // tile's blocks); a direct load of any size fills one 4-byte LDS slot per
    // lane
    static constexpr int SA_BYTES = Op::MX && !Op::SG ? BM * 4 : 0;
    static constexpr int SB_BYTES = Op::MX && !Op::SG ? BN * 4 : 0;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    static constexpr int LDS_BYTES = S * STAGE_BYTES;
    static constexpr int NA = BM / RPL / WAVES;            // direct loads per wave per K tile
    static constexpr int NB = BN / RPL / WAVES;
    static constexpr int NSA = Op::MX && !Op::SG ? 1 : 0;  // 4-byte scale loads: 64 rows each
    static constexpr int NSB = Op::MX && !Op::SG ? 1 : 0;
    static constexpr int LOADS = NA + NB + NSA + NSB;
    static_assert(WAVES == 4 || WAVES == 8, "four or eight waves");
    static_assert(WAVES == 4 || !Op::MX || Op::SG, "eight waves: MX with scale groups only");
    static_assert((ROWB == 64 && CH == 4 && RPL == 16) || (ROWB == 128 && CH == 8 && RPL == 8),
                  "64- or 128-byte LDS rows");
    static_assert(NA % 2 == 0 && NB % 2 == 0, "loads split in halves; swizzle parity");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((S - 2) * LOADS < 64, "vmcnt range");
    static_assert(!Op::MX || (BM == 256 && BN == 256), "MX scale loads assume 256-row tiles");
};

// Constants of the two-stage early-release ring for one format and tile.
template <class Op, int BM, int BN>
struct EarlyPlan {
    using G = RingGeometry<Op, BM, BN, 2>;
    static constexpr int NKS = Op::NKS;
    // matrix-core blocks of 32x32 (16x16 on the 16x16x32 format) per wave tile
    static constexpr bool S16 = Op::S16;
    static constexpr int BLK = S16 ? 16 : 32, TI = G::WM / BLK, TJ = G::WN / BLK;
    static constexpr int NM = TI * TJ;                      // matrix-core instructions per k-step
    static constexpr int RPF = Op::MX && !Op::FP4 ? 2 : 1;  // LDS reads per fragment
    static constexpr int BPK = Op::BK * Op::EPU / 32;       // scale blocks per K tile
    static constexpr int GK = 16 / BPK;                     // K tiles per scale group
    static constexpr int UNR = Op::SG ? GK : 1;             // K tiles per K-loop trip
    static constexpr int SW = BPK / 4;                      // scale words per row and K tile
    static constexpr int FRAG_READS = (TI + TJ) * RPF;
    static constexpr int AM = Op::AM;                       // phase A
    static constexpr int XM = Op::XM, YM = NKS * NM - AM - XM;   // phases X and Y
    static constexpr int LOADS = G::LOADS;
    static constexpr int LX = Op::LX, LY = Op::LY, LA = LOADS - LX - LY, YA = Op::YA, YK = Op::YK;
    // LDS: the two stages, then (scale groups) two buffers of 16 bytes per
    // A and B row
    static constexpr int SG_BYTES = Op::SG ? 2 * (BM + BN) * 16 : 0;
    // direct loads per wave for one scale group: one 16-byte load of 64 rows
    // per wave and operand with four waves, one of either operand with eight
    static constexpr int GROUP_LOADS = Op::SG ? 8 / G::WAVES : 0;
    static constexpr int WAVES = G::WAVES;
    static_assert(G::CH == 8, "128-byte LDS rows");
    static_assert(AM > 0 && XM > 0 && YM > 0 && LX > 0 && LY >= 0 && LA >= 0, "phase split");
    static_assert(YA >= 1 && YA <= TI, "first A fragment read in phase Y");
    static_assert(YK >= 0 && YK < NKS && AM + XM >= (YK + 1) * NM,
                  "phase Y overwrites only k-steps whose instructions precede it");
    static_assert(LX <= XM && LY <= YM && LA <= AM, "at most one load per matrix-core instruction");
    static_assert(!Op::SG || UNR % 2 == 0, "scale-word register sets alternate by unrolled copy");
};

// ------------------------------------------------------------------ steps
//
// Iteration g consumes K tile g (K tiles counted over all tiles of the
// workgroup), which sits in stage g % 2.  The prologue is iteration g = -1
// without its matrix-core work.
enum RingStep {
    RS_READ_TAIL,       // K tile g's fragments not read in the last phase Y
    RS_ISSUE_PENDING,   // direct loads [LX+LY, LOADS) of K tile g+1
    RS_MFMA_A,          // matrix-core instructions [0, AM) of K tile g
    RS_WAIT_LGKM,       // this wave's LDS reads have returned (lgkmcnt(0))
    RS_BARRIER,         // workgroup barrier
    RS_ISSUE_X,         // direct loads [0, LX) of K tile g+2
    RS_MFMA_X,          // instructions [AM, AM+XM)
    RS_WAIT_VM,         // at most LX of this wave's direct loads in flight
    RS_READ_HEAD,       // K tile g+1's first fragments
    RS_READ_SCALES,     // K tile g+1's scale words (MX)
    RS_ISSUE_Y,         // direct loads [LX, LX+LY) of K tile g+2
    RS_MFMA_Y,          // instructions [AM+XM, NKS*NM)
    RS_ISSUE_GROUP,     // scale groups: at a group's first K tile, the next group
    // prologue only
    RS_ISSUE_GROUP0,    // scale group 0
    RS_ISSUE_FIRST,     // every direct load of K tile g+1 = 0
    RS_ISSUE_SECOND,    // direct loads [0, LX+LY) of K tile g+2 = 1
    RS_WAIT_VM_PRO,     // at most LX+LY of this wave's direct loads in flight
    RS_NSTEPS
};

// The prologue (g = -1): K tile 0 whole and scale group 0, then K tile 1 but
// its last LA loads (the first phase A issues those: a direct load always
// writes LDS, so no placeholder load may target a stage in use); K tile 0's
// first fragments read once every wave's loads of it have landed.
constexpr int kEarlyPrologue[] = {RS_ISSUE_GROUP0, RS_ISSUE_FIRST, RS_ISSUE_SECOND, RS_WAIT_VM_PRO,
                                  RS_BARRIER, RS_READ_HEAD, RS_READ_SCALES};

// One K-tile iteration: phase A, barrier 1 (free: stage g % 2 read by every
// wave), phase X, barrier 2 (ready: K tile g+1 landed for every wave),
// phase Y.  The waits and barriers are also fences for the compiler's
// scheduler: no instruction moves across them.
constexpr int kEarlyLoop[] = {RS_READ_TAIL, RS_ISSUE_PENDING, RS_MFMA_A, RS_WAIT_LGKM, RS_BARRIER,
                              RS_ISSUE_X, RS_MFMA_X, RS_WAIT_VM, RS_BARRIER, RS_READ_HEAD,
                              RS_READ_SCALES, RS_ISSUE_Y, RS_MFMA_Y, RS_ISSUE_GROUP};

constexpr int kEarlyPrologueSteps = sizeof(kEarlyPrologue) / sizeof(kEarlyPrologue[0]);
constexpr int kEarlyLoopSteps = sizeof(kEarlyLoop) / sizeof(kEarlyLoop[0]);

// What one direct-load step issues: K tile g + ktile, loads [lo, hi) of
// that K tile (0 .. NA-1 the A rows, then B rows, then MX scale words), into
// stage (g + ktile) % 2.  ktile = 0 marks a step that issues nothing.
struct LoadStep {
    int ktile, lo, hi;
};

template <class P>
constexpr LoadStep load_step(int step)
{
    return step == RS_ISSUE_PENDING ? LoadStep{1, P::LX + P::LY, P::LOADS}
         : step == RS_ISSUE_X       ? LoadStep{2, 0, P::LX}
         : step == RS_ISSUE_Y       ? LoadStep{2, P::LX, P::LX + P::LY}
         : step == RS_ISSUE_FIRST   ? LoadStep{1, 0, P::LOADS}
         : step == RS_ISSUE_SECOND  ? LoadStep{2, 0, P::LX + P::LY}
                                    : LoadStep{0, 0, 0};
}

// Direct loads a wait step lets stay in flight (-1: not a direct-load wait).
template <class P>
constexpr int vm_wait(int step)
{
    return step == RS_WAIT_VM ? P::LX : step == RS_WAIT_VM_PRO ? P::LX + P::LY : -1;
}

// K tile (relative to g) whose stage a read step reads: READ_TAIL reads K
// tile g, READ_HEAD and READ_SCALES K tile g+1 (READ_SCALES reads the scale
// group buffer of that K tile's group when the format has scale groups, else
// the stage).  -1: not a read step.
constexpr int read_ktile(int step)
{
    return step == RS_READ_TAIL ? 0 : (step == RS_READ_HEAD || step == RS_READ_SCALES) ? 1 : -1;
}

// Scale groups (formats with SG): group q covers K tiles [q GK, (q+1) GK)
// and lives in group buffer q % 2.  RS_ISSUE_GROUP in iteration g issues
// group g / GK + 1 when g is a group's first K tile; RS_ISSUE_GROUP0 issues
// group 0.
constexpr int group_buffer(int q) { return q & 1; }

} // namespace mce
