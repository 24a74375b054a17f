// Fused attention forward on the matrix cores: for every batch b, head h and
// query row i,  o(i,:) = softmax_j(scale * q(i,:) . k(j,:)) v(j,:),  with bf16
// Q, K, V, fp32 accumulation and an online softmax, the score (S),
// probability (P) and output (O) tiles living in registers and LDS ("B200
// TMEM Lifecycle Planner", section A2 trigger 2 and section E steps 1-7: the
// S/P/O tiles of attention, their storage, reuse and hand-offs; here the
// accumulator store is the register file and the staging store LDS).
//
// Workgroup: 128 query rows of one (batch, head), four waves of 32 rows;
// keys in tiles of 64.  Per key tile and wave:
//   S (32 x 64)  = Q (32 x D) . K^T        two 32x32 blocks, D/16 k-steps each
//   online softmax on S (base 2), P = bf16(exp2(S - m))
//   O (32 x D)  += P (32 x 64) . V         D/32 blocks, four k-steps each
// on v_mfma_f32_32x32x16_bf16.  Both products feed the "B" side first, so
// every accumulator holds its block transposed: lane l owns query row l % 32
// and 16 columns (8q + 4h + c, h = l / 32), so row maxima and sums stay in a
// lane, plus one exchange with lane l ^ 32.
//
// The columns of S are keys in a permuted order: column j = 8q + 4h + c is
// key pi(j) = 16(q >> 1) + 8h + 4(q & 1) + c of its 32-key block (the K row
// the instruction's lane j % 32 reads).  Then the eight accumulators
// 8t .. 8t+7 of a lane are keys 16t + 8h .. 16t + 8h + 7 of the block in
// order, exactly the P operand a lane supplies for k-step t of the P V
// product: P goes from the S accumulators to that product with no exchange
// between lanes.
//
// Data movement per key tile: the K and V tiles (64 rows of D bf16 each) by
// direct loads (buffer_load ... lds, bounds-checked: keys past seq_k read as
// zero) into double-buffered, XOR-swizzled LDS tiles stored as in memory.  A
// P V operand fragment (eight consecutive keys of one d) is two transposing
// LDS reads (ds_read_b64_tr_b16: each lane addresses 4 d of one key row and
// receives one d of four key rows), so V needs no pass through registers.
// One barrier per key tile: the loads of tile j+1 are in flight while tile
// j is consumed.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "attn_layout.hpp"
#include "sched.hpp"

namespace mce {
namespace {

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 *lds_v4i16_t;

constexpr int ABM = 128;   // query rows per workgroup
constexpr int ABN = 64;    // keys per key tile

template <int D>
struct AttnGeom {
    static constexpr int ROWK = D * 2;                 // bytes per K row in LDS
    static constexpr int CHK = ROWK / 16;              // 16-byte chunks per K row
    static constexpr int K_BYTES = ABN * ROWK;         // one K tile
    static constexpr int V_BYTES = K_BYTES;            // one V tile, the same layout
    static constexpr int LDS = 2 * (K_BYTES + V_BYTES);
    static constexpr int KS = D / 16;                  // k-steps of S
    static constexpr int DB = D / 32;                  // 32-column blocks of O
    static constexpr int KLOADS = K_BYTES / 1024 / 4;  // K (and V) direct loads per wave and tile
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
};

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm_0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void sync_wg() { asm volatile("s_barrier" ::: "memory"); }

template <int D, bool CAUSAL, bool NEG, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_fwd(AttnArgs a)
{
    using G = AttnGeom<D>;
    __shared__ __attribute__((aligned(1024))) char smem[G::LDS];
    char *kbuf = smem;                          // [2][K_BYTES]
    char *vbuf = smem + 2 * G::K_BYTES;         // [2][V_BYTES]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;

    // workgroup -> (batch*head, query tile): XCD-major slots, so the query
    // tiles of one head (sharing its K and V) run on one XCD's L2; the
    // heaviest causal tiles first
    const int n_qt = (a.seq_q + ABM - 1) / ABM;
    const int slot = xcd_major(blockIdx.x, gridDim.x);
    const int bh = slot / n_qt;
    const int qt = n_qt - 1 - slot % n_qt;
    const int q0 = qt * ABM;
    const int row = q0 + wave * 32 + l32;       // this lane's query row

    const size_t qo_base = (size_t)bh * a.seq_q * D;
    const size_t kv_base = (size_t)bh * a.seq_k * D;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(a.Q + qo_base, (uint32_t)((size_t)a.seq_q * D * 2));

    // keys this tile of query rows may see
    const int kv_end_vis = CAUSAL ? q0 + ABM - 1 + a.seq_k - a.seq_q + 1 : a.seq_k;
    const int kv_end = kv_end_vis < a.seq_k ? kv_end_vis : a.seq_k;
    const int ntiles = kv_end > 0 ? (kv_end + ABN - 1) / ABN : 0;
    const int diag = row + a.seq_k - a.seq_q;   // causal: last key this row sees

    // Q fragments: lane (row, h), k-step s: d = 16s + 8h .. +7
    bf16x8 qf[G::KS];
#pragma unroll
    for (int s = 0; s < G::KS; ++s) {
        const uint32_t off = (uint32_t)((row * D + 16 * s + 8 * h) * 2);
        const intx4 v = __builtin_bit_cast(intx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rq, row < a.seq_q ? off : OOB_OFFSET, 0, 0));
        qf[s] = __builtin_bit_cast(bf16x8, v);
    }

    // K tile loads: this wave's KLOADS direct loads of 1 KiB; lane l writes
    // row (wave*KLOADS + t) * RPL + l / CHK at physical chunk l % CHK and so
    // fetches logical chunk (l % CHK) ^ swz_attn_k(row).  Each tile gets a
    // buffer resource based at its first key whose record count ends at
    // seq_k (keys past it read as zeros), so a lane's offsets are constants.
    constexpr int RPL = 1024 / G::ROWK;
    uint32_t kvoff[G::KLOADS], vvoff[G::KLOADS];
#pragma unroll
    for (int t = 0; t < G::KLOADS; ++t) {
        const int r = (wave * G::KLOADS + t) * RPL + lane / G::CHK;
        kvoff[t] = (uint32_t)((r * D + ((lane % G::CHK) ^ swz_attn_k(r, D)) * 8) * 2);
        vvoff[t] = (uint32_t)((r * D + ((lane % G::CHK) ^ swz_attn_v(r, D)) * 8) * 2);
    }
    auto tile_rsrc = [&](const uint16_t *base, int tile) {
        const int key0 = tile * ABN;
        const int left = a.seq_k - key0;
        return make_rsrc(base + kv_base + (size_t)key0 * D, left > 0 ? (uint32_t)left * D * 2 : 0u);
    };
    auto issue_k = [&](int tile, int buf) {
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(a.K, tile);
#pragma unroll
        for (int t = 0; t < G::KLOADS; ++t) {
            const uint32_t voff = kvoff[t];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (lds_ptr_t)(kbuf + buf * G::K_BYTES + (wave * G::KLOADS + t) * 1024), 16, voff, 0, 0,
                0);
        }
    };
    // The V tile likewise (its own swizzle)
    auto issue_v = [&](int tile, int buf) {
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(a.V, tile);
#pragma unroll
        for (int t = 0; t < G::KLOADS; ++t) {
            const uint32_t voff = vvoff[t];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (lds_ptr_t)(vbuf + buf * G::V_BYTES + (wave * G::KLOADS + t) * 1024), 16, voff, 0, 0,
                0);
        }
    };
    // P V operand of block b (d = 32b + l % 32), keys 8h .. 8h + 7 of k-step
    // ts, from two transposing reads q = 0, 1: in 16-lane group g = (l % 32)
    // / 16, lane L = l % 16 addresses key row 16 ts + 8h + 4q + L / 4 at
    // d = 32b + 16g + 4 (L % 4) (8 bytes), and receives d = 32b + 16g + L of
    // the four key rows 16 ts + 8h + 4q .. +3.  The key rows' swizzle
    // depends only on L / 4 (the rest is a multiple of 4), so each block's
    // address is a lane constant plus (16 ts + 4q) rows.
    int vaddr[G::DB];
    {
        const int L = lane & 15, g = l32 >> 4;
        const int r = 8 * h + (L >> 2);
#pragma unroll
        for (int b = 0; b < G::DB; ++b) {
            const int d = 32 * b + 16 * g + 4 * (L & 3);
            vaddr[b] = r * G::ROWK + (((2 * d) >> 4) ^ swz_attn_v(r, D)) * 16 + ((2 * d) & 15);
        }
    }
    auto read_vf = [&](int buf, int b, int ts) -> bf16x8 {
        const char *p0 = vbuf + buf * G::V_BYTES + vaddr[b] + 16 * ts * G::ROWK;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)p0);
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(p0 + 4 * G::ROWK));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    floatx16 o_acc[G::DB];
#pragma unroll
    for (int b = 0; b < G::DB; ++b)
        o_acc[b] = zero16();
    // Reference maximum of this row in base-2 logits (-inf: no visible key
    // yet).  It moves only when a tile's maximum exceeds it by more than
    // TAU, so most tiles skip the rescale of O; the probabilities exp2(x -
    // m_ref) are then at most 2^TAU, which fp32 sums and bf16 hold with the
    // same relative rounding.
    constexpr float TAU = 8.0f;
    float m_ref = -__builtin_inff();
    float l_run = 0.0f;                // this lane's share of the row's normaliser
    const float c = a.scale_log2;
    const float ninf = -__builtin_inff();
    // raw scores are ranked by s * c: by their maximum for c >= 0, their
    // minimum for c < 0 (NEG)
    auto better = [](float x, float y) { return NEG ? __builtin_fminf(x, y) : __builtin_fmaxf(x, y); };

    // K row read by this lane for the S products, and its swizzle
    const int krow = attn_key_of_col(l32);
    const int kswz = swz_attn_k(krow, D);   // rows 32b + krow share it (b adds no low bits)

    if (ntiles > 0) {
        issue_k(0, 0);
        issue_v(0, 0);
        wait_vm0();
        sync_wg();
    }
    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool more = j + 1 < ntiles;
        if (more) {
            issue_k(j + 1, buf ^ 1);
            issue_v(j + 1, buf ^ 1);
        }
        // Causal: a key tile wholly past the diagonal of this wave's last row
        // is masked for every row of the wave (its probabilities are zero
        // and its maximum -inf), so the wave skips its products and softmax
        // and only takes part in the loads and the barrier.
        const int key0 = j * ABN;
        if (!CAUSAL || key0 <= q0 + 32 * wave + 31 + a.seq_k - a.seq_q) {
            // ---- S = Q K^T (two 32-key blocks): the two blocks' accumulators
            // alternate (independent chains), and each k-step's K fragments are
            // read one k-step ahead of their products
            const char *kb = kbuf + buf * G::K_BYTES;
            floatx16 sacc[2];
            sacc[0] = zero16();
            sacc[1] = zero16();
            {
                const char *krp0 = kb + krow * G::ROWK, *krp1 = kb + (32 + krow) * G::ROWK;
                bf16x8 kf[2][2];
                kf[0][0] = *(const bf16x8 *)(krp0 + (h ^ kswz) * 16);
                kf[0][1] = *(const bf16x8 *)(krp1 + (h ^ kswz) * 16);
#pragma unroll
                for (int s = 0; s < G::KS; ++s) {
                    if (s + 1 < G::KS) {
                        kf[(s + 1) & 1][0] = *(const bf16x8 *)(krp0 + ((2 * (s + 1) + h) ^ kswz) * 16);
                        kf[(s + 1) & 1][1] = *(const bf16x8 *)(krp1 + ((2 * (s + 1) + h) ^ kswz) * 16);
                    }
                    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s & 1][0], qf[s], sacc[0], 0, 0, 0);
                    sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s & 1][1], qf[s], sacc[1], 0, 0, 0);
                }
            }
            // ---- online softmax.  Tiles that every row of this wave sees
            // whole skip the mask.
            const bool whole = key0 + ABN <= a.seq_k &&
                               (!CAUSAL || key0 + ABN - 1 <= q0 + 32 * wave + a.seq_k - a.seq_q);
            // this tile's maximum logit of the row (-inf: nothing visible); on
            // masked tiles the scores are scaled here and masked keys set to
            // -inf, so the exponent below multiplies by 1 instead of c
            float tm;
            if (whole) {
                float ext = sacc[0][0];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        ext = better(ext, sacc[blk][r]);
                tm = ext * c;
            } else {
                tm = ninf;
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + 32 * blk + attn_key_of_col(8 * (r >> 2) + 4 * h + (r & 3));
                        const bool vis = key < a.seq_k && (!CAUSAL || key <= diag);
                        sacc[blk][r] = vis ? sacc[blk][r] * c : ninf;
                        tm = __builtin_fmaxf(tm, sacc[blk][r]);
                    }
            }
            const float c_eff = whole ? c : 1.0f;
            tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32));
            if (__builtin_amdgcn_ballot_w64(tm > m_ref + TAU)) {
                const float m_new = __builtin_fmaxf(m_ref, tm);
                const float alpha = m_new == ninf ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
                m_ref = m_new;
                l_run *= alpha;
#pragma unroll
                for (int b = 0; b < G::DB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o_acc[b][r] *= alpha;
            }
            const float mu = m_ref == ninf ? 0.0f : m_ref;
            float psum = 0.0f;
            bf16x8 pf[2][2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][8 * t + e], c_eff, -mu));
                        psum += pr;
                        pf[blk][t][e] = (__bf16)pr;
                    }
                }
            l_run += psum;
            // ---- O += P V (four k-steps of 16 keys): the DB blocks of O
            // alternate within each k-step (independent chains), and each
            // k-step's V fragments are read one k-step ahead
            {
                bf16x8 vf[2][G::DB];
#pragma unroll
                for (int b = 0; b < G::DB; ++b)
                    vf[0][b] = read_vf(buf, b, 0);
#pragma unroll
                for (int ts = 0; ts < 4; ++ts) {
                    if (ts + 1 < 4) {
#pragma unroll
                        for (int b = 0; b < G::DB; ++b)
                            vf[(ts + 1) & 1][b] = read_vf(buf, b, ts + 1);
                    }
#pragma unroll
                    for (int b = 0; b < G::DB; ++b)
                        o_acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ts & 1][b], pf[ts >> 1][ts & 1], o_acc[b],
                                                                           0, 0, 0);
                }
            }
        }
        // ---- the barrier: every wave's reads of this tile are done and
        // the next tile's K and V are in LDS
        wait_vm0();
        wait_lgkm_0();
        sync_wg();
    }

    // ---- epilogue: normalise, convert, store (rows past seq_q are not stored)
    const float l_row = l_run + __shfl_xor(l_run, 32);
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
    if (row < a.seq_q) {
#pragma unroll
        for (int b = 0; b < G::DB; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 32 * b + 8 * q + 4 * h;
                const size_t idx = qo_base + (size_t)row * D + d;
                const floatx16 &o = o_acc[b];
                if constexpr (OUT == OUT_BF16) {
                    *(u16x4 *)((uint16_t *)a.O + idx) =
                        u16x4{f32_to_bf16_rne(o[4 * q] * inv), f32_to_bf16_rne(o[4 * q + 1] * inv),
                              f32_to_bf16_rne(o[4 * q + 2] * inv), f32_to_bf16_rne(o[4 * q + 3] * inv)};
                } else {
                    *(floatx4 *)((float *)a.O + idx) =
                        floatx4{o[4 * q] * inv, o[4 * q + 1] * inv, o[4 * q + 2] * inv, o[4 * q + 3] * inv};
                }
            }
    }
    wait_vm0();
}

template <int D, bool CAUSAL, bool NEG>
hipError_t launch_attn_s(const AttnArgs &a, hipStream_t s)
{
    const int n_qt = (a.seq_q + ABM - 1) / ABM;
    const long grid = (long)a.batch * a.heads * n_qt;
    if (a.o_dtype == OUT_BF16)
        hipLaunchKernelGGL((attention_fwd<D, CAUSAL, NEG, OUT_BF16>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((attention_fwd<D, CAUSAL, NEG, OUT_F32>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t s)
{
    return a.scale_log2 < 0.0f ? launch_attn_s<D, CAUSAL, true>(a, s) : launch_attn_s<D, CAUSAL, false>(a, s);
}

} // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t s)
{
    if (a.dim == 64)
        return a.causal ? launch_attn_d<64, true>(a, s) : launch_attn_d<64, false>(a, s);
    if (a.dim == 128)
        return a.causal ? launch_attn_d<128, true>(a, s) : launch_attn_d<128, false>(a, s);
    return hipErrorInvalidValue;
}

} // namespace mce
