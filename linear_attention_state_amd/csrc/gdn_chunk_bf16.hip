// Chunked Gated DeltaNet replay for gfx950: bf16 MFMA operands, fp32 accumulation and
// fp32 state.
//
// Recurrence (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.3,
// Eq. (1), state stored dv x dk so the key-space operator acts from the right):
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = S_t q_t.
//
// Chunked (WY) form used here, for a chunk of n <= 64 tokens entering with state S:
//   gamma_t = sum_{u<=t} g_u                          (log-space gate cumsum, g = log alpha)
//   L_ti    = beta_t e^{gamma_t - gamma_i} k_t.k_i     (i < t),  A = (I + L)^{-1}
//   U0      = A diag(beta) V,   W = A diag(beta e^gamma) K
//   U'      = U0 - W S^T                               (rows u_t of the per-token delta)
//   O       = diag(e^gamma) Q S^T + P U',   P_ti = e^{gamma_t - gamma_i} q_t.k_i (i <= t)
//   S      <- e^{gamma_n} S + U'^T diag(e^{gamma_n - gamma}) K
// This follows from unrolling the recurrence inside the chunk: with
// u_t = beta_t (v_t - alpha_t S_{t-1} k_t) one has S_t = alpha_t S_{t-1} + u_t k_t^T, and
// stacking u_t gives (I + L) U' = diag(beta) V - diag(beta e^gamma) K S^T.
//
// Precision: q, k, v enter the MFMAs as their exact bf16 inputs.  The unit diagonal of A
// is applied exactly in fp32 (U0 = diag(beta) V + (A - I) diag(beta) V, same for W).
// U' is split into bf16 hi + lo parts for the state update, and P and U' are both split
// for P U' (hi*hi + hi*lo + lo*hi).  Everything else is a single bf16 rounding.
//
// Work decomposition: one workgroup of DV/32 waves per (sequence, value head); two
// workgroups share a CU (LDS <= 80 KiB, <= 256 registers per lane) so that one's
// barriers and latencies hide behind the other's MFMA work.  Wave w owns value columns
// [32w, 32w + 32) of the state, kept in MFMA accumulator registers as S^T tiles (dk rows
// x 32 dv columns).  Per chunk:
//   P0  stage K (loaded one chunk ahead, with g and beta); gate cumsum and the exp2 tables;
//       issue this chunk's Q and V loads and the next chunk's K, g, beta loads
//   P1  K K^T lower 16x16 tiles on 16x16x32 MFMA, masked and decayed into L: the
//       off-diagonal blocks row-major in bf16 (LDS); the wave that forms a diagonal block
//       inverts it in registers at once, as (I - L)(I + L^2)(I + L^4)(I + L^8) (the block
//       is nilpotent), each product from bf16 hi / lo splits on 16x16x16 MFMA with fp32
//       accumulation; stage Q
//   P2  the rest of A = (I + L)^{-1}: wave j forms block column j of A - I by 16x16x16
//       MFMA merges.  The Q K^T tiles are spread over the waves (1, 3, 3, 3: wave 0 has the
//       longest merge chain)
//   P3  U0 (own value columns, V read straight from HBM in operand order) and -W (to LDS);
//       K^T operands come from the row-major K tile through LDS transpose reads
//   P4  P (bf16 hi/lo) to LDS, over the dead (A - I) tiles
//   P5  U' = U0 + (-W) S^T and Y = Q S^T in one pass over the state operands; then
//       O = e^gamma q_scale Y + P U', stored, and after it the state update
//       S <- e^{gamma_n} S + U'^T D K (the output accumulators are free by then)
// The state-only variant (WITH_O = false) drops Q, Q K^T, P and O.
//
// PREP = true is the first kernel of the split schedule (few heads): one workgroup per
// (sequence, chunk, value head) runs P0-P4 only -- nothing there depends on the state -- and
// writes the chunk's operands -W, K^T, P hi / lo, U0 and the gate tables to a record in the
// workspace as MFMA operand fragments; gdn_scan_split.hip then runs the state part with the
// state split along dv.
// An accumulator feeds the next product directly as its B operand: the contraction index
// is permuted the same way on both operands (see kperm()).
#include "gdn_mfma.h"

#include <type_traits>

namespace tr {
namespace {

using namespace gdn;

constexpr int RS_T = CH + 8;           // row stride (elements) of 64-column bf16 tiles
constexpr int RS_L = CH + 4;           // row stride of the fp32 L tile

// 32x32x16 MFMA layouts (lane l, half h = l / 32):
//   A operand: row l % 32, k = 8h + i;  B operand: column l % 32, k = 8h + i;
//   accumulator register j: row 8 (j / 4) + 4h + (j % 4), column l % 32.
// When an accumulator (rows = contraction index) is reused as a B operand, k-step s of
// 16 rows takes registers 8 (s % 2) .. 8 (s % 2) + 7 of row tile s / 2, which hold rows
// 16 s + {4h .. 4h+3} and 16 s + 8 + {4h .. 4h+3}.  kperm() reads a partner row in that
// same order, and the transpose reads below fetch token columns in it.
__device__ __forceinline__ int acc_row(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

__device__ __forceinline__ bf16x8 kperm(const bf16* row, int s, int h) {
    return cat(*reinterpret_cast<const bf16x4*>(row + 16 * s + 4 * h),
               *reinterpret_cast<const bf16x4*>(row + 16 * s + 8 + 4 * h));
}
__device__ __forceinline__ void acc_to_b_split(const f32x16& t, int s, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        bf16x2 h, l;
        split2(t[8 * (s & 1) + i], t[8 * (s & 1) + i + 1], h, l);
        hi[i] = h[0]; hi[i + 1] = h[1];
        lo[i] = l[0]; lo[i + 1] = l[1];
    }
}
__device__ __forceinline__ bf16x8 acc_to_b(const f32x16& t, int s) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)t[8 * (s & 1) + i];
    return r;
}
template <int DK, int DV>
struct Smem {
    bf16 K[CH][DK + 16];        // key rows (padding keeps the transpose reads conflict-free)
    bf16 Q[CH][DK + 8];         // query rows
    union {
        struct {
            bf16 Lb[CH][RS_T];      // L row-major in bf16 (off-diagonal blocks used): P1 .. P2
        } l;
        bf16 Wn[CH][DK + 8];    // -W rows: P3 .. P5
    } lw;
    union {
        struct { bf16 Nb[CH][RS_T]; bf16 Nbg[CH][RS_T]; } n;   // (A-I) diag(beta), (A-I) diag(beta e^g): P2 .. P3
        struct { bf16 Ph[CH][RS_T]; bf16 Pl[CH][RS_T]; } p;    // P hi / lo: P4 .. P5
    } np;
    bf16 Ad[4][16][24];         // diagonal 16x16 blocks of A (bf16 merge operands)
    bf16 AdT[4][16][24];        // the same blocks transposed
    // per-token tables of the chunk (padded tokens: g = beta = 0)
    float g2[CH];               // gamma_t * log2(e)
    float bt[CH];               // beta_t
    float bg[CH];               // beta_t e^{gamma_t}
    float eg[CH];               // e^{gamma_t}
    float qeg[CH];              // q_scale e^{gamma_t}
    float dec[CH];              // e^{gamma_last - gamma_t}
};

// WITH_O: per-token outputs are produced (Q is loaded, Q K^T and P formed, O stored); without
// them the kernel is the state-only scan.
template <int DK, int DV, bool WITH_O, bool PREP>
__global__ void __launch_bounds__(DV * 2, 2)
gdn_chunk_bf16_kernel(const SeqOrder order, int ordered, const bf16* __restrict__ q, const bf16* __restrict__ k,
                      const bf16* __restrict__ v, const float* __restrict__ g,
                      const float* __restrict__ beta, const int32_t* __restrict__ cu,
                      int B, int Hqk, int Hv, float q_scale, int uniform_len, long long state_bstride,
                      const float* state_in, int state_identity, float* state_out, bf16* __restrict__ o,
                      unsigned char* __restrict__ ws, long long rec_per_head, int cmax)
{
    constexpr int NW = DV / 32;            // waves; wave w owns dv columns [32w, 32w+32)
    constexpr int NT = NW * 64;
    constexpr int KT_TILES = DK / 32;      // S^T row tiles per wave
    constexpr int KSTEPS_D = DK / 16;      // 32x32x16 k-steps over dk
    constexpr int TPR = DK / 8;            // threads per staged key/query row (16 B each)
    constexpr int RPP = NT / TPR;          // rows per pass
    constexpr int NPASS = CH / RPP;
    constexpr int G_PER_WAVE = (10 + NW - 1) / NW;          // K K^T tiles per wave (P1)
    // Q K^T tiles (P2): wave w takes tiles [qk_begin(w), qk_begin(w + 1)); the waves with the
    // longer inverse merge chains (low w) take fewer.
    // With four waves, wave 0 (the longest inverse merge chain) takes tile 0 and waves 1..3
    // take three tiles each; each count runs as straight-line code, so no branch splits the
    // product chains.  Tiles are numbered row by row: (0,0) (1,0) (1,1) (2,0) ...
    constexpr int QK_PER_WAVE = NW == 4 ? 3 : 6;
    auto qk_begin = [](int w) { return NW == 4 ? (w == 0 ? 0 : 3 * w - 2) : (w == 0 ? 0 : (w == 1 ? 4 : 10)); };

    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<DK, DV>& sm = *reinterpret_cast<Smem<DK, DV>*>(smem_raw);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto qk_tile = [&](int it, int& rb, int& cb) {
        const int tt = qk_begin(wave) + it;
        rb = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
        cb = tt - rb * (rb + 1) / 2;
    };
    auto qk_live = [&](int it) { return NW == 4 || qk_begin(wave) + it < qk_begin(wave + 1); };
    // runs f(std::integral_constant<int, n>) with this wave's tile count n
    auto with_qk_count = [&](auto&& f) {
        if constexpr (NW == 4) {
            if (wave == 0) f(std::integral_constant<int, 1>{});
            else f(std::integral_constant<int, 3>{});
        } else {
            f(std::integral_constant<int, QK_PER_WAVE>{});
        }
    };
    int lane = tid & 63;
    int l32 = lane & 31;
    int h2 = lane >> 5;
    int l16 = lane & 15;
    int g4 = lane >> 4;
    // transpose-read addressing: row offset p and column offset within a 32-wide tile
    int tr_p = (lane & 15) >> 2;
    int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // Workgroup order.  blockIdx % 8 picks the XCD.  Fused: units (sequence, query/key head)
    // are dealt round-robin to the XCDs in rank order (sequences longest first when ordered),
    // and the value heads of a unit follow one another on its XCD, so the second reader of
    // each key/query tile finds it in that XCD's L2.  PREP: items (sequence, chunk, value
    // head) in contiguous ranges per XCD, value head fastest.
    const int G = Hv / Hqk;
    int b, hv, item = 0;
    if (PREP) {
        const int per_xcd = (int)(gridDim.x / 8);
        item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
        if (item >= B * Hv * cmax) return;
        b = item / (Hv * cmax);
        hv = item % Hv;
    } else {
        const int r = (int)(blockIdx.x / 8);
        const int u = (r / G) * 8 + (int)(blockIdx.x % 8);
        if (u >= B * Hqk) return;
        b = (ordered & 1) ? seq_at(u / Hqk) : u / Hqk;
        hv = (u % Hqk) * G + r % G;
    }
    (void)order;
    const int hq = hv / G;
    const int bos = cu ? cu[b] : b * uniform_len;
    const int len = cu ? cu[b + 1] - bos : uniform_len;
    const int n_chunks = (len + CH - 1) / CH;
    const int c_begin = PREP ? (item / Hv) % cmax : 0;
    const int c_end = PREP ? c_begin + 1 : n_chunks;
    if (PREP && c_begin >= n_chunks) return;
    const int col0 = 32 * wave;

    // Buffer views of this (sequence, head): rows past the sequence end read as zero.
    const uint32_t kq_stride = (uint32_t)Hqk * DK * 2;     // bytes between token rows
    const uint32_t v_stride = (uint32_t)Hv * DV * 2;
    const uint32_t gb_stride = (uint32_t)Hv * 4;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + ((size_t)bos * Hqk + hq) * DK, (uint32_t)len * kq_stride);
    // a null q or v reads as zeros (empty resource)
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q ? q + ((size_t)bos * Hqk + hq) * DK : nullptr, q ? (uint32_t)len * kq_stride : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v ? v + ((size_t)bos * Hv + hv) * DV : nullptr, v ? (uint32_t)len * v_stride : 0u);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(g + (size_t)bos * Hv + hv, (uint32_t)len * gb_stride);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(beta + (size_t)bos * Hv + hv, (uint32_t)len * gb_stride);
    // outputs: stores past the sequence end fall outside the resource and are dropped
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(WITH_O ? o + ((size_t)bos * Hv + hv) * DV : nullptr,
                                                WITH_O ? (uint32_t)len * v_stride : 0u);

    // ---- state: S^T tiles, tile r covers dk rows [32r, 32r+32), columns = own dv cols
    f32x16 St[KT_TILES];
    const size_t sbase = (size_t)b * state_bstride + (size_t)hv * DV * DK + (size_t)(col0 + l32) * DK;
#pragma unroll
    for (int r = 0; r < KT_TILES; ++r) {
        if (PREP) break;
        if (state_identity) {
            // S = I: element (dv col0 + l32, dk 32 r + 8 q4 + 4 h2 + i)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    St[r][4 * q4 + i] = (32 * r + 8 * q4 + 4 * h2 + i == col0 + l32) ? 1.f : 0.f;
        } else if (state_in) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(state_in + sbase + 32 * r + 8 * q4 + 4 * h2);
#pragma unroll
                for (int i = 0; i < 4; ++i) St[r][4 * q4 + i] = x[i];
            }
        } else {
            St[r] = zero16();
        }
    }

    // (A - I) tiles above the diagonal inside each 32-row band are read as zeros and never
    // written by the inverse; P4 rewrites them as zeros each chunk (the tiles alias P).
    for (int i = tid; i < CH * RS_T; i += NT) {
        (&sm.np.n.Nb[0][0])[i] = (bf16)0.f;
        (&sm.np.n.Nbg[0][0])[i] = (bf16)0.f;
    }

    // ---- loads (zero past the end of the sequence)
    bf16x8 pk[NPASS], pq[NPASS];
    float pg = 0.f, pb = 0.f;
    int kq_row = tid / TPR;
    int kq_col = (tid % TPR) * 8;
    // K and the gates are prefetched one chunk ahead; Q is loaded at the start of its own
    // chunk and staged at the end of P1 (register budget).
    auto fetch_kq = [&](int c) {
        const uint32_t voff = (uint32_t)kq_row * kq_stride + (uint32_t)kq_col * 2;
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const uint32_t soff = (uint32_t)(c * CH + RPP * p) * kq_stride;
            pk[p] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, voff, soff, 0));
        }
        if (wave == 0) {
            const uint32_t soff = (uint32_t)(c * CH) * gb_stride;
            pg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)lane * gb_stride, soff, 0));
            pb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)lane * gb_stride, soff, 0));
        }
    };
    // The first chunk's K and tables are also staged here (the top of the loop stages them once
    // more): with its loads consumed before the loop, the compiler's wait at the top of the loop
    // is for the prefetch alone, not for the previous chunk's output stores issued after it.
    auto stage = [&]() {
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
            *reinterpret_cast<bf16x8*>(&sm.K[kq_row + RPP * p][kq_col]) = pk[p];
        if (wave == 0) {
            const float g2 = wave_prefix_sum(pg) * LOG2E;
            const float g2_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g2), 63));
            const float e = __builtin_amdgcn_exp2f(g2);
            sm.g2[lane] = g2;
            sm.bt[lane] = pb;
            sm.bg[lane] = pb * e;
            sm.eg[lane] = e;
            sm.qeg[lane] = q_scale * e;
            sm.dec[lane] = __builtin_amdgcn_exp2f(g2_last - g2);
        }
    };
    if (c_begin < c_end) {
        fetch_kq(c_begin);
        stage();
    }

    // With unequal lengths, or when all workgroups fit in one round, the two workgroups that
    // share a CU take turns at issue priority chunk by chunk, by the parity of their wave slot:
    // otherwise the one dispatched first keeps it throughout.  Measured on 64 hits of 205 to
    // 6,554 tokens: 1.43 -> 1.39 ms.  With equal lengths over several rounds it measured 1-2%
    // slower (an early finisher lets the next round start sooner), so it is off there.
    const int slot = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 4) & 1);   // HW_ID wave_id, bit 0
    for (int c = c_begin; c < c_end; ++c) {
        if (!PREP && (ordered & 2)) {
            if ((slot + c) & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        // Recompute the lane-derived indices every chunk: left loop-invariant, the compiler
        // hoists dozens of per-lane LDS addresses out of the loop and spills them.
        asm volatile("" : "+v"(lane));
        l32 = lane & 31; h2 = lane >> 5; l16 = lane & 15; g4 = lane >> 4;
        tr_p = (lane & 15) >> 2; tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        kq_row = (64 * wave + lane) / TPR; kq_col = ((64 * wave + lane) % TPR) * 8;
        const int t0 = bos + c * CH;
        const int nval = min(CH, len - c * CH);

        // -------------------------------------------------------------- P0: stage
        stage();
        // This chunk's Q and V are issued after the tables: the gate values reloaded above
        // must not queue behind them.
        if (WITH_O) {
            const uint32_t voff = (uint32_t)kq_row * kq_stride + (uint32_t)kq_col * 2;
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const uint32_t soff = (uint32_t)(c * CH + RPP * p) * kq_stride;
                pq[p] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, voff, soff, 0));
            }
        }

        // V of this wave's columns in B-operand order (k-step s holds tokens
        // 16s + 4h + {0..3} and 16s + 8 + 4h + {0..3}); consumed in P3.
        bf16x8 vc[4];
        {
            const uint32_t voff = (uint32_t)(4 * h2) * v_stride + (uint32_t)(col0 + l32) * 2;
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t soff = (uint32_t)(c * CH + 16 * s + (i & 3) + ((i >> 2) << 3)) * v_stride;
                    vc[s][i] = __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rv, voff, soff, 0));
                }
        }

        if (c + 1 < c_end) fetch_kq(c + 1);
        lds_barrier();

        // ------------------------------------------------------------- P1: K K^T -> L
        // Diagonal tiles come out with lane (n, q) holding rows 4q..4q+3 of column n; the wave
        // that forms one inverts it at once (below).  Off-diagonal tiles are formed transposed
        // (operands swapped), so lane (m, q) holds row m, columns 4q..4q+3, stored as bf16
        // rows for the merges' A operands.
        //
        // The diagonal blocks D_b = (I + L_bb)^{-1}: L_bb is strictly lower triangular
        // (nilpotent), so
        //     D_b = (I - L)(I + L^2)(I + L^4)(I + L^8),
        // each product from hi / lo bf16 splits (about 2^-16 relative, far below the bf16
        // rounding that every later use of D_b applies).  The raw tile K_b K_b^T is symmetric,
        // so the accumulator that holds it in accumulator layout (lane (n, q): rows 4q..4q+3
        // of column n) also holds it in row layout (lane (m, q): row m, columns 4q..4q+3):
        // both layouts of L_bb come from one product, with the mask and decay applied per
        // layout.
        auto invert_diag = [&](int b, const f32x4& raw) {
            const int base = 16 * b;
            const int ci = base + l16;                    // this lane's column (acc) / row (row layout)
            const int r0 = base + 4 * g4;                 // rows (acc) / columns (row layout) r0..r0+3
            const float gi = sm.g2[ci], bi = sm.bt[ci];
            const f32x4 gt = tab4(sm.g2, r0), bt = tab4(sm.bt, r0);
            f32x4 La, Lr;                                 // L_bb in accumulator and row layout
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                La[j] = (ci < r0 + j) ? bt[j] * __builtin_amdgcn_exp2f(gt[j] - gi) * raw[j] : 0.f;
                Lr[j] = (ci > r0 + j) ? bi * __builtin_amdgcn_exp2f(gi - gt[j]) * raw[j] : 0.f;
            }
            const f32x4 L2a = mm16x3(Lr, La, zero4()), L2r = mm16x3(La, Lr, zero4());
            const f32x4 L4a = mm16x3(L2r, L2a, zero4()), L4r = mm16x3(L2a, L2r, zero4());
            const f32x4 L8r = mm16x3(L4a, L4r, zero4());
            f32x4 D;                                      // I - L, accumulator layout
#pragma unroll
            for (int j = 0; j < 4; ++j) D[j] = (r0 + j == ci ? 1.f : 0.f) - La[j];
            D = mm16x3(L2r, D, D);
            D = mm16x3(L4r, D, D);
            D = mm16x3(L8r, D, D);                        // lane (n, g): D[4g + j][n]
            const float bgn = sm.bg[ci];
            bf16x4 ad;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g4 + j;
                ad[j] = (bf16)D[j];
                const float nn = r > l16 ? D[j] : 0.f;    // strictly lower part: A - I
                sm.np.n.Nb[base + r][base + l16] = (bf16)(nn * bi);
                sm.np.n.Nbg[base + r][base + l16] = (bf16)(nn * bgn);
            }
            *reinterpret_cast<bf16x4*>(&sm.AdT[b][l16][4 * g4]) = ad;
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.Ad[b][4 * g4 + j][l16] = ad[j];
        };
        auto l_off = [&](int rb, int cb, const f32x4& acc) {
            const int t = 16 * rb + l16;                  // row (later token)
            const int c0 = 16 * cb + 4 * g4;              // columns c0..c0+3 (earlier tokens)
            const float gt = sm.g2[t], bt = sm.bt[t];
            const f32x4 gi = tab4(sm.g2, c0);
            bf16x4 lv;
#pragma unroll
            for (int j = 0; j < 4; ++j) lv[j] = (bf16)(bt * __builtin_amdgcn_exp2f(gt - gi[j]) * acc[j]);
            *reinterpret_cast<bf16x4*>(&sm.lw.l.Lb[t][c0]) = lv;
        };
        if constexpr (NW == 4) {
            // Wave w: the diagonal tile (w, w) and two off-diagonal tiles, with no branches so
            // that the three product chains and their LDS reads overlap:
            //   w0: (1,0) (2,0)   w1: (2,1) (3,1)   w2: (3,2) (3,0)   w3: (3,0) (3,2) (repeats;
            // the same values land in the same places).  Tables: 2 bits per block index.
            constexpr uint32_t R1 = 1 | 2 << 2 | 3 << 4 | 3 << 6, C1 = 0 | 1 << 2 | 2 << 4 | 0 << 6;
            constexpr uint32_t R2 = 2 | 3 << 2 | 3 << 4 | 3 << 6, C2 = 0 | 1 << 2 | 0 << 4 | 2 << 6;
            const int r1 = (R1 >> (2 * wave)) & 3, c1 = (C1 >> (2 * wave)) & 3;
            const int r2 = (R2 >> (2 * wave)) & 3, c2 = (C2 >> (2 * wave)) & 3;
            const bf16* pd = &sm.K[(16 * wave + l16) & (CH - 1)][8 * g4];
            const bf16* pa1 = &sm.K[(16 * c1 + l16) & (CH - 1)][8 * g4];
            const bf16* pb1 = &sm.K[(16 * r1 + l16) & (CH - 1)][8 * g4];
            const bf16* pa2 = &sm.K[(16 * c2 + l16) & (CH - 1)][8 * g4];
            const bf16* pb2 = &sm.K[(16 * r2 + l16) & (CH - 1)][8 * g4];
            f32x4 ad = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const bf16x8 xd = *reinterpret_cast<const bf16x8*>(pd + 32 * s);
                const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(pa1 + 32 * s);
                const bf16x8 y1 = *reinterpret_cast<const bf16x8*>(pb1 + 32 * s);
                const bf16x8 x2 = *reinterpret_cast<const bf16x8*>(pa2 + 32 * s);
                const bf16x8 y2 = *reinterpret_cast<const bf16x8*>(pb2 + 32 * s);
                ad = mma16k32(xd, xd, ad);
                a1 = mma16k32(x1, y1, a1);
                a2 = mma16k32(x2, y2, a2);
            }
            invert_diag(wave, ad);
            l_off(r1, c1, a1);
            l_off(r2, c2, a2);
        } else {
#pragma unroll
            for (int it = 0; it < G_PER_WAVE; ++it) {
                const int tt = wave + NW * it;
                if (tt < 10) {
                    const int rb = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
                    const int cb = tt - rb * (rb + 1) / 2;
                    const bool diag = rb == cb;
                    const bf16* xrow = &sm.K[16 * (diag ? rb : cb) + l16][0];
                    const bf16* krow = &sm.K[16 * (diag ? cb : rb) + l16][0];
                    f32x4 acc = zero4();
#pragma unroll
                    for (int s = 0; s < DK / 32; ++s)
                        acc = mma16k32(*reinterpret_cast<const bf16x8*>(xrow + 32 * s + 8 * g4),
                                       *reinterpret_cast<const bf16x8*>(krow + 32 * s + 8 * g4), acc);
                    if (diag) invert_diag(rb, acc);
                    else l_off(rb, cb, acc);
                }
            }
        }
        if (WITH_O) {
#pragma unroll
            for (int p = 0; p < NPASS; ++p)
                *reinterpret_cast<bf16x8*>(&sm.Q[kq_row + RPP * p][kq_col]) = pq[p];
        }
        lds_barrier();

        // ------------------- P2: A = (I + L)^{-1} off the diagonal; Q K^T tiles on every wave
        // Off-diagonal blocks, one block column per wave:
        // A_ij = -A_ii sum_{k=j}^{i-1} L_ik A_kj on 16x16x16 bf16 MFMA.  16x16x16 layouts: the A
        // operand lane (m = l % 16, q = l / 16) holds row m, k = 4q..4q+3; the B operand and the
        // accumulator hold rows 4q..4q+3 of column l % 16, so a result feeds the next product's
        // B operand as it stands.
        f32x4 tacc[QK_PER_WAVE];
        {
            auto opL = [&](int i, int kb) {          // A operand: L block (i, kb)
                return *reinterpret_cast<const bf16x4*>(&sm.lw.l.Lb[16 * i + l16][16 * kb + 4 * g4]);
            };
            auto opAd = [&](int i) {                 // A operand: diagonal block A_ii (row layout)
                return *reinterpret_cast<const bf16x4*>(&sm.Ad[i][l16][4 * g4]);
            };
            auto opBd = [&](int kb) {                // B operand: diagonal block A_kk
                return *reinterpret_cast<const bf16x4*>(&sm.AdT[kb][l16][4 * g4]);
            };
            // Block (i, j) of A - I is -(A_ii T); its transpose -(T^T A_ii^T) comes out of the MFMA
            // in row order (lane (n, q) holds row n, columns 4q..4q+3), so it is written as
            // 8-byte row segments.  T enters as the A operand in its accumulator layout (which
            // reads as T^T), A_ii as the B operand in row layout (which reads as A_ii^T).
            for (int j = wave; j < 3; j += NW) {
                // Every operand of block column j's chain is read before the chain starts (block
                // indices clamped to 3; a clamped operand is never used), so the chain waits
                // only on its own products.
                const int j1 = j + 1, j2 = min(j + 2, 3);
                const bf16x4 dj = opBd(j);
                const bf16x4 l10 = opL(j1, j), l20 = opL(j2, j), l21 = opL(j2, j1);
                const bf16x4 l30 = opL(3, j), l31 = opL(3, j1), l32 = opL(3, j2);
                const bf16x4 d1 = opAd(j1), d2 = opAd(j2), d3 = opAd(3);
                const int c0 = 16 * j + 4 * g4;
                const f32x4 bt = tab4(sm.bt, c0), bg = tab4(sm.bg, c0);
                auto emit = [&](int i, const bf16x4& di, const bf16x4& tneg) {
                    const f32x4 rows = mma16(tneg, di, zero4());
                    bf16x4 nb, ng;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        nb[e] = (bf16)(rows[e] * bt[e]);
                        ng[e] = (bf16)(rows[e] * bg[e]);
                    }
                    *reinterpret_cast<bf16x4*>(&sm.np.n.Nb[16 * i + l16][c0]) = nb;
                    *reinterpret_cast<bf16x4*>(&sm.np.n.Nbg[16 * i + l16][c0]) = ng;
                };
                // A_{j+1,j}, A_{j+2,j} as B operands (a1 unused when j + 1 = 3, a2 unless j = 0)
                const bf16x4 t1 = to_bf4(mma16(l10, dj, zero4()), -1.f);
                const bf16x4 a1 = to_bf4(mma16(d1, t1, zero4()), 1.f);
                emit(j1, d1, t1);
                if (j + 2 <= 3) {
                    const bf16x4 t2 = to_bf4(mma16(l21, a1, mma16(l20, dj, zero4())), -1.f);
                    const bf16x4 a2 = to_bf4(mma16(d2, t2, zero4()), 1.f);
                    emit(j2, d2, t2);
                    if (j == 0) {
                        f32x4 acc = mma16(l30, dj, zero4());
                        acc = mma16(l31, a1, acc);
                        acc = mma16(l32, a2, acc);
                        emit(3, d3, to_bf4(acc, -1.f));
                    }
                }
            }
            if (WITH_O) {
                // Q K^T lower 16x16 tiles, kept in registers until P4.  Operands swapped: lane
                // (t, q) ends with row 16 rb + t of Q K^T, columns 16 cb + 4q .. 16 cb + 4q + 3.
                with_qk_count([&](auto n_c) {
                    constexpr int N = decltype(n_c)::value;
                    const bf16* qrow[N];
                    const bf16* krow[N];
#pragma unroll
                    for (int it = 0; it < N; ++it) {
                        int rb, cb;
                        qk_tile(it, rb, cb);
                        qrow[it] = &sm.Q[(16 * rb + l16) & (CH - 1)][8 * g4];
                        krow[it] = &sm.K[(16 * cb + l16) & (CH - 1)][8 * g4];
                        tacc[it] = zero4();
                    }
#pragma unroll
                    for (int s = 0; s < DK / 32; ++s)
#pragma unroll
                        for (int it = 0; it < N; ++it)
                            if (qk_live(it))
                                tacc[it] = mma16k32(*reinterpret_cast<const bf16x8*>(krow[it] + 32 * s),
                                                    *reinterpret_cast<const bf16x8*>(qrow[it] + 32 * s), tacc[it]);
                });
            }
        }
        lds_barrier();

        // --------------------------------------------------------- P3: U0 and -W
        f32x16 U[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x16 acc = zero16();
#pragma unroll
            for (int s = 0; s < 2 * rt + 2; ++s)             // A = (I + L)^{-1} is lower triangular
                acc = mma32(kperm(&sm.np.n.Nb[32 * rt + l32][0], s, h2), vc[s], acc);
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const f32x4 bt = tab4(sm.bt, 32 * rt + 8 * j4 + 4 * h2);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * j4 + e;
                    acc[j] += bt[e] * (float)vc[2 * rt + (j >> 3)][j & 7];
                }
            }
            U[rt] = acc;
        }
        for (int ct = wave; ct < DK / 32; ct += NW) {
            bf16x8 kb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kb[s] = cat(lds_tr4(&sm.K[16 * s + 4 * h2 + tr_p][32 * ct + tr_c]),
                            lds_tr4(&sm.K[16 * s + 8 + 4 * h2 + tr_p][32 * ct + tr_c]));
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                // the K row segments of the unit-diagonal term, read before the products
                bf16x4 kt[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    kt[q] = *reinterpret_cast<const bf16x4*>(&sm.K[32 * rt + l32][32 * ct + 8 * q + 4 * h2]);
                // W^T tile (operands swapped): lane (t = l32, h) holds token 32 rt + t, dk columns
                // 32 ct + 8 q + 4 h + {0..3} -- 8-byte row segments of -W
                f32x16 acc = zero16();
#pragma unroll
                for (int s = 0; s < 2 * rt + 2; ++s)
                    acc = mma32(kb[s], kperm(&sm.np.n.Nbg[32 * rt + l32][0], s, h2), acc);
                const int t = 32 * rt + l32;
                const float bgt = sm.bg[t];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 32 * ct + 8 * q + 4 * h2;
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (bf16)(-(acc[4 * q + e] + bgt * (float)kt[q][e]));
                    *reinterpret_cast<bf16x4*>(&sm.lw.Wn[t][c]) = w;
                }
            }
        }
        lds_barrier();

        unsigned char* rec = nullptr;
        if constexpr (PREP) {
            // the chunk's record: operand fragments, 64 lanes x 16 bytes each
            rec = ws + ((size_t)hv * rec_per_head + (size_t)(bos / CH + b + c)) * split_record_bytes(DK, DV);
            for (int f = wave; f < 2 * KSTEPS_D; f += NW) {          // -W and Q, (row tile, k-step)
                const int rt = f / KSTEPS_D, s = f % KSTEPS_D;
                *reinterpret_cast<bf16x8*>(rec + split_wn_off() + (size_t)(f * 64 + lane) * 16) =
                    kperm(&sm.lw.Wn[32 * rt + l32][0], s, h2);
                if (WITH_O)
                    *reinterpret_cast<bf16x8*>(rec + split_q_off(DK) + (size_t)(f * 64 + lane) * 16) =
                        kperm(&sm.Q[32 * rt + l32][0], s, h2);
            }
            for (int f = wave; f < 4 * KT_TILES; f += NW) {          // K^T, (token k-step, dk tile)
                const int s = f / KT_TILES, r = f % KT_TILES;
                *reinterpret_cast<bf16x8*>(rec + split_kt_off(DK) + (size_t)(f * 64 + lane) * 16) =
                    cat(lds_tr4(&sm.K[16 * s + 4 * h2 + tr_p][32 * r + tr_c]),
                        lds_tr4(&sm.K[16 * s + 8 + 4 * h2 + tr_p][32 * r + tr_c]));
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)                           // U0 of this wave's columns
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = U[rt][4 * q4 + i];
                    *reinterpret_cast<f32x4*>(rec + split_u0_off(DK) + (size_t)((wave * 2 + rt) * 64 + lane) * 64 + q4 * 16) = x;
                }
            if (tid < CH) {
                const int row = tid / 16, i4 = 4 * (tid % 16);
                const float* t = row == 0 ? sm.bt : (row == 1 ? sm.qeg : (row == 2 ? sm.dec : sm.eg));
                *reinterpret_cast<f32x4*>(rec + split_tab_off(DK, DV) + (row * CH + i4) * 4) = tab4(t, i4);
            }
        }

        // ------------------------------------------------------------ P4: P to LDS
        if (WITH_O) {
            with_qk_count([&](auto n_c) {
                constexpr int N = decltype(n_c)::value;
#pragma unroll
                for (int it = 0; it < N; ++it) {
                    if (qk_live(it)) {
                        int rb, cb;
                        qk_tile(it, rb, cb);
                        const int t = 16 * rb + l16;
                        const int c0 = 16 * cb + 4 * g4;
                        const float gt = sm.g2[t];
                        const f32x4 gi = tab4(sm.g2, c0);
                        f32x4 p;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            p[j] = (c0 + j <= t) ? q_scale * __builtin_amdgcn_exp2f(gt - gi[j]) * tacc[it][j] : 0.f;
                        bf16x4 ph, pl;
                        split_bf4(p, ph, pl);
                        *reinterpret_cast<bf16x4*>(&sm.np.p.Ph[t][c0]) = ph;
                        *reinterpret_cast<bf16x4*>(&sm.np.p.Pl[t][c0]) = pl;
                    }
                }
            });
            // the zero blocks above the diagonal inside each 32-row band (also zero for A - I):
            // (band, hi / lo) = (w & 1, w >> 1) for wave w when there are four waves
#pragma unroll
            for (int z = 0; z < 4 / NW; ++z) {
                const int zb = NW == 4 ? wave : 2 * wave + z;
                const int band = zb & 1;
                bf16* zp = (zb >> 1) ? &sm.np.p.Pl[32 * band + l16][32 * band + 16 + 4 * g4]
                                     : &sm.np.p.Ph[32 * band + l16][32 * band + 16 + 4 * g4];
                *reinterpret_cast<bf16x4*>(zp) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            }
        }
        lds_barrier();

        if constexpr (PREP) {
            if (WITH_O) {
                for (int f = wave; f < 12; f += NW) {       // P hi then lo, (rt, s) with s < 2 rt + 2
                    const int hl = f / 6, ff = f % 6;
                    const int rt = ff < 2 ? 0 : 1, s = ff < 2 ? ff : ff - 2;
                    const bf16* row = hl ? &sm.np.p.Pl[32 * rt + l32][0] : &sm.np.p.Ph[32 * rt + l32][0];
                    *reinterpret_cast<bf16x8*>(rec + (hl ? split_pl_off(DK) : split_ph_off(DK)) + (size_t)(ff * 64 + lane) * 16) =
                        kperm(row, s, h2);
                }
            }
            continue;
        }

        // ------------------------------------------------ P5: state-dependent part
        // U' = U0 + (-W) S^T and, with outputs, Y = Q S^T: one conversion of each state operand
        // feeds up to four independent accumulators.
        f32x16 Y[2];
        if (WITH_O) {
            Y[0] = zero16();
            Y[1] = zero16();
        }
#pragma unroll
        for (int s = 0; s < KSTEPS_D; ++s) {
            const bf16x8 sb = acc_to_b(St[s >> 1], s);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                U[rt] = mma32(kperm(&sm.lw.Wn[32 * rt + l32][0], s, h2), sb, U[rt]);
                if (WITH_O) Y[rt] = mma32(kperm(&sm.Q[32 * rt + l32][0], s, h2), sb, Y[rt]);
            }
        }
        // Outputs first: O = diag(q_scale e^gamma) Y + P U' (P and U' split hi / lo), stored before
        // the state update so that its accumulators are free during the update.
        if (WITH_O) {
            bf16x8 uh[4], ul[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) acc_to_b_split(U[s >> 1], s, uh[s], ul[s]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const f32x4 e = tab4(sm.qeg, 32 * rt + 8 * j4 + 4 * h2);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Y[rt][4 * j4 + i] *= e[i];
                }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    if (s < 2 * rt + 2) {                  // P is lower triangular
                        const bf16x8 ph = kperm(&sm.np.p.Ph[32 * rt + l32][0], s, h2);
                        const bf16x8 pl = kperm(&sm.np.p.Pl[32 * rt + l32][0], s, h2);
                        Y[rt] = mma32(ph, uh[s], Y[rt]);
                        Y[rt] = mma32(ph, ul[s], Y[rt]);
                        Y[rt] = mma32(pl, uh[s], Y[rt]);
                    }
                }
            // O as 32-bit words: for each token pair (t, t + 1) a lane holds, lanes 2m and 2m + 1
            // swap halves and store columns (2m, 2m + 1) of tokens t and t + 1 respectively
            // (half the store instructions of 16-bit stores, the same cache lines).
            const uint32_t ooff = (uint32_t)(4 * h2 + (l32 & 1)) * v_stride + (uint32_t)(col0 + (l32 & ~1)) * 2;
            const uint32_t sel = (l32 & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const uint32_t own = __builtin_bit_cast(uint32_t, bf16x2{(bf16)Y[rt][j], (bf16)Y[rt][j + 1]});
                    const uint32_t partner = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
                    const uint32_t wv = __builtin_amdgcn_perm(partner, own, sel);
                    const uint32_t soff = (uint32_t)(c * CH + 32 * rt + 8 * (j >> 2) + (j & 3)) * v_stride;
                    __builtin_amdgcn_raw_buffer_store_b32(wv, ro, ooff, soff, 0);
                }
        }
        // S <- e^{gamma_n} S + U'^T diag(e^{gamma_n - gamma}) K (U' split hi / lo)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const f32x4 d = tab4(sm.dec, 32 * rt + 8 * j4 + 4 * h2);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[rt][4 * j4 + i] *= d[i];
            }
        const float decay = sm.eg[CH - 1];
#pragma unroll
        for (int r = 0; r < KT_TILES; ++r)
#pragma unroll
            for (int j = 0; j < 16; ++j) St[r][j] *= decay;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 dh, dl;
            acc_to_b_split(U[s >> 1], s, dh, dl);
#pragma unroll
            for (int r = 0; r < KT_TILES; ++r) {
                const bf16x8 a = cat(lds_tr4(&sm.K[16 * s + 4 * h2 + tr_p][32 * r + tr_c]),
                                     lds_tr4(&sm.K[16 * s + 8 + 4 * h2 + tr_p][32 * r + tr_c]));
                St[r] = mma32(a, dh, St[r]);
                St[r] = mma32(a, dl, St[r]);
            }
        }
        lds_barrier();
    }

    // ---- write the final state
    if (PREP) return;
#pragma unroll
    for (int r = 0; r < KT_TILES; ++r) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = St[r][4 * q4 + i];
            *reinterpret_cast<f32x4*>(state_out + sbase + 32 * r + 8 * q4 + 4 * h2) = x;
        }
    }
}

template <int DK, int DV, bool WITH_O, bool PREP>
hipError_t launch_variant(const GdnArgs& a, const SplitPlan* plan, const SeqOrder* order, hipStream_t stream) {
    constexpr auto kern = gdn_chunk_bf16_kernel<DK, DV, WITH_O, PREP>;
    const size_t smem = sizeof(Smem<DK, DV>);
    const hipError_t e = ensure_dynamic_smem<kern>(smem);
    if (e != hipSuccess) return e;
    // a multiple of 8 blocks (one share per XCD); fused: ceil(units / 8) rounds of 8 units
    const long long units = (long long)a.B * a.Hqk;
    const long long blocks = PREP ? ((long long)a.B * a.Hv * plan->cmax + 7) / 8 * 8
                                  : (units + 7) / 8 * 8 * (a.Hv / a.Hqk);
    const dim3 grid((unsigned)blocks);
    const dim3 block(DV * 2);
    SeqOrder ord{};
    if (order) ord = *order;
    // flags: bit 0, sequences in the given order; bit 1, the two workgroups of a CU take
    // turns at issue priority (unequal lengths, or one partial round of workgroups)
    const int cus = device_cu_count();
    const bool one_round = cus > 0 && blocks <= 2LL * cus;
    const int flags = (order ? 1 : 0) | ((order || one_round) ? 2 : 0);
    hipLaunchKernelGGL(kern, grid, block, smem, stream, ord, flags,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta, a.cu_seqlens,
                       a.B, a.Hqk, a.Hv, a.q_scale, a.uniform_len, (long long)a.state_bstride,
                       a.state_in, a.state_identity, a.state_out, (bf16*)a.o,
                       PREP ? (unsigned char*)plan->ws : nullptr, PREP ? (long long)plan->rec_per_head : 0LL,
                       PREP ? plan->cmax : 0);
    return hipGetLastError();
}

template <int DK, int DV, bool PREP>
hipError_t launch(const GdnArgs& a, const SplitPlan* plan, const SeqOrder* order, hipStream_t stream) {
    return a.o ? launch_variant<DK, DV, true, PREP>(a, plan, order, stream)
               : launch_variant<DK, DV, false, PREP>(a, plan, order, stream);
}

template <bool PREP>
hipError_t launch_dims(const GdnArgs& a, const SplitPlan* plan, const SeqOrder* order, hipStream_t stream) {
    if (a.dk == 128 && a.dv == 128) return launch<128, 128, PREP>(a, plan, order, stream);
    if (a.dk == 64 && a.dv == 64) return launch<64, 64, PREP>(a, plan, order, stream);
    if (a.dk == 128 && a.dv == 64) return launch<128, 64, PREP>(a, plan, order, stream);
    if (a.dk == 64 && a.dv == 128) return launch<64, 128, PREP>(a, plan, order, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gdn_chunk_bf16(const GdnArgs& a, hipStream_t stream, const SeqOrder* order) {
    return launch_dims<false>(a, nullptr, order, stream);
}

hipError_t launch_gdn_prep_bf16(const GdnArgs& a, const SplitPlan& plan, hipStream_t stream) {
    return launch_dims<true>(a, &plan, nullptr, stream);
}

}  // namespace tr
