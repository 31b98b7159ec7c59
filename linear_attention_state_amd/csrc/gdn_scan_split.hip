// State scan of the split schedule: the inter-chunk part of the chunked Gated DeltaNet
// replay with each state split along dv across workgroups, for requests with few heads.
//
// Rows of the state S (dv x dk) evolve independently given the chunk's key-side operators
// (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.3, Eq. (1): the
// operator T_t acts from the right, so row i of S_t depends only on row i of S_{t-1} and
// entry i of v_t).  The prep kernel (gdn_chunk_bf16.hip, PREP mode) has already written,
// for every chunk, -W = -A diag(beta e^gamma) K, K^T, P = e^{gamma_t - gamma_i} q_scale
// q_t.k_i (hi / lo), U0 = A diag(beta) V and the gate tables, as MFMA operand fragments.
// Here a workgroup of two waves owns 32 value columns of one (sequence, value head), and the
// pair splits each chunk's products between them.  Wave h forms U' = U0 + (-W) S^T and
// Y = Q S^T for token rows [32 h, 32 h + 32) over all of dk, splits its rows' U' and
// U' diag(dec) into the bf16 hi / lo operands of the next products and swaps them with its
// partner through LDS; wave h stores the outputs of its rows,
//     O  = diag(q_scale e^gamma) Y + P U'      (stored as 32-bit words of two value columns),
// and updates its half of the state tiles (dk rows [dk h / 2, dk (h + 1) / 2)),
//     S <- e^{gamma_n} S + U'^T diag(e^{gamma_n - gamma}) K,
// then hands the bf16 operands of those rows to its partner for the next chunk's pass.  Every
// accumulator sums its terms in the fused kernel's order, with the same operand splits (U' hi /
// lo in the state update, P and U' hi / lo in P U'), so both schedules give the same bits.
//
// Data movement: each chunk's fragments go straight from memory to LDS (buffer_load ...
// lds), two stages deep, so chunk c + 1 lands while chunk c computes.  Each wave issues an
// equal share of the stage's 1 KiB pieces and waits for its own; a barrier then publishes
// the stage, and the first pass's fragments of the next chunk are read into registers
// before the loop turns.  Every LDS read is one lane's 16 bytes of a fragment (conflict-free, and a
// plain read: the compiler can then tell that the next stage's loads do not touch the
// stage being read, and adds no wait for them).
#include "gdn_mfma.h"

#include <type_traits>

namespace tr {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int CH = 64;

__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}
__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = lo[i]; r[4 + i] = hi[i]; }
    return r;
}
// 32x32x16 accumulator -> B operand: k-step s takes registers 8 (s % 2) .. + 7 of row tile
// s / 2 (rows 16 s + {4h .. 4h+3} and 16 s + 8 + {4h .. 4h+3}).
__device__ __forceinline__ bf16x8 acc_to_b(const f32x16& t, int s) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)t[8 * (s & 1) + i];
    return r;
}
__device__ __forceinline__ void acc_to_b_split(const f32x16& t, int s, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        bf16x2 h, l;
        gdn::split2(t[8 * (s & 1) + i], t[8 * (s & 1) + i + 1], h, l);
        hi[i] = h[0]; hi[i + 1] = h[1];
        lo[i] = l[0]; lo[i + 1] = l[1];
    }
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Fragment f of a fragment array: this lane's 16 bytes.
template <int N>
__device__ __forceinline__ bf16x8 frag(const bf16 (&a)[N], int f, int lane) {
    return *reinterpret_cast<const bf16x8*>(&a[(f * 64 + lane) * 8]);
}

template <int DK>
struct Stage {
    bf16 Wn[2 * (DK / 16) * 512]; // -W fragments
    bf16 Q[2 * (DK / 16) * 512];  // Q fragments
    bf16 KT[4 * (DK / 32) * 512]; // K^T fragments
    bf16 Ph[6 * 512];             // P hi fragments
    bf16 Pl[6 * 512];             // P lo fragments
    float U0[2 * 64 * 16];        // U0 accumulators of this workgroup's 32 columns (row tiles 0, 1)
    float tab[4][CH];             // beta, q_scale e^gamma, e^{gamma_last - gamma}, e^gamma
};
// What the two waves of a pair hand each other: the bf16 hi / lo operands of their U' rows --
// of U' diag(dec) for the state update (both waves) and of U' for P U' (wave 0 to wave 1) --
// and the bf16 state operands of a half of the dk rows.
template <int DK>
struct Swap {
    bf16 D[2][4 * 64 * 8];        // [wave][(k-step 0/1 of its rows) x (hi, lo)] fragments
    bf16 Uo[4 * 64 * 8];          // wave 0's U' hi / lo for k-steps 0, 1
    bf16 Sb[2][(DK / 32) * 64 * 8];
};

constexpr int kScanWaves = 2;   // waves per scan workgroup: one pair on 32 value columns

// The stage's 1 KiB pieces in issue order: -W, Q [WITH_O], K^T, P hi, P lo [WITH_O], U0,
// tables, each a contiguous KiB of the record.
template <int DK, bool WITH_O>
struct Pieces {
    static constexpr int WN = 2 * (DK / 16);
    static constexpr int Q = WITH_O ? 2 * (DK / 16) : 0;
    static constexpr int KT = 4 * (DK / 32);
    static constexpr int P = WITH_O ? 12 : 0;
    static constexpr int U0 = 8;
    static constexpr int TOTAL = WN + Q + KT + P + U0 + 1;
};

// Wave W's pieces (every kScanWaves-th, from W) of one chunk's stage; the list is fixed at
// compile time.
template <int DK, int DV, bool WITH_O, int W>
__device__ __forceinline__ void issue_pieces(Stage<DK>& S, __amdgpu_buffer_rsrc_t rr, uint32_t rec_soff,
                                             uint32_t u0_base, uint32_t lane16) {
    using PC = Pieces<DK, WITH_O>;
#pragma unroll
    for (int p = W; p < PC::TOTAL; p += kScanWaves) {
        int i = p;
        bf16* dst;
        uint32_t off;
        if (i < PC::WN) { dst = &S.Wn[i * 512]; off = (uint32_t)split_wn_off() + i * 1024; }
        else if ((i -= PC::WN) < PC::Q) { dst = &S.Q[i * 512]; off = (uint32_t)split_q_off(DK) + i * 1024; }
        else if ((i -= PC::Q) < PC::KT) { dst = &S.KT[i * 512]; off = (uint32_t)split_kt_off(DK) + i * 1024; }
        else if ((i -= PC::KT) < PC::P) {
            dst = i < 6 ? &S.Ph[i * 512] : &S.Pl[(i - 6) * 512];
            off = (uint32_t)(i < 6 ? split_ph_off(DK) + i * 1024 : split_pl_off(DK) + (i - 6) * 1024);
        } else if ((i -= PC::P) < PC::U0) {
            dst = reinterpret_cast<bf16*>(&S.U0[i * 256]); off = (uint32_t)split_u0_off(DK) + u0_base + i * 1024;
        } else {
            dst = reinterpret_cast<bf16*>(&S.tab[0][0]); off = (uint32_t)split_tab_off(DK, DV);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr)dst, 16, lane16, rec_soff + off, 0, 0);
    }
}

template <int DK, int DV, bool WITH_O>
__global__ void __launch_bounds__(64 * kScanWaves, 1)
gdn_scan_split_kernel(const int32_t* __restrict__ cu, int B, int Hv,
                      int uniform_len, long long state_bstride, const float* state_in, float* state_out,
                      bf16* __restrict__ o, const unsigned char* __restrict__ ws, long long rec_per_head)
{
    using PC = Pieces<DK, WITH_O>;
    constexpr int NG = DV / 32;                 // workgroups (32 columns each) per (sequence, head)
    constexpr int KT_TILES = DK / 32;
    constexpr int KSTEPS_D = DK / 16;
    constexpr int HT = KT_TILES / 2;            // state tiles per wave
    constexpr int HS = KSTEPS_D / 2;            // state k-steps per wave
    constexpr uint32_t REC = (uint32_t)split_record_bytes(DK, DV);
    // each wave's memory operations between its wait for a stage and the wait before it:
    // its pieces of the next stage and its output stores
    constexpr int OWN_PIECES = (PC::TOTAL + kScanWaves - 1) / kScanWaves;
    constexpr int O_STORES = WITH_O ? 8 : 0;
    static_assert(OWN_PIECES + O_STORES <= 63, "more memory operations in flight than vmcnt counts");

    extern __shared__ __align__(16) unsigned char smem_raw[];
    Stage<DK>* st = reinterpret_cast<Stage<DK>*>(smem_raw);
    Swap<DK>& sw = *reinterpret_cast<Swap<DK>*>(smem_raw + 2 * sizeof(Stage<DK>));

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // The pair's two waves run the same steps on different rows; with the wave index a
    // compile-time constant every register array below is indexed statically.
    auto run = [&](auto hc) {
        constexpr int h = decltype(hc)::value;     // this wave's row tile and dk half
        int lane = threadIdx.x & 63;
        // consecutive items (the column groups of one head, then the heads sharing a key head)
        // stay on one XCD (blockIdx % 8 picks it) so they meet the same data in its L2
        const int per_xcd = (int)(gridDim.x / 8);
        const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
        if (item >= B * Hv * NG) return;
        const int grp = item % NG;
        const int hv = (item / NG) % Hv;
        const int b = item / (NG * Hv);
        const int bos = cu ? cu[b] : b * uniform_len;
        const int len = cu ? cu[b + 1] - bos : uniform_len;
        const int n_chunks = (len + CH - 1) / CH;
        const int col0 = 32 * grp;                  // the pair's first value column

        const uint32_t v_stride = (uint32_t)Hv * DV * 2;
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(ws + ((size_t)hv * rec_per_head + (size_t)(bos / CH + b)) * REC,
                                                    (uint32_t)n_chunks * REC);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(WITH_O ? o + ((size_t)bos * Hv + hv) * DV : nullptr,
                                                    WITH_O ? (uint32_t)len * v_stride : 0u);
        const uint32_t u0_base = (uint32_t)grp * 8192;   // this workgroup's U0 fragments

        // Issue this wave's pieces of chunk c into stage sidx (the other wave issues the rest).
        auto issue_stage = [&](int c, int sidx) {
            const uint32_t rec_soff = (uint32_t)c * REC;
            Stage<DK>& S = st[sidx];
            const uint32_t lane16 = (uint32_t)(threadIdx.x & 63) * 16;
            issue_pieces<DK, DV, WITH_O, h>(S, rr, rec_soff, u0_base, lane16);
        };

        int l32 = lane & 31, h2 = lane >> 5;
        // ---- state: this wave's S^T tiles (dk rows [32 (h HT + i), +32) x the pair's 32 columns)
        f32x16 St[HT];
        const size_t sbase = (size_t)b * state_bstride + (size_t)hv * DV * DK + (size_t)(col0 + l32) * DK;
#pragma unroll
        for (int i = 0; i < HT; ++i) {
            const int r = h * HT + i;
            if (state_in) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(state_in + sbase + 32 * r + 8 * q4 + 4 * h2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) St[i][4 * q4 + e] = x[e];
                }
            } else {
                St[i] = zero16();
            }
        }

        // bf16 state operands of every k-step: this wave's from its own tiles, the partner's from LDS
        bf16x8 sb[KSTEPS_D];
        auto own_sb = [&]() {
#pragma unroll
            for (int i = 0; i < HS; ++i) {
                const int s = h * HS + i;
                sb[s] = acc_to_b(St[(s >> 1) - h * HT], s);
                *reinterpret_cast<bf16x8*>(&sw.Sb[h][(i * 64 + lane) * 8]) = sb[s];
            }
        };
        auto partner_sb = [&]() {
#pragma unroll
            for (int i = 0; i < HS; ++i) sb[(1 - h) * HS + i] = frag(sw.Sb[1 - h], i, lane);
        };

        // The U'/Y pass's fragments (-W, Q of this wave's row tile) of chunk c are read at the end of
        // iteration c - 1, after the stage has landed: the reads cannot drift down to their uses
        // across the loop edge, so the pass's products find their operands in registers.
        bf16x8 fw[KSTEPS_D], fq[KSTEPS_D];
        auto read_pass = [&](const Stage<DK>& S) {
#pragma unroll
            for (int s = 0; s < KSTEPS_D; ++s) {
                fw[s] = frag(S.Wn, h * KSTEPS_D + s, lane);
                if (WITH_O) fq[s] = frag(S.Q, h * KSTEPS_D + s, lane);
            }
        };
        if (n_chunks > 0) {
            issue_stage(0, 0);
            own_sb();
            asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            if (1 < n_chunks) issue_stage(1, 1);
            read_pass(st[0]);
            partner_sb();
        }
        for (int c = 0; c < n_chunks; ++c) {
            asm volatile("" : "+v"(lane));
            l32 = lane & 31; h2 = (lane >> 5) & 1;
            const Stage<DK>& S = st[c & 1];

            // U' = U0 + (-W) S^T and Y = Q S^T for row tile h, k-steps in order
            f32x16 U[2], Y;     // U[h] only: the partner's rows arrive as split operands
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&S.U0[(h * 64 + lane) * 16 + 4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) U[h][4 * q4 + e] = x[e];
            }
            if (WITH_O) Y = zero16();
#pragma unroll
            for (int s = 0; s < KSTEPS_D; ++s) {
                U[h] = mma32(fw[s], sb[s], U[h]);
                if (WITH_O) Y = mma32(fq[s], sb[s], Y);
            }
            // this wave's rows: U' hi / lo for P U' (k-steps 2h, 2h + 1) and U' diag(dec) hi / lo
            // for the state update, handed to the partner (each split once, by the wave that
            // holds the rows)
            bf16x8 uh[4], ul[4], dh[4], dl[4];
            if (WITH_O) {
#pragma unroll
                for (int s = 2 * h; s < 2 * h + 2; ++s) acc_to_b_split(U[h], s, uh[s], ul[s]);
            }
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const f32x4 d = *reinterpret_cast<const f32x4*>(&S.tab[2][32 * h + 8 * j4 + 4 * h2]);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[h][4 * j4 + i] *= d[i];
            }
#pragma unroll
            for (int s = 2 * h; s < 2 * h + 2; ++s) {
                acc_to_b_split(U[h], s, dh[s], dl[s]);
                *reinterpret_cast<bf16x8*>(&sw.D[h][((2 * (s - 2 * h)) * 64 + lane) * 8]) = dh[s];
                *reinterpret_cast<bf16x8*>(&sw.D[h][((2 * (s - 2 * h) + 1) * 64 + lane) * 8]) = dl[s];
                if (WITH_O && h == 0) {
                    *reinterpret_cast<bf16x8*>(&sw.Uo[((2 * s) * 64 + lane) * 8]) = uh[s];
                    *reinterpret_cast<bf16x8*>(&sw.Uo[((2 * s + 1) * 64 + lane) * 8]) = ul[s];
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int s = 2 * (1 - h); s < 2 * (1 - h) + 2; ++s) {
                dh[s] = frag(sw.D[1 - h], 2 * (s - 2 * (1 - h)), lane);
                dl[s] = frag(sw.D[1 - h], 2 * (s - 2 * (1 - h)) + 1, lane);
            }
            if (WITH_O && h == 1) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    uh[s] = frag(sw.Uo, 2 * s, lane);
                    ul[s] = frag(sw.Uo, 2 * s + 1, lane);
                }
            }
            if (WITH_O) {
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const f32x4 e = *reinterpret_cast<const f32x4*>(&S.tab[1][32 * h + 8 * j4 + 4 * h2]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Y[4 * j4 + i] *= e[i];
                }
            }
            // S <- e^{gamma_n} S + U'^T diag(e^{gamma_n - gamma}) K (this wave's tiles) and O = Y + P U'
            const float decay = S.tab[3][CH - 1];
#pragma unroll
            for (int i = 0; i < HT; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) St[i][j] *= decay;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int i = 0; i < HT; ++i) {
                    const bf16x8 a = frag(S.KT, s * KT_TILES + h * HT + i, lane);
                    St[i] = mma32(a, dh[s], St[i]);
                    St[i] = mma32(a, dl[s], St[i]);
                }
                if (WITH_O && s < 2 * h + 2) {                 // P is lower triangular
                    const int f = h == 0 ? s : 2 + s;
                    const bf16x8 ph = frag(S.Ph, f, lane);
                    const bf16x8 pl = frag(S.Pl, f, lane);
                    Y = mma32(ph, uh[s], Y);
                    Y = mma32(ph, ul[s], Y);
                    Y = mma32(pl, uh[s], Y);
                }
            }
            if (WITH_O) {
                // O as 32-bit words: lane (l, half) holds column col0 + l of tokens 8 q + 4 half + {0..3}
                // of row tile h; for each token pair (t, t + 1), lanes 2m and 2m + 1 swap halves and
                // store columns (2m, 2m + 1) of tokens t and t + 1 respectively, so each store
                // instruction covers whole 64-byte row runs.
                const uint32_t ooff = (uint32_t)(4 * h2 + (l32 & 1)) * v_stride + (uint32_t)(col0 + (l32 & ~1)) * 2;
                const uint32_t sel = (l32 & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const uint32_t own = __builtin_bit_cast(uint32_t, bf16x2{(bf16)Y[j], (bf16)Y[j + 1]});
                    const uint32_t partner = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
                    const uint32_t wv = __builtin_amdgcn_perm(partner, own, sel);
                    const uint32_t soff = (uint32_t)(c * CH + 32 * h + 8 * (j >> 2) + (j & 3)) * v_stride;
                    __builtin_amdgcn_raw_buffer_store_b32(wv, ro, ooff, soff, 0);
                }
            }
            if (c + 1 < n_chunks) {
                // Hand this wave's state operands to the partner, wait for this wave's share of
                // chunk c + 1 (only this chunk's output stores were issued after it), then for
                // everyone's; the barrier also ends every wave's reads of this chunk's stage (which
                // the issue of chunk c + 2 overwrites) and of the partner's swapped rows.
                own_sb();
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)" :: "i"(O_STORES) : "memory");
                __builtin_amdgcn_s_barrier();
                if (c + 2 < n_chunks) issue_stage(c + 2, c & 1);
                read_pass(st[(c + 1) & 1]);
                partner_sb();
            }
        }

        // ---- write this wave's part of the final state
#pragma unroll
        for (int i = 0; i < HT; ++i) {
            const int r = h * HT + i;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = St[i][4 * q4 + e];
                *reinterpret_cast<f32x4*>(state_out + sbase + 32 * r + 8 * q4 + 4 * h2) = x;
            }
        }
    };
    if (wave == 0) run(std::integral_constant<int, 0>());
    else run(std::integral_constant<int, 1>());
}

template <int DK, int DV, bool WITH_O>
hipError_t launch_scan(const GdnArgs& a, const SplitPlan& plan, hipStream_t stream) {
    constexpr auto kern = gdn_scan_split_kernel<DK, DV, WITH_O>;
    const size_t smem = 2 * sizeof(Stage<DK>) + sizeof(Swap<DK>);
    const hipError_t e = ensure_dynamic_smem<kern>(smem);
    if (e != hipSuccess) return e;
    const long long items = (long long)a.B * a.Hv * (DV / 32);
    const dim3 grid((unsigned)((items + 7) / 8 * 8));
    hipLaunchKernelGGL(kern, grid, dim3(64 * kScanWaves), smem, stream,
                       a.cu_seqlens, a.B, a.Hv,
                       a.uniform_len, (long long)a.state_bstride, a.state_in, a.state_out, (bf16*)a.o,
                       (const unsigned char*)plan.ws, (long long)plan.rec_per_head);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dv(const GdnArgs& a, const SplitPlan& plan, hipStream_t stream) {
    return a.o ? launch_scan<DK, DV, true>(a, plan, stream) : launch_scan<DK, DV, false>(a, plan, stream);
}

}  // namespace

hipError_t launch_gdn_scan_split_bf16(const GdnArgs& a, const SplitPlan& plan, hipStream_t stream) {
    if (a.dk == 128 && a.dv == 128) return launch_dv<128, 128>(a, plan, stream);
    if (a.dk == 64 && a.dv == 64) return launch_dv<64, 64>(a, plan, stream);
    if (a.dk == 128 && a.dv == 64) return launch_dv<128, 64>(a, plan, stream);
    if (a.dk == 64 && a.dv == 128) return launch_dv<64, 128>(a, plan, stream);
    return hipErrorInvalidValue;
}

}  // namespace tr
