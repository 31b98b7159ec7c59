// State scan of the split schedule: the inter-chunk part of the chunked Gated DeltaNet
// replay with each state split along dv across workgroups, for requests with few heads.
//
// Rows of the state S (dv x dk) evolve independently given the chunk's key-side operators
// (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.3, Eq. (1): the
// operator T_t acts from the right, so row i of S_t depends only on row i of S_{t-1} and
// entry i of v_t).  The prep kernel (gdn_chunk_bf16.hip, PREP mode) has already written,
// for every chunk, -W = -A diag(beta e^gamma) K, K^T, P = e^{gamma_t - gamma_i} q_scale
// q_t.k_i (hi / lo), U0 = A diag(beta) V and the gate tables, as MFMA operand fragments.
// Here a workgroup of NWB waves owns NWB x 32 value columns of one (sequence, value head);
// wave w keeps S^T for its 32 columns in MFMA accumulators and per chunk computes
//     U' = U0 + (-W) S^T,   Y = Q S^T
//     S <- e^{gamma_n} S + U'^T diag(e^{gamma_n - gamma}) K
//     O  = diag(q_scale e^gamma) Y + P U'      (stored as 32-bit words of two value columns)
// with the same operand splits as the fused kernel (U' hi / lo in the state update, P and U'
// hi / lo in P U').
//
// Data movement: each chunk's fragments go straight from memory to LDS (buffer_load ...
// lds), two stages deep, so chunk c + 1 lands while chunk c computes.  Each wave issues an
// equal share of the stage's 1 KiB pieces and waits for its own; a barrier then publishes
// the stage, and the first pass's fragments of the next chunk are read into registers
// before the loop turns.  Every LDS read is one lane's 16 bytes of a fragment (conflict-free, and a
// plain read: the compiler can then tell that the next stage's loads do not touch the
// stage being read, and adds no wait for them).
#include "internal.h"

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
    for (int i = 0; i < 8; ++i) {
        const float x = t[8 * (s & 1) + i];
        const bf16 xh = (bf16)x;
        hi[i] = xh;
        lo[i] = (bf16)(x - (float)xh);
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

template <int DK, int NWB>
struct Stage {
    bf16 Wn[2 * (DK / 16) * 512]; // -W fragments
    bf16 Q[2 * (DK / 16) * 512];  // Q fragments
    bf16 KT[4 * (DK / 32) * 512]; // K^T fragments
    bf16 Ph[6 * 512];             // P hi fragments
    bf16 Pl[6 * 512];             // P lo fragments
    float U0[NWB * 2 * 64 * 16];  // U0 accumulators of this workgroup's waves
    float tab[4][CH];             // beta, q_scale e^gamma, e^{gamma_last - gamma}, e^gamma
};

// The stage's 1 KiB pieces in issue order: -W, Q [WITH_O], K^T, P hi, P lo [WITH_O], U0,
// tables, each a contiguous KiB of the record.
template <int DK, int NWB, bool WITH_O>
struct Pieces {
    static constexpr int WN = 2 * (DK / 16);
    static constexpr int Q = WITH_O ? 2 * (DK / 16) : 0;
    static constexpr int KT = 4 * (DK / 32);
    static constexpr int P = WITH_O ? 12 : 0;
    static constexpr int U0 = NWB * 8;
    static constexpr int TOTAL = WN + Q + KT + P + U0 + 1;
};

// Wave W's pieces (every NWB-th, from W) of one chunk's stage; the list is fixed at compile
// time.
template <int DK, int DV, int NWB, bool WITH_O, int W>
__device__ __forceinline__ void issue_pieces(Stage<DK, NWB>& S, __amdgpu_buffer_rsrc_t rr, uint32_t rec_soff,
                                             uint32_t u0_base, uint32_t lane16) {
    using PC = Pieces<DK, NWB, WITH_O>;
#pragma unroll
    for (int p = W; p < PC::TOTAL; p += NWB) {
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

template <int DK, int DV, int NWB, bool WITH_O>
__global__ void __launch_bounds__(64 * NWB, 1)
gdn_scan_split_kernel(const int32_t* __restrict__ cu, int B, int Hv,
                      int uniform_len, long long state_bstride, const float* state_in, float* state_out,
                      bf16* __restrict__ o, const unsigned char* __restrict__ ws, long long rec_per_head)
{
    using PC = Pieces<DK, NWB, WITH_O>;
    constexpr int NG = DV / (32 * NWB);         // workgroups per (sequence, head)
    constexpr int KT_TILES = DK / 32;
    constexpr int KSTEPS_D = DK / 16;
    constexpr uint32_t REC = (uint32_t)split_record_bytes(DK, DV);
    // each wave's memory operations between its wait for a stage and the wait before it:
    // its pieces of the next stage and its output stores
    constexpr int OWN_PIECES = (PC::TOTAL + NWB - 1) / NWB;
    constexpr int O_STORES = WITH_O ? 16 : 0;
    static_assert(OWN_PIECES + O_STORES <= 63, "more memory operations in flight than vmcnt counts");

    extern __shared__ __align__(16) unsigned char smem_raw[];
    Stage<DK, NWB>* st = reinterpret_cast<Stage<DK, NWB>*>(smem_raw);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int col0 = 32 * (grp * NWB + wave);   // this wave's first value column

    const uint32_t v_stride = (uint32_t)Hv * DV * 2;
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(ws + ((size_t)hv * rec_per_head + (size_t)(bos / CH + b)) * REC,
                                                (uint32_t)n_chunks * REC);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(WITH_O ? o + ((size_t)bos * Hv + hv) * DV : nullptr,
                                                WITH_O ? (uint32_t)len * v_stride : 0u);
    const uint32_t u0_base = (uint32_t)(grp * NWB) * 8192;   // this workgroup's U0 fragments

    // Issue this wave's pieces of chunk c into stage sidx (the other waves issue the rest).
    auto issue_stage = [&](int c, int sidx) {
        const uint32_t rec_soff = (uint32_t)c * REC;
        Stage<DK, NWB>& S = st[sidx];
        const uint32_t lane16 = (uint32_t)(threadIdx.x & 63) * 16;
        if (wave == 0) issue_pieces<DK, DV, NWB, WITH_O, 0>(S, rr, rec_soff, u0_base, lane16);
        else if (NWB > 1 && wave == 1) issue_pieces<DK, DV, NWB, WITH_O, 1>(S, rr, rec_soff, u0_base, lane16);
        else if (NWB > 2 && wave == 2) issue_pieces<DK, DV, NWB, WITH_O, 2>(S, rr, rec_soff, u0_base, lane16);
        else if (NWB > 3) issue_pieces<DK, DV, NWB, WITH_O, 3>(S, rr, rec_soff, u0_base, lane16);
    };

    int l32 = lane & 31, h2 = lane >> 5;
    // ---- state: S^T tiles (dk rows x this wave's 32 value columns)
    f32x16 St[KT_TILES];
    const size_t sbase = (size_t)b * state_bstride + (size_t)hv * DV * DK + (size_t)(col0 + l32) * DK;
#pragma unroll
    for (int r = 0; r < KT_TILES; ++r) {
        if (state_in) {
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

    // The U'/Y pass's fragments (-W, Q) of chunk c are read at the end of iteration c - 1,
    // after the stage has landed: the reads cannot drift down to their uses across the loop
    // edge, so the pass's products find their operands in registers.
    bf16x8 fw[2 * KSTEPS_D], fq[2 * KSTEPS_D];
    auto read_pass = [&](const Stage<DK, NWB>& S) {
#pragma unroll
        for (int f = 0; f < 2 * KSTEPS_D; ++f) {
            fw[f] = frag(S.Wn, f, lane);
            if (WITH_O) fq[f] = frag(S.Q, f, lane);
        }
    };
    if (n_chunks > 0) {
        issue_stage(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (1 < n_chunks) issue_stage(1, 1);
        read_pass(st[0]);
    }
    for (int c = 0; c < n_chunks; ++c) {
        asm volatile("" : "+v"(lane));
        l32 = lane & 31; h2 = (lane >> 5) & 1;
        const Stage<DK, NWB>& S = st[c & 1];

        // U0 of this wave's columns (accumulator registers as the prep kernel left them)
        f32x16 U[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&S.U0[((wave * 2 + rt) * 64 + lane) * 16 + 4 * q4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[rt][4 * q4 + i] = x[i];
            }

        // U' = U0 + (-W) S^T and Y = Q S^T in one pass over the state operands
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
                U[rt] = mma32(fw[rt * KSTEPS_D + s], sb, U[rt]);
                if (WITH_O) Y[rt] = mma32(fq[rt * KSTEPS_D + s], sb, Y[rt]);
            }
        }
        bf16x8 uh[4], ul[4];
        if (WITH_O) {
#pragma unroll
            for (int s = 0; s < 4; ++s) acc_to_b_split(U[s >> 1], s, uh[s], ul[s]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const f32x4 e = *reinterpret_cast<const f32x4*>(&S.tab[1][32 * rt + 8 * j4 + 4 * h2]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Y[rt][4 * j4 + i] *= e[i];
                }
        }
        // S <- e^{gamma_n} S + U'^T diag(e^{gamma_n - gamma}) K and O = Y + P U'
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const f32x4 d = *reinterpret_cast<const f32x4*>(&S.tab[2][32 * rt + 8 * j4 + 4 * h2]);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[rt][4 * j4 + i] *= d[i];
            }
        const float decay = S.tab[3][CH - 1];
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
                const bf16x8 a = frag(S.KT, s * KT_TILES + r, lane);
                St[r] = mma32(a, dh, St[r]);
                St[r] = mma32(a, dl, St[r]);
            }
            if (WITH_O) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    if (s < 2 * rt + 2) {                  // P is lower triangular
                        const int f = rt == 0 ? s : 2 + s;
                        const bf16x8 ph = frag(S.Ph, f, lane);
                        const bf16x8 pl = frag(S.Pl, f, lane);
                        Y[rt] = mma32(ph, uh[s], Y[rt]);
                        Y[rt] = mma32(ph, ul[s], Y[rt]);
                        Y[rt] = mma32(pl, uh[s], Y[rt]);
                    }
                }
            }
        }
        if (WITH_O) {
            // O as 32-bit words: lane (l, h) holds column col0 + l of tokens 8 q + 4 h + {0..3}
            // (per row tile); for each token pair (t, t + 1), lanes 2m and 2m + 1 swap halves and
            // store columns (2m, 2m + 1) of tokens t and t + 1 respectively, so each store
            // instruction covers whole 64-byte row runs.
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
        if (c + 1 < n_chunks) {
            // Wait for this wave's share of chunk c + 1 (only this chunk's output stores were
            // issued after it), then for everyone's; the barrier also ends every wave's reads of
            // this chunk's stage, which the issue of chunk c + 2 overwrites.
            asm volatile("s_waitcnt vmcnt(%0)" :: "i"(O_STORES) : "memory");
            __builtin_amdgcn_s_barrier();
            if (c + 2 < n_chunks) issue_stage(c + 2, c & 1);
            read_pass(st[(c + 1) & 1]);
        }
    }

    // ---- write the final state
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

constexpr int kScanWaves = 2;   // waves (32 value columns each) per scan workgroup

template <int DK, int DV, bool WITH_O>
hipError_t launch_scan(const GdnArgs& a, const SplitPlan& plan, hipStream_t stream) {
    auto kern = gdn_scan_split_kernel<DK, DV, kScanWaves, WITH_O>;
    const size_t smem = 2 * sizeof(Stage<DK, kScanWaves>);
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const long long items = (long long)a.B * a.Hv * (DV / (32 * kScanWaves));
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
