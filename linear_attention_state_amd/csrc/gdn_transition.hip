// Transition product of a replayed span, Phi = T_1 T_2 ... T_n with T_t = alpha_t (I - beta_t
// k_t k_t^T): the recurrence of reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制",
// section 2.3, Eq. (1), started from S = I with every value zero.  By section 2.3's split of
// the rebuilt state (the start carried through the span's operators plus the replay from
// zero), S_a Phi is the part of S_m that a replay from zero leaves out.
//
// The decays are scalars, so they are kept out of the matrix product: the kernels form
// (I - beta_1 k_1 k_1^T) ... (I - beta_n k_n k_n^T) and the sum of the gates, and the caller
// either receives that log scale or has it applied once at the end.  Every factor has norm at
// most 1 for beta |k|^2 <= 2, so the product stays in range without the decay.
//
// transition_segment_kernel: token-serial fp32.  A workgroup of 256 threads takes 16 rows of
// one (sequence, segment, head); a row is spread over 16 lanes, lane j holding E = d / 16 key
// columns in groups of four, 4 j + 64 q + {0..3} for group q (so the 16 lanes' 16-byte LDS
// reads of a key row are contiguous and conflict-free).  Per token: row . k over the row's
// lanes (E fused multiply-adds,
// then a four-step sum by DPP row rotations), then row -= beta (row . k) k^T (E more).  Keys
// of 32 tokens at a time are staged in LDS as fp32 (bf16 keys are converted once there, not
// once per row), double-buffered behind register loads of the next 32 tokens.
//
// The product is associative, so a span with few heads is cut into segments that run side by
// side from I; transition_chain_kernel then multiplies each head's segment products in order
// on fp32 MFMA (16x16x4): a workgroup takes 16 rows of Phi with one wave per 16 columns, the
// running 16-row block shared through LDS and the next factor's columns loaded into registers
// while the current factor is applied.
#include "internal.h"

namespace tr {
namespace {

constexpr int LPR = 16;            // lanes per row
constexpr int NTH = 256;           // threads per segment workgroup
constexpr int ROWS = NTH / LPR;    // rows per segment workgroup
constexpr int TC = 32;             // tokens per staged block
static_assert(ROWS == kTransitionRows, "the host plan counts workgroups of kTransitionRows rows");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));  // row_ror:8
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));  // row_ror:4
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));  // row_ror:2
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));  // row_ror:1
    return x;
}

// 16 bytes of inputs as fp32 (bf16 converts exactly).
template <typename TI>
__device__ __forceinline__ void to_f32(const u32x4& w, float* out) {
    if constexpr (sizeof(TI) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned int u = w[e];                // a scalar: a cast of the vector element
            out[e] = __builtin_bit_cast(float, u);      // itself would read element 0
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = __builtin_bit_cast(float, w[e] << 16);
            out[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xffff0000u);
        }
    }
}

// Items are (sequence, segment, head, row block) with seg_len > 0, else (sequence, head, row
// block) over whole sequences, the row blocks of one (sequence, segment, head) on one XCD.  A sequence of one segment (or none) writes its result to
// phi_out / log_scale_out; longer ones write every segment's product and gate sum to the
// records for transition_chain_kernel.
template <int D, typename TI>
__global__ void __launch_bounds__(NTH)
transition_segment_kernel(const TI* __restrict__ k, const float* __restrict__ g, const float* __restrict__ beta,
                          const int32_t* __restrict__ cu, int Hqk, int Hv, int seg_len, int seg_max, int n_pairs,
                          float* __restrict__ seg_phi, float* __restrict__ seg_log,
                          float* __restrict__ phi_out, float* __restrict__ log_scale_out)
{
    constexpr int E = D / LPR;                          // key columns per lane
    constexpr int VEC = 16 / sizeof(TI);                // inputs per 16-byte load
    constexpr int KLOADS = TC * D / VEC / NTH;          // 16-byte key loads per thread per block
    static_assert(KLOADS >= 1 && KLOADS * VEC * NTH == TC * D, "staging covers the block");
    __shared__ __align__(16) float sK[2][TC][D];
    __shared__ __align__(16) float sB[2][TC];
    __shared__ float sG[2][TC];

    int pair, rb;                                       // pair = (sequence or sequence-segment, head)
    xcd_item((int)blockIdx.x, D / ROWS, pair, rb);
    if (pair >= n_pairs) return;                        // the whole workgroup, before any barrier
    const int hv = pair % Hv;
    const int bs = pair / Hv;
    const int b = seg_len > 0 ? bs / seg_max : bs;
    const int seg = seg_len > 0 ? bs % seg_max : 0;
    const int hq = hv / (Hv / Hqk);
    const int tid = (int)threadIdx.x;
    const int lr = tid / LPR, j = tid % LPR;
    const int r = rb * ROWS + lr;                       // row of the product
    auto col = [&](int e) { return 4 * LPR * (e / 4) + 4 * j + e % 4; };   // key column of S[e]
    int bos = cu[b];
    int len = cu[b + 1] - bos;
    bool to_records = false;
    if (seg_len > 0) {
        const int nseg = max(1, (len + seg_len - 1) / seg_len);
        if (seg >= nseg) return;                        // the whole workgroup, before any barrier
        to_records = nseg > 1;
        bos += seg * seg_len;
        len = min(seg_len, len - seg * seg_len);
    }

    float S[E];
#pragma unroll
    for (int e = 0; e < E; ++e) S[e] = (col(e) == r) ? 1.f : 0.f;

    u32x4 rk[KLOADS];
    float rg = 0.f, rbeta = 0.f;
    auto fetch = [&](int c0) {
        const int n = min(TC, len - c0);
#pragma unroll
        for (int i = 0; i < KLOADS; ++i) {
            const int idx = tid + NTH * i;
            const int t = idx / (D / VEC), c = (idx % (D / VEC)) * VEC;
            rk[i] = t < n ? *reinterpret_cast<const u32x4*>(k + ((size_t)(bos + c0 + t) * Hqk + hq) * D + c)
                          : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < TC) {
            rg = tid < n ? g[(size_t)(bos + c0 + tid) * Hv + hv] : 0.f;
            rbeta = tid < n ? beta[(size_t)(bos + c0 + tid) * Hv + hv] : 0.f;
        }
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KLOADS; ++i) {
            const int idx = tid + NTH * i;
            const int t = idx / (D / VEC), c = (idx % (D / VEC)) * VEC;
            float x[VEC];
            to_f32<TI>(rk[i], x);
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                *reinterpret_cast<f32x4*>(&sK[buf][t][c + e]) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};
        }
        if (tid < TC) {
            sB[buf][tid] = rbeta;
            sG[buf][tid] = rg;
        }
    };
    // one token: row -= beta (row . k) k^T; kr points at the token's key column 4 j
    auto step = [&](const float* kr, float bt) {
        float kv[E];
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(kr + 4 * LPR * (e / 4));
            kv[e] = x[0]; kv[e + 1] = x[1]; kv[e + 2] = x[2]; kv[e + 3] = x[3];
        }
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e += 2) {
            p0 = fmaf(S[e], kv[e], p0);
            p1 = fmaf(S[e + 1], kv[e + 1], p1);
        }
        const float c = -bt * row16_sum(p0 + p1);
#pragma unroll
        for (int e = 0; e < E; ++e) S[e] = fmaf(c, kv[e], S[e]);
    };

    float log_sum = 0.f;                                // thread 0: the gates summed in token order
    int buf = 0;
    if (len > 0) {
        fetch(0);
        put(0);
    }
    __syncthreads();
    for (int c0 = 0; c0 < len; c0 += TC) {
        const int n = min(TC, len - c0);
        const bool more = c0 + TC < len;
        if (more) fetch(c0 + TC);                       // lands while this block is applied
        if (tid == 0)
            for (int t = 0; t < n; ++t) log_sum += sG[buf][t];
        int t = 0;
        for (; t + 4 <= n; t += 4) {
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sB[buf][t]);
#pragma unroll
            for (int u = 0; u < 4; ++u) step(&sK[buf][t + u][4 * j], b4[u]);
        }
        for (; t < n; ++t) step(&sK[buf][t][4 * j], sB[buf][t]);
        __syncthreads();                                // every thread is done with buffer buf
        if (more) {
            put(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }

    if (to_records) {
        float* dst = seg_phi + (((size_t)bs * Hv + hv) * D + r) * D;
#pragma unroll
        for (int e = 0; e < E; e += 4) *reinterpret_cast<f32x4*>(dst + col(e)) = f32x4{S[e], S[e + 1], S[e + 2], S[e + 3]};
        if (tid == 0 && rb == 0) seg_log[(size_t)bs * Hv + hv] = log_sum;
        return;
    }
    // the gate sum reaches every thread through LDS (sG is free after the last barrier)
    if (tid == 0) sG[0][0] = log_sum;
    __syncthreads();
    const float ls = sG[0][0];
    const float scale = log_scale_out ? 1.f : __expf(ls);
    float* dst = phi_out + (((size_t)b * Hv + hv) * D + r) * D;
#pragma unroll
    for (int e = 0; e < E; e += 4)
        *reinterpret_cast<f32x4*>(dst + col(e)) = f32x4{scale * S[e], scale * S[e + 1], scale * S[e + 2], scale * S[e + 3]};
    if (log_scale_out && tid == 0 && rb == 0) log_scale_out[(size_t)b * Hv + hv] = ls;
}

// Phi = P_0 P_1 ... P_{nseg-1} for every (sequence, head) cut into several segments.  A
// workgroup of D / 16 waves takes 16 rows of one head's product (the head's row blocks on one
// XCD, so each factor comes from memory once per head); wave w owns columns
// [16 w, 16 w + 16).  Per factor, R_new[:, cols] = R P_s[:, cols] on v_mfma_f32_16x16x4_f32:
// the A operand is R from LDS, the B operand the factor's columns from memory.  The
// contraction index is visited in the order that lets each lane read its A values as one
// 16-byte LDS load: at step 4 kk + i, lane group gq = lane / 16 takes k = 16 kk + 4 gq + i.
template <int D>
__global__ void __launch_bounds__(D * 4)
transition_chain_kernel(const int32_t* __restrict__ cu, int Hv, int seg_len, int seg_max, int n_pairs,
                        const float* __restrict__ seg_phi, const float* __restrict__ seg_log,
                        float* __restrict__ phi_out, float* __restrict__ log_scale_out)
{
    constexpr int NW = D / 16;                          // waves, one per 16 columns
    constexpr int SR = D + 8;                           // LDS row stride: conflict-free 16-byte reads
    constexpr int KS = D / 4;                           // MFMA steps per factor
    __shared__ __align__(16) float sR[16 * SR];
    int pair, rb;                                       // pair = (sequence, head)
    xcd_item((int)blockIdx.x, D / 16, pair, rb);
    if (pair >= n_pairs) return;
    const int b = pair / Hv;
    const int hv = pair % Hv;
    const int len = cu[b + 1] - cu[b];
    const int nseg = max(1, (len + seg_len - 1) / seg_len);
    if (nseg < 2) return;                               // written in place by the segment kernel
    const int tid = (int)threadIdx.x;
    const int w = tid / 64, lane = tid % 64, m = lane % 16, gq = lane / 16;
    const size_t mat = (size_t)D * D;
    auto factor = [&](int s) { return seg_phi + ((size_t)(b * seg_max + s) * Hv + hv) * mat; };

    // rows [16 rb, 16 rb + 16) of P_0 into LDS
    {
        const float* P0 = factor(0) + (size_t)rb * 16 * D;
#pragma unroll
        for (int i = 0; i < 16 * D / 4 / (NW * 64); ++i) {
            const int idx = (tid + NW * 64 * i) * 4;
            *reinterpret_cast<f32x4*>(&sR[(idx / D) * SR + idx % D]) = *reinterpret_cast<const f32x4*>(P0 + idx);
        }
    }
    // B operand of a factor: step 4 kk + i takes row 16 kk + 4 gq + i, column 16 w + m
    float bn[KS];
    auto load_b = [&](int s) {
        const float* P = factor(s) + (size_t)16 * w + m;
#pragma unroll
        for (int v = 0; v < KS; ++v) bn[v] = P[(size_t)(16 * (v / 4) + 4 * gq + v % 4) * D];
    };
    load_b(1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 1; s < nseg; ++s) {
        float bc[KS];
#pragma unroll
        for (int v = 0; v < KS; ++v) bc[v] = bn[v];
        if (s + 1 < nseg) load_b(s + 1);                // lands while this factor is applied
        __syncthreads();                                // R is in LDS
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(&sR[m * SR + 16 * kk + 4 * gq]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (kk % 2 == 0) a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bc[4 * kk + i], a0, 0, 0, 0);
                else a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bc[4 * kk + i], a1, 0, 0, 0);
            }
        }
        acc = a0 + a1;
        if (s + 1 < nseg) {
            __syncthreads();                            // every wave is done reading R
            // accumulator layout: lane (m, gq) holds rows 4 gq + i of column 16 w + m
#pragma unroll
            for (int i = 0; i < 4; ++i) sR[(4 * gq + i) * SR + 16 * w + m] = acc[i];
        }
    }
    float ls = 0.f;
    for (int s = 0; s < nseg; ++s) ls += seg_log[(size_t)(b * seg_max + s) * Hv + hv];
    const float scale = log_scale_out ? 1.f : __expf(ls);
    float* dst = phi_out + ((size_t)b * Hv + hv) * mat + (size_t)(rb * 16) * D + 16 * w + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(size_t)(4 * gq + i) * D] = scale * acc[i];
    if (log_scale_out && rb == 0 && tid == 0) log_scale_out[(size_t)b * Hv + hv] = ls;
}

template <int D, typename TI>
hipError_t launch_d(const GdnArgs& a, const Segments& sg, hipStream_t stream) {
    const long long sets = sg.seg_len > 0 ? (long long)a.B * sg.seg_max : (long long)a.B;
    const long long pairs = sets * a.Hv;
    if (xcd_grid(pairs, D / ROWS) > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((transition_segment_kernel<D, TI>), dim3((unsigned)xcd_grid(pairs, D / ROWS)), dim3(NTH), 0, stream,
                       (const TI*)a.k, a.g, a.beta, a.cu_seqlens, a.Hqk, a.Hv, sg.seg_len, sg.seg_max, (int)pairs,
                       sg.phi, sg.log, a.state_out, a.log_scale_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sg.seg_len <= 0) return e;
    const long long heads = (long long)a.B * a.Hv;
    hipLaunchKernelGGL((transition_chain_kernel<D>), dim3((unsigned)xcd_grid(heads, D / 16)), dim3(D * 4), 0, stream,
                       a.cu_seqlens, a.Hv, sg.seg_len, sg.seg_max, (int)heads, (const float*)sg.phi,
                       (const float*)sg.log, a.state_out, a.log_scale_out);
    return hipGetLastError();
}

template <typename TI>
hipError_t launch(const GdnArgs& a, const Segments& sg, hipStream_t stream) {
    // from I with no values: square products, packed lengths on the device
    if (!a.state_identity || a.o || a.v || a.state_in || !a.cu_seqlens || a.dk != a.dv)
        return hipErrorInvalidValue;
    if (sg.seg_len > 0 && (sg.seg_max < 2 || !sg.phi || !sg.log)) return hipErrorInvalidValue;
    if (a.dk == 128) return launch_d<128, TI>(a, sg, stream);
    if (a.dk == 64) return launch_d<64, TI>(a, sg, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gdn_transition(const GdnArgs& a, bool keys_bf16, const Segments& sg, hipStream_t stream) {
    return keys_bf16 ? launch<__bf16>(a, sg, stream) : launch<float>(a, sg, stream);
}

}  // namespace tr
