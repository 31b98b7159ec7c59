// Token-serial Gated DeltaNet recurrence in fp32, for fp32 inputs.
//
// Reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.3, Eq. (1), with
// the state stored dv x dk: S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
// which is the same matrix as alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T;
// read-out o_t = S_t (q_scale q_t).  The operator acts from the right, so every row of S
// evolves on its own: row r needs only its own dot product with k_t and entry r of v_t.
//
// Work decomposition: a workgroup of 256 threads takes 16 rows of one (sequence, value head);
// a row is spread over 16 lanes, lane j holding E = dk / 16 key columns in groups of four,
// 4 j + 64 g + {0..3} for group g, so that the 16 lanes' 16-byte LDS reads of a key (or query)
// row are contiguous and free of bank conflicts.  Per
// token a row costs E fused multiply-adds per lane for S k, a four-step sum across its 16
// lanes (DPP row rotations, so every lane ends with the total), and E more for the update:
// the serial chain per token is a few dozen cycles instead of dk dependent steps in one
// thread.  Keys (and queries, with outputs) of 64 tokens are staged in LDS, double-buffered:
// the next chunk's loads are issued into registers before the current chunk is processed, and
// written to the other buffer after it; tokens go four at a time, so the LDS reads of the
// next tokens are issued ahead of the current token's dependent chain.  This path serves fp32
// inputs, where bf16 MFMA operands would not be exact.
#include "internal.h"

namespace tr {
namespace {

constexpr int LPR = 16;           // lanes per state row
constexpr int NTH = 256;          // threads per workgroup
constexpr int ROWS = NTH / LPR;   // state rows per workgroup
constexpr int TC = 64;            // tokens per staged chunk

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));  // row_ror:8
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));  // row_ror:4
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));  // row_ror:2
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));  // row_ror:1
    return x;
}

// E consecutive inputs as fp32 (bf16 converts exactly).
template <int E, typename TI>
__device__ __forceinline__ void load_f32(const TI* p, float* out) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = (float)p[e];
}

template <int DK, typename TI, bool WITH_O>
__global__ void __launch_bounds__(NTH)
gdn_token_f32_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                     const TI* __restrict__ v, const float* __restrict__ g,
                     const float* __restrict__ beta, const int32_t* __restrict__ cu,
                     int Hqk, int Hv, int DV, float q_scale, int uniform_len, long long state_bstride,
                     const float* state_in, float* state_out, TI* __restrict__ o)
{
    constexpr int E = DK / LPR;                         // key columns per lane
    constexpr int VEC = 16 / sizeof(TI);                // inputs per 16-byte load
    constexpr int KLOADS = TC * DK / VEC / NTH;         // 16-byte loads of a chunk's keys per thread
    static_assert(KLOADS * VEC * NTH == TC * DK, "staging covers the chunk");
    __shared__ __align__(16) TI sK[2][TC][DK];
    __shared__ __align__(16) TI sQ[WITH_O ? 2 : 1][WITH_O ? TC : 1][DK];
    __shared__ float sA[2][TC], sB[2][TC];
    __shared__ float sV[2][TC][ROWS];

    const int row_blocks = DV / ROWS;
    const int item = (int)blockIdx.x;                   // (sequence, head, row block)
    const int hv = (item / row_blocks) % Hv;
    const int rb = item % row_blocks;
    const int b = item / (Hv * row_blocks);
    const int hq = hv / (Hv / Hqk);
    const int tid = (int)threadIdx.x;
    const int lr = tid / LPR, j = tid % LPR;
    const int r = rb * ROWS + lr;                       // state row (value index)
    const int bos = cu ? cu[b] : b * uniform_len;
    const int len = cu ? cu[b + 1] - bos : uniform_len;
    const size_t sbase = (size_t)b * state_bstride + ((size_t)hv * DV + r) * DK;
    auto col = [&](int e) { return 4 * LPR * (e / 4) + 4 * j + e % 4; };   // key column of S[e]

    float S[E];
#pragma unroll
    for (int e = 0; e < E; ++e) S[e] = state_in ? state_in[sbase + col(e)] : 0.f;

    // chunk staging registers: keys (and queries), this workgroup's values, gates
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 rk[KLOADS], rq[WITH_O ? KLOADS : 1];
    float rv[TC * ROWS / NTH], ra = 0.f, rbeta = 0.f;
    auto fetch = [&](int c0) {
        const int n = min(TC, len - c0);
#pragma unroll
        for (int i = 0; i < KLOADS; ++i) {
            const int idx = tid + NTH * i;
            const int t = idx / (DK / VEC), c = (idx % (DK / VEC)) * VEC;
            const size_t off = ((size_t)(bos + c0 + t) * Hqk + hq) * DK + c;
            rk[i] = t < n ? *reinterpret_cast<const u32x4*>(k + off) : u32x4{0u, 0u, 0u, 0u};
            if (WITH_O) rq[i] = t < n ? *reinterpret_cast<const u32x4*>(q + off) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < TC * ROWS / NTH; ++i) {
            const int idx = tid + NTH * i;
            const int t = idx / ROWS, rr = idx % ROWS;
            rv[i] = (t < n && v) ? (float)v[((size_t)(bos + c0 + t) * Hv + hv) * DV + rb * ROWS + rr] : 0.f;
        }
        if (tid < TC) {
            ra = tid < n ? g[(size_t)(bos + c0 + tid) * Hv + hv] : 0.f;
            rbeta = tid < n ? beta[(size_t)(bos + c0 + tid) * Hv + hv] : 0.f;
        }
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KLOADS; ++i) {
            const int idx = tid + NTH * i;
            const int t = idx / (DK / VEC), c = (idx % (DK / VEC)) * VEC;
            *reinterpret_cast<u32x4*>(&sK[buf][t][c]) = rk[i];
            if (WITH_O) *reinterpret_cast<u32x4*>(&sQ[WITH_O ? buf : 0][WITH_O ? t : 0][c]) = rq[WITH_O ? i : 0];
        }
#pragma unroll
        for (int i = 0; i < TC * ROWS / NTH; ++i) {
            const int idx = tid + NTH * i;
            sV[buf][idx / ROWS][idx % ROWS] = rv[i];
        }
        if (tid < TC) {
            sA[buf][tid] = __expf(ra);
            sB[buf][tid] = rbeta;
        }
    };

    int buf = 0;
    if (len > 0) {
        fetch(0);
        put(0);
    }
    __syncthreads();
    for (int c0 = 0; c0 < len; c0 += TC) {
        const int n = min(TC, len - c0);
        const bool more = c0 + TC < len;
        if (more) fetch(c0 + TC);                       // lands while this chunk is processed
        auto step = [&](int t) {
            float kv[E];
#pragma unroll
            for (int e = 0; e < E; e += 4) load_f32<4>(&sK[buf][t][col(e)], kv + e);
            const float a = sA[buf][t], bt = sB[buf][t], vr = sV[buf][t][lr];
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int e = 0; e < E; e += 2) {
                p0 = fmaf(S[e], kv[e], p0);
                p1 = fmaf(S[e + 1], kv[e + 1], p1);
            }
            const float sk = row16_sum(p0 + p1);
            const float coef = bt * (vr - a * sk);
#pragma unroll
            for (int e = 0; e < E; ++e) S[e] = fmaf(a, S[e], coef * kv[e]);
            if (WITH_O) {
                float qv[E];
#pragma unroll
                for (int e = 0; e < E; e += 4) load_f32<4>(&sQ[WITH_O ? buf : 0][WITH_O ? t : 0][col(e)], qv + e);
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int e = 0; e < E; e += 2) {
                    s0 = fmaf(S[e], qv[e], s0);
                    s1 = fmaf(S[e + 1], qv[e + 1], s1);
                }
                const float so = row16_sum(s0 + s1);
                if (j == 0) o[((size_t)(bos + c0 + t) * Hv + hv) * DV + r] = (TI)(q_scale * so);
            }
        };
        int t = 0;
        for (; t + 4 <= n; t += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) step(t + u);
        }
        for (; t < n; ++t) step(t);
        __syncthreads();                                // every thread is done with buffer buf
        if (more) {
            put(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) state_out[sbase + col(e)] = S[e];
}

template <int DK, typename TI>
hipError_t launch_dk(const GdnArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.Hv * (a.dv / ROWS)));
    if (a.o) {
        hipLaunchKernelGGL((gdn_token_f32_kernel<DK, TI, true>), grid, dim3(NTH), 0, stream,
                           (const TI*)a.q, (const TI*)a.k, (const TI*)a.v, a.g, a.beta,
                           a.cu_seqlens, a.Hqk, a.Hv, a.dv, a.q_scale, a.uniform_len, (long long)a.state_bstride,
                           a.state_in, a.state_out, (TI*)a.o);
    } else {
        hipLaunchKernelGGL((gdn_token_f32_kernel<DK, TI, false>), grid, dim3(NTH), 0, stream,
                           (const TI*)a.q, (const TI*)a.k, (const TI*)a.v, a.g, a.beta,
                           a.cu_seqlens, a.Hqk, a.Hv, a.dv, a.q_scale, a.uniform_len, (long long)a.state_bstride,
                           a.state_in, a.state_out, (TI*)nullptr);
    }
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_token(const GdnArgs& a, hipStream_t stream) {
    if (a.dv % ROWS != 0 || a.state_identity || a.log_scale_out) return hipErrorInvalidValue;
    if (a.dk == 128) return launch_dk<128, TI>(a, stream);
    if (a.dk == 64) return launch_dk<64, TI>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gdn_token_f32(const GdnArgs& a, hipStream_t stream) { return launch_token<float>(a, stream); }

}  // namespace tr
