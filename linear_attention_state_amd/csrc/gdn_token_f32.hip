// Token-serial Gated DeltaNet recurrence in fp32, for fp32 inputs.
//
// Reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.3, Eq. (1), with
// the state stored dv x dk: S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
// which is the same matrix as alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T;
// read-out o_t = S_t (q_scale q_t).
//
// One workgroup per (sequence, value head); thread r owns state row r (dk fp32 values in
// registers), so every product is a per-thread dot product with no cross-thread
// reduction.  Keys and queries of 32 tokens at a time are staged in LDS and read by all
// threads.  This path serves fp32 inputs, where bf16 MFMA operands would not be exact, and
// the transition product of bf16 inputs, which wants fp32 arithmetic (its inputs are read
// as bf16 and converted exactly).
#include "internal.h"

namespace tr {
namespace {

constexpr int CH = 32;            // tokens staged per pass (keeps static LDS at 32 KiB for dk = 128)

template <int DK, typename TI>
__global__ void __launch_bounds__(128)
gdn_token_f32_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                     const TI* __restrict__ v, const float* __restrict__ g,
                     const float* __restrict__ beta, const int32_t* __restrict__ cu,
                     int Hqk, int Hv, int DV, float q_scale, int uniform_len, long long state_bstride,
                     const float* state_in, int state_identity, float* state_out, TI* __restrict__ o,
                     float* log_scale_out)
{
    __shared__ float sK[CH][DK];
    __shared__ float sQ[CH][DK];
    __shared__ float sA[CH];
    __shared__ float sB[CH];

    const int b = blockIdx.x / Hv;
    const int hv = blockIdx.x % Hv;
    const int hq = hv / (Hv / Hqk);
    const int r = threadIdx.x;            // state row (value index); blockDim.x == DV
    const int bos = cu ? cu[b] : b * uniform_len;
    const int len = cu ? cu[b + 1] - bos : uniform_len;
    const size_t sbase = (size_t)b * state_bstride + ((size_t)hv * DV + r) * DK;

    float log_sum = 0.f;
    float S[DK];
#pragma unroll
    for (int c = 0; c < DK; ++c) S[c] = state_identity ? (c == r ? 1.f : 0.f) : (state_in ? state_in[sbase + c] : 0.f);

    for (int c0 = 0; c0 < len; c0 += CH) {
        const int n = min(CH, len - c0);
        __syncthreads();
        for (int i = threadIdx.x; i < n * DK; i += blockDim.x) {
            const int t = i / DK, c = i % DK;
            const size_t off = ((size_t)(bos + c0 + t) * Hqk + hq) * DK + c;
            sK[t][c] = (float)k[off];
            sQ[t][c] = q ? (float)q[off] : 0.f;   // q may be null when o is
        }
        for (int t = threadIdx.x; t < n; t += blockDim.x) {
            const float gt = g[(size_t)(bos + c0 + t) * Hv + hv];
            // with log_scale_out, the decay is kept out of S and summed in log space instead
            sA[t] = log_scale_out ? 1.f : __expf(gt);
            sB[t] = beta[(size_t)(bos + c0 + t) * Hv + hv];
        }
        if (log_scale_out && threadIdx.x == 0)
            for (int t = 0; t < n; ++t) log_sum += g[(size_t)(bos + c0 + t) * Hv + hv];
        __syncthreads();
        for (int t = 0; t < n; ++t) {
            const size_t tok = (size_t)(bos + c0 + t) * Hv + hv;
            const float a = sA[t];
            float sk = 0.f;
#pragma unroll
            for (int c = 0; c < DK; ++c) sk = fmaf(S[c], sK[t][c], sk);
            const float coef = sB[t] * ((v ? (float)v[tok * DV + r] : 0.f) - a * sk);   // null v: zero values
            float so = 0.f;
#pragma unroll
            for (int c = 0; c < DK; ++c) {
                S[c] = fmaf(a, S[c], coef * sK[t][c]);
                so = fmaf(S[c], sQ[t][c], so);
            }
            if (o) o[tok * DV + r] = (TI)(q_scale * so);
        }
    }
#pragma unroll
    for (int c = 0; c < DK; ++c) state_out[sbase + c] = S[c];
    if (log_scale_out && threadIdx.x == 0) log_scale_out[(size_t)b * Hv + hv] = log_sum;
}

}  // namespace

template <typename TI>
hipError_t launch_token(const GdnArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.Hv));
    const dim3 block((unsigned)a.dv);
    if (a.dk == 128) {
        hipLaunchKernelGGL((gdn_token_f32_kernel<128, TI>), grid, block, 0, stream,
                           (const TI*)a.q, (const TI*)a.k, (const TI*)a.v, a.g, a.beta,
                           a.cu_seqlens, a.Hqk, a.Hv, a.dv, a.q_scale, a.uniform_len, (long long)a.state_bstride,
                           a.state_in, a.state_identity, a.state_out, (TI*)a.o, a.log_scale_out);
    } else if (a.dk == 64) {
        hipLaunchKernelGGL((gdn_token_f32_kernel<64, TI>), grid, block, 0, stream,
                           (const TI*)a.q, (const TI*)a.k, (const TI*)a.v, a.g, a.beta,
                           a.cu_seqlens, a.Hqk, a.Hv, a.dv, a.q_scale, a.uniform_len, (long long)a.state_bstride,
                           a.state_in, a.state_identity, a.state_out, (TI*)a.o, a.log_scale_out);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gdn_token_f32(const GdnArgs& a, hipStream_t stream) { return launch_token<float>(a, stream); }
hipError_t launch_gdn_token_f32_bf16in(const GdnArgs& a, hipStream_t stream) { return launch_token<__bf16>(a, stream); }

}  // namespace tr
