// State algebra and single-token steps around the replay:
//   state_compose_kernel  out = e^ls S_c Phi (+ S_hat): the linearity of the recurrence in its
//                         starting state (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制",
//                         section 2.3, the decomposition of S_m into the propagated start and the
//                         replayed part), used for the exact truncation error E_m = S_a Phi and
//                         for continuing from a checkpoint.
//   gdn_decode_kernel     one recurrence step per (sequence, value head) on a resident state
//                         (section 2.3 Eq. (1) with the read-out after the update), the step that
//                         follows the replay when the new suffix is generated (section 2.2, step 4).
#include "internal.h"

namespace tr {
namespace {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- out = e^ls S_c Phi (+ S_hat)
// One 64x64 output tile per workgroup of 256 threads (4x4 outputs each), k in slices of 32
// through LDS.  fp32 throughout.
__global__ void __launch_bounds__(256)
state_compose_kernel(const float* __restrict__ S_c, const float* __restrict__ Phi,
                     const float* __restrict__ log_scale, const float* S_hat, float* out, int dv, int dk)
{
    __shared__ float sA[64][32 + 1];
    __shared__ float sB[32][64 + 4];
    const int tiles_c = dk / 64, tiles = (dv / 64) * tiles_c;
    const int n = blockIdx.x / tiles;
    const int t = blockIdx.x % tiles;
    const int r0 = (t / tiles_c) * 64, c0 = (t % tiles_c) * 64;
    const float* A = S_c + (size_t)n * dv * dk;
    const float* P = Phi + (size_t)n * dk * dk;
    const int tid = threadIdx.x;
    const int tr = tid >> 4, tc = tid & 15;
    const float scale = log_scale ? expf(log_scale[n]) : 1.f;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < dk; k0 += 32) {
        for (int i = tid; i < 64 * 32; i += 256) {
            sA[i >> 5][i & 31] = A[(size_t)(r0 + (i >> 5)) * dk + k0 + (i & 31)];
            sB[i >> 6][i & 63] = P[(size_t)(k0 + (i >> 6)) * dk + c0 + (i & 63)];
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < 32; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { a[i] = sA[4 * tr + i][kk]; b[i] = sB[kk][4 * tc + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const size_t off = (size_t)n * dv * dk + (size_t)(r0 + 4 * tr + i) * dk + c0 + 4 * tc;
        f32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = scale * acc[i][j];
        if (S_hat) x += *reinterpret_cast<const f32x4*>(S_hat + off);
        *reinterpret_cast<f32x4*>(out + off) = x;
    }
}

// ---------------------------------------------------------------- one recurrence step
// Workgroup per (sequence, value head); DK / 8 lanes share one state row, 8 fp32 each:
//   s <- alpha s + beta (v_r - alpha s.k) k,   o_r = q_scale s.q
template <int DK, bool BF16>
__global__ void __launch_bounds__(256)
gdn_decode_kernel(const DecodeArgs a)
{
    constexpr int LPR = DK / 8;               // lanes per state row
    constexpr int RPP = 256 / LPR;            // rows per pass
    const int b = blockIdx.x / a.Hv;
    const int hv = blockIdx.x % a.Hv;
    const int hq = hv / (a.Hv / a.Hqk);
    const int tid = threadIdx.x;
    const int cl = (tid % LPR) * 8;
    const size_t kq = ((size_t)b * a.Hqk + hq) * DK + cl;
    const size_t head = (size_t)b * a.Hv + hv;
    float kv[8], qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (BF16) {
            kv[i] = (float)((const bf16*)a.k)[kq + i];
            qv[i] = (float)((const bf16*)a.q)[kq + i];
        } else {
            kv[i] = ((const float*)a.k)[kq + i];
            qv[i] = ((const float*)a.q)[kq + i];
        }
    }
    const float alpha = expf(a.g[head]);
    const float bt = a.beta[head];
    float* S = a.state + head * a.dv * DK;
    for (int r = tid / LPR; r < a.dv; r += RPP) {
        float* row = S + (size_t)r * DK + cl;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(row);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(row + 4);
        float s[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        float sk = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sk = fmaf(s[i], kv[i], sk);
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) sk += __shfl_xor(sk, m, 64);
        const float vr = BF16 ? (float)((const bf16*)a.v)[head * a.dv + r] : ((const float*)a.v)[head * a.dv + r];
        const float coef = bt * (vr - alpha * sk);
        float so = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = fmaf(alpha, s[i], coef * kv[i]);
            so = fmaf(s[i], qv[i], so);
        }
        *reinterpret_cast<f32x4*>(row) = f32x4{s[0], s[1], s[2], s[3]};
        *reinterpret_cast<f32x4*>(row + 4) = f32x4{s[4], s[5], s[6], s[7]};
        if (a.o) {
#pragma unroll
            for (int m = 1; m < LPR; m <<= 1) so += __shfl_xor(so, m, 64);
            if (tid % LPR == 0) {
                if (BF16) ((bf16*)a.o)[head * a.dv + r] = (bf16)(a.q_scale * so);
                else ((float*)a.o)[head * a.dv + r] = a.q_scale * so;
            }
        }
    }
}

}  // namespace

hipError_t launch_state_compose(const float* S_c, const float* Phi, const float* log_scale, const float* S_hat,
                                float* out, int N, int dv, int dk, hipStream_t stream) {
    const unsigned blocks = (unsigned)N * (unsigned)((dv / 64) * (dk / 64));
    hipLaunchKernelGGL(state_compose_kernel, dim3(blocks), dim3(256), 0, stream, S_c, Phi, log_scale, S_hat, out,
                       dv, dk);
    return hipGetLastError();
}

hipError_t launch_gdn_decode(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.Hv));
    if (a.dk == 128) {
        if (a.is_bf16) hipLaunchKernelGGL((gdn_decode_kernel<128, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((gdn_decode_kernel<128, false>), grid, dim3(256), 0, stream, a);
    } else if (a.dk == 64) {
        if (a.is_bf16) hipLaunchKernelGGL((gdn_decode_kernel<64, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((gdn_decode_kernel<64, false>), grid, dim3(256), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tr
