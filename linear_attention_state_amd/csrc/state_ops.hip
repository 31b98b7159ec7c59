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
// fp32 MFMA (16x16x4).  A workgroup of DK / 16 waves takes 16 rows of one matrix's output (the
// matrix's row blocks on one XCD, so Phi comes from memory once per matrix); wave w owns
// columns [16 w, 16 w + 16).  The A operand is the row block of S_c staged in LDS (rows padded
// to DK + 8 floats, so each lane's 16-byte read is conflict-free), the B operand Phi's column
// slab from memory.  The contraction index is visited in the order that lets each lane read
// its A values as one 16-byte load: at step 4 kk + i, lane group gq = lane / 16 takes
// k = 16 kk + 4 gq + i.
template <int DK>
__global__ void __launch_bounds__(DK * 4)
state_compose_kernel(const float* __restrict__ S_c, const float* __restrict__ Phi,
                     const float* __restrict__ log_scale, const float* S_hat, float* out, int N, int dv)
{
    constexpr int NW = DK / 16;                         // waves, one per 16 columns
    constexpr int SR = DK + 8;
    constexpr int KS = DK / 4;                          // MFMA steps
    __shared__ __align__(16) float sA[16 * SR];
    int n, rb;
    xcd_item((int)blockIdx.x, dv / 16, n, rb);
    if (n >= N) return;
    const int tid = (int)threadIdx.x;
    const int w = tid / 64, lane = tid % 64, m = lane % 16, gq = lane / 16;
    const float* A = S_c + ((size_t)n * dv + (size_t)rb * 16) * DK;
    const float* P = Phi + (size_t)n * DK * DK + 16 * w + m;
    float bv[KS];
#pragma unroll
    for (int v = 0; v < KS; ++v) bv[v] = P[(size_t)(16 * (v / 4) + 4 * gq + v % 4) * DK];
#pragma unroll
    for (int i = 0; i < 16 * DK / 4 / (NW * 64); ++i) {
        const int idx = (tid + NW * 64 * i) * 4;
        *reinterpret_cast<f32x4*>(&sA[(idx / DK) * SR + idx % DK]) = *reinterpret_cast<const f32x4*>(A + idx);
    }
    __syncthreads();
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK / 16; ++kk) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&sA[m * SR + 16 * kk + 4 * gq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (kk % 2 == 0) a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bv[4 * kk + i], a0, 0, 0, 0);
            else a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bv[4 * kk + i], a1, 0, 0, 0);
        }
    }
    const f32x4 acc = a0 + a1;
    const float scale = log_scale ? expf(log_scale[n]) : 1.f;
    // accumulator layout: lane (m, gq) holds rows 4 gq + i of column 16 w + m
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const size_t off = ((size_t)n * dv + 16 * rb + 4 * gq + i) * DK + 16 * w + m;
        float x = scale * acc[i];
        if (S_hat) x += S_hat[off];
        out[off] = x;
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
    const long long blocks = xcd_grid(N, dv / 16);
    if (blocks > 0x7fffffffLL || dv % 16 != 0) return hipErrorInvalidValue;
    if (dk == 128)
        hipLaunchKernelGGL((state_compose_kernel<128>), dim3((unsigned)blocks), dim3(512), 0, stream, S_c, Phi, log_scale,
                           S_hat, out, N, dv);
    else if (dk == 64)
        hipLaunchKernelGGL((state_compose_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, stream, S_c, Phi, log_scale,
                           S_hat, out, N, dv);
    else
        return hipErrorInvalidValue;
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
