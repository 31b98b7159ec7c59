// Kernels of the LA-layer body around the recurrence, for the group replay:
//   rmsnorm_kernel      y = bf16( x / sqrt(mean(x^2) + eps) * gain )
//   gemm_tn_kernel      C = A B^T on bf16 MFMA (A [M x K], B [N x K], both K-contiguous),
//                       batched over groups with per-group weights, with two epilogues:
//                       EPI_LAYER_IN : per-head L2 norm of q and k (q also x dk^-1/2),
//                                      bf16 v, g = -softplus(z_a), beta = sigmoid(z_b)
//                       EPI_RESIDUAL : x_out = bf16( x_in + C )
// The pages only say that the keys, values and gates are produced inside the group
// (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.1 symbol table);
// this is the plainest Gated DeltaNet layer body with the stated widths.
#include "internal.h"

namespace tr {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// --------------------------------------------------------------------------- RMSNorm
// One wave per row of d elements (d % 512 == 0 handled as d / 512 passes of 8 per lane).
__global__ void __launch_bounds__(256)
rmsnorm_kernel(const bf16* __restrict__ x, bf16* __restrict__ y, PtrTable gain, int rows_per_group,
               int rows, int d, float eps)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const bf16* xr = x + (size_t)row * d;
    const bf16* gr = (const bf16*)gain.p[row / rows_per_group];
    float ss = 0.f;
    for (int c = lane * 8; c < d; c += 512) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) { const float f = (float)v[i]; ss = fmaf(f, f, ss); }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    bf16* yr = y + (size_t)row * d;
    for (int c = lane * 8; c < d; c += 512) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c);
        bf16x8 o;
        if (gr) {
            const bf16x8 gv = *reinterpret_cast<const bf16x8*>(gr + c);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)v[i] * r * (float)gv[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)v[i] * r);
        }
        *reinterpret_cast<bf16x8*>(yr + c) = o;
    }
}

// --------------------------------------------------------------------------- GEMM
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;            // bf16 elements per staged row
constexpr int STAGE_STRIDE = BN + 4;          // fp32 elements per epilogue row

enum { EPI_LAYER_IN = 0, EPI_RESIDUAL = 1 };

struct GemmParams {
    const bf16* A;            // [G*M, K]
    PtrTable b0, b1, b2, b3;  // weight row blocks (see row_src)
    int n0, n1, n2, n3;       // rows in each block: N = n0 + n1 + n2 + n3
    int G, M, K, N;
    int n_mt, n_nt;           // tiles per group
    // EPI_LAYER_IN
    bf16* q; bf16* k; bf16* v; float* g; float* beta;
    int Hqk, Hv;
    float q_scale;
    // EPI_RESIDUAL
    const bf16* x_in; bf16* x_out;
};

__device__ __forceinline__ const bf16* row_src(const GemmParams& p, int g, int n) {
    if (n < p.n0) return (const bf16*)p.b0.p[g] + (size_t)n * p.K;
    n -= p.n0;
    if (n < p.n1) return (const bf16*)p.b1.p[g] + (size_t)n * p.K;
    n -= p.n1;
    if (n < p.n2) return (const bf16*)p.b2.p[g] + (size_t)n * p.K;
    n -= p.n2;
    if (n < p.n3) return (const bf16*)p.b3.p[g] + (size_t)n * p.K;
    return nullptr;
}

__device__ __forceinline__ float softplus_f(float z) { return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))); }
__device__ __forceinline__ float sigmoid_f(float z) {
    const float e = expf(-fabsf(z));
    return z >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

template <int EPI>
__global__ void __launch_bounds__(256, 2)
gemm_tn_kernel(const GemmParams p)
{
    __shared__ __align__(16) bf16 smem[2 * 2 * BM * LDS_STRIDE];   // [buf][A|B][row][k]
    bf16 (*sA)[BM][LDS_STRIDE] = reinterpret_cast<bf16 (*)[BM][LDS_STRIDE]>(smem);
    bf16 (*sB)[BN][LDS_STRIDE] = reinterpret_cast<bf16 (*)[BN][LDS_STRIDE]>(smem + 2 * BM * LDS_STRIDE);

    // XCD-aware tile order: consecutive logical tiles (same weight tile, successive row
    // tiles) land on the same XCD, whose L2 then serves the shared weight rows.
    const int n_tiles = p.G * p.n_mt * p.n_nt;
    const int per_xcd = (int)((gridDim.x + 7) / 8);
    const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (logical >= n_tiles) return;
    const int mt = logical % p.n_mt;
    const int nt = (logical / p.n_mt) % p.n_nt;
    const int g = logical / (p.n_mt * p.n_nt);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h2 = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    // loader: thread covers 16 B of rows r0 + 32 i, i = 0..3, column chunk kc
    const int lr = tid >> 3;
    const int kc = (tid & 7) * 8;
    const bf16* a_src[4];
    const bf16* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = mt * BM + lr + 32 * i;
        a_src[i] = (m < p.M) ? p.A + ((size_t)g * p.M + m) * p.K : nullptr;
        b_src[i] = row_src(p, g, nt * BN + lr + 32 * i);
    }
    bf16x8 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (a_src[i]) ra[i] = *reinterpret_cast<const bf16x8*>(a_src[i] + k0 + kc);
            else { for (int e = 0; e < 8; ++e) ra[i][e] = (bf16)0.f; }
            if (b_src[i]) rb[i] = *reinterpret_cast<const bf16x8*>(b_src[i] + k0 + kc);
            else { for (int e = 0; e < 8; ++e) rb[i][e] = (bf16)0.f; }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<bf16x8*>(&sA[buf][lr + 32 * i][kc]) = ra[i];
            *reinterpret_cast<bf16x8*>(&sB[buf][lr + 32 * i][kc]) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = p.K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                af[i] = *reinterpret_cast<const bf16x8*>(&sA[cur][64 * wm + 32 * i + l32][16 * kk + 8 * h2]);
                bfr[i] = *reinterpret_cast<const bf16x8*>(&sB[cur][64 * wn + 32 * i + l32][16 * kk + 8 * h2]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mma32(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < KT) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: stage the fp32 tile in LDS, then rows are processed by thread pairs
    float (*stage)[STAGE_STRIDE] = reinterpret_cast<float (*)[STAGE_STRIDE]>(smem);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * h2 + (e & 3);
                stage[r][64 * wn + 32 * j + l32] = acc[i][j][e];
            }
    __syncthreads();

    const int row = tid >> 1;            // tile row
    const int half = tid & 1;            // columns [64 half, 64 half + 64)
    const int m = mt * BM + row;
    const bool valid = m < p.M;
    const size_t grow = (size_t)g * p.M + m;      // global token row
    const float* srow = &stage[row][64 * half];

    if (EPI == EPI_RESIDUAL) {
        if (!valid) return;
        const int n0 = nt * BN + 64 * half;
        const bf16* xi = p.x_in + grow * p.N + n0;
        bf16* xo = p.x_out + grow * p.N + n0;
#pragma unroll
        for (int c = 0; c < 64; c += 8) {
            const bf16x8 xv = *reinterpret_cast<const bf16x8*>(xi + c);
            bf16x8 ov;
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] = (bf16)((float)xv[e] + srow[c + e]);
            *reinterpret_cast<bf16x8*>(xo + c) = ov;
        }
        return;
    }

    // EPI_LAYER_IN: tile nt is one q head, one k head, one v head, or the gate logits
    const int nq = p.Hqk, nk = 2 * p.Hqk, nv = 2 * p.Hqk + p.Hv;
    if (nt < nk) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 64; ++c) ss = fmaf(srow[c], srow[c], ss);
        ss += __shfl_xor(ss, 1, 64);
        const bool is_q = nt < nq;
        const float scale = (is_q ? p.q_scale : 1.f) / sqrtf(ss + 1e-6f);
        if (!valid) return;
        const int head = is_q ? nt : nt - nq;
        bf16* dst = (is_q ? p.q : p.k) + (grow * p.Hqk + head) * 128 + 64 * half;
#pragma unroll
        for (int c = 0; c < 64; c += 8) {
            bf16x8 ov;
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] = (bf16)(srow[c + e] * scale);
            *reinterpret_cast<bf16x8*>(dst + c) = ov;
        }
    } else if (nt < nv) {
        if (!valid) return;
        bf16* dst = p.v + (grow * p.Hv + (nt - nk)) * 128 + 64 * half;
#pragma unroll
        for (int c = 0; c < 64; c += 8) {
            bf16x8 ov;
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] = (bf16)srow[c + e];
            *reinterpret_cast<bf16x8*>(dst + c) = ov;
        }
    } else {
        if (!valid) return;
        // columns [0, Hv) are the gate logits z_a, [Hv, 2 Hv) the write logits z_b
        for (int c = 64 * half; c < 64 * half + 64 && c < 2 * p.Hv; ++c) {
            const float z = stage[row][c];
            if (c < p.Hv) p.g[grow * p.Hv + c] = -softplus_f(z);
            else p.beta[grow * p.Hv + (c - p.Hv)] = sigmoid_f(z);
        }
    }
}

unsigned grid_for(int tiles) { return (unsigned)(((tiles + 7) / 8) * 8); }

}  // namespace

hipError_t launch_rmsnorm(const bf16* x, bf16* y, const PtrTable& gain, int G, int n, int d, float eps,
                          hipStream_t stream) {
    const int rows = G * n;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                       x, y, gain, n, rows, d, eps);
    return hipGetLastError();
}

hipError_t launch_layer_in_gemm(const bf16* y, const PtrTable& w_qk, const PtrTable& w_v, const PtrTable& w_a,
                                const PtrTable& w_b, int G, int n, int d, int Hqk, int Hv,
                                bf16* q, bf16* k, bf16* v, float* g, float* beta, hipStream_t stream) {
    GemmParams p{};
    p.A = y; p.b0 = w_qk; p.b1 = w_v; p.b2 = w_a; p.b3 = w_b;
    p.n0 = 2 * Hqk * 128; p.n1 = Hv * 128; p.n2 = Hv; p.n3 = Hv;
    p.G = G; p.M = n; p.K = d; p.N = p.n0 + p.n1 + p.n2 + p.n3;
    p.n_mt = (n + BM - 1) / BM;
    p.n_nt = 2 * Hqk + Hv + 1;       // one tile per head, plus one for the 2 Hv gate columns
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.Hqk = Hqk; p.Hv = Hv;
    p.q_scale = 1.0f / sqrtf(128.0f);
    const int tiles = G * p.n_mt * p.n_nt;
    hipLaunchKernelGGL(gemm_tn_kernel<EPI_LAYER_IN>, dim3(grid_for(tiles)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_out_residual_gemm(const bf16* o, const PtrTable& w_o, int G, int n, int din, int d,
                                    const bf16* x_in, bf16* x_out, hipStream_t stream) {
    GemmParams p{};
    p.A = o; p.b0 = w_o; p.n0 = d;
    p.G = G; p.M = n; p.K = din; p.N = d;
    p.n_mt = (n + BM - 1) / BM;
    p.n_nt = d / BN;
    p.x_in = x_in; p.x_out = x_out;
    const int tiles = G * p.n_mt * p.n_nt;
    hipLaunchKernelGGL(gemm_tn_kernel<EPI_RESIDUAL>, dim3(grid_for(tiles)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tr
