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
// Work decomposition: one workgroup per (sequence, value head).  Wave w owns value
// columns [32w, 32w + 32) of the state, kept in MFMA accumulator registers as S^T tiles
// (dk rows x 32 dv columns).  Chunk-local quantities (L, A, W, P) are shared through LDS.
// The accumulator layout of one product is fed straight back as the B operand of the
// next by permuting the contraction index consistently on both operands (see kperm()).
#include "internal.h"

namespace tr {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;                 // tokens per chunk
constexpr int RS_T = CH + 8;           // row stride (elements) of token-contiguous tiles
constexpr int RS_L = CH + 4;           // row stride of the fp32 L tile

__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// 32x32x16 MFMA layouts (lane l, half h = l / 32):
//   A operand: row l % 32, k = 8h + i;  B operand: column l % 32, k = 8h + i;
//   accumulator register j: row 8 (j / 4) + 4h + (j % 4), column l % 32.
// When an accumulator (rows = contraction index) is reused as a B operand, k-step s of
// 16 rows takes registers 8 (s % 2) .. 8 (s % 2) + 7 of row tile s / 2, which hold rows
// 16 s + {4h .. 4h+3} and 16 s + 8 + {4h .. 4h+3}.  kperm() reads the partner operand's
// row in that same order.
__device__ __forceinline__ int acc_row(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

__device__ __forceinline__ bf16x8 kperm(const bf16* row, int s, int h) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 16 * s + 4 * h);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 * s + 8 + 4 * h);
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = lo[i]; r[4 + i] = hi[i]; }
    return r;
}
__device__ __forceinline__ bf16x8 kstd(const bf16* row, int s, int h) {
    return *reinterpret_cast<const bf16x8*>(row + 16 * s + 8 * h);
}
// B operand for k-step s from an fp32 accumulator tile (registers 8 (s % 2) ..).
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

template <int DK, int DV>
struct Smem {
    bf16 K[CH][DK + 8];         // token rows
    bf16 Q[CH][DK + 8];
    bf16 KT[DK][RS_T];          // key columns: K^T, token contiguous
    bf16 VT[DV][RS_T];          // V^T
    union {
        float L[CH][RS_L];      // strictly lower L (fp32), live until the inverse is done
        bf16 W[CH][DK + 8];     // W rows, live from the W product to the end of the chunk
    } lw;
    bf16 Ab[CH][RS_T];          // blocks of A = (I + L)^{-1} as bf16 merge operands
    bf16 Nb[CH][RS_T];          // (A - I) diag(beta)
    bf16 Nbg[CH][RS_T];         // (A - I) diag(beta e^gamma)
    bf16 Ph[CH][RS_T];          // P, bf16 high part
    bf16 Pl[CH][RS_T];          // P, bf16 low part
    float gam[CH];
    float beta[CH];
};

template <int DK, int DV>
__global__ void __launch_bounds__(DV * 2, 1)
gdn_chunk_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                      const bf16* __restrict__ v, const float* __restrict__ g,
                      const float* __restrict__ beta, const int32_t* __restrict__ cu,
                      int B, int Hqk, int Hv, float q_scale, int uniform_len, long long state_bstride,
                      const float* state_in, float* state_out, bf16* __restrict__ o)
{
    constexpr int NW = DV / 32;            // waves; wave w owns dv columns [32w, 32w+32)
    constexpr int NT = NW * 64;            // threads
    constexpr int KT_TILES = DK / 32;      // S^T row tiles per wave
    constexpr int KSTEPS_D = DK / 16;      // k-steps over dk

    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<DK, DV>& sm = *reinterpret_cast<Smem<DK, DV>*>(smem_raw);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h2 = lane >> 5;              // half of the wave (32x32 layouts)
    const int l16 = lane & 15;
    const int g4 = lane >> 4;              // quarter of the wave (16x16 layouts)

    const int b = blockIdx.x / Hv;
    const int hv = blockIdx.x % Hv;
    const int hq = hv / (Hv / Hqk);
    const int bos = cu ? cu[b] : b * uniform_len;
    const int len = cu ? cu[b + 1] - bos : uniform_len;
    const int n_chunks = (len + CH - 1) / CH;
    const int col0 = 32 * wave;            // this wave's first dv column

    // ---- state: S^T tiles, tile r covers dk rows [32r, 32r+32), columns = own dv cols
    f32x16 St[KT_TILES];
    {
        const size_t base = (size_t)b * state_bstride + (size_t)hv * DV * DK;
#pragma unroll
        for (int r = 0; r < KT_TILES; ++r) {
            if (state_in) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int dk0 = 32 * r + 8 * q4 + 4 * h2;
                    const f32x4 x = *reinterpret_cast<const f32x4*>(state_in + base + (size_t)(col0 + l32) * DK + dk0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) St[r][4 * q4 + i] = x[i];
                }
            } else {
                St[r] = zero16();
            }
        }
    }

    // Nb / Nbg: blocks above the diagonal are never written below; clear them once.
    for (int i = tid; i < CH * RS_T; i += NT) {
        (&sm.Nb[0][0])[i] = (bf16)0.f;
        (&sm.Nbg[0][0])[i] = (bf16)0.f;
    }

    for (int c = 0; c < n_chunks; ++c) {
        const int t0 = bos + c * CH;
        const int nval = min(CH, len - c * CH);

        // ------------------------------------------------------------ load the chunk
        {
            constexpr int TPR_K = DK / 8;              // threads per key row (16 B each)
            constexpr int RPP_K = NT / TPR_K;          // rows per pass
            const int cc = (tid % TPR_K) * 8;
            for (int row = tid / TPR_K; row < CH; row += RPP_K) {
                bf16x8 kx, qx;
                if (row < nval) {
                    const size_t off = ((size_t)(t0 + row) * Hqk + hq) * DK + cc;
                    kx = *reinterpret_cast<const bf16x8*>(k + off);
                    qx = *reinterpret_cast<const bf16x8*>(q + off);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) { kx[i] = (bf16)0.f; qx[i] = (bf16)0.f; }
                }
                *reinterpret_cast<bf16x8*>(&sm.K[row][cc]) = kx;
                *reinterpret_cast<bf16x8*>(&sm.Q[row][cc]) = qx;
#pragma unroll
                for (int i = 0; i < 8; ++i) sm.KT[cc + i][row] = kx[i];
            }
            constexpr int TPR_V = DV / 8;
            constexpr int RPP_V = NT / TPR_V;
            const int cv = (tid % TPR_V) * 8;
            for (int row = tid / TPR_V; row < CH; row += RPP_V) {
                bf16x8 vx;
                if (row < nval) {
                    vx = *reinterpret_cast<const bf16x8*>(v + ((size_t)(t0 + row) * Hv + hv) * DV + cv);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) vx[i] = (bf16)0.f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) sm.VT[cv + i][row] = vx[i];
            }
            if (wave == 0) {
                // log-space gate cumsum over the chunk (padded tokens: g = 0, beta = 0)
                float gv = 0.f, bv = 0.f;
                if (lane < nval) {
                    gv = g[(size_t)(t0 + lane) * Hv + hv];
                    bv = beta[(size_t)(t0 + lane) * Hv + hv];
                }
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float up = __shfl_up(gv, off, 64);
                    if (lane >= off) gv += up;
                }
                sm.gam[lane] = gv;
                sm.beta[lane] = bv;
            }
        }
        __syncthreads();

        // ------------------------------------- K K^T -> L and Q K^T -> P (3 lower tiles each)
        // tiles: 0..2 = G(0,0), G(1,0), G(1,1); 3..5 = the same for Q K^T
        for (int tile = wave; tile < 6; tile += NW) {
            const bool is_p = tile >= 3;
            const int tt = is_p ? tile - 3 : tile;
            const int rb = tt == 0 ? 0 : 1;
            const int cb = tt == 2 ? 1 : 0;
            const bf16 (*X)[DK + 8] = is_p ? sm.Q : sm.K;
            f32x16 acc = zero16();
#pragma unroll
            for (int s = 0; s < KSTEPS_D; ++s)
                acc = mma32(kstd(&X[32 * rb + l32][0], s, h2), kstd(&sm.K[32 * cb + l32][0], s, h2), acc);
            const int ci = 32 * cb + l32;          // column index i (token)
            const float gi = sm.gam[ci];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rt = 32 * rb + acc_row(j, h2);     // row index t (token)
                const float dec = __expf(sm.gam[rt] - gi);
                if (!is_p) {
                    sm.lw.L[rt][ci] = (ci < rt) ? sm.beta[rt] * dec * acc[j] : 0.f;
                } else {
                    const float p = (ci <= rt) ? q_scale * dec * acc[j] : 0.f;
                    const bf16 ph = (bf16)p;
                    sm.Ph[rt][ci] = ph;
                    sm.Pl[rt][ci] = (bf16)(p - (float)ph);
                }
            }
        }
        __syncthreads();

        // ------------------------------------------------ A = (I + L)^{-1}, blocked by 16
        // diagonal blocks: forward substitution in fp32, one block per wave (column per lane)
        for (int blk = wave; blk < 4; blk += NW) {
            const int j = l16;
            const int base = 16 * blk;
            float a[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = (t == j) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < t; ++i) acc -= sm.lw.L[base + t][base + i] * a[i];
                a[t] = acc;
            }
            if (lane < 16) {
                const float bj = sm.beta[base + j];
                const float bgj = bj * __expf(sm.gam[base + j]);
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    sm.Ab[base + t][base + j] = (bf16)a[t];
                    const float n = (t > j) ? a[t] : 0.f;
                    sm.Nb[base + t][base + j] = (bf16)(n * bj);
                    sm.Nbg[base + t][base + j] = (bf16)(n * bgj);
                }
            }
        }
        __syncthreads();
        // off-diagonal blocks by distance: A_ij = -A_ii sum_{k=j}^{i-1} L_ik A_kj
        for (int dist = 1; dist < 4; ++dist) {
            const int n_blocks = 4 - dist;
            for (int bi = wave; bi < n_blocks; bi += NW) {
                const int i = bi + dist;
                const int j = bi;
                f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
                for (int kb = j; kb < i; ++kb) {
                    bf16x4 la, ab;
                    const float* lrow = &sm.lw.L[16 * i + l16][16 * kb + 4 * g4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        la[r] = (bf16)lrow[r];
                        ab[r] = sm.Ab[16 * kb + 4 * g4 + r][16 * j + l16];
                    }
                    t4 = mma16(la, ab, t4);
                }
                bf16x4 da, tb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    da[r] = sm.Ab[16 * i + l16][16 * i + 4 * g4 + r];
                    tb[r] = (bf16)(-t4[r]);
                }
                f32x4 res = {0.f, 0.f, 0.f, 0.f};
                res = mma16(da, tb, res);
                const int cj = 16 * j + l16;
                const float bj = sm.beta[cj];
                const float bgj = bj * __expf(sm.gam[cj]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rt = 16 * i + 4 * g4 + r;
                    sm.Ab[rt][cj] = (bf16)res[r];
                    sm.Nb[rt][cj] = (bf16)(res[r] * bj);
                    sm.Nbg[rt][cj] = (bf16)(res[r] * bgj);
                }
            }
            __syncthreads();
        }

        // ------------------------------------------- U0 (own dv columns) and W (dk tiles)
        f32x16 U[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x16 acc = zero16();
            const int ns = rt == 0 ? 2 : 4;          // A is lower triangular
            for (int s = 0; s < ns; ++s)
                acc = mma32(kstd(&sm.Nb[32 * rt + l32][0], s, h2), kstd(&sm.VT[col0 + l32][0], s, h2), acc);
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int t = 32 * rt + 8 * j4 + 4 * h2;
                const bf16x4 vv = *reinterpret_cast<const bf16x4*>(&sm.VT[col0 + l32][t]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[4 * j4 + r] += sm.beta[t + r] * (float)vv[r];
            }
            U[rt] = acc;
        }
        for (int ct = wave; ct < DK / 32; ct += NW) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x16 acc = zero16();
                const int ns = rt == 0 ? 2 : 4;
                for (int s = 0; s < ns; ++s)
                    acc = mma32(kstd(&sm.Nbg[32 * rt + l32][0], s, h2), kstd(&sm.KT[32 * ct + l32][0], s, h2), acc);
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int t = 32 * rt + 8 * j4 + 4 * h2;
                    const bf16x4 kk = *reinterpret_cast<const bf16x4*>(&sm.KT[32 * ct + l32][t]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float w = acc[4 * j4 + r] + sm.beta[t + r] * __expf(sm.gam[t + r]) * (float)kk[r];
                        sm.lw.W[t + r][32 * ct + l32] = (bf16)w;
                    }
                }
            }
        }
        __syncthreads();

        // ------------------------------------------------------ state-dependent part
        bf16x8 Sb[KSTEPS_D];
#pragma unroll
        for (int s = 0; s < KSTEPS_D; ++s) Sb[s] = acc_to_b(St[s >> 1], s);

        // U' = U0 - W S^T ;  Y = Q S^T
        f32x16 Y[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x16 x = zero16();
#pragma unroll
            for (int s = 0; s < KSTEPS_D; ++s) x = mma32(kperm(&sm.lw.W[32 * rt + l32][0], s, h2), Sb[s], x);
#pragma unroll
            for (int j = 0; j < 16; ++j) U[rt][j] -= x[j];
            if (o) {
                f32x16 y = zero16();
#pragma unroll
                for (int s = 0; s < KSTEPS_D; ++s) y = mma32(kperm(&sm.Q[32 * rt + l32][0], s, h2), Sb[s], y);
                Y[rt] = y;
            }
        }

        // O = diag(e^gamma) Y + P U'
        if (o) {
            bf16x8 uh[4], ul[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) acc_to_b_split(U[s >> 1], s, uh[s], ul[s]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x16 acc = zero16();
                const int ns = rt == 0 ? 2 : 4;
#pragma unroll
                for (int s = 0; s < ns; ++s) {
                    const bf16x8 ph = kperm(&sm.Ph[32 * rt + l32][0], s, h2);
                    const bf16x8 pl = kperm(&sm.Pl[32 * rt + l32][0], s, h2);
                    acc = mma32(ph, uh[s], acc);
                    acc = mma32(ph, ul[s], acc);
                    acc = mma32(pl, uh[s], acc);
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int t = 32 * rt + acc_row(j, h2);
                    if (t < nval) {
                        const float val = q_scale * __expf(sm.gam[t]) * Y[rt][j] + acc[j];
                        o[((size_t)(t0 + t) * Hv + hv) * DV + col0 + l32] = (bf16)val;
                    }
                }
            }
        }

        // S <- e^{gamma_n} S + U'^T diag(e^{gamma_n - gamma}) K
        {
            const float gl = sm.gam[CH - 1];
            bf16x8 dh[4], dl[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                f32x16 tmp;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int j = 8 * (s & 1) + i;
                    const int t = 32 * (s >> 1) + acc_row(j, h2);
                    tmp[j] = U[s >> 1][j] * __expf(gl - sm.gam[t]);
                }
                acc_to_b_split(tmp, s, dh[s], dl[s]);
            }
            const float decay = __expf(gl);
#pragma unroll
            for (int r = 0; r < KT_TILES; ++r) {
                f32x16 acc;
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[j] = St[r][j] * decay;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 a = kperm(&sm.KT[32 * r + l32][0], s, h2);
                    acc = mma32(a, dh[s], acc);
                    acc = mma32(a, dl[s], acc);
                }
                St[r] = acc;
            }
        }
        __syncthreads();
    }

    // ---- write the final state
    {
        const size_t base = (size_t)b * state_bstride + (size_t)hv * DV * DK;
#pragma unroll
        for (int r = 0; r < KT_TILES; ++r) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int dk0 = 32 * r + 8 * q4 + 4 * h2;
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = St[r][4 * q4 + i];
                *reinterpret_cast<f32x4*>(state_out + base + (size_t)(col0 + l32) * DK + dk0) = x;
            }
        }
    }
}

template <int DK, int DV>
hipError_t launch(const GdnArgs& a, hipStream_t stream) {
    auto kern = gdn_chunk_bf16_kernel<DK, DV>;
    const size_t smem = sizeof(Smem<DK, DV>);
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(a.B * a.Hv));
    const dim3 block(DV * 2);
    hipLaunchKernelGGL(kern, grid, block, smem, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta, a.cu_seqlens,
                       a.B, a.Hqk, a.Hv, a.q_scale, a.uniform_len, (long long)a.state_bstride,
                       a.state_in, a.state_out, (bf16*)a.o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_chunk_bf16(const GdnArgs& a, hipStream_t stream) {
    if (a.dk == 128 && a.dv == 128) return launch<128, 128>(a, stream);
    if (a.dk == 64 && a.dv == 64) return launch<64, 64>(a, stream);
    if (a.dk == 128 && a.dv == 64) return launch<128, 64>(a, stream);
    if (a.dk == 64 && a.dv == 128) return launch<64, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace tr
