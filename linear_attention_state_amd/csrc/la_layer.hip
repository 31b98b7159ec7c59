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

#include <cstddef>

namespace tr {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// --------------------------------------------------------------------------- RMSNorm
// One wave per row of d elements (d % 8 == 0), 8 per lane per 512-column pass.  A row of up
// to 512 * RMS_MAXP columns stays in registers between the sum of squares and the scaling, so
// x is read once; wider rows are read twice.
constexpr int RMS_MAXP = 8;
__device__ __forceinline__ bf16x8 rms_scale(const bf16x8& v, const bf16* gr, int c, float r) {
    bf16x8 o;
    if (gr) {
        const bf16x8 gv = *reinterpret_cast<const bf16x8*>(gr + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)v[i] * r * (float)gv[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)v[i] * r);
    }
    return o;
}

__global__ void __launch_bounds__(256)
rmsnorm_kernel(const bf16* __restrict__ x, bf16* __restrict__ y, PtrTable gain, int rows_per_group,
               int rows, int d, float eps)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const bf16* xr = x + (size_t)row * d;
    bf16* yr = y + (size_t)row * d;
    const bf16* gr = (const bf16*)gain.p[row / rows_per_group];
    float ss = 0.f;
    if (d <= 512 * RMS_MAXP) {
        bf16x8 v[RMS_MAXP];
#pragma unroll
        for (int p = 0; p < RMS_MAXP; ++p) {
            const int c = 512 * p + lane * 8;
            if (c < d) {
                v[p] = *reinterpret_cast<const bf16x8*>(xr + c);
#pragma unroll
                for (int i = 0; i < 8; ++i) { const float f = (float)v[p][i]; ss = fmaf(f, f, ss); }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
        const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
        for (int p = 0; p < RMS_MAXP; ++p) {
            const int c = 512 * p + lane * 8;
            if (c < d) *reinterpret_cast<bf16x8*>(yr + c) = rms_scale(v[p], gr, c, r);
        }
        return;
    }
    for (int c = lane * 8; c < d; c += 512) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) { const float f = (float)v[i]; ss = fmaf(f, f, ss); }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane * 8; c < d; c += 512)
        *reinterpret_cast<bf16x8*>(yr + c) = rms_scale(*reinterpret_cast<const bf16x8*>(xr + c), gr, c, r);
}

// --------------------------------------------------------------------------- GEMM
// 256x256 output tile per workgroup of 8 waves (2 x 4 waves of 128x64, 16x16x32 bf16 MFMA).
// The K loop streams 64-wide slices through a 2-slot LDS ring (64 KB per slot) with direct
// global-to-LDS loads, issued one slice ahead.  Each 128-byte LDS row holds its eight 16-byte
// chunks in a row-dependent order so that the operand reads hit distinct banks.
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES_N = 4, TM = 4, TN = 2;            // wave grid 2 x 4, wave tile 128 x 64
constexpr int FM = 2 * TM, FN = 2 * TN;               // 16x16 product tiles per wave: 8 x 4
constexpr int NTHREADS = 512;
constexpr int ROW_BYTES = BK * 2;                    // 128
constexpr int SLOT_BYTES = (BM + BN) * ROW_BYTES;    // A rows then B rows: 64 KB
constexpr int RING_BYTES = 2 * SLOT_BYTES;           // 128 KB
// Epilogue staging, one private region per wave (its 128 x 64 outputs): bf16 rows of 72 for
// the layer-in outputs, or fp32 rows of 68 for the residual (64 tokens per pass).
constexpr int STG_BF16_ROW = 64 + 8, STG_F32_ROW = 64 + 4;
constexpr int STG_WAVE_BYTES = 128 * STG_BF16_ROW * 2;                 // 18 KB
static_assert(64 * STG_F32_ROW * 4 <= STG_WAVE_BYTES, "fp32 half tile fits the wave's region");
constexpr int SSBUF_OFFSET = 8 * STG_WAVE_BYTES;                       // row sums of squares
constexpr int SMEM_BYTES = SSBUF_OFFSET + 8 * 4 * 32 * 4;              // 148 KB
static_assert(SMEM_BYTES >= RING_BYTES, "the staging reuses the ring");
constexpr int LOADS_PER_WAVE = SLOT_BYTES / 1024 / (NTHREADS / 64);   // 1 KB per load instruction
constexpr int GROUP_M = 8;                           // row tiles per band of the tile order

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

// Entry g of the pointer table at byte offset table_off of the kernel's argument block, read
// straight from the kernel-argument segment (GemmParams is the kernel's only argument, at
// offset 0).  Indexing the by-value argument with a variable would copy the whole block to
// scratch memory.
__device__ __forceinline__ const bf16* table_entry(size_t table_off, int g) {
    typedef const __attribute__((address_space(4))) unsigned char kchar;
    typedef const bf16* const __attribute__((address_space(4))) kptr;
    kchar* ka = (kchar*)__builtin_amdgcn_kernarg_segment_ptr();
    return *reinterpret_cast<kptr*>(ka + table_off + sizeof(void*) * (size_t)g);
}

__device__ __forceinline__ const bf16* row_src(const GemmParams& p, int g, int n) {
    if (n < p.n0) return table_entry(offsetof(GemmParams, b0), g) + (size_t)n * p.K;
    n -= p.n0;
    if (n < p.n1) return table_entry(offsetof(GemmParams, b1), g) + (size_t)n * p.K;
    n -= p.n1;
    if (n < p.n2) return table_entry(offsetof(GemmParams, b2), g) + (size_t)n * p.K;
    n -= p.n2;
    if (n < p.n3) return table_entry(offsetof(GemmParams, b3), g) + (size_t)n * p.K;
    return nullptr;
}

// Gates on the hardware exp2 / log2 (about 1 ulp each).  softplus(z) = max(z, 0) + log1p(t),
// t = e^{-|z|} in (0, 1]; log1p(t) is taken as log(u) with u = 1 + t rounded, corrected to first
// order for that rounding: log(1 + t) = log(u) - (u - 1 - t) / u + O(((u - 1 - t) / u)^2).
__device__ __forceinline__ float softplus_f(float z) {
    const float t = __expf(-fabsf(z));
    const float u = 1.f + t;
    return fmaxf(z, 0.f) + (__logf(u) - ((u - 1.f) - t) / u);
}
__device__ __forceinline__ float sigmoid_f(float z) {
    const float t = __expf(-fabsf(z));
    const float r = 1.f / (1.f + t);
    return z >= 0.f ? r : t * r;
}

// Physical position of logical 16-byte chunk c in slot row r is c ^ chunk_swz(r).  A 16-byte
// LDS read is checked for bank conflicts over 32 lanes at a time (512 bytes): the 32 lanes of
// a fragment read rows r..r+15 at two chunk positions, and with this order the 32 slots fall
// on 32 distinct 16-byte bank groups (so do 16- and 64-lane groups).  The row-XOR order
// (r ^ r >> 3) & 7 was conflict-free over 16 lanes only, and measured bank-conflict stalls on
// 17% of the cycles.
__device__ __forceinline__ int chunk_swz(int r) { return (r >> 1) & 7; }

typedef __attribute__((address_space(3))) void lds_void;

template <int EPI>
__global__ void __launch_bounds__(NTHREADS, 1)
gemm_tn_kernel(const GemmParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];

    // Tile order: blocks of consecutive logical tiles go to one XCD (blockIdx % 8 picks the
    // XCD), and inside a group the tiles run in bands of GROUP_M row tiles, so the tiles that
    // an XCD holds at once share a few A row tiles and weight tiles in its L2.
    const int per_group = p.n_mt * p.n_nt;
    const int n_tiles = p.G * per_group;
    const int per_xcd = (int)((gridDim.x + 7) / 8);
    const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (logical >= n_tiles) return;
    const int g = logical / per_group;
    const int t = logical % per_group;
    const int band = GROUP_M * p.n_nt;
    const int first_m = (t / band) * GROUP_M;
    const int rows_in_band = min(p.n_mt - first_m, GROUP_M);
    const int mt = first_m + (t % band) % rows_in_band;
    const int nt = (t % band) / rows_in_band;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    // Column blocks rotate with the row half (waves w and w + 4 share SIMD w % 4), so the two
    // live waves of a tile with one live column block (the gate columns) run on two SIMDs.
    const int wm = wave / WAVES_N, wn = (wave + wm) % WAVES_N;

    // Loader: load instruction i of a slot fills slot rows [8i, 8i + 8) (rows 0..255 are A,
    // 256..511 are B); lane l writes bytes [16l, 16l + 16) of its 1 KB, i.e. row l / 8, chunk
    // position l % 8.  Rows past M (or past the weight blocks) repeat a valid row: their
    // results are never stored.
    const bf16* src[LOADS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < LOADS_PER_WAVE; ++j) {
        const int r = (wave * LOADS_PER_WAVE + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ chunk_swz(r);
        if (r < BM) {
            const int m = min(mt * BM + r, p.M - 1);
            src[j] = p.A + ((size_t)g * p.M + m) * p.K + 8 * c;
        } else {
            const bf16* br = row_src(p, g, nt * BN + r - BM);
            src[j] = (br ? br : row_src(p, g, 0)) + 8 * c;
        }
    }
    auto issue = [&](int kt) {
        unsigned char* slot = smem + (kt & 1) * SLOT_BYTES + wave * LOADS_PER_WAVE * 1024;   // ring: [0, RING_BYTES)
#pragma unroll
        for (int j = 0; j < LOADS_PER_WAVE; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(src[j] + kt * BK), (lds_void*)(slot + 1024 * j), 16, 0, 0);
    };

    // acc[i][j] element e of lane (l16, g4) is output row (token) 128 wm + 16 i + l16 and
    // column 64 wn + 16 j + 4 g4 + e: the operands are swapped, so each lane holds one token
    // and runs of 4 consecutive output columns.
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

    // A wave whose 128 x 64 block lies wholly past the last row or column (the last row tile
    // of a group, the gate tile) still loads and meets the barriers but skips its products,
    // so the live waves of a ragged tile have their SIMDs to themselves.
    const bool live = mt * BM + wm * TM * 32 < p.M && nt * BN + wn * TN * 32 < p.N;
    const int KT = __builtin_amdgcn_readfirstlane(p.K / BK);
    issue(0);
    for (int kt = 0; kt < KT; ++kt) {
        // slice kt is in LDS once this wave's loads are done and every wave has passed here;
        // passing also means every wave is done reading the slot that slice kt + 1 overwrites
        asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kt + 1 < KT) issue(kt + 1);
        if (!live) continue;
        const unsigned char* slot = smem + (kt & 1) * SLOT_BYTES;
        // two 32-deep k-steps per slice; lane (l16, g4) reads row l16 of each 16-row fragment,
        // 16-byte chunk 4 ks + g4 (the 16 lanes of one chunk hit distinct banks)
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * TM * 32 + 16 * i + l16;
                af[i] = *reinterpret_cast<const bf16x8*>(slot + r * ROW_BYTES + 16 * ((4 * ks + g4) ^ chunk_swz(r)));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = BM + wn * TN * 32 + 16 * j + l16;
                bfr[j] = *reinterpret_cast<const bf16x8*>(slot + r * ROW_BYTES + 16 * ((4 * ks + g4) ^ chunk_swz(r)));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mma16(bfr[j], af[i], acc[i][j]);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- epilogue.  Each wave turns its 128 x 64 block around in a private LDS region, then
    // writes whole 128-byte row runs.
    unsigned char* stg = smem + wave * STG_WAVE_BYTES;
    const int rr = lane >> 3;                 // read-back: row within a group of 8, 16-byte chunk
    const int rc = (lane & 7) * 8;            // first of 8 columns
    if (EPI == EPI_RESIDUAL) {
        float* st = reinterpret_cast<float*>(stg);
        // rows [64 half, 64 half + 64) of the wave's block: product tiles 4 half .. 4 half + 3
        auto put = [&](int half) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    *reinterpret_cast<f32x4*>(st + (16 * ii + l16) * STG_F32_ROW + 16 * j + 4 * g4) = acc[4 * half + ii][j];
        };
        // x_in / x_out through buffer views of this wave's rows: rows past M read as zero and
        // their stores are dropped, so the row loop has no branches and the x_in loads can be
        // issued before the staging.
        const int n0 = nt * BN + wn * TN * 32 + rc;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row0 = mt * BM + wm * TM * 32 + 64 * half;
            const int rows = max(0, min(64, p.M - row0));
            const size_t base = ((size_t)g * p.M + row0) * p.N;
            const uint32_t bytes = (uint32_t)rows * (uint32_t)p.N * 2u;
            const __amdgpu_buffer_rsrc_t rin = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16*>(p.x_in + base), (short)0, (int)bytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(
                p.x_out + base, (short)0, (int)bytes, 0x00020000);
            bf16x8 xv[8];
            uint32_t off[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int row = 8 * t + rr;
                off[t] = n0 < p.N ? ((uint32_t)row * (uint32_t)p.N + (uint32_t)n0) * 2u : 0xFFFFFFF0u;
                xv[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rin, off[t], 0, 0));
            }
            put(half);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int row = 8 * t + rr;
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(st + row * STG_F32_ROW + rc);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(st + row * STG_F32_ROW + rc + 4);
                bf16x8 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ov[e] = (bf16)((float)xv[t][e] + v0[e]);
                    ov[4 + e] = (bf16)((float)xv[t][4 + e] + v1[e]);
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(f32x4, ov), rout, off[t], 0, 0);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next half lands
        }
        return;
    }

    // EPI_LAYER_IN.  128-column segments: q heads, k heads, v heads, then one segment of gate
    // logits ([0, Hv) z_a, [Hv, 2 Hv) z_b).  A segment spans waves wn and wn ^ 1; the row sums
    // of squares for the q / k L2 norms meet through LDS.
    // row sums of squares: the four lanes (l16, 0..3) of a token hold its 64 columns of this wave
    float ss[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) t = fmaf(acc[i][j][e], acc[i][j][e], t);
        t += __shfl_xor(t, 16, 64);
        ss[i] = t + __shfl_xor(t, 32, 64);
    }
    float* ssbuf = reinterpret_cast<float*>(smem + SSBUF_OFFSET);      // [waves][FM][16]
    if (g4 == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) ssbuf[((wm * WAVES_N + wn) * FM + i) * 16 + l16] = ss[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < FM; ++i) ss[i] += ssbuf[((wm * WAVES_N + (wn ^ 1)) * FM + i) * 16 + l16];

    const int seg = 2 * nt + (wn >> 1);
    const int nq = p.Hqk, nk = 2 * p.Hqk, nv = 2 * p.Hqk + p.Hv;
    if (seg < nv) {
        // q, k (L2-normalised rows, q also scaled) or v: bf16 through the wave's staging rows
        const bool is_qk = seg < nk, is_q = seg < nq;
        bf16* st = reinterpret_cast<bf16*>(stg);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float scale = is_qk ? (is_q ? p.q_scale : 1.f) / sqrtf(ss[i] + 1e-6f) : 1.f;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = (bf16)(acc[i][j][e] * scale);
                *reinterpret_cast<bf16x4*>(st + (16 * i + l16) * STG_BF16_ROW + 16 * j + 4 * g4) = ov;
            }
        }
        bf16* base = is_qk ? (is_q ? p.q : p.k) : p.v;
        const int heads = is_qk ? p.Hqk : p.Hv;
        const int head = is_qk ? (is_q ? seg : seg - nq) : seg - nk;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int row = 8 * t + rr;                          // 0..127
            const int m = mt * BM + wm * TM * 32 + row;
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(st + row * STG_BF16_ROW + rc);
            if (m < p.M)
                *reinterpret_cast<bf16x8*>(base + (((size_t)g * p.M + m) * heads + head) * 128 + (wn & 1) * 64 + rc) = x;
        }
    } else if (seg == nv) {
        // gate logits: few columns, written from registers
        const int cseg = (wn & 1) * TN * 32 + 4 * g4;
        auto gates = [&](const f32x4 (&a)[FN], int i) {
            const int m = mt * BM + wm * TM * 32 + 16 * i + l16;
            if (m >= p.M) return;
            const size_t grow = (size_t)g * p.M + m;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int cg0 = cseg + 16 * j;                      // four consecutive columns
                if (cg0 >= 2 * p.Hv) continue;
                if ((p.Hv & 3) == 0) {                              // all four in g or all in beta
                    const bool is_g = cg0 < p.Hv;
                    f32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float z = a[j][e];
                        r[e] = is_g ? -softplus_f(z) : sigmoid_f(z);
                    }
                    float* dst = is_g ? p.g + grow * p.Hv + cg0 : p.beta + grow * p.Hv + (cg0 - p.Hv);
                    *reinterpret_cast<f32x4*>(dst) = r;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int cg = cg0 + e;
                        const float z = a[j][e];
                        if (cg < p.Hv) p.g[grow * p.Hv + cg] = -softplus_f(z);
                        else if (cg < 2 * p.Hv) p.beta[grow * p.Hv + (cg - p.Hv)] = sigmoid_f(z);
                    }
                }
            }
        };
#pragma unroll
        for (int i = 0; i < FM; ++i) gates(acc[i], i);
    }
}

unsigned grid_for(int tiles) { return (unsigned)(((tiles + 7) / 8) * 8); }

template <int EPI>
hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
    const hipError_t e = ensure_dynamic_smem<gemm_tn_kernel<EPI>>(SMEM_BYTES);
    if (e != hipSuccess) return e;
    const int tiles = p.G * p.n_mt * p.n_nt;
    hipLaunchKernelGGL(gemm_tn_kernel<EPI>, dim3(grid_for(tiles)), dim3(NTHREADS), SMEM_BYTES, stream, p);
    return hipGetLastError();
}

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
    // 128-column segments: one per head, plus one for the 2 Hv gate columns; two per tile
    p.n_nt = (2 * Hqk + Hv + 1 + 1) / 2;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.Hqk = Hqk; p.Hv = Hv;
    p.q_scale = 1.0f / sqrtf(128.0f);
    return launch_gemm<EPI_LAYER_IN>(p, stream);
}

hipError_t launch_out_residual_gemm(const bf16* o, const PtrTable& w_o, int G, int n, int din, int d,
                                    const bf16* x_in, bf16* x_out, hipStream_t stream) {
    GemmParams p{};
    p.A = o; p.b0 = w_o; p.n0 = d;
    p.G = G; p.M = n; p.K = din; p.N = d;
    p.n_mt = (n + BM - 1) / BM;
    p.n_nt = (d + BN - 1) / BN;
    p.x_in = x_in; p.x_out = x_out;
    return launch_gemm<EPI_RESIDUAL>(p, stream);
}

}  // namespace tr
