// Host side of the C ABI declared in include/tailreplay.h: argument validation, error
// reporting, tail selection, and dispatch to the HIP kernels.  Every check runs before the
// first HIP call, so a rejected request enqueues nothing.
#include "tailreplay.h"

#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

tr_status fail(tr_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

tr_status ok() {
    g_last_error.clear();
    return TR_OK;
}

bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("TR_DEBUG_SYNC");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

tr_status finish_launch(hipError_t e, hipStream_t stream, const char* what) {
    if (e != hipSuccess) return fail(TR_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    if (debug_sync()) {
        e = hipStreamSynchronize(stream);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return fail(TR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    }
    return ok();
}

bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }

typedef __bf16 bf16;

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of tr_group_replay: the running hidden x, the normalised y, q, k, v, g, beta, o.
struct GroupLayout {
    size_t x, y, q, k, v, o, g, beta, total;
    GroupLayout(int32_t G, int32_t n, int32_t d, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv) {
        const size_t rows = (size_t)G * n;
        size_t off = 0;
        auto take = [&](size_t bytes) { const size_t at = off; off += align_up(bytes); return at; };
        x = take(rows * d * 2);
        y = take(rows * d * 2);
        q = take(rows * Hqk * dk * 2);
        k = take(rows * Hqk * dk * 2);
        v = take(rows * Hv * dv * 2);
        o = take(rows * Hv * dv * 2);
        g = take(rows * Hv * 4);
        beta = take(rows * Hv * 4);
        total = off;
    }
};

tr_status check_layer_dims(const char* fn, int32_t G, int32_t L, int32_t n, int32_t d, int32_t Hqk, int32_t Hv,
                           int32_t dk, int32_t dv, float eps) {
    if (G < 1 || L < 1 || n < 1) return fail(TR_ERR_INVALID_ARG, "%s: need G, L, n_tokens >= 1", fn);
    if (Hqk < 1 || Hv < 1 || Hv % Hqk != 0)
        return fail(TR_ERR_INVALID_ARG, "%s: need Hv a positive multiple of Hqk (Hqk=%d, Hv=%d)", fn, Hqk, Hv);
    if (dk != 128 || dv != 128) return fail(TR_ERR_UNSUPPORTED, "%s: the layer path supports dk = dv = 128", fn);
    if (d < 128 || d % 128 != 0) return fail(TR_ERR_UNSUPPORTED, "%s: d_model must be a multiple of 128", fn);
    if (Hv > 64) return fail(TR_ERR_UNSUPPORTED, "%s: Hv <= 64 supported", fn);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(TR_ERR_INVALID_ARG, "%s: rms_eps must be finite and >= 0", fn);
    if ((int64_t)G * n > INT32_MAX / 64) return fail(TR_ERR_INVALID_ARG, "%s: too many tokens", fn);
    return TR_OK;
}

tr_status check_weights(const char* fn, const tr_la_weights* w, bool need_o, int gi, int li) {
    if (!w->w_qk || !w->w_v || !w->w_a || !w->w_b || (need_o && !w->w_o))
        return fail(TR_ERR_INVALID_ARG, "%s: null weight pointer (group %d, layer %d)", fn, gi, li);
    return TR_OK;
}

// Projection GEMM for G blocks; weights of block g are wp[g * stride + offset].
hipError_t project(const void* y, const tr_la_weights* const* wp, int stride, int offset, int G, int n, int d,
                   int Hqk, int Hv, bf16* q, bf16* k, bf16* v, float* g, float* beta, hipStream_t s) {
    for (int g0 = 0; g0 < G; g0 += tr::kMaxGroupsPerLaunch) {
        const int gb = std::min(tr::kMaxGroupsPerLaunch, G - g0);
        tr::PtrTable wqk{}, wv{}, wa{}, wb{};
        for (int i = 0; i < gb; ++i) {
            const tr_la_weights* w = wp[(size_t)(g0 + i) * stride + offset];
            wqk.p[i] = w->w_qk; wv.p[i] = w->w_v; wa.p[i] = w->w_a; wb.p[i] = w->w_b;
        }
        const size_t r0 = (size_t)g0 * n;
        const hipError_t e = tr::launch_layer_in_gemm((const bf16*)y + r0 * d, wqk, wv, wa, wb, gb, n, d, Hqk, Hv,
                                                      q + r0 * Hqk * 128, k + r0 * Hqk * 128, v + r0 * Hv * 128,
                                                      g + r0 * Hv, beta + r0 * Hv, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// RMSNorm then projections for G blocks (y is scratch of [G, n, d] bf16).
hipError_t layer_inputs(const void* x, const tr_la_weights* const* wp, int stride, int offset, int G, int n, int d,
                        int Hqk, int Hv, float eps, bf16* y, bf16* q, bf16* k, bf16* v, float* g, float* beta,
                        hipStream_t s) {
    for (int g0 = 0; g0 < G; g0 += tr::kMaxGroupsPerLaunch) {
        const int gb = std::min(tr::kMaxGroupsPerLaunch, G - g0);
        tr::PtrTable gain{};
        for (int i = 0; i < gb; ++i) gain.p[i] = wp[(size_t)(g0 + i) * stride + offset]->rms_gain;
        const size_t r0 = (size_t)g0 * n * d;
        const hipError_t e = tr::launch_rmsnorm((const bf16*)x + r0, y + r0, gain, gb, n, d, eps, s);
        if (e != hipSuccess) return e;
    }
    return project(y, wp, stride, offset, G, n, d, Hqk, Hv, q, k, v, g, beta, s);
}

hipError_t output_residual(const void* x_in, const void* o, const tr_la_weights* const* wp, int stride, int offset,
                           int G, int n, int d, int din, void* x_out, hipStream_t s) {
    for (int g0 = 0; g0 < G; g0 += tr::kMaxGroupsPerLaunch) {
        const int gb = std::min(tr::kMaxGroupsPerLaunch, G - g0);
        tr::PtrTable wo{};
        for (int i = 0; i < gb; ++i) wo.p[i] = wp[(size_t)(g0 + i) * stride + offset]->w_o;
        const size_t r0 = (size_t)g0 * n;
        hipError_t e = tr::launch_out_residual_gemm((const bf16*)o + r0 * din, wo, gb, n, din, d,
                                                    (const bf16*)x_in + r0 * d, (bf16*)x_out + r0 * d, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// tr_group_replay's workspace, carved as GroupLayout says.
struct GroupBuffers {
    bf16 *x, *y, *q, *k, *v, *o;
    float *g, *beta;
    GroupBuffers(void* workspace, const GroupLayout& lay) {
        unsigned char* ws = (unsigned char*)workspace;
        x = (bf16*)(ws + lay.x); y = (bf16*)(ws + lay.y); q = (bf16*)(ws + lay.q); k = (bf16*)(ws + lay.k);
        v = (bf16*)(ws + lay.v); o = (bf16*)(ws + lay.o); g = (float*)(ws + lay.g); beta = (float*)(ws + lay.beta);
    }
};

// The LA layers of groups [g0, g1) on one stream: every layer from the zero state, the last one
// state-only.  Each group's rows of the workspace buffers are its own, so disjoint group ranges
// could run on different streams at once (measured: two halves side by side on two streams were
// slower than one stream, the projection products already fill the chip).
hipError_t group_chain(const void* h_tail, const tr_la_weights* const* wp, int32_t g0, int32_t g1, int32_t L,
                       int32_t n, int32_t d, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, float eps,
                       float* states_out, const GroupBuffers& buf, hipStream_t s) {
    const int32_t G = g1 - g0;
    const size_t r0 = (size_t)g0 * n;
    bf16* x = buf.x + r0 * d;
    bf16* y = buf.y + r0 * d;
    bf16* q = buf.q + r0 * Hqk * dk;
    bf16* k = buf.k + r0 * Hqk * dk;
    bf16* v = buf.v + r0 * Hv * dv;
    bf16* o = buf.o + r0 * Hv * dv;
    float* g = buf.g + r0 * Hv;
    float* beta = buf.beta + r0 * Hv;
    const tr_la_weights* const* w = wp + (size_t)g0 * L;
    const int64_t state_elems = (int64_t)Hv * dv * dk;
    const void* x_cur = (const bf16*)h_tail + r0 * d;
    for (int32_t li = 0; li < L; ++li) {
        const bool last = li == L - 1;
        // projections in front of the recurrence (stride L through the weight table)
        hipError_t e = layer_inputs(x_cur, w, L, li, G, n, d, Hqk, Hv, eps, y, q, k, v, g, beta, s);
        if (e != hipSuccess) return e;
        // the recurrence from the zero state; the last layer keeps its state only
        tr::GdnArgs a;
        a.state_identity = 0;
        a.log_scale_out = nullptr;
        a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
        a.cu_seqlens = nullptr; a.uniform_len = n;
        a.B = G; a.T = G * n; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.q_scale = 1.0f;
        a.state_in = nullptr; a.state_out = states_out + ((int64_t)g0 * L + li) * state_elems;
        a.state_bstride = (int64_t)L * state_elems;
        a.o = last ? nullptr : o; a.max_len = n;
        e = tr::launch_gdn_chunk_bf16(a, s);
        if (e != hipSuccess) return e;
        if (!last) {
            e = output_residual(x_cur, o, w, L, li, G, n, d, Hv * dv, x, s);
            if (e != hipSuccess) return e;
            x_cur = x;
        }
        if (debug_sync()) {
            e = hipStreamSynchronize(s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* tr_last_error(void) { return g_last_error.c_str(); }

const char* tr_version(void) { return "tailreplay 0.1 (gfx950)"; }

int64_t tr_tail_length(int64_t m, int32_t r_num, int32_t r_den) {
    if (m < 0) { fail(TR_ERR_INVALID_ARG, "tr_tail_length: m = %lld is negative", (long long)m); return -1; }
    if (r_den <= 0 || r_num <= 0 || r_num > r_den) {
        fail(TR_ERR_INVALID_ARG, "tr_tail_length: need 0 < r_num <= r_den (got %d/%d)", r_num, r_den);
        return -1;
    }
    // ceil(m * r_num / r_den) without overflow: m < 2^63, r_num <= r_den < 2^31
    const int64_t qm = m / r_den, rm = m % r_den;
    const int64_t k = qm * r_num + (rm * (int64_t)r_num + r_den - 1) / r_den;
    ok();
    return k;
}

tr_status tr_tail_seqlens(const int64_t* m_host, int32_t B, int32_t r_num, int32_t r_den,
                          int32_t* cu_seqlens_host, int64_t* tail_start_host) {
    if (!m_host || !cu_seqlens_host) return fail(TR_ERR_INVALID_ARG, "tr_tail_seqlens: null pointer");
    if (B < 0) return fail(TR_ERR_INVALID_ARG, "tr_tail_seqlens: B = %d is negative", B);
    int64_t total = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t k = tr_tail_length(m_host[b], r_num, r_den);
        if (k < 0) return fail(TR_ERR_INVALID_ARG, "tr_tail_seqlens: hit %d: %s", b, g_last_error.c_str());
        total += k;
        if (total > INT32_MAX) return fail(TR_ERR_INVALID_ARG, "tr_tail_seqlens: total tail tokens exceed INT32_MAX");
    }
    cu_seqlens_host[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t k = tr_tail_length(m_host[b], r_num, r_den);
        cu_seqlens_host[b + 1] = cu_seqlens_host[b] + (int32_t)k;
        if (tail_start_host) tail_start_host[b] = m_host[b] - k;
    }
    return ok();
}

}  // extern "C"

namespace {

// Shared argument checks of the varlen recurrence entry points; sets *max_len.
tr_status check_gdn(const char* fn, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                    int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, tr_dtype dt,
                    int32_t* max_len) {
    if (B < 1) return fail(TR_ERR_INVALID_ARG, "%s: B = %d, need B >= 1", fn, B);
    if (T < 0) return fail(TR_ERR_INVALID_ARG, "%s: T = %d is negative", fn, T);
    if (Hqk < 1 || Hv < 1) return fail(TR_ERR_INVALID_ARG, "%s: head counts must be >= 1 (Hqk=%d, Hv=%d)", fn, Hqk, Hv);
    if (Hv % Hqk != 0) return fail(TR_ERR_INVALID_ARG, "%s: Hv = %d is not a multiple of Hqk = %d", fn, Hv, Hqk);
    if (dt != TR_BF16 && dt != TR_F32) return fail(TR_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
    if (!supported_head_dim(dk) || !supported_head_dim(dv))
        return fail(TR_ERR_UNSUPPORTED, "%s: dk = %d, dv = %d; supported head dims are 64 and 128", fn, dk, dv);
    if ((int64_t)B * Hv > INT32_MAX) return fail(TR_ERR_INVALID_ARG, "%s: B * Hv too large", fn);
    if (!cu_seqlens_host || !cu_seqlens_dev) return fail(TR_ERR_INVALID_ARG, "%s: null cu_seqlens", fn);
    if (cu_seqlens_host[0] != 0) return fail(TR_ERR_INVALID_ARG, "%s: cu_seqlens[0] = %d, must be 0", fn, cu_seqlens_host[0]);
    int32_t ml = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t l = cu_seqlens_host[b + 1] - cu_seqlens_host[b];
        if (cu_seqlens_host[b + 1] < cu_seqlens_host[b])
            return fail(TR_ERR_INVALID_ARG, "%s: cu_seqlens decreases at %d", fn, b + 1);
        if (l > ml) ml = l;
    }
    if (cu_seqlens_host[B] != T)
        return fail(TR_ERR_INVALID_ARG, "%s: cu_seqlens[B] = %d but T = %d", fn, cu_seqlens_host[B], T);
    // the kernels address one sequence's rows with 32-bit byte offsets
    const int64_t esize = dt == TR_BF16 ? 2 : 4;
    if ((int64_t)ml * std::max((int64_t)Hqk * dk, (int64_t)Hv * dv) * esize > INT32_MAX)
        return fail(TR_ERR_INVALID_ARG, "%s: a sequence of %d tokens is too long for these head sizes", fn, ml);
    *max_len = ml;
    return TR_OK;
}

// Schedule of the bf16 recurrence (tr_gdn_set_schedule).  The split schedule is chosen
// automatically when the fused one would leave most of the chip idle: at most kSplitMaxSlices
// 32-column state slices in all, one round of the scan's workgroups (a pair of waves per
// slice, one workgroup per CU).  Measured at 1,639 tokens, dk = dv = 128 (fused / split, us):
// 16 heads 194 / 80, 64 heads 196 / 117, 128 heads 199 / 238.
std::atomic<int> g_schedule{TR_SCHEDULE_AUTO};
constexpr int64_t kSplitMaxSlices = 256;

bool use_split(int32_t B, int32_t Hv, int32_t dv, tr_dtype dt) {
    if (dt != TR_BF16) return false;
    const int s = g_schedule.load(std::memory_order_relaxed);
    if (s == TR_SCHEDULE_FUSED) return false;
    if (s == TR_SCHEDULE_SPLIT) return true;
    return (int64_t)B * Hv * (dv / 32) <= kSplitMaxSlices;
}

int64_t split_records_per_head(int32_t B, int32_t T) { return ((int64_t)T + 63) / 64 + B; }

size_t split_workspace_bytes(int32_t B, int32_t T, int32_t Hv, int32_t dk, int32_t dv) {
    return (size_t)Hv * (size_t)split_records_per_head(B, T) * tr::split_record_bytes(dk, dv);
}

hipError_t launch_gdn(const tr::GdnArgs& a, tr_dtype dt, hipStream_t s) {
    return (dt == TR_BF16) ? tr::launch_gdn_chunk_bf16(a, s) : tr::launch_gdn_token_f32(a, s);
}

// Segments of tr_gdn_transition.  The product of a span's operators is associative, so with
// few (sequence, head) pairs to run, each span is cut into segments of seg_len tokens that run
// side by side from I, and their products are multiplied in order afterwards.  The plan aims
// the segments at kTransitionWgs workgroups of 16 rows (three per CU on 256 CUs; four, as many
// as their LDS allows, cost one more product in the chain and measured no faster on a
// 1,639-token span of 16 heads) and depends only on the lengths, the head count and d, so a
// result does not change with the device.
constexpr int64_t kTransitionWgs = 768;
constexpr int64_t kTransitionMinSeg = 128;   // shorter segments cost more to multiply than to run
constexpr int64_t kTransitionMaxSegs = 16;   // the products are multiplied one after another
struct TransitionPlan {
    tr::Segments sg;
    size_t bytes = 0;
};
TransitionPlan transition_plan(const int32_t* cu, int32_t B, int32_t Hv, int32_t d, int32_t max_len) {
    TransitionPlan p;
    const int64_t per_seq = (int64_t)Hv * (d / tr::kTransitionRows);   // workgroups of one whole span
    if ((int64_t)B * per_seq * 2 > kTransitionWgs) return p;
    const int64_t segs = (kTransitionWgs + per_seq - 1) / per_seq;   // segments in all
    int64_t seg = std::max<int64_t>(((int64_t)cu[B] + segs - 1) / segs, kTransitionMinSeg);
    seg = std::max<int64_t>(seg, (max_len + kTransitionMaxSegs - 1) / kTransitionMaxSegs);
    const int64_t smax = (max_len + seg - 1) / seg;
    if (smax < 2) return p;
    p.sg.seg_len = (int32_t)seg;
    p.sg.seg_max = (int32_t)smax;
    const size_t mats = (size_t)B * smax * Hv;
    p.bytes = align_up(mats * d * d * sizeof(float)) + align_up(mats * sizeof(float));
    return p;
}

}  // namespace

extern "C" {

tr_status tr_gdn_set_schedule(tr_schedule schedule) {
    if (schedule != TR_SCHEDULE_AUTO && schedule != TR_SCHEDULE_FUSED && schedule != TR_SCHEDULE_SPLIT)
        return fail(TR_ERR_INVALID_ARG, "tr_gdn_set_schedule: unknown schedule %d", (int)schedule);
    g_schedule.store((int)schedule, std::memory_order_relaxed);
    return ok();
}

tr_schedule tr_gdn_get_schedule(void) { return (tr_schedule)g_schedule.load(std::memory_order_relaxed); }

size_t tr_gdn_replay_workspace_size(const int32_t* cu_seqlens_host, int32_t B, int32_t Hqk, int32_t Hv,
                                    int32_t dk, int32_t dv, tr_dtype dt) {
    static const char* fn = "tr_gdn_replay_workspace_size";
    if (!cu_seqlens_host || B < 1) { fail(TR_ERR_INVALID_ARG, "%s: need cu_seqlens_host and B >= 1", fn); return 0; }
    int32_t max_len = 0;
    // the device copy is not needed here: pass the host array for the null check
    if (check_gdn(fn, cu_seqlens_host, cu_seqlens_host, B, cu_seqlens_host[B], Hqk, Hv, dk, dv, dt, &max_len) != TR_OK)
        return 0;
    ok();
    return use_split(B, Hv, dv, dt) ? split_workspace_bytes(B, cu_seqlens_host[B], Hv, dk, dv) : 0;
}

}  // extern "C"

namespace {

// Device scratch of tr_gdn_replay_noalloc: the split schedule's records for requests up to
// kNoallocScratchBytes, in a file-scope device array that every GPU the library runs on holds
// until the process ends.  The host-side name is not a device address: its address on each
// device comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoallocScratchBytes = TR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

tr_status noalloc_scratch(const char* fn, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TR_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(TR_ERR_UNSUPPORTED, "%s: device %d beyond the 64 the library tracks", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(TR_ERR_HIP, "%s: hipGetSymbolAddress of the static scratch: %s", fn,
                        e != hipSuccess ? hipGetErrorString(e) : "null address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TR_OK;
}

// tr_gdn_replay and tr_gdn_replay_noalloc: with noalloc set, the split schedule's records go
// to the static scratch (workspace arguments unused).
tr_status gdn_replay_impl(const char* fn, const void* q, const void* k, const void* v,
                          const float* g, const float* beta,
                          const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                          int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                          tr_dtype dt, float q_scale,
                          const float* state_in, float* state_out, void* o,
                          void* workspace, size_t workspace_bytes, bool noalloc, void* stream) {
    int32_t max_len = 0;
    const tr_status st = check_gdn(fn, cu_seqlens_host, cu_seqlens_dev, B, T, Hqk, Hv, dk, dv, dt, &max_len);
    if (st != TR_OK) return st;
    if (!(q_scale > 0.f) || !std::isfinite(q_scale))
        return fail(TR_ERR_INVALID_ARG, "%s: q_scale must be finite and > 0", fn);
    if (!state_out) return fail(TR_ERR_INVALID_ARG, "%s: null state_out", fn);
    if (T > 0 && (!q || !k || !v || !g || !beta)) return fail(TR_ERR_INVALID_ARG, "%s: null input pointer", fn);
    if ((((uintptr_t)q | (uintptr_t)k) & 15) != 0)
        return fail(TR_ERR_INVALID_ARG, "%s: q and k must be 16-byte aligned (rows are read in 16-byte pieces)", fn);
    const bool split = use_split(B, Hv, dv, dt);
    const size_t need = split ? split_workspace_bytes(B, T, Hv, dk, dv) : 0;
    if (noalloc && need > kNoallocScratchBytes)
        return fail(TR_ERR_WORKSPACE, "%s: the split schedule needs %zu bytes of scratch for this request, more "
                    "than the %zu the library holds; use tr_gdn_replay with a workspace, or TR_SCHEDULE_FUSED "
                    "(no scratch)", fn, need, kNoallocScratchBytes);
    if (noalloc && need > 0) {
        const tr_status ss = noalloc_scratch(fn, &workspace);
        if (ss != TR_OK) return ss;
        workspace_bytes = kNoallocScratchBytes;
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(TR_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace ? workspace_bytes : (size_t)0, need);
    if (need > 0 && ((uintptr_t)workspace & 15) != 0)
        return fail(TR_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
    if (split && (int64_t)((max_len + 63) / 64) * (int64_t)tr::split_record_bytes(dk, dv) > INT32_MAX)
        return fail(TR_ERR_INVALID_ARG, "%s: a sequence of %d tokens is too long for the split schedule", fn, max_len);

    tr::GdnArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.cu_seqlens = cu_seqlens_dev;
    a.B = B; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.q_scale = q_scale;
    a.state_in = state_in; a.state_identity = 0; a.state_out = state_out; a.o = o; a.max_len = max_len;
    a.log_scale_out = nullptr;
    a.uniform_len = 0; a.state_bstride = (int64_t)Hv * dv * dk;
    hipStream_t s = (hipStream_t)stream;
    if (!split) {
        // Fused schedule: with unequal lengths, the longest sequences go first so that they do
        // not start in the last round of workgroups.
        if (dt == TR_BF16 && B > 1 && B <= tr::kMaxOrdered) {
            bool uniform = true;
            for (int32_t b = 1; b < B && uniform; ++b)
                uniform = cu_seqlens_host[b + 1] - cu_seqlens_host[b] == cu_seqlens_host[1] - cu_seqlens_host[0];
            if (!uniform) {
                int32_t idx[tr::kMaxOrdered];
                for (int32_t b = 0; b < B; ++b) idx[b] = b;
                std::stable_sort(idx, idx + B, [&](int32_t x, int32_t y) {
                    return cu_seqlens_host[x + 1] - cu_seqlens_host[x] > cu_seqlens_host[y + 1] - cu_seqlens_host[y];
                });
                tr::SeqOrder order{};
                for (int32_t r = 0; r < B; ++r) order.idx[r] = (uint16_t)idx[r];
                return finish_launch(tr::launch_gdn_chunk_bf16(a, s, &order), s, fn);
            }
        }
        return finish_launch(launch_gdn(a, dt, s), s, fn);
    }
    // split schedule: chunk-parallel prep into the workspace, then the state scan split along dv
    tr::SplitPlan plan;
    plan.ws = workspace;
    plan.rec_per_head = split_records_per_head(B, T);
    plan.cmax = (max_len + 63) / 64;
    hipError_t e = plan.cmax > 0 ? tr::launch_gdn_prep_bf16(a, plan, s) : hipSuccess;
    if (e == hipSuccess) e = tr::launch_gdn_scan_split_bf16(a, plan, s);
    return finish_launch(e, s, fn);
}

}  // namespace

extern "C" {

tr_status tr_gdn_replay(const void* q, const void* k, const void* v,
                        const float* g, const float* beta,
                        const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                        tr_dtype dt, float q_scale,
                        const float* state_in, float* state_out, void* o,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_replay_impl("tr_gdn_replay", q, k, v, g, beta, cu_seqlens_host, cu_seqlens_dev, B, T, Hqk, Hv, dk, dv,
                           dt, q_scale, state_in, state_out, o, workspace, workspace_bytes, false, stream);
}

tr_status tr_gdn_replay_noalloc(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                                int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                                tr_dtype dt, float q_scale,
                                const float* state_in, float* state_out, void* o, void* stream) {
    return gdn_replay_impl("tr_gdn_replay_noalloc", q, k, v, g, beta, cu_seqlens_host, cu_seqlens_dev, B, T, Hqk, Hv,
                           dk, dv, dt, q_scale, state_in, state_out, o, nullptr, 0, true, stream);
}

size_t tr_gdn_transition_workspace_size(const int32_t* cu_seqlens_host, int32_t B, int32_t Hqk, int32_t Hv,
                                        int32_t d, tr_dtype dt) {
    static const char* fn = "tr_gdn_transition_workspace_size";
    if (!cu_seqlens_host || B < 1) { fail(TR_ERR_INVALID_ARG, "%s: need cu_seqlens_host and B >= 1", fn); return 0; }
    int32_t max_len = 0;
    // the device copy is not needed here: pass the host array for the null check
    if (check_gdn(fn, cu_seqlens_host, cu_seqlens_host, B, cu_seqlens_host[B], Hqk, Hv, d, d, dt, &max_len) != TR_OK)
        return 0;
    ok();
    return transition_plan(cu_seqlens_host, B, Hv, d, max_len).bytes;
}

tr_status tr_gdn_transition(const void* k, const float* g, const float* beta,
                            const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                            int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t d,
                            tr_dtype dt, float* phi_out, float* log_scale_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
    static const char* fn = "tr_gdn_transition";
    int32_t max_len = 0;
    const tr_status st = check_gdn(fn, cu_seqlens_host, cu_seqlens_dev, B, T, Hqk, Hv, d, d, dt, &max_len);
    if (st != TR_OK) return st;
    if (!phi_out) return fail(TR_ERR_INVALID_ARG, "%s: null phi_out", fn);
    if (T > 0 && (!k || !g || !beta)) return fail(TR_ERR_INVALID_ARG, "%s: null input pointer", fn);
    if (((uintptr_t)k & 15) != 0)
        return fail(TR_ERR_INVALID_ARG, "%s: k must be 16-byte aligned (rows are read in 16-byte pieces)", fn);
    TransitionPlan plan = transition_plan(cu_seqlens_host, B, Hv, d, max_len);
    if (plan.bytes > 0) {
        if (!workspace || workspace_bytes < plan.bytes)
            return fail(TR_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace ? workspace_bytes : 0,
                        plan.bytes);
        if (((uintptr_t)workspace & 15) != 0) return fail(TR_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
        const size_t mats = (size_t)B * plan.sg.seg_max * Hv;
        plan.sg.phi = (float*)workspace;
        plan.sg.log = (float*)((unsigned char*)workspace + align_up(mats * d * d * sizeof(float)));
    }

    // The recurrence from S = I with zero values: S_m = I T_{a+1} ... T_m, in fp32 arithmetic
    // for either input type (a product of many operators keeps every rounding it meets).
    tr::GdnArgs a;
    a.q = nullptr; a.k = k; a.v = nullptr; a.g = g; a.beta = beta; a.cu_seqlens = cu_seqlens_dev;
    a.B = B; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.dk = d; a.dv = d; a.q_scale = 1.f;
    a.state_in = nullptr; a.state_identity = 1; a.state_out = phi_out; a.o = nullptr; a.max_len = max_len;
    a.log_scale_out = log_scale_out;
    a.uniform_len = 0; a.state_bstride = (int64_t)Hv * d * d;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = tr::launch_gdn_transition(a, dt == TR_BF16, plan.sg, s);
    return finish_launch(e, s, fn);
}

tr_status tr_state_compose(const float* S_c, const float* phi, const float* log_scale, const float* S_hat,
                           float* out, int32_t N, int32_t dv, int32_t dk, void* stream) {
    static const char* fn = "tr_state_compose";
    if (N < 1) return fail(TR_ERR_INVALID_ARG, "%s: N = %d, need N >= 1", fn, N);
    if (!supported_head_dim(dk) || !supported_head_dim(dv))
        return fail(TR_ERR_UNSUPPORTED, "%s: dk = %d, dv = %d; supported head dims are 64 and 128", fn, dk, dv);
    if (!S_c || !phi || !out) return fail(TR_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (out == S_c || out == phi) return fail(TR_ERR_INVALID_ARG, "%s: out may alias only S_hat", fn);
    if ((int64_t)N * (dv / 64) * (dk / 64) > INT32_MAX) return fail(TR_ERR_INVALID_ARG, "%s: N too large", fn);
    hipStream_t s = (hipStream_t)stream;
    return finish_launch(tr::launch_state_compose(S_c, phi, log_scale, S_hat, out, N, dv, dk, s), s, fn);
}

tr_status tr_gdn_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                        int32_t B, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, tr_dtype dt, float q_scale,
                        float* state, void* o, void* stream) {
    static const char* fn = "tr_gdn_decode";
    if (B < 1) return fail(TR_ERR_INVALID_ARG, "%s: B = %d, need B >= 1", fn, B);
    if (Hqk < 1 || Hv < 1) return fail(TR_ERR_INVALID_ARG, "%s: head counts must be >= 1 (Hqk=%d, Hv=%d)", fn, Hqk, Hv);
    if (Hv % Hqk != 0) return fail(TR_ERR_INVALID_ARG, "%s: Hv = %d is not a multiple of Hqk = %d", fn, Hv, Hqk);
    if (dt != TR_BF16 && dt != TR_F32) return fail(TR_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
    if (!supported_head_dim(dk) || !supported_head_dim(dv))
        return fail(TR_ERR_UNSUPPORTED, "%s: dk = %d, dv = %d; supported head dims are 64 and 128", fn, dk, dv);
    if (!(q_scale > 0.f) || !std::isfinite(q_scale))
        return fail(TR_ERR_INVALID_ARG, "%s: q_scale must be finite and > 0", fn);
    if ((int64_t)B * Hv > INT32_MAX) return fail(TR_ERR_INVALID_ARG, "%s: B * Hv too large", fn);
    if (!q || !k || !v || !g || !beta || !state) return fail(TR_ERR_INVALID_ARG, "%s: null pointer", fn);
    tr::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.B = B; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.is_bf16 = dt == TR_BF16; a.q_scale = q_scale;
    a.state = state; a.o = o;
    hipStream_t s = (hipStream_t)stream;
    return finish_launch(tr::launch_gdn_decode(a, s), s, fn);
}

size_t tr_la_layer_inputs_workspace_size(int32_t G, int32_t n_tokens, int32_t d_model) {
    if (G < 1 || n_tokens < 1 || d_model < 1) return 0;
    return align_up((size_t)G * n_tokens * d_model * 2);
}

tr_status tr_la_layer_inputs(const void* x, const tr_la_weights* const* w,
                             int32_t G, int32_t n_tokens, int32_t d_model,
                             int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, float rms_eps,
                             void* q, void* k, void* v, float* g_out, float* beta_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
    static const char* fn = "tr_la_layer_inputs";
    tr_status st = check_layer_dims(fn, G, 1, n_tokens, d_model, Hqk, Hv, dk, dv, rms_eps);
    if (st != TR_OK) return st;
    if (!x || !w || !q || !k || !v || !g_out || !beta_out) return fail(TR_ERR_INVALID_ARG, "%s: null pointer", fn);
    for (int32_t gi = 0; gi < G; ++gi) {
        if (!w[gi]) return fail(TR_ERR_INVALID_ARG, "%s: null weights for block %d", fn, gi);
        st = check_weights(fn, w[gi], false, gi, 0);
        if (st != TR_OK) return st;
    }
    const size_t need = tr_la_layer_inputs_workspace_size(G, n_tokens, d_model);
    if (!workspace || workspace_bytes < need)
        return fail(TR_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    return finish_launch(layer_inputs(x, w, 1, 0, G, n_tokens, d_model, Hqk, Hv, rms_eps, (bf16*)workspace,
                                      (bf16*)q, (bf16*)k, (bf16*)v, g_out, beta_out, s), s, fn);
}

tr_status tr_la_output_residual(const void* x_in, const void* o, const tr_la_weights* const* w,
                                int32_t G, int32_t n_tokens, int32_t d_model, int32_t Hv, int32_t dv,
                                void* x_out, void* stream) {
    static const char* fn = "tr_la_output_residual";
    if (G < 1 || n_tokens < 1) return fail(TR_ERR_INVALID_ARG, "%s: need G >= 1 and n_tokens >= 1", fn);
    if (d_model < 128 || d_model % 128 != 0) return fail(TR_ERR_UNSUPPORTED, "%s: d_model must be a multiple of 128", fn);
    if (Hv < 1 || dv < 1 || ((int64_t)Hv * dv) % 64 != 0)
        return fail(TR_ERR_UNSUPPORTED, "%s: Hv * dv must be a positive multiple of 64", fn);
    if (!x_in || !o || !w || !x_out) return fail(TR_ERR_INVALID_ARG, "%s: null pointer", fn);
    for (int32_t gi = 0; gi < G; ++gi)
        if (!w[gi] || !w[gi]->w_o) return fail(TR_ERR_INVALID_ARG, "%s: null w_o for block %d", fn, gi);
    hipStream_t s = (hipStream_t)stream;
    return finish_launch(output_residual(x_in, o, w, 1, 0, G, n_tokens, d_model, Hv * dv, x_out, s), s, fn);
}

tr_status tr_rmsnorm(const void* x, const void* const* gain, int32_t G, int32_t n_tokens, int32_t d_model,
                     float rms_eps, void* y, void* stream) {
    static const char* fn = "tr_rmsnorm";
    if (G < 1 || n_tokens < 1) return fail(TR_ERR_INVALID_ARG, "%s: need G >= 1 and n_tokens >= 1", fn);
    if (d_model < 128 || d_model % 128 != 0) return fail(TR_ERR_UNSUPPORTED, "%s: d_model must be a multiple of 128", fn);
    if (!(rms_eps >= 0.f) || !std::isfinite(rms_eps)) return fail(TR_ERR_INVALID_ARG, "%s: rms_eps must be finite and >= 0", fn);
    if (!x || !y || !gain) return fail(TR_ERR_INVALID_ARG, "%s: null pointer", fn);
    hipStream_t s = (hipStream_t)stream;
    for (int g0 = 0; g0 < G; g0 += tr::kMaxGroupsPerLaunch) {
        const int gb = std::min(tr::kMaxGroupsPerLaunch, G - g0);
        tr::PtrTable gt{};
        for (int i = 0; i < gb; ++i) gt.p[i] = gain[g0 + i];
        const size_t r0 = (size_t)g0 * n_tokens * d_model;
        const hipError_t e = tr::launch_rmsnorm((const bf16*)x + r0, (bf16*)y + r0, gt, gb, n_tokens, d_model,
                                                rms_eps, s);
        if (e != hipSuccess) return finish_launch(e, s, fn);
    }
    return finish_launch(hipSuccess, s, fn);
}

tr_status tr_la_project(const void* y, const tr_la_weights* const* w,
                        int32_t G, int32_t n_tokens, int32_t d_model,
                        int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                        void* q, void* k, void* v, float* g_out, float* beta_out, void* stream) {
    static const char* fn = "tr_la_project";
    tr_status st = check_layer_dims(fn, G, 1, n_tokens, d_model, Hqk, Hv, dk, dv, 0.f);
    if (st != TR_OK) return st;
    if (!y || !w || !q || !k || !v || !g_out || !beta_out) return fail(TR_ERR_INVALID_ARG, "%s: null pointer", fn);
    for (int32_t gi = 0; gi < G; ++gi) {
        if (!w[gi]) return fail(TR_ERR_INVALID_ARG, "%s: null weights for block %d", fn, gi);
        st = check_weights(fn, w[gi], false, gi, 0);
        if (st != TR_OK) return st;
    }
    hipStream_t s = (hipStream_t)stream;
    return finish_launch(project(y, w, 1, 0, G, n_tokens, d_model, Hqk, Hv, (bf16*)q, (bf16*)k, (bf16*)v,
                                 g_out, beta_out, s), s, fn);
}

size_t tr_group_replay_workspace_size(int32_t G, int32_t L, int32_t n_tokens, int32_t d_model,
                                      int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv) {
    if (G < 1 || L < 1 || n_tokens < 1 || d_model < 1 || Hqk < 1 || Hv < 1 || dk < 1 || dv < 1) return 0;
    return GroupLayout(G, n_tokens, d_model, Hqk, Hv, dk, dv).total;
}

tr_status tr_group_replay(const void* h_tail, const tr_la_weights* w,
                          int32_t G, int32_t L, int32_t n_tokens, int32_t d_model,
                          int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, float rms_eps,
                          float* states_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
    static const char* fn = "tr_group_replay";
    tr_status st = check_layer_dims(fn, G, L, n_tokens, d_model, Hqk, Hv, dk, dv, rms_eps);
    if (st != TR_OK) return st;
    if (!h_tail || !w || !states_out) return fail(TR_ERR_INVALID_ARG, "%s: null pointer", fn);
    for (int32_t gi = 0; gi < G; ++gi)
        for (int32_t li = 0; li < L; ++li) {
            st = check_weights(fn, &w[(size_t)gi * L + li], li < L - 1, gi, li);
            if (st != TR_OK) return st;
        }
    const GroupLayout lay(G, n_tokens, d_model, Hqk, Hv, dk, dv);
    if (!workspace || workspace_bytes < lay.total)
        return fail(TR_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, lay.total);

    hipStream_t s = (hipStream_t)stream;
    std::vector<const tr_la_weights*> wp((size_t)G * L);
    for (size_t i = 0; i < wp.size(); ++i) wp[i] = &w[i];
    const GroupBuffers buf(workspace, lay);
    const hipError_t e = group_chain(h_tail, wp.data(), 0, G, L, n_tokens, d_model, Hqk, Hv, dk, dv, rms_eps,
                                     states_out, buf, s);
    return finish_launch(e, s, fn);
}

}  // extern "C"
