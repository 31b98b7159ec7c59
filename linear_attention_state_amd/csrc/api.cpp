// Host side of the C ABI declared in include/tailreplay.h: argument validation, error
// reporting, tail selection, and dispatch to the HIP kernels.  Every check runs before the
// first HIP call, so a rejected request enqueues nothing.
#include "tailreplay.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

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

tr_status tr_gdn_replay(const void* q, const void* k, const void* v,
                        const float* g, const float* beta,
                        const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                        tr_dtype dt, float q_scale,
                        const float* state_in, float* state_out, void* o,
                        void* stream) {
    static const char* fn = "tr_gdn_replay";
    if (B < 1) return fail(TR_ERR_INVALID_ARG, "%s: B = %d, need B >= 1", fn, B);
    if (T < 0) return fail(TR_ERR_INVALID_ARG, "%s: T = %d is negative", fn, T);
    if (Hqk < 1 || Hv < 1) return fail(TR_ERR_INVALID_ARG, "%s: head counts must be >= 1 (Hqk=%d, Hv=%d)", fn, Hqk, Hv);
    if (Hv % Hqk != 0) return fail(TR_ERR_INVALID_ARG, "%s: Hv = %d is not a multiple of Hqk = %d", fn, Hv, Hqk);
    if (dt != TR_BF16 && dt != TR_F32) return fail(TR_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
    if (!supported_head_dim(dk) || !supported_head_dim(dv))
        return fail(TR_ERR_UNSUPPORTED, "%s: dk = %d, dv = %d; supported head dims are 64 and 128", fn, dk, dv);
    if (!(q_scale > 0.f) || !std::isfinite(q_scale))
        return fail(TR_ERR_INVALID_ARG, "%s: q_scale must be finite and > 0", fn);
    if ((int64_t)B * Hv > INT32_MAX) return fail(TR_ERR_INVALID_ARG, "%s: B * Hv too large", fn);
    if (!cu_seqlens_host || !cu_seqlens_dev) return fail(TR_ERR_INVALID_ARG, "%s: null cu_seqlens", fn);
    if (!state_out) return fail(TR_ERR_INVALID_ARG, "%s: null state_out", fn);
    if (T > 0 && (!q || !k || !v || !g || !beta)) return fail(TR_ERR_INVALID_ARG, "%s: null input pointer", fn);
    if (cu_seqlens_host[0] != 0) return fail(TR_ERR_INVALID_ARG, "%s: cu_seqlens[0] = %d, must be 0", fn, cu_seqlens_host[0]);
    int32_t max_len = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t l = cu_seqlens_host[b + 1] - cu_seqlens_host[b];
        if (cu_seqlens_host[b + 1] < cu_seqlens_host[b])
            return fail(TR_ERR_INVALID_ARG, "%s: cu_seqlens decreases at %d", fn, b + 1);
        if (l > max_len) max_len = l;
    }
    if (cu_seqlens_host[B] != T)
        return fail(TR_ERR_INVALID_ARG, "%s: cu_seqlens[B] = %d but T = %d", fn, cu_seqlens_host[B], T);

    tr::GdnArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.cu_seqlens = cu_seqlens_dev;
    a.B = B; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.q_scale = q_scale;
    a.state_in = state_in; a.state_out = state_out; a.o = o; a.max_len = max_len;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = (dt == TR_BF16) ? tr::launch_gdn_chunk_bf16(a, s) : tr::launch_gdn_token_f32(a, s);
    return finish_launch(e, s, fn);
}

size_t tr_la_layer_inputs_workspace_size(int32_t G, int32_t n_tokens, int32_t d_model) {
    if (G < 1 || n_tokens < 0 || d_model < 1) return 0;
    return (size_t)G * n_tokens * d_model * 2;
}

tr_status tr_la_layer_inputs(const void*, const tr_la_weights* const*, int32_t, int32_t, int32_t,
                             int32_t, int32_t, int32_t, int32_t, float, void*, void*, void*, float*, float*,
                             void*, size_t, void*) {
    return fail(TR_ERR_UNSUPPORTED, "tr_la_layer_inputs: not available in this build");
}

tr_status tr_la_output_residual(const void*, const void*, const tr_la_weights* const*, int32_t, int32_t,
                                int32_t, int32_t, int32_t, void*, void*) {
    return fail(TR_ERR_UNSUPPORTED, "tr_la_output_residual: not available in this build");
}

size_t tr_group_replay_workspace_size(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) {
    return 0;
}

tr_status tr_group_replay(const void*, const tr_la_weights*, int32_t, int32_t, int32_t, int32_t,
                          int32_t, int32_t, int32_t, int32_t, float, float*, void*, size_t, void*) {
    return fail(TR_ERR_UNSUPPORTED, "tr_group_replay: not available in this build");
}

}  // extern "C"
