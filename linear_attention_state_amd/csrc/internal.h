// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tr {

// One tr_gdn_replay request after host-side validation.
struct GdnArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;   // device
    int32_t B, T, Hqk, Hv, dk, dv;
    float q_scale;
    const float* state_in;       // may be null (zero state)
    float* state_out;
    void* o;                     // may be null (state-only)
    int32_t max_len;             // longest sequence (host-computed)
};

// Chunked WY-form recurrence, bf16 operands, fp32 state (gdn_chunk_bf16.hip).
hipError_t launch_gdn_chunk_bf16(const GdnArgs& a, hipStream_t stream);
// Token-serial recurrence in fp32 for fp32 inputs (gdn_token_f32.hip).
hipError_t launch_gdn_token_f32(const GdnArgs& a, hipStream_t stream);

// Group path (la_layer.hip).
struct LayerInputsArgs {
    const void* x;               // [G, n, d] bf16
    const void* const* w_qk;     // device array of G pointers
    const void* const* w_v;
    const void* const* w_a;
    const void* const* w_b;
    const void* const* gain;     // entries may be null
    int32_t G, n, d, Hqk, Hv, dk, dv;
    float rms_eps;
    void* q; void* k; void* v; float* g; float* beta;
    void* y;                     // workspace: [G, n, d] bf16 normalised hidden
};
hipError_t launch_la_layer_inputs(const LayerInputsArgs& a, hipStream_t stream);

struct OutResArgs {
    const void* x_in;            // [G, n, d] bf16
    const void* o;               // [G*n, Hv*dv] bf16
    const void* const* w_o;      // device array of G pointers
    int32_t G, n, d, din;
    void* x_out;
};
hipError_t launch_la_output_residual(const OutResArgs& a, hipStream_t stream);

}  // namespace tr
