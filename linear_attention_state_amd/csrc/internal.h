// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace tr {

// hipFuncSetAttribute(max dynamic shared memory) once per (kernel, device) in the process
// rather than on every launch.
template <auto KERN>
hipError_t ensure_dynamic_smem(size_t smem) {
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (done.load(std::memory_order_acquire) & (1ull << dev)) return hipSuccess;
    e = hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e == hipSuccess) done.fetch_or(1ull << dev, std::memory_order_acq_rel);
    return e;
}

// Compute units of the current device, queried once per device (0 if the query fails).
inline int device_cu_count() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups are dealt to the 8 XCDs round robin by index.  Item -> (pair, row block) such
// that the rb_count row blocks of one pair (a matrix, or a (sequence, head)) share an XCD and so
// its L2: the operands they all read are then fetched from memory once per pair.  A grid of
// xcd_grid(pairs, rb_count) = 8 rb_count ceil(pairs / 8) items covers every pair; items past
// the last pair have nothing to do.
__device__ __forceinline__ void xcd_item(int item, int rb_count, int& pair, int& rb) {
    const int xcd = item % 8, slot = item / 8;
    pair = (slot / rb_count) * 8 + xcd;
    rb = slot % rb_count;
}
inline long long xcd_grid(long long pairs, int rb_count) { return 8LL * rb_count * ((pairs + 7) / 8); }

// One tr_gdn_replay request after host-side validation.
struct GdnArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;   // device, or null: every sequence has uniform_len tokens
    int32_t uniform_len;
    int64_t state_bstride;       // elements between sequences in state_in / state_out
    int32_t B, T, Hqk, Hv, dk, dv;
    float q_scale;
    const float* state_in;       // may be null (zero state)
    int32_t state_identity;      // 1: start every (sequence, head) from I (dk == dv); state_in unused
    float* log_scale_out;        // transition only: non-null keeps the decay out of state_out
                                 // and writes sum(g) per (sequence, head) here, [B, Hv]
    float* state_out;
    void* o;                     // may be null (state-only)
    int32_t max_len;             // longest sequence (host-computed)
    // v may be null: every value vector is zero.  q may be null when o is null.
};

// Chunked WY-form recurrence, bf16 operands, fp32 state (gdn_chunk_bf16.hip).
// The fused kernel takes the sequences longest first when the host passes an order (at most
// kMaxOrdered sequences of unequal lengths): the longest replays then start in the first
// round of workgroups instead of wherever they fall in the packing.
constexpr int kMaxOrdered = 256;
struct SeqOrder {
    uint16_t idx[kMaxOrdered];   // idx[rank] = sequence
};
hipError_t launch_gdn_chunk_bf16(const GdnArgs& a, hipStream_t stream, const SeqOrder* order = nullptr);

// Split schedule for few heads: a chunk-parallel prep kernel writes one record per
// (value head, chunk) to the workspace, then the state scan runs with each state split
// along dv across workgroups (gdn_scan_split.hip).  A record holds MFMA operand fragments
// of the 32x32x16 bf16 layouts: fragment = 64 lanes x 16 bytes, lane l's 8 values in the
// order the operand takes them (row or column l % 32, contraction 16 s + 4 h + {0..3},
// 16 s + 8 + 4 h + {0..3}, h = l / 32).  In order, bytes:
//   -W          [row tile rt < 2][k-step s < dk/16]          (A operand of -W S^T)
//   Q           [row tile rt < 2][k-step s < dk/16]          (B operand of S Q^T)
//   K^T         [k-step s < 4][dk tile r < dk/32]            (A operand of the state update)
//   P hi, P lo  [(rt, s), s < 2 rt + 2: 6 fragments] each    (B operand of (P U')^T)
//   U0          [dv tile w < dv/32][rt < 2][lane][16 fp32]   (accumulator registers)
//   tables      [4][64] fp32: beta, q_scale e^gamma, e^{gamma_last - gamma}, e^gamma
// Records of sequence b sit at index floor(cu[b] / 64) + b + chunk within each head, which
// never collide and stay below ceil(T / 64) + B.
constexpr size_t split_wn_off() { return 0; }
constexpr size_t split_q_off(int dk) { return (size_t)dk * 128; }
constexpr size_t split_kt_off(int dk) { return split_q_off(dk) + (size_t)dk * 128; }
constexpr size_t split_ph_off(int dk) { return split_kt_off(dk) + (size_t)dk * 128; }
constexpr size_t split_pl_off(int dk) { return split_ph_off(dk) + 6 * 1024; }
constexpr size_t split_u0_off(int dk) { return split_pl_off(dk) + 6 * 1024; }
constexpr size_t split_tab_off(int dk, int dv) { return split_u0_off(dk) + (size_t)dv * 256; }
constexpr size_t split_record_bytes(int dk, int dv) { return split_tab_off(dk, dv) + 4 * 64 * 4; }
struct SplitPlan {
    void* ws;                    // records, [Hv][rec_per_head]
    int64_t rec_per_head;        // ceil(T / 64) + B
    int32_t cmax;                // most chunks in one sequence
};
hipError_t launch_gdn_prep_bf16(const GdnArgs& a, const SplitPlan& plan, hipStream_t stream);
hipError_t launch_gdn_scan_split_bf16(const GdnArgs& a, const SplitPlan& plan, hipStream_t stream);
// Token-serial recurrence in fp32 for fp32 inputs (gdn_token_f32.hip).
hipError_t launch_gdn_token_f32(const GdnArgs& a, hipStream_t stream);

// Transition product of a span from I with no values (gdn_transition.hip); a.state_out receives
// [B, Hv, d, d] and a.log_scale_out (if non-null) the gate sums, else the decay is applied.
// With seg_len > 0 every sequence of n tokens is cut into max(1, ceil(n / seg_len)) <= seg_max
// segments that run side by side, each from I; a sequence of several segments writes their
// products to phi[(b * seg_max + s) * Hv + h] ([d, d] each) and gate sums to
// log[(b * seg_max + s) * Hv + h], and a second kernel multiplies them in order.
constexpr int kTransitionRows = 16;   // rows of one head's product per segment workgroup
struct Segments {
    int32_t seg_len = 0;     // 0: one pass over every whole sequence
    int32_t seg_max = 1;
    float* phi = nullptr;
    float* log = nullptr;
};
hipError_t launch_gdn_transition(const GdnArgs& a, bool keys_bf16, const Segments& sg, hipStream_t stream);

// State algebra and single-token steps (state_ops.hip).
// out[n] = exp(log_scale[n]) S_c[n] Phi[n] (+ S_hat[n]) for n < N (log_scale may be null); S_c, S_hat, out [N, dv, dk], Phi [N, dk, dk], fp32.
hipError_t launch_state_compose(const float* S_c, const float* Phi, const float* log_scale, const float* S_hat,
                                float* out, int N, int dv, int dk, hipStream_t stream);
// One recurrence step per (sequence, value head) on a resident state, in place.
struct DecodeArgs {
    const void* q; const void* k; const void* v;   // [B, Hqk, dk], [B, Hqk, dk], [B, Hv, dv]
    const float* g; const float* beta;             // [B, Hv]
    int32_t B, Hqk, Hv, dk, dv;
    int32_t is_bf16;
    float q_scale;
    float* state;                                  // [B, Hv, dv, dk], updated in place
    void* o;                                       // [B, Hv, dv] or null
};
hipError_t launch_gdn_decode(const DecodeArgs& a, hipStream_t stream);

// Group path (la_layer.hip).  Per-group weight pointers travel in kernel arguments.
constexpr int kMaxGroupsPerLaunch = 16;
struct PtrTable {
    const void* p[kMaxGroupsPerLaunch];
};
hipError_t launch_rmsnorm(const __bf16* x, __bf16* y, const PtrTable& gain, int G, int n, int d, float eps,
                          hipStream_t stream);
hipError_t launch_layer_in_gemm(const __bf16* y, const PtrTable& w_qk, const PtrTable& w_v, const PtrTable& w_a,
                                const PtrTable& w_b, int G, int n, int d, int Hqk, int Hv,
                                __bf16* q, __bf16* k, __bf16* v, float* g, float* beta, hipStream_t stream);
hipError_t launch_out_residual_gemm(const __bf16* o, const PtrTable& w_o, int G, int n, int din, int d,
                                    const __bf16* x_in, __bf16* x_out, hipStream_t stream);

}  // namespace tr
