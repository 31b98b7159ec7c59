/*
 * CPU oracle for the Gated DeltaNet (GDN) state replay -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load this
 * file's library.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制",
 * section 2.3, Eq. (1), with the layout remark that follows it):
 *
 *   S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   alpha_t = exp(g_t) in (0, 1],  S in R^{dv x dk}.
 *
 * The pages write T_i S_{i-1} with T_i = alpha_i (I - beta_i k_i k_i^T); with the
 * state stored as dv x dk the key-space operator has to act from the right, and
 * since T_i is symmetric this is the transpose of the printed form.  The pages
 * print no read-out; the reading taken here is the standard GDN one,
 * o_t = S_t (q_scale * q_t), with the state *after* token t's update.
 *
 * Evaluation: plain token loop in double precision.  The right product with the
 * operator is expanded as S - beta (S k) k^T, which is the same matrix; nothing is
 * chunked, blocked or reordered across tokens.
 *
 * Layouts (token-major, packed over sequences by cu_seqlens):
 *   q, k : [T, Hqk, dk]     v, o : [T, Hv, dv]     g, beta : [T, Hv]
 *   state_in, state_out : [B, Hv, dv, dk] (dk contiguous); state_in may be NULL
 *   (zero state, the replay start in section 2.2 step 2) and may alias state_out.
 *   Value head h reads query/key head h / (Hv / Hqk).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int oracle_gdn(const double* q, const double* k, const double* v,
               const double* g, const double* beta, const int32_t* cu_seqlens,
               int32_t B, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
               double q_scale, const double* state_in, double* state_out,
               double* o)
{
    if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk != 0)
        return 1;
    for (int32_t b = 0; b < B; ++b)
        if (cu_seqlens[b + 1] < cu_seqlens[b]) return 1;
    const int32_t per_qk = Hv / Hqk;
    const int64_t n_pairs = (int64_t)B * Hv;
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < n_pairs; ++p) {
        const int32_t b = (int32_t)(p / Hv);
        const int32_t h = (int32_t)(p % Hv);
        const int32_t j = h / per_qk;
        double* S = (double*)malloc(sizeof(double) * (size_t)dv * (size_t)dk);
        if (!S) {
#pragma omp atomic write
            err = 2;
            continue;
        }
        const size_t state_off = ((size_t)b * Hv + h) * (size_t)dv * dk;
        if (state_in)
            memcpy(S, state_in + state_off, sizeof(double) * (size_t)dv * dk);
        else
            memset(S, 0, sizeof(double) * (size_t)dv * dk);

        for (int64_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) {
            const double* kt = k + ((size_t)t * Hqk + j) * dk;
            const double* qt = q + ((size_t)t * Hqk + j) * dk;
            const double* vt = v + ((size_t)t * Hv + h) * dv;
            const double alpha = exp(g[(size_t)t * Hv + h]);
            const double bt = beta[(size_t)t * Hv + h];
            for (int32_t r = 0; r < dv; ++r) {
                double* row = S + (size_t)r * dk;
                double sk = 0.0;
                for (int32_t c = 0; c < dk; ++c) sk += row[c] * kt[c];
                /* row <- alpha*(row - beta*(row.k) k^T) + beta*v_r k^T */
                for (int32_t c = 0; c < dk; ++c)
                    row[c] = alpha * (row[c] - bt * sk * kt[c]) + bt * vt[r] * kt[c];
            }
            if (o) {
                double* ot = o + ((size_t)t * Hv + h) * dv;
                for (int32_t r = 0; r < dv; ++r) {
                    const double* row = S + (size_t)r * dk;
                    double acc = 0.0;
                    for (int32_t c = 0; c < dk; ++c) acc += row[c] * qt[c];
                    ot[r] = q_scale * acc;
                }
            }
        }
        memcpy(state_out + state_off, S, sizeof(double) * (size_t)dv * dk);
        free(S);
    }
    return err;
}

/* Number of threads OpenMP will use for the loop above (reported by the CPU baseline). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
