/*
 * oracle.h -- plain, slow CPU reference for the KV-cached MAR decoding hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and it never calls it.
 *
 * Every floating-point result is computed in double precision from inputs that
 * the caller has widened exactly (bf16 and fp32 both widen to double without
 * rounding).  Loops are plain scalar loops; OpenMP splits only independent
 * (sequence, head) or sequence units and never changes an evaluation order.
 *
 * Sources (titles of the pages the method is described on):
 *   [MARche-notes]  "MARche: Fast Masked Autoregressive Image Generation with
 *                    Cache-Aware Attention" (paper-notes page), Method:
 *                    Overall Architecture, Key Designs 1-3, Eq. 1-2, flowchart.
 *   [MARche-review] the Pith review of the same paper: "What carries the
 *                    argument", Assumptions & free parameters.
 *   [LazyMAR-notes] "LazyMAR: Accelerating Masked Autoregressive Models via
 *                    Feature Caching" (paper-notes page), Key designs
 *                    (token cache, condition cache, cache-reuse-refresh).
 */
#ifndef MAR_ORACLE_H
#define MAR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of OpenMP threads the oracle will use (1 when built without OpenMP). */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

/*
 * Cache-aware attention, written as its plain definition
 * ([MARche-notes] Key Design 2, Eq. 1-2; [MARche-review] "What carries the
 * argument": the split into an active and a cached path, merged by the safe
 * online softmax, equals ordinary softmax attention over the union of the two
 * key/value sets).  So the oracle forms that union explicitly:
 *   keys   = [K_A rows 0..A-1 ; K_cache rows cached_idx[b][0..Nc-1]]
 *   values = the same rows of V_A / V_cache
 * and for each active query i computes
 *   s_j = scale * <q_i, key_j>,  p_j = exp(s_j - max s) / sum_j exp(s_j - max s),
 *   out_i = sum_j p_j value_j,   lse_i = max s + ln sum_j exp(s_j - max s).
 * Layouts (row-major): q_a,k_a,v_a [B,H,A,D]; k_cache,v_cache [B,H,N,D];
 * cached_idx [B,ldc] (first Nc entries used); out [B,H,A,D]; lse [B,H,A]
 * (may be NULL).  Returns 0, or -1 when a cached index is out of [0,N).
 */
int oracle_cache_attention(const double* q_a, const double* k_a, const double* v_a,
                           const double* k_cache, const double* v_cache,
                           const int32_t* cached_idx, int64_t ldc,
                           int64_t B, int64_t H, int64_t N, int64_t A, int64_t Nc,
                           int64_t D, double scale, double* out, double* lse);

/*
 * Layer-2 relevance scores ([MARche-notes] Key Design 1; figure 3 caption on
 * the review page): attention probabilities from every generating query to
 * every token of the sequence (full attention over all N tokens), averaged
 * over heads and over the generating queries:
 *   score[b][j] = 1/(H*G) * sum_h sum_g softmax_j(scale * <q[b,h,g], k[b,h,j]>).
 * q_gen [B,H,G,D]; k_full [B,H,N,D]; scores [B,N].
 */
void oracle_refresh_scores(const double* q_gen, const double* k_full,
                           int64_t B, int64_t H, int64_t G, int64_t N, int64_t D,
                           double scale, double* scores);

/*
 * Top-K refresh selection and the active / cached partition
 * ([MARche-notes] Overall Architecture and Key Design 1).
 * Tokens listed in gp_idx[b][0..n_gp-1] (this step's generating tokens and
 * the previous step's caching tokens) are not candidates.  The remaining
 * tokens are sorted by (score descending, index ascending) with qsort and the
 * first K become the refreshing tokens.
 * Outputs, per sequence b:
 *   active_idx[b][0..n_gp-1]      = gp_idx[b][0..n_gp-1] (copied)
 *   active_idx[b][n_gp..n_gp+K-1] = refreshing tokens in sorted order,
 *                                   -1 where fewer than K tokens are eligible
 *   cached_idx[b][0..]            = ascending indices that are neither in
 *                                   gp_idx nor refreshing, -1 padded to ld_cached
 *   cached_len[b]                 = number of such indices (may exceed
 *                                   ld_cached; then only ld_cached are written)
 * gp_idx entries outside [0,N) are ignored.
 */
void oracle_refresh_select(const double* scores, const int32_t* gp_idx, int64_t ld_gp,
                           int64_t n_gp, int64_t K, int64_t B, int64_t N,
                           int32_t* active_idx, int64_t ld_act,
                           int32_t* cached_idx, int64_t ld_cached, int32_t* cached_len);

/*
 * KV cache update ([MARche-review] abstract: only the tokens that need
 * recomputation are updated; [MARche-notes] Key Design 3 and flowchart: the
 * whole cache is rewritten on a periodic full refresh).  Works on raw bytes
 * of elem_bytes per element so that the result is comparable bit for bit.
 *   idx != NULL: cache[b][h][idx[b][m]][:] = new[b][h][m][:] for m < M;
 *                indices outside [0,N) are skipped and counted.
 *   idx == NULL: full refresh, M must equal N, cache = new.
 * Returns the number of skipped indices (counted once per (b,m)).
 */
int64_t oracle_kv_scatter(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          const int32_t* idx, int64_t B, int64_t H, int64_t N, int64_t M,
                          int64_t D, int64_t elem_bytes);

/*
 * Cosine-similarity token gate ([LazyMAR-notes] Key designs, token cache:
 * in layers past the first three, a token whose current feature is
 * cosine-similar to its cached feature reuses the cache).
 *   cos[b][j]   = <x_j, y_j> / max(|x_j| * |y_j|, eps)
 *   reuse[b][j] = cos[b][j] >= tau
 *   compute_idx[b][..] = ascending j with reuse == 0, -1 padded to N
 *   compute_len[b]     = their count
 * x, y [B,N,W]; cos [B,N]; reuse [B,N]; compute_idx [B,N]; compute_len [B].
 */
void oracle_cos_gate(const double* x, const double* y, int64_t B, int64_t N, int64_t W,
                     double tau, double eps, double* cos_out, uint8_t* reuse,
                     int32_t* compute_idx, int32_t* compute_len);

/*
 * The mask and compaction of oracle_cos_gate alone, from given cosines.  Used
 * to check a device's integer outputs against its own cosines (the decision is
 * then taken on the same values on both sides).
 */
void oracle_gate_from_cos(const double* cos_in, int64_t B, int64_t N, double tau,
                          uint8_t* reuse, int32_t* compute_idx, int32_t* compute_len);

/*
 * Classifier-free-guidance residual cache ([LazyMAR-notes] Key designs,
 * condition cache): keep residual = cond - uncond from a fully computed step,
 * and on a reuse step approximate uncond as cond - residual.
 *   mode 0 (store): residual = cond - uncond;   u = uncond
 *   mode 1 (reuse): uncond_out = cond - residual; u = uncond_out
 *   guided (optional, may be NULL): u + w * (cond - u)  (the usual guidance mix)
 * Each result is evaluated in double and rounded once to float.
 */
void oracle_cfg_residual(const float* cond, const float* uncond, float* residual,
                         float* uncond_out, float* guided, double w, int mode, int64_t n);

#ifdef __cplusplus
}
#endif

#endif /* MAR_ORACLE_H */
