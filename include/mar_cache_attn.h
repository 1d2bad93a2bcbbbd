/*
 * mar_cache_attn.h -- C ABI of libmarca, the MI355X (gfx950) library for the
 * per-step hot path of KV-cached masked-autoregressive (MAR) image decoding.
 *
 * The method is described on these pages (cited by title and section):
 *   [MARche]  "MARche: Fast Masked Autoregressive Image Generation with
 *             Cache-Aware Attention": the paper-notes page (Method: Overall
 *             Architecture, flowchart, Key Designs 1-3 with Eq. 1-2) and the
 *             Pith review page ("What carries the argument", Assumptions &
 *             free parameters, figure 3 caption).
 *   [LazyMAR] "LazyMAR: Accelerating Masked Autoregressive Models via Feature
 *             Caching": the paper-notes page (Key designs: token cache,
 *             condition cache, periodic cache-reuse-refresh).
 *
 * Conventions shared by every entry point
 *   - Return value: MAR_OK (0) or a negative mar_status.  No exception or
 *     abort crosses the ABI.  Argument checks happen on the host before any
 *     GPU work is queued; a failed check queues nothing.
 *   - Ownership: every buffer pointer is caller-owned device memory (the
 *     library never allocates, frees or retains buffers, and keeps no state
 *     between calls; mar_refresh_topk_noalloc's own device array is the one
 *     exception, described there).  Host-side arguments are marked (host).
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Calls are asynchronous on it; the caller synchronises.
 *   - Layouts: dense row-major; [B,H,N,D] means index ((b*H+h)*N+n)*D+d.
 *   - dtype: MAR_F32 (float) or MAR_BF16 (bfloat16 inputs, float accumulation,
 *     bfloat16 outputs rounded to nearest even).
 *   - Alignment: tensor base pointers must be 16-byte aligned (any torch or
 *     hipMalloc allocation is); MAR_E_RANGE otherwise.
 *   - Calls on one stream are ordered; calls that write the same buffer from
 *     different streams race.
 */
#ifndef MAR_CACHE_ATTN_H
#define MAR_CACHE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mar_status {
    MAR_OK = 0,
    MAR_E_NULL = -1,        /* a required pointer is NULL                        */
    MAR_E_SHAPE = -2,       /* a size is non-positive or sizes are inconsistent  */
    MAR_E_DTYPE = -3,       /* unknown dtype                                      */
    MAR_E_RANGE = -4,       /* an argument is outside its documented range        */
    MAR_E_WORKSPACE = -5,   /* workspace missing or smaller than required         */
    MAR_E_LAUNCH = -6,      /* the HIP runtime rejected a kernel launch           */
    MAR_E_UNSUPPORTED = -7  /* valid, but not implemented (e.g. head dim != 64)   */
} mar_status;

typedef enum mar_dtype { MAR_F32 = 0, MAR_BF16 = 1 } mar_dtype;

/* Static, never-NULL description of a status code. */
const char* mar_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int mar_version(void);

/*
 * Cache-aware attention  ([MARche] Key Design 2, Eq. 1-2; Overall Architecture).
 *
 * For every sequence b, head h and active query i < A:
 *   keys   = [k_a[b,h,0..A-1,:] ; k_cache[b,h,cached_idx[b,c],:] for c < Nc]
 *   values = the same rows of v_a / v_cache
 *   out[b,h,i,:] = softmax_j(scale * <q_a[b,h,i,:], key_j>) . values
 *   lse[b,h,i]   = natural log of sum_j exp(scale * <q_a[b,h,i,:], key_j>)
 * computed without forming the concatenation: the fresh active path and the
 * stored cached path are streamed as separate sources and folded into one
 * running (max, sum, weighted sum) state -- the safe online softmax merge.
 *
 *   q_a, k_a, v_a     [B,H,A,D]  fresh queries/keys/values of the active tokens
 *   k_cache, v_cache  [B,H,N,D]  stored keys/values of all N tokens (read only)
 *   cached_idx        [B,ldc] int32; the first Nc entries of row b are the
 *                     token positions of the cached set.  Precondition: they
 *                     lie in [0,N) and do not repeat an active token; an entry
 *                     outside [0,N) (e.g. the -1 padding mar_refresh_topk
 *                     writes) is skipped, never read out of bounds.
 *   out               [B,H,A,D]  same dtype as the inputs
 *   lse               [B,H,A] float, may be NULL
 *   scale             softmax temperature, positive and finite (usually 1/sqrt(D));
 *                     MAR_E_RANGE otherwise
 * Requires 1 <= A, 0 <= Nc, A + Nc <= N, ldc >= Nc, D == 64 (else
 * MAR_E_UNSUPPORTED).  Nc == 0 is plain attention over the active set (A == N
 * is the full-attention layer).  The output does not depend on the order of
 * the cached list.  cached_idx may be NULL when Nc == 0.
 */
int mar_cache_attn_fwd(const void* q_a, const void* k_a, const void* v_a,
                       const void* k_cache, const void* v_cache,
                       const int32_t* cached_idx, int ldc,
                       void* out, float* lse,
                       int B, int H, int N, int A, int Nc, int D,
                       float scale, int dtype, void* stream);

/*
 * Cache-aware attention with per-sequence set sizes  ([LazyMAR] Key designs,
 * token cache: each sequence recomputes only the tokens its gate selects, so
 * the active and cached sets differ in size from sequence to sequence;
 * [MARche] Key Design 2, Eq. 1-2, for the attention itself).
 *
 * As mar_cache_attn_fwd, with A and Nc read as capacities:
 *   a_len [B] device int32: sequence b has An = min(max(a_len[b], 0), A)
 *         active rows -- the first An rows of its q_a/k_a/v_a blocks;
 *   c_len [B] device int32: its first min(max(c_len[b], 0), Nc) entries of
 *         cached_idx are its cached set.
 * Rows of out (and lse) at or past An are not written.  A sequence with An = 0
 * computes nothing.  Requirements and errors as for mar_cache_attn_fwd,
 * except that A <= N and Nc <= N replace A + Nc <= N (the capacities are
 * maxima over sequences), plus a_len and c_len != NULL.
 */
int mar_cache_attn_fwd_ragged(const void* q_a, const void* k_a, const void* v_a,
                              const void* k_cache, const void* v_cache,
                              const int32_t* cached_idx, int ldc,
                              const int32_t* a_len, const int32_t* c_len,
                              void* out, float* lse,
                              int B, int H, int N, int A, int Nc, int D,
                              float scale, int dtype, void* stream);

/*
 * Cache-aware attention fused with the cache update of the active rows
 * ([MARche] Overall Architecture: attention over the active and cached sets
 * as one fused operator; abstract on the Pith page: only the recomputed
 * tokens' cache entries are updated).
 *
 * Computes exactly what mar_cache_attn_fwd computes and, in the same pass,
 * writes the fresh active rows into the caches:
 *   k_cache[b,h,active_idx[b*ld_act+i],:] = k_a[b,h,i,:]  (and V),  i < A
 * -- the partial update of mar_kv_scatter_refresh with idx = active_idx and
 * M = A -- from the registers that already hold those rows, so the rows are
 * read from memory once.
 *   active_idx  [B,ld_act] int32: token positions of the A active rows;
 *               NULL means the full refresh of a refresh step ([MARche] Key
 *               Design 3): every token is active (A == N, Nc == 0) and row i
 *               goes to cache row i -- full attention over all N tokens
 *               together with the cache rewrite of mar_kv_scatter_refresh
 *               with idx = NULL.
 *   err_count   device int32, may be NULL: +1 per (sequence, entry) outside
 *               [0,N); such entries are skipped.
 * Precondition: the active positions of a sequence are distinct and none of
 * them is among its first Nc cached entries (the cached set is the
 * complement of the active set), so no cache row is both read and written;
 * otherwise the value read for such a row is unspecified.  Requirements and
 * errors as for mar_cache_attn_fwd, plus ld_act >= A when active_idx is
 * given; active_idx == NULL with A != N or Nc != 0 returns MAR_E_NULL.
 */
int mar_cache_attn_fwd_update(const void* q_a, const void* k_a, const void* v_a,
                              void* k_cache, void* v_cache,
                              const int32_t* cached_idx, int ldc,
                              const int32_t* active_idx, int ld_act, int32_t* err_count,
                              void* out, float* lse,
                              int B, int H, int N, int A, int Nc, int D,
                              float scale, int dtype, void* stream);

/*
 * The per-sequence form of mar_cache_attn_fwd_update, for LazyMAR's token
 * cache ([LazyMAR] Key designs, token cache: each sequence recomputes the
 * tokens its gate selects, and their fresh K/V replace the cached ones;
 * [MARche] Key Design 2, Eq. 1-2, for the attention).
 *
 * Computes exactly what mar_cache_attn_fwd_ragged computes (a_len, c_len and
 * the capacities A, Nc as there) and, in the same pass, writes each
 * sequence's fresh active rows into the caches:
 *   k_cache[b,h,active_idx[b*ld_act+i],:] = k_a[b,h,i,:]  (and V),  i < An
 * where An = min(max(a_len[b], 0), A).  Entries of active_idx at or past a
 * sequence's An are not read (the gate's compute list, -1 padded, passes as
 * is); an entry before An outside [0,N) is skipped and, with err_count
 * non-NULL, counted once per sequence.
 * Precondition as for mar_cache_attn_fwd_update: a sequence's first An
 * active positions are distinct and none of them is among its first
 * min(c_len[b], Nc) cached entries.  Requires bf16 (MAR_E_UNSUPPORTED
 * otherwise), D == 64, 16 <= A (MAR_E_UNSUPPORTED), N <= 8192, ld_act >= A,
 * plus the requirements of mar_cache_attn_fwd_ragged; active_idx, a_len and
 * c_len must not be NULL (MAR_E_NULL).
 */
int mar_cache_attn_fwd_ragged_update(const void* q_a, const void* k_a, const void* v_a,
                                     void* k_cache, void* v_cache,
                                     const int32_t* cached_idx, int ldc,
                                     const int32_t* active_idx, int ld_act,
                                     const int32_t* a_len, const int32_t* c_len,
                                     int32_t* err_count, void* out, float* lse,
                                     int B, int H, int N, int A, int Nc, int D,
                                     float scale, int dtype, void* stream);

/*
 * Layer-2 full attention that also emits the refresh relevance partials
 * ([MARche] Key Design 1 and figure 3 on the Pith page: the refreshing tokens
 * are ranked by layer 2's attention from the generating tokens to every
 * token, averaged over heads; Overall Architecture: one fused operator).
 *
 * Computes what mar_cache_attn_fwd computes for a full-attention layer
 * (A == N, no cached rows; out and lse as there), and in the same pass
 *   partials[(b*H + h)*N + j] = sum over g < G of
 *       softmax_j(scale * <q[b,h,gen_idx[b*ld_gen + g],:], k[b,h,j,:]>)
 * -- the per-head sums of the generating queries' probabilities that
 * mar_refresh_select turns into scores and the active / cached partition, so
 * that the selection does not read K again.
 *   q, k, v     [B,H,N,D]   layer 2's queries, keys and values of all N tokens
 *   out         [B,H,N,D];  lse [B,H,N] float, may be NULL
 *   gen_idx     [B,ld_gen] int32: the G generating tokens' positions; an entry
 *               outside [0,N) contributes nothing
 *   partials    [B,H,N] float, partials_bytes >= B*H*N*4 (MAR_E_WORKSPACE)
 * Requires bf16 (MAR_E_UNSUPPORTED otherwise), D == 64, 64 < N <= 320,
 * 1 <= G <= 16, ld_gen >= G; scale positive and finite.  The probabilities
 * are fp32 and normalised by their exact fp32 sums.
 */
int mar_cache_attn_fwd_scores(const void* q, const void* k, const void* v,
                              void* out, float* lse,
                              const int32_t* gen_idx, int ld_gen, int G,
                              float* partials, size_t partials_bytes,
                              int B, int H, int N, int D, float scale, int dtype, void* stream);

/*
 * KV cache update  ([MARche] abstract on the Pith page: only the tokens that
 * need recomputation are updated; Key Design 3 and flowchart: every 3rd step
 * a periodic full refresh rewrites the whole cache).
 *
 *   idx != NULL  partial update: for m < M, with j = idx[b*ld_idx + m],
 *                k_cache[b,h,j,:] = k_new[b,h,m,:] and likewise for V.
 *                Entries outside [0,N) (including -1 padding) are skipped;
 *                each skipped (b,m) adds 1 to *err_count when err_count is
 *                not NULL (device int32, caller zeroes it).  Precondition:
 *                no position repeats within a row (the last writer would be
 *                unspecified).
 *   idx == NULL  full refresh: M must equal N; the caches become copies of
 *                k_new / v_new.
 *   k_cache, v_cache [B,H,N,D] (in/out);  k_new, v_new [B,H,M,D].
 * Rows are copied bit for bit.  Requires D*sizeof(dtype) to be a multiple of
 * 16 bytes, ld_idx >= M when idx != NULL.
 */
int mar_kv_scatter_refresh(void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new,
                           const int32_t* idx, int ld_idx, int32_t* err_count,
                           int B, int H, int N, int M, int D, int dtype, void* stream);

/* Bytes of device workspace mar_refresh_topk needs (B*H*N floats). */
size_t mar_refresh_topk_workspace(int B, int H, int N);

/*
 * Selective KV refresh: relevance scores, top-K refreshing tokens and the
 * active / cached partition  ([MARche] Key Design 1 and figure 3: layer-2
 * attention from the generating tokens to every token, averaged over heads,
 * ranked, top-K refresh; Overall Architecture: active = generating + previous
 * caching + refreshing tokens, cached = all others).
 *
 *   q_gen    [B,H,G,D]  layer-2 queries of the G generating tokens
 *   k_full   [B,H,N,D]  layer-2 keys of all N tokens
 *   gp_idx   [B,ld_gp] int32: the first n_gp entries of row b are the
 *            generating and previous-step tokens (never candidates; entries
 *            outside [0,N) are ignored).
 *   scores   [B,N] float out:
 *            scores[b,j] = 1/(H*G) * sum_h sum_g softmax_j(scale*<q,k_j>)
 *   active_idx [B,ld_act] int32 out: gp_idx row copied to [0,n_gp), then the
 *            K refreshing tokens in (score descending, index ascending)
 *            order; -1 where fewer than K tokens are eligible.
 *   cached_idx [B,ld_cached] int32 out: ascending positions that are neither
 *            in gp_idx nor refreshing, -1 padded to ld_cached.
 *   cached_len [B] int32 out: the number of such positions (if it exceeds
 *            ld_cached only ld_cached are written).
 *   workspace  >= mar_refresh_topk_workspace(B,H,N) bytes of device memory.
 * Ties between equal scores go to the lower token index.  Requires 1 <= G <= 64,
 * 0 <= K, n_gp + K <= N, ld_gp >= n_gp, ld_act >= n_gp + K,
 * ld_cached >= N - n_gp - K, N <= 4096, D == 64.
 * Deterministic: no floating-point atomics.
 */
int mar_refresh_topk(const void* q_gen, const void* k_full,
                     const int32_t* gp_idx, int ld_gp, int n_gp,
                     int K, float scale,
                     float* scores,
                     int32_t* active_idx, int ld_act,
                     int32_t* cached_idx, int ld_cached, int32_t* cached_len,
                     void* workspace, size_t ws_bytes,
                     int B, int H, int G, int N, int D, int dtype, void* stream);

/*
 * The selection half of mar_refresh_topk, from per-head partials such as
 * mar_cache_attn_fwd_scores writes ([MARche] Key Design 1: the K highest
 * head-averaged scores among the tokens outside G and P are refreshed;
 * Overall Architecture: active = generating + previous + refreshing tokens).
 *   partials [B,H,N] float: per (sequence, head, token) sums over the G
 *            generating queries of their softmax probabilities
 *   scores[b,j] = 1/(H*G) * sum_h partials[b,h,j]  (summed over h in order)
 * and gp_idx, K, active_idx, cached_idx, cached_len exactly as in
 * mar_refresh_topk (ties to the lower index; -1 where fewer than K tokens
 * are eligible).  Requires partials_bytes >= B*H*N*4 (MAR_E_WORKSPACE),
 * 1 <= G, 0 <= K, n_gp + K <= N, ld_gp >= n_gp, ld_act >= n_gp + K,
 * ld_cached >= N - n_gp - K, N <= 4096.
 */
int mar_refresh_select(const float* partials, size_t partials_bytes,
                       const int32_t* gp_idx, int ld_gp, int n_gp, int K,
                       float* scores,
                       int32_t* active_idx, int ld_act,
                       int32_t* cached_idx, int ld_cached, int32_t* cached_len,
                       int B, int H, int G, int N, void* stream);

/*
 * mar_refresh_topk without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, fixed serving loops,
 * harnesses that forbid allocation.  It calls no hipMalloc, hipFree or
 * allocating library routine.
 *
 * Arguments, outputs and errors as for mar_refresh_topk.  The per-(sequence,
 * head, token) partial scores go to a device array inside the library of
 * MAR_REFRESH_TOPK_SCRATCH_BYTES bytes, one per device, which each device the
 * call runs on holds until the process ends; its address is looked up on the
 * first call on a device (the device of `stream`, the current one for the
 * null stream).  B*H*N*4 bytes must fit in it, else MAR_E_WORKSPACE and
 * nothing is queued (8 MiB: e.g. 256 sequences x 20 heads x 320 tokens, or
 * 64 x 16 x 1088).  Every call writes all the partials it reads, so no state
 * carries over from one call to the next, but all calls on one device share
 * the array: calls that overlap on one device (two streams, two host threads)
 * race and give unspecified results.  MAR_E_LAUNCH if the runtime cannot give
 * the array's address.
 */
#define MAR_REFRESH_TOPK_SCRATCH_BYTES ((size_t)8 << 20)
int mar_refresh_topk_noalloc(const void* q_gen, const void* k_full,
                             const int32_t* gp_idx, int ld_gp, int n_gp,
                             int K, float scale,
                             float* scores,
                             int32_t* active_idx, int ld_act,
                             int32_t* cached_idx, int ld_cached, int32_t* cached_len,
                             int B, int H, int G, int N, int D, int dtype, void* stream);

/*
 * Cosine-similarity token gate  ([LazyMAR] Key designs, token cache: in the
 * layers past the first three, a token whose current feature is close in
 * cosine similarity to its cached feature reuses the cached computation).
 *
 *   x_cur, x_cached [B,N,W]   features of the same tokens now / when cached
 *   cos_out     [B,N] float   <x,y> / max(|x|*|y|, eps)
 *   reuse_mask  [B,N] uint8   1 iff cos_out >= tau (compared in float)
 *   compute_idx [B,N] int32   ascending positions with reuse 0, -1 padded
 *   compute_len [B]   int32   their count
 *   reuse_idx   [B,N] int32   (may be NULL) ascending positions with reuse 1,
 *                             -1 padded: the cached list of the ragged
 *                             attention over the recomputed tokens
 *   reuse_len   [B]   int32   (NULL iff reuse_idx is) their count, N - compute_len
 * Requires W*sizeof(dtype) to be a multiple of 16 bytes, N <= 65536.  Exactly
 * one of reuse_idx, reuse_len NULL: MAR_E_NULL.
 */
int mar_cos_gate(const void* x_cur, const void* x_cached, float tau, float eps,
                 float* cos_out, uint8_t* reuse_mask,
                 int32_t* compute_idx, int32_t* compute_len,
                 int32_t* reuse_idx, int32_t* reuse_len,
                 int B, int N, int W, int dtype, void* stream);

/*
 * Classifier-free-guidance residual cache  ([LazyMAR] Key designs, condition
 * cache: residual = cond - uncond is kept from a fully computed step and the
 * unconditional output of a reuse step is approximated as cond - residual).
 *
 *   mode MAR_CFG_STORE: residual[i] = cond[i] - uncond[i];  u = uncond
 *   mode MAR_CFG_REUSE: uncond_out[i] = cond[i] - residual[i]; u = uncond_out
 *   guided_out (may be NULL): u + cfg_scale * (cond - u), the usual guidance
 *            mix (not stated on the pages; provided for the caller's sampler).
 * float32 throughout, each operation rounded separately (no fused
 * multiply-add), so results are reproducible bit for bit.  Buffers [n_elems].
 */
enum { MAR_CFG_STORE = 0, MAR_CFG_REUSE = 1 };
int mar_cfg_residual(const float* cond, const float* uncond, float* residual,
                     float* uncond_out, float* guided_out, float cfg_scale,
                     int mode, int64_t n_elems, void* stream);

/*
 * Step schedule (host only)  ([MARche] flowchart and Key Design 3: full
 * refresh when step % period == 0, which includes step 0; Key Design 1: a
 * fixed active budget shared by generating, previous and refreshing tokens;
 * [LazyMAR] warm-up steps are computed in full).
 *
 * Step t generates the tokens order[o_t, o_t + counts[t]) of the generation
 * order, o_t = counts[0] + ... + counts[t-1]; the previous step's tokens are
 * order[o_{t-1}, o_t), so previous-then-generating is the single slice
 * order[prev_begin, gen_begin + n_gen).
 */
typedef struct mar_step_plan {
    int32_t step;
    int32_t refresh;     /* 1: every layer full attention + full cache rewrite */
    int32_t gen_begin;   /* o_t                                               */
    int32_t n_gen;       /* |G| = counts[t]                                   */
    int32_t prev_begin;  /* o_{t-1}                                           */
    int32_t n_prev;      /* |P| = counts[t-1] (0 at t = 0)                    */
    int32_t n_refresh;   /* K = clamp(budget - |G| - |P|, 0, n_tokens-|G|-|P|) */
    int32_t n_active;    /* |G|+|P|+K on cache-aware steps, n_tokens otherwise */
    int32_t n_cached;    /* n_tokens - n_active                               */
} mar_step_plan;

/* counts (host) [n_steps]; fills *out.  MAR_E_RANGE if step is out of range or
 * a count is negative, MAR_E_SHAPE if period < 1. */
int mar_plan_step(const int32_t* counts, int n_steps, int step, int n_tokens,
                  int budget, int period, int warmup, mar_step_plan* out);

/* Role of a (1-based) layer in a planned step, as a bit set:
 *   MAR_LAYER_CACHE  cache-aware attention over the active set (else full);
 *   MAR_LAYER_SELECT this layer's attention picks the refreshing tokens;
 *   MAR_LAYER_GATE   [LazyMAR] the cosine gate applies (layers past the
 *                    ungated ones, on reuse steps).
 * Negative mar_status on bad arguments. */
enum { MAR_LAYER_CACHE = 1, MAR_LAYER_SELECT = 2, MAR_LAYER_GATE = 4 };
int mar_layer_flags(const mar_step_plan* plan, int layer, int n_full_layers,
                    int select_layer, int ungated_layers);

#ifdef __cplusplus
}
#endif

#endif /* MAR_CACHE_ATTN_H */
