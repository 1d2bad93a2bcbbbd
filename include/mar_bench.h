/*
 * mar_bench.h -- C ABI of libmarca_bench: measurement kernels that put the
 * cache-aware attention of libmarca in context.  They are not part of the
 * decoding path and the path never calls them.  Conventions (status codes,
 * dtypes, layouts, caller-owned device buffers, asynchronous calls on
 * `stream`) are those of mar_cache_attn.h.
 */
#ifndef MAR_BENCH_H
#define MAR_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "mar_cache_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The memory operations of mar_cache_attn_fwd's one-wave kernel at A <= 64
 * queries per (sequence, head) unit, without its arithmetic: the floor of
 * that access pattern on this chip.  Reads q_a, k_a, v_a [B,H,A,D], the first
 * Nc entries of each cached_idx row [B,ldc] and the cache rows they name in
 * k_cache, v_cache [B,H,N,D], exactly as the attention does (entries outside
 * [0,N) are not dereferenced).  write_out != 0: writes the A rows of each
 * unit of out [B,H,A,D] with meaningless values, as many bytes as the
 * attention's output; write_out == 0: reads only.
 * Requires bf16 (MAR_E_UNSUPPORTED otherwise), D == 64, 1 <= A <= 64,
 * A + Nc <= N, Nc <= 8192, ldc >= Nc.
 */
int mar_bench_attn_pattern(const void* q_a, const void* k_a, const void* v_a,
                           const void* k_cache, const void* v_cache,
                           const int32_t* cached_idx, int ldc, void* out, int write_out,
                           int B, int H, int N, int A, int Nc, int D, int dtype, void* stream);

/*
 * The concatenation that standard attention performs before attending over
 * the active and the cached tokens ([MARche] paper-notes page, Key Design 2;
 * Pith review page, figure 7: standard versus cache-aware attention).  For
 * T = A + Nc:
 *   k_cat[b,h,r,:] = k_a[b,h,r,:]                         r < A
 *   k_cat[b,h,r,:] = k_cache[b,h,cached_idx[b*ldc + r-A],:] A <= r < T
 * and likewise for V.  k_cat, v_cat [B,H,T,D]; k_a, v_a [B,H,A,D];
 * k_cache, v_cache [B,H,N,D].  An entry outside [0,N) leaves its row as it
 * was.  Rows are copied bit for bit.  Requires D*sizeof(dtype) to be a
 * multiple of 16 bytes, ldc >= Nc.
 */
int mar_bench_kv_concat(void* k_cat, void* v_cat, const void* k_a, const void* v_a,
                        const void* k_cache, const void* v_cache,
                        const int32_t* cached_idx, int ldc,
                        int B, int H, int N, int A, int Nc, int D, int dtype, void* stream);

/*
 * The two floors of the full-attention layer (mar_cache_attn_fwd with
 * A == N, Nc == 0, more than 64 tokens: [MARche] Key Design 3, layers 1-2
 * and every layer of a refresh step) and, with k_cache and v_cache given, of
 * the refresh-step layer (mar_cache_attn_fwd_update with no active list: the
 * same attention, every row of k and v also written to k_cache, v_cache
 * [B,H,N,D]), measured with the decoding path's own kernel in a measurement
 * mode:
 *   MAR_BENCH_FLOOR_ARITH   its arithmetic, LDS traffic and barriers alone:
 *                           every global load reads past its buffer (zeros,
 *                           no memory traffic) and nothing is stored;
 *   MAR_BENCH_FLOOR_MEMORY  its memory operations alone: it reads q, k, v
 *                           [B,H,N,D] and writes out [B,H,N,D] (meaningless
 *                           values) -- and the caches -- exactly as the layer
 *                           does, without the per-chunk math.
 * k_cache and v_cache are both NULL or both given (MAR_E_NULL otherwise).
 * Requires bf16 (MAR_E_UNSUPPORTED otherwise), D == 64, 64 < N <= 8192;
 * another mode is MAR_E_RANGE.
 */
enum { MAR_BENCH_FLOOR_ARITH = 1, MAR_BENCH_FLOOR_MEMORY = 2 };
int mar_bench_dense_floor(const void* q, const void* k, const void* v, void* k_cache,
                          void* v_cache, void* out, int mode, int B, int H, int N, int D,
                          int dtype, void* stream);

/*
 * The same two floors for the cache-aware layers whose active queries fill
 * several waves ([MARche] Key Design 2, Eq. 1-2, at the high-res length; the
 * [LazyMAR] notes page, token cache: each sequence's recomputed tokens),
 * measured with the decoding path's workgroup kernel in the modes above:
 *   - uniform counts, no update (active_idx, a_len, c_len all NULL): the
 *     layer of mar_cache_attn_fwd with A active rows and Nc cached entries,
 *     A + Nc <= N;
 *   - per-sequence counts with the cache update (active_idx, a_len, c_len
 *     all given): the layer of mar_cache_attn_fwd_ragged_update, with A and
 *     Nc as capacities (each <= N) and ld_act >= A.
 * Arguments as for those calls: q_a, k_a, v_a, out [B,H,A,D]; k_cache,
 * v_cache [B,H,N,D]; cached_idx [B,ldc]; active_idx [B,ld_act]; a_len, c_len
 * [B].  The arithmetic-only mode writes neither out nor the caches; the
 * memory-only mode writes out (meaningless values) and, with the update,
 * the caches as the layer does.  Requires bf16, D == 64, A > 64, Nc >= 1,
 * N <= 8192 and the staged lists within the workgroup's LDS
 * (MAR_E_UNSUPPORTED otherwise; a_len without c_len is MAR_E_NULL, and so
 * is a missing pointer).  The other combinations of the optional lists are
 * MAR_E_UNSUPPORTED; another mode is MAR_E_RANGE.
 */
int mar_bench_cached_floor(const void* q_a, const void* k_a, const void* v_a, void* k_cache,
                           void* v_cache, const int32_t* cached_idx, int ldc,
                           const int32_t* active_idx, int ld_act, const int32_t* a_len,
                           const int32_t* c_len, void* out, int mode, int B, int H, int N, int A,
                           int Nc, int D, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAR_BENCH_H */
