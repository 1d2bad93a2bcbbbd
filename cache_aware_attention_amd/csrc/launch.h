// launch.h -- internal interface between the host-side argument checks
// (abi.cpp) and the HIP translation units that own the kernels.  Plain C++
// types only, so abi.cpp builds without HIP headers.  Every launcher assumes
// its arguments were already validated and returns MAR_OK or MAR_E_LAUNCH.
#pragma once
#include <cstddef>
#include <cstdint>

#include "mar_cache_attn.h"

namespace marca {

int launch_cache_attn(const void* q_a, const void* k_a, const void* v_a,
                      const void* k_cache, const void* v_cache,
                      const int32_t* cached_idx, int ldc, void* out, float* lse,
                      int B, int H, int N, int A, int Nc, float scale, int dtype,
                      void* stream);

int launch_cache_attn_ragged(const void* q_a, const void* k_a, const void* v_a,
                             const void* k_cache, const void* v_cache, const int32_t* cached_idx,
                             int ldc, const int32_t* a_len, const int32_t* c_len, void* out,
                             float* lse, int B, int H, int N, int A, int Nc, float scale,
                             int dtype, void* stream);

int launch_cache_attn_update(const void* q_a, const void* k_a, const void* v_a, void* k_cache,
                             void* v_cache, const int32_t* cached_idx, int ldc,
                             const int32_t* active_idx, int ld_act, int32_t* err_count, void* out,
                             float* lse, int B, int H, int N, int A, int Nc, float scale,
                             int dtype, void* stream);
int launch_cache_attn_ragged_update(const void* q_a, const void* k_a, const void* v_a,
                                    void* k_cache, void* v_cache, const int32_t* cached_idx,
                                    int ldc, const int32_t* active_idx, int ld_act,
                                    const int32_t* a_len, const int32_t* c_len,
                                    int32_t* err_count, void* out, float* lse, int B, int H,
                                    int N, int A, int Nc, float scale, void* stream);

// Layer 2's full attention (A = N <= 320, no cached rows, bf16) that also
// writes the generating queries' per-head probability sums into partials.
int launch_cache_attn_scores(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* gen_idx, int ld_gen, int G, float* partials, int B,
                             int H, int N, float scale, void* stream);

int launch_kv_scatter(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int32_t* idx, int ld_idx, int32_t* err_count,
                      int B, int H, int N, int M, int row_bytes, void* stream);

int launch_refresh_topk(const void* q_gen, const void* k_full,
                        const int32_t* gp_idx, int ld_gp, int n_gp, int K, float scale,
                        float* scores, int32_t* active_idx, int ld_act,
                        int32_t* cached_idx, int ld_cached, int32_t* cached_len,
                        float* workspace, int B, int H, int G, int N, int dtype,
                        void* stream);

// The selection half of launch_refresh_topk, from per-head partials [B,H,N].
int launch_refresh_select(const float* partials, const int32_t* gp_idx, int ld_gp, int n_gp,
                          int K, float* scores, int32_t* active_idx, int ld_act,
                          int32_t* cached_idx, int ld_cached, int32_t* cached_len, int B, int H,
                          int G, int N, void* stream);

// The allocation-free top-K: the partial scores go to the library's own
// per-device array of kTopkScratchBytes (B*H*N floats must fit; checked by
// the caller).
constexpr size_t kTopkScratchBytes = MAR_REFRESH_TOPK_SCRATCH_BYTES;
int launch_refresh_topk_noalloc(const void* q_gen, const void* k_full,
                                const int32_t* gp_idx, int ld_gp, int n_gp, int K, float scale,
                                float* scores, int32_t* active_idx, int ld_act,
                                int32_t* cached_idx, int ld_cached, int32_t* cached_len,
                                int B, int H, int G, int N, int dtype, void* stream);

int launch_cos_gate(const void* x_cur, const void* x_cached, float tau, float eps,
                    float* cos_out, uint8_t* reuse_mask, int32_t* compute_idx,
                    int32_t* compute_len, int32_t* reuse_idx, int32_t* reuse_len, int B, int N,
                    int W, int dtype, void* stream);

int launch_cfg_residual(const float* cond, const float* uncond, float* residual,
                        float* uncond_out, float* guided_out, float cfg_scale, int mode,
                        int64_t n, void* stream);

}  // namespace marca
