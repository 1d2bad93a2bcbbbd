// abi.cpp -- the extern "C" entry points of libmarca: argument checks on the
// host, then dispatch to the kernel launchers.  Contains no HIP code, so a
// rejected call never touches the GPU runtime.
#include <cstdint>

#include "launch.h"
#include "mar_cache_attn.h"

namespace {

constexpr int kHeadDim = 64;
constexpr int kMaxTopkTokens = 4096;
constexpr int kMaxGenQueries = 64;
constexpr int kMaxGateTokens = 65536;
constexpr int kMaxRaggedUpdateTokens = 8192;  // the MFMA attention kernels' limit

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int elem_bytes(int dtype) { return dtype == MAR_F32 ? 4 : (dtype == MAR_BF16 ? 2 : 0); }

}  // namespace

extern "C" const char* mar_status_string(int status) {
    switch (status) {
        case MAR_OK: return "ok";
        case MAR_E_NULL: return "a required pointer is NULL";
        case MAR_E_SHAPE: return "non-positive or inconsistent sizes";
        case MAR_E_DTYPE: return "unknown dtype";
        case MAR_E_RANGE: return "argument outside its documented range";
        case MAR_E_WORKSPACE: return "workspace missing or too small";
        case MAR_E_LAUNCH: return "kernel launch failed";
        case MAR_E_UNSUPPORTED: return "unsupported configuration";
        default: return "unknown status";
    }
}

extern "C" int mar_version(void) { return 100; }

// ragged: A and Nc are per-sequence capacities, each at most N (one
// sequence's active plus cached counts are its own business).
static int check_cache_attn(const void* q_a, const void* k_a, const void* v_a,
                            const void* k_cache, const void* v_cache, const int32_t* cached_idx,
                            int ldc, const void* out, int B, int H, int N, int A, int Nc, int D,
                            float scale, int dtype, bool ragged = false) {
    if (!q_a || !k_a || !v_a || !k_cache || !v_cache || !out) return MAR_E_NULL;
    if (Nc > 0 && !cached_idx) return MAR_E_NULL;
    if (elem_bytes(dtype) == 0) return MAR_E_DTYPE;
    if (B < 1 || H < 1 || N < 1 || A < 1 || D < 1 || Nc < 0) return MAR_E_SHAPE;
    if (ragged ? (A > N || Nc > N) : ((long long)A + Nc > N)) return MAR_E_SHAPE;
    if (Nc > 0 && ldc < Nc) return MAR_E_SHAPE;
    if (D != kHeadDim) return MAR_E_UNSUPPORTED;
    if (!(scale > 0.f) || scale > 3.0e38f) return MAR_E_RANGE;  // positive and finite
    if (!aligned16(q_a) || !aligned16(k_a) || !aligned16(v_a) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return MAR_E_RANGE;
    return MAR_OK;
}

extern "C" int mar_cache_attn_fwd(const void* q_a, const void* k_a, const void* v_a,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* cached_idx, int ldc, void* out, float* lse,
                                  int B, int H, int N, int A, int Nc, int D, float scale,
                                  int dtype, void* stream) {
    const int st = check_cache_attn(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, B, H,
                                    N, A, Nc, D, scale, dtype);
    if (st != MAR_OK) return st;
    return marca::launch_cache_attn(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse,
                                    B, H, N, A, Nc, scale, dtype, stream);
}

extern "C" int mar_cache_attn_fwd_ragged(const void* q_a, const void* k_a, const void* v_a,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* cached_idx, int ldc,
                                         const int32_t* a_len, const int32_t* c_len, void* out,
                                         float* lse, int B, int H, int N, int A, int Nc, int D,
                                         float scale, int dtype, void* stream) {
    if (!a_len || !c_len) return MAR_E_NULL;
    const int st = check_cache_attn(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, B, H,
                                    N, A, Nc, D, scale, dtype, true);
    if (st != MAR_OK) return st;
    return marca::launch_cache_attn_ragged(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc,
                                           a_len, c_len, out, lse, B, H, N, A, Nc, scale, dtype,
                                           stream);
}

extern "C" int mar_cache_attn_fwd_ragged_update(const void* q_a, const void* k_a,
                                                const void* v_a, void* k_cache, void* v_cache,
                                                const int32_t* cached_idx, int ldc,
                                                const int32_t* active_idx, int ld_act,
                                                const int32_t* a_len, const int32_t* c_len,
                                                int32_t* err_count, void* out, float* lse, int B,
                                                int H, int N, int A, int Nc, int D, float scale,
                                                int dtype, void* stream) {
    if (!active_idx || !a_len || !c_len) return MAR_E_NULL;
    const int st = check_cache_attn(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, B, H,
                                    N, A, Nc, D, scale, dtype, true);
    if (st != MAR_OK) return st;
    if (ld_act < A) return MAR_E_SHAPE;
    if (dtype != MAR_BF16 || A < 16 || N > kMaxRaggedUpdateTokens) return MAR_E_UNSUPPORTED;
    return marca::launch_cache_attn_ragged_update(q_a, k_a, v_a, k_cache, v_cache, cached_idx,
                                                  ldc, active_idx, ld_act, a_len, c_len,
                                                  err_count, out, lse, B, H, N, A, Nc, scale,
                                                  stream);
}

extern "C" int mar_cache_attn_fwd_update(const void* q_a, const void* k_a, const void* v_a,
                                         void* k_cache, void* v_cache,
                                         const int32_t* cached_idx, int ldc,
                                         const int32_t* active_idx, int ld_act,
                                         int32_t* err_count, void* out, float* lse, int B, int H,
                                         int N, int A, int Nc, int D, float scale, int dtype,
                                         void* stream) {
    const int st = check_cache_attn(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, B, H,
                                    N, A, Nc, D, scale, dtype);
    if (st != MAR_OK) return st;
    // No list: a full refresh, which needs every token active.
    if (!active_idx && !(A == N && Nc == 0)) return MAR_E_NULL;
    if (active_idx && ld_act < A) return MAR_E_SHAPE;
    return marca::launch_cache_attn_update(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc,
                                           active_idx, ld_act, err_count, out, lse, B, H, N, A,
                                           Nc, scale, dtype, stream);
}

extern "C" int mar_cache_attn_fwd_scores(const void* q, const void* k, const void* v, void* out,
                                         float* lse, const int32_t* gen_idx, int ld_gen, int G,
                                         float* partials, size_t partials_bytes, int B, int H,
                                         int N, int D, float scale, int dtype, void* stream) {
    const int st = check_cache_attn(q, k, v, k, v, nullptr, 0, out, B, H, N, N, 0, D, scale,
                                    dtype);
    if (st != MAR_OK) return st;
    if (!gen_idx || !partials) return MAR_E_NULL;
    if (G < 1 || ld_gen < G) return MAR_E_SHAPE;
    if (dtype != MAR_BF16 || N <= 64 || N > 320 || G > 16) return MAR_E_UNSUPPORTED;
    if (partials_bytes < (size_t)B * H * N * sizeof(float)) return MAR_E_WORKSPACE;
    return marca::launch_cache_attn_scores(q, k, v, out, lse, gen_idx, ld_gen, G, partials, B, H,
                                           N, scale, stream);
}

extern "C" int mar_kv_scatter_refresh(void* k_cache, void* v_cache, const void* k_new,
                                      const void* v_new, const int32_t* idx, int ld_idx,
                                      int32_t* err_count, int B, int H, int N, int M, int D,
                                      int dtype, void* stream) {
    if (!k_cache || !v_cache || !k_new || !v_new) return MAR_E_NULL;
    const int eb = elem_bytes(dtype);
    if (eb == 0) return MAR_E_DTYPE;
    if (B < 1 || H < 1 || N < 1 || M < 0 || D < 1) return MAR_E_SHAPE;
    if (idx == nullptr && M != N) return MAR_E_SHAPE;
    if (idx != nullptr && ld_idx < M) return MAR_E_SHAPE;
    if ((D * eb) % 16 != 0) return MAR_E_UNSUPPORTED;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
        return MAR_E_RANGE;
    return marca::launch_kv_scatter(k_cache, v_cache, k_new, v_new, idx, ld_idx, err_count, B, H,
                                    N, M, D * eb, stream);
}

extern "C" size_t mar_refresh_topk_workspace(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1) return 0;
    return (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

// Checks shared by both top-K entry points (everything but the workspace).
static int check_refresh_topk(const void* q_gen, const void* k_full, const int32_t* gp_idx,
                              int ld_gp, int n_gp, int K, float scale, const float* scores,
                              const int32_t* active_idx, int ld_act, const int32_t* cached_idx,
                              int ld_cached, const int32_t* cached_len, int B, int H, int G,
                              int N, int D, int dtype) {
    if (!q_gen || !k_full || !scores || !active_idx || !cached_idx || !cached_len)
        return MAR_E_NULL;
    if (n_gp > 0 && !gp_idx) return MAR_E_NULL;
    if (elem_bytes(dtype) == 0) return MAR_E_DTYPE;
    if (B < 1 || H < 1 || G < 1 || N < 1 || D < 1 || n_gp < 0) return MAR_E_SHAPE;
    if (K < 0 || (long long)n_gp + K > N) return MAR_E_RANGE;
    if (G > kMaxGenQueries) return MAR_E_UNSUPPORTED;
    if (n_gp > 0 && ld_gp < n_gp) return MAR_E_SHAPE;
    if (ld_act < n_gp + K || ld_act < 1) return MAR_E_SHAPE;
    if (ld_cached < N - n_gp - K || ld_cached < 1) return MAR_E_SHAPE;
    if (D != kHeadDim || N > kMaxTopkTokens) return MAR_E_UNSUPPORTED;
    if (!(scale == scale)) return MAR_E_RANGE;
    if (!aligned16(q_gen) || !aligned16(k_full)) return MAR_E_RANGE;
    return MAR_OK;
}

extern "C" int mar_refresh_topk(const void* q_gen, const void* k_full, const int32_t* gp_idx,
                                int ld_gp, int n_gp, int K, float scale, float* scores,
                                int32_t* active_idx, int ld_act, int32_t* cached_idx,
                                int ld_cached, int32_t* cached_len, void* workspace,
                                size_t ws_bytes, int B, int H, int G, int N, int D, int dtype,
                                void* stream) {
    const int st = check_refresh_topk(q_gen, k_full, gp_idx, ld_gp, n_gp, K, scale, scores,
                                      active_idx, ld_act, cached_idx, ld_cached, cached_len, B,
                                      H, G, N, D, dtype);
    if (st != MAR_OK) return st;
    if (!workspace) return MAR_E_WORKSPACE;
    if (ws_bytes < mar_refresh_topk_workspace(B, H, N)) return MAR_E_WORKSPACE;
    if (!aligned16(workspace)) return MAR_E_RANGE;
    return marca::launch_refresh_topk(q_gen, k_full, gp_idx, ld_gp, n_gp, K, scale, scores,
                                      active_idx, ld_act, cached_idx, ld_cached, cached_len,
                                      static_cast<float*>(workspace), B, H, G, N, dtype, stream);
}

extern "C" int mar_refresh_select(const float* partials, size_t partials_bytes,
                                  const int32_t* gp_idx, int ld_gp, int n_gp, int K,
                                  float* scores, int32_t* active_idx, int ld_act,
                                  int32_t* cached_idx, int ld_cached, int32_t* cached_len, int B,
                                  int H, int G, int N, void* stream) {
    if (!partials || !scores || !active_idx || !cached_idx || !cached_len) return MAR_E_NULL;
    if (n_gp > 0 && !gp_idx) return MAR_E_NULL;
    if (B < 1 || H < 1 || G < 1 || N < 1 || n_gp < 0) return MAR_E_SHAPE;
    if (K < 0 || (long long)n_gp + K > N) return MAR_E_RANGE;
    if (n_gp > 0 && ld_gp < n_gp) return MAR_E_SHAPE;
    if (ld_act < n_gp + K || ld_act < 1) return MAR_E_SHAPE;
    if (ld_cached < N - n_gp - K || ld_cached < 1) return MAR_E_SHAPE;
    if (N > kMaxTopkTokens) return MAR_E_UNSUPPORTED;
    if (partials_bytes < mar_refresh_topk_workspace(B, H, N)) return MAR_E_WORKSPACE;
    return marca::launch_refresh_select(partials, gp_idx, ld_gp, n_gp, K, scores, active_idx,
                                        ld_act, cached_idx, ld_cached, cached_len, B, H, G, N,
                                        stream);
}

extern "C" int mar_refresh_topk_noalloc(const void* q_gen, const void* k_full,
                                        const int32_t* gp_idx, int ld_gp, int n_gp, int K,
                                        float scale, float* scores, int32_t* active_idx,
                                        int ld_act, int32_t* cached_idx, int ld_cached,
                                        int32_t* cached_len, int B, int H, int G, int N, int D,
                                        int dtype, void* stream) {
    const int st = check_refresh_topk(q_gen, k_full, gp_idx, ld_gp, n_gp, K, scale, scores,
                                      active_idx, ld_act, cached_idx, ld_cached, cached_len, B,
                                      H, G, N, D, dtype);
    if (st != MAR_OK) return st;
    if (mar_refresh_topk_workspace(B, H, N) > marca::kTopkScratchBytes) return MAR_E_WORKSPACE;
    return marca::launch_refresh_topk_noalloc(q_gen, k_full, gp_idx, ld_gp, n_gp, K, scale,
                                              scores, active_idx, ld_act, cached_idx, ld_cached,
                                              cached_len, B, H, G, N, dtype, stream);
}

extern "C" int mar_cos_gate(const void* x_cur, const void* x_cached, float tau, float eps,
                            float* cos_out, uint8_t* reuse_mask, int32_t* compute_idx,
                            int32_t* compute_len, int32_t* reuse_idx, int32_t* reuse_len, int B,
                            int N, int W, int dtype, void* stream) {
    if (!x_cur || !x_cached || !cos_out || !reuse_mask || !compute_idx || !compute_len)
        return MAR_E_NULL;
    if ((reuse_idx == nullptr) != (reuse_len == nullptr)) return MAR_E_NULL;
    const int eb = elem_bytes(dtype);
    if (eb == 0) return MAR_E_DTYPE;
    if (B < 1 || N < 1 || W < 1) return MAR_E_SHAPE;
    if ((W * eb) % 16 != 0 || N > kMaxGateTokens) return MAR_E_UNSUPPORTED;
    if (!(tau == tau) || !(eps >= 0.f)) return MAR_E_RANGE;
    if (!aligned16(x_cur) || !aligned16(x_cached)) return MAR_E_RANGE;
    return marca::launch_cos_gate(x_cur, x_cached, tau, eps, cos_out, reuse_mask, compute_idx,
                                  compute_len, reuse_idx, reuse_len, B, N, W, dtype, stream);
}

extern "C" int mar_cfg_residual(const float* cond, const float* uncond, float* residual,
                                float* uncond_out, float* guided_out, float cfg_scale, int mode,
                                int64_t n_elems, void* stream) {
    if (mode != MAR_CFG_STORE && mode != MAR_CFG_REUSE) return MAR_E_RANGE;
    if (!cond || !residual) return MAR_E_NULL;
    if (mode == MAR_CFG_STORE && !uncond) return MAR_E_NULL;
    if (mode == MAR_CFG_REUSE && !uncond_out) return MAR_E_NULL;
    if (n_elems < 0) return MAR_E_SHAPE;
    if (!aligned16(cond) || !aligned16(residual) || (uncond && !aligned16(uncond)) ||
        (uncond_out && !aligned16(uncond_out)) || (guided_out && !aligned16(guided_out)))
        return MAR_E_RANGE;
    return marca::launch_cfg_residual(cond, uncond, residual, uncond_out, guided_out, cfg_scale,
                                      mode, n_elems, stream);
}
