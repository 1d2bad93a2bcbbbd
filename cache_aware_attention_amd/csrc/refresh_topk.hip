// refresh_topk.hip -- selective KV refresh for KV-cached MAR decoding (gfx950).
//
// "MARche" paper-notes page, Key Design 1 (and figure 3 on the Pith review
// page): during the layer-2 full attention, the attention weights from every
// generating token to every token are averaged over heads into one relevance
// score per token; the K highest-scoring tokens (outside this step's
// generating tokens and the previous step's caching tokens) are recomputed.
// Overall Architecture: active = generating + caching + refreshing tokens,
// cached = every other token.
//
// Kernel 1 (one workgroup per (sequence, head)): two passes over the head's
// keys per group of up to 16 queries -- pass 1 builds each query's softmax
// max and normaliser with the running (max, sum) rule, pass 2 sums the
// normalised probabilities over the queries into a per-(b,h,token) partial.
// Kernel 2 (one workgroup per sequence): sums the partials over heads in a
// fixed order (no float atomics, deterministic), ranks the eligible tokens
// with a bitonic sort of 64-bit keys (orderable score << 32 | ~index, so equal
// scores put the lower index first), emits the refreshing tokens, and
// compacts the ascending cached complement with a block prefix sum.
#include "device_util.h"
#include "launch.h"

namespace marca {
namespace {

constexpr int kD = 64;
constexpr int kQG = 16;  // queries per pass group
constexpr int kThreads = 256;

__device__ __forceinline__ void load_row(const float* p, float (&x)[kD]) {
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 a = reinterpret_cast<const float4*>(p)[c];
        x[4 * c] = a.x; x[4 * c + 1] = a.y; x[4 * c + 2] = a.z; x[4 * c + 3] = a.w;
    }
}
__device__ __forceinline__ void load_row(const uint16_t* p, float (&x)[kD]) {
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[c];
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
            x[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
}
__device__ __forceinline__ float load1(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load1(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

// Merge two running softmax states (max m, sum l) in base 2.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float a = (m == -INFINITY) ? 0.f : l * exp2f(m - M);
    const float c = (m2 == -INFINITY) ? 0.f : l2 * exp2f(m2 - M);
    m = M;
    l = a + c;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void refresh_scores_kernel(
    const T* __restrict__ q_gen, const T* __restrict__ k_full, float* __restrict__ ws, int G,
    int N, float scale_log2) {
    __shared__ float q_s[kQG][kD];
    __shared__ float red_m[kThreads / kWave][kQG], red_l[kThreads / kWave][kQG];
    __shared__ float stat_m[kQG], stat_inv[kQG];
    extern __shared__ float acc_s[];  // [N]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int u = blockIdx.x;
    const T* K = k_full + (size_t)u * N * kD;

    for (int j = tid; j < N; j += kThreads) acc_s[j] = 0.f;

    for (int g0 = 0; g0 < G; g0 += kQG) {
        const int ng = min(kQG, G - g0);
        __syncthreads();
        for (int e = tid; e < kQG * kD; e += kThreads) {
            const int gq = e / kD, d = e % kD;
            q_s[gq][d] = (gq < ng) ? load1(q_gen, ((size_t)u * G + g0 + gq) * kD + d) * scale_log2
                                   : 0.f;
        }
        __syncthreads();

        // Pass 1: per-query running max / normaliser over this thread's keys.
        float m[kQG], l[kQG];
#pragma unroll
        for (int gq = 0; gq < kQG; ++gq) {
            m[gq] = -INFINITY;
            l[gq] = 0.f;
        }
        for (int j = tid; j < N; j += kThreads) {
            float kr[kD];
            load_row(K + (size_t)j * kD, kr);
#pragma unroll
            for (int gq = 0; gq < kQG; ++gq) {
                if (gq < ng) {
                    float s = 0.f;
#pragma unroll
                    for (int d = 0; d < kD; ++d) s = fmaf(q_s[gq][d], kr[d], s);
                    merge_ml(m[gq], l[gq], s, 1.f);
                }
            }
        }
#pragma unroll
        for (int gq = 0; gq < kQG; ++gq) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float mo = __shfl_xor(m[gq], o, kWave);
                const float lo = __shfl_xor(l[gq], o, kWave);
                merge_ml(m[gq], l[gq], mo, lo);
            }
            if (lane == 0) {
                red_m[wid][gq] = m[gq];
                red_l[wid][gq] = l[gq];
            }
        }
        __syncthreads();
        if (tid < kQG) {
            float mm = red_m[0][tid], ll = red_l[0][tid];
            for (int w = 1; w < kThreads / kWave; ++w) merge_ml(mm, ll, red_m[w][tid], red_l[w][tid]);
            stat_m[tid] = mm;
            stat_inv[tid] = (ll > 0.f) ? 1.f / ll : 0.f;
        }
        __syncthreads();

        // Pass 2: sum of normalised probabilities over the group's queries.
        for (int j = tid; j < N; j += kThreads) {
            float kr[kD];
            load_row(K + (size_t)j * kD, kr);
            float a = 0.f;
#pragma unroll
            for (int gq = 0; gq < kQG; ++gq) {
                if (gq < ng) {
                    float s = 0.f;
#pragma unroll
                    for (int d = 0; d < kD; ++d) s = fmaf(q_s[gq][d], kr[d], s);
                    a += exp2f(s - stat_m[gq]) * stat_inv[gq];
                }
            }
            acc_s[j] += a;
        }
    }
    __syncthreads();
    for (int j = tid; j < N; j += kThreads) ws[(size_t)u * N + j] = acc_s[j];
}

__device__ __forceinline__ uint64_t rank_key(float s, int j) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(ord) << 32) | static_cast<uint64_t>(0xffffffffu - (uint32_t)j);
}

__global__ __launch_bounds__(kThreads) void refresh_select_kernel(
    const float* __restrict__ ws, const int32_t* __restrict__ gp_idx, int ld_gp, int n_gp, int K,
    float inv_hg, float* __restrict__ scores, int32_t* __restrict__ active_idx, int ld_act,
    int32_t* __restrict__ cached_idx, int ld_cached, int32_t* __restrict__ cached_len, int H,
    int N, int NP) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* keys = reinterpret_cast<uint64_t*>(smem);    // [NP]
    uint8_t* state = smem + (size_t)NP * sizeof(uint64_t);  // [N]: 0 cand, 1 G/P, 2 refresh
    __shared__ int scan_scratch[kThreads / kWave];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;

    for (int j = tid; j < N; j += kThreads) state[j] = 0;
    __syncthreads();
    for (int m = tid; m < n_gp; m += kThreads) {
        const int j = gp_idx[(size_t)b * ld_gp + m];
        active_idx[(size_t)b * ld_act + m] = j;
        if (j >= 0 && j < N) state[j] = 1;
    }
    __syncthreads();
    for (int j = tid; j < NP; j += kThreads) {
        uint64_t key = 0;
        if (j < N) {
            float s = 0.f;
            for (int h = 0; h < H; ++h) s += ws[((size_t)b * H + h) * N + j];
            s *= inv_hg;
            scores[(size_t)b * N + j] = s;
            if (state[j] == 0) key = rank_key(s, j);
        }
        keys[j] = key;
    }
    __syncthreads();

    // Bitonic sort, descending.
    for (int k = 2; k <= NP; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            for (int i = tid; i < NP; i += kThreads) {
                const int ixj = i ^ jj;
                if (ixj > i) {
                    const uint64_t a = keys[i], c = keys[ixj];
                    const bool first_half = (i & k) == 0;
                    if (first_half ? (a < c) : (a > c)) {
                        keys[i] = c;
                        keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }

    for (int r = tid; r < K; r += kThreads) {
        const uint64_t key = keys[r];
        int j = -1;
        if (key != 0) {
            j = (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
            state[j] = 2;
        }
        active_idx[(size_t)b * ld_act + n_gp + r] = j;
    }
    __syncthreads();

    // Ascending compaction of the remaining candidates (state 0).
    const int per = (N + kThreads - 1) / kThreads;
    const int j0 = tid * per;
    const int j1 = min(N, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += (state[j] == 0);
    int total = 0;
    int pos = block_exclusive_scan<kThreads>(cnt, scan_scratch, &total);
    int32_t* crow = cached_idx + (size_t)b * ld_cached;
    for (int j = j0; j < j1; ++j)
        if (state[j] == 0) {
            if (pos < ld_cached) crow[pos] = j;
            ++pos;
        }
    for (int t = total + tid; t < ld_cached; t += kThreads) crow[t] = -1;
    if (tid == 0) cached_len[b] = total;
}

}  // namespace

int launch_refresh_topk(const void* q_gen, const void* k_full, const int32_t* gp_idx, int ld_gp,
                        int n_gp, int K, float scale, float* scores, int32_t* active_idx,
                        int ld_act, int32_t* cached_idx, int ld_cached, int32_t* cached_len,
                        float* workspace, int B, int H, int G, int N, int dtype,
                        void* stream_v) {
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    const float scale_log2 = scale * 1.4426950408889634f;
    const size_t lds1 = (size_t)N * sizeof(float);
    if (dtype == MAR_BF16) {
        hipLaunchKernelGGL(refresh_scores_kernel<uint16_t>, dim3(B * H), dim3(kThreads), lds1,
                           stream, static_cast<const uint16_t*>(q_gen),
                           static_cast<const uint16_t*>(k_full), workspace, G, N, scale_log2);
    } else {
        hipLaunchKernelGGL(refresh_scores_kernel<float>, dim3(B * H), dim3(kThreads), lds1, stream,
                           static_cast<const float*>(q_gen), static_cast<const float*>(k_full),
                           workspace, G, N, scale_log2);
    }
    int st = status_from_launch();
    if (st != MAR_OK) return st;
    int NP = 1;
    while (NP < N) NP <<= 1;
    const size_t lds2 = (size_t)NP * sizeof(uint64_t) + (size_t)N;
    const float inv_hg = 1.f / (float)(H * G);
    hipLaunchKernelGGL(refresh_select_kernel, dim3(B), dim3(kThreads), lds2, stream, workspace,
                       gp_idx, ld_gp, n_gp, K, inv_hg, scores, active_idx, ld_act, cached_idx,
                       ld_cached, cached_len, H, N, NP);
    return status_from_launch();
}

}  // namespace marca
