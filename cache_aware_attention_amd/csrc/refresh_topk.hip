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
// Kernel 1 (one workgroup per (sequence, head)) writes each token's
// probability summed over the generating queries into a per-(b,h,token)
// partial.  bf16: the score tiles run on MFMA.  Up to 16 generating queries
// and 320 keys the scores stay in registers from the MFMA to the per-key
// sums; otherwise, when the head's [queries x keys] score block fits in LDS,
// the keys are read once (scores kept in LDS, then per-query max / sum, then
// per-key sums), else two passes over the keys (running (max, sum) per
// query, then normalised sums).  fp32 uses a plain FMA version.
// Kernel 2 (one workgroup per sequence): sums the partials over heads in a
// fixed order (no float atomics, deterministic), ranks the eligible tokens by
// counting larger 64-bit keys with wave ballots (orderable score << 32 |
// ~index, so equal scores put the lower index first), emits the refreshing
// tokens, and
// compacts the ascending cached complement with a block prefix sum.
#include <mutex>

#include "device_util.h"
#include "launch.h"

namespace marca {
namespace {

constexpr int kD = 64;
constexpr int kThreads = 256;
constexpr size_t kMaxScoreLds = 64 * 1024;  // single-pass scores when [QT*16][N+16] floats fit
// Register-resident scores: 4 waves x 5 key tiles per unit (up to 320 keys).
constexpr int kRegWaves = 4;
constexpr int kRegTiles = 5;

// Merge two running softmax states (max m, sum l) in base 2.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float a = (m == -INFINITY) ? 0.f : l * exp2f(m - M);
    const float c = (m2 == -INFINITY) ? 0.f : l2 * exp2f(m2 - M);
    m = M;
    l = a + c;
}

// fp32 version of kernel 1: plain FMA, one generating query at a time with
// block-wide max and sum reductions (three sweeps over the head's keys per
// query; this path serves float inputs, not the bf16 decoding shapes).
__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red_s) {
    v = is_max ? wave_max(v) : wave_sum(v);
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) red_s[wid] = v;
    __syncthreads();
    float r = red_s[0];
    for (int w = 1; w < kThreads / kWave; ++w) r = is_max ? fmaxf(r, red_s[w]) : r + red_s[w];
    return r;
}

__device__ __forceinline__ float dot_row(const float* q_s, const float* k) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 a = reinterpret_cast<const float4*>(k)[c];
        s = fmaf(q_s[4 * c], a.x, s);
        s = fmaf(q_s[4 * c + 1], a.y, s);
        s = fmaf(q_s[4 * c + 2], a.z, s);
        s = fmaf(q_s[4 * c + 3], a.w, s);
    }
    return s;
}

__global__ __launch_bounds__(kThreads) void refresh_scores_f32_kernel(
    const float* __restrict__ q_gen, const float* __restrict__ k_full, float* __restrict__ ws,
    int G, int N, float scale_log2) {
    __shared__ float q_s[kD];
    __shared__ float red_s[kThreads / kWave];
    extern __shared__ float acc_s[];  // [N]
    const int tid = threadIdx.x;
    const int u = blockIdx.x;
    const float* K = k_full + (size_t)u * N * kD;
    for (int j = tid; j < N; j += kThreads) acc_s[j] = 0.f;
    for (int g = 0; g < G; ++g) {
        __syncthreads();
        if (tid < kD) q_s[tid] = q_gen[((size_t)u * G + g) * kD + tid] * scale_log2;
        __syncthreads();
        float mloc = -INFINITY;
        for (int j = tid; j < N; j += kThreads) mloc = fmaxf(mloc, dot_row(q_s, K + (size_t)j * kD));
        const float M = block_reduce(mloc, true, red_s);
        float lloc = 0.f;
        for (int j = tid; j < N; j += kThreads) lloc += exp2f(dot_row(q_s, K + (size_t)j * kD) - M);
        const float inv = 1.f / block_reduce(lloc, false, red_s);
        for (int j = tid; j < N; j += kThreads)
            acc_s[j] += exp2f(dot_row(q_s, K + (size_t)j * kD) - M) * inv;
    }
    __syncthreads();
    for (int j = tid; j < N; j += kThreads) ws[(size_t)u * N + j] = acc_s[j];
}

// bf16 path of kernel 1 on MFMA.  Workgroup of 4 waves per (sequence, head);
// S = Q K^T tiles of 16 queries x 16 keys on v_mfma_f32_16x16x32_bf16 (Q as
// the A operand, 16-byte pieces of key rows as the B operand), so a lane
// holds S[query 4g+i][key m16].  Pass 1 keeps a running (max, sum) per query
// over the wave's key tiles, merged across the 16 lanes of a group and then
// across the waves; pass 2 recomputes S (the head's keys are re-read, mostly
// from L2), normalises, and sums over the queries in registers and two lane
// shuffles.  Each key tile belongs to one wave, so no accumulation races.
template <int QT>
__global__ __launch_bounds__(kThreads) void refresh_scores_mfma_kernel(
    const uint16_t* __restrict__ q_gen, const uint16_t* __restrict__ k_full,
    float* __restrict__ ws, int G, int N, float scale_log2) {
    constexpr int kWaves = kThreads / kWave;
    __shared__ float red_m[kWaves][QT * 16], red_l[kWaves][QT * 16];
    __shared__ float stat_m[QT * 16], stat_inv[QT * 16];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int g = lane >> 4, m16 = lane & 15;
    const int u = blockIdx.x;

    bf16x8_t qa[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int q = qt * 16 + m16;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        if (q < G) {
            const uint4* p = reinterpret_cast<const uint4*>(q_gen + ((size_t)u * G + q) * kD);
            lo = p[g];
            hi = p[4 + g];
        }
        qa[qt][0] = __builtin_bit_cast(bf16x8_t, lo);
        qa[qt][1] = __builtin_bit_cast(bf16x8_t, hi);
    }
    const uint16_t* K = k_full + (size_t)u * N * kD;
    const int ntiles = (N + 15) / 16;

    auto tile_scores = [&](int t, f32x4_t (&s)[QT]) {
        const int key = 16 * t + m16;
        const uint4* p = reinterpret_cast<const uint4*>(K + (size_t)(key < N ? key : 0) * kD);
        const bf16x8_t k0 = __builtin_bit_cast(bf16x8_t, p[g]);
        const bf16x8_t k1 = __builtin_bit_cast(bf16x8_t, p[4 + g]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qt][0], k0, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qt][1], k1, acc, 0, 0, 0);
            s[qt] = acc;
        }
    };

    // Pass 1: running max / sum per query over this wave's key tiles.
    float m[QT][4], l[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[qt][i] = -INFINITY;
            l[qt][i] = 0.f;
        }
    for (int t = w; t < ntiles; t += kWaves) {
        f32x4_t s[QT];
        tile_scores(t, s);
        const bool valid = 16 * t + m16 < N;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = valid ? s[qt][i] * scale_log2 : -INFINITY;
                const float M = fmaxf(m[qt][i], v);
                const float Mr = (M == -INFINITY) ? 0.f : M;
                l[qt][i] = l[qt][i] * __builtin_amdgcn_exp2f(m[qt][i] - Mr) +
                           __builtin_amdgcn_exp2f(v - Mr);
                m[qt][i] = M;
            }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1)
                merge_ml(m[qt][i], l[qt][i], __shfl_xor(m[qt][i], o, kWave),
                         __shfl_xor(l[qt][i], o, kWave));
            if (m16 == 0) {
                red_m[w][qt * 16 + 4 * g + i] = m[qt][i];
                red_l[w][qt * 16 + 4 * g + i] = l[qt][i];
            }
        }
    __syncthreads();
    if (tid < QT * 16) {
        float mm = red_m[0][tid], ll = red_l[0][tid];
        for (int v = 1; v < kWaves; ++v) merge_ml(mm, ll, red_m[v][tid], red_l[v][tid]);
        stat_m[tid] = (mm == -INFINITY) ? 0.f : mm;
        stat_inv[tid] = (tid < G && ll > 0.f) ? 1.f / ll : 0.f;  // padded queries add 0
    }
    __syncthreads();

    // Pass 2: normalised probabilities summed over the queries, per key.
    float sm[QT][4], si[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sm[qt][i] = stat_m[qt * 16 + 4 * g + i];
            si[qt][i] = stat_inv[qt * 16 + 4 * g + i];
        }
    for (int t = w; t < ntiles; t += kWaves) {
        f32x4_t s[QT];
        tile_scores(t, s);
        float col = 0.f;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                col += __builtin_amdgcn_exp2f(s[qt][i] * scale_log2 - sm[qt][i]) * si[qt][i];
        col += __shfl_xor(col, 16, kWave);
        col += __shfl_xor(col, 32, kWave);
        const int key = 16 * t + m16;
        if (g == 0 && key < N) ws[(size_t)u * N + key] = col;
    }
}

// Single-pass bf16 path of kernel 1, used when the head's score block fits
// in LDS: every wave computes S = Q K^T for its key tiles on MFMA (as above)
// and writes scale_log2 * S to LDS ([query][key], row stride NS = N + 16
// floats so the four lane groups of a tile store hit different banks); then
// one wave per query reduces its row to (max, 1/sum); then one thread per
// key sums exp2(S - max) / sum over the queries.  Each key row is read from
// HBM once.
template <int QT>
__global__ __launch_bounds__(kThreads) void refresh_scores_lds_kernel(
    const uint16_t* __restrict__ q_gen, const uint16_t* __restrict__ k_full,
    float* __restrict__ ws, int G, int N, int NS, float scale_log2) {
    constexpr int kWaves = kThreads / kWave;
    constexpr int kBatch = 8;  // key tiles whose loads a wave issues together
    extern __shared__ float s_lds[];  // [QT * 16][NS]
    __shared__ float stat_m[QT * 16], stat_inv[QT * 16];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int g = lane >> 4, m16 = lane & 15;
    const int u = blockIdx.x;

    bf16x8_t qa[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int q = qt * 16 + m16;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        if (q < G) {
            const uint4* p = reinterpret_cast<const uint4*>(q_gen + ((size_t)u * G + q) * kD);
            lo = p[g];
            hi = p[4 + g];
        }
        qa[qt][0] = __builtin_bit_cast(bf16x8_t, lo);
        qa[qt][1] = __builtin_bit_cast(bf16x8_t, hi);
    }
    const uint16_t* K = k_full + (size_t)u * N * kD;
    const int ntiles = (N + 15) / 16;

    for (int t0 = w; t0 < ntiles; t0 += kWaves * kBatch) {
        uint4 kr[kBatch][2];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {  // missing tiles / keys read key row 0
            const int key = 16 * (t0 + kWaves * b) + m16;
            const uint4* p = reinterpret_cast<const uint4*>(K + (size_t)(key < N ? key : 0) * kD);
            kr[b][0] = p[g];
            kr[b][1] = p[4 + g];
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int t = t0 + kWaves * b;
            const int key = 16 * t + m16;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    qa[qt][0], __builtin_bit_cast(bf16x8_t, kr[b][0]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    qa[qt][1], __builtin_bit_cast(bf16x8_t, kr[b][1]), acc, 0, 0, 0);
                if (t < ntiles && key < N) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s_lds[(qt * 16 + 4 * g + i) * NS + key] = acc[i] * scale_log2;
                }
            }
        }
    }
    __syncthreads();

    for (int q = w; q < G; q += kWaves) {
        const float* row = s_lds + (size_t)q * NS;
        float m = -INFINITY;
        for (int j = lane; j < N; j += kWave) m = fmaxf(m, row[j]);
        m = wave_max(m);
        float l = 0.f;
        for (int j = lane; j < N; j += kWave) l += __builtin_amdgcn_exp2f(row[j] - m);
        l = wave_sum(l);
        if (lane == 0) {
            stat_m[q] = m;
            stat_inv[q] = 1.f / l;
        }
    }
    __syncthreads();

    for (int j = tid; j < N; j += kThreads) {
        float col = 0.f;
        for (int q = 0; q < G; ++q)
            col += __builtin_amdgcn_exp2f(s_lds[(size_t)q * NS + j] - stat_m[q]) * stat_inv[q];
        ws[(size_t)u * N + j] = col;
    }
}

// Register-resident bf16 path of kernel 1 for short sequences: up to 16
// generating queries and at most W * TPW key tiles.  W waves per (sequence,
// head) unit; wave w keeps the scores of its tiles t = w + W k (k < TPW) in
// registers from the MFMA to the per-key sums, so nothing of the score block
// goes through LDS (only the W partial row maxima and sums when W > 1).  At
// 320 tokens and one wave per unit every unit of a decoding batch is resident
// at once, two waves per SIMD, each with all of its key rows in flight.
// The order of every reduction is fixed: over the wave's tiles in k order,
// then a butterfly over the 16 lanes of a row, then over the waves in w
// order, and per key over the four rows i of a lane, then across the lane
// groups (xor 16, then xor 32); equal key rows therefore get equal scores.
template <int TPW, int W>
__global__ __launch_bounds__(64 * W) void refresh_scores_reg_kernel(
    const uint16_t* __restrict__ q_gen, const uint16_t* __restrict__ k_full,
    float* __restrict__ ws, int G, int N, float scale_log2) {
    __shared__ float red[2][W][16];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = (W > 1) ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) : 0;
    const int g = lane >> 4, m16 = lane & 15;
    const int u = blockIdx.x;

    // Q operand: query m16, dims 8g..8g+7 and 32+8g..32+8g+7 (zero past G).
    uint4 qlo = make_uint4(0, 0, 0, 0), qhi = qlo;
    if (m16 < G) {
        const uint4* p = reinterpret_cast<const uint4*>(q_gen + ((size_t)u * G + m16) * kD);
        qlo = p[g];
        qhi = p[4 + g];
    }
    const bf16x8_t qa0 = __builtin_bit_cast(bf16x8_t, qlo);
    const bf16x8_t qa1 = __builtin_bit_cast(bf16x8_t, qhi);
    const uint16_t* K = k_full + (size_t)u * N * kD;

    // Every tile's key rows are requested before the first MFMA, as whole
    // 128-byte rows with streaming loads (lane: piece kpiece of key
    // 16 (w + W k) + 8h + m16 % 8), then exchanged into the operand layout
    // (piece g and 4 + g of key 16 (w + W k) + m16); a key past N (partial
    // or missing tile) reads row 0 and is masked below.
    const int kpiece = (m16 < 8) ? g : 4 + g;
    uint4 kr[TPW][2];
#pragma unroll
    for (int k = 0; k < TPW; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 16 * (w + W * k) + 8 * h + (m16 & 7);
            kr[k][h] = ld_stream(reinterpret_cast<const uint4*>(K + (size_t)(key < N ? key : 0) * kD) +
                                 kpiece);
        }
#pragma unroll
    for (int k = 0; k < TPW; ++k) swap_row_halves(kr[k][0], kr[k][1], kr[k][0], kr[k][1]);
    // s[k][i] = scale_log2 * S[query 4g+i][key 16 (w + W k) + m16]
    f32x4_t s[TPW];
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, __builtin_bit_cast(bf16x8_t, kr[k][0]),
                                                      acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, __builtin_bit_cast(bf16x8_t, kr[k][1]),
                                                      acc, 0, 0, 0);
        const bool ok = 16 * (w + W * k) + m16 < N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[k][i] = ok ? acc[i] * scale_log2 : -INFINITY;
            mx[i] = fmaxf(mx[i], s[k][i]);
        }
    }
    // Row maxima over all N keys (finite: key 0 is in wave 0's first tile).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], o, kWave));
    }
    if constexpr (W > 1) {
        if (m16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[0][w][4 * g + i] = mx[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = red[0][0][4 * g + i];
#pragma unroll
            for (int v = 1; v < W; ++v) m = fmaxf(m, red[0][v][4 * g + i]);
            mx[i] = m;
        }
    }
    // Probabilities (unnormalised) in place, and the row sums.
    float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < TPW; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[k][i] = __builtin_amdgcn_exp2f(s[k][i] - mx[i]);
            l[i] += s[k][i];
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) l[i] += __shfl_xor(l[i], o, kWave);
    }
    if constexpr (W > 1) {
        if (m16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[1][w][4 * g + i] = l[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = red[1][0][4 * g + i];
#pragma unroll
            for (int v = 1; v < W; ++v) t += red[1][v][4 * g + i];
            l[i] = t;
        }
    }
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = (4 * g + i < G) ? 1.f / l[i] : 0.f;  // padded queries add 0
    // Per key: the normalised probabilities summed over the queries.
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        float col = s[k][0] * inv[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) col += s[k][i] * inv[i];
        col += __shfl_xor(col, 16, kWave);
        col += __shfl_xor(col, 32, kWave);
        const int key = 16 * (w + W * k) + m16;
        if (g == 0 && key < N) ws[(size_t)u * N + key] = col;
    }
}

// Token j's partials summed over the H heads in head order, with the loads of
// a batch of heads issued together (a loop of dependent load-add steps would
// wait for each load in turn).
__device__ __forceinline__ float head_sum(const float* __restrict__ ws, int b, int H, int N, int j) {
    constexpr int kBatch = 16;
    float s = 0.f;
    for (int h0 = 0; h0 < H; h0 += kBatch) {
        float v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            v[i] = (h0 + i < H) ? ws[((size_t)b * H + h0 + i) * N + j] : 0.f;
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (h0 + i < H) s += v[i];
    }
    return s;
}

__device__ __forceinline__ uint64_t rank_key(float s, int j) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(ord) << 32) | static_cast<uint64_t>(0xffffffffu - (uint32_t)j);
}

// Kernel 2.  The rank of an eligible token is the number of eligible tokens
// whose 64-bit key is larger; keys are unique (the index is part of the key),
// so ranks are a permutation and the K smallest ranks are the refreshing
// tokens in (score descending, index ascending) order.  Each wave ranks
// tokens w, w + kSelWaves, ...; lane l holds keys l, l + 64, ... and one
// ballot per 64 keys counts the larger ones.
// NB > 0 (N <= 64 NB <= 2048): all keys sit in NB registers per lane, so the
// ballots need no bounds test; four tokens are ranked per step, which keeps
// four independent compare / count chains in flight, and the ascending
// compaction takes its positions from a ballot per wave.  A wave ranks at
// most 64 tokens (one per lane) per round and a thread compacts one token
// per round: one round up to 1024 tokens, two up to 2048.  NB == 0 is the
// general form for longer sequences, which reads the keys past the first 512
// from LDS inside the counting loop.
constexpr int kSelThreads = 1024;  // 16 waves: more compare / count chains in flight per CU
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelMaxRegBlocks = 32;  // the register-block path: up to 2048 tokens
static_assert(kSelThreads == kSelWaves * kWave && kSelWaves * kWave * 2 >= kSelMaxRegBlocks * kWave,
              "selection: two rounds of one token per thread cover the register-block path");
template <int NB>
__global__ __launch_bounds__(kSelThreads) void refresh_select_kernel(
    const float* __restrict__ ws, const int32_t* __restrict__ gp_idx, int ld_gp, int n_gp, int K,
    float inv_hg, float* __restrict__ scores, int32_t* __restrict__ active_idx, int ld_act,
    int32_t* __restrict__ cached_idx, int ld_cached, int32_t* __restrict__ cached_len, int H,
    int N) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* keys = reinterpret_cast<uint64_t*>(smem);   // [N], 0 = not eligible
    uint8_t* state = smem + (size_t)N * sizeof(uint64_t);  // [N]: 0 cand, 1 G/P, 2 refresh
    __shared__ int scan_scratch[kSelWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int b = blockIdx.x;
    int32_t* arow = active_idx + (size_t)b * ld_act;

    // Both global reads (the G/P list and the head partials of this thread's
    // first token) are issued before the first barrier so their latencies
    // overlap.
    const int gp0 = (tid < n_gp) ? gp_idx[(size_t)b * ld_gp + tid] : -1;
    const float s0 = (tid < N) ? head_sum(ws, b, H, N, tid) : 0.f;  // fixed order
    for (int j = tid; j < N; j += kSelThreads) state[j] = 0;
    for (int r = tid; r < K; r += kSelThreads) arow[n_gp + r] = -1;  // fewer eligible than K
    __syncthreads();
    for (int m = tid; m < n_gp; m += kSelThreads) {
        const int j = (m == tid) ? gp0 : gp_idx[(size_t)b * ld_gp + m];
        arow[m] = j;
        if (j >= 0 && j < N) state[j] = 1;
    }
    __syncthreads();
    for (int j = tid; j < N; j += kSelThreads) {
        float s = (j != tid) ? head_sum(ws, b, H, N, j) : s0;
        s *= inv_hg;
        scores[(size_t)b * N + j] = s;
        keys[j] = (state[j] == 0) ? rank_key(s, j) : 0ull;
    }
    __syncthreads();

    int32_t* crow = cached_idx + (size_t)b * ld_cached;
    if constexpr (NB > 0) {
        static_assert(NB <= kSelMaxRegBlocks, "register blocks");
        constexpr int kRounds = (NB * kWave + kSelThreads - 1) / kSelThreads;  // 1 or 2
        uint64_t kr[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int i = lane + kWave * k;
            kr[k] = (i < N) ? keys[i] : 0ull;  // 0 is never larger than an eligible key
        }
        // Round rd: lane l holds the key of token base + kSelWaves * l, base =
        // wu + kSelThreads * rd.  Tokens at or past N read key 0 and are
        // skipped like ineligible ones; nt <= 64, so the lane index of every
        // step stays below 64.
        const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
        for (int rd = 0; rd < kRounds; ++rd) {
            const int base = wu + kSelThreads * rd;
            const int jl = base + kSelWaves * lane;
            const uint64_t kl = (jl < N) ? keys[jl] : 0ull;
            const int nt = (N > base) ? min(kWave, (N - base + kSelWaves - 1) / kSelWaves) : 0;
            for (int e0 = 0; e0 < nt; e0 += 4) {
                uint64_t kj[4];
                int cnt[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(kl), e0 + q);
                    const uint32_t hi =
                        __builtin_amdgcn_readlane(static_cast<uint32_t>(kl >> 32), e0 + q);
                    kj[q] = (static_cast<uint64_t>(hi) << 32) | lo;
                    cnt[q] = 0;
                }
#pragma unroll
                for (int k = 0; k < NB; ++k)
#pragma unroll
                    for (int q = 0; q < 4; ++q) cnt[q] += __popcll(__ballot(kr[k] > kj[q]));
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (kj[q] != 0 && cnt[q] < K && lane == 0) {
                        const int j = base + kSelWaves * (e0 + q);
                        arow[n_gp + cnt[q]] = j;
                        state[j] = 2;
                    }
            }
        }
        __syncthreads();

        // Ascending compaction: in round rd thread tid holds token
        // tid + kSelThreads * rd; a round's positions follow the earlier ones.
        int done = 0;
#pragma unroll
        for (int rd = 0; rd < kRounds; ++rd) {
            const int t = tid + kSelThreads * rd;
            const bool c = t < N && state[t] == 0;
            const uint64_t m = __ballot(c);
            const int below = __builtin_amdgcn_mbcnt_hi(
                static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
            if (lane == 0) scan_scratch[w] = __popcll(m);
            __syncthreads();
            int pos = done + below, total = 0;
#pragma unroll
            for (int v = 0; v < kSelWaves; ++v) {
                const int sv = scan_scratch[v];
                pos += (v < w) ? sv : 0;
                total += sv;
            }
            if (c && pos < ld_cached) crow[pos] = t;
            done += total;
            __syncthreads();  // every wave has read scan_scratch before the next round writes it
        }
        for (int t = done + tid; t < ld_cached; t += kSelThreads) crow[t] = -1;
        if (tid == 0) cached_len[b] = done;
        return;
    }

    // The first kRegs * 64 keys live in registers; keys past them (N > 512)
    // are read from LDS in the counting loop.
    constexpr int kRegs = 8;
    uint64_t kr[kRegs];
#pragma unroll
    for (int k = 0; k < kRegs; ++k) {
        const int i = lane + kWave * k;
        kr[k] = (i < N) ? keys[i] : 0ull;  // 0 is never larger than an eligible key
    }
    const int nblk = (N + kWave - 1) / kWave;
    // The wave's tokens j = w + kSelWaves * (64 t + l): lane l fetches the key
    // of its token for round t, and the round then walks the 64 tokens with
    // the key taken from that lane (readlane), so no LDS access sits in the
    // inner loop.
    for (int t0 = w; t0 < N; t0 += kSelWaves * kWave) {
        const int jl = t0 + kSelWaves * lane;
        const uint64_t kl = (jl < N) ? keys[jl] : 0ull;
        const int nt = min(kWave, (N - t0 + kSelWaves - 1) / kSelWaves);
        for (int e = 0; e < nt; ++e) {
            const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(kl), e);
            const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(kl >> 32), e);
            const uint64_t kj = (static_cast<uint64_t>(hi) << 32) | lo;
            if (kj == 0) continue;  // not eligible (wave-uniform)
            int cnt = 0;
#pragma unroll
            for (int k = 0; k < kRegs; ++k)
                if (k < nblk) cnt += __popcll(__ballot(kr[k] > kj));
            for (int i0 = kRegs * kWave; i0 < N; i0 += kWave) {
                const int i = i0 + lane;
                cnt += __popcll(__ballot(i < N && keys[i] > kj));
            }
            if (cnt < K && lane == 0) {
                const int j = t0 + kSelWaves * e;
                arow[n_gp + cnt] = j;
                state[j] = 2;
            }
        }
    }
    __syncthreads();

    // Ascending compaction of the remaining candidates (state 0).
    const int per = (N + kSelThreads - 1) / kSelThreads;
    const int j0 = tid * per;
    const int j1 = min(N, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += (state[j] == 0);
    int total = 0;
    int pos = block_exclusive_scan<kSelThreads>(cnt, scan_scratch, &total);
    for (int j = j0; j < j1; ++j)
        if (state[j] == 0) {
            if (pos < ld_cached) crow[pos] = j;
            ++pos;
        }
    for (int t = total + tid; t < ld_cached; t += kSelThreads) crow[t] = -1;
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
        const int qt = (G + 15) / 16;
        const dim3 grid(B * H), block(kThreads);
        const uint16_t* q = static_cast<const uint16_t*>(q_gen);
        const uint16_t* k = static_cast<const uint16_t*>(k_full);
        const int NS = N + 16;
        const size_t lds_s = (size_t)qt * 16 * NS * sizeof(float);
        if (qt == 1 && (N + 15) / 16 <= kRegTiles * kRegWaves) {
            hipLaunchKernelGGL((refresh_scores_reg_kernel<kRegTiles, kRegWaves>), grid,
                               dim3(kRegWaves * kWave), 0, stream, q, k, workspace, G, N,
                               scale_log2);
        } else if (lds_s <= kMaxScoreLds) {
            switch (qt) {
                case 1: hipLaunchKernelGGL(refresh_scores_lds_kernel<1>, grid, block, lds_s, stream, q, k, workspace, G, N, NS, scale_log2); break;
                case 2: hipLaunchKernelGGL(refresh_scores_lds_kernel<2>, grid, block, lds_s, stream, q, k, workspace, G, N, NS, scale_log2); break;
                case 3: hipLaunchKernelGGL(refresh_scores_lds_kernel<3>, grid, block, lds_s, stream, q, k, workspace, G, N, NS, scale_log2); break;
                default: hipLaunchKernelGGL(refresh_scores_lds_kernel<4>, grid, block, lds_s, stream, q, k, workspace, G, N, NS, scale_log2); break;
            }
        } else {
            switch (qt) {
                case 1: hipLaunchKernelGGL(refresh_scores_mfma_kernel<1>, grid, block, 0, stream, q, k, workspace, G, N, scale_log2); break;
                case 2: hipLaunchKernelGGL(refresh_scores_mfma_kernel<2>, grid, block, 0, stream, q, k, workspace, G, N, scale_log2); break;
                case 3: hipLaunchKernelGGL(refresh_scores_mfma_kernel<3>, grid, block, 0, stream, q, k, workspace, G, N, scale_log2); break;
                default: hipLaunchKernelGGL(refresh_scores_mfma_kernel<4>, grid, block, 0, stream, q, k, workspace, G, N, scale_log2); break;
            }
        }
    } else {
        hipLaunchKernelGGL(refresh_scores_f32_kernel, dim3(B * H), dim3(kThreads), lds1, stream,
                           static_cast<const float*>(q_gen), static_cast<const float*>(k_full),
                           workspace, G, N, scale_log2);
    }
    const int st = status_from_launch();
    if (st != MAR_OK) return st;
    return launch_refresh_select(workspace, gp_idx, ld_gp, n_gp, K, scores, active_idx, ld_act,
                                 cached_idx, ld_cached, cached_len, B, H, G, N, stream_v);
}

int launch_refresh_select(const float* workspace, const int32_t* gp_idx, int ld_gp, int n_gp,
                          int K, float* scores, int32_t* active_idx, int ld_act,
                          int32_t* cached_idx, int ld_cached, int32_t* cached_len, int B, int H,
                          int G, int N, void* stream_v) {
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    const size_t lds2 = (size_t)N * sizeof(uint64_t) + (size_t)N;
    const float inv_hg = 1.f / (float)(H * G);
#define MARCA_SELECT(NB)                                                                     \
    hipLaunchKernelGGL(refresh_select_kernel<NB>, dim3(B), dim3(kSelThreads), lds2, stream,     \
                       workspace, gp_idx, ld_gp, n_gp, K, inv_hg, scores, active_idx, ld_act,   \
                       cached_idx, ld_cached, cached_len, H, N)
    // one instantiation per block count up to 8, then a few sizes up to 32
    // (blocks past N hold key 0 and count nothing)
    const int nb = (N + kWave - 1) / kWave;
    switch (nb) {
        case 1: MARCA_SELECT(1); break;
        case 2: MARCA_SELECT(2); break;
        case 3: MARCA_SELECT(3); break;
        case 4: MARCA_SELECT(4); break;
        case 5: MARCA_SELECT(5); break;
        case 6: MARCA_SELECT(6); break;
        case 7: MARCA_SELECT(7); break;
        case 8: MARCA_SELECT(8); break;
        default:
            if (nb <= 12) MARCA_SELECT(12);
            else if (nb <= 16) MARCA_SELECT(16);
            else if (nb <= 18) MARCA_SELECT(18);
            else if (nb <= 24) MARCA_SELECT(24);
            else if (nb <= kSelMaxRegBlocks) MARCA_SELECT(32);
            else MARCA_SELECT(0);
            break;
    }
#undef MARCA_SELECT
    return status_from_launch();
}

// ---------------------------------------------------------------------------
// Allocation-free form (mar_refresh_topk_noalloc), for callers that cannot
// allocate device memory.  The per-(sequence, head, token) partial scores go
// to `scratch`, a file-scope device array of kTopkScratchBytes: each device
// that runs the call holds its own copy at its own address until the process
// ends.  In host code the array's name is only a host-side stand-in, so the
// device address is looked up once per device with hipGetSymbolAddress (on
// the device of the call's stream) and only that address is passed to the
// kernels.  Every scores kernel writes each of the B*H*N partials before the
// selection reads them, so the array needs no clearing between calls; calls
// that overlap on one device share it and race.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) float scratch[kTopkScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream` (the current
// device for the null stream), looked up on the first call on that device.
int scratch_address(hipStream_t stream, float** out) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MAR_E_LAUNCH;
    int dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) {
        (void)hipGetLastError();
        return MAR_E_LAUNCH;
    }
    if (dev < 0 || dev >= kMaxDevices) return MAR_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return MAR_E_LAUNCH;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return MAR_E_LAUNCH;
        }
        g_scratch_dev[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_dev[dev];
    return MAR_OK;
}

}  // namespace

int launch_refresh_topk_noalloc(const void* q_gen, const void* k_full, const int32_t* gp_idx,
                                int ld_gp, int n_gp, int K, float scale, float* scores,
                                int32_t* active_idx, int ld_act, int32_t* cached_idx,
                                int ld_cached, int32_t* cached_len, int B, int H, int G, int N,
                                int dtype, void* stream_v) {
    float* ws = nullptr;
    const int st = scratch_address(static_cast<hipStream_t>(stream_v), &ws);
    if (st != MAR_OK) return st;
    return launch_refresh_topk(q_gen, k_full, gp_idx, ld_gp, n_gp, K, scale, scores, active_idx,
                               ld_act, cached_idx, ld_cached, cached_len, ws, B, H, G, N, dtype,
                               stream_v);
}

}  // namespace marca
