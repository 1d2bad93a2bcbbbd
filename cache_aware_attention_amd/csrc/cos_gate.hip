// cos_gate.hip -- LazyMAR token gate on gfx950.
//
// "LazyMAR" paper-notes page, Key designs (token cache): past the first three
// layers, a token whose current feature is cosine-similar to the feature it
// had when its cached value was computed skips recomputation.  Kernel 1
// computes one cosine per token (16-byte streaming loads, float accumulation of <x,y>,
// |x|^2, |y|^2 per lane, then a wave reduction) and the reuse decision
// cos >= tau in float: several tokens per wave with all their loads in
// flight for widths up to 256 pieces of 16 bytes, one token per wave above.
// Kernel 2 (one workgroup per sequence) packs the positions to recompute in
// ascending order with a block prefix sum, and optionally the positions that
// reuse (every position before a thread's range that is not recomputed
// reuses, so one scan places both lists).
#include "device_util.h"
#include "launch.h"

namespace marca {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void acc_piece(uint4 a, uint4 c, float& xy, float& xx, float& yy) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
    const uint32_t wc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float x0 = __uint_as_float(wa[k] << 16), x1 = __uint_as_float(wa[k] & 0xffff0000u);
        const float y0 = __uint_as_float(wc[k] << 16), y1 = __uint_as_float(wc[k] & 0xffff0000u);
        xy = fmaf(x0, y0, xy); xy = fmaf(x1, y1, xy);
        xx = fmaf(x0, x0, xx); xx = fmaf(x1, x1, xx);
        yy = fmaf(y0, y0, yy); yy = fmaf(y1, y1, yy);
    }
}
__device__ __forceinline__ void acc_piece(float4 a, float4 c, float& xy, float& xx, float& yy) {
    xy = fmaf(a.x, c.x, xy); xy = fmaf(a.y, c.y, xy); xy = fmaf(a.z, c.z, xy); xy = fmaf(a.w, c.w, xy);
    xx = fmaf(a.x, a.x, xx); xx = fmaf(a.y, a.y, xx); xx = fmaf(a.z, a.z, xx); xx = fmaf(a.w, a.w, xx);
    yy = fmaf(c.x, c.x, yy); yy = fmaf(c.y, c.y, yy); yy = fmaf(c.z, c.z, yy); yy = fmaf(c.w, c.w, yy);
}

// One wave per token; V is the 16-byte vector type of the element type.
template <typename V>
__global__ __launch_bounds__(kThreads) void cosine_kernel(const V* __restrict__ x,
                                                          const V* __restrict__ y,
                                                          float* __restrict__ cos_out,
                                                          uint8_t* __restrict__ reuse,
                                                          long long tokens, int pieces, float tau,
                                                          float eps) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long t = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    if (t >= tokens) return;  // wave-uniform
    const V* xr = x + (size_t)t * pieces;
    const V* yr = y + (size_t)t * pieces;
    float xy = 0.f, xx = 0.f, yy = 0.f;
    int p = lane;
    for (; p + kWave < pieces; p += 2 * kWave) {
        const V a0 = ld_stream(xr + p), c0 = ld_stream(yr + p), a1 = ld_stream(xr + p + kWave),
                c1 = ld_stream(yr + p + kWave);
        acc_piece(a0, c0, xy, xx, yy);
        acc_piece(a1, c1, xy, xx, yy);
    }
    if (p < pieces) acc_piece(ld_stream(xr + p), ld_stream(yr + p), xy, xx, yy);
    xy = wave_sum(xy);
    xx = wave_sum(xx);
    yy = wave_sum(yy);
    if (lane == 0) {
        const float den = fmaxf(sqrtf(xx) * sqrtf(yy), eps);
        const float c = xy / den;
        cos_out[t] = c;
        reuse[t] = (c >= tau) ? 1 : 0;
    }
}

// Several tokens per wave: kTPW tokens, kPPL 16-byte pieces per lane per
// vector (pieces = W / elements-per-piece <= 64 * kPPL).  All loads of the
// wave's tokens are issued before any arithmetic, so a wave keeps
// 2 * kTPW * kPPL loads in flight; reductions stay in registers (DPP and
// row swaps).  A token past the end reads the last token and is not stored.
template <typename V, int kTPW, int kPPL>
__global__ __launch_bounds__(kThreads) void cosine_multi_kernel(
    const V* __restrict__ x, const V* __restrict__ y, float* __restrict__ cos_out,
    uint8_t* __restrict__ reuse, long long tokens, int pieces, float tau, float eps) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long t0 =
        ((long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave) * kTPW;
    if (t0 >= tokens) return;  // wave-uniform
    V xa[kTPW][kPPL], ya[kTPW][kPPL];
#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
        const long long t = (t0 + k < tokens) ? t0 + k : tokens - 1;
        const V* xr = x + (size_t)t * pieces;
        const V* yr = y + (size_t)t * pieces;
#pragma unroll
        for (int i = 0; i < kPPL; ++i) {
            const int p = lane + kWave * i;
            const int pc = (p < pieces) ? p : 0;  // lanes past the row reload piece 0 (unused)
            xa[k][i] = ld_stream(xr + pc);
            ya[k][i] = ld_stream(yr + pc);
        }
    }
    float xy[kTPW], xx[kTPW], yy[kTPW];
#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
        xy[k] = 0.f;
        xx[k] = 0.f;
        yy[k] = 0.f;
#pragma unroll
        for (int i = 0; i < kPPL; ++i)
            if (lane + kWave * i < pieces) acc_piece(xa[k][i], ya[k][i], xy[k], xx[k], yy[k]);
    }
#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
        const float sxy = wave_sum(xy[k]);
        const float sxx = wave_sum(xx[k]);
        const float syy = wave_sum(yy[k]);
        if (lane == k && t0 + k < tokens) {
            const float den = fmaxf(sqrtf(sxx) * sqrtf(syy), eps);
            const float c = sxy / den;
            cos_out[t0 + k] = c;
            reuse[t0 + k] = (c >= tau) ? 1 : 0;
        }
    }
}

template <typename V, int kTPW>
void launch_cosine_multi(const void* x, const void* y, float* cos_out, uint8_t* reuse,
                         long long tokens, int pieces, float tau, float eps, hipStream_t stream) {
    const long long waves = (tokens + kTPW - 1) / kTPW;
    const long long blocks = (waves + kThreads / kWave - 1) / (kThreads / kWave);
    const V* xv = static_cast<const V*>(x);
    const V* yv = static_cast<const V*>(y);
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch ((pieces + kWave - 1) / kWave) {
        case 1: hipLaunchKernelGGL((cosine_multi_kernel<V, kTPW, 1>), grid, block, 0, stream, xv, yv, cos_out, reuse, tokens, pieces, tau, eps); break;
        case 2: hipLaunchKernelGGL((cosine_multi_kernel<V, kTPW, 2>), grid, block, 0, stream, xv, yv, cos_out, reuse, tokens, pieces, tau, eps); break;
        case 3: hipLaunchKernelGGL((cosine_multi_kernel<V, kTPW, 3>), grid, block, 0, stream, xv, yv, cos_out, reuse, tokens, pieces, tau, eps); break;
        default: hipLaunchKernelGGL((cosine_multi_kernel<V, kTPW, 4>), grid, block, 0, stream, xv, yv, cos_out, reuse, tokens, pieces, tau, eps); break;
    }
}

__global__ __launch_bounds__(kThreads) void compact_kernel(const uint8_t* __restrict__ reuse,
                                                           int32_t* __restrict__ compute_idx,
                                                           int32_t* __restrict__ compute_len,
                                                           int32_t* __restrict__ reuse_idx,
                                                           int32_t* __restrict__ reuse_len,
                                                           int N) {
    __shared__ int scan_scratch[kThreads / kWave];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const uint8_t* r = reuse + (size_t)b * N;
    const int per = (N + kThreads - 1) / kThreads;
    const int j0 = min(N, tid * per);
    const int j1 = min(N, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += (r[j] == 0);
    int total = 0;
    int pos = block_exclusive_scan<kThreads>(cnt, scan_scratch, &total);
    int pos_r = j0 - pos;  // the reusing positions before j0
    int32_t* row = compute_idx + (size_t)b * N;
    int32_t* rrow = reuse_idx != nullptr ? reuse_idx + (size_t)b * N : nullptr;
    for (int j = j0; j < j1; ++j) {
        if (r[j] == 0)
            row[pos++] = j;
        else if (rrow != nullptr)
            rrow[pos_r++] = j;
    }
    for (int t = total + tid; t < N; t += kThreads) row[t] = -1;
    if (rrow != nullptr)
        for (int t = N - total + tid; t < N; t += kThreads) rrow[t] = -1;
    if (tid == 0) {
        compute_len[b] = total;
        if (reuse_len != nullptr) reuse_len[b] = N - total;
    }
}

}  // namespace

int launch_cos_gate(const void* x_cur, const void* x_cached, float tau, float eps,
                    float* cos_out, uint8_t* reuse_mask, int32_t* compute_idx,
                    int32_t* compute_len, int32_t* reuse_idx, int32_t* reuse_len, int B, int N,
                    int W, int dtype, void* stream_v) {
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    const long long tokens = (long long)B * N;
    const int waves_per_block = kThreads / kWave;
    const long long blocks = (tokens + waves_per_block - 1) / waves_per_block;
    const int pieces = (dtype == MAR_BF16) ? W / 8 : W / 4;  // 16-byte pieces per token
    if (pieces <= 4 * kWave) {
        if (dtype == MAR_BF16)
            launch_cosine_multi<uint4, 4>(x_cur, x_cached, cos_out, reuse_mask, tokens, pieces,
                                          tau, eps, stream);
        else
            launch_cosine_multi<float4, 2>(x_cur, x_cached, cos_out, reuse_mask, tokens, pieces,
                                           tau, eps, stream);
    } else if (dtype == MAR_BF16) {
        hipLaunchKernelGGL(cosine_kernel<uint4>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           static_cast<const uint4*>(x_cur), static_cast<const uint4*>(x_cached),
                           cos_out, reuse_mask, tokens, W / 8, tau, eps);
    } else {
        hipLaunchKernelGGL(cosine_kernel<float4>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, static_cast<const float4*>(x_cur),
                           static_cast<const float4*>(x_cached), cos_out, reuse_mask, tokens,
                           W / 4, tau, eps);
    }
    int st = status_from_launch();
    if (st != MAR_OK) return st;
    hipLaunchKernelGGL(compact_kernel, dim3(B), dim3(kThreads), 0, stream, reuse_mask, compute_idx,
                       compute_len, reuse_idx, reuse_len, N);
    return status_from_launch();
}

}  // namespace marca
