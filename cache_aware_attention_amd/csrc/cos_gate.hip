// cos_gate.hip -- LazyMAR token gate on gfx950.
//
// "LazyMAR" paper-notes page, Key designs (token cache): past the first three
// layers, a token whose current feature is cosine-similar to the feature it
// had when its cached value was computed skips recomputation.  Kernel 1
// computes one cosine per token (a wave per token: 16-byte loads, float
// accumulation of <x,y>, |x|^2, |y|^2, butterfly reduction) and the reuse
// decision cos >= tau in float.  Kernel 2 (one workgroup per sequence) packs
// the positions to recompute in ascending order with a block prefix sum.
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
        const V a0 = xr[p], c0 = yr[p], a1 = xr[p + kWave], c1 = yr[p + kWave];
        acc_piece(a0, c0, xy, xx, yy);
        acc_piece(a1, c1, xy, xx, yy);
    }
    if (p < pieces) acc_piece(xr[p], yr[p], xy, xx, yy);
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

__global__ __launch_bounds__(kThreads) void compact_kernel(const uint8_t* __restrict__ reuse,
                                                           int32_t* __restrict__ compute_idx,
                                                           int32_t* __restrict__ compute_len,
                                                           int N) {
    __shared__ int scan_scratch[kThreads / kWave];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const uint8_t* r = reuse + (size_t)b * N;
    const int per = (N + kThreads - 1) / kThreads;
    const int j0 = tid * per;
    const int j1 = min(N, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += (r[j] == 0);
    int total = 0;
    int pos = block_exclusive_scan<kThreads>(cnt, scan_scratch, &total);
    int32_t* row = compute_idx + (size_t)b * N;
    for (int j = j0; j < j1; ++j)
        if (r[j] == 0) row[pos++] = j;
    for (int t = total + tid; t < N; t += kThreads) row[t] = -1;
    if (tid == 0) compute_len[b] = total;
}

}  // namespace

int launch_cos_gate(const void* x_cur, const void* x_cached, float tau, float eps,
                    float* cos_out, uint8_t* reuse_mask, int32_t* compute_idx,
                    int32_t* compute_len, int B, int N, int W, int dtype, void* stream_v) {
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    const long long tokens = (long long)B * N;
    const int waves_per_block = kThreads / kWave;
    const long long blocks = (tokens + waves_per_block - 1) / waves_per_block;
    if (dtype == MAR_BF16) {
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
                       compute_len, N);
    return status_from_launch();
}

}  // namespace marca
