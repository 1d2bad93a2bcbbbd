// cfg_residual.hip -- LazyMAR condition cache on gfx950.
//
// "LazyMAR" paper-notes page, Key designs (condition cache): the difference
// between the conditional and unconditional outputs changes little between
// adjacent steps, so a fully computed step stores residual = cond - uncond and
// a reuse step runs only the conditional branch and takes
// uncond = cond - residual.  Optionally the usual guidance mix
// u + w * (cond - u) is produced in the same pass.
//
// Elementwise float32, four elements per thread, each operation rounded on
// its own: contraction into fused multiply-adds is switched off for this
// file so the results are reproducible bit for bit.
#include "device_util.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace marca {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float guided_mix(float u, float c, float w) {
    const float d = c - u;
    const float wd = w * d;
    return u + wd;
}

__global__ __launch_bounds__(kThreads) void cfg_store_kernel(
    const float* __restrict__ cond, const float* __restrict__ uncond, float* __restrict__ residual,
    float* __restrict__ guided, float w, long long n) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    const long long n4 = n / 4;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 c = reinterpret_cast<const float4*>(cond)[i];
        const float4 u = reinterpret_cast<const float4*>(uncond)[i];
        reinterpret_cast<float4*>(residual)[i] = make_float4(c.x - u.x, c.y - u.y, c.z - u.z, c.w - u.w);
        if (guided != nullptr)
            reinterpret_cast<float4*>(guided)[i] =
                make_float4(guided_mix(u.x, c.x, w), guided_mix(u.y, c.y, w),
                            guided_mix(u.z, c.z, w), guided_mix(u.w, c.w, w));
    }
    for (long long i = n4 * 4 + (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        residual[i] = cond[i] - uncond[i];
        if (guided != nullptr) guided[i] = guided_mix(uncond[i], cond[i], w);
    }
}

__global__ __launch_bounds__(kThreads) void cfg_reuse_kernel(
    const float* __restrict__ cond, const float* __restrict__ residual,
    float* __restrict__ uncond_out, float* __restrict__ guided, float w, long long n) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    const long long n4 = n / 4;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 c = reinterpret_cast<const float4*>(cond)[i];
        const float4 r = reinterpret_cast<const float4*>(residual)[i];
        const float4 u = make_float4(c.x - r.x, c.y - r.y, c.z - r.z, c.w - r.w);
        reinterpret_cast<float4*>(uncond_out)[i] = u;
        if (guided != nullptr)
            reinterpret_cast<float4*>(guided)[i] =
                make_float4(guided_mix(u.x, c.x, w), guided_mix(u.y, c.y, w),
                            guided_mix(u.z, c.z, w), guided_mix(u.w, c.w, w));
    }
    for (long long i = n4 * 4 + (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float u = cond[i] - residual[i];
        uncond_out[i] = u;
        if (guided != nullptr) guided[i] = guided_mix(u, cond[i], w);
    }
}

}  // namespace

int launch_cfg_residual(const float* cond, const float* uncond, float* residual,
                        float* uncond_out, float* guided_out, float cfg_scale, int mode,
                        int64_t n, void* stream_v) {
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    if (n == 0) return MAR_OK;
    long long blocks = (n / 4 + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    if (mode == MAR_CFG_STORE)
        hipLaunchKernelGGL(cfg_store_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           cond, uncond, residual, guided_out, cfg_scale, (long long)n);
    else
        hipLaunchKernelGGL(cfg_reuse_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           cond, residual, uncond_out, guided_out, cfg_scale, (long long)n);
    return status_from_launch();
}

}  // namespace marca
