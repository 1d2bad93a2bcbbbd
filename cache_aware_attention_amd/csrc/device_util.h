// device_util.h -- small device helpers shared by the HIP kernels of libmarca
// (bf16 conversion, 64-lane wave reductions, prefix scans).  gfx950 only.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "mar_cache_attn.h"

namespace marca {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bfloat16 <-> float.  Widening is exact; narrowing uses gfx950's
// v_cvt_pk_bf16_f32 (round to nearest even, NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Two floats -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return static_cast<uint16_t>(pack_bf16x2(f, 0.f) & 0xffffu);
}

// Reductions over the 64 lanes of a wave, register-only: DPP steps within
// 16-lane rows (quad xor 1, quad xor 2, half-row mirror, row mirror), then
// gfx950's row swaps (permlane16 / permlane32).  Every lane ends with the
// same bits, and the combination order is fixed, so results are
// deterministic.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = op(v, dpp_mov<0xb1>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_mov<0x4e>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_mov<0x141>(v));  // row_half_mirror
    v = op(v, dpp_mov<0x140>(v));  // row_mirror
    const uint32_t u = __float_as_uint(v);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(v);
    auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// Exclusive prefix sum of one int per thread over a block of kThreads
// threads (multiple of 64).  `scratch` holds kThreads/64 ints of LDS.
// Returns the exclusive prefix; *total receives the block sum.
template <int kThreads>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) scratch[wid] = incl;
    __syncthreads();
    int wave_off = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        int s = scratch[w];
        if (w < wid) wave_off += s;
        sum += s;
    }
    __syncthreads();
    *total = sum;
    return wave_off + incl - v;
}

inline int status_from_launch() {
    return hipGetLastError() == hipSuccess ? MAR_OK : MAR_E_LAUNCH;
}

}  // namespace marca
