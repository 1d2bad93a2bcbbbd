// device_util.h -- small device helpers shared by the HIP kernels of libmarca
// (bf16 conversion, 64-lane wave reductions, prefix scans, streaming loads,
// the whole-row / MFMA-operand exchange).  gfx950 only.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "mar_cache_attn.h"

namespace marca {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
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

// The number of compute units of the device `stream` runs on (the current
// device for the null stream), asked once per device and kept.
inline int compute_units(hipStream_t stream, int* cus) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> known[kMaxDev];
    int dev = 0;
    if ((stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) {
        (void)hipGetLastError();
        return MAR_E_LAUNCH;
    }
    int n = (dev >= 0 && dev < kMaxDev) ? known[dev].load(std::memory_order_relaxed) : 0;
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            return MAR_E_LAUNCH;
        }
        if (dev >= 0 && dev < kMaxDev) known[dev].store(n, std::memory_order_relaxed);
    }
    *cus = n;
    return MAR_OK;
}

// Streaming 16-byte load (nontemporal: the line is not kept for reuse).  On
// this chip such loads sustain more HBM read bandwidth than plain loads for
// data that is read once, as every K/V row of the attention is.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 ld_stream(const float4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
}
// Streaming 16-byte store (nontemporal).
__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
}
// Cache-policy bits of a streaming (nontemporal) buffer load or store.
constexpr int kStreamPolicy = 2;

// Buffer resource over `bytes` bytes at p (raw buffer, range-checked: an
// offset at or past `bytes` reads zero / drops the store).  p and bytes are
// wave-uniform; taking them through readfirstlane keeps the descriptor in
// scalar registers.  A pointer the compiler also holds in vector registers
// (for per-lane address selects) would otherwise make every buffer access a
// readfirstlane loop behind a wait for all outstanding loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    void* q = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Two layouts of 16 rows x 128 bytes held in two 16-byte registers per lane
// (lane (g, m16): g = lane / 16, m16 = lane % 16):
//  * operand layout (A/B operand of v_mfma_f32_16x16x32_bf16 over 64 head
//    dims): x0 = piece g and x1 = piece 4 + g of row m16;
//  * whole-row layout: r_h = piece (m16 < 8 ? g : 4 + g) of row 8h + m16 % 8,
//    so one register of the 64 lanes covers 8 complete rows.
// A load or store of whole rows moves complete 128-byte lines (a streaming
// load of half-rows fetches each line twice).  Each direction exchanges the
// upper 8 lanes' first register with the lower 8 lanes' second one within
// each 16-lane row: two DPP row shifts by 8 per dword, under bank masks.
__device__ __forceinline__ void swap_row_halves(uint4 a, uint4 b, uint4& x, uint4& y) {
    const u32x4_t a4 = __builtin_bit_cast(u32x4_t, a);
    const u32x4_t b4 = __builtin_bit_cast(u32x4_t, b);
    u32x4_t xo, yo;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        // lanes 8..15 of each row take b of lane - 8; lanes 0..7 keep a
        xo[d] = __builtin_amdgcn_update_dpp(a4[d], b4[d], 0x118, 0xf, 0xc, false);
        // lanes 0..7 take a of lane + 8; lanes 8..15 keep b
        yo[d] = __builtin_amdgcn_update_dpp(b4[d], a4[d], 0x108, 0xf, 0x3, false);
    }
    x = __builtin_bit_cast(uint4, xo);
    y = __builtin_bit_cast(uint4, yo);
}

}  // namespace marca
