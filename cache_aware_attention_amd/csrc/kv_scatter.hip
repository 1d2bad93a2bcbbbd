// kv_scatter.hip -- KV cache update for KV-cached MAR decoding on gfx950.
//
// Partial update: the freshly projected K/V rows of the active tokens are
// written into the per-layer cache at their token positions (only tokens that
// were recomputed are updated -- "MARche" abstract on the Pith review page).
// Full refresh: on every third step the whole cache is rewritten ("MARche"
// paper-notes page, Key Design 3 and flowchart).
//
// Both are pure data movement: 16-byte vector loads/stores, every byte of
// the source read once and every destination byte written once.  The partial
// kernel assigns one thread per 16-byte piece of a (b, m, h) row pair, so a
// wave covers whole 128-byte rows (bf16, D = 64) and stays coalesced.
#include "device_util.h"
#include "launch.h"

namespace marca {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Threads = B * M * H * pieces (pieces = row_bytes / 16), K and V in the same
// thread.  Index order: piece fastest, then h, then m, then b.
__global__ __launch_bounds__(256) void scatter_rows_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const uint4* __restrict__ k_new,
    const uint4* __restrict__ v_new, const int32_t* __restrict__ idx, int ld_idx,
    int32_t* __restrict__ err_count, int H, int N, int M, int pieces, long long total) {
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const int piece = (int)(t % pieces);
    long long r = t / pieces;
    const int h = (int)(r % H);
    r /= H;
    const int m = (int)(r % M);
    const int b = (int)(r / M);
    const int j = idx[(size_t)b * ld_idx + m];
    if (j < 0 || j >= N) {
        if (err_count != nullptr && h == 0 && piece == 0) atomicAdd(err_count, 1);
        return;
    }
    const size_t src = (((size_t)b * H + h) * M + m) * pieces + piece;
    const size_t dst = (((size_t)b * H + h) * N + j) * pieces + piece;
    // Nontemporal stores: the rows are read again only at a later step, and
    // streaming them out now keeps their write-back out of the next kernel.
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, k_new[src]),
                                reinterpret_cast<u32x4_t*>(k_cache + dst));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v_new[src]),
                                reinterpret_cast<u32x4_t*>(v_cache + dst));
}

// Full rewrite: grid-stride copy of n16 16-byte pieces of both tensors, four
// pieces in flight per thread per iteration.
__global__ __launch_bounds__(256) void copy_full_kernel(uint4* __restrict__ k_cache,
                                                        uint4* __restrict__ v_cache,
                                                        const uint4* __restrict__ k_new,
                                                        const uint4* __restrict__ v_new,
                                                        long long n16) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 k0 = k_new[i], k1 = k_new[i + stride], k2 = k_new[i + 2 * stride],
                    k3 = k_new[i + 3 * stride];
        const uint4 v0 = v_new[i], v1 = v_new[i + stride], v2 = v_new[i + 2 * stride],
                    v3 = v_new[i + 3 * stride];
        k_cache[i] = k0;
        k_cache[i + stride] = k1;
        k_cache[i + 2 * stride] = k2;
        k_cache[i + 3 * stride] = k3;
        v_cache[i] = v0;
        v_cache[i + stride] = v1;
        v_cache[i + 2 * stride] = v2;
        v_cache[i + 3 * stride] = v3;
    }
    for (; i < n16; i += stride) {
        k_cache[i] = k_new[i];
        v_cache[i] = v_new[i];
    }
}

}  // namespace

int launch_kv_scatter(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int32_t* idx, int ld_idx, int32_t* err_count, int B, int H, int N,
                      int M, int row_bytes, void* stream_v) {
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    const int pieces = row_bytes / 16;
    uint4* kc = static_cast<uint4*>(k_cache);
    uint4* vc = static_cast<uint4*>(v_cache);
    const uint4* kn = static_cast<const uint4*>(k_new);
    const uint4* vn = static_cast<const uint4*>(v_new);
    if (idx == nullptr) {
        const long long n16 = (long long)B * H * N * pieces;
        // ~8 waves per CU of 256 CUs, each thread moving 4 pieces per pass
        long long blocks = (n16 + 256 * 4 - 1) / (256 * 4);
        if (blocks > 2048) blocks = 2048;
        if (blocks < 1) blocks = 1;
        hipLaunchKernelGGL(copy_full_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kc, vc,
                           kn, vn, n16);
        return status_from_launch();
    }
    const long long total = (long long)B * M * H * pieces;
    if (total == 0) return MAR_OK;
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kc, vc,
                       kn, vn, idx, ld_idx, err_count, H, N, M, pieces, total);
    return status_from_launch();
}

}  // namespace marca
