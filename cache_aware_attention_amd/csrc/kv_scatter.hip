// kv_scatter.hip -- KV cache update for KV-cached MAR decoding on gfx950.
//
// Partial update: the freshly projected K/V rows of the active tokens are
// written into the per-layer cache at their token positions (only tokens that
// were recomputed are updated -- "MARche" abstract on the Pith review page).
// Full refresh: on every third step the whole cache is rewritten ("MARche"
// paper-notes page, Key Design 3 and flowchart).
//
// Both are pure data movement: 16-byte streaming loads/stores, every byte of
// the source read once and every destination byte written once.  The partial
// kernel assigns one thread per 16-byte piece of a (b, m, h) row pair, so a
// wave covers whole 128-byte rows (bf16, D = 64) and stays coalesced.
#include "device_util.h"
#include "launch.h"

namespace marca {
namespace {

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
    st_stream(k_cache + dst, ld_stream(k_new + src));
    st_stream(v_cache + dst, ld_stream(v_new + src));
}

// Full rewrite: each wave copies contiguous groups of 4 KB of both tensors
// (four 1 KB pieces in flight per tensor), grid-stride over the groups, with
// streaming loads and stores (whole lines, read and written once); the tail
// below one group goes piece by piece.
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(256) void copy_full_kernel(uint4* __restrict__ k_cache,
                                                        uint4* __restrict__ v_cache,
                                                        const uint4* __restrict__ k_new,
                                                        const uint4* __restrict__ v_new,
                                                        long long n16) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const long long n_waves = (long long)gridDim.x * blockDim.x / kWave;
    constexpr long long kGroup = kCopyUnroll * kWave;  // pieces per group
    const long long n_groups = n16 / kGroup;
    for (long long gi = wave; gi < n_groups; gi += n_waves) {
        const long long base = gi * kGroup + lane;
        uint4 k[kCopyUnroll], v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            k[u] = ld_stream(k_new + base + u * kWave);
            v[u] = ld_stream(v_new + base + u * kWave);
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            st_stream(k_cache + base + u * kWave, k[u]);
            st_stream(v_cache + base + u * kWave, v[u]);
        }
    }
    const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (long long i = n_groups * kGroup + tid; i < n16; i += (long long)gridDim.x * blockDim.x) {
        st_stream(k_cache + i, ld_stream(k_new + i));
        st_stream(v_cache + i, ld_stream(v_new + i));
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
        // two waves per SIMD (512 workgroups of 4 waves), fewer for small copies
        long long blocks = (n16 + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
        if (blocks > 512) blocks = 512;
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
