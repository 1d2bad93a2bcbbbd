// bench_kernels.hip -- measurement kernels of libmarca_bench.  They are not
// part of the decoding path; the benchmark uses them to put the cache-aware
// attention's time in context.
//
//  * attn_pattern_kernel: the memory operations of the one-wave cache-aware
//    attention kernel (A <= 64 queries per unit) with an XOR fold in place of
//    its arithmetic: the unit's cached list staged in LDS (entries outside
//    [0, N) become missing rows), Q read as whole 128-byte rows, the virtual
//    sequence [A active rows ; Nc cached rows] read in 32-row chunks as whole
//    rows with streaming loads (four row lookups per chunk, the same chunks in
//    flight as the attention), and -- with WRITE -- the A output rows written
//    with streaming stores.  Its time is the floor of that access pattern.
//  * concat_rows_kernel: the concatenation that standard attention needs
//    before it can attend over the active and the cached tokens ("MARche"
//    paper-notes page, Key Design 2: the standard way concatenates the stored
//    and the fresh keys and values; the Pith review page, figure 7: runtime of
//    standard versus cache-aware attention).  Row r of the output is active
//    row r for r < A and cached row cached_idx[r - A] after that.
//  * the full-attention kernel of the decoding path (attn_dense.h) in its two
//    measurement modes: its arithmetic alone (every global load past the
//    buffer, no memory traffic, no output) and its memory operations alone
//    (no per-chunk math): the two floors that bound the full-attention layer.
#include <type_traits>

#include "attn_cached.h"
#include "device_util.h"
#include "mar_bench.h"

namespace marca {
namespace {

template <bool WRITE, int NQT>
__global__ __launch_bounds__(64) void attn_pattern_kernel(
    const uint16_t* __restrict__ q_a, const uint16_t* __restrict__ k_a,
    const uint16_t* __restrict__ v_a, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ cached_idx, int ldc,
    uint16_t* __restrict__ out, int H, int N, int A, int Nc) {
    constexpr int kPF = NQT <= 3 ? 2 : 1;  // chunks in flight, as in the attention
    extern __shared__ int32_t list_s[];     // [max(Nc, 1)]
    const int lane = threadIdx.x;
    const int g = lane >> 4, m16 = lane & 15;
    const int kpiece = (m16 < 8) ? g : 4 + g;
    const int u = blockIdx.x;
    const int32_t* cl = cached_idx + static_cast<size_t>(u / H) * ldc;
    for (int c = lane; c < Nc; c += kWave) {
        const int n = cl[c];
        list_s[c] = (n >= 0 && n < N) ? n : -1;
    }
    __syncthreads();  // one wave: orders the list writes before the reads
    const uint16_t* ka = k_a + static_cast<size_t>(u) * A * kD;
    const uint16_t* va = v_a + static_cast<size_t>(u) * A * kD;
    const uint16_t* kc = k_cache + static_cast<size_t>(u) * N * kD;
    const uint16_t* vc = v_cache + static_cast<size_t>(u) * N * kD;
    uint32_t fold = 0;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int qi = min(16 * qt + 8 * h + (m16 & 7), A - 1);
            const uint4 q = ld_stream(reinterpret_cast<const uint4*>(
                                          q_a + (static_cast<size_t>(u) * A + qi) * kD) + kpiece);
            fold ^= q.x ^ q.w;
        }
    const int T = A + Nc;
    const int nchunks = (T + kChunk - 1) / kChunk;
    // Row r of [active ; cached]: missing rows (past T, skipped entries) read
    // active row 0, as in the attention.
    auto issue = [&](int c, uint4 (&kk)[4], uint4 (&vv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = min(c, nchunks) * kChunk + 8 * k + (m16 & 7);
            const int j = r - A;
            const int n = (j >= 0 && j < Nc) ? list_s[j] : -1;
            const bool cached = n >= 0;
            const int ofs = (cached ? n : (r < A ? r : 0)) * kD + 8 * kpiece;
            vv[k] = ld_stream(reinterpret_cast<const uint4*>((cached ? vc : va) + ofs));
            kk[k] = ld_stream(reinterpret_cast<const uint4*>((cached ? kc : ka) + ofs));
        }
    };
    auto eat = [&](const uint4 (&kk)[4], const uint4 (&vv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) fold ^= kk[k].x ^ kk[k].w ^ vv[k].y ^ vv[k].z;
    };
    uint4 kb[kPF + 1][4], vb[kPF + 1][4];
#pragma unroll
    for (int i = 0; i < kPF; ++i) issue(i, kb[i], vb[i]);
    // Chunk c sits in buffer c % (kPF + 1); every step requests a chunk
    // (past the end: missing rows), as the attention does.
    int c = 0;
    for (; c + kPF < nchunks; c += kPF + 1) {
#pragma unroll
        for (int i = 0; i <= kPF; ++i) {
            issue(c + i + kPF, kb[(i + kPF) % (kPF + 1)], vb[(i + kPF) % (kPF + 1)]);
            eat(kb[i], vb[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < kPF; ++i)
        if (c + i < nchunks) eat(kb[i], vb[i]);
    if constexpr (WRITE) {
        u32x4_t w = {fold, fold ^ 1u, fold ^ 2u, fold ^ 3u};
        u32x4_t* orow = reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(u) * A * kD);
#pragma unroll
        for (int k = 0; k < 2 * NQT; ++k) {
            const int row = 8 * k + (lane >> 3);
            if (row < A) __builtin_nontemporal_store(w, orow + row * 8 + (lane & 7));
        }
    } else if (fold == 0x9e3779b9u) {
        out[static_cast<size_t>(u) * A * kD] = 1;  // keeps the loads; practically never taken
    }
}

// One thread per 16-byte piece of an output row, K and V together.  Index
// order: piece fastest, then the row r of T = A + Nc, then the unit.
__global__ __launch_bounds__(256) void concat_rows_kernel(
    uint4* __restrict__ k_cat, uint4* __restrict__ v_cat, const uint4* __restrict__ k_a,
    const uint4* __restrict__ v_a, const uint4* __restrict__ k_cache,
    const uint4* __restrict__ v_cache, const int32_t* __restrict__ cached_idx, int ldc, int H,
    int N, int A, int Nc, int pieces, long long total) {
    const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const int piece = static_cast<int>(t % pieces);
    long long rest = t / pieces;
    const int T = A + Nc;
    const int r = static_cast<int>(rest % T);
    const long long u = rest / T;
    const size_t dst = (static_cast<size_t>(u) * T + r) * pieces + piece;
    if (r < A) {
        const size_t src = (static_cast<size_t>(u) * A + r) * pieces + piece;
        st_stream(k_cat + dst, ld_stream(k_a + src));
        st_stream(v_cat + dst, ld_stream(v_a + src));
        return;
    }
    const int n = cached_idx[static_cast<size_t>(u / H) * ldc + (r - A)];
    if (n < 0 || n >= N) return;  // skipped entry: the row is left as it was
    const size_t src = (static_cast<size_t>(u) * N + n) * pieces + piece;
    st_stream(k_cat + dst, ld_stream(k_cache + src));
    st_stream(v_cat + dst, ld_stream(v_cache + src));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace marca

extern "C" int mar_bench_attn_pattern(const void* q_a, const void* k_a, const void* v_a,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* cached_idx, int ldc, void* out,
                                      int write_out, int B, int H, int N, int A, int Nc, int D,
                                      int dtype, void* stream) {
    using namespace marca;
    if (!q_a || !k_a || !v_a || !k_cache || !v_cache || !out) return MAR_E_NULL;
    if (Nc > 0 && !cached_idx) return MAR_E_NULL;
    if (dtype != MAR_BF16) return MAR_E_UNSUPPORTED;
    if (B < 1 || H < 1 || N < 1 || A < 1 || Nc < 0 || (long long)A + Nc > N) return MAR_E_SHAPE;
    if (Nc > 0 && ldc < Nc) return MAR_E_SHAPE;
    if (D != kD || A > 64 || Nc > 8192) return MAR_E_UNSUPPORTED;
    if (!aligned16(q_a) || !aligned16(k_a) || !aligned16(v_a) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return MAR_E_RANGE;
    const size_t lds = static_cast<size_t>(Nc > 0 ? Nc : 1) * 4;
    const dim3 grid(B * H), block(64);
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto q = static_cast<const uint16_t*>(q_a);
    auto ka = static_cast<const uint16_t*>(k_a);
    auto va = static_cast<const uint16_t*>(v_a);
    auto kc = static_cast<const uint16_t*>(k_cache);
    auto vc = static_cast<const uint16_t*>(v_cache);
    auto o = static_cast<uint16_t*>(out);
    auto go = [&](auto w_tag, auto nqt_tag) {
        constexpr bool W = decltype(w_tag)::value;
        constexpr int Q = decltype(nqt_tag)::value;
        hipLaunchKernelGGL((attn_pattern_kernel<W, Q>), grid, block, lds, s, q, ka, va, kc, vc,
                           cached_idx, ldc, o, H, N, A, Nc);
    };
    using T1 = std::true_type;
    using F0 = std::false_type;
    const int nqt = (A + 15) / 16;
    switch (nqt) {
        case 1: write_out ? go(T1{}, std::integral_constant<int, 1>{}) : go(F0{}, std::integral_constant<int, 1>{}); break;
        case 2: write_out ? go(T1{}, std::integral_constant<int, 2>{}) : go(F0{}, std::integral_constant<int, 2>{}); break;
        case 3: write_out ? go(T1{}, std::integral_constant<int, 3>{}) : go(F0{}, std::integral_constant<int, 3>{}); break;
        default: write_out ? go(T1{}, std::integral_constant<int, 4>{}) : go(F0{}, std::integral_constant<int, 4>{}); break;
    }
    return status_from_launch();
}

extern "C" int mar_bench_kv_concat(void* k_cat, void* v_cat, const void* k_a, const void* v_a,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* cached_idx, int ldc, int B, int H, int N, int A,
                                   int Nc, int D, int dtype, void* stream) {
    using namespace marca;
    if (!k_cat || !v_cat || !k_a || !v_a || !k_cache || !v_cache) return MAR_E_NULL;
    if (Nc > 0 && !cached_idx) return MAR_E_NULL;
    const int eb = dtype == MAR_BF16 ? 2 : (dtype == MAR_F32 ? 4 : 0);
    if (eb == 0) return MAR_E_DTYPE;
    if (B < 1 || H < 1 || N < 1 || A < 0 || Nc < 0 || D < 1) return MAR_E_SHAPE;
    if (Nc > 0 && ldc < Nc) return MAR_E_SHAPE;
    if ((D * eb) % 16 != 0) return MAR_E_UNSUPPORTED;
    if (!aligned16(k_cat) || !aligned16(v_cat) || !aligned16(k_a) || !aligned16(v_a) ||
        !aligned16(k_cache) || !aligned16(v_cache))
        return MAR_E_RANGE;
    const int pieces = D * eb / 16;
    const long long total = static_cast<long long>(B) * H * (A + Nc) * pieces;
    if (total == 0) return MAR_OK;
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(concat_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cat),
                       static_cast<uint4*>(v_cat), static_cast<const uint4*>(k_a),
                       static_cast<const uint4*>(v_a), static_cast<const uint4*>(k_cache),
                       static_cast<const uint4*>(v_cache), cached_idx, ldc, H, N, A, Nc, pieces,
                       total);
    return status_from_launch();
}

extern "C" int mar_bench_dense_floor(const void* q, const void* k, const void* v,
                                     void* k_cache, void* v_cache, void* out, int mode, int B,
                                     int H, int N, int D, int dtype, void* stream) {
    using namespace marca;
    if (!q || !k || !v || !out) return MAR_E_NULL;
    if ((k_cache == nullptr) != (v_cache == nullptr)) return MAR_E_NULL;
    const bool update = k_cache != nullptr;
    if (dtype != MAR_BF16) return MAR_E_UNSUPPORTED;
    if (B < 1 || H < 1 || N < 1) return MAR_E_SHAPE;
    if (D != kD || N <= 64 || N > 8192) return MAR_E_UNSUPPORTED;
    if (mode != MAR_BENCH_FLOOR_ARITH && mode != MAR_BENCH_FLOOR_MEMORY) return MAR_E_RANGE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MAR_E_RANGE;
    if (update && (!aligned16(k_cache) || !aligned16(v_cache))) return MAR_E_RANGE;
    auto qq = static_cast<const uint16_t*>(q);
    auto kk = static_cast<const uint16_t*>(k);
    auto vv = static_cast<const uint16_t*>(v);
    auto o = static_cast<uint16_t*>(out);
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto kc = static_cast<uint16_t*>(k_cache);
    auto vc = static_cast<uint16_t*>(v_cache);
    const float scale_log2 = 0.125f * 1.4426950408889634f;
    if (mode == MAR_BENCH_FLOOR_ARITH)
        return update ? launch_dense_wg<true, kLabArith>(qq, kk, vv, kc, vc, o, nullptr, B, H, N,
                                                         scale_log2, s)
                      : launch_dense_wg<false, kLabArith>(qq, kk, vv, nullptr, nullptr, o, nullptr,
                                                          B, H, N, scale_log2, s);
    return update ? launch_dense_wg<true, kLabMemory>(qq, kk, vv, kc, vc, o, nullptr, B, H, N,
                                                      scale_log2, s)
                  : launch_dense_wg<false, kLabMemory>(qq, kk, vv, nullptr, nullptr, o, nullptr, B,
                                                       H, N, scale_log2, s);
}

extern "C" int mar_bench_cached_floor(const void* q_a, const void* k_a, const void* v_a,
                                      void* k_cache, void* v_cache, const int32_t* cached_idx,
                                      int ldc, const int32_t* active_idx, int ld_act,
                                      const int32_t* a_len, const int32_t* c_len, void* out,
                                      int mode, int B, int H, int N, int A, int Nc, int D,
                                      int dtype, void* stream) {
    using namespace marca;
    if (!q_a || !k_a || !v_a || !k_cache || !v_cache || !cached_idx || !out) return MAR_E_NULL;
    if ((a_len == nullptr) != (c_len == nullptr)) return MAR_E_NULL;
    const bool ragged = a_len != nullptr;
    const bool update = active_idx != nullptr;
    if (ragged != update) return MAR_E_UNSUPPORTED;  // the two forms the decoding path runs
    if (dtype != MAR_BF16) return MAR_E_UNSUPPORTED;
    if (B < 1 || H < 1 || N < 1 || A < 1 || Nc < 1) return MAR_E_SHAPE;
    // per-sequence counts: A and Nc are capacities, each at most N
    if (ragged ? (A > N || Nc > N) : (static_cast<long long>(A) + Nc > N)) return MAR_E_SHAPE;
    if (ldc < Nc || (update && ld_act < A)) return MAR_E_SHAPE;
    if (D != kD || A <= 64 || N > 8192) return MAR_E_UNSUPPORTED;
    if (cached_wg_lds(update, A, Nc) > kCachedWgMaxLds) return MAR_E_UNSUPPORTED;
    if (mode != MAR_BENCH_FLOOR_ARITH && mode != MAR_BENCH_FLOOR_MEMORY) return MAR_E_RANGE;
    if (!aligned16(q_a) || !aligned16(k_a) || !aligned16(v_a) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return MAR_E_RANGE;
    auto q = static_cast<const uint16_t*>(q_a);
    auto k = static_cast<const uint16_t*>(k_a);
    auto v = static_cast<const uint16_t*>(v_a);
    auto kc = static_cast<const uint16_t*>(k_cache);
    auto vc = static_cast<const uint16_t*>(v_cache);
    auto o = static_cast<uint16_t*>(out);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale_log2 = 0.125f * 1.4426950408889634f;
    auto go = [&](auto lab_tag) {
        constexpr int kLab = decltype(lab_tag)::value;
        return update ? launch_cached_wg<true, true, kLab>(q, k, v, kc, vc, cached_idx, ldc, o,
                                                            nullptr, B, H, N, A, Nc, scale_log2,
                                                            active_idx, ld_act, nullptr, a_len,
                                                            c_len, s)
                      : launch_cached_wg<false, false, kLab>(q, k, v, kc, vc, cached_idx, ldc, o,
                                                              nullptr, B, H, N, A, Nc, scale_log2,
                                                              nullptr, 0, nullptr, nullptr,
                                                              nullptr, s);
    };
    return mode == MAR_BENCH_FLOOR_ARITH ? go(std::integral_constant<int, kLabArith>{})
                                         : go(std::integral_constant<int, kLabMemory>{});
}
