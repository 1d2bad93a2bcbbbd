// attn_dense.h -- the per-chunk tile math of the workgroup attention kernels
// and the full-attention kernel built on it (gfx950).
//
// Operation ("MARche" paper-notes page, Key Design 2, Eq. 1-2, and Key
// Design 3: layers 1-2 and every layer of a refresh step attend over all
// tokens): softmax attention of each query over the keys/values of its
// (sequence, head) unit, streamed in 32-row chunks through one running
// (max, sum, weighted sum) state.  cache_attn.hip builds the decoding path's
// kernels from this file (the cache-aware workgroup kernel shares wg_chunk);
// the measurement library instantiates the full-attention kernel's
// measurement modes (LAB below) to time its arithmetic and its memory traffic
// apart.
#pragma once

#include <algorithm>
#include <type_traits>

#include "device_util.h"

namespace marca {
namespace {

constexpr int kD = 64;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kChunk = 32;          // key rows per chunk (two 16-row MFMA tiles)
// A query's reference maximum is raised (and its state rescaled) only when a
// score passes it by more than this many log2 units, so probabilities stay
// at most 2^kRescaleLog2.
constexpr float kRescaleLog2 = 8.f;

union U4 {
    uint4 u;
    bf16x8_t v;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) {
    U4 t;
    t.u = x;
    return t.v;
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_t;

// Byte offset of logical 16-byte piece `piece` of 128-byte row r in a
// swizzled LDS tile.
__device__ __forceinline__ int swz(int r, int piece) { return r * 128 + ((piece ^ (r & 7)) << 4); }

// Transposing 8-byte LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lane i receives element (i mod 4) of the 8-byte chunk addressed by
// lane 4e + i/4 of the group, for e = 0..3.
__device__ __forceinline__ uint2 lds_tr_b64(const unsigned char* p) {
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(p));
    return __builtin_bit_cast(uint2, v);
}

// Maximum over lanes l, l^16, l^32, l^48 (register-only lane swaps).
__device__ __forceinline__ float max_over_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(x);
    auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr int kWgWaves = 4;
constexpr int kWgNqt = 5;
constexpr int kWgTile = kChunk * 128;  // bytes of one K or V chunk tile
constexpr int kHalfTile = kWgTile / 2;  // its rows 16..31

// The softmax state of a wave's NQT 16-query tiles in the workgroup kernels:
// the Q operands (B of S^T = K Q^T: lane holds query m16 of the tile, head
// dims [8g, 8g+8) and [32+8g, 32+8g+8)), each query's reference mc (the
// maximum of its scaled scores s * scale_log2 from the first chunk, raised by
// rescales), and the O^T and row-sum accumulators.
template <int NQT>
struct WgTiles {
    bf16x8_t qf[NQT][2];
    float mc[NQT];
    f32x4_t oacc[NQT][4], lacc[NQT];
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            mc[qt] = 0.f;
            lacc[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
};

// One 32-key chunk of the workgroup kernels for a wave's NQT query tiles: the
// K tile kt and V tile vt in LDS (swizzled rows), the lane's K operand and
// V^T transposing-read offsets kofs, vofs in the tile's first 16 rows (the
// same offsets plus kHalfTile address rows 16..31: the swizzle repeats every
// 8 rows).  kFull: every key row of the chunk
// exists; kFirst: chunk 0, which sets the references.  CACHED: rows is the
// chunk's row mask (bit k: row 32c + k exists); otherwise the rows at or past
// A are missing (only a partial last chunk has any).  NT: the tiles computed,
// the first NT of the wave's NQT (a wave with fewer queries skips the rest).
template <int NQT, bool CACHED, bool kFull, bool kFirst, int NT = NQT>
__device__ __forceinline__ void wg_chunk(WgTiles<NQT>& st, const unsigned char* kt,
                                         const unsigned char* vt, const int (&kofs)[2],
                                         const int (&vofs)[4], int c, int A, uint32_t rows,
                                         float scale_log2, int g) {
    const bf16x8_t ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    uint4 kop[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        kop[t][0] = *reinterpret_cast<const uint4*>(kt + kofs[0] + t * kHalfTile);
        kop[t][1] = *reinterpret_cast<const uint4*>(kt + kofs[1] + t * kHalfTile);
    }
    bf16x8_t va[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const uint2 lo = lds_tr_b64(vt + vofs[dt]);
        const uint2 hi = lds_tr_b64(vt + vofs[dt] + kHalfTile);
        va[dt] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
    const int r0 = c * kChunk;
    // CACHED: the score MFMAs start from 0 for a key row that exists and
    // from -inf for one that does not (rows: the chunk's row mask, uniform),
    // so every chunk takes the same path; the per-row values are formed only
    // for a chunk with a missing row (a partial last chunk or skipped list
    // entries).  Otherwise (no cached rows) only the partial last chunk
    // masks, here: the lane's key rows 16t + 4g + i that exist, at bits
    // 16t + i.
    f32x4_t bias[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    if constexpr (CACHED) {
        if (__builtin_expect(rows != ~0u, 0)) {
            const uint32_t have = rows >> (4 * g);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    bias[t][i] = ((have >> (16 * t + i)) & 1u) ? 0.f : -INFINITY;
        }
    }
    uint32_t have = 0;
    if constexpr (!kFull && !CACHED) {
        {
            const int left = A - r0 - 4 * g;  // rows past A do not exist
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) have |= (16 * t + i < left ? 1u : 0u) << (16 * t + i);
        }
    }
    auto scores = [&](int qt, float (&x)[8]) __attribute__((always_inline)) {
        f32x4_t s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4_t acc = CACHED ? bias[t] : f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[t][0]), st.qf[qt][0], acc,
                                                          0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[t][1]), st.qf[qt][1], acc,
                                                          0, 0, 0);
            s[t] = acc;
        }
        if constexpr (!kFull && !CACHED) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((have >> (16 * t + i)) & 1u)) s[t][i] = -INFINITY;
        }
        if constexpr (kFirst) {
            const float m1 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
            const float m2 = fmaxf(fmaxf(s[0][3], s[1][0]), s[1][1]);
            const float ms = fmaxf(fmaxf(s[1][2], s[1][3]), fmaxf(m1, m2));
            st.mc[qt] = max_over_groups(ms) * scale_log2;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * t + i] = fmaf(s[t][i], scale_log2, -st.mc[qt]);
    };
    auto xmax = [&](const float (&x)[8]) __attribute__((always_inline)) {
        const float m1 = fmaxf(fmaxf(x[0], x[1]), x[2]);
        const float m2 = fmaxf(fmaxf(x[3], x[4]), x[5]);
        return fmaxf(fmaxf(x[6], x[7]), fmaxf(m1, m2));
    };
    // A query's maximum moved far up: rescale (rare; kept off the
    // straight-line path so it is not turned into selects).
    auto rescale = [&](int qt, float mx, float (&x)[8]) __attribute__((always_inline)) {
        const float up = max_over_groups(mx);
        if (up > kRescaleLog2) {
            const float alpha = __builtin_amdgcn_exp2f(-up);
            st.lacc[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) st.oacc[qt][dt] *= alpha;
            st.mc[qt] += up;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] -= up;
        }
    };
    auto exps = [&](const float (&x)[8], float (&p)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i]);
    };
    auto finish = [&](int qt, const float (&p)[8]) __attribute__((always_inline)) {
        U4 pk;
        pk.u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
        st.lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk.v, st.lacc[qt], 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            st.oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pk.v,
                                                                   st.oacc[qt][dt], 0, 0, 0);
    };
    // Query tiles in pairs: both tiles' chains sit in one basic block
    // (one rescale test per pair), so their instructions interleave.
    // The exponentials are taken before the test, which only decides
    // whether they are taken again after a rescale (rare), so they need
    // not wait for the maximum; the block that ends at a pair's test
    // then also holds the previous pair's conversions and P V MFMAs and
    // this pair's score MFMAs, which issue among the exponentials.
    // Every one of the NT tiles is computed, also past nq (those rows repeat
    // the last query and are never stored): a per-pair test would end the
    // basic block early.
    static_assert(NT >= 1 && NT <= NQT, "tiles computed");
#pragma unroll
    for (int qt = 0; qt < NT; qt += 2) {
        if (qt + 1 < NT) {
            float x0[8], x1[8], p0[8], p1[8];
            scores(qt, x0);
            scores(qt + 1, x1);
            exps(x0, p0);
            exps(x1, p1);
            if constexpr (!kFirst) {
                const float m0 = xmax(x0), m1 = xmax(x1);
                if (__builtin_expect(__any(fmaxf(m0, m1) > kRescaleLog2), 0)) {
                    rescale(qt, m0, x0);
                    rescale(qt + 1, m1, x1);
                    exps(x0, p0);
                    exps(x1, p1);
                }
            }
            finish(qt, p0);
            finish(qt + 1, p1);
        } else {
            float x0[8], p0[8];
            scores(qt, x0);
            exps(x0, p0);
            if constexpr (!kFirst) {
                const float m0 = xmax(x0);
                if (__builtin_expect(__any(m0 > kRescaleLog2), 0)) {
                    rescale(qt, m0, x0);
                    exps(x0, p0);
                }
            }
            finish(qt, p0);
        }
    }
}

// ---------------------------------------------------------------------------
// Dense kernel: no cached rows and more queries per unit than one wave holds
// (A > 64): the full-attention layers, and with UPDATE a refresh step's
// layer (row r of k_a/v_a is also written to cache row r; A == N).  Work
// items are (unit, block of up to kDenseQ queries), nb = ceil(A / kDenseQ)
// blocks per unit.  A grid of persistent workgroups (kWgWaves waves x 16
// kWgNqt queries, kDensePerCu per compute unit) takes items s = blockIdx.x,
// blockIdx.x + gridDim.x, ...  The chunk stream runs on from one item to the
// next: while chunk c of an item is computed, the workgroup requests the
// stream's next chunk (chunk c + 1, or chunk 0 of its next item) and row
// block c of its next item's queries, which goes to an LDS copy of that
// item's Q.  An item thus starts from data already on chip.  (With one item
// per workgroup, the workgroups that start together all wait for their
// queries at once while the chip idles, once per round of workgroups.)
//  * Item s belongs to XCD s mod 8 (workgroups go round-robin over the 8 and
//    gridDim.x is a multiple of 8); the nb blocks of a unit are consecutive
//    items of one XCD, which run side by side and share the unit's chunks
//    through that XCD's L2.
//  * UPDATE: the loading lanes write each chunk they load into the caches;
//    of a unit's blocks, block c mod nb writes chunk c.
//  * The per-chunk math is wg_chunk's.  Q rows load with streaming loads;
//    so do K/V rows when a unit has one block (SHARED = false).  With several
//    blocks (SHARED) the K/V loads are plain, since the unit's other blocks
//    read the same chunks from L2 at about the same time (streaming loads
//    there cost 3-4% at 1088 tokens; plain ones cost 4-5% at 320).
// ---------------------------------------------------------------------------
constexpr int kDenseQ = kWgWaves * 16 * kWgNqt;  // queries per item
constexpr int kDenseLds = 4 * kWgTile + kDenseQ * kD * 2 + kWgWaves * 2048;
constexpr int kDensePerCu = 2;  // resident workgroups per compute unit (register-bound)
static_assert(kDenseLds <= 64 * 1024, "static LDS");
static_assert(kDenseQ % kChunk == 0, "Q row blocks follow the chunks");

// LAB (measurement builds only; the decoding path uses kLabNone): kLabArith
// keeps every instruction but turns each global load into a range-checked
// load past the buffer (zeros, no memory traffic) and drops the output and
// lse stores (and, with UPDATE, the cache writes) -- the kernel's
// arithmetic, LDS traffic and barriers alone; kLabMemory skips the per-chunk
// math -- its loads, LDS stores, barriers, cache writes and output stores
// alone.
constexpr int kLabNone = 0, kLabArith = 1, kLabMemory = 2;

template <bool UPDATE, bool SHARED, int LAB = kLabNone>
__global__ __launch_bounds__(64 * kWgWaves) __attribute__((amdgpu_waves_per_eu(2, 8)))
void attn_dense_kernel(const uint16_t* __restrict__ q_a, const uint16_t* __restrict__ k_a,
                       const uint16_t* __restrict__ v_a, uint16_t* __restrict__ k_cache,
                       uint16_t* __restrict__ v_cache, uint16_t* __restrict__ out,
                       float* __restrict__ lse, int units, int A, int nb, float scale_log2) {
    constexpr int NQT = kWgNqt;
    constexpr int kQ = 16 * NQT;  // queries per wave
    constexpr uint32_t kOut = 0x80000000u;  // past any buffer: a load reads zeros, a store is dropped
    __shared__ __align__(16) unsigned char lds[kDenseLds];  // 2 x (K tile, V tile); Q; output staging
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int m16 = lane & 15;
    unsigned char* const qs = lds + 4 * kWgTile;                // Q rows of an item, swizzled
    unsigned char* const ot = qs + kDenseQ * kD * 2 + w * 2048;  // this wave's output staging
    const int nchunks = (A + kChunk - 1) / kChunk;
    const int nitems = ((units + 7) / 8) * 8 * nb;
    const uint32_t unit_bytes = static_cast<uint32_t>(A) * kD * 2;
    // Item s: unit (s / 8 / nb) * 8 + s mod 8, block (s / 8) mod nb; an item
    // past the last unit is skipped.
    auto unit_of = [&](int s) { return ((s >> 3) / nb) * 8 + (s & 7); };
    auto block_of = [&](int s) { return (s >> 3) % nb; };
    auto next_item = [&](int s) {
        for (s += gridDim.x; s < nitems && unit_of(s) >= units; s += gridDim.x) {
        }
        return s < nitems ? s : -1;
    };
    auto rsrc = [&](const uint16_t* base, int u) {
        return uniform_rsrc(base + static_cast<size_t>(u) * A * kD, unit_bytes);
    };
    // Q rows are read once: streaming loads.  K/V rows too, unless the unit
    // has several blocks (SHARED), whose workgroups read them from L2 again.
    auto ldq = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t ofs) __attribute__((always_inline)) {
        if constexpr (LAB == kLabArith) ofs = kOut;
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, ofs, 0, kStreamPolicy));
    };
    auto ld = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t ofs) __attribute__((always_inline)) {
        if constexpr (LAB == kLabArith) ofs = kOut;
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, ofs, 0, SHARED ? 0 : kStreamPolicy));
    };
    // Loading lane: piece tid % 8 of row tid / 8 of a 32-row block.
    const int lrow = tid >> 3;
    const uint32_t piece = 16 * (tid & 7);
    const int lofs = swz(lrow, tid & 7);
    auto put_rows = [&](int u, int c, const uint4& kk, const uint4& vv) __attribute__((always_inline)) {
        if constexpr (LAB == kLabArith) return;  // no memory traffic
        // the cache rows of chunk c of unit u (a row past A is dropped)
        const int r = c * kChunk + lrow;
        const uint32_t off = r < A ? static_cast<uint32_t>(r) * (kD * 2) + piece : kOut;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, kk), rsrc(k_cache, u), off, 0, kStreamPolicy);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, vv), rsrc(v_cache, u), off, 0, kStreamPolicy);
    };

    int s = blockIdx.x;
    while (s < nitems && unit_of(s) >= units) s += gridDim.x;
    if (s >= nitems) return;  // uniform over the workgroup, before any barrier
    {
        // The first item's Q rows and chunk 0, requested together.
        const int u = unit_of(s), qb = block_of(s);
        const __amdgpu_buffer_rsrc_t rq = rsrc(q_a, u);
        uint4 qv[kDenseQ / kChunk];
#pragma unroll
        for (int i = 0; i < kDenseQ / kChunk; ++i) {
            const int r = qb * kDenseQ + i * kChunk + lrow;  // a row past A reads zero
            qv[i] = ldq(rq, static_cast<uint32_t>(r) * (kD * 2) + piece);
        }
        const uint4 kk = ld(rsrc(k_a, u), static_cast<uint32_t>(lrow) * (kD * 2) + piece);
        const uint4 vv = ld(rsrc(v_a, u), static_cast<uint32_t>(lrow) * (kD * 2) + piece);
#pragma unroll
        for (int i = 0; i < kDenseQ / kChunk; ++i)
            *reinterpret_cast<uint4*>(qs + swz(i * kChunk + lrow, tid & 7)) = qv[i];
        *reinterpret_cast<uint4*>(lds + lofs) = kk;
        *reinterpret_cast<uint4*>(lds + kWgTile + lofs) = vv;
        if constexpr (UPDATE)
            if (qb == 0) put_rows(u, 0, kk, vv);
        __syncthreads();
    }

    // LDS offsets: the K operand pieces g and 4 + g of key row 16t + m16 and
    // the V^T transposing reads (as in the workgroup kernel).
    int vofs[4], kofs[2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        vofs[dt] = swz(4 * g + (m16 >> 2), 2 * dt + ((m16 & 3) >> 1)) + ((m16 & 1) << 3);
    kofs[0] = swz(m16, g);
    kofs[1] = swz(m16, 4 + g);
    WgTiles<NQT> st;
    uint4 sk, sv, sq;  // the staged chunk rows and the next item's Q row

    // Item s, its chunk 0 in LDS buffer P (chunk c in buffer (P + c) mod 2),
    // its Q in qs; sn: the workgroup's next item (-1: none).
    auto run_item = [&](int s, int sn, auto par_tag) __attribute__((always_inline)) {
        constexpr int P = decltype(par_tag)::value;
        const int u = unit_of(s), qb = block_of(s);
        const int un = sn >= 0 ? unit_of(sn) : 0, qbn = sn >= 0 ? block_of(sn) : 0;
        const int nqb = min(A - qb * kDenseQ, kDenseQ);  // the item's queries (>= 1)
        const int q0 = qb * kDenseQ + w * kQ;            // this wave's first query
        const int nq = min(A - q0, kQ);                  // <= 0: the wave loads and waits only
        {
            int lq = lane;  // opaque copy, so that these offsets are not hoisted (see below)
            asm volatile("" : "+v"(lq));
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int r = min(w * kQ + 16 * qt + (lq & 15), nqb - 1);  // rows past the end repeat the last
                st.qf[qt][0] = as_bf16x8(*reinterpret_cast<const uint4*>(qs + swz(r, lq >> 4)));
                st.qf[qt][1] = as_bf16x8(*reinterpret_cast<const uint4*>(qs + swz(r, 4 + (lq >> 4))));
            }
        }
        __syncthreads();  // every wave holds its Q before the next item's rows land
        st.reset();
        const __amdgpu_buffer_rsrc_t rk = rsrc(k_a, u), rv = rsrc(v_a, u);
        const __amdgpu_buffer_rsrc_t rkn = rsrc(k_a, un), rvn = rsrc(v_a, un), rqn = rsrc(q_a, un);
        // Step c: request the stream's next chunk and row block c of the next
        // item's Q, compute chunk c, store what was requested and wait for
        // every wave.  Every step issues the same loads (out-of-range offsets
        // where there is nothing to load: no traffic), so the compiler's
        // memory-counter waits stay exact.
        auto step = [&](int c, auto buf_tag, auto full_tag, auto first_tag) __attribute__((always_inline)) {
            constexpr int BI = decltype(buf_tag)::value;
            const bool own = c + 1 < nchunks;  // uniform
            const uint32_t row_ofs = static_cast<uint32_t>(lrow) * (kD * 2) + piece;
            const uint32_t ofs = own ? static_cast<uint32_t>((c + 1) * kChunk) * (kD * 2) + row_ofs
                                     : (sn >= 0 ? row_ofs : kOut);
            sk = ld(own ? rk : rkn, ofs);
            sv = ld(own ? rv : rvn, ofs);
            const bool qrow = sn >= 0 && c * kChunk < kDenseQ;  // uniform
            sq = ldq(rqn, qrow ? static_cast<uint32_t>(qbn * kDenseQ + c * kChunk) * (kD * 2) + row_ofs : kOut);
            if (LAB != kLabMemory && nq > 0)
                wg_chunk<NQT, false, decltype(full_tag)::value, decltype(first_tag)::value>(
                    st, lds + BI * 2 * kWgTile, lds + BI * 2 * kWgTile + kWgTile, kofs, vofs, c, A,
                    ~0u, scale_log2, g);
            *reinterpret_cast<uint4*>(lds + (BI ^ 1) * 2 * kWgTile + lofs) = sk;
            *reinterpret_cast<uint4*>(lds + (BI ^ 1) * 2 * kWgTile + kWgTile + lofs) = sv;
            if (c * kChunk < kDenseQ) *reinterpret_cast<uint4*>(qs + swz(c * kChunk + lrow, tid & 7)) = sq;
            if constexpr (UPDATE) {
                if (own ? (c + 1) % nb == qb : (sn >= 0 && qbn == 0))  // uniform
                    put_rows(own ? u : un, own ? c + 1 : 0, sk, sv);
            }
            __syncthreads();
        };
        using Bp = std::integral_constant<int, P>;
        using Bq = std::integral_constant<int, P ^ 1>;
        using T1 = std::true_type;
        using F0 = std::false_type;
        // The chunks without rows past A, in pairs, then the partial last
        // chunk if A is not a multiple of 32: only that one masks.
        const int nfull = A / kChunk;  // >= 2 (A > 64)
        step(0, Bp{}, T1{}, T1{});
        int c = 1;
        for (; c + 1 < nfull; c += 2) {
            step(c, Bq{}, T1{}, F0{});
            step(c + 1, Bp{}, T1{}, F0{});
        }
        if (c < nfull) step(c++, Bq{}, T1{}, F0{});
        if (c < nchunks) {
            if (c & 1)
                step(c, Bq{}, F0{}, F0{});
            else
                step(c, Bp{}, F0{}, F0{});
        }
        // Finalise through this wave's own staging area, one 16-query tile at
        // a time, so that every (nontemporal) store writes whole 128-byte rows.
        if (nq > 0) {
            // The lane's offsets are derived here from an opaque copy of its
            // index: offsets the compiler could hoist out of the item loop
            // would stay live across every chunk step and be spilled.
            int lf = lane;
            asm volatile("" : "+v"(lf));
            const int gf = lf >> 4, mf = lf & 15;
            u32x4_t* orow = reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(u) * A * kD +
                                                       static_cast<size_t>(q0) * kD);
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                if (qt * 16 >= nq) continue;
                const float l = st.lacc[qt][0];
                const float inv = 1.f / l;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const uint2 v2 = make_uint2(
                        pack_bf16x2(st.oacc[qt][dt][0] * inv, st.oacc[qt][dt][1] * inv),
                        pack_bf16x2(st.oacc[qt][dt][2] * inv, st.oacc[qt][dt][3] * inv));
                    *reinterpret_cast<uint2*>(ot + swz(mf, 2 * dt + (gf >> 1)) + ((gf & 1) << 3)) = v2;
                }
                const int row = 16 * qt + mf;
                if (LAB != kLabArith && lse != nullptr && gf == 0 && row < nq)
                    lse[static_cast<size_t>(u) * A + q0 + row] = (st.mc[qt] + log2f(l)) * kLn2;
                __builtin_amdgcn_wave_barrier();  // the tile's writes before its reads (one wave)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int r = 8 * k + (lf >> 3);
                    const u32x4_t v4 = *reinterpret_cast<const u32x4_t*>(ot + swz(r, lf & 7));
                    if (LAB != kLabArith && 16 * qt + r < nq)
                        __builtin_nontemporal_store(v4, orow + (16 * qt + r) * 8 + (lf & 7));
                }
                __builtin_amdgcn_wave_barrier();  // the reads before the next tile's writes
            }
        }
    };

    int par = 0;  // the LDS buffer of the current item's chunk 0
    while (s >= 0) {
        const int sn = next_item(s);
        if (par == 0)
            run_item(s, sn, std::integral_constant<int, 0>{});
        else
            run_item(s, sn, std::integral_constant<int, 1>{});
        par ^= nchunks & 1;
        s = sn;
    }
}

template <bool UPDATE, int LAB = kLabNone>
int launch_dense_wg(const uint16_t* q_a, const uint16_t* k_a, const uint16_t* v_a,
                    uint16_t* k_cache, uint16_t* v_cache, uint16_t* out, float* lse, int B, int H,
                    int A, float scale_log2, hipStream_t stream) {
    const int units = B * H;
    const int nb = (A + kDenseQ - 1) / kDenseQ;
    const int items = ((units + 7) / 8) * 8 * nb;
    int cus = 0;
    if (const int st = compute_units(stream, &cus); st != MAR_OK) return st;
    const int grid = std::min(items, std::max(8, (kDensePerCu * cus) / 8 * 8));
    if (nb == 1)
        hipLaunchKernelGGL((attn_dense_kernel<UPDATE, false, LAB>), dim3(grid), dim3(64 * kWgWaves), 0,
                           stream, q_a, k_a, v_a, k_cache, v_cache, out, lse, units, A, nb, scale_log2);
    else
        hipLaunchKernelGGL((attn_dense_kernel<UPDATE, true, LAB>), dim3(grid), dim3(64 * kWgWaves), 0,
                           stream, q_a, k_a, v_a, k_cache, v_cache, out, lse, units, A, nb, scale_log2);
    return status_from_launch();
}


}  // namespace
}  // namespace marca
