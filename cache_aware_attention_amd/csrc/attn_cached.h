// attn_cached.h -- the workgroup attention kernel for units whose queries
// fill several waves (gfx950): the cache-aware layers with more than 64
// active rows (the high-res layers, LazyMAR's per-sequence recomputed rows)
// and layer 2's full attention with the refresh partials.
//
// Operation ("MARche" paper-notes page, Overall Architecture and Key Design
// 2, Eq. 1-2: attention of the active queries over the fresh active rows and
// the stored rows of the cached tokens, merged through one running softmax
// state; the "LazyMAR" notes page, token cache: per-sequence sets of
// recomputed tokens).  cache_attn.hip launches it on the decoding path; the
// measurement library instantiates its measurement modes (LAB, as for the
// full-attention kernel) to time its arithmetic and its memory traffic apart.
#pragma once

#include <type_traits>

#include "attn_dense.h"

namespace marca {
namespace {

// ---------------------------------------------------------------------------
// Workgroup kernel: more queries per unit than one wave holds (A > 64).  One
// workgroup of W waves per (unit, block of W * 16 * NQT queries).  Each 32-row
// K/V chunk of the unit's sequence is loaded once per workgroup into a
// double-buffered LDS tile, and every wave reads its MFMA operands from there.
// A unit's K/V then crosses the L2-to-CU path once per workgroup instead of
// once per 64-query wave, which is what bounds the one-wave kernel once a unit
// has several query groups.
//  * CACHED = false only for layer 2's scores pass (SCORES below; the other
//    full-attention layers run attn_dense_kernel): W = 4, NQT = 5, one
//    workgroup per unit of at most 320 tokens, the keys rows 0..A-1 of
//    k_a/v_a, read with range-checked buffer loads (a row past A reads as
//    zero and is masked).
//  * CACHED = true (the cache-aware layers with several query groups, W = 2
//    or 4, NQT = 4): the sequence is [the A active rows ; the Nc cached rows
//    at the staged list's token positions].  The list is staged in LDS once
//    (entries outside [0, N) become -1) together with one flag per chunk that
//    says whether every row of the chunk exists; only chunks without that
//    flag carry the masking.  With UPDATE the loading lanes of the unit's
//    first block write the active rows into the caches at active_idx.
//    RAGGED: per-sequence counts, min(a_len[b], A) active rows and
//    min(c_len[b], Nc) cached entries (A and Nc stay the row stride and the
//    list capacity); rows past a sequence's active count are not written,
//    neither to out nor (with UPDATE) to the caches.
// The MFMA tiles are those of attn_mfma_kernel.  The softmax state differs:
//  * each query keeps one reference mc, a maximum of its scaled scores
//    s * scale_log2, set from the first chunk (active rows, at least the
//    first of which exists, so the reference is finite);
//  * a tile computes x = s * scale_log2 - mc first and tests max(x) against
//    kRescaleLog2 (an inline constant), so no raw maximum or threshold has
//    to stay in registers;
//  * the query tiles go in pairs under one rescale test, so both tiles'
//    exponentials and conversions sit in one basic block and interleave.
// The first chunk sets the same reference in both kernels, so a unit that
// needs no later rescale gets the same bits from both.
// LAB (measurement modes, cached rows only; outputs meaningless): kLabArith
// reads every chunk as zeros with no memory traffic and skips the cache and
// output stores (the LDS staging of the output keeps the arithmetic live);
// kLabMemory issues every load, LDS store, barrier and store but skips the
// per-chunk math.
// ---------------------------------------------------------------------------
//  * SCORES (no cached rows, no update, one workgroup per unit of at most 320
//    tokens: layer 2's full attention on a cached step): every K chunk stays
//    in LDS (at its own slot instead of the double buffer) and each query's
//    reference is recorded; after the last chunk the waves score the unit's
//    generating queries (gen_idx, at most 16) against the K held in LDS and
//    write their softmax probabilities summed over those queries, per key --
//    the per-head partials the refresh selection reads ("MARche" paper-notes
//    page, Key Design 1: the top-K reads layer 2's attention from the
//    generating tokens; without this the scores kernel reads K again).  The
//    probabilities are exp2(s c - m) / l in fp32 with the query's attention
//    reference m and l their exact fp32 sum over the keys.
template <int NQT, int W, bool UPDATE, bool CACHED, bool RAGGED = false, bool SCORES = false,
          int LAB = kLabNone>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 8)))
void attn_wg_kernel(const uint16_t* __restrict__ q_a, const uint16_t* __restrict__ k_a,
                    const uint16_t* __restrict__ v_a, uint16_t* k_cache, uint16_t* v_cache,
                    uint16_t* __restrict__ out, float* __restrict__ lse, int units, int A,
                    int n_blocks, float scale_log2, const int32_t* __restrict__ cached_idx,
                    int ldc, int H, int N, int Nc, const int32_t* __restrict__ active_idx,
                    int ld_act, int32_t* __restrict__ err_count,
                    const int32_t* __restrict__ a_len = nullptr,
                    const int32_t* __restrict__ c_len = nullptr,
                    const int32_t* __restrict__ gen_idx = nullptr, int ld_gen = 0, int G = 0,
                    float* __restrict__ partials = nullptr) {
    static_assert(W == 1 || W == 2 || W == 4, "waves per workgroup");
    static_assert(!RAGGED || CACHED, "per-sequence counts: cached rows");
    static_assert(!SCORES || (!CACHED && !UPDATE && W == 4), "scores: layer 2's full attention");
    static_assert(CACHED || SCORES, "the full-attention layers run attn_dense_kernel");
    static_assert(LAB == kLabNone || (CACHED && !SCORES), "measurement modes: cached rows");
    constexpr int kQ = 16 * NQT;         // queries per wave
    constexpr int kPasses = 4 / W;       // load passes per chunk (8 W rows each)
    // The chunk loads (whole rows, 8 lanes per row): streaming with cached
    // rows; plain for the scores pass.
    constexpr int kWgLoadPolicy = CACHED ? kStreamPolicy : 0;
    __shared__ __align__(16) unsigned char lds[4 * kWgTile];  // 2 buffers x (K tile, V tile)
    static_assert(4 * kWgTile >= W * 2048, "the output staging reuses the K/V tiles");
    // CACHED: the staged lists after the tiles, [max(Nc, 1)] entries, the
    // chunk flags [nchunks], and with UPDATE the active positions [A].
    extern __shared__ __align__(16) int32_t wg_lists[];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int m16 = lane & 15;

    int u, qb;
    if (n_blocks == 1) {
        u = blockIdx.x;
        qb = 0;
    } else {  // the blocks of one unit on one XCD (workgroups go round-robin over the 8)
        const int xcd = blockIdx.x & 7;
        const int slot = blockIdx.x >> 3;
        u = (slot / n_blocks) * 8 + xcd;
        qb = slot % n_blocks;
        if (u >= units) return;  // uniform over the workgroup, before any barrier
    }
    // The unit's counts: An active rows (A is their stride) and Ncn cached
    // entries (Nc is the list capacity).
    int An = A, Ncn = Nc;
    if constexpr (RAGGED) {
        An = min(max(a_len[u / H], 0), A);
        Ncn = min(max(c_len[u / H], 0), Nc);
        if (qb * W * kQ >= An) return;  // no queries in this block (uniform, before any barrier)
    }
    // This wave's queries: nt 16-query tiles from q0.  CACHED: the block's
    // tiles are spread evenly over its waves, one more for `extra` of them,
    // a choice that rotates with the workgroup so no SIMD always takes the
    // larger share (a ragged count of ~170 then keeps all four waves busy
    // with three tiles or two, instead of three waves with four and one
    // idle).  Otherwise kQ queries per wave.
    int q0 = (qb * W + w) * kQ, nt = NQT;
    if constexpr (CACHED) {
        const int qbase = qb * W * kQ;
        const int tiles = (min(An - qbase, W * kQ) + 15) / 16;  // An > qbase here
        const int base = tiles / W, extra = tiles % W;
        const int rot = static_cast<int>(blockIdx.x % W);
        int t0 = 0;
        for (int v = 0; v < w; ++v) t0 += base + ((v + rot) % W < extra ? 1 : 0);
        nt = base + ((w + rot) % W < extra ? 1 : 0);
        q0 = qbase + 16 * t0;
    }
    const int nq = min(An - q0, 16 * nt);  // <= 0: the wave loads and waits, computes nothing
    const size_t ub = static_cast<size_t>(u) * A * kD;
    // CACHED: the active rows fill chunks [0, na) (the last one padded), the
    // cached rows start on the next chunk: row A0 + j is cached entry j.
    const int na = (An + kChunk - 1) / kChunk;
    const int A0 = CACHED ? na * kChunk : A;
    const int T = CACHED ? A0 + Ncn : A;  // rows of the unit's (padded) sequence
    const int nchunks = (T + kChunk - 1) / kChunk;
    const __amdgpu_buffer_rsrc_t rka = uniform_rsrc(k_a + ub, A * kD * 2);
    const __amdgpu_buffer_rsrc_t rva = uniform_rsrc(v_a + ub, A * kD * 2);
    const size_t cb = static_cast<size_t>(u) * N * kD;  // the unit's cache rows (CACHED)

    int32_t* cidx_s = wg_lists;                       // [max(Nc, 1)]
    int32_t* cflag_s = cidx_s + (Nc > 0 ? Nc : 1);    // [nchunks]
    int32_t* aidx_s = cflag_s + nchunks;              // [A] with UPDATE
    // Loading lane: piece tid % 8 of rows 8 W p + tid / 8 (p < kPasses) of the
    // chunk, for K and V, by range-checked buffer loads (an offset past the
    // buffer reads as zero).  A row past A (no cached rows), a skipped cached
    // entry or a row past the sequence reads as zero and is masked.
    const int lrow = tid >> 3;
    const __amdgpu_buffer_rsrc_t rkc = uniform_rsrc(k_cache + (CACHED ? cb : 0), CACHED ? N * kD * 2 : 0);
    const __amdgpu_buffer_rsrc_t rvc = uniform_rsrc(v_cache + (CACHED ? cb : 0), CACHED ? N * kD * 2 : 0);
    auto load = [&](int c, uint4 (&kk)[kPasses], uint4 (&vv)[kPasses]) __attribute__((always_inline)) {
        constexpr uint32_t kOut = 0x80000000u;  // past any buffer: reads as zero
        auto ld = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t ofs) __attribute__((always_inline)) {
            // kLabArith: every load reads as zero, with no memory traffic
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, LAB == kLabArith ? kOut : ofs, 0, kWgLoadPolicy));
        };
        const int r0 = c * kChunk;
        const uint32_t piece = 16 * (tid & 7);
        if (!CACHED || r0 < An) {  // active rows (uniform; a row past A reads as zero)
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const uint32_t ofs = static_cast<uint32_t>(r0 + 8 * W * p + lrow) * (kD * 2) + piece;
                kk[p] = ld(rka, ofs);
                vv[p] = ld(rva, ofs);
            }
        } else {  // cached rows at the staged positions (the index read is in bounds)
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int j = r0 - A0 + 8 * W * p + lrow;
                const int n = cidx_s[min(j, Nc - 1)];
                const uint32_t ofs = (j < Ncn && n >= 0) ? static_cast<uint32_t>(n) * (kD * 2) + piece : kOut;
                kk[p] = ld(rkc, ofs);
                vv[p] = ld(rvc, ofs);
            }
        }
    };
    // SCORES: K chunk c at its own slot of the dynamic LDS, kall + c * kWgTile.
    unsigned char* kall = reinterpret_cast<unsigned char*>(wg_lists);
    auto put = [&](int buf, int c, const uint4 (&kk)[kPasses], const uint4 (&vv)[kPasses]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int lofs = swz(8 * W * p + lrow, tid & 7);
            if constexpr (SCORES) {
                if (c < nchunks) *reinterpret_cast<uint4*>(kall + c * kWgTile + lofs) = kk[p];
            } else {
                *reinterpret_cast<uint4*>(lds + buf * 2 * kWgTile + lofs) = kk[p];
            }
            *reinterpret_cast<uint4*>(lds + buf * 2 * kWgTile + kWgTile + lofs) = vv[p];
        }
        if constexpr (UPDATE && LAB != kLabArith) {
            // The row's target cache row, or an offset past the buffer, which
            // the range check drops: a row past A or a skipped entry.
            constexpr uint32_t kSkip = 0x80000000u;
            constexpr int kNT = 2;  // nontemporal (streaming) store
            const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(k_cache + cb, N * kD * 2);
            const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(v_cache + cb, N * kD * 2);
            if (c * kChunk < An) {  // uniform: the chunk holds active rows
#pragma unroll
                for (int p = 0; p < kPasses; ++p) {
                    const int r = c * kChunk + 8 * W * p + lrow;
                    const int n = (r >= A) ? -1 : aidx_s[r];
                    const uint32_t off = (n >= 0) ? static_cast<uint32_t>(n) * (kD * 2) + 16 * (tid & 7)
                                                  : kSkip;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, kk[p]), rk, off, 0, kNT);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, vv[p]), rv, off, 0, kNT);
                }
            }
        }
    };

    // Q operands (B of S^T = K Q^T): lane holds query m16 of tile qt, head
    // dims [8g, 8g+8) and [32+8g, 32+8g+8).  Rows past the end load the last
    // query; they are never stored.
    WgTiles<NQT> st;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int qi = max(min(q0 + qt * 16 + m16, An - 1), 0);
        const uint4* p = reinterpret_cast<const uint4*>(q_a + ub + static_cast<size_t>(qi) * kD);
        st.qf[qt][0] = as_bf16x8(p[g]);
        st.qf[qt][1] = as_bf16x8(p[4 + g]);
    }
    // LDS byte offsets: the V^T transposing reads as in attn_mfma_kernel, and
    // the K operand pieces g and 4+g of key row 16t + m16.
    int vofs[4], kofs[2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        vofs[dt] = swz(4 * g + (m16 >> 2), 2 * dt + ((m16 & 3) >> 1)) + ((m16 & 1) << 3);
    kofs[0] = swz(m16, g);
    kofs[1] = swz(m16, 4 + g);

    // mc: the reference maximum of each query's scaled scores s * scale_log2
    // (set from the first chunk: active rows, the first of which exists).
    st.reset();

    // NT: the tiles the wave computes (its whole chunk loop is instantiated
    // per tile count, so each copy keeps the registers of one).
    auto compute = [&](int c, int buf, uint32_t rows, auto full_tag, auto first_tag, auto nt_tag) __attribute__((always_inline)) {
        const unsigned char* kt = SCORES ? kall + c * kWgTile : lds + buf * 2 * kWgTile;
        const unsigned char* vt = lds + buf * 2 * kWgTile + kWgTile;
        wg_chunk<NQT, CACHED, decltype(full_tag)::value, decltype(first_tag)::value,
                 decltype(nt_tag)::value>(st, kt, vt, kofs, vofs, c, A, rows, scale_log2, g);
    };

    // Chunk c sits in LDS buffer c % 2.  Each step requests chunk c + 1 into
    // the staging registers, computes chunk c, stores chunk c + 1 into the
    // other buffer (whose chunk c - 1 every wave finished before the previous
    // barrier) and waits at the barrier.  Every step issues the same loads
    // (past the last chunk at out-of-range offsets, which read zeros without
    // touching memory), so the compiler's memory-counter waits stay exact.
    uint4 sk[kPasses], sv[kPasses];
    load(0, sk, sv);  // chunk 0 holds active rows only (A > 64): no list needed
    if constexpr (CACHED) {
        // Stage the cached list (entries outside [0, N) become -1); the first
        // kStage entries per thread are requested together.
        const int b = u / H;
        const int32_t* cg = cached_idx + static_cast<size_t>(b) * ldc;
        constexpr int kStage = 8;
        int32_t iv[kStage];
#pragma unroll
        for (int k = 0; k < kStage; ++k) {
            const int c = tid + 64 * W * k;
            iv[k] = (c < Ncn) ? cg[c] : -1;
        }
#pragma unroll
        for (int k = 0; k < kStage; ++k) {
            const int c = tid + 64 * W * k;
            if (c < Ncn) cidx_s[c] = (iv[k] >= 0 && iv[k] < N) ? iv[k] : -1;
        }
        for (int c = tid + 64 * W * kStage; c < Ncn; c += 64 * W) {
            const int n = cg[c];
            cidx_s[c] = (n >= 0 && n < N) ? n : -1;
        }
        if constexpr (UPDATE) {
            // Only the unit's first block writes the active rows; an entry
            // outside [0, N) is skipped and, once per sequence, counted.
            // RAGGED: entries past the sequence's count are not read.
            const int32_t* ag = active_idx + static_cast<size_t>(b) * ld_act;
            for (int r = tid; r < A; r += 64 * W) {
                if (r >= An) {
                    aidx_s[r] = -1;
                    continue;
                }
                const int n = ag[r];
                const bool ok = n >= 0 && n < N;
                aidx_s[r] = (ok && qb == 0) ? n : -1;
                if (!ok && err_count != nullptr && qb == 0 && u % H == 0) atomicAdd(err_count, 1);
            }
        }
        __syncthreads();
        // Chunk c's row mask, bit k set when row 32c + k exists: one ballot
        // per 64 rows (the index read is in bounds for every lane).
        for (int base = 64 * w; base < nchunks * kChunk; base += 64 * W) {
            const int r = base + lane;
            const int n = cidx_s[min(max(r - A0, 0), Nc - 1)];
            const bool ok = (r < A0) ? r < An : (r < T && n >= 0);
            const uint64_t m = __ballot(ok);
            if (lane == 0) {
                cflag_s[base / kChunk] = static_cast<int32_t>(static_cast<uint32_t>(m));
                if (base / kChunk + 1 < nchunks)
                    cflag_s[base / kChunk + 1] = static_cast<int32_t>(static_cast<uint32_t>(m >> 32));
            }
        }
        // (the barrier after the first chunk's tile stores orders these)
    }
    put(0, 0, sk, sv);
    __syncthreads();
    auto step = [&](int c, auto buf_tag, auto full_tag, auto first_tag, auto nt_tag, uint32_t rows = ~0u) __attribute__((always_inline)) {
        constexpr int BI = decltype(buf_tag)::value;
        load(c + 1, sk, sv);  // past the last chunk: out-of-range offsets, no traffic
        if (LAB != kLabMemory && nq > 0) compute(c, BI, rows, full_tag, first_tag, nt_tag);
        put(BI ^ 1, c + 1, sk, sv);
        __syncthreads();
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using T1 = std::true_type;
    using F0 = std::false_type;
    using NA = std::integral_constant<int, NQT>;
    if constexpr (!CACHED) {
        // The chunks without rows past A, in pairs (constant buffer indices),
        // then the partial last chunk if A is not a multiple of 32: only that
        // one carries the masking.
        const int nfull = A / kChunk;  // >= 2 (A > 64)
        step(0, B0{}, T1{}, T1{}, NA{});
        int c = 1;
        for (; c + 1 < nfull; c += 2) {
            step(c, B1{}, T1{}, F0{}, NA{});
            step(c + 1, B0{}, T1{}, F0{}, NA{});
        }
        if (c < nfull) step(c++, B1{}, T1{}, F0{}, NA{});
        if (c < nchunks) {
            if (c & 1)
                step(c, B1{}, F0{}, F0{}, NA{});
            else
                step(c, B0{}, F0{}, F0{}, NA{});
        }
    } else {
        // Every chunk's scores start from its row mask (uniform).  Chunk 0
        // sets the references; it holds active rows only, all of them unless
        // a sequence's count is below 32.  The loop runs at the wave's tile
        // count (every copy passes the same barriers).
        auto chunks = [&](auto nt_tag) __attribute__((always_inline)) {
            auto step_any = [&](int c, auto buf_tag) __attribute__((always_inline)) {
                step(c, buf_tag, T1{}, F0{}, nt_tag,
                     __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(cflag_s[c])));
            };
            step(0, B0{}, T1{}, T1{}, nt_tag,
                 __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(cflag_s[0])));
            int c = 1;
            for (; c + 1 < nchunks; c += 2) {
                step_any(c, B1{});
                step_any(c + 1, B0{});
            }
            if (c < nchunks) step_any(c, B1{});
        };
        static_assert(NQT == 4, "cached workgroup tiles");
        if (nt >= 4)
            chunks(std::integral_constant<int, 4>{});
        else if (nt == 3)
            chunks(std::integral_constant<int, 3>{});
        else if (nt == 2)
            chunks(std::integral_constant<int, 2>{});
        else  // one tile, or none (nq <= 0: the wave only loads)
            chunks(std::integral_constant<int, 1>{});
    }

    if constexpr (SCORES) {
        // The references of this wave's queries, for the scores below.
        float* mq_s = reinterpret_cast<float*>(kall + nchunks * kWgTile);
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            if (g == 0 && 16 * qt + m16 < nq) mq_s[q0 + 16 * qt + m16] = st.mc[qt];
    }

    // Finalise through this wave's 2 KB of the (now free) LDS tiles, one
    // 16-query tile at a time, so that every (nontemporal) store writes
    // whole 128-byte rows.  (SCORES: the output first, so its accumulators
    // are free before the scores; a wave without queries stays for the
    // barriers that follow.)
    if (!SCORES && nq <= 0) return;
    unsigned char* ot = lds + w * 2048;
    u32x4_t* orow = reinterpret_cast<u32x4_t*>(out + ub + static_cast<size_t>(q0) * kD);
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        if (qt * 16 >= nq) continue;
        const float l = st.lacc[qt][0];
        const float inv = 1.f / l;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const uint2 v2 = make_uint2(pack_bf16x2(st.oacc[qt][dt][0] * inv, st.oacc[qt][dt][1] * inv),
                                        pack_bf16x2(st.oacc[qt][dt][2] * inv, st.oacc[qt][dt][3] * inv));
            *reinterpret_cast<uint2*>(ot + swz(m16, 2 * dt + (g >> 1)) + ((g & 1) << 3)) = v2;
        }
        const int row = 16 * qt + m16;
        if (LAB != kLabArith && lse != nullptr && g == 0 && row < nq)
            lse[static_cast<size_t>(u) * A + q0 + row] = (st.mc[qt] + log2f(l)) * kLn2;
        __builtin_amdgcn_wave_barrier();  // the tile's writes before its reads (one wave)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = 8 * k + (lane >> 3);
            const u32x4_t v4 = *reinterpret_cast<const u32x4_t*>(ot + swz(r, lane & 7));
            if (LAB != kLabArith && 16 * qt + r < nq)
                __builtin_nontemporal_store(v4, orow + (16 * qt + r) * 8 + (lane & 7));
        }
        __builtin_amdgcn_wave_barrier();  // the reads before the next tile's writes
    }

    if constexpr (SCORES) {
        // References of this wave's queries, then the generating queries'
        // probabilities against the K chunks held in LDS.  Lane (g, m16) holds
        // S[generating query 4g + i][key 16t + m16] of key tile t (the scores
        // kernel's layout: Q as the A operand, K as the B operand).
        float* mq_s = reinterpret_cast<float*>(kall + nchunks * kWgTile);  // [nchunks * 32]
        float* red_s = mq_s + nchunks * kChunk;                             // [W][16]
        const int32_t* gi = gen_idx + static_cast<size_t>(u / H) * ld_gen;
        const int gq = (m16 < G) ? gi[m16] : -1;  // this lane's A-operand query
        const bool gq_ok = gq >= 0 && gq < A;
        uint4 qlo = make_uint4(0, 0, 0, 0), qhi = qlo;
        if (gq_ok) {
            const uint4* pq = reinterpret_cast<const uint4*>(q_a + ub + static_cast<size_t>(gq) * kD);
            qlo = pq[g];
            qhi = pq[4 + g];
        }
        __syncthreads();  // the references are in LDS
        float mg[4];
        bool row_ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // the generating query of row 4g + i
            const int r = 4 * g + i;
            const int pos = (r < G) ? gi[r] : -1;
            row_ok[i] = pos >= 0 && pos < A;
            mg[i] = row_ok[i] ? mq_s[pos] : 0.f;
        }
        constexpr int kTiles = (5 * 64) / (16 * W);  // 16-key tiles per wave at 320 keys
        const int ntiles = 2 * nchunks;
        float e[kTiles][4];
        float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            const int t = w + W * k;  // uniform
            const int key = 16 * t + m16;
            f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
            if (t < ntiles) {
                const unsigned char* kt = kall + (t >> 1) * kWgTile;
                const int r = 16 * (t & 1) + m16;
                const uint4 k0 = *reinterpret_cast<const uint4*>(kt + swz(r, g));
                const uint4 k1 = *reinterpret_cast<const uint4*>(kt + swz(r, 4 + g));
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qlo), as_bf16x8(k0), sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qhi), as_bf16x8(k1), sacc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[k][i] = (t < ntiles && key < A && row_ok[i])
                              ? __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -mg[i]))
                              : 0.f;
                l[i] += e[k][i];
            }
        }
        // Row sums: over the 16 lanes of a row, then over the waves in order.
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) l[i] += __shfl_xor(l[i], o, kWave);
        if (m16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) red_s[w * 16 + 4 * g + i] = l[i];
        __syncthreads();
        float inv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = red_s[4 * g + i];
#pragma unroll
            for (int v = 1; v < W; ++v) t += red_s[v * 16 + 4 * g + i];
            inv[i] = row_ok[i] ? 1.f / t : 0.f;
        }
        // Per key: the probabilities summed over the generating queries.
        float* pu = partials + static_cast<size_t>(u) * A;
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            float col = e[k][0] * inv[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) col += e[k][i] * inv[i];
            col += __shfl_xor(col, 16, kWave);
            col += __shfl_xor(col, 32, kWave);
            const int key = 16 * (w + W * k) + m16;
            if (g == 0 && key < A) pu[key] = col;
        }
    }
}

// Dynamic LDS of the cached workgroup kernel: the staged list, the chunk
// flags and (UPDATE) the active positions.
inline size_t cached_wg_lds(bool update, int A, int Nc) {
    // the kernel's chunk count: the active rows padded to whole chunks, then
    // the cached rows
    const int nchunks = (A + kChunk - 1) / kChunk + (Nc + kChunk - 1) / kChunk;
    return static_cast<size_t>((Nc > 0 ? Nc : 1) + nchunks + (update ? A : 0)) * 4;
}
constexpr size_t kCachedWgMaxLds = 48 * 1024;  // + 16 KB of tiles: 64 KB per workgroup

template <bool UPDATE, bool RAGGED, int LAB = kLabNone>
int launch_cached_wg(const uint16_t* q_a, const uint16_t* k_a, const uint16_t* v_a,
                     const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* cached_idx,
                     int ldc, uint16_t* out, float* lse, int B, int H, int N, int A, int Nc,
                     float scale_log2, const int32_t* active_idx, int ld_act, int32_t* err_count,
                     const int32_t* a_len, const int32_t* c_len, hipStream_t stream) {
    const int units = B * H;
    const size_t lds = cached_wg_lds(UPDATE, A, Nc);  // <= kCachedWgMaxLds (checked by the caller)
    auto go = [&](auto nqt_tag, auto waves_tag) {
        constexpr int kNqt = decltype(nqt_tag)::value;
        constexpr int kW = decltype(waves_tag)::value;
        constexpr int kPerBlock = kW * 16 * kNqt;
        const int nb = (A + kPerBlock - 1) / kPerBlock;
        const int grid = (nb == 1) ? units : ((units + 7) / 8) * 8 * nb;
        hipLaunchKernelGGL((attn_wg_kernel<kNqt, kW, UPDATE, true, RAGGED, false, LAB>), dim3(grid),
                           dim3(64 * kW), lds, stream, q_a, k_a, v_a,
                           const_cast<uint16_t*>(k_cache), const_cast<uint16_t*>(v_cache), out,
                           lse, units, A, nb, scale_log2, cached_idx, ldc, H, N, Nc, active_idx,
                           ld_act, err_count, a_len, c_len);
        return status_from_launch();
    };
    using Q4 = std::integral_constant<int, 4>;
    // two waves up to 128 queries, four beyond (more blocks past 256).  (With
    // per-sequence counts, four waves of 48 queries instead, so that a block
    // whose counts sit below the capacity leaves fewer tile slots empty, made
    // the high-res gated layers slower: their sequences past 192 queries then
    // stream the unit's K/V a second time.)
    return (A <= 2 * 64) ? go(Q4{}, std::integral_constant<int, 2>{})
                         : go(Q4{}, std::integral_constant<int, 4>{});
}

}  // namespace
}  // namespace marca
