// cache_attn.hip -- cache-aware attention for KV-cached MAR decoding on gfx950.
//
// Operation ("MARche" paper-notes page, Key Design 2, Eq. 1-2): every active
// query attends over two key/value sources -- the fresh active rows (K_A, V_A)
// and the stored rows of the cached set (K_C, V_C, gathered from the per-layer
// cache through the cached index list) -- and the two partial softmax sums are
// merged with the safe online softmax instead of concatenating the sources.
// Here both sources are streamed through one running (max m, sum l, weighted
// sum o) state: active rows first, cached rows after, in chunks of 32 rows;
// at each chunk boundary (the active/cached boundary among them) the state is
// rescaled by 2^(m_old - m_new), which is the same merge rule.
//
// Five code paths:
//  * attn_mfma_kernel (bf16, A >= 16): one wave per (sequence, head) unit and
//    query group of up to 64 queries.  S^T = K Q^T and O^T = V^T P^T run on
//    v_mfma_f32_16x16x32_bf16; K goes straight from HBM into MFMA operand
//    registers (each lane loads 16-byte pieces of one 128-byte key row), V is
//    staged through a swizzled LDS tile and read back with the transposing
//    ds_read_b64_tr_b16 as the PV operand.  The next chunk's loads are issued
//    before the current chunk is computed.  The unit's cached index list is
//    staged in LDS once.  Separate instantiations serve per-sequence counts,
//    the fused cache update, and the case with no cached rows, whose keys are
//    contiguous rows read at fixed per-lane offsets.  With few units, several
//    waves per unit each stream a range of its chunks and merge their states.
//  * attn_wg_kernel (attn_cached.h; bf16, A > 64, cached rows): a workgroup
//    per unit (per block of its queries) shares each K/V chunk through a
//    double-buffered LDS tile among its 2 or 4 waves, the block's 16-query
//    tiles spread evenly over them (also with per-sequence counts); the same
//    MFMA tiles, with the softmax reference kept in scaled units and the
//    query tiles in pairs.  Its 4 x 80-query form without cached rows serves
//    layer 2's pass that also yields the refresh scores.
//  * attn_dense_kernel (attn_dense.h, with the per-chunk tile math it shares
//    with attn_wg_kernel; bf16, A > 64, no cached rows: the full-attention
//    layers and a refresh step's layers): persistent workgroups of 4 waves x
//    80 queries, whose chunk stream runs on from one (unit, query block) item
//    to the next together with the next item's queries.
//  * attn_f32_mfma_kernel (fp32, A >= 16): one wave per unit and query group,
//    S^T and O^T on v_mfma_f32_16x16x4_f32 with every operand loaded from
//    memory straight into the layout the products take (no LDS tile).
//  * attn_unit_kernel (fp32 below 16 queries or past 8192 tokens, bf16 below
//    16 queries): a workgroup per unit and block of 64 queries streams 64-row
//    K/V chunks through LDS; fp32 FMAs.
//
// Head dim is fixed at 64 (MAR-B/L/H all use 64).  The cached index list is
// sanitised: an entry outside [0, N) is skipped, never dereferenced.  Inputs
// are NaN-free (a precondition of the ABI); this file is compiled with
// -fno-honor-nans, so maxima of matrix-core results need no quieting step.
#include <type_traits>

#include "attn_cached.h"
#include "device_util.h"
#include "launch.h"

namespace marca {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Per-unit vector path (fp32 inputs below 16 active queries or past 8192
// tokens; bf16 below 16 active queries, where a 16-wide MFMA tile would be
// mostly empty): fp32 FMAs throughout.
//
// A workgroup of 4 waves per (sequence, head) unit and block of 64 queries
// streams the unit's virtual sequence [active rows ; cached rows] in chunks
// of 64 rows through LDS, so every K/V row is read from memory once per
// block.  Wave w holds queries 16w .. 16w+15 of the block: lane (kg, qi)
// keeps query qi's 64 scaled elements in registers and scores keys kg + 4i
// (i < 16) of the chunk against the K tile; the chunk's maximum, the
// rescale of the running (max, sum, weighted sum) state -- the merge of the
// two partial softmax sums, applied chunk by chunk across the active/cached
// boundary -- and the probabilities follow; the probabilities go through an
// LDS tile so that lane (kg, qi) can accumulate the weighted sum of V over
// all 64 keys for head dims 16kg .. 16kg+15.  LDS rows are padded to 68
// floats (rows four banks apart), so the reads are conflict-free.  A cached
// entry outside [0, N) and rows past the sequence are masked, never read.
// ---------------------------------------------------------------------------
constexpr int kUnitQ = 64;      // queries per workgroup
constexpr int kUnitChunk = 64;  // key rows per chunk
constexpr int kRowPad = 68;     // floats per LDS row
constexpr int kPPad = 65;       // floats per query row of the probability tile

__device__ __forceinline__ void load16(const float* p, float (&x)[16]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float4 a = reinterpret_cast<const float4*>(p)[c];
        x[4 * c] = a.x; x[4 * c + 1] = a.y; x[4 * c + 2] = a.z; x[4 * c + 3] = a.w;
    }
}
__device__ __forceinline__ void load16(const uint16_t* p, float (&x)[16]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[c];
        const uint32_t wv[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[8 * c + 2 * k] = __uint_as_float(wv[k] << 16);
            x[8 * c + 2 * k + 1] = __uint_as_float(wv[k] & 0xffff0000u);
        }
    }
}
__device__ __forceinline__ void store1(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store1(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

template <typename T>
__global__ __launch_bounds__(256) void attn_unit_kernel(
    const T* __restrict__ q_a, const T* __restrict__ k_a, const T* __restrict__ v_a,
    const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ cached_idx, int ldc, T* __restrict__ out,
    float* __restrict__ lse, int H, int N, int A, int Nc, float scale_log2,
    const int32_t* __restrict__ a_len, const int32_t* __restrict__ c_len) {
    __shared__ __align__(16) float ks[kUnitChunk * kRowPad];
    __shared__ __align__(16) float vs[kUnitChunk * kRowPad];
    __shared__ float ps[4][16 * kPPad];
    __shared__ int rowok_s[kUnitChunk];
    const int tid = threadIdx.x;
    const int w = tid / kWave, lane = tid & (kWave - 1);
    const int qi = lane & 15, kg = lane >> 4;
    const int u = blockIdx.x;
    const int b = u / H;
    // A and Nc are the row stride / list capacity; per-sequence counts may be smaller.
    const int An = (a_len != nullptr) ? min(max(a_len[b], 0), A) : A;
    const int Ncn = (c_len != nullptr) ? min(max(c_len[b], 0), Nc) : Nc;
    if (static_cast<int>(blockIdx.y) * kUnitQ >= An) return;  // uniform, before any barrier
    const int q = blockIdx.y * kUnitQ + 16 * w + qi;             // this lane's query
    const bool has_q = q < An;

    float qr[64];
    {
        const T* qp = q_a + (static_cast<size_t>(u) * A + min(q, An - 1)) * kD;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float x[16];
            load16(qp + 16 * c, x);
#pragma unroll
            for (int e = 0; e < 16; ++e) qr[16 * c + e] = x[e] * scale_log2;
        }
    }
    float m = -INFINITY, l = 0.f, o[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = 0.f;

    const int32_t* cidx = cached_idx + static_cast<size_t>(b) * ldc;
    const int T_rows = An + Ncn;
    const int lrow = tid >> 2, lq = tid & 3;  // loading thread: row, quarter of the row
    for (int r0 = 0; r0 < T_rows; r0 += kUnitChunk) {
        // Load the chunk's K and V rows (a thread: 16 elements of one row).
        {
            const int r = r0 + lrow;
            const T* kp = nullptr;
            const T* vp = nullptr;
            if (r < An) {
                kp = k_a + (static_cast<size_t>(u) * A + r) * kD;
                vp = v_a + (static_cast<size_t>(u) * A + r) * kD;
            } else if (r < T_rows) {
                const int n = cidx[r - An];
                if (n >= 0 && n < N) {
                    kp = k_cache + (static_cast<size_t>(u) * N + n) * kD;
                    vp = v_cache + (static_cast<size_t>(u) * N + n) * kD;
                }
            }
            float kx[16], vx[16];
            if (kp != nullptr) {
                load16(kp + 16 * lq, kx);
                load16(vp + 16 * lq, vx);
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) kx[e] = vx[e] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                *reinterpret_cast<float4*>(ks + lrow * kRowPad + 16 * lq + 4 * c) =
                    make_float4(kx[4 * c], kx[4 * c + 1], kx[4 * c + 2], kx[4 * c + 3]);
                *reinterpret_cast<float4*>(vs + lrow * kRowPad + 16 * lq + 4 * c) =
                    make_float4(vx[4 * c], vx[4 * c + 1], vx[4 * c + 2], vx[4 * c + 3]);
            }
            if (lq == 0) rowok_s[lrow] = (kp != nullptr) ? 1 : 0;
        }
        __syncthreads();
        // Scores of query qi against keys kg + 4i of the chunk.
        float sc[16];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = kg + 4 * i;
            const float* kr = ks + j * kRowPad;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float4 k4 = *reinterpret_cast<const float4*>(kr + 4 * c);
                acc = fmaf(qr[4 * c], k4.x, acc);
                acc = fmaf(qr[4 * c + 1], k4.y, acc);
                acc = fmaf(qr[4 * c + 2], k4.z, acc);
                acc = fmaf(qr[4 * c + 3], k4.w, acc);
            }
            sc[i] = rowok_s[j] ? acc : -INFINITY;
            mx = fmaxf(mx, sc[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float mn = fmaxf(m, mx);
        const float mu = (mn == -INFINITY) ? 0.f : mn;  // no valid key yet: every term is 0
        const float alpha = exp2f(m - mu);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float pv = exp2f(sc[i] - mu);
            ps[w][qi * kPPad + kg + 4 * i] = pv;
            psum += pv;
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        l = l * alpha + psum;
#pragma unroll
        for (int d = 0; d < 16; ++d) o[d] *= alpha;
        m = mn;
        __syncthreads();  // the probability tile is complete
        // o[d] += sum over the chunk's keys j of p(qi, j) * V[j][16kg + d]
        for (int j = 0; j < kUnitChunk; ++j) {
            const float pj = ps[w][qi * kPPad + j];
            const float* vr = vs + j * kRowPad + 16 * kg;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4 v4 = *reinterpret_cast<const float4*>(vr + 4 * c);
                o[4 * c] = fmaf(pj, v4.x, o[4 * c]);
                o[4 * c + 1] = fmaf(pj, v4.y, o[4 * c + 1]);
                o[4 * c + 2] = fmaf(pj, v4.z, o[4 * c + 2]);
                o[4 * c + 3] = fmaf(pj, v4.w, o[4 * c + 3]);
            }
        }
        __syncthreads();  // every wave is done with the tiles
    }
    if (!has_q) return;
    const size_t orow = (static_cast<size_t>(u) * A + q) * kD + 16 * kg;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < 16; ++d) store1(out, orow + d, o[d] * inv);
    if (lse != nullptr && kg == 0)
        lse[static_cast<size_t>(u) * A + q] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// MFMA path (bf16, A >= 16)
//
// One 64-lane wave per (sequence, head) unit and group of up to 16*NQT
// queries.  The virtual key/value sequence [active rows ; cached rows] is
// streamed in chunks of 32 rows; one or two further chunks are in flight
// while one is computed.  Per chunk:
//  * K goes from HBM straight into MFMA operand registers: lane (g, m16)
//    loads 16-byte pieces g and 4+g of key row 16t + m16, which is the A
//    operand layout of S^T = K Q^T on v_mfma_f32_16x16x32_bf16.  Each load
//    instruction reads 64-byte halves of 16 rows.
//  * V is loaded as whole 128-byte rows (lane l: row 8k + l/8, piece l%8, so
//    one instruction reads 8 complete rows), stored to LDS with the 16-byte
//    piece p of row r at slot p ^ (r & 7), and read back with the transposing
//    ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T.
//  * The S^T accumulator layout (lane (g, m16) holds keys 16t + 4g + i of
//    query m16) is directly the B operand P^T of the PV product, with k-slot
//    j <-> key row 16(j>>2) + 4g + (j&3); the V^T reads use the same map.
//  * Online softmax in base 2 with a lazily updated reference max: the state
//    is rescaled only when a score exceeds the reference by more than
//    kRescaleLog2 (in log2 units), so probabilities stay <= 2^kRescaleLog2.
//    Rescaling by 2^(m_old - m_new) folds chunk after chunk -- the active
//    rows first, the cached rows after -- into one (max, sum, weighted sum)
//    state, which is the merge rule of the two partial softmax sums.
//  * The softmax denominator is accumulated by one more MFMA with an all-ones
//    A operand, so numerator and denominator sum the same bf16 probabilities.
// Rows past the end of the sequence and cached entries outside [0, N) load
// active row 0 instead (always valid) and are masked to -inf.  The unit's
// cached index list is staged in LDS once; chunks made only of active rows
// are requested before that list arrives.  The output tile goes through LDS
// so that every store instruction writes whole 128-byte rows.
// ---------------------------------------------------------------------------
constexpr int kQueriesPerGroup = 64;
constexpr int kMaxMfmaTokens = 8192;
// LDS per one-wave workgroup that still fits 8 of them in a CU's 160 KB.
constexpr size_t kStashLdsMax = 20 * 1024;
// Chunks in flight ahead of the one computed: two where the registers allow
// (up to 48 queries per wave), one for 64 queries.
constexpr int prefetch_depth(int nqt) { return nqt <= 3 ? 2 : 1; }

// Row r of the virtual sequence [active ; cached] of one unit: its element
// offset in the active block (is_c false) or the unit's cache rows (is_c
// true), and whether it exists.  Missing rows are active row 0.
__device__ __forceinline__ int row_ofs(int r, int A, int Nc, const int32_t* cidx_s, bool& is_c,
                                       bool& ok) {
    const int c = r - A;
    const bool is_a = r < A;
    const bool in_c = static_cast<unsigned>(c) < static_cast<unsigned>(Nc);
    const int n = cidx_s[in_c ? c : 0];  // the list area holds at least one entry
    ok = is_a || (in_c && n >= 0);
    is_c = !is_a && ok;
    return (is_c ? n : (is_a ? r : 0)) * kD;
}

// Registers of one chunk in flight.
struct ChunkRegs {
    uint4 k[2][2];   // K rows 16t..16t+15 in the whole-row layout (see swap_row_halves)
    uint4 v[4];      // V in the same layout: piece kpiece of row 8k + m16 % 8
    uint32_t valid;  // bit j: key row j of the chunk exists (wave-uniform)
};

// UPDATE: also write the unit's fresh active K/V rows into the caches at
// their token positions (active_idx), from the registers that already hold
// them for the attention.  The rows read from the caches are the cached set,
// which is disjoint from the active positions, so the reads and the writes of
// one unit never touch the same row and different units never share a row.
// RAGGED: per-sequence active / cached counts from a_len / c_len (a separate
// instantiation, so the uniform-count kernel carries none of it).
// SPLIT > 1: few units (small batches).  A workgroup of SPLIT waves per unit,
// each wave streaming its own contiguous range of the unit's chunks; the
// waves' partial (max, sum, weighted sum) states are then merged pairwise
// through LDS with the same rule as the chunk-to-chunk merge, and the first
// wave writes the output.
// DENSE: no cached rows (Nc == 0, the full-attention layers): the unit's keys
// are rows 0..A-1 of k_a/v_a, read with range-checked buffer loads at
// per-lane offsets fixed for the whole sequence.  A row past A reads as zero
// and is masked like a missing row.
// STASH (with UPDATE, one wave per unit): the active rows are copied to LDS as
// they are read and written into the caches after the last chunk, beside the
// output, instead of while the cached rows are being read (the cache writes
// then no longer compete with the reads of every wave's first chunks).
template <int NQT, bool UPDATE, bool RAGGED, bool DENSE, int SPLIT = 1, bool STASH = false>
__global__ __launch_bounds__(64 * SPLIT) __attribute__((amdgpu_waves_per_eu(2, 8)))
void attn_mfma_kernel(const uint16_t* __restrict__ q_a, const uint16_t* __restrict__ k_a,
                      const uint16_t* __restrict__ v_a, const uint16_t* k_cache,
                      const uint16_t* v_cache, const int32_t* __restrict__ cached_idx, int ldc,
                      uint16_t* __restrict__ out, float* __restrict__ lse, int units, int H,
                      int N, int A, int Nc, int n_groups, float scale_log2,
                      const int32_t* __restrict__ active_idx, int ld_act,
                      int32_t* __restrict__ err_count, const int32_t* __restrict__ a_len,
                      const int32_t* __restrict__ c_len) {
    constexpr int kPF = prefetch_depth(NQT);
    static_assert(kPF >= 1 && kPF <= 3, "prefetch depth");
    constexpr int kTileBytes = (16 * NQT * 128 > kChunk * 128) ? 16 * NQT * 128 : kChunk * 128;
    static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4 || SPLIT == 8, "split");
    // With SPLIT > 1 each wave has its own V tile; after the chunks the same
    // bytes hold the partial states being merged (kState floats per lane).
    constexpr int kState = NQT * 18;  // per tile: 16 weighted sums, max, sum
    constexpr int kRegionBytes = (SPLIT / 2) * 64 * kState * 4 > SPLIT * kTileBytes
                                     ? (SPLIT / 2) * 64 * kState * 4
                                     : SPLIT * kTileBytes;
    static_assert(!STASH || (UPDATE && !DENSE && SPLIT == 1), "stash: fused update, one wave");
    extern __shared__ __align__(16) unsigned char smem[];
    const int wv = (SPLIT > 1) ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
    unsigned char* tile = smem + wv * kTileBytes;  // V chunk, later the output tile
    unsigned char* stash = smem + kRegionBytes;    // STASH: [A] K rows, then [A] V rows
    int32_t* cidx_s = reinterpret_cast<int32_t*>(smem + kRegionBytes +
                                                 (STASH ? 2 * A * kD * 2 : 0));  // [max(Nc, 1)]
    int32_t* aidx_s = cidx_s + (Nc > 0 ? Nc : 1);                                // [A] with UPDATE

    const int lane = (SPLIT > 1) ? static_cast<int>(threadIdx.x & 63) : static_cast<int>(threadIdx.x);
    const int g = lane >> 4;    // lane group: k-slot group of the MFMA operands
    const int m16 = lane & 15;  // row / column within a 16x16 tile

    // Work mapping.  With several query groups per unit, the groups of one
    // unit are placed on the same XCD (workgroups are dealt round-robin over
    // the 8 XCDs), so the second group's key/value reads hit that XCD's L2.
    int u, qg;
    if (n_groups == 1) {
        u = blockIdx.x;
        qg = 0;
    } else {
        const int xcd = blockIdx.x & 7;
        const int slot = blockIdx.x >> 3;
        u = (slot / n_groups) * 8 + xcd;
        qg = slot % n_groups;
        if (u >= units) return;  // uniform over the (one-wave) workgroup
    }
    const int b = u / H;
    // A and Nc are the row stride of q_a/k_a/v_a/out and the list capacity;
    // with per-sequence lengths the unit's counts An <= A, Ncn <= Nc.
    int An = A, Ncn = Nc;
    if constexpr (RAGGED) {
        An = min(max(a_len[b], 0), A);
        Ncn = min(max(c_len[b], 0), Nc);
    }
    const int q0 = qg * kQueriesPerGroup;
    if constexpr (RAGGED)
        if (q0 >= An) return;  // no queries in this group (uniform; before any barrier)
    const int nq = min(An - q0, 16 * NQT);  // queries of this group (>= 1)

    const uint16_t* ka_u = k_a + static_cast<size_t>(u) * A * kD;
    const uint16_t* va_u = v_a + static_cast<size_t>(u) * A * kD;
    const uint16_t* kc_u = k_cache + static_cast<size_t>(u) * N * kD;
    const uint16_t* vc_u = v_cache + static_cast<size_t>(u) * N * kD;
    const int T = An + Ncn;
    const int nchunks = (T + kChunk - 1) / kChunk;
    // This wave's chunks [cb, ce) (all of them unless SPLIT > 1).
    int cb = 0, ce = nchunks;
    if constexpr (SPLIT > 1) {
        const int per = (nchunks + SPLIT - 1) / SPLIT;
        cb = min(wv * per, nchunks);
        ce = min(cb + per, nchunks);
    }
    static_assert(!DENSE || !RAGGED, "dense rows: uniform counts only");
    const __amdgpu_buffer_rsrc_t rka = uniform_rsrc(ka_u, An * kD * 2);
    const __amdgpu_buffer_rsrc_t rva = uniform_rsrc(va_u, An * kD * 2);
    const int k_lofs = (m16 & 7) * (kD * 2) + 16 * ((m16 < 8) ? g : 4 + g);  // K: whole rows

    // The first entries of the cached list are requested first: they gate
    // every chunk that holds a cached row.
    constexpr int kIdxRegs = 8;
    const int32_t* cidx_g = cached_idx + static_cast<size_t>(b) * ldc;
    int32_t iv[kIdxRegs];
#pragma unroll
    for (int k = 0; k < kIdxRegs; ++k) {
        const int c = lane + kWave * k;
        iv[k] = (!DENSE && c < Ncn) ? cidx_g[c] : -1;
    }

    // Q tile as the B operand of S^T = K Q^T: lane holds query m16 of tile qt,
    // head dims [8g, 8g+8) (k-step 0) and [32+8g, 32+8g+8) (k-step 1).
    // Queries past the group's end load its last query; they are never stored.
    // Loaded as whole rows (lane: piece kpiece of query 16qt + 8h + m16 % 8)
    // and exchanged into the operand layout.
    const int kpiece = (m16 < 8) ? g : 4 + g;
    bf16x8_t qf[NQT][2];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        uint4 qr[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int qi = q0 + min(qt * 16 + 8 * h + (m16 & 7), nq - 1);
            qr[h] = ld_stream(reinterpret_cast<const uint4*>(
                                  q_a + (static_cast<size_t>(u) * A + qi) * kD) + kpiece);
        }
        uint4 x, y;
        swap_row_halves(qr[0], qr[1], x, y);
        qf[qt][0] = as_bf16x8(x);
        qf[qt][1] = as_bf16x8(y);
    }

    // A chunk at or past the wave's range end (requested only to keep every
    // step's loads alike) is made of rows past the sequence: missing rows,
    // which read active row 0 (one line per load instruction) or, in the
    // dense form, past the buffer (zeros, no memory traffic).
    auto issue = [&](int c, ChunkRegs& cr) __attribute__((always_inline)) {
        const int r0 = (c < ce ? c : nchunks) * kChunk;
        if constexpr (DENSE) {
            const int rb = r0 * (kD * 2);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                cr.v[k] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rva, rb + k_lofs + 1024 * k, 0, kStreamPolicy));
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    cr.k[t][h] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(rka, rb + k_lofs + 2048 * t + 1024 * h,
                                                                     0, kStreamPolicy));
            cr.valid = 0;
            return;
        }
        // K and V as whole rows at one row lookup per 8 rows: lane (g, m16)
        // loads piece kpiece of row 8k + m16 % 8 (k = 2t + h for K); lanes
        // 0..7 see rows 8k + 0..7.  V is requested first: it is consumed
        // first (into LDS).
        uint32_t valid = 0;
        int ofs[4];
        bool cached[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bool ok;
            ofs[k] = row_ofs(r0 + 8 * k + (m16 & 7), An, Ncn, cidx_s, cached[k], ok) + 8 * kpiece;
            valid |= static_cast<uint32_t>(__ballot(ok) & 0xffull) << (8 * k);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            cr.v[k] = ld_stream(reinterpret_cast<const uint4*>((cached[k] ? vc_u : va_u) + ofs[k]));
#pragma unroll
        for (int k = 0; k < 4; ++k)
            cr.k[k >> 1][k & 1] =
                ld_stream(reinterpret_cast<const uint4*>((cached[k] ? kc_u : ka_u) + ofs[k]));
        cr.valid = valid;
    };

    // Stage the cached list (entries outside [0, N) become -1).
    auto stage_list = [&]() __attribute__((always_inline)) {
        if constexpr (DENSE && !UPDATE) return;
#pragma unroll
        for (int k = 0; k < kIdxRegs; ++k) {
            const int c = lane + kWave * k;
            if (c < Ncn) cidx_s[c] = (iv[k] >= 0 && iv[k] < N) ? iv[k] : -1;
        }
        for (int c = lane + kWave * kIdxRegs; c < Ncn; c += kWave) {
            const int n = cidx_g[c];
            cidx_s[c] = (n >= 0 && n < N) ? n : -1;
        }
        if constexpr (UPDATE) {
            // One query group writes each row (see the stores below).  An entry
            // outside [0, N) is skipped and, once per sequence, counted.  With
            // no list (A == N, a full refresh) row r goes to cache row r; the
            // dense instantiation then needs no staged list at all.
            const int32_t* ag = active_idx ? active_idx + static_cast<size_t>(b) * ld_act : nullptr;
            for (int r = lane; r < An && (!DENSE || ag != nullptr); r += kWave) {
                const int n = ag ? ag[r] : r;
                const bool ok = n >= 0 && n < N;
                aidx_s[r] = (ok && (DENSE || qg == 0)) ? n : -1;
                if (!ok && err_count != nullptr && qg == 0 && u % H == 0 && wv == 0)
                    atomicAdd(err_count, 1);
            }
        }
        __syncthreads();  // one wave: orders the list writes before the reads below
    };

    // Chunk i (i < kPF) starts in cr[i].  A first chunk made only of active
    // rows does not need the cached list and is requested before it arrives.
    // When the sequence has fewer than kPF chunks the spare buffers load
    // chunks past the end (never used), so every path issues the same loads.
    ChunkRegs cr[kPF + 1];
    if constexpr (SPLIT == 1) {
        if (An >= kChunk) {
            issue(0, cr[0]);
            stage_list();
        } else {
            stage_list();
            issue(0, cr[0]);
        }
#pragma unroll
        for (int k = 1; k < kPF; ++k) issue(k, cr[k]);
    } else {
        // A wave with no chunks (cb == ce) requests a chunk past its range
        // and never computes it.
        if ((cb + 1) * kChunk <= An) {
            issue(cb, cr[0]);
            stage_list();
        } else {
            stage_list();
            issue(cb, cr[0]);
        }
#pragma unroll
        for (int k = 1; k < kPF; ++k) issue(cb + k, cr[k]);
    }
    // Per-lane LDS byte offsets of the V^T transposing reads: lane s of its
    // 16-lane group addresses key row 16h + 4g + s/4, head dims 16dt + 4(s%4).
    int vofs[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            vofs[h][dt] = swz(16 * h + 4 * g + (m16 >> 2), 2 * dt + ((m16 & 3) >> 1)) +
                          ((m16 & 1) << 3);
    const int vst = swz(m16 & 7, kpiece);  // V store slot, + 1024 per 8 rows

    const float thr_raw = kRescaleLog2 / scale_log2;
    bool tile_on[NQT];
    float mref[NQT], mc[NQT], mthr[NQT];
    f32x4_t oacc[NQT][4], lacc[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        tile_on[qt] = qt * 16 < nq;
        mref[qt] = -INFINITY;
        mthr[qt] = -INFINITY;
        mc[qt] = 0.f;
        lacc[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const bf16x8_t ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));

    auto compute = [&](int c, const ChunkRegs& ch) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<uint4*>(tile + vst + 1024 * k) = ch.v[k];
        if constexpr (UPDATE) {
            // wave-uniform: the chunk holds active rows, written by the
            // unit's first query group (dense: every chunk holds active rows,
            // and the query groups take turns, chunk c written by group
            // c mod n_groups)
            if constexpr (STASH) {
                if (c * kChunk < An) {  // wave-uniform: the chunk holds active rows
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int r = c * kChunk + 8 * k + (m16 & 7);
                        if (r < An) {
                            *reinterpret_cast<uint4*>(stash + swz(r, kpiece)) = ch.k[k >> 1][k & 1];
                            *reinterpret_cast<uint4*>(stash + A * kD * 2 + swz(r, kpiece)) = ch.v[k];
                        }
                    }
                }
            } else if (DENSE ? c % n_groups == qg : c * kChunk < An) {
                // Buffer stores: an offset past the unit's N rows (inactive
                // lane, skipped entry) is dropped by the range check.
                constexpr uint32_t kSkip = 0x80000000u;
                constexpr int kNT = 2;  // cache-policy bits: nontemporal (streaming) store
                const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(kc_u, N * kD * 2);
                const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(vc_u, N * kD * 2);
                // K and V are held as whole rows (see issue): every store
                // writes 8 complete 128-byte rows; K row 8k + m16 % 8 is in
                // k[k / 2][k % 2], V's in v[k].
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = c * kChunk + 8 * k + (m16 & 7);
                    const int n = (r >= An) ? -1 : (DENSE && active_idx == nullptr) ? r : aidx_s[r];
                    const uint32_t off =
                        (n >= 0) ? static_cast<uint32_t>(n) * (kD * 2) + 16 * kpiece : kSkip;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4_t, ch.k[k >> 1][k & 1]), rk, off, 0, kNT);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, ch.v[k]), rv,
                                                           off, 0, kNT);
                }
            }
        }
        bf16x8_t va[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const uint2 lo = lds_tr_b64(tile + vofs[0][dt]);
            const uint2 hi = lds_tr_b64(tile + vofs[1][dt]);
            va[dt] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
        // K rows into the operand layout: kop[t][0] = piece g, kop[t][1] =
        // piece 4 + g of key row 16t + m16.
        uint4 kop[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) swap_row_halves(ch.k[t][0], ch.k[t][1], kop[t][0], kop[t][1]);
        // wave-uniform
        const bool full = DENSE ? (c * kChunk + kChunk <= An) : ch.valid == 0xffffffffu;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            if (!tile_on[qt]) continue;  // wave-uniform
            // S^T tiles: lane holds S^T[key 16t + 4g + i][query m16] in s[t][i].
            f32x4_t s[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[t][0]), qf[qt][0],
                                                              acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[t][1]), qf[qt][1],
                                                              acc, 0, 0, 0);
                s[t] = acc;
            }
            if (!full) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (DENSE ? (c * kChunk + 16 * t + 4 * g + i >= An)
                                  : !((ch.valid >> (16 * t + 4 * g + i)) & 1u))
                            s[t][i] = -INFINITY;
            }
            const float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
            if (__any(mx > mthr[qt])) {  // a query's maximum moved far up: rescale
                const float mnew = fmaxf(mref[qt], max_over_groups(mx));
                const float alpha = (mref[qt] == -INFINITY)
                                        ? 0.f
                                        : __builtin_amdgcn_exp2f((mref[qt] - mnew) * scale_log2);
                lacc[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] *= alpha;
                mref[qt] = mnew;
                mc[qt] = mnew * scale_log2;
                mthr[qt] = mnew + thr_raw;
            }
            float p[8];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p[4 * t + i] = __builtin_amdgcn_exp2f(fmaf(s[t][i], scale_log2, -mc[qt]));
            U4 pk;
            pk.u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                              pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
            lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk.v, lacc[qt], 0, 0, 0);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pk.v,
                                                                       oacc[qt][dt], 0, 0, 0);
        }
    };

    // Chunk c lives in cr[c % (kPF + 1)].  Each step requests chunk c + kPF
    // into the buffer chunk c - 1 just left, then computes chunk c.  Near the
    // end the request is for a chunk past the range (see issue: it reads one
    // line per load, or nothing), so every step issues the same loads and the
    // compiler's memory-counter waits stay exact with kPF chunks in flight (a
    // conditional request would make them wait for everything).  The loop is
    // unrolled by kPF + 1 so every register buffer index is a constant.
    auto step = [&](int c, auto buf_tag) __attribute__((always_inline)) {
        constexpr int BI = decltype(buf_tag)::value;
        constexpr int BN = (BI + kPF) % (kPF + 1);
        __builtin_amdgcn_s_setprio(3);  // requests first: they keep HBM busy
        issue(c + kPF, cr[BN]);
        __builtin_amdgcn_s_setprio(0);
        compute(c, cr[BI]);
    };
    // Whole groups without guards (so the state at the loop back edge is the
    // same on every path), then the last nchunks mod (kPF + 1) chunks.
    int c = cb;
    for (; c + kPF < ce; c += kPF + 1) {
        step(c, std::integral_constant<int, 0>{});
        step(c + 1, std::integral_constant<int, 1>{});
        if constexpr (kPF >= 2) step(c + 2, std::integral_constant<int, 2>{});
        if constexpr (kPF >= 3) step(c + 3, std::integral_constant<int, 3>{});
    }
    if (c < ce) step(c, std::integral_constant<int, 0>{});
    if constexpr (kPF >= 2)
        if (c + 1 < ce) step(c + 1, std::integral_constant<int, 1>{});
    if constexpr (kPF >= 3)
        if (c + 2 < ce) step(c + 2, std::integral_constant<int, 2>{});

    if constexpr (SPLIT > 1) {
        // Pairwise merge: in round r the wave r past a multiple of 2r hands
        // its state to that multiple through LDS.  A state whose maximum is
        // still -inf (the wave saw no valid key) contributes nothing.
        float* mbuf = reinterpret_cast<float*>(smem);
        __syncthreads();  // every wave is done with its V tile
#pragma unroll
        for (int r = 1; r < SPLIT; r <<= 1) {
            float* st = mbuf + (wv / (2 * r)) * (64 * kState);
            if ((wv & (2 * r - 1)) == r) {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            st[(qt * 18 + 4 * dt + i) * 64 + lane] = oacc[qt][dt][i];
                    st[(qt * 18 + 16) * 64 + lane] = mref[qt];
                    st[(qt * 18 + 17) * 64 + lane] = lacc[qt][0];
                }
            }
            __syncthreads();
            if ((wv & (2 * r - 1)) == 0) {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    const float mb = st[(qt * 18 + 16) * 64 + lane];
                    const float lb = st[(qt * 18 + 17) * 64 + lane];
                    const bool va = mref[qt] != -INFINITY;
                    const bool vb = mb != -INFINITY;
                    const float mcb = mb * scale_log2;
                    const float mcm = fmaxf(va ? mc[qt] : -INFINITY, vb ? mcb : -INFINITY);
                    const float fa = va ? __builtin_amdgcn_exp2f(mc[qt] - mcm) : 0.f;
                    const float fb = vb ? __builtin_amdgcn_exp2f(mcb - mcm) : 0.f;
                    const float l = lacc[qt][0] * fa + lb * fb;
                    lacc[qt] = f32x4_t{l, l, l, l};
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            oacc[qt][dt][i] =
                                oacc[qt][dt][i] * fa + st[(qt * 18 + 4 * dt + i) * 64 + lane] * fb;
                    if (vb && (!va || mb > mref[qt])) {
                        mref[qt] = mb;
                        mc[qt] = mcb;
                    }
                }
            }
            __syncthreads();
        }
        if (wv != 0) return;  // after the last barrier
    }

    if constexpr (STASH) {
        // The stashed active rows into the caches at their token positions:
        // 8 whole rows per store, skipped entries dropped by the range check.
        __syncthreads();  // one wave: orders the stash writes before the reads
        constexpr uint32_t kSkip = 0x80000000u;
        const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(kc_u, N * kD * 2);
        const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(vc_u, N * kD * 2);
        for (int k = 0; k < (An + 7) / 8; ++k) {
            const int r = 8 * k + (m16 & 7);
            const int n = (r < An) ? aidx_s[r] : -1;
            const uint32_t off = (n >= 0) ? static_cast<uint32_t>(n) * (kD * 2) + 16 * kpiece : kSkip;
            const uint4 kr = *reinterpret_cast<const uint4*>(stash + swz(r, kpiece));
            const uint4 vr = *reinterpret_cast<const uint4*>(stash + A * kD * 2 + swz(r, kpiece));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, kr), rk, off, 0,
                                                   kStreamPolicy);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, vr), rv, off, 0,
                                                   kStreamPolicy);
        }
    }

    // Finalise: lane holds O[query 16qt + m16][16dt + 4g + i] = oacc[qt][dt][i]
    // and the softmax denominator of that query in every lacc[qt][i].  The
    // tile goes through LDS (same swizzle) and leaves as whole rows.
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        if (!tile_on[qt]) continue;
        const float l = lacc[qt][0];
        const float inv = 1.f / l;
        const int row = 16 * qt + m16;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const uint2 w = make_uint2(pack_bf16x2(oacc[qt][dt][0] * inv, oacc[qt][dt][1] * inv),
                                       pack_bf16x2(oacc[qt][dt][2] * inv, oacc[qt][dt][3] * inv));
            *reinterpret_cast<uint2*>(tile + swz(row, 2 * dt + (g >> 1)) + ((g & 1) << 3)) = w;
        }
        const int qi = q0 + row;
        if (lse != nullptr && g == 0 && row < nq)
            lse[static_cast<size_t>(u) * A + qi] = (mc[qt] + log2f(l)) * kLn2;
    }
    if constexpr (SPLIT > 1)
        __builtin_amdgcn_wave_barrier();  // only the first wave is left
    else
        __syncthreads();  // one wave: orders the tile writes before the reads
    u32x4_t* orow = reinterpret_cast<u32x4_t*>(out + (static_cast<size_t>(u) * A + q0) * kD);
#pragma unroll
    for (int k = 0; k < 2 * NQT; ++k) {
        const int row = 8 * k + (lane >> 3);
        if (row < nq) {
            const u32x4_t w = *reinterpret_cast<const u32x4_t*>(tile + swz(row, lane & 7));
            __builtin_nontemporal_store(w, orow + row * 8 + (lane & 7));
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 matrix-core path (fp32 inputs, A >= 16): one wave per (sequence, head)
// unit and group of up to 16*NQT queries, as attn_mfma_kernel, on
// v_mfma_f32_16x16x4_f32 (lane l supplies A[l%16][l/16] and B[l/16][l%16];
// the output has lane l holding rows 4(l/16)..4(l/16)+3 of column l%16).
// Which head dims or keys a product's four k-slots take, and which dims its
// output rows stand for, is free as long as the operands agree, so every
// operand comes from memory already in place and there is no LDS tile:
//  * S^T = K Q^T over 16-key chunks, in 16 steps: step 4j + e gives lane
//    (g, m) head dim 16j + 4g + e of key row m and of query m.  Load j of a
//    lane is floats [16j + 4g, +4) of its row, so one load instruction reads
//    64 contiguous bytes of each of 16 rows.  The output gives lane (g, m) the
//    scores of keys 4g..4g+3 against query m.
//  * O^T = V^T P^T, per 16-dim output tile dt, in 4 steps: step s gives lane
//    (g, m) key 4g + s, i.e. its own probability p[s] as the B operand and
//    V[key 4g+s][dim pi(dt, m)] as the A operand, with output row i of tile
//    dt standing for dim pi(dt, i) = 16(i % 4) + 4(i / 4) + dt.  A lane loads
//    V rows 4g..4g+3 at floats [16(m % 4) + 4(m / 4), +4) (16 lanes read each
//    whole row) and ends holding O[m][16r + 4g + dt] = oacc[dt][r], stored
//    with one instruction per r writing 64 contiguous bytes of 16 rows.
// The softmax state follows attn_mfma_kernel (a reference maximum per query,
// the state rescaled when a chunk's maximum passes it by kRescaleLog2); the
// probabilities stay in fp32, and each lane keeps the row sum over its own
// keys, summed over the four lane groups at the end.  The cached list is
// staged in LDS; missing rows read active row 0 and are masked.
// ---------------------------------------------------------------------------
constexpr int kF32Chunk = 16;  // key rows per chunk

// Sum over lanes l, l^16, l^32, l^48 (register-only lane swaps).
__device__ __forceinline__ float sum_over_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(x);
    auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Registers of one fp32 chunk in flight: K floats [16j + 4g, +4) of key row m
// (j < 4), V floats [16(m % 4) + 4(m / 4), +4) of key rows 4g+s, and the
// chunk's row mask.
struct F32Chunk {
    float4 k[4];
    float4 v[4];
    uint32_t valid;  // bit j: key row j of the chunk exists (wave-uniform)
};

template <int NQT, bool RAGGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void attn_f32_mfma_kernel(const float* __restrict__ q_a, const float* __restrict__ k_a,
                          const float* __restrict__ v_a, const float* __restrict__ k_cache,
                          const float* __restrict__ v_cache, const int32_t* __restrict__ cached_idx,
                          int ldc, float* __restrict__ out, float* __restrict__ lse, int units,
                          int H, int N, int A, int Nc, int n_groups, float scale_log2,
                          const int32_t* __restrict__ a_len, const int32_t* __restrict__ c_len) {
    constexpr int kPF = (NQT <= 3) ? 2 : 1;  // chunks in flight
    extern __shared__ __align__(16) int32_t f32_cidx_s[];  // [max(Nc, 1)]
    const int lane = threadIdx.x;
    const int g = lane >> 4;
    const int m = lane & 15;

    // The query groups of one unit sit on one XCD (workgroups go round-robin
    // over the 8), so the later groups' K/V reads hit that XCD's L2.
    int u, qg;
    if (n_groups == 1) {
        u = blockIdx.x;
        qg = 0;
    } else {
        const int xcd = blockIdx.x & 7;
        const int slot = blockIdx.x >> 3;
        u = (slot / n_groups) * 8 + xcd;
        qg = slot % n_groups;
        if (u >= units) return;  // uniform (one-wave workgroup)
    }
    const int b = u / H;
    int An = A, Ncn = Nc;
    if constexpr (RAGGED) {
        An = min(max(a_len[b], 0), A);
        Ncn = min(max(c_len[b], 0), Nc);
    }
    const int q0 = qg * kQueriesPerGroup;
    if (q0 >= An) return;  // no queries in this group (uniform; RAGGED only)
    const int nq = min(An - q0, 16 * NQT);

    const float* ka_u = k_a + static_cast<size_t>(u) * A * kD;
    const float* va_u = v_a + static_cast<size_t>(u) * A * kD;
    const float* kc_u = k_cache + static_cast<size_t>(u) * N * kD;
    const float* vc_u = v_cache + static_cast<size_t>(u) * N * kD;
    const int T = An + Ncn;
    const int nchunks = (T + kF32Chunk - 1) / kF32Chunk;

    // The list's first entries are requested before the queries.
    constexpr int kIdxRegs = 8;
    const int32_t* cidx_g = cached_idx + static_cast<size_t>(b) * ldc;
    int32_t iv[kIdxRegs];
#pragma unroll
    for (int k = 0; k < kIdxRegs; ++k) {
        const int c = lane + kWave * k;
        iv[k] = (c < Ncn) ? cidx_g[c] : -1;
    }
    // Query operands: lane (g, m) holds floats [16j + 4g, +4) (j < 4) of
    // query 16qt + m (past the group's end: its last query, never stored).
    float4 qv[NQT][4];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int qi = q0 + min(16 * qt + m, nq - 1);
        const float4* qp = reinterpret_cast<const float4*>(q_a + (static_cast<size_t>(u) * A + qi) * kD);
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[qt][j] = ld_stream(qp + 4 * j + g);
    }
    // Stage the cached list (entries outside [0, N) become -1).
#pragma unroll
    for (int k = 0; k < kIdxRegs; ++k) {
        const int c = lane + kWave * k;
        if (c < Ncn) f32_cidx_s[c] = (iv[k] >= 0 && iv[k] < N) ? iv[k] : -1;
    }
    for (int c = lane + kWave * kIdxRegs; c < Ncn; c += kWave) {
        const int n = cidx_g[c];
        f32_cidx_s[c] = (n >= 0 && n < N) ? n : -1;
    }
    __syncthreads();  // one wave: orders the list writes before the reads

    auto issue = [&](int c, F32Chunk& cr) __attribute__((always_inline)) {
        const int r0 = c * kF32Chunk;
        bool is_c, ok;
        const int ko = row_ofs(r0 + m, An, Ncn, f32_cidx_s, is_c, ok) + 4 * g;
        cr.valid = static_cast<uint32_t>(__ballot(ok) & 0xffffull);
        const float4* kp = reinterpret_cast<const float4*>((is_c ? kc_u : ka_u) + ko);
#pragma unroll
        for (int j = 0; j < 4; ++j) cr.k[j] = ld_stream(kp + 4 * j);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bool vc, vok;
            const int vo = row_ofs(r0 + 4 * g + s, An, Ncn, f32_cidx_s, vc, vok) + 16 * (m & 3) + 4 * (m >> 2);
            cr.v[s] = ld_stream(reinterpret_cast<const float4*>((vc ? vc_u : va_u) + vo));
        }
    };

    const float thr_raw = kRescaleLog2 / scale_log2;
    float mref[NQT], mc[NQT], mthr[NQT], lsum[NQT];
    f32x4_t oacc[NQT][4];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        mref[qt] = -INFINITY;
        mthr[qt] = -INFINITY;
        mc[qt] = 0.f;
        lsum[qt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    auto f4 = [](const float4& x, int j) __attribute__((always_inline)) {
        return j == 0 ? x.x : (j == 1 ? x.y : (j == 2 ? x.z : x.w));
    };

    auto compute = [&](const F32Chunk& ch) __attribute__((always_inline)) {
        // S^T tiles of all query tiles, step by step (NQT independent chains).
        f32x4_t sc[NQT];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) sc[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 16; ++s)
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
                sc[qt] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4(ch.k[s >> 2], s & 3),
                                                              f4(qv[qt][s >> 2], s & 3), sc[qt], 0,
                                                              0, 0);
        // Masking, then every tile's probabilities against its current
        // reference before the one rescale test of the chunk, which only
        // decides whether they are taken again (rare).  Tiles past the
        // group's queries repeat its last query and are never stored; they
        // are computed too, so the chunk stays one basic block.
        if (ch.valid != 0xffffu) {  // wave-uniform
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((ch.valid >> (4 * g + i)) & 1u)) sc[qt][i] = -INFINITY;
        }
        float mx[NQT], p[NQT][4];
        bool up = false;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            mx[qt] = fmaxf(fmaxf(sc[qt][0], sc[qt][1]), fmaxf(sc[qt][2], sc[qt][3]));
            up = up || (mx[qt] > mthr[qt]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[qt][i] = __builtin_amdgcn_exp2f(fmaf(sc[qt][i], scale_log2, -mc[qt]));
        }
        if (__builtin_expect(__any(up), 0)) {  // a query's maximum moved far up: rescale
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const float mnew = fmaxf(mref[qt], max_over_groups(mx[qt]));
                if (mnew > mthr[qt] || mref[qt] == -INFINITY) {
                    const float alpha = (mref[qt] == -INFINITY)
                                            ? 0.f
                                            : __builtin_amdgcn_exp2f((mref[qt] - mnew) * scale_log2);
                    lsum[qt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] *= alpha;
                    mref[qt] = mnew;
                    mc[qt] = mnew * scale_log2;
                    mthr[qt] = mnew + thr_raw;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        p[qt][i] = __builtin_amdgcn_exp2f(fmaf(sc[qt][i], scale_log2, -mc[qt]));
                }
            }
        }
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            lsum[qt] += (p[qt][0] + p[qt][1]) + (p[qt][2] + p[qt][3]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4(ch.v[s], dt), p[qt][s],
                                                                       oacc[qt][dt], 0, 0, 0);
        }
    };

    // Chunk c lives in cr[c % (kPF + 1)]; each step requests chunk c + kPF
    // (past the end: rows that do not exist, which read active row 0) and
    // computes chunk c, so every step issues the same loads.
    F32Chunk cr[kPF + 1];
#pragma unroll
    for (int k = 0; k < kPF; ++k) issue(k, cr[k]);
    auto step = [&](int c, auto buf_tag) __attribute__((always_inline)) {
        constexpr int BI = decltype(buf_tag)::value;
        constexpr int BN = (BI + kPF) % (kPF + 1);
        issue(c + kPF, cr[BN]);
        compute(cr[BI]);
    };
    int c = 0;
    for (; c + kPF < nchunks; c += kPF + 1) {
        step(c, std::integral_constant<int, 0>{});
        step(c + 1, std::integral_constant<int, 1>{});
        if constexpr (kPF >= 2) step(c + 2, std::integral_constant<int, 2>{});
    }
    if (c < nchunks) step(c, std::integral_constant<int, 0>{});
    if constexpr (kPF >= 2)
        if (c + 1 < nchunks) step(c + 1, std::integral_constant<int, 1>{});

    // Finalise: lane (g, m) writes dims [16r + 4g, +4) (r < 4) of query 16qt + m.
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int row = 16 * qt + m;
        if (16 * qt >= nq) continue;  // wave-uniform
        const float l = sum_over_groups(lsum[qt]);
        const float inv = 1.f / l;
        if (row < nq) {
            float4* orow = reinterpret_cast<float4*>(out + (static_cast<size_t>(u) * A + q0 + row) * kD + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float4 w = make_float4(oacc[qt][0][r] * inv, oacc[qt][1][r] * inv,
                                             oacc[qt][2][r] * inv, oacc[qt][3][r] * inv);
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, w),
                                            reinterpret_cast<u32x4_t*>(orow + 4 * r));
            }
            if (lse != nullptr && g == 0)
                lse[static_cast<size_t>(u) * A + q0 + row] = (mc[qt] + log2f(l)) * kLn2;
        }
    }
}


// Layer 2's full attention with the refresh partials (SCORES): one workgroup
// of 4 waves x 80 queries per unit of at most 320 tokens; dynamic LDS: the K
// chunks, the query references and the cross-wave sums.
int launch_scores_wg(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                     float* lse, const int32_t* gen_idx, int ld_gen, int G, float* partials,
                     int B, int H, int N, float scale_log2, hipStream_t stream) {
    const int units = B * H;
    const int nchunks = (N + kChunk - 1) / kChunk;
    const size_t lds = static_cast<size_t>(nchunks) * kWgTile + static_cast<size_t>(nchunks) * kChunk * 4 +
                       kWgWaves * 16 * 4;
    hipLaunchKernelGGL((attn_wg_kernel<kWgNqt, kWgWaves, false, false, false, true>), dim3(units),
                       dim3(64 * kWgWaves), lds, stream, q, k, v, const_cast<uint16_t*>(k),
                       const_cast<uint16_t*>(v), out, lse, units, N, 1, scale_log2, nullptr, 0, H,
                       N, 0, nullptr, 0, nullptr, nullptr, nullptr, gen_idx, ld_gen, G, partials);
    return status_from_launch();
}

template <int NQT, bool UPDATE>
int launch_mfma(const uint16_t* q_a, const uint16_t* k_a, const uint16_t* v_a,
                const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* cached_idx,
                int ldc, uint16_t* out, float* lse, int B, int H, int N, int A, int Nc,
                int n_groups, float scale_log2, const int32_t* active_idx, int ld_act,
                int32_t* err_count, const int32_t* a_len, const int32_t* c_len,
                hipStream_t stream) {
    const int units = B * H;
    const int grid = (n_groups == 1) ? units : ((units + 7) / 8) * 8 * n_groups;
    constexpr size_t kTileBytes = (16 * NQT * 128 > kChunk * 128) ? 16 * NQT * 128 : kChunk * 128;
    const bool dense = a_len == nullptr && Nc == 0;  // no cached rows
    const bool list = UPDATE && (active_idx != nullptr || !dense);
    const size_t lds = kTileBytes + static_cast<size_t>(Nc > 0 ? Nc : 1) * 4 +
                       (list ? static_cast<size_t>(A) * 4 : 0);
    if (dense) {
        hipLaunchKernelGGL((attn_mfma_kernel<NQT, UPDATE, false, true>), dim3(grid), dim3(64), lds,
                           stream, q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse,
                           units, H, N, A, Nc, n_groups, scale_log2, active_idx, ld_act,
                           err_count, a_len, c_len);
        return status_from_launch();
    }
    // The fused update stashes the active rows in LDS when the stash still
    // leaves room for two waves per SIMD (8 one-wave workgroups per CU).
    const size_t lds_stash = lds + static_cast<size_t>(A) * kD * 2 * 2;
    if constexpr (UPDATE) {
        if (a_len == nullptr && n_groups == 1 && lds_stash <= kStashLdsMax) {
            hipLaunchKernelGGL((attn_mfma_kernel<NQT, true, false, false, 1, true>), dim3(grid),
                               dim3(64), lds_stash, stream, q_a, k_a, v_a, k_cache, v_cache,
                               cached_idx, ldc, out, lse, units, H, N, A, Nc, n_groups,
                               scale_log2, active_idx, ld_act, err_count, a_len, c_len);
            return status_from_launch();
        }
    }
    if (a_len != nullptr)
        hipLaunchKernelGGL((attn_mfma_kernel<NQT, UPDATE, true, false>), dim3(grid), dim3(64), lds,
                           stream, q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse,
                           units, H, N, A, Nc, n_groups, scale_log2, active_idx, ld_act,
                           err_count, a_len, c_len);
    else
        hipLaunchKernelGGL((attn_mfma_kernel<NQT, UPDATE, false, false>), dim3(grid), dim3(64), lds,
                           stream, q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse,
                           units, H, N, A, Nc, n_groups, scale_log2, active_idx, ld_act,
                           err_count, a_len, c_len);
    return status_from_launch();
}

// Waves per workgroup for few units: double while the (unit, group) count
// times the waves stays within a quarter of the chip's wave slots (256 CUs x
// 8; with more work items the one-wave kernel already keeps HBM busy, and a
// split of 768 MAR-B units measured slower) and every wave keeps at least one
// chunk; 4 at most with 64 queries per group (the merge's LDS).
constexpr int kWaveSlots = 2048 / 4;
constexpr size_t split_region(int nqt, int split) {
    const size_t tile = (16 * nqt * 128 > kChunk * 128) ? 16 * nqt * 128 : kChunk * 128;
    const size_t merge = static_cast<size_t>(split / 2) * 64 * nqt * 18 * 4;
    return merge > split * tile ? merge : split * tile;
}
inline size_t split_lds(int nqt, int split, bool update, int A, int Nc) {
    return split_region(nqt, split) + static_cast<size_t>(Nc > 0 ? Nc : 1) * 4 +
           (update ? static_cast<size_t>(A) * 4 : 0);
}
inline int split_for(int units, int n_groups, int nchunks, int nqt) {
    const int cap = (nqt >= 4) ? 4 : 8;
    int s = 1;
    while (s < cap && static_cast<long>(units) * n_groups * 2 * s <= kWaveSlots &&
           nchunks >= 2 * s)
        s *= 2;
    return s;
}

// SPLIT > 1: one workgroup of SPLIT waves per (unit, query group).
template <int NQT, bool UPDATE, int SPLIT>
int launch_split(const uint16_t* q_a, const uint16_t* k_a, const uint16_t* v_a,
                 const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* cached_idx,
                 int ldc, uint16_t* out, float* lse, int B, int H, int N, int A, int Nc,
                 int n_groups, float scale_log2, const int32_t* active_idx, int ld_act,
                 int32_t* err_count, const int32_t* a_len, const int32_t* c_len,
                 hipStream_t stream) {
    const int units = B * H;
    const int grid = (n_groups == 1) ? units : ((units + 7) / 8) * 8 * n_groups;
    static_assert(split_region(NQT, SPLIT) <= 56 * 1024, "split workgroup LDS");
    const size_t lds = split_lds(NQT, SPLIT, UPDATE, A, Nc);  // <= 64 KB (checked by the caller)
    if (a_len != nullptr)
        hipLaunchKernelGGL((attn_mfma_kernel<NQT, UPDATE, true, false, SPLIT>), dim3(grid),
                           dim3(64 * SPLIT), lds, stream, q_a, k_a, v_a, k_cache, v_cache,
                           cached_idx, ldc, out, lse, units, H, N, A, Nc, n_groups, scale_log2,
                           active_idx, ld_act, err_count, a_len, c_len);
    else
        hipLaunchKernelGGL((attn_mfma_kernel<NQT, UPDATE, false, false, SPLIT>), dim3(grid),
                           dim3(64 * SPLIT), lds, stream, q_a, k_a, v_a, k_cache, v_cache,
                           cached_idx, ldc, out, lse, units, H, N, A, Nc, n_groups, scale_log2,
                           active_idx, ld_act, err_count, a_len, c_len);
    return status_from_launch();
}

template <int NQT, bool UPDATE>
int launch_maybe_split(const uint16_t* q, const uint16_t* ka, const uint16_t* va,
                       const uint16_t* kc, const uint16_t* vc, const int32_t* cached_idx,
                       int ldc, uint16_t* o, float* lse, int B, int H, int N, int A, int Nc,
                       int n_groups, float scale_log2, const int32_t* active_idx, int ld_act,
                       int32_t* err_count, const int32_t* a_len, const int32_t* c_len,
                       hipStream_t stream) {
    const bool dense = a_len == nullptr && Nc == 0;
    int split = dense ? 1 : split_for(B * H, n_groups, (A + Nc + kChunk - 1) / kChunk, NQT);
    // fewer waves when the staged lists would not fit the workgroup's 64 KB
    while (split > 1 && split_lds(NQT, split, UPDATE, A, Nc) > 64 * 1024) split /= 2;
    switch (split) {
        case 2:
            return launch_split<NQT, UPDATE, 2>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H,
                                                N, A, Nc, n_groups, scale_log2, active_idx, ld_act,
                                                err_count, a_len, c_len, stream);
        case 4:
            return launch_split<NQT, UPDATE, 4>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H,
                                                N, A, Nc, n_groups, scale_log2, active_idx, ld_act,
                                                err_count, a_len, c_len, stream);
        case 8:
            if constexpr (NQT < 4)
                return launch_split<NQT, UPDATE, 8>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B,
                                                    H, N, A, Nc, n_groups, scale_log2, active_idx,
                                                    ld_act, err_count, a_len, c_len, stream);
            [[fallthrough]];
        default:
            return launch_mfma<NQT, UPDATE>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H, N,
                                            A, Nc, n_groups, scale_log2, active_idx, ld_act,
                                            err_count, a_len, c_len, stream);
    }
}

template <bool UPDATE>
int dispatch_mfma(const uint16_t* q, const uint16_t* ka, const uint16_t* va, const uint16_t* kc,
                  const uint16_t* vc, const int32_t* cached_idx, int ldc, uint16_t* o, float* lse,
                  int B, int H, int N, int A, int Nc, float scale_log2, const int32_t* active_idx,
                  int ld_act, int32_t* err_count, const int32_t* a_len, const int32_t* c_len,
                  hipStream_t stream) {
    // All tokens active and no cached rows, more queries than one wave holds:
    // the workgroup kernel (with UPDATE only for the full refresh, row r to
    // cache row r).
    if (a_len == nullptr && Nc == 0 && A > kQueriesPerGroup &&
        (!UPDATE || active_idx == nullptr))
        return launch_dense_wg<UPDATE>(q, ka, va, const_cast<uint16_t*>(kc),
                                       const_cast<uint16_t*>(vc), o, lse, B, H, A, scale_log2,
                                       stream);
    const int n_groups = (A + kQueriesPerGroup - 1) / kQueriesPerGroup;
    // Cached rows and several query groups per unit (capacities, with
    // per-sequence counts): the workgroup kernel shares each chunk among the
    // unit's groups, unless there are so few units that several waves per
    // unit (one per chunk range) fill the chip better, or the staged lists
    // would not fit.
    if (Nc > 0 && n_groups > 1 && cached_wg_lds(UPDATE, A, Nc) <= kCachedWgMaxLds &&
        split_for(B * H, n_groups, (A + Nc + kChunk - 1) / kChunk, 4) == 1) {
        if (a_len == nullptr)
            return launch_cached_wg<UPDATE, false>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B,
                                                   H, N, A, Nc, scale_log2, active_idx, ld_act,
                                                   err_count, nullptr, nullptr, stream);
        return launch_cached_wg<UPDATE, true>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H, N,
                                              A, Nc, scale_log2, active_idx, ld_act, err_count,
                                              a_len, c_len, stream);
    }
    const int nqt = (n_groups > 1) ? 4 : (A + 15) / 16;
    switch (nqt) {
        case 1:
            return launch_maybe_split<1, UPDATE>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H,
                                                 N, A, Nc, n_groups, scale_log2, active_idx,
                                                 ld_act, err_count, a_len, c_len, stream);
        case 2:
            return launch_maybe_split<2, UPDATE>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H,
                                                 N, A, Nc, n_groups, scale_log2, active_idx,
                                                 ld_act, err_count, a_len, c_len, stream);
        case 3:
            return launch_maybe_split<3, UPDATE>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H,
                                                 N, A, Nc, n_groups, scale_log2, active_idx,
                                                 ld_act, err_count, a_len, c_len, stream);
        default:
            return launch_maybe_split<4, UPDATE>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H,
                                                 N, A, Nc, n_groups, scale_log2, active_idx,
                                                 ld_act, err_count, a_len, c_len, stream);
    }
}

}  // namespace

namespace {

// fp32 inputs, A >= 16: attn_f32_mfma_kernel, one wave per (unit, group of up
// to 64 queries), the groups of a unit on one XCD.
int launch_f32_mfma(const float* q_a, const float* k_a, const float* v_a, const float* k_cache,
                    const float* v_cache, const int32_t* cached_idx, int ldc, float* out,
                    float* lse, int B, int H, int N, int A, int Nc, float scale_log2,
                    const int32_t* a_len, const int32_t* c_len, hipStream_t stream) {
    const int units = B * H;
    const int n_groups = (A + kQueriesPerGroup - 1) / kQueriesPerGroup;
    const int grid = (n_groups == 1) ? units : ((units + 7) / 8) * 8 * n_groups;
    const size_t lds = static_cast<size_t>(Nc > 0 ? Nc : 1) * 4;
    const int nqt = (n_groups > 1) ? 4 : (A + 15) / 16;
    auto go = [&](auto nqt_tag) {
        constexpr int kNqt = decltype(nqt_tag)::value;
        if (a_len != nullptr)
            hipLaunchKernelGGL((attn_f32_mfma_kernel<kNqt, true>), dim3(grid), dim3(64), lds,
                               stream, q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse,
                               units, H, N, A, Nc, n_groups, scale_log2, a_len, c_len);
        else
            hipLaunchKernelGGL((attn_f32_mfma_kernel<kNqt, false>), dim3(grid), dim3(64), lds,
                               stream, q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse,
                               units, H, N, A, Nc, n_groups, scale_log2, a_len, c_len);
        return status_from_launch();
    };
    switch (nqt) {
        case 1: return go(std::integral_constant<int, 1>{});
        case 2: return go(std::integral_constant<int, 2>{});
        case 3: return go(std::integral_constant<int, 3>{});
        default: return go(std::integral_constant<int, 4>{});
    }
}

int launch_attn_impl(const void* q_a, const void* k_a, const void* v_a, const void* k_cache,
                     const void* v_cache, const int32_t* cached_idx, int ldc, void* out,
                     float* lse, int B, int H, int N, int A, int Nc, float scale, int dtype,
                     const int32_t* a_len, const int32_t* c_len, void* stream_v) {
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    const float scale_log2 = scale * kLog2e;
    if (cached_idx == nullptr) ldc = 0;  // only legal with Nc == 0: never dereferenced
    if (dtype == MAR_BF16 && A >= 16 && N <= kMaxMfmaTokens) {
        const uint16_t* q = static_cast<const uint16_t*>(q_a);
        const uint16_t* ka = static_cast<const uint16_t*>(k_a);
        const uint16_t* va = static_cast<const uint16_t*>(v_a);
        const uint16_t* kc = static_cast<const uint16_t*>(k_cache);
        const uint16_t* vc = static_cast<const uint16_t*>(v_cache);
        uint16_t* o = static_cast<uint16_t*>(out);
        return dispatch_mfma<false>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H, N, A, Nc,
                                    scale_log2, nullptr, 0, nullptr, a_len, c_len, stream);
    }
    if (dtype == MAR_F32 && A >= 16 && N <= kMaxMfmaTokens)
        return launch_f32_mfma(static_cast<const float*>(q_a), static_cast<const float*>(k_a),
                               static_cast<const float*>(v_a), static_cast<const float*>(k_cache),
                               static_cast<const float*>(v_cache), cached_idx, ldc,
                               static_cast<float*>(out), lse, B, H, N, A, Nc, scale_log2, a_len,
                               c_len, static_cast<hipStream_t>(stream_v));
    const dim3 grid(B * H, (A + kUnitQ - 1) / kUnitQ);
    if (dtype == MAR_BF16) {
        hipLaunchKernelGGL(attn_unit_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(q_a), static_cast<const uint16_t*>(k_a),
                           static_cast<const uint16_t*>(v_a), static_cast<const uint16_t*>(k_cache),
                           static_cast<const uint16_t*>(v_cache), cached_idx, ldc,
                           static_cast<uint16_t*>(out), lse, H, N, A, Nc, scale_log2, a_len,
                           c_len);
    } else {
        hipLaunchKernelGGL(attn_unit_kernel<float>, grid, dim3(256), 0, stream,
                           static_cast<const float*>(q_a), static_cast<const float*>(k_a),
                           static_cast<const float*>(v_a), static_cast<const float*>(k_cache),
                           static_cast<const float*>(v_cache), cached_idx, ldc,
                           static_cast<float*>(out), lse, H, N, A, Nc, scale_log2, a_len, c_len);
    }
    return status_from_launch();
}

}  // namespace

int launch_cache_attn(const void* q_a, const void* k_a, const void* v_a, const void* k_cache,
                      const void* v_cache, const int32_t* cached_idx, int ldc, void* out,
                      float* lse, int B, int H, int N, int A, int Nc, float scale, int dtype,
                      void* stream_v) {
    return launch_attn_impl(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse, B, H, N,
                            A, Nc, scale, dtype, nullptr, nullptr, stream_v);
}

int launch_cache_attn_ragged(const void* q_a, const void* k_a, const void* v_a,
                             const void* k_cache, const void* v_cache, const int32_t* cached_idx,
                             int ldc, const int32_t* a_len, const int32_t* c_len, void* out,
                             float* lse, int B, int H, int N, int A, int Nc, float scale,
                             int dtype, void* stream_v) {
    return launch_attn_impl(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse, B, H, N,
                            A, Nc, scale, dtype, a_len, c_len, stream_v);
}

int launch_cache_attn_scores(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* gen_idx, int ld_gen, int G, float* partials, int B,
                             int H, int N, float scale, void* stream_v) {
    return launch_scores_wg(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                            static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse,
                            gen_idx, ld_gen, G, partials, B, H, N, scale * kLog2e,
                            static_cast<hipStream_t>(stream_v));
}

int launch_cache_attn_update(const void* q_a, const void* k_a, const void* v_a, void* k_cache,
                             void* v_cache, const int32_t* cached_idx, int ldc,
                             const int32_t* active_idx, int ld_act, int32_t* err_count, void* out,
                             float* lse, int B, int H, int N, int A, int Nc, float scale,
                             int dtype, void* stream_v) {
    if (dtype == MAR_BF16 && A >= 16 && N <= kMaxMfmaTokens) {
        if (cached_idx == nullptr) ldc = 0;
        return dispatch_mfma<true>(
            static_cast<const uint16_t*>(q_a), static_cast<const uint16_t*>(k_a),
            static_cast<const uint16_t*>(v_a), static_cast<const uint16_t*>(k_cache),
            static_cast<const uint16_t*>(v_cache), cached_idx, ldc, static_cast<uint16_t*>(out),
            lse, B, H, N, A, Nc, scale * kLog2e, active_idx, ld_act, err_count, nullptr, nullptr,
            static_cast<hipStream_t>(stream_v));
    }
    // Row-wise path: the attention, then the row scatter on the same stream
    // (the two touch disjoint cache rows, so the order does not matter).
    const int st = launch_cache_attn(q_a, k_a, v_a, k_cache, v_cache, cached_idx, ldc, out, lse,
                                     B, H, N, A, Nc, scale, dtype, stream_v);
    if (st != MAR_OK) return st;
    const int row_bytes = kD * (dtype == MAR_BF16 ? 2 : 4);
    return launch_kv_scatter(k_cache, v_cache, k_a, v_a, active_idx, ld_act, err_count, B, H, N,
                             A, row_bytes, stream_v);
}

int launch_cache_attn_ragged_update(const void* q_a, const void* k_a, const void* v_a,
                                    void* k_cache, void* v_cache, const int32_t* cached_idx,
                                    int ldc, const int32_t* active_idx, int ld_act,
                                    const int32_t* a_len, const int32_t* c_len,
                                    int32_t* err_count, void* out, float* lse, int B, int H,
                                    int N, int A, int Nc, float scale, void* stream_v) {
    // bf16, A >= 16, N <= kMaxMfmaTokens (checked by the caller): the MFMA
    // kernels, whose per-sequence instantiations write rows [0, An) only.
    return dispatch_mfma<true>(
        static_cast<const uint16_t*>(q_a), static_cast<const uint16_t*>(k_a),
        static_cast<const uint16_t*>(v_a), static_cast<const uint16_t*>(k_cache),
        static_cast<const uint16_t*>(v_cache), cached_idx, ldc, static_cast<uint16_t*>(out), lse,
        B, H, N, A, Nc, scale * kLog2e, active_idx, ld_act, err_count, a_len, c_len,
        static_cast<hipStream_t>(stream_v));
}

}  // namespace marca
