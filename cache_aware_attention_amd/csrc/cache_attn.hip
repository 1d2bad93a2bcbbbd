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
// Two code paths:
//  * attn_mfma_kernel (bf16, A >= 16): one wave per (sequence, head) unit and
//    query group of up to 64 queries.  S^T = K Q^T and O^T = V^T P^T run on
//    v_mfma_f32_16x16x32_bf16; K goes straight from HBM into MFMA operand
//    registers (each lane loads 16-byte pieces of one 128-byte key row), V is
//    staged through LDS (padded rows) so each lane can read the 8 key rows of
//    one d column it needs for the PV operand.  The next chunk's loads are
//    issued before the current chunk is computed.  The unit's cached index
//    list is staged in LDS once.
//  * attn_rowwise_kernel (fp32 any A, bf16 A < 16): one wave per query, one
//    lane per head-dim element; plain FMA.  Exact-precision path for fp32.
//
// Head dim is fixed at 64 (MAR-B/L/H all use 64).  The cached index list is
// sanitised: an entry outside [0, N) is skipped, never dereferenced.
#include "device_util.h"
#include "launch.h"

namespace marca {
namespace {

constexpr int kD = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Row-wise path
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const float* p, int c, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[2 * c];
    const float4 b = reinterpret_cast<const float4*>(p)[2 * c + 1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, int c, float (&x)[8]) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[c];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}
__device__ __forceinline__ float load1(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load1(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store1(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store1(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

template <typename T>
__global__ __launch_bounds__(256) void attn_rowwise_kernel(
    const T* __restrict__ q_a, const T* __restrict__ k_a, const T* __restrict__ v_a,
    const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ cached_idx, int ldc, T* __restrict__ out,
    float* __restrict__ lse, int H, int N, int A, int Nc, float scale_log2) {
    __shared__ float q_s[4][kD];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int u = blockIdx.x;  // (b, h) unit
    const int b = u / H;
    const int i = blockIdx.y * 4 + wid;  // query of this wave
    const bool has_query = i < A;
    q_s[wid][lane] = has_query ? load1(q_a, ((size_t)u * A + i) * kD + lane) * scale_log2
                               : 0.f;
    __syncthreads();
    if (!has_query) return;  // no block-wide barrier after this point

    const int n_rows = A + Nc;
    const int32_t* cidx = cached_idx + (size_t)b * ldc;
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int r0 = 0; r0 < n_rows; r0 += kWave) {
        const int r = r0 + lane;
        long long off_k = -1, off_v = -1;
        if (r < A) {
            off_k = ((long long)u * A + r) * kD;
            off_v = off_k;
        } else if (r < n_rows) {
            const int n = cidx[r - A];
            if (n >= 0 && n < N) {
                off_k = ((long long)u * N + n) * kD + (1ll << 62);  // tag: cache source
                off_v = off_k;
            }
        }
        const bool valid = off_k >= 0;
        float s = -INFINITY;
        if (valid) {
            const bool from_cache = off_k >= (1ll << 62);
            const T* krow = from_cache ? k_cache + (off_k - (1ll << 62)) : k_a + off_k;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < kD / 8; ++c) {
                float x[8];
                load8(krow, c, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(q_s[wid][8 * c + e], x[e], acc);
            }
            s = acc;
        }
        const float mc = wave_max(s);
        const float mn = fmaxf(m, mc);
        if (mn == -INFINITY) continue;  // wave-uniform: nothing valid yet
        const float alpha = exp2f(m - mn);
        const float p = valid ? exp2f(s - mn) : 0.f;
        l = l * alpha + wave_sum(p);
        o *= alpha;
        const int cnt = min(kWave, n_rows - r0);
        for (int j = 0; j < cnt; ++j) {
            const float pj = __shfl(p, j, kWave);
            const long long ov = __shfl(off_v, j, kWave);
            if (pj != 0.f) {
                const bool from_cache = ov >= (1ll << 62);
                const T* vrow = from_cache ? v_cache + (ov - (1ll << 62)) : v_a + ov;
                o = fmaf(pj, load1(vrow, lane), o);
            }
        }
        m = mn;
    }
    const size_t orow = ((size_t)u * A + i) * kD;
    store1(out, orow + lane, l > 0.f ? o / l : 0.f);
    if (lse != nullptr && lane == 0) lse[(size_t)u * A + i] = (l > 0.f) ? (m + log2f(l)) * kLn2
                                                                        : -INFINITY;
}

// ---------------------------------------------------------------------------
// MFMA path (bf16, A >= 16)
// ---------------------------------------------------------------------------
constexpr int kChunk = 32;         // key rows per iteration (two 16-row MFMA tiles)
constexpr int kVStride = 80;       // LDS row stride of staged V, in bf16 (160 bytes)
constexpr int kQueriesPerGroup = 64;
constexpr int kMaxMfmaTokens = 8192;

union U4 {
    uint4 u;
    bf16x8_t v;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) {
    U4 t;
    t.u = x;
    return t.v;
}

// Element offset of key/value row r of the virtual sequence [active ; cached]
// from the unit's active base (r < A) or cache base (otherwise), with a flag
// for "row exists".  Branch-free: invalid rows point at active row 0, which
// always exists (A >= 1), and are zeroed / masked by the caller.
struct RowRef {
    const uint16_t* p;
    bool ok;
};
__device__ __forceinline__ RowRef row_ref(int r, int A, int Nc, const int32_t* cidx_s,
                                          const uint16_t* base_a, const uint16_t* base_c) {
    const int c = r - A;
    const bool in_c = (c >= 0) && (c < Nc);
    const int n = cidx_s[in_c ? c : 0];  // cidx_s has at least one entry
    const bool is_a = r < A;
    const bool ok = is_a || (in_c && n >= 0);
    const uint16_t* pa = base_a + (size_t)(is_a ? r : 0) * kD;
    const uint16_t* pc = base_c + (size_t)(n >= 0 ? n : 0) * kD;
    RowRef ref;
    ref.p = (!is_a && ok) ? pc : pa;
    ref.ok = ok;
    return ref;
}

__device__ __forceinline__ uint4 zero_unless(bool ok, uint4 x) {
    return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
}

template <int NQT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void attn_mfma_kernel(const uint16_t* __restrict__ q_a, const uint16_t* __restrict__ k_a,
                      const uint16_t* __restrict__ v_a, const uint16_t* __restrict__ k_cache,
                      const uint16_t* __restrict__ v_cache,
                      const int32_t* __restrict__ cached_idx, int ldc,
                      uint16_t* __restrict__ out, float* __restrict__ lse, int units, int H,
                      int N, int A, int Nc, int n_groups, float scale_log2) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* Vs = reinterpret_cast<uint16_t*>(smem);                         // [32][80]
    int32_t* cidx_s = reinterpret_cast<int32_t*>(smem + kChunk * kVStride * 2); // [Nc]

    const int lane = threadIdx.x;
    const int g = lane >> 4;    // lane group: k-slot group of MFMA operands
    const int m16 = lane & 15;  // row/column within a 16x16 tile

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
        if (u >= units) return;  // before any barrier: the whole workgroup exits
    }
    const int b = u / H;

    // Stage the sequence's cached list (sanitised) in LDS.
    const int32_t* cidx_g = cached_idx + (size_t)b * ldc;
    for (int c = lane; c < Nc; c += kWave) {
        const int n = cidx_g[c];
        cidx_s[c] = (n >= 0 && n < N) ? n : -1;
    }

    // Q tile as the B operand of S^T = K Q^T: lane holds query m16 of tile qt,
    // head-dim elements [8g, 8g+8) (k-step 0) and [32+8g, 32+8g+8) (k-step 1).
    const int q0 = qg * kQueriesPerGroup;
    bf16x8_t qf[NQT][2];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int qi = q0 + qt * 16 + m16;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        if (qi < A) {
            const uint4* p = reinterpret_cast<const uint4*>(q_a + ((size_t)u * A + qi) * kD);
            lo = p[g];
            hi = p[4 + g];
        }
        qf[qt][0] = as_bf16x8(lo);
        qf[qt][1] = as_bf16x8(hi);
    }

    const uint16_t* ka_u = k_a + (size_t)u * A * kD;
    const uint16_t* va_u = v_a + (size_t)u * A * kD;
    const uint16_t* kc_u = k_cache + (size_t)u * N * kD;
    const uint16_t* vc_u = v_cache + (size_t)u * N * kD;
    const int T = A + Nc;
    const int nchunks = (T + kChunk - 1) / kChunk;

    __syncthreads();  // cidx_s visible

    // Loader roles.  K: lane loads row (16t + m16) of the chunk, pieces g and
    // 4+g (16 bytes each).  V: lane loads row (lane & 31), pieces 4*(lane>>5)+k.
    const int vrow_l = lane & 31;
    const int vpiece0 = (lane >> 5) * 4;

    uint4 kA[2][2], kB[2][2], vA[4], vB[4];
    uint32_t mA[2], mB[2];
    bool okA, okB;

    // Loads are unconditional: a missing row (past the end, or an invalid
    // cached index) reads active row 0 instead.  Its scores are masked to
    // -inf through `mk`, and its V row is replaced by zeros when staged, so
    // it contributes nothing.
    auto load_chunk = [&](int c, uint4 (&kr)[2][2], uint4 (&vr)[4], uint32_t (&mk)[2],
                          bool& vok) {
        const int base = c * kChunk;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const RowRef rk = row_ref(base + 16 * t + m16, A, Nc, cidx_s, ka_u, kc_u);
            const uint4* p = reinterpret_cast<const uint4*>(rk.p);
            kr[t][0] = p[g];
            kr[t][1] = p[4 + g];
            mk[t] = static_cast<uint32_t>(__ballot(rk.ok) & 0xffffull);
        }
        const RowRef rv = row_ref(base + vrow_l, A, Nc, cidx_s, va_u, vc_u);
        const uint4* pv = reinterpret_cast<const uint4*>(rv.p);
#pragma unroll
        for (int k = 0; k < 4; ++k) vr[k] = pv[vpiece0 + k];
        vok = rv.ok;
    };

    float mrow[NQT], lrow[NQT];
    f32x4_t oacc[NQT][4];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        mrow[qt] = -INFINITY;
        lrow[qt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // One chunk: stage its V rows in LDS, start loading chunk c+1 into the
    // other buffer set (its latency overlaps this chunk's math), then fold the
    // chunk into the running softmax state.
    auto step = [&](int c, const uint4 (&kc)[2][2], const uint4 (&vc)[4], const uint32_t (&mk)[2],
                    bool vok, uint4 (&kn)[2][2], uint4 (&vn)[4], uint32_t (&mn_)[2], bool& vokn) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<uint4*>(Vs + vrow_l * kVStride + (vpiece0 + k) * 8) =
                zero_unless(vok, vc[k]);
        if (c + 1 < nchunks) load_chunk(c + 1, kn, vn, mn_, vokn);
        __syncthreads();

        // V^T operands: row m16 <-> head dims 4*m16 + dt (dt = output tile),
        // k-slot j <-> key row 16*(j>>2) + 4g + (j&3) of the chunk; one 8-byte
        // LDS read per slot serves all four tiles.
        bf16x8_t va[4];
        {
            uint2 w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kr = 16 * (j >> 2) + 4 * g + (j & 3);
                w[j] = *reinterpret_cast<const uint2*>(Vs + kr * kVStride + 4 * m16);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                uint32_t e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t word = (dt < 2) ? w[j].x : w[j].y;
                    e[j] = (dt & 1) ? (word >> 16) : (word & 0xffffu);
                }
                U4 t;
                t.u = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                 e[6] | (e[7] << 16));
                va[dt] = t.v;
            }
        }

#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            // S^T tiles: lane holds S^T[key 16t + 4g + i][query m16] in s[t][i].
            f32x4_t s[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[t][0]), qf[qt][0],
                                                              acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[t][1]), qf[qt][1],
                                                              acc, 0, 0, 0);
                s[t] = acc;
            }
            // Online softmax for query m16; P^T packed as the B operand of
            // O^T = V^T P^T with the same k-slot <-> key row map as va.
            float v[8];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = (mk[t] >> (4 * g + i)) & 1u;
                    v[4 * t + i] = ok ? s[t][i] * scale_log2 : -INFINITY;
                }
            float mx = v[0];
#pragma unroll
            for (int k = 1; k < 8; ++k) mx = fmaxf(mx, v[k]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const float mnew = fmaxf(mrow[qt], mx);
            const float mref = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrow[qt] - mref);
            float p[8], ps = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                p[k] = __builtin_amdgcn_exp2f(v[k] - mref);
                ps += p[k];
            }
            lrow[qt] = lrow[qt] * alpha + ps;
            mrow[qt] = mnew;
            U4 pk;
            pk.u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                              pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                oacc[qt][dt] *= alpha;
                oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pk.v, oacc[qt][dt],
                                                                       0, 0, 0);
            }
        }
        __syncthreads();  // all V reads done before the next chunk overwrites Vs
    };

    load_chunk(0, kA, vA, mA, okA);
    for (int c = 0; c < nchunks; c += 2) {
        step(c, kA, vA, mA, okA, kB, vB, mB, okB);
        if (c + 1 < nchunks) step(c + 1, kB, vB, mB, okB, kA, vA, mA, okA);
    }

    // Finalise: lane holds O[query m16][16g + 4i + dt] = oacc[qt][dt][i].
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        float l = lrow[qt];
        l += __shfl_xor(l, 16, kWave);
        l += __shfl_xor(l, 32, kWave);
        const int qi = q0 + qt * 16 + m16;
        if (qi < A) {
            const float inv = 1.f / l;
            uint32_t wv[8];
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float lo = oacc[qt][e & 3][e >> 2] * inv;
                const float hi = oacc[qt][(e + 1) & 3][(e + 1) >> 2] * inv;
                wv[e / 2] = pack_bf16x2(lo, hi);
            }
            uint4* dst = reinterpret_cast<uint4*>(out + ((size_t)u * A + qi) * kD + 16 * g);
            dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
            if (lse != nullptr && g == 0) lse[(size_t)u * A + qi] = (mrow[qt] + log2f(l)) * kLn2;
        }
    }
}

template <int NQT>
int launch_mfma(const uint16_t* q_a, const uint16_t* k_a, const uint16_t* v_a,
                const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* cached_idx,
                int ldc, uint16_t* out, float* lse, int B, int H, int N, int A, int Nc,
                int n_groups, float scale_log2, hipStream_t stream) {
    const int units = B * H;
    const int grid = (n_groups == 1) ? units : ((units + 7) / 8) * 8 * n_groups;
    const size_t lds = (size_t)kChunk * kVStride * 2 + (size_t)(Nc > 0 ? Nc : 1) * 4;
    hipLaunchKernelGGL(attn_mfma_kernel<NQT>, dim3(grid), dim3(64), lds, stream, q_a, k_a, v_a,
                       k_cache, v_cache, cached_idx, ldc, out, lse, units, H, N, A, Nc, n_groups,
                       scale_log2);
    return status_from_launch();
}

}  // namespace

int launch_cache_attn(const void* q_a, const void* k_a, const void* v_a, const void* k_cache,
                      const void* v_cache, const int32_t* cached_idx, int ldc, void* out,
                      float* lse, int B, int H, int N, int A, int Nc, float scale, int dtype,
                      void* stream_v) {
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
        const int n_groups = (A + kQueriesPerGroup - 1) / kQueriesPerGroup;
        const int nqt = (n_groups > 1) ? 4 : (A + 15) / 16;
        switch (nqt) {
            case 1: return launch_mfma<1>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H, N, A, Nc, n_groups, scale_log2, stream);
            case 2: return launch_mfma<2>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H, N, A, Nc, n_groups, scale_log2, stream);
            case 3: return launch_mfma<3>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H, N, A, Nc, n_groups, scale_log2, stream);
            default: return launch_mfma<4>(q, ka, va, kc, vc, cached_idx, ldc, o, lse, B, H, N, A, Nc, n_groups, scale_log2, stream);
        }
    }
    const dim3 grid(B * H, (A + 3) / 4);
    if (dtype == MAR_BF16) {
        hipLaunchKernelGGL(attn_rowwise_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(q_a), static_cast<const uint16_t*>(k_a),
                           static_cast<const uint16_t*>(v_a), static_cast<const uint16_t*>(k_cache),
                           static_cast<const uint16_t*>(v_cache), cached_idx, ldc,
                           static_cast<uint16_t*>(out), lse, H, N, A, Nc, scale_log2);
    } else {
        hipLaunchKernelGGL(attn_rowwise_kernel<float>, grid, dim3(256), 0, stream,
                           static_cast<const float*>(q_a), static_cast<const float*>(k_a),
                           static_cast<const float*>(v_a), static_cast<const float*>(k_cache),
                           static_cast<const float*>(v_cache), cached_idx, ldc,
                           static_cast<float*>(out), lse, H, N, A, Nc, scale_log2);
    }
    return status_from_launch();
}

}  // namespace marca
