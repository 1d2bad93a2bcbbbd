/*
 * oracle.c -- plain CPU reference for the KV-cached MAR decoding hot path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Scalar double-precision loops,
 * written from the definitions the method pages state; no blocking, fusion or
 * reordering beyond what those definitions say.  OpenMP parallelises only
 * across independent (sequence, head) or sequence units.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double dot(const double* a, const double* b, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* ------------------------------------------------------------------------ */
/* Cache-aware attention as softmax attention over the union of both paths.  */
/* ------------------------------------------------------------------------ */
int oracle_cache_attention(const double* q_a, const double* k_a, const double* v_a,
                           const double* k_cache, const double* v_cache,
                           const int32_t* cached_idx, int64_t ldc,
                           int64_t B, int64_t H, int64_t N, int64_t A, int64_t Nc,
                           int64_t D, double scale, double* out, double* lse) {
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < Nc; ++c) {
            int32_t j = cached_idx[b * ldc + c];
            if (j < 0 || j >= N) return -1;
        }
    const int64_t T = A + Nc; /* size of the union of the two key/value sets */
    int64_t units = B * H;
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < units; ++u) {
        int64_t b = u / H;
        /* Row pointers of the union: active rows first, then cached rows. */
        const double** krow = (const double**)malloc((size_t)(T > 0 ? T : 1) * sizeof(double*));
        const double** vrow = (const double**)malloc((size_t)(T > 0 ? T : 1) * sizeof(double*));
        double* s = (double*)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
        for (int64_t j = 0; j < A; ++j) {
            krow[j] = k_a + (u * A + j) * D;
            vrow[j] = v_a + (u * A + j) * D;
        }
        for (int64_t c = 0; c < Nc; ++c) {
            int64_t n = cached_idx[b * ldc + c];
            krow[A + c] = k_cache + (u * N + n) * D;
            vrow[A + c] = v_cache + (u * N + n) * D;
        }
        for (int64_t i = 0; i < A; ++i) {
            const double* q = q_a + (u * A + i) * D;
            double mx = -INFINITY;
            for (int64_t j = 0; j < T; ++j) {
                s[j] = scale * dot(q, krow[j], D);
                if (s[j] > mx) mx = s[j];
            }
            double denom = 0.0;
            for (int64_t j = 0; j < T; ++j) denom += exp(s[j] - mx);
            double* o = out + (u * A + i) * D;
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < T; ++j) acc += exp(s[j] - mx) * vrow[j][d];
                o[d] = acc / denom;
            }
            if (lse) lse[u * A + i] = mx + log(denom);
        }
        free(krow);
        free(vrow);
        free(s);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Layer-2 head- and query-averaged attention probabilities.                */
/* ------------------------------------------------------------------------ */
void oracle_refresh_scores(const double* q_gen, const double* k_full,
                           int64_t B, int64_t H, int64_t G, int64_t N, int64_t D,
                           double scale, double* scores) {
#pragma omp parallel for schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        double* acc = scores + b * N;
        double* s = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            const double* K = k_full + (b * H + h) * N * D;
            for (int64_t g = 0; g < G; ++g) {
                const double* q = q_gen + ((b * H + h) * G + g) * D;
                double mx = -INFINITY;
                for (int64_t j = 0; j < N; ++j) {
                    s[j] = scale * dot(q, K + j * D, D);
                    if (s[j] > mx) mx = s[j];
                }
                double denom = 0.0;
                for (int64_t j = 0; j < N; ++j) denom += exp(s[j] - mx);
                for (int64_t j = 0; j < N; ++j) acc[j] += exp(s[j] - mx) / denom;
            }
        }
        double inv = (H * G > 0) ? 1.0 / (double)(H * G) : 0.0;
        for (int64_t j = 0; j < N; ++j) acc[j] *= inv;
        free(s);
    }
}

/* ------------------------------------------------------------------------ */
/* Sort-based top-K with lowest-index tie-break, and the cached complement. */
/* ------------------------------------------------------------------------ */
typedef struct {
    double score;
    int32_t idx;
} cand_t;

static int cand_cmp(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->score > b->score) return -1; /* larger score first */
    if (a->score < b->score) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx); /* then lower index */
}

void oracle_refresh_select(const double* scores, const int32_t* gp_idx, int64_t ld_gp,
                           int64_t n_gp, int64_t K, int64_t B, int64_t N,
                           int32_t* active_idx, int64_t ld_act,
                           int32_t* cached_idx, int64_t ld_cached, int32_t* cached_len) {
#pragma omp parallel for schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        /* state: 0 = eligible candidate, 1 = generating/caching, 2 = refreshing */
        unsigned char* state = (unsigned char*)calloc((size_t)(N > 0 ? N : 1), 1);
        cand_t* cand = (cand_t*)malloc((size_t)(N > 0 ? N : 1) * sizeof(cand_t));
        for (int64_t m = 0; m < n_gp; ++m) {
            int32_t j = gp_idx[b * ld_gp + m];
            active_idx[b * ld_act + m] = j;
            if (j >= 0 && j < N) state[j] = 1;
        }
        int64_t n_cand = 0;
        for (int64_t j = 0; j < N; ++j)
            if (state[j] == 0) {
                cand[n_cand].score = scores[b * N + j];
                cand[n_cand].idx = (int32_t)j;
                ++n_cand;
            }
        qsort(cand, (size_t)n_cand, sizeof(cand_t), cand_cmp);
        for (int64_t r = 0; r < K; ++r) {
            if (r < n_cand) {
                active_idx[b * ld_act + n_gp + r] = cand[r].idx;
                state[cand[r].idx] = 2;
            } else {
                active_idx[b * ld_act + n_gp + r] = -1;
            }
        }
        int64_t c = 0;
        for (int64_t j = 0; j < N; ++j)
            if (state[j] == 0) {
                if (c < ld_cached) cached_idx[b * ld_cached + c] = (int32_t)j;
                ++c;
            }
        for (int64_t t = c; t < ld_cached; ++t) cached_idx[b * ld_cached + t] = -1;
        cached_len[b] = (int32_t)c;
        free(state);
        free(cand);
    }
}

/* ------------------------------------------------------------------------ */
/* KV cache row update (partial) or full rewrite.                           */
/* ------------------------------------------------------------------------ */
int64_t oracle_kv_scatter(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          const int32_t* idx, int64_t B, int64_t H, int64_t N, int64_t M,
                          int64_t D, int64_t elem_bytes) {
    const int64_t row = D * elem_bytes;
    unsigned char* kc = (unsigned char*)k_cache;
    unsigned char* vc = (unsigned char*)v_cache;
    const unsigned char* kn = (const unsigned char*)k_new;
    const unsigned char* vn = (const unsigned char*)v_new;
    if (idx == NULL) {
        memcpy(kc, kn, (size_t)(B * H * N * row));
        memcpy(vc, vn, (size_t)(B * H * N * row));
        return 0;
    }
    int64_t skipped = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m) {
            int32_t j = idx[b * M + m];
            if (j < 0 || j >= N) {
                ++skipped;
                continue;
            }
            for (int64_t h = 0; h < H; ++h) {
                memcpy(kc + ((b * H + h) * N + j) * row, kn + ((b * H + h) * M + m) * row, (size_t)row);
                memcpy(vc + ((b * H + h) * N + j) * row, vn + ((b * H + h) * M + m) * row, (size_t)row);
            }
        }
    return skipped;
}

/* ------------------------------------------------------------------------ */
/* Cosine gate.                                                             */
/* ------------------------------------------------------------------------ */
void oracle_gate_from_cos(const double* cos_in, int64_t B, int64_t N, double tau,
                          uint8_t* reuse, int32_t* compute_idx, int32_t* compute_len) {
    for (int64_t b = 0; b < B; ++b) {
        int64_t c = 0;
        for (int64_t j = 0; j < N; ++j) {
            int r = cos_in[b * N + j] >= tau;
            reuse[b * N + j] = (uint8_t)r;
            if (!r) compute_idx[b * N + c++] = (int32_t)j;
        }
        for (int64_t t = c; t < N; ++t) compute_idx[b * N + t] = -1;
        compute_len[b] = (int32_t)c;
    }
}

void oracle_cos_gate(const double* x, const double* y, int64_t B, int64_t N, int64_t W,
                     double tau, double eps, double* cos_out, uint8_t* reuse,
                     int32_t* compute_idx, int32_t* compute_len) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < B * N; ++t) {
        const double* xt = x + t * W;
        const double* yt = y + t * W;
        double xy = dot(xt, yt, W);
        double nx = sqrt(dot(xt, xt, W));
        double ny = sqrt(dot(yt, yt, W));
        double den = nx * ny;
        if (den < eps) den = eps;
        cos_out[t] = xy / den;
    }
    oracle_gate_from_cos(cos_out, B, N, tau, reuse, compute_idx, compute_len);
}

/* ------------------------------------------------------------------------ */
/* CFG residual store / reuse.                                              */
/* ------------------------------------------------------------------------ */
void oracle_cfg_residual(const float* cond, const float* uncond, float* residual,
                         float* uncond_out, float* guided, double w, int mode, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        double c = (double)cond[i];
        double u;
        if (mode == 0) {
            u = (double)uncond[i];
            residual[i] = (float)(c - u);
        } else {
            u = (double)(float)(c - (double)residual[i]);
            uncond_out[i] = (float)u;
        }
        if (guided) guided[i] = (float)(u + w * (c - u));
    }
}
