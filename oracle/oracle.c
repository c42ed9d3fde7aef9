/*
 * CPU oracle for SpecPrefill's token-importance estimator and chunk selection.
 *
 * TEST INFRASTRUCTURE ONLY. It exists to check the GPU library: only the test
 * suite, the package's smoke check and the benchmark's CPU-baseline leg may
 * load or call it. It shares no code with the GPU path.
 *
 * Plain, slow and direct: every quantity is computed from its definition, in
 * double precision for the scoring, and in the pinned fp32 / integer / double
 * steps stated below for the selection (so that a GPU fed the same float32
 * importance array can reproduce the kept set bit for bit).
 *
 * Sources (web pages; cited by title and section):
 *  [SP-R]  "Speculative Prefill: Turbocharging TTFT with Lightweight and
 *          Training-Free Token Importance Estimation" (paper review page):
 *          section "Core algorithm" (attention-score speculation, look-ahead,
 *          max-mean aggregation, chunk selection and pooling, position-ID
 *          recovery) and section "Core formulas" (attention score, token
 *          importance aggregation, chunk score, top-K).
 *  [SP-G]  "SpecPrefill - Implementation Guide": "How It Works" (core
 *          algorithm, token importance, chunk selection), "v3 Improvements"
 *          (cumulative attention mass selection, structural token boosting),
 *          "v3.1 Optimizations" (score normalisation to [0,1]) and
 *          "Configuration Reference" (defaults of the SP_* variables).
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes of the repository):
 *  - query rows are the N look-ahead rows at positions M..M+N-1; row j's
 *    softmax runs over the M+j+1 keys it can see (causal), and importance is
 *    reported for the M prompt keys only;
 *  - logits are scaled by 1/sqrt(d) unless a scale is given;
 *  - query head h reads kv-head floor(h / (H/Hkv));
 *  - importance_i = (1/N) sum_j max_{l,h} a_{l,h,j,i} (the review's formula
 *    sums over the look-ahead index, written with a mismatched letter);
 *  - robust normalisation (percentile clip, clipped z-score): see normalise;
 *  - selection: min-max normalise (all 1 when max == min), boost first then
 *    last, fixed point 2^32, chunk sums, average pool over chunks with the
 *    window clipped at the edges (mean over the tokens actually in the
 *    window), rank by (pooled key desc, chunk index asc); top-K keeps
 *    max(1, ceil(rate * nc)) chunks, mass mode walks the ranking adding each
 *    chunk's own mass until it reaches mass * total; kept tokens ascend, with
 *    position id = pos_base + i;
 *  - threshold selection (oracle_select_threshold) follows the steps of the
 *    Implementation Guide's own program on the raw scores; the cap keeps
 *    every (n / max_keep)-th kept token and ends with the last kept one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_TOPK = 0, ORC_MASS = 1 };

static double elem(const void* base, int dtype, size_t idx) {
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16; /* bf16 -> f32 exactly */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int check_dims(int dtype, int L, int H, int Hkv, int d, int N, int M) {
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    if (L < 1 || H < 1 || Hkv < 1 || d < 1 || N < 1 || M < 1) return -1;
    if (H % Hkv != 0) return -1;
    return 0;
}

/*
 * One row of look-ahead attention: for layer l, query head h, look-ahead step
 * j, the softmax of the scaled logits of query position M+j over the M+j+1
 * keys it can see ([SP-R] Core formulas: a_ij = Softmax(Q_{M+j} K^T)_i).
 *   Q: [L][H][N][d], K: [L][Hkv][M+N][d] (f32, or bf16 bit patterns)
 *   p: out, M+j+1 doubles (probabilities of keys 0..M+j)
 */
int oracle_softmax_row(const void* Q, const void* K, int dtype, int L, int H, int Hkv, int d,
                       int N, int M, double scale, int l, int h, int j, double* p) {
    if (check_dims(dtype, L, H, Hkv, d, N, M)) return -1;
    if (l < 0 || l >= L || h < 0 || h >= H || j < 0 || j >= N) return -1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    const int G = H / Hkv;
    const int g = h / G;
    const long nk = (long)M + j + 1;
    const size_t qoff = (((size_t)l * H + h) * N + j) * (size_t)d;
    const size_t kbase = ((size_t)l * Hkv + g) * (size_t)(M + N) * (size_t)d;

    double* q = (double*)malloc(sizeof(double) * (size_t)d);
    if (!q) return -2;
    for (int t = 0; t < d; ++t) q[t] = elem(Q, dtype, qoff + t);

    double m = -INFINITY;
    for (long i = 0; i < nk; ++i) {
        double s = 0.0;
        const size_t koff = kbase + (size_t)i * d;
        for (int t = 0; t < d; ++t) s += q[t] * elem(K, dtype, koff + t);
        p[i] = scale * s;
        if (p[i] > m) m = p[i];
    }
    double Z = 0.0;
    for (long i = 0; i < nk; ++i) {
        p[i] = exp(p[i] - m);
        Z += p[i];
    }
    for (long i = 0; i < nk; ++i) p[i] /= Z;
    free(q);
    return 0;
}

/*
 * Token importance ([SP-R] Core formulas, token importance aggregation;
 * [SP-G] How It Works, token importance): max over query heads, max over
 * layers, mean over the N look-ahead steps.
 *   importance: out, M doubles.
 * Rows (l, h, j) are independent and run in parallel over nthreads threads
 * (<= 0: the OpenMP default); each thread keeps its own running max.
 */
int oracle_score(const void* Q, const void* K, int dtype, int L, int H, int Hkv, int d, int N,
                 int M, double scale, int nthreads, double* importance) {
    if (check_dims(dtype, L, H, Hkv, d, N, M)) return -1;
    const size_t SM = (size_t)N * (size_t)M;
    double* S = (double*)calloc(SM, sizeof(double)); /* S[j][i] = max_{l,h} a */
    if (!S) return -2;
    const long nrows = (long)L * H * N;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* Sp = (double*)calloc(SM, sizeof(double));
        double* p = (double*)malloc(sizeof(double) * (size_t)(M + N));
        if (!Sp || !p) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            fail = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long r = 0; r < nrows; ++r) {
            if (!Sp || !p) continue;
            const int l = (int)(r / ((long)H * N));
            const int h = (int)((r / N) % H);
            const int j = (int)(r % N);
            oracle_softmax_row(Q, K, dtype, L, H, Hkv, d, N, M, scale, l, h, j, p);
            double* Sj = Sp + (size_t)j * M;
            for (int i = 0; i < M; ++i)
                if (p[i] > Sj[i]) Sj[i] = p[i];
        }
#ifdef _OPENMP
#pragma omp critical
#endif
        {
            if (Sp)
                for (size_t k = 0; k < SM; ++k)
                    if (Sp[k] > S[k]) S[k] = Sp[k];
        }
        free(Sp);
        free(p);
    }
    if (!fail) {
        for (int i = 0; i < M; ++i) {
            double acc = 0.0;
            for (int j = 0; j < N; ++j) acc += S[(size_t)j * M + i];
            importance[i] = acc / (double)N;
        }
    }
    free(S);
    return fail ? -2 : 0;
}

/*
 * Importance with the query row of the last prompt token as one more step
 * ([SP-G] How It Works, Attention Capture (cb_eval): the attention row of
 * the last query position is captured during the prefill, like each
 * look-ahead step's, and the importance averages over all captured steps).
 * That row, at position M-1, sees the M prompt keys 0..M-1:
 *   importance_i = (sum_{j<N} S_j[i] + X[i]) / (N + 1),
 *   S_j[i] = max_{l,h} a_{l,h,j,i} (as in oracle_score),
 *   X[i]   = max_{l,h} softmax_{i'<M}(scale <Q_last[l][h], K[l][h/G][i']>)_i.
 *   Q_last: [L][H][d]; importance: out, M doubles.
 */
int oracle_score_lastrow(const void* Q, const void* Q_last, const void* K, int dtype, int L,
                         int H, int Hkv, int d, int N, int M, double scale, int nthreads,
                         double* importance) {
    if (check_dims(dtype, L, H, Hkv, d, N, M)) return -1;
    int rc = oracle_score(Q, K, dtype, L, H, Hkv, d, N, M, scale, nthreads, importance);
    if (rc) return rc;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    const int G = H / Hkv;
    double* X = (double*)calloc((size_t)M, sizeof(double));
    if (!X) return -2;
    int fail = 0;
    /* rows (l, h) in parallel, each thread with its own running max */
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* Xp = (double*)calloc((size_t)M, sizeof(double));
        double* p = (double*)malloc(sizeof(double) * (size_t)M);
        if (!Xp || !p) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            fail = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long r = 0; r < (long)L * H; ++r) {
            if (!Xp || !p) continue;
            const int l = (int)(r / H), h = (int)(r % H);
            const size_t qoff = ((size_t)l * H + h) * (size_t)d;
            const size_t kbase = ((size_t)l * Hkv + h / G) * (size_t)(M + N) * (size_t)d;
            double m = -INFINITY;
            for (int i = 0; i < M; ++i) {
                double s = 0.0;
                for (int t = 0; t < d; ++t)
                    s += elem(Q_last, dtype, qoff + t) * elem(K, dtype, kbase + (size_t)i * d + t);
                p[i] = scale * s;
                if (p[i] > m) m = p[i];
            }
            double Z = 0.0;
            for (int i = 0; i < M; ++i) {
                p[i] = exp(p[i] - m);
                Z += p[i];
            }
            for (int i = 0; i < M; ++i)
                if (p[i] / Z > Xp[i]) Xp[i] = p[i] / Z;
        }
#ifdef _OPENMP
#pragma omp critical
#endif
        {
            if (Xp)
                for (int i = 0; i < M; ++i)
                    if (Xp[i] > X[i]) X[i] = Xp[i];
        }
        free(Xp);
        free(p);
    }
    /* importance currently holds (1/N) sum_j S_j */
    if (!fail)
        for (int i = 0; i < M; ++i) importance[i] = (importance[i] * N + X[i]) / (N + 1);
    free(X);
    return fail ? -2 : 0;
}

/* ------------------------------------------------------------------------------------- */
/* selection                                                                              */
/* ------------------------------------------------------------------------------------- */

enum { ORC_NORM_MINMAX = 0, ORC_NORM_PERCENTILE = 1, ORC_NORM_ZSCORE = 2 };

static int cmp_f32_asc(const void* a, const void* b) {
    const float x = *(const float*)a, y = *(const float*)b;
    return (x < y) ? -1 : (x > y);
}

/* v = (x - lo) / (hi - lo) in fp32 (a subtraction and one IEEE division), or
 * 1 everywhere when hi == lo; with clamp, values outside [0, 1] are clamped
 * and a degenerate range gives 1 for x >= hi and 0 below. */
static void scale_to_unit(const float* x, int M, float lo, float hi, int clamp, float* v) {
    const float range = hi - lo;
    for (int i = 0; i < M; ++i) {
        if (range > 0.0f) {
            float num = x[i] - lo;
            v[i] = num / range;
            if (clamp) {
                if (v[i] < 0.0f) v[i] = 0.0f;
                if (v[i] > 1.0f) v[i] = 1.0f;
            }
        } else {
            v[i] = (clamp && x[i] < hi) ? 0.0f : 1.0f;
        }
    }
}

/*
 * Normalisation of the scores to [0, 1] before boosting.
 *  - min-max ([SP-G] v3.1 item 5): v = (x - min) / (max - min), all 1 when
 *    max == min.
 *  - percentile clip ([SP-G] Limitations item 5 names percentile-based
 *    normalisation as the remedy for outliers; the reading: clip to two order
 *    statistics, then min-max between them): with s the scores sorted
 *    ascending, lo = s[floor(p_lo (M-1))], hi = s[ceil(p_hi (M-1))] (indices
 *    evaluated in double from the float parameters, 0 <= p_lo < p_hi <= 1);
 *    v = clamp((x - lo) / (hi - lo), 0, 1), or (x >= hi ? 1 : 0) when hi == lo.
 *    p_lo = 0, p_hi = 1 is min-max exactly.
 *  - clipped z-score (same passage names z-score normalisation; the reading:
 *    standardise, clip at +-c standard deviations, map [-c, c] onto [0, 1]).
 *    Statistics are taken exactly on a 16-bit grid of the min-max values u
 *    (a z-score is unchanged by the positive affine map to u):
 *    y = rint(u * 2^16) (integers in [0, 65536]), S1 = sum y, S2 = sum y^2,
 *    D = M S2 - S1^2 (exact; M^2 times the variance of y). D == 0: v = 1
 *    everywhere. Otherwise z = (double)(M y - S1) / sqrt((double) D) (the
 *    integer M y - S1 is exact in double; (double) D rounds once), clipped to
 *    [-c, c], and v = (float)((z + c) / (2 c)), every step one IEEE double
 *    operation. c = p_hi > 0; p_lo must be 0.
 * Returns 0, or -1 on invalid parameters.
 */
static int normalise(const float* x, int M, int norm, float p_lo, float p_hi, float* v) {
    float mn = x[0], mx = x[0];
    for (int i = 1; i < M; ++i) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    if (norm == ORC_NORM_MINMAX) {
        scale_to_unit(x, M, mn, mx, 0, v);
        return 0;
    }
    if (norm == ORC_NORM_PERCENTILE) {
        if (!(p_lo >= 0.0f && p_lo < p_hi && p_hi <= 1.0f)) return -1;
        float* s = (float*)malloc(sizeof(float) * (size_t)M);
        if (!s) return -2;
        memcpy(s, x, sizeof(float) * (size_t)M);
        qsort(s, (size_t)M, sizeof(float), cmp_f32_asc);
        const long i_lo = (long)floor((double)p_lo * (double)(M - 1));
        const long i_hi = (long)ceil((double)p_hi * (double)(M - 1));
        const float lo = s[i_lo], hi = s[i_hi];
        free(s);
        scale_to_unit(x, M, lo, hi, 1, v);
        return 0;
    }
    if (norm == ORC_NORM_ZSCORE) {
        if (!(p_lo == 0.0f && p_hi > 0.0f) || !isfinite(p_hi)) return -1;
        scale_to_unit(x, M, mn, mx, 0, v); /* u: the min-max values */
        uint64_t S1 = 0, S2 = 0;
        int64_t* y = (int64_t*)malloc(sizeof(int64_t) * (size_t)M);
        if (!y) return -2;
        for (int i = 0; i < M; ++i) {
            y[i] = (int64_t)llrint((double)(v[i] * 65536.0f));
            S1 += (uint64_t)y[i];
            S2 += (uint64_t)(y[i] * y[i]);
        }
        const unsigned __int128 D =
            (unsigned __int128)M * S2 - (unsigned __int128)S1 * S1;
        if (D == 0) {
            for (int i = 0; i < M; ++i) v[i] = 1.0f;
        } else {
            const double sd = sqrt((double)D);
            const double c = (double)p_hi;
            for (int i = 0; i < M; ++i) {
                double z = (double)((int64_t)M * y[i] - (int64_t)S1) / sd;
                if (z < -c) z = -c;
                if (z > c) z = c;
                v[i] = (float)((z + c) / (2.0 * c));
            }
        }
        free(y);
        return 0;
    }
    return -1;
}

typedef struct {
    double key;
    long idx;
} ranked_t;

/* pooled key descending, then chunk index ascending */
static int rank_cmp(const void* a, const void* b) {
    const ranked_t* x = (const ranked_t*)a;
    const ranked_t* y = (const ranked_t*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

/*
 * Chunk selection and compaction for one prompt of M tokens.
 *   importance : M float32 scores
 *   mode       : 0 = top-K keep rate ([SP-R] Core formulas, chunk score and
 *                top-K; [SP-G] Chunk Selection), 1 = cumulative mass
 *                ([SP-G] v3 Improvements 1)
 *   boosts     : [SP-G] v3 Improvements 2; normalisation: [SP-G] v3.1 item 5
 *                (min-max) or [SP-G] Limitations item 5 (percentile clip,
 *                clipped z-score; see normalise)
 *   pooling    : [SP-R] Core algorithm, chunk selection and pooling
 *   outputs    : kept_idx[n] = base_index + i, pos_ids[n] = pos_base + i for
 *                every token i of every kept chunk, ascending ([SP-R] Core
 *                algorithm, position-ID recovery); *n_kept.
 *   debug outputs (each may be NULL): v[M] normalised+boosted values,
 *   q[M] fixed-point values, C[nc] chunk masses, key[nc] pooled keys,
 *   kept_chunk[nc] 0/1.
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_select(const float* importance, int M, int chunk, int pool_k, int mode,
                  float keep_rate, float mass, int first_n, float first_mult, int last_n,
                  float last_mult, int norm, float norm_lo, float norm_hi, long pos_base,
                  long base_index, int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept,
                  float* v_out, uint64_t* q_out, uint64_t* C_out, double* key_out,
                  uint8_t* kept_chunk_out) {
    if (M < 1 || chunk < 1 || pool_k < 1 || (pool_k % 2) == 0) return -1;
    if (mode == ORC_TOPK && !(keep_rate > 0.0f && keep_rate <= 1.0f)) return -1;
    if (mode == ORC_MASS && !(mass > 0.0f && mass <= 1.0f)) return -1;
    if (mode != ORC_TOPK && mode != ORC_MASS) return -1;
    if (first_n < 0 || last_n < 0 || !(first_mult >= 0.0f) || !(last_mult >= 0.0f)) return -1;

    const long nc = (M + chunk - 1) / chunk;
    float* v = (float*)malloc(sizeof(float) * (size_t)M);
    uint64_t* C = (uint64_t*)calloc((size_t)nc, sizeof(uint64_t));
    uint64_t* len = (uint64_t*)calloc((size_t)nc, sizeof(uint64_t));
    double* key = (double*)malloc(sizeof(double) * (size_t)nc);
    ranked_t* rk = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)nc);
    uint8_t* keep = (uint8_t*)calloc((size_t)nc, 1);
    if (!v || !C || !len || !key || !rk || !keep) {
        free(v); free(C); free(len); free(key); free(rk); free(keep);
        return -2;
    }

    /* normalisation to [0, 1] (min-max, percentile clip or clipped z-score) */
    const int nrc = normalise(importance, M, norm, norm_lo, norm_hi, v);
    if (nrc) {
        free(v); free(C); free(len); free(key); free(rk); free(keep);
        return nrc;
    }
    for (int i = 0; i < M; ++i) {
        /* structural boosts: first, then last (both apply where they overlap) */
        if (i < first_n) v[i] = v[i] * first_mult;
        if (i >= M - last_n) v[i] = v[i] * last_mult;
    }

    /* fixed point (v * 2^32, round to nearest even), chunk sums */
    for (int i = 0; i < M; ++i) {
        float scaled = v[i] * 4294967296.0f;
        uint64_t qi = (uint64_t)llrint((double)scaled);
        if (q_out) q_out[i] = qi;
        C[i / chunk] += qi;
        len[i / chunk] += 1;
    }

    /* 1-D average pool over chunks, stride 1, window clipped at the edges */
    const long hw = (pool_k - 1) / 2;
    for (long c = 0; c < nc; ++c) {
        uint64_t P = 0, T = 0;
        for (long c2 = c - hw; c2 <= c + hw; ++c2) {
            if (c2 < 0 || c2 >= nc) continue;
            P += C[c2];
            T += len[c2];
        }
        key[c] = (double)P / (double)T;
        rk[c].key = key[c];
        rk[c].idx = c;
    }
    qsort(rk, (size_t)nc, sizeof(ranked_t), rank_cmp);

    if (mode == ORC_TOPK) {
        long K = (long)ceil((double)keep_rate * (double)nc);
        if (K < 1) K = 1;
        if (K > nc) K = nc;
        for (long r = 0; r < K; ++r) keep[rk[r].idx] = 1;
    } else {
        uint64_t total = 0;
        for (long c = 0; c < nc; ++c) total += C[c];
        const double thr = (double)mass * (double)total;
        uint64_t cum = 0;
        for (long r = 0; r < nc; ++r) {
            keep[rk[r].idx] = 1;
            cum += C[rk[r].idx];
            if ((double)cum >= thr) break;
        }
    }

    int32_t n = 0;
    for (long c = 0; c < nc; ++c) {
        if (!keep[c]) continue;
        long i1 = (c + 1) * chunk < M ? (c + 1) * chunk : M;
        for (long i = c * chunk; i < i1; ++i) {
            kept_idx[n] = (int32_t)(base_index + i);
            pos_ids[n] = (int32_t)(pos_base + i);
            ++n;
        }
    }
    *n_kept = n;

    if (v_out) memcpy(v_out, v, sizeof(float) * (size_t)M);
    if (C_out) memcpy(C_out, C, sizeof(uint64_t) * (size_t)nc);
    if (key_out) memcpy(key_out, key, sizeof(double) * (size_t)nc);
    if (kept_chunk_out) memcpy(kept_chunk_out, keep, (size_t)nc);
    free(v); free(C); free(len); free(key); free(rk); free(keep);
    return 0;
}

/* float comparison for qsort, descending */
static int desc_f32(const void* a, const void* b) {
    const float x = *(const float*)a, y = *(const float*)b;
    return (x > y) ? -1 : (x < y);
}

/*
 * Threshold chunk selection as the Implementation Guide's own program performs
 * it: [SP-G] "Full Source Code" (its chunk selection and the cap on sparse
 * tokens), "How It Works" / Chunk Selection (the first 4 and last 2 tokens are
 * always kept) and "Configuration Reference" (SP_MAX_KEEP). On the raw float32
 * scores x[0..M):
 *  1. eff_min = min(min_tok, max(4, M / 10)); with keep_rate >= 1 or
 *     M <= eff_min every token is kept;
 *  2. chunk means a_c = (float)(s_c / n_c), s_c the double sum of the chunk's
 *     scores in index order, n_c its token count;
 *  3. K = max(1, ceil(nc * keep_rate)) with the product in single precision;
 *     t = the K-th largest a_c; every chunk with a_c >= t is kept (equal
 *     means may keep more than K chunks);
 *  4. tokens 0..3 and, when M > 4, M-2 and M-1 are kept;
 *  5. while fewer than eff_min tokens are kept, tokens of the chunks with
 *     a_c < t are added in index order;
 *  6. the kept tokens ascend; if max_keep > 0 and more than max_keep are kept,
 *     only every (n / max_keep)-th of them is kept, at most max_keep, the last
 *     of which is replaced by the last kept token.
 * Outputs as for oracle_select. Returns 0, or -1 on invalid arguments.
 */
int oracle_select_threshold(const float* x, int M, int chunk, float keep_rate, int min_tok,
                            int max_keep, long pos_base, long base_index, int32_t* kept_idx,
                            int32_t* pos_ids, int32_t* n_kept) {
    if (M < 1 || chunk < 1 || !(keep_rate > 0.0f) || min_tok < 0 || max_keep < 0) return -1;
    const int four = 4, tenth = M / 10;
    const int floor_min = tenth > four ? tenth : four;
    const int eff_min = min_tok < floor_min ? min_tok : floor_min;
    uint8_t* keep = (uint8_t*)calloc((size_t)M, 1);
    if (!keep) return -2;
    int all = keep_rate >= 1.0f || M <= eff_min;
    if (all) {
        memset(keep, 1, (size_t)M);
    } else {
        const long nc = (M + chunk - 1) / chunk;
        float* a = (float*)malloc(sizeof(float) * (size_t)nc);
        float* sorted = (float*)malloc(sizeof(float) * (size_t)nc);
        if (!a || !sorted) {
            free(a); free(sorted); free(keep);
            return -2;
        }
        for (long c = 0; c < nc; ++c) {
            const long i0 = c * chunk, i1 = (c + 1) * chunk < M ? (c + 1) * chunk : M;
            double s = 0.0;
            for (long i = i0; i < i1; ++i) s += (double)x[i];
            a[c] = (float)(s / (double)(i1 - i0));
            sorted[c] = a[c];
        }
        const float prod = (float)nc * keep_rate;
        long K = (long)ceilf(prod);
        if (K < 1) K = 1;
        qsort(sorted, (size_t)nc, sizeof(float), desc_f32);
        const float t = sorted[K - 1];
        long n = 0;
        for (long c = 0; c < nc; ++c) {
            if (!(a[c] >= t)) continue;
            const long i1 = (c + 1) * chunk < M ? (c + 1) * chunk : M;
            for (long i = c * chunk; i < i1; ++i) keep[i] = 1, ++n;
        }
        const int always[6] = {0, 1, 2, 3, M - 2, M - 1};
        const int n_always = M > 4 ? 6 : 4;
        for (int k = 0; k < n_always; ++k)
            if (always[k] < M && !keep[always[k]]) keep[always[k]] = 1, ++n;
        for (long c = 0; c < nc && n < eff_min; ++c) {
            if (a[c] >= t) continue;
            const long i1 = (c + 1) * chunk < M ? (c + 1) * chunk : M;
            for (long i = c * chunk; i < i1 && n < eff_min; ++i)
                if (!keep[i]) keep[i] = 1, ++n;
        }
        free(a);
        free(sorted);
    }
    int32_t n = 0;
    for (long i = 0; i < M; ++i)
        if (keep[i]) kept_idx[n++] = (int32_t)i;
    free(keep);
    if (max_keep > 0 && n > max_keep) {
        const int32_t step = n / max_keep, last = kept_idx[n - 1];
        int32_t m = 0;
        for (int32_t i = 0; i < n && m < max_keep; i += step) kept_idx[m++] = kept_idx[i];
        kept_idx[m - 1] = last;
        n = m;
    }
    for (int32_t k = 0; k < n; ++k) {
        pos_ids[k] = (int32_t)(pos_base + kept_idx[k]);
        kept_idx[k] = (int32_t)(base_index + kept_idx[k]);
    }
    *n_kept = n;
    return 0;
}
