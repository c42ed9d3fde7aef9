/*
 * Seeded synthetic inputs for look-ahead token scoring.
 *
 * This file draws random numbers and lays them out; it holds none of the
 * scoring or selection arithmetic. Both the CPU oracle's tests and the GPU
 * path's tests/benchmarks read the arrays it fills.
 *
 * Every element is a pure function of (seed, tag, coordinates): a
 * counter-based generator (SplitMix64's finaliser applied to a Weyl sequence
 * keyed per stream), so any slice of any tensor can be generated on its own,
 * in parallel, in any order, with identical results.
 *
 * Distribution (the "planted direction" workload of the scoring method's
 * synthetic benchmark):
 *   noise ~ N(0,1) (tabulated inverse CDF, one normal per 64-bit draw)
 *   u[r][l][g] = z / |z|, z ~ N(0, I_d)               (one unit direction per
 *                                                      request, layer, kv-head)
 *   K[r][l][g][i][t] = noise + (planted[i] ? 2*u[t] : 0)
 *   Q[r][l][h][j][t] = noise + 2*u[r][l][h / (H/Hkv)][t]
 * Values are formed in double, rounded to float32 (round-to-nearest-even) and,
 * for bf16 storage, rounded again from float32 to bf16 (nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define TAG_K 0x4b4b4b4b01ULL
#define TAG_Q 0x5151515102ULL
#define TAG_U 0x5555555503ULL
#define TAG_P 0x5050505004ULL
#define TAG_S 0x5353535305ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Key of one stream: seed, a tag naming the tensor, and up to three
 * coordinates, each folded in through the finaliser. */
static inline uint64_t stream_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b,
                                  uint64_t c) {
    uint64_t k = mix64(seed + 0x9e3779b97f4a7c15ULL);
    k = mix64(k ^ tag);
    k = mix64(k + 0x632be59bd9b4e019ULL * (a + 1));
    k = mix64(k + 0x8cb92ba72f3d8dd7ULL * (b + 1));
    k = mix64(k + 0xd6e8feb86659fd93ULL * (c + 1));
    return k;
}

static inline uint64_t draw(uint64_t key, uint64_t idx) {
    return mix64(key + (idx + 1) * 0x9e3779b97f4a7c15ULL);
}

/*
 * Standard normals by inverse transform: z = Phi^-1(q) with Phi^-1 tabulated at
 * the 65537 nodes q_k = (k + 0.5) / 65537 and interpolated linearly. The high
 * 32 bits of a draw pick the segment (16 bits) and the position inside it
 * (16 bits). Range is +-4.33; mean 0, variance 1 - 3e-4. The table is built once
 * per process from erfc by Newton's method, to full double precision.
 */
#define NT 65536
static double g_icdf[NT + 1];

static double phi_cdf(double z) { return 0.5 * erfc(-z * 0.70710678118654752440); }

static double inv_phi(double q) {
    /* bracket by bisection (Phi is monotone), then polish with Newton steps */
    double lo = -9.0, hi = 9.0;
    for (int it = 0; it < 40; ++it) {
        double mid = 0.5 * (lo + hi);
        if (phi_cdf(mid) < q) lo = mid; else hi = mid;
    }
    double z = 0.5 * (lo + hi);
    for (int it = 0; it < 3; ++it) {
        double pdf = 0.39894228040143267794 * exp(-0.5 * z * z);
        z -= (phi_cdf(z) - q) / pdf;
    }
    return z;
}

__attribute__((constructor)) static void build_icdf(void) {
    for (int k = 0; k <= NT; ++k) g_icdf[k] = inv_phi(((double)k + 0.5) / (double)(NT + 1));
}

static inline double normal_of(uint64_t h) {
    uint32_t top = (uint32_t)(h >> 32);
    uint32_t k = top >> 16;
    double f = (double)(top & 0xffffu) * (1.0 / 65536.0);
    return g_icdf[k] + f * (g_icdf[k + 1] - g_icdf[k]);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7fffu + lsb;
    return (uint16_t)(b >> 16);
}

/* unit direction u[0..d) for (seed, r, l, g) */
void synth_direction(uint64_t seed, int64_t r, int64_t l, int64_t g, int32_t d, double* u) {
    uint64_t key = stream_key(seed, TAG_U, (uint64_t)r, (uint64_t)l, (uint64_t)g);
    double n2 = 0.0;
    for (int32_t t = 0; t < d; ++t) {
        u[t] = normal_of(draw(key, (uint64_t)t));
        n2 += u[t] * u[t];
    }
    double inv = 1.0 / sqrt(n2);
    for (int32_t t = 0; t < d; ++t) u[t] *= inv;
}

static inline void store(void* out, int32_t dtype, int64_t idx, double v) {
    float f = (float)v;
    if (dtype == 0)
        ((float*)out)[idx] = f;
    else
        ((uint16_t*)out)[idx] = f32_to_bf16_rne(f);
}

/*
 * Q of request r, layout [L][H][N][d] starting at `out` (dtype 0 = f32,
 * 1 = bf16 bit patterns). plant_scale multiplies u (2.0 in the workloads).
 */
void synth_fill_q(uint64_t seed, int64_t r, int32_t L, int32_t H, int32_t Hkv, int32_t N,
                  int32_t d, int32_t dtype, double plant_scale, void* out) {
    const int32_t G = H / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t l = 0; l < L; ++l)
        for (int32_t h = 0; h < H; ++h) {
            double u[1024];
            synth_direction(seed, r, l, h / G, d, u);
            uint64_t key = stream_key(seed, TAG_Q, (uint64_t)r, (uint64_t)l, (uint64_t)h);
            for (int32_t j = 0; j < N; ++j)
                for (int32_t t = 0; t < d; ++t) {
                    int64_t e = (int64_t)j * d + t;
                    double v = normal_of(draw(key, (uint64_t)e)) + plant_scale * u[t];
                    store(out, dtype, (((int64_t)l * H + h) * N + j) * d + t, v);
                }
        }
}

/*
 * K of request r: n_keys = M + N rows per (l, g). Element (l, g, i, t) goes to
 * out[(l*Hkv + g) * plane_stride + (key_offset + i) * d + t]; so a contiguous
 * [L][Hkv][M+N][d] tensor uses plane_stride = (M+N)*d, key_offset = 0, and a
 * packed ragged tensor [L][Hkv][T][d] uses plane_stride = T*d and the request's
 * first key row as key_offset. planted[i] != 0 adds plant_scale*u to row i.
 */
void synth_fill_k(uint64_t seed, int64_t r, int32_t L, int32_t Hkv, int64_t n_keys, int32_t d,
                  int32_t dtype, double plant_scale, const uint8_t* planted, void* out,
                  int64_t plane_stride, int64_t key_offset) {
    const int64_t BLK = 1024;
    const int64_t nblk = (n_keys + BLK - 1) / BLK;
#pragma omp parallel for collapse(3) schedule(static)
    for (int32_t l = 0; l < L; ++l)
        for (int32_t g = 0; g < Hkv; ++g)
            for (int64_t b = 0; b < nblk; ++b) {
                double u[1024];
                synth_direction(seed, r, l, g, d, u);
                uint64_t key = stream_key(seed, TAG_K, (uint64_t)r, (uint64_t)l, (uint64_t)g);
                int64_t i0 = b * BLK, i1 = i0 + BLK < n_keys ? i0 + BLK : n_keys;
                int64_t base = ((int64_t)l * Hkv + g) * plane_stride;
                for (int64_t i = i0; i < i1; ++i) {
                    double add = planted[i] ? plant_scale : 0.0;
                    for (int32_t t = 0; t < d; ++t) {
                        int64_t e = i * d + t;
                        double v = normal_of(draw(key, (uint64_t)e)) + add * u[t];
                        store(out, dtype, base + (key_offset + i) * d + t, v);
                    }
                }
            }
}

/* n uniform 64-bit draws of stream (seed, tag=S, r, which) */
void synth_uniform_u64(uint64_t seed, int64_t r, int64_t which, int64_t n, uint64_t* out) {
    uint64_t key = stream_key(seed, TAG_S, (uint64_t)r, (uint64_t)which, 0);
    for (int64_t i = 0; i < n; ++i) out[i] = draw(key, (uint64_t)i);
}

/*
 * Choose k distinct chunk indices out of nc (partial Fisher-Yates driven by the
 * stream (seed, P, r)); result in chosen[0..k), in draw order.
 */
void synth_choose(uint64_t seed, int64_t r, int64_t nc, int64_t k, int64_t* perm_scratch,
                  int64_t* chosen) {
    uint64_t key = stream_key(seed, TAG_P, (uint64_t)r, 0, 0);
    for (int64_t i = 0; i < nc; ++i) perm_scratch[i] = i;
    for (int64_t i = 0; i < k; ++i) {
        uint64_t h = draw(key, (uint64_t)i);
        int64_t span = nc - i;
        int64_t jdx = i + (int64_t)(h % (uint64_t)span);
        int64_t tmp = perm_scratch[i];
        perm_scratch[i] = perm_scratch[jdx];
        perm_scratch[jdx] = tmp;
        chosen[i] = perm_scratch[i];
    }
}
