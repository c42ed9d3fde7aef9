// Chunk selection of one prompt: the steps, shared by the selection kernel
// (one workgroup of 1024 threads per request, or a grid of them for one long
// prompt) and the fused scoring launch (one workgroup of 512 threads after
// the scores, on chunk masses the streaming workgroups summed for long
// prompts).
//
// Steps ("SpecPrefill - Implementation Guide": v3.1 item 5 min-max
// normalisation, v3 item 2 structural boosts, v3 item 1 cumulative attention
// mass, How It Works chunk selection; "Speculative Prefill" review page, Core
// algorithm: chunk means, 1-D average pooling across chunks, top-K chunks,
// position-ID recovery):
//   v_i = (x_i - min) / (max - min) (1 when max == min), boosts (first, then
//   last), q_i = rint(v_i * 2^32) as uint64, chunk sums C_c, pooled keys
//   key_c = sum C / sum len over the clipped window, rank (key desc, index asc),
//   keep K chunks (top-K) or the shortest ranked prefix reaching mass * total
//   (mass), emit kept tokens ascending with their position ids. The ranking
//   is never materialised: a radix select over the keys' bits finds the key
//   of the last kept rank, and ties on it are settled by index.
// Every step is exact or a single IEEE-rounded operation (fp32 sub/div/mul,
// u64 -> f64 conversion, f64 div and mul), and sums are integer, so the
// result is the same however the work is split across threads or
// workgroups: a CPU doing the same steps in any order reproduces it bit for
// bit. Compiled with -ffp-contract=off.
#pragma once

#include <math.h>

#include "sp_internal.h"
#include "sp_slots.h"

namespace sp {

constexpr int kLd = 16;         // importance loads in flight per thread
constexpr int kSeg = 16;        // contiguous elements a thread quantises per tile
constexpr int kDigit = 11;      // radix select: key bits per round
constexpr int kBins = 1 << kDigit;
constexpr int kFinal = 64;      // candidates ranked exactly, one per thread
constexpr int kRankBatch = 8;   // candidates read at a time while ranking

// Workgroup shape of the selection: NT threads (1024 for the selection
// kernel, 512 inside the fused scoring launch).
template <int NT>
struct SelCfg {
    static constexpr int kThreads = NT;
    static constexpr int kWaves = NT / 64;
    static constexpr int kScanPer = kSelMaxChunks / NT;  // chunks per thread
    static constexpr int kTile = NT * kSeg;              // elements per staged tile
    static_assert(kScanPer * NT == kSelMaxChunks, "chunks split evenly over threads");
};

template <int NT>
struct SelectShared {
    using C_ = SelCfg<NT>;
    unsigned long long C[kSelMaxChunks];     // chunk masses
    // staged importance tile (one pad word after every kSeg, so that a thread's
    // contiguous segment reads are bank-conflict free) while chunk masses are
    // accumulated; afterwards the arrays of the selection
    union {
        float stage[C_::kTile + C_::kTile / kSeg];
        struct {
            unsigned long long S[kSelMaxChunks + 1]; // prefix sums, then the ties' exclusive cumulatives
            int off[kSelMaxChunks];                  // kept flags, then their exclusive scan
            int klist[kSelMaxChunks];                // kept chunks in index order
        };
        struct {                                  // radix select rounds
            unsigned long long hmass[2][kBins];   // mass of each digit's candidates
            unsigned int hcount[2][kBins];        //   and their count (two sets, alternating rounds)
        };
    };
    unsigned long long ck[kFinal], cmass[kFinal];  // the last candidates: key, mass,
    unsigned int ci[kFinal];                        //   chunk index,
    int ckeep[kFinal];                              //   kept or not
    int ncand;
    unsigned long long wtmp[C_::kWaves];
    unsigned long long bc_prefix, bc_mass; // broadcast of a round's result
    unsigned int bc_count, bc_ties;
    float fmin[C_::kWaves], fmax[C_::kWaves];
    unsigned long long zs[2];             // (z-score) sums of y and y^2
    float pct[2];                         // (percentile) the two order statistics
    unsigned long long rand_[C_::kWaves], ror_[C_::kWaves];  // AND / OR of the keys per wave
    int kc;                               // number of kept chunks
};

// Inclusive scan across a wave with lane moves: shifts within rows of 16,
// then row 0's total into row 1 (and row 2's into row 3), then rows 0-1's
// total into rows 2-3 (rows not selected keep the 0 they are given).
__device__ __forceinline__ unsigned wave_scan_u32(unsigned v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return (unsigned)x;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)v, CTRL, ROWS, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(v >> 32), CTRL, ROWS, 0xf, false);
    return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}

// The same scan for 64-bit values (each half moved, then a 64-bit add).
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long v) {
    v += dpp_u64<0x111, 0xf>(v);
    v += dpp_u64<0x112, 0xf>(v);
    v += dpp_u64<0x114, 0xf>(v);
    v += dpp_u64<0x118, 0xf>(v);
    v += dpp_u64<0x142, 0xa>(v);
    v += dpp_u64<0x143, 0xc>(v);
    return v;
}

// Bitwise AND and OR across a wave (butterflies: quad swaps, half-row and
// row mirrors, then the row and half-wave swaps).
template <bool AND>
__device__ __forceinline__ unsigned wave_bitwise(unsigned v) {
    auto op = [](unsigned a, unsigned b) { return AND ? (a & b) : (a | b); };
    v = op(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, true));
    v = op(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, true));
    v = op(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, true));
    v = op(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, true));
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(r16[0], r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(r32[0], r32[1]);
}
template <bool AND>
__device__ __forceinline__ unsigned long long wave_bitwise64(unsigned long long v) {
    return ((unsigned long long)wave_bitwise<AND>((unsigned)(v >> 32)) << 32) |
           wave_bitwise<AND>((unsigned)v);
}

__device__ __forceinline__ bool ranks_before(unsigned long long ka, unsigned int ia,
                                             unsigned long long kb, unsigned int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// In-place exclusive scan of data[0..n) (n <= kSelMaxChunks) by NT threads;
// returns the total.
template <typename T, int NT>
__device__ T block_excl_scan(T* data, int n, unsigned long long* wtmp) {
    constexpr int kScanPer = SelCfg<NT>::kScanPer;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int i0 = tid * kScanPer;
    T loc[kScanPer];
    T run = 0;
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
        loc[e] = (i0 + e < n) ? data[i0 + e] : (T)0;
        run += loc[e];
    }
    T incl;
    if constexpr (sizeof(T) == 8) incl = (T)wave_scan_u64((unsigned long long)run);
    else incl = (T)wave_scan_u32((unsigned)run);
    if (lane == 63) wtmp[w] = (unsigned long long)incl;
    __syncthreads();
    T wbase = 0, total = 0;
    for (int x = 0; x < SelCfg<NT>::kWaves; ++x) {
        const T t = (T)wtmp[x];
        if (x < w) wbase += t;
        total += t;
    }
    T ex = wbase + incl - run;
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
        if (i0 + e < n) data[i0 + e] = ex;
        ex += loc[e];
    }
    __syncthreads();
    return total;
}

// Order-preserving map of float bits to unsigned keys (and back): negative
// values have all bits flipped, others only the sign bit.
__device__ __forceinline__ unsigned f32_key(float f) {
    const unsigned b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_f32(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The k-th smallest (0-based) of x[0..M): a radix select over the keys'
// bits (digits of 11, 11 and 10 bits from the top; a histogram of the
// candidates' digit in LDS, one pad word per 32 bins so that wave 0's lanes
// read their 32-bin groups without bank conflicts). hist holds 2112 words.
template <int NT>
__device__ float order_stat(const float* __restrict__ x, int M, int k, unsigned* hist,
                            unsigned long long* bc_prefix, unsigned* bc_count) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    unsigned prefix = 0u, pmask = 0u;
    const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
    for (int rnd = 0; rnd < 3; ++rnd) {
        const int sh = shifts[rnd];
        const unsigned dmask = (1u << widths[rnd]) - 1u;
        for (int d = tid; d < 2048 + 64; d += NT) hist[d] = 0u;
        __syncthreads();
        for (int i = tid; i < M; i += NT) {
            const unsigned key = f32_key(x[i]);
            if ((key & pmask) == prefix) {
                const unsigned d = (key >> sh) & dmask;
                atomicAdd(&hist[d + (d >> 5)], 1u);
            }
        }
        __syncthreads();
        if (w == 0) {
            // lane L sums bins 32 L .. 32 L + 31; the first lane whose
            // inclusive count exceeds k holds the digit, then one lane per bin
            unsigned c = 0u;
            for (int j = 0; j < 32; ++j) c += hist[lane * 33 + j];
            const unsigned incl = wave_scan_u32(c);
            const unsigned long long bal = __ballot(incl > (unsigned)k);
            const int F = bal ? __builtin_ctzll(bal) : 63;
            const unsigned before = __shfl(incl - c, F);
            const unsigned cb = lane < 32 ? hist[F * 33 + lane] : 0u;
            const unsigned incl2 = wave_scan_u32(cb);
            const unsigned long long bal2 = __ballot(lane < 32 && before + incl2 > (unsigned)k);
            const int J = bal2 ? __builtin_ctzll(bal2) : 0;
            if (lane == J) {
                *bc_prefix = (unsigned long long)(F * 32 + J);
                *bc_count = before + incl2 - cb;
            }
        }
        __syncthreads();
        prefix |= (unsigned)*bc_prefix << sh;
        pmask |= dmask << sh;
        k -= (int)*bc_count;
        __syncthreads();
    }
    return key_f32(prefix);
}

// A non-negative 128-bit integer rounded to the nearest double (ties to even):
// the top 64 bits with the rest folded into a sticky bit, converted, scaled.
__device__ __forceinline__ double u128_to_f64(unsigned __int128 v) {
    const unsigned long long hi = (unsigned long long)(v >> 64);
    if (hi == 0ull) return (double)(unsigned long long)v;
    const int sh = 64 - __builtin_clzll(hi);
    unsigned long long m = (unsigned long long)(v >> sh);
    if ((unsigned long long)v & ((1ull << sh) - 1ull)) m |= 1ull;
    return ldexp((double)m, sh);
}

// The min-max value u of one score: the correctly rounded quotient
// (x - mn) / range by a reciprocal and one correction (Markstein): with
// both operands scaled by a power of two taking range into [1, 2)
// (a2 = (x - mn) * scale in one rounding), y = 1/range rounded,
// q0 = a2 * y and the exact residual a2 - q0 * range, q0 + residual * y
// rounds to the IEEE quotient (a quotient too small for that is too
// small to survive the fixed point); a plain division when the range is
// subnormal or near the top of the range; 1 when max == min.
struct MinMaxNorm {
    float mn, range, dscale, drange, dnms, drcp;
    bool dfast;
    __device__ __forceinline__ void init(float mn_, float mx_) {
        mn = mn_;
        range = mx_ - mn_;
        const int rexp = (int)((__float_as_uint(range) >> 23) & 255);  // range's exponent field
        dfast = range > 0.f && rexp >= 1 && rexp <= 253;                // normal, scale representable
        dscale = dfast ? __uint_as_float((unsigned)(254 - rexp) << 23) : 1.f;
        drange = range * dscale;
        dnms = -mn * dscale;
        drcp = __fdiv_rn(1.0f, drange);
    }
    __device__ __forceinline__ float value(float xv) const {
        if (dfast) {
            const float a2 = fmaf(xv, dscale, dnms);
            const float q0 = a2 * drcp;
            return fmaf(fmaf(-q0, drange, a2), drcp, q0);
        }
        return range > 0.f ? __fdiv_rn(xv - mn, range) : 1.0f;
    }
};

// The fixed-point mass of token i (of M) with normalised value v: the boosts
// (first, then last), then rint(v * 2^32) as uint64.
__device__ __forceinline__ unsigned long long token_mass(float v, int i, int M, const SelectParamsDev& p) {
    float q = v;
    if (i < p.first_n) q = q * p.first_mult;
    if (i >= M - p.last_n) q = q * p.last_mult;
    return (unsigned long long)rintf(q * 4294967296.0f);
}

template <int NT>
__device__ void select_ranked(SelectShared<NT>& sh, const SelectParamsDev& p, int M, int base, int pb,
                              int32_t* __restrict__ kept, int32_t* __restrict__ pos,
                              int32_t* __restrict__ nkept_out);

// The selection of one prompt x[0..M) by a workgroup of NT threads, in the
// steps above; sh is the workgroup's LDS. kept and pos receive the kept
// tokens (kept[n] = base + i, pos[n] = pb + i), *nkept_out their count, or -1
// when some score is not finite (then nothing else is written).
template <int NT>
__device__ void select_prompt(SelectShared<NT>& sh, const SelectParamsDev& p, const float* __restrict__ x,
                              int M, int base, int pb, int32_t* __restrict__ kept,
                              int32_t* __restrict__ pos, int32_t* __restrict__ nkept_out) {
    using C_ = SelCfg<NT>;
    constexpr int kSelThreads = NT, kSelWaves = C_::kWaves, kTile = C_::kTile;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int chunk = p.chunk;
    const int nc = (M + chunk - 1) / chunk;

    // 1. min and max (exact in any order); kLd loads in flight per thread,
    // indices past the end re-read the last element
    // (a NaN or infinite score, which a scoring call that timed out leaves,
    // makes the request's count -1 and leaves its outputs untouched)
    // (the first kLd loads are the first tile of step 2 in the same layout:
    // they stay in registers for it)
    static_assert(kSelThreads * kLd == kTile && kLd == kSeg, "step 1's first loads are step 2's first tile");
    float mn = INFINITY, mx = -INFINITY;
    int nonfinite = 0;
    float tile0[kLd];
#pragma unroll
    for (int k = 0; k < kLd; ++k) tile0[k] = x[min(k * kSelThreads + tid, M - 1)];
#pragma unroll
    for (int k = 0; k < kLd; ++k) {
        nonfinite |= (__float_as_uint(tile0[k]) & 0x7f800000u) == 0x7f800000u;
        mn = fminf(mn, tile0[k]);
        mx = fmaxf(mx, tile0[k]);
    }
    for (int t0 = kSelThreads * kLd; t0 < M; t0 += kSelThreads * kLd) {
        float v[kLd];
#pragma unroll
        for (int k = 0; k < kLd; ++k) v[k] = x[min(t0 + k * kSelThreads + tid, M - 1)];
#pragma unroll
        for (int k = 0; k < kLd; ++k) {
            nonfinite |= (__float_as_uint(v[k]) & 0x7f800000u) == 0x7f800000u;
            mn = fminf(mn, v[k]);
            mx = fmaxf(mx, v[k]);
        }
    }
    if (__syncthreads_or(nonfinite)) {
        if (tid == 0) *nkept_out = -1;
        return;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if (lane == 0) {
        sh.fmin[w] = mn;
        sh.fmax[w] = mx;
    }
    for (int c = tid; c < nc; c += kSelThreads) sh.C[c] = 0ull;
    __syncthreads();
    mn = sh.fmin[0];
    mx = sh.fmax[0];
    for (int x2 = 1; x2 < kSelWaves; ++x2) {
        mn = fminf(mn, sh.fmin[x2]);
        mx = fmaxf(mx, sh.fmax[x2]);
    }
    MinMaxNorm nm;
    nm.init(mn, mx);
    const float range = nm.range;
    const bool dfast = nm.dfast;
    const float dscale = nm.dscale, drange = nm.drange, dnms = nm.dnms, drcp = nm.drcp;
    auto minmax_value = [&](float xv) __attribute__((always_inline)) { return nm.value(xv); };

    // Robust normalisations ("SpecPrefill - Implementation Guide",
    // Limitations item 5). Percentile clip: v = clamp((x - lo) / (hi - lo), 0, 1)
    // between two order statistics of the scores (v = x >= hi ? 1 : 0 when
    // they are equal). Clipped z-score: from the exact integer sums of the
    // min-max values on a 2^-16 grid, y = rint(u 2^16), S1 = sum y,
    // S2 = sum y^2, D = M S2 - S1^2; z = (M y - S1) / sqrt(D) clipped to
    // [-c, c] and v = (z + c) / (2c) in double, then rounded to float (1
    // everywhere when D = 0). Every step is exact or one IEEE operation.
    float plo = 0.f, phi = 0.f;
    long long zS1 = 0;
    double zsd = 0.0, zc = 0.0;
    bool zflat = true;
    if (p.norm == SP_NORM_PERCENTILE) {
        const int i_lo = (int)floor((double)p.norm_lo * (double)(M - 1));
        const int i_hi = (int)ceil((double)p.norm_hi * (double)(M - 1));
        unsigned* hist = (unsigned*)sh.hcount[0];
        plo = order_stat<NT>(x, M, i_lo, hist, &sh.bc_prefix, &sh.bc_count);
        phi = order_stat<NT>(x, M, i_hi, hist, &sh.bc_prefix, &sh.bc_count);
    } else if (p.norm == SP_NORM_ZSCORE) {
        unsigned long long s1 = 0ull, s2 = 0ull;
        for (int i = tid; i < M; i += kSelThreads) {
            const unsigned long long y = (unsigned long long)rintf(minmax_value(x[i]) * 65536.0f);
            s1 += y;
            s2 += y * y;
        }
        if (tid < 2) sh.zs[tid] = 0ull;
        __syncthreads();
        atomicAdd(&sh.zs[0], s1);
        atomicAdd(&sh.zs[1], s2);
        __syncthreads();
        const unsigned long long S1 = sh.zs[0], S2 = sh.zs[1];
        const unsigned __int128 D = (unsigned __int128)(unsigned)M * S2 - (unsigned __int128)S1 * S1;
        zflat = D == 0;
        zsd = sqrt(u128_to_f64(D));
        zS1 = (long long)S1;
        zc = (double)p.norm_hi;
    }
    const float prange = phi - plo;
    auto robust_value = [&](float xv) __attribute__((always_inline)) {
        if (p.norm == SP_NORM_PERCENTILE) {
            if (!(prange > 0.f)) return xv < phi ? 0.0f : 1.0f;
            const float v = __fdiv_rn(xv - plo, prange);
            return v < 0.f ? 0.0f : (v > 1.f ? 1.0f : v);
        }
        if (zflat) return 1.0f;
        const long long y = (long long)rintf(minmax_value(xv) * 65536.0f);
        double z = (double)((long long)M * y - zS1) / zsd;
        z = z < -zc ? -zc : (z > zc ? zc : z);
        return (float)((z + zc) / (2.0 * zc));
    };

    // 2-3. normalise, boost, fixed point, chunk sums. Tiles of kTile elements
    // are staged in LDS with coalesced loads; each thread then takes kSeg
    // contiguous elements and adds each run of one chunk to that chunk's mass.
    // (the next tile's loads are issued before this tile is processed)
    float v[kSeg];
#pragma unroll
    for (int k = 0; k < kSeg; ++k) v[k] = tile0[k];
    for (int t0 = 0; t0 < M; t0 += kTile) {
#pragma unroll
        for (int k = 0; k < kSeg; ++k) {
            const int l = k * kSelThreads + tid;
            sh.stage[l + l / kSeg] = v[k];
        }
        __syncthreads();
        if (t0 + kTile < M) {
#pragma unroll
            for (int k = 0; k < kSeg; ++k) v[k] = x[min(t0 + kTile + k * kSelThreads + tid, M - 1)];
        }
        const int g0 = t0 + tid * kSeg;  // first element of this thread's segment
        if (g0 < M) {
            float xv[kSeg];
#pragma unroll
            for (int e = 0; e < kSeg; ++e) xv[e] = sh.stage[tid * (kSeg + 1) + e];
            float vq[kSeg];
            if (p.norm != SP_NORM_MINMAX) {
                for (int e = 0; e < kSeg; ++e) vq[e] = robust_value(xv[e]);
            } else if (dfast) {
#pragma unroll
                for (int e = 0; e < kSeg; ++e) {
                    const float a2 = fmaf(xv[e], dscale, dnms);
                    const float q0 = a2 * drcp;
                    vq[e] = fmaf(fmaf(-q0, drange, a2), drcp, q0);
                }
            } else if (range > 0.f) {
#pragma unroll
                for (int e = 0; e < kSeg; ++e) vq[e] = __fdiv_rn(xv[e] - mn, range);
            } else {
#pragma unroll
                for (int e = 0; e < kSeg; ++e) vq[e] = 1.0f;
            }
            const bool boosted = g0 < p.first_n || g0 + kSeg > M - p.last_n;
            if (!boosted && g0 + kSeg <= M && chunk % kSeg == 0) {
                // the whole segment lies in one chunk, inside the prompt, unboosted
                unsigned long long run = 0ull;
#pragma unroll
                for (int e = 0; e < kSeg; ++e) run += (unsigned long long)rintf(vq[e] * 4294967296.0f);
                atomicAdd(&sh.C[g0 / chunk], run);
            } else {
                asm volatile("");  // (keep this path a branch)
                unsigned long long qv[kSeg];
#pragma unroll
                for (int e = 0; e < kSeg; ++e) {
                    const int i = g0 + e;
                    qv[e] = i < M ? token_mass(vq[e], i, M, p) : 0ull;
                }
                int c = g0 / chunk;
                int next = (c + 1) * chunk;  // first element of the next chunk
                unsigned long long run = 0ull;
#pragma unroll
                for (int e = 0; e < kSeg; ++e) {
                    if (g0 + e == next && next < M) {  // (past the prompt's end only zeros follow)
                        atomicAdd(&sh.C[c], run);
                        run = 0ull;
                        ++c;
                        next += chunk;
                    }
                    run += qv[e];
                }
                atomicAdd(&sh.C[c], run);
            }
        }
        __syncthreads();
    }

    select_ranked<NT>(sh, p, M, base, pb, kept, pos, nkept_out);
}

// Steps 4-7 from the chunk masses in sh.C[0..nc) (nc = ceil(M / chunk)): the
// pooled keys, the ranking, the kept chunks and the kept tokens.
template <int NT>
__device__ void select_ranked(SelectShared<NT>& sh, const SelectParamsDev& p, int M, int base, int pb,
                              int32_t* __restrict__ kept, int32_t* __restrict__ pos,
                              int32_t* __restrict__ nkept_out) {
    using C_ = SelCfg<NT>;
    constexpr int kSelThreads = NT, kSelWaves = C_::kWaves;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int chunk = p.chunk;
    const int nc = (M + chunk - 1) / chunk;

    // 4. pooled keys from prefix sums: key_c = (S[hi+1] - S[lo]) / tokens in
    // window, held as the bits of the (non-negative) double, which order like
    // the values; thread tid holds chunks e * kSelThreads + tid
    for (int c = tid; c < nc; c += kSelThreads) sh.S[c] = sh.C[c];
    __syncthreads();
    const unsigned long long total = block_excl_scan<unsigned long long, NT>(sh.S, nc, sh.wtmp);
    if (tid == 0) sh.S[nc] = total;
    __syncthreads();
    const int hw = (p.pool_k - 1) / 2;
    const int last_len = M - (nc - 1) * chunk;
    constexpr int kPer = C_::kScanPer;
    unsigned long long key[kPer], cm[kPer];
    bool valid[kPer];
    unsigned long long kand = ~0ull, kor = 0ull;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int c = tid + e * kSelThreads;
        valid[e] = c < nc;
        key[e] = 0ull;
        cm[e] = 0ull;
        if (valid[e]) {
            const int lo = c - hw < 0 ? 0 : c - hw;
            const int hi = c + hw > nc - 1 ? nc - 1 : c + hw;
            const unsigned long long P = sh.S[hi + 1] - sh.S[lo];
            const long long T = (long long)(hi - lo + 1) * chunk - (hi == nc - 1 ? chunk - last_len : 0);
            key[e] = (unsigned long long)__double_as_longlong((double)P / (double)T);
            cm[e] = sh.C[c];
            kand &= key[e];
            kor |= key[e];
        }
    }

    // 5. The kept chunks are the first kc in rank order (key descending, then
    // index ascending): top-K takes kc = max(1, ceil(rate * nc)); mass walks
    // the ranking adding own masses and stops at the first rank whose
    // cumulative mass reaches mass * total (all chunks if none does). Instead
    // of sorting, a radix select over the key bits narrows down the keys
    // around the last kept rank, with the count and mass of all keys above
    // them; the few left are ranked exactly (equal keys: lowest index first).
    const bool topk = p.mode == SP_SELECT_TOPK;
    long long kc_topk = 0;
    double thr = 0.0;
    bool keep_all = false;
    if (topk) {
        kc_topk = (long long)ceil((double)p.keep_rate * (double)nc);
        if (kc_topk < 1) kc_topk = 1;
        if (kc_topk > nc) kc_topk = nc;
    } else {
        thr = (double)p.mass * (double)total;
        keep_all = !((double)total >= thr);  // no rank reaches the threshold
    }
    // Rounds fix kDigit bits at a time from the highest bit where keys
    // differ, keeping the candidates (keys matching prefix on the bits of
    // fmask) that contain the last kept rank, until at most kFinal are left or
    // all bits are fixed. Keys above the candidates rank before all of them.
    // With at most kFinal chunks there are no rounds: every chunk is a
    // candidate (fmask and prefix 0).
    int hi = -1;
    unsigned long long fmask = 0ull, prefix = 0ull;
    if (nc > kFinal && !keep_all) {
        kand = wave_bitwise64<true>(kand);
        kor = wave_bitwise64<false>(kor);
        if (lane == 0) {
            sh.rand_[w] = kand;
            sh.ror_[w] = kor;
        }
        __syncthreads();
        kand = ~0ull;
        kor = 0ull;
        for (int x2 = 0; x2 < kSelWaves; ++x2) {
            kand &= sh.rand_[x2];
            kor |= sh.ror_[x2];
        }
        const unsigned long long diff = kand ^ kor;  // bits where the keys differ
        hi = diff == 0ull ? -1 : 63 - __builtin_clzll(diff);
        fmask = hi >= 63 ? 0ull : ~0ull << (hi + 1);
        prefix = kand & fmask;
    }
    unsigned long long above_mass = 0ull;
    unsigned int above_count = 0u;
    unsigned int ncand = (unsigned)nc;
    for (int rnd = 0; hi >= 0 && ncand > (unsigned)kFinal && !keep_all; ++rnd) {
        const int hb = rnd & 1;
        const int lo = hi - (kDigit - 1) > 0 ? hi - (kDigit - 1) : 0;
        const int nbits = hi - lo + 1;
        const int nbins = 1 << nbits;
        const unsigned long long dmask = (unsigned long long)(nbins - 1);
        if (rnd == 0) {
            for (int d = tid; d < kBins; d += kSelThreads) {
                sh.hcount[0][d] = 0u;
                sh.hmass[0][d] = 0ull;
            }
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            if (valid[e] && (key[e] & fmask) == prefix) {
                const int d = (int)((key[e] >> lo) & dmask);
                // (transposed: wave 0's lane L reads digits 32 (63 - L) + b
                // at b * 64 + 63 - L, conflict-free)
                const int h = (d & 31) * 64 + (d >> 5);
                atomicAdd(&sh.hcount[hb][h], 1u);
                if (!topk) atomicAdd(&sh.hmass[hb][h], cm[e]);
            }
        __syncthreads();
        if (w == 0) {
            // lane L sums digits 32 (63 - L) .. 32 (63 - L) + 31, so lanes
            // ascend as digits descend (digits >= nbins are empty)
            const int a0 = 63 - lane;
            unsigned int lc = 0u;
            unsigned long long lm = 0ull;
            if (topk) {
#pragma unroll
                for (int j = 0; j < 32; ++j) lc += sh.hcount[hb][j * 64 + a0];
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    lc += sh.hcount[hb][j * 64 + a0];
                    lm += sh.hmass[hb][j * 64 + a0];
                }
            }
            const unsigned int ic = wave_scan_u32(lc);
            const unsigned long long im = topk ? 0ull : wave_scan_u64(lm);
            // the first digit (descending) whose inclusive cumulative reaches the target
            const bool reach = topk ? (long long)(above_count + ic) >= kc_topk
                                    : (double)(above_mass + im) >= thr;
            const unsigned long long bal = __ballot(reach);
            const int F = bal ? __builtin_ctzll(bal) : 63;
            // counts before lane F's digits, then lane F's digits one per lane, descending
            const unsigned int cF = __shfl(ic - lc, F);
            const unsigned long long mF = topk ? 0ull : __shfl(im - lm, F);
            const bool mine = lane < 32;
            const int hF = (31 - (lane & 31)) * 64 + (63 - F);
            const unsigned int c1 = mine ? sh.hcount[hb][hF] : 0u;
            const unsigned long long m1 = (mine && !topk) ? sh.hmass[hb][hF] : 0ull;
            const unsigned int ic1 = wave_scan_u32(c1);
            const unsigned long long im1 = topk ? 0ull : wave_scan_u64(m1);
            const bool reach1 = mine && (topk ? (long long)(above_count + cF + ic1) >= kc_topk
                                              : (double)(above_mass + mF + im1) >= thr);
            const unsigned long long bal1 = __ballot(reach1);
            const int J = bal1 ? __builtin_ctzll(bal1) : 0;
            if (lane == J) {
                sh.bc_prefix = prefix | ((unsigned long long)(32 * (63 - F) + 31 - J) << lo);
                sh.bc_count = above_count + cF + ic1 - c1;
                sh.bc_mass = above_mass + mF + im1 - m1;
                sh.bc_ties = c1;
            }
        } else {
            // the next round's histogram set
            for (int x2 = tid - 64; x2 < kBins; x2 += kSelThreads - 64) {
                sh.hcount[hb ^ 1][x2] = 0u;
                sh.hmass[hb ^ 1][x2] = 0ull;
            }
        }
        __syncthreads();
        prefix = sh.bc_prefix;
        above_count = sh.bc_count;
        above_mass = sh.bc_mass;
        ncand = sh.bc_ties;
        fmask |= dmask << lo;
        hi = lo - 1;
    }
    __syncthreads();  // the histograms alias S

    // The last candidates: at most kFinal are ranked exactly, one per thread;
    // more can only remain when all their bits are fixed, i.e. they are equal
    // keys, and then their index order decides (a scan).
    bool keep[kPer];
    int slot[kPer];
    const bool exact = !keep_all && ncand <= (unsigned)kFinal;
    if (exact) {
        if (tid == 0) sh.ncand = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            slot[e] = -1;
            if (valid[e] && (key[e] & fmask) == prefix) {
                const int sl = atomicAdd(&sh.ncand, 1);
                if (sl < kFinal) {
                    slot[e] = sl;
                    sh.ck[sl] = key[e];
                    sh.ci[sl] = (unsigned)(tid + e * kSelThreads);
                    sh.cmass[sl] = cm[e];
                }
            }
        }
        __syncthreads();
        // slots up to the next multiple of kRankBatch: entries that rank
        // before none (key 0 with an index past every chunk)
        const int n = sh.ncand < kFinal ? sh.ncand : kFinal;
        const int npad = (n + kRankBatch - 1) / kRankBatch * kRankBatch;
        if (tid >= n && tid < npad) {
            sh.ck[tid] = 0ull;
            sh.ci[tid] = ~0u;
            sh.cmass[tid] = 0ull;
        }
        __syncthreads();
        {
            if (tid < n) {
                const unsigned long long mk = sh.ck[tid];
                const unsigned int mi = sh.ci[tid];
                unsigned int rank = 0u;
                unsigned long long before = 0ull;
                // kRankBatch candidates' loads in flight at a time
                for (int j0 = 0; j0 < npad; j0 += kRankBatch) {
                    unsigned long long kk[kRankBatch], mm[kRankBatch];
                    unsigned int ii[kRankBatch];
#pragma unroll
                    for (int u = 0; u < kRankBatch; ++u) {
                        kk[u] = sh.ck[j0 + u];
                        ii[u] = sh.ci[j0 + u];
                        mm[u] = sh.cmass[j0 + u];
                    }
#pragma unroll
                    for (int u = 0; u < kRankBatch; ++u) {
                        const bool b = ranks_before(kk[u], ii[u], mk, mi);
                        rank += b ? 1u : 0u;
                        before += mm[u] & (0ull - (unsigned long long)b);  // (every load used)
                    }
                }
                sh.ckeep[tid] = topk ? (long long)(above_count + rank) < kc_topk
                                      : (double)(above_mass + before) < thr;
            }
        }
        __syncthreads();
    } else if (!keep_all) {
        for (int c = tid; c < nc; c += kSelThreads) sh.S[c] = 0ull;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            if (valid[e] && (key[e] & fmask) == prefix) sh.S[tid + e * kSelThreads] = topk ? 1ull : cm[e];
        __syncthreads();
        block_excl_scan<unsigned long long, NT>(sh.S, nc, sh.wtmp);
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int c = tid + e * kSelThreads;
        bool k = false;
        if (valid[e]) {
            if (keep_all || (key[e] & fmask) > prefix) {
                k = true;
            } else if ((key[e] & fmask) == prefix) {
                if (exact) {
                    k = slot[e] >= 0 && sh.ckeep[slot[e]];
                } else {
                    const unsigned long long before = sh.S[c];
                    k = topk ? (long long)(above_count + before) < kc_topk
                             : (double)(above_mass + before) < thr;
                }
            }
        }
        keep[e] = k;
    }
    __syncthreads();

    // 6. kept chunks in index order: klist by an exclusive scan of the flags
#pragma unroll
    for (int e = 0; e < kPer; ++e)
        if (valid[e]) sh.off[tid + e * kSelThreads] = keep[e] ? 1 : 0;
    __syncthreads();
    const int kc = block_excl_scan<int, NT>(sh.off, nc, sh.wtmp);
#pragma unroll
    for (int e = 0; e < kPer; ++e)
        if (valid[e] && keep[e]) sh.klist[sh.off[tid + e * kSelThreads]] = tid + e * kSelThreads;
    __syncthreads();

    // 7. emit kept tokens ascending (coalesced over output positions). Every
    // kept chunk but chunk nc - 1 (last in the list when kept) holds chunk
    // tokens, so output o lies in kept chunk min(o / chunk, kc - 1).
    const bool last_kept = kc > 0 && sh.klist[kc - 1] == nc - 1;
    const int n_kept = kc * chunk - (last_kept ? chunk - last_len : 0);
    for (int o = tid; o < n_kept; o += kSelThreads) {
        int k = o / chunk;
        if (k > kc - 1) k = kc - 1;
        const int i = sh.klist[k] * chunk + (o - k * chunk);
        kept[o] = base + i;
        pos[o] = pb + i;
    }
    if (tid == 0) *nkept_out = n_kept;
}

// The selection of one long prompt by a grid of W workgroups (W = gridDim.x,
// all resident at once) with min-max normalisation: workgroup b takes chunks
// [nc b / W, nc (b + 1) / W) and publishes the min and max of their scores
// (or a mark that one is not finite); once all W are there, it sums those
// chunks' fixed-point masses (exact, so the split does not change them) and
// publishes each as two tagged words; workgroup 0 gathers every chunk's mass
// and runs steps 4-7. slots: [0, 2 W) the ranges, from kSelDistChunkSlot the
// masses (low, high) of chunk c at 2 c. Every wait gives up after spin ticks
// of the 100 MHz clock (then n_kept = -1).
constexpr int kSelDistChunkSlot = 2 * 256;

template <int NT>
__device__ void select_distributed(SelectShared<NT>& sh, const SelectParamsDev& p, const float* __restrict__ x,
                                   int M, int pb, int32_t* __restrict__ kept, int32_t* __restrict__ pos,
                                   int32_t* __restrict__ nkept_out, unsigned long long* slots, unsigned E,
                                   unsigned long long spin) {
    using C_ = SelCfg<NT>;
    constexpr int kSelWaves = C_::kWaves;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int W = (int)gridDim.x, b = (int)blockIdx.x;
    const int chunk = p.chunk;
    const int nc = (M + chunk - 1) / chunk;
    const int c0 = (int)((long long)nc * b / W), c1 = (int)((long long)nc * (b + 1) / W);
    const int e0 = c0 * chunk, e1 = min(M, c1 * chunk);
    const unsigned long long Et = (unsigned long long)E << 32;

    // 1. this range's min and max (exact in any order)
    float mn = INFINITY, mx = -INFINITY;
    int nonfinite = 0;
    for (int i = e0 + tid; i < e1; i += NT) {
        const float v = x[i];
        nonfinite |= (__float_as_uint(v) & 0x7f800000u) == 0x7f800000u;
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if (lane == 0) {
        sh.fmin[w] = mn;
        sh.fmax[w] = mx;
    }
    const bool nf = __syncthreads_or(nonfinite);
    if (tid == 0) {
        for (int x2 = 1; x2 < kSelWaves; ++x2) {
            mn = fminf(mn, sh.fmin[x2]);
            mx = fmaxf(mx, sh.fmax[x2]);
        }
        st64u(slots + 2 * b, Et | __float_as_uint(fminf(mn, sh.fmin[0])));
        st64u(slots + 2 * b + 1, Et | (nf ? kNonFiniteMark : __float_as_uint(fmaxf(mx, sh.fmax[0]))));
    }

    // 2. the prompt's min and max from every range (lane x reads range x)
    if (w == 0) {
        float gmn = INFINITY, gmx = -INFINITY;
        bool bad = false;
        const unsigned long long t0 = wall_clock64();
        while (true) {
            bool miss = false, nfx = false;
            gmn = INFINITY;
            gmx = -INFINITY;
            if (lane < W) {
                const unsigned long long lo = ld64(slots + 2 * lane), hi = ld64(slots + 2 * lane + 1);
                miss = !(tag_is(lo, E) && tag_is(hi, E));
                nfx = (unsigned)hi == kNonFiniteMark;
                gmn = tag_value(lo);
                gmx = tag_value(hi);
            }
            if (__ballot(miss) == 0) {
                bad = __ballot(nfx) != 0;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            if (wall_clock64() - t0 > spin) {
                bad = true;
                break;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            gmn = fminf(gmn, __shfl_xor(gmn, o));
            gmx = fmaxf(gmx, __shfl_xor(gmx, o));
        }
        if (lane == 0) {
            sh.pct[0] = gmn;
            sh.pct[1] = gmx;
            sh.ncand = bad ? 1 : 0;
        }
    }
    __syncthreads();
    if (sh.ncand) {
        // (a non-finite score, or a range that never came)
        if (b == 0 && tid == 0) *nkept_out = -1;
        return;
    }
    MinMaxNorm nm;
    nm.init(sh.pct[0], sh.pct[1]);

    // 3. this range's chunk masses
    for (int c = c0 + tid; c < c1; c += NT) sh.C[c - c0] = 0ull;
    __syncthreads();
    for (int i = e0 + tid; i < e1; i += NT) atomicAdd(&sh.C[i / chunk - c0], token_mass(nm.value(x[i]), i, M, p));
    __syncthreads();
    for (int c = c0 + tid; c < c1; c += NT) {
        const unsigned long long v = sh.C[c - c0];
        st64u(slots + kSelDistChunkSlot + 2 * c, Et | (unsigned)v);
        st64u(slots + kSelDistChunkSlot + 2 * c + 1, Et | (unsigned)(v >> 32));
    }
    if (b != 0) return;
    __syncthreads();  // (the gather rewrites C)

    // 4. workgroup 0: every chunk's mass, then the ranking
    constexpr int P = kSelMaxChunks / NT;  // chunks per thread
    unsigned long long lo[P], hi[P];
    unsigned pend = 0;  // bit e: chunk tid + e NT not seen yet
#pragma unroll
    for (int e = 0; e < P; ++e) {
        lo[e] = hi[e] = 0ull;
        if (tid + e * NT < nc) pend |= 1u << e;
    }
    bool expired = false;
    const unsigned long long t0 = wall_clock64();
    while (true) {
#pragma unroll
        for (int e = 0; e < P; ++e)
            if ((pend >> e) & 1) {
                const unsigned long long* sl = slots + kSelDistChunkSlot + 2 * (tid + e * NT);
                lo[e] = ld64(sl);
                hi[e] = ld64(sl + 1);
            }
        unsigned np = 0;
#pragma unroll
        for (int e = 0; e < P; ++e)
            if (((pend >> e) & 1) && !(tag_is(lo[e], E) && tag_is(hi[e], E))) np |= 1u << e;
        pend = np;
        if (__ballot(pend != 0) == 0) break;
        __builtin_amdgcn_s_sleep(2);
        if (wall_clock64() - t0 > spin) {
            expired = true;
            break;
        }
    }
#pragma unroll
    for (int e = 0; e < P; ++e)
        if (tid + e * NT < nc) sh.C[tid + e * NT] = (unsigned long long)(unsigned)lo[e] | (hi[e] << 32);
    if (__syncthreads_or(expired)) {
        if (tid == 0) *nkept_out = -1;
        return;
    }
    select_ranked<NT>(sh, p, M, 0, pb, kept, pos, nkept_out);
}

}  // namespace sp
