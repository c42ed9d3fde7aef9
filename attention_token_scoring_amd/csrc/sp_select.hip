// Chunk selection and compaction on gfx950: one workgroup per request.
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
//   (mass), emit kept tokens ascending with their position ids.
// Every step is exact or a single IEEE-rounded operation (fp32 sub/div/mul,
// u64 -> f64 conversion, f64 div and mul), and sums are integer, so the
// result is the same however the work is split across threads: a CPU doing
// the same steps in any order reproduces it bit for bit. Compiled with
// -ffp-contract=off.
#include <math.h>

#include "sp_internal.h"

namespace sp {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxChunks = 4096;
constexpr int kSelBatch = 256;  // requests per launch (offsets travel in the kernel arguments)

struct SelectBatch {
    int cu[kSelBatch + 1];      // prompt offsets of the requests in this launch
    int pos_base[kSelBatch];
    int first;                  // index of this launch's first request (for n_kept)
};

struct SelectShared {
    unsigned long long C[kMaxChunks];     // chunk masses
    unsigned long long S[kMaxChunks + 1]; // prefix sums, then sort keys, then ranked cumsums
    unsigned int idx[kMaxChunks];         // chunk index in rank order
    int off[kMaxChunks];                  // kept-token offset of each kept chunk (compacted)
    int klist[kMaxChunks];                // kept chunks in index order
    unsigned long long wtmp[kSelWaves];
    float fmin[kSelWaves], fmax[kSelWaves];
    int kc;                               // number of kept chunks
};

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const T u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// In-place exclusive scan of data[0..n) (n <= 4 * kSelThreads); returns the total.
template <typename T>
__device__ T block_excl_scan(T* data, int n, unsigned long long* wtmp) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int i0 = tid * 4;
    T loc[4];
    T run = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        loc[e] = (i0 + e < n) ? data[i0 + e] : (T)0;
        run += loc[e];
    }
    T incl = wave_incl_scan<T>(run, lane);
    if (lane == 63) wtmp[w] = (unsigned long long)incl;
    __syncthreads();
    T wbase = 0, total = 0;
    for (int x = 0; x < kSelWaves; ++x) {
        const T t = (T)wtmp[x];
        if (x < w) wbase += t;
        total += t;
    }
    T ex = wbase + incl - run;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (i0 + e < n) data[i0 + e] = ex;
        ex += loc[e];
    }
    __syncthreads();
    return total;
}

__device__ __forceinline__ bool ranks_before(unsigned long long ka, unsigned int ia,
                                             unsigned long long kb, unsigned int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectBatch b, SelectParamsDev p,
                                                             const float* __restrict__ x_all,
                                                             int32_t* __restrict__ kept_all,
                                                             int32_t* __restrict__ pos_all,
                                                             int32_t* __restrict__ nkept_all) {
    extern __shared__ unsigned long long smem_raw[];
    SelectShared& sh = *reinterpret_cast<SelectShared*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = blockIdx.x;
    const int base = b.cu[r];
    const int M = b.cu[r + 1] - base;
    const float* x = x_all + base;
    const int chunk = p.chunk;
    const int nc = (M + chunk - 1) / chunk;

    // 1. min and max (exact in any order)
    float mn = INFINITY, mx = -INFINITY;
    for (int i = tid; i < M; i += kSelThreads) {
        const float v = x[i];
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
    for (int c = tid; c < nc; c += kSelThreads) sh.C[c] = 0ull;
    __syncthreads();
    mn = sh.fmin[0];
    mx = sh.fmax[0];
    for (int x2 = 1; x2 < kSelWaves; ++x2) {
        mn = fminf(mn, sh.fmin[x2]);
        mx = fmaxf(mx, sh.fmax[x2]);
    }
    const float range = mx - mn;

    // 2-3. normalise, boost, fixed point, chunk sums
    const bool pow2 = (chunk & (chunk - 1)) == 0;
    const int seg = chunk < 64 ? chunk : 64;
    for (int blk = w; blk * 64 < M; blk += kSelWaves) {
        const int i = blk * 64 + lane;
        unsigned long long q = 0ull;
        if (i < M) {
            float v = 1.0f;
            if (range > 0.f) v = __fdiv_rn(x[i] - mn, range);
            if (i < p.first_n) v = v * p.first_mult;
            if (i >= M - p.last_n) v = v * p.last_mult;
            q = (unsigned long long)rintf(v * 4294967296.0f);
        }
        if (pow2) {
            for (int o = seg >> 1; o > 0; o >>= 1) q += __shfl_xor(q, o);
            if ((lane & (seg - 1)) == 0 && i < M) {
                if (chunk <= 64)
                    sh.C[i / chunk] = q;
                else
                    atomicAdd(&sh.C[i / chunk], q);
            }
        } else if (i < M) {
            atomicAdd(&sh.C[i / chunk], q);
        }
    }
    __syncthreads();

    // 4. pooled keys from prefix sums: key_c = (S[hi+1] - S[lo]) / tokens in window
    for (int c = tid; c < nc; c += kSelThreads) sh.S[c] = sh.C[c];
    __syncthreads();
    const unsigned long long total = block_excl_scan<unsigned long long>(sh.S, nc, sh.wtmp);
    if (tid == 0) sh.S[nc] = total;
    __syncthreads();
    const int hw = (p.pool_k - 1) / 2;
    const int last_len = M - (nc - 1) * chunk;
    unsigned long long kb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = tid + e * kSelThreads;
        kb[e] = 0ull;
        if (c < nc) {
            const int lo = c - hw < 0 ? 0 : c - hw;
            const int hi = c + hw > nc - 1 ? nc - 1 : c + hw;
            const unsigned long long P = sh.S[hi + 1] - sh.S[lo];
            const long long T = (long long)(hi - lo + 1) * chunk - (hi == nc - 1 ? chunk - last_len : 0);
            const double key = (double)P / (double)T;
            kb[e] = (unsigned long long)__double_as_longlong(key) + 1ull;  // 0 marks padding
        }
    }
    int ncp = 1;
    while (ncp < nc) ncp <<= 1;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = tid + e * kSelThreads;
        if (c < ncp) {
            sh.S[c] = kb[e];
            sh.idx[c] = (unsigned)c;
        }
    }
    __syncthreads();

    // 5. bitonic sort into rank order: key descending, then index ascending
    for (int k = 2; k <= ncp; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            for (int i = tid; i < ncp; i += kSelThreads) {
                const int l = i ^ jj;
                if (l > i) {
                    const unsigned long long ka = sh.S[i], kl = sh.S[l];
                    const unsigned ia = sh.idx[i], il = sh.idx[l];
                    const bool l_first = ranks_before(kl, il, ka, ia);
                    const bool up = (i & k) == 0;
                    if (up == l_first) {
                        sh.S[i] = kl;
                        sh.S[l] = ka;
                        sh.idx[i] = il;
                        sh.idx[l] = ia;
                    }
                }
            }
            __syncthreads();
        }
    }

    // 6. number of kept chunks
    if (p.mode == SP_SELECT_TOPK) {
        if (tid == 0) {
            long long K = (long long)ceil((double)p.keep_rate * (double)nc);
            if (K < 1) K = 1;
            if (K > nc) K = nc;
            sh.kc = (int)K;
        }
    } else {
        // ranked cumulative own masses; kept = (ranks whose cumsum is still below
        // the threshold) + 1, since the cumsum only grows
        for (int i = tid; i < nc; i += kSelThreads) sh.S[i] = sh.C[sh.idx[i]];
        if (tid == 0) sh.kc = 0;
        __syncthreads();
        block_excl_scan<unsigned long long>(sh.S, nc, sh.wtmp);
        const double thr = (double)p.mass * (double)total;
        int below = 0;
        for (int i = tid; i < nc; i += kSelThreads) {
            const unsigned long long incl = sh.S[i] + sh.C[sh.idx[i]];
            below += ((double)incl < thr) ? 1 : 0;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) below += __shfl_xor(below, o);
        if (lane == 0) atomicAdd(&sh.kc, below);
        __syncthreads();
        if (tid == 0) sh.kc = sh.kc + 1 > nc ? nc : sh.kc + 1;
    }
    __syncthreads();

    // 7. kept flags in chunk order -> offsets of kept tokens
    const int kc = sh.kc;
    for (int c = tid; c < nc; c += kSelThreads) sh.off[c] = 0;
    __syncthreads();
    for (int i = tid; i < kc; i += kSelThreads) sh.off[sh.idx[i]] = 1;
    __syncthreads();
    // klist position of each kept chunk (exclusive scan of the flags)
    for (int c = tid; c < nc; c += kSelThreads) sh.klist[c] = sh.off[c];
    __syncthreads();
    block_excl_scan<int>(sh.klist, nc, sh.wtmp);
    // kept chunk k (in index order) -> chunk id; token offsets by scan of lengths
    for (int c = tid; c < nc; c += kSelThreads) {
        if (sh.off[c]) {
            const int k = sh.klist[c];
            sh.idx[k] = (unsigned)c;  // rank order no longer needed
        }
    }
    __syncthreads();
    for (int k = tid; k < kc; k += kSelThreads) {
        const int c = (int)sh.idx[k];
        sh.off[k] = (c == nc - 1) ? last_len : chunk;
    }
    __syncthreads();
    const int n_kept = block_excl_scan<int>(sh.off, kc, sh.wtmp);

    // 8. emit kept tokens ascending (coalesced over output positions)
    int32_t* kept = kept_all + base;
    int32_t* pos = pos_all + base;
    const int pb = b.pos_base[r];
    for (int o = tid; o < n_kept; o += kSelThreads) {
        int lo = 0, hi = kc - 1;  // last k with off[k] <= o
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.off[mid] <= o) lo = mid; else hi = mid - 1;
        }
        const int i = (int)sh.idx[lo] * chunk + (o - sh.off[lo]);
        kept[o] = base + i;
        pos[o] = pb + i;
    }
    if (tid == 0) nkept_all[b.first + r] = n_kept;
}

size_t select_shared_bytes() { return sizeof(SelectShared); }

// Launches the selection of requests [0, R) whose prompt offsets are cu[0..R].
hipError_t launch_select(const SelectParamsDev& p, const int64_t* cu, const int32_t* pos_base,
                         int R, const float* importance, int32_t* kept_idx, int32_t* pos_ids,
                         int32_t* n_kept, hipStream_t stream) {
    const size_t lds = sizeof(SelectShared);
    hipError_t e = hipFuncSetAttribute((const void*)&select_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    for (int r0 = 0; r0 < R; r0 += kSelBatch) {
        const int nr = R - r0 < kSelBatch ? R - r0 : kSelBatch;
        SelectBatch b;
        for (int i = 0; i <= nr; ++i) b.cu[i] = (int)cu[r0 + i];
        for (int i = 0; i < nr; ++i) b.pos_base[i] = pos_base ? pos_base[r0 + i] : 0;
        b.first = r0;
        hipLaunchKernelGGL(select_kernel, dim3(nr), dim3(kSelThreads), lds, stream, b, p,
                           importance, kept_idx, pos_ids, n_kept);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sp
