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
//   (mass), emit kept tokens ascending with their position ids. The ranking
//   is never materialised: a radix select over the keys' bits finds the key
//   of the last kept rank, and ties on it are settled by index.
// Every step is exact or a single IEEE-rounded operation (fp32 sub/div/mul,
// u64 -> f64 conversion, f64 div and mul), and sums are integer, so the
// result is the same however the work is split across threads: a CPU doing
// the same steps in any order reproduces it bit for bit. Compiled with
// -ffp-contract=off.
#include "sp_select_core.h"

namespace sp {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxThreshChunks = 4096;  // (the threshold mode's bitonic sort)
constexpr int kSelBatch = 256;  // requests per launch (offsets travel in the kernel arguments)

struct SelectBatch {
    int cu[kSelBatch + 1];      // prompt offsets of the requests in this launch
    int pos_base[kSelBatch];
    int first;                  // index of this launch's first request (for n_kept)
};

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectBatch b, SelectParamsDev p,
                                                             const float* __restrict__ x_all,
                                                             int32_t* __restrict__ kept_all,
                                                             int32_t* __restrict__ pos_all,
                                                             int32_t* __restrict__ nkept_all) {
    extern __shared__ unsigned long long smem_raw[];
    SelectShared<kSelThreads>& sh = *reinterpret_cast<SelectShared<kSelThreads>*>(smem_raw);
    const int r = blockIdx.x;
    const int base = b.cu[r];
    select_prompt<kSelThreads>(sh, p, x_all + base, b.cu[r + 1] - base, base, b.pos_base[r], kept_all + base,
                               pos_all + base, nkept_all + b.first + r);
}

// ---------------------------------------------------------------------------------------
// Threshold selection: the steps of the Implementation Guide's own program
// ("SpecPrefill - Implementation Guide", Full Source Code: its chunk selection
// and the cap on sparse tokens; How It Works, chunk selection: the first 4 and
// last 2 tokens always kept; Configuration Reference: SP_MAX_KEEP), on the raw
// scores: chunk means (double sums in index order, rounded to float), a
// threshold at the K-th largest mean (K = max(1, ceil(nc * keep_rate)), the
// product in single precision) keeping every chunk that reaches it, tokens
// 0..3 and (M > 4) M-2, M-1, a fill of the dropped chunks' tokens in index
// order up to eff_min = min(min_tok, max(4, M / 10)) tokens, everything when
// keep_rate >= 1 or M <= eff_min, and with max_keep > 0 a cap to every
// (n / max_keep)-th kept token, the last one replaced by the last kept token.
// One workgroup per request; each chunk's mean is one thread's sequential sum,
// so the result does not depend on how the work is split.
// ---------------------------------------------------------------------------------------
struct ThreshShared {
    float a[kMaxThreshChunks];     // chunk means
    float srt[kMaxThreshChunks];   // the means sorted descending (padded with -inf)
    int cnt[kMaxThreshChunks];     // free tokens of dropped chunks, then their exclusive scan
    int off[kMaxThreshChunks];     // kept tokens per chunk, then their exclusive scan
    unsigned long long wtmp[kSelWaves];
    float thr;
    int total;
};

__device__ __forceinline__ int always_in(int i0, int i1, int M) {
    // tokens of [i0, i1) among 0..3 and, when M > 4, M-2 and M-1
    int n = 0;
    for (int t = 0; t < 4 && t < M; ++t) n += t >= i0 && t < i1;
    if (M > 4)
        for (int t = M - 2; t < M; ++t) n += t >= i0 && t < i1 && t > 3;
    return n;
}

__device__ __forceinline__ bool is_always(int t, int M) { return t < 4 || (M > 4 && t >= M - 2); }

__global__ __launch_bounds__(kSelThreads) void select_threshold_kernel(
    SelectBatch b, SelectParamsDev p, const float* __restrict__ x_all, int32_t* __restrict__ kept_all,
    int32_t* __restrict__ pos_all, int32_t* __restrict__ nkept_all) {
    extern __shared__ unsigned long long smem_raw[];
    ThreshShared& sh = *reinterpret_cast<ThreshShared*>(smem_raw);
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int base = b.cu[r];
    const int M = b.cu[r + 1] - base;
    const float* x = x_all + base;
    const int chunk = p.chunk;
    const int nc = (M + chunk - 1) / chunk;
    const int pb = b.pos_base[r];
    int32_t* kept = kept_all + base;
    int32_t* pos = pos_all + base;
    const int eff_min = min(p.min_tok, max(4, M / 10));
    // non-finite scores: count -1, outputs untouched (as in select_kernel)
    int nonfinite = 0;
    for (int i = tid; i < M; i += kSelThreads)
        nonfinite |= (__float_as_uint(x[i]) & 0x7f800000u) == 0x7f800000u;
    if (__syncthreads_or(nonfinite)) {
        if (tid == 0) nkept_all[b.first + r] = -1;
        return;
    }
    int n;
    if (p.keep_rate >= 1.0f || M <= eff_min) {
        for (int o = tid; o < M; o += kSelThreads) {
            kept[o] = base + o;
            pos[o] = pb + o;
        }
        n = M;
    } else {
        // 1. chunk means
        for (int c = tid; c < nc; c += kSelThreads) {
            const int i0 = c * chunk, i1 = min(i0 + chunk, M);
            double sum = 0.0;
            for (int i = i0; i < i1; ++i) sum += (double)x[i];
            const float mean = (float)(sum / (double)(i1 - i0));
            sh.a[c] = mean;
            sh.srt[c] = mean;
        }
        int np2 = 1;
        while (np2 < nc) np2 <<= 1;
        for (int c = nc + tid; c < np2; c += kSelThreads) sh.srt[c] = -INFINITY;
        __syncthreads();
        // 2. bitonic sort, descending
        for (int k = 2; k <= np2; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < np2; i += kSelThreads) {
                    const int l = i ^ j;
                    if (l > i) {
                        const float u = sh.srt[i], v = sh.srt[l];
                        if ((i & k) == 0 ? u < v : u > v) {
                            sh.srt[i] = v;
                            sh.srt[l] = u;
                        }
                    }
                }
                __syncthreads();
            }
        }
        // 3. threshold: the K-th largest mean
        int K = (int)ceilf(__fmul_rn((float)nc, p.keep_rate));
        if (K < 1) K = 1;
        if (K > nc) K = nc;
        const float thr = sh.srt[K - 1];
        // 4. per chunk: kept tokens before the fill, and free tokens of dropped
        // chunks (those the fill may take, in index order)
        for (int c = tid; c < nc; c += kSelThreads) {
            const int i0 = c * chunk, i1 = min(i0 + chunk, M);
            const int al = always_in(i0, i1, M);
            const bool keep_c = sh.a[c] >= thr;
            sh.off[c] = keep_c ? i1 - i0 : al;
            sh.cnt[c] = keep_c ? 0 : i1 - i0 - al;
        }
        __syncthreads();
        const int n_base = block_excl_scan<int, kSelThreads>(sh.off, nc, sh.wtmp);  // (off: scanned, unused)
        block_excl_scan<int, kSelThreads>(sh.cnt, nc, sh.wtmp);
        const int need = max(eff_min - n_base, 0);
        // 5. final kept count per chunk (the fill takes need tokens in index order)
        for (int c = tid; c < nc; c += kSelThreads) {
            const int i0 = c * chunk, i1 = min(i0 + chunk, M);
            const int al = always_in(i0, i1, M);
            const bool keep_c = sh.a[c] >= thr;
            const int free_c = keep_c ? 0 : i1 - i0 - al;
            const int take = min(max(need - sh.cnt[c], 0), free_c);
            sh.off[c] = keep_c ? i1 - i0 : al + take;
            sh.cnt[c] = take;  // (each thread rewrites only its own chunks)
        }
        __syncthreads();
        n = block_excl_scan<int, kSelThreads>(sh.off, nc, sh.wtmp);
        // 6. emit: output o lies in the last chunk whose offset is <= o
        for (int o = tid; o < n; o += kSelThreads) {
            int lo = 0, hi = nc - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh.off[mid] <= o) lo = mid;
                else hi = mid - 1;
            }
            const int c = lo, i0 = c * chunk, i1 = min(i0 + chunk, M);
            int i;
            if (sh.a[c] >= thr) {
                i = i0 + (o - sh.off[c]);
            } else {
                // the j-th kept token of a dropped chunk: its always-kept tokens
                // and its first `take` other tokens, ascending
                int j = o - sh.off[c], others = 0;
                i = i0;
                for (int t = i0; t < i1; ++t) {
                    bool k;
                    if (is_always(t, M)) {
                        k = true;
                    } else {
                        k = others < sh.cnt[c];
                        ++others;
                    }
                    if (k) {
                        if (j == 0) {
                            i = t;
                            break;
                        }
                        --j;
                    }
                }
            }
            kept[o] = base + i;
            pos[o] = pb + i;
        }
    }
    // 7. cap: every step-th kept token, the last replaced by the last kept one;
    // rounds of kSelThreads outputs read before they are written (a round
    // writes below every index a later round reads)
    if (p.max_keep > 0 && n > p.max_keep) {
        __threadfence_block();
        __syncthreads();
        const int step = n / p.max_keep;
        const int32_t last = kept[n - 1];
        for (int o0 = 0; o0 < p.max_keep; o0 += kSelThreads) {
            const int o = o0 + tid;
            int32_t v = 0;
            if (o < p.max_keep) v = o == p.max_keep - 1 ? last : kept[o * step];
            __syncthreads();
            if (o < p.max_keep) {
                kept[o] = v;
                pos[o] = pb + (v - base);
            }
            __threadfence_block();
            __syncthreads();
        }
        n = p.max_keep;
    }
    if (tid == 0) nkept_all[b.first + r] = n;
}

// One long prompt by several workgroups (min-max normalisation): see
// select_distributed.
__global__ __launch_bounds__(kSelThreads) void select_dist_kernel(SelectParamsDev p, const float* __restrict__ x,
                                                                  int M, int pb, int32_t* __restrict__ kept,
                                                                  int32_t* __restrict__ pos,
                                                                  int32_t* __restrict__ nkept,
                                                                  unsigned long long* slots, unsigned epoch,
                                                                  unsigned long long spin) {
    extern __shared__ unsigned long long smem_raw[];
    SelectShared<kSelThreads>& sh = *reinterpret_cast<SelectShared<kSelThreads>*>(smem_raw);
    select_distributed<kSelThreads>(sh, p, x, M, pb, kept, pos, nkept, slots, epoch, spin);
}

size_t select_shared_bytes() { return sizeof(SelectShared<kSelThreads>); }

// Launches the selection of one prompt of M >= kSelGridMin tokens by a grid of
// workgroups (about 2048 tokens each, 2 to 64 of them: one lane per range in
// the exchange, and all resident at once on an idle device) on a workspace
// of kSelDistBytes.
hipError_t launch_select_dist(const SelectParamsDev& p, const float* importance, int M, int pos_base,
                              int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept, void* ws, unsigned epoch,
                              unsigned long long spin, int cus, hipStream_t stream) {
    const size_t lds = sizeof(SelectShared<kSelThreads>);
    hipError_t e = hipFuncSetAttribute((const void*)&select_dist_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int W = (M + 2047) / 2048;
    if (W > 64) W = 64;
    if (W > cus) W = cus;
    if (W < 2) W = 2;
    hipLaunchKernelGGL(select_dist_kernel, dim3(W), dim3(kSelThreads), lds, stream, p, importance, M, pos_base,
                       kept_idx, pos_ids, n_kept, (unsigned long long*)ws, epoch, spin);
    return hipGetLastError();
}

// Launches the selection of requests [0, R) whose prompt offsets are cu[0..R].
hipError_t launch_select(const SelectParamsDev& p, const int64_t* cu, const int32_t* pos_base,
                         int R, const float* importance, int32_t* kept_idx, int32_t* pos_ids,
                         int32_t* n_kept, hipStream_t stream) {
    const bool threshold = p.mode == SP_SELECT_THRESHOLD;
    const size_t lds = threshold ? sizeof(ThreshShared) : sizeof(SelectShared<kSelThreads>);
    const void* fn = threshold ? (const void*)&select_threshold_kernel : (const void*)&select_kernel;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    for (int r0 = 0; r0 < R; r0 += kSelBatch) {
        const int nr = R - r0 < kSelBatch ? R - r0 : kSelBatch;
        SelectBatch b;
        for (int i = 0; i <= nr; ++i) b.cu[i] = (int)cu[r0 + i];
        for (int i = 0; i < nr; ++i) b.pos_base[i] = pos_base ? pos_base[r0 + i] : 0;
        b.first = r0;
        if (threshold)
            hipLaunchKernelGGL(select_threshold_kernel, dim3(nr), dim3(kSelThreads), lds, stream, b,
                               p, importance, kept_idx, pos_ids, n_kept);
        else
            hipLaunchKernelGGL(select_kernel, dim3(nr), dim3(kSelThreads), lds, stream, b, p,
                               importance, kept_idx, pos_ids, n_kept);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sp
