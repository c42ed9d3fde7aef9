// Sparse-prefill batch: the rows (token ids, or any fixed-size records) of the
// kept tokens, in kept order ("SpecPrefill - Implementation Guide", Full
// Source Code: the target's sparse batch takes the input token of each kept
// index, at its original position). The kept counts are read on the device,
// so no host synchronisation is needed between selection and gather.
#include "sp_internal.h"

namespace sp {

constexpr int kGatherThreads = 256;
constexpr int kGatherBatch = 128;  // requests per launch (offsets travel in the kernel arguments)

struct GatherBatch {
    long long cu[kGatherBatch];  // output (and kept-list) offset of each request
    int first;                   // index of the launch's first request (for n_kept)
};

// Request blockIdx.y: dst row cu[r] + o = src row kept[cu[r] + o], o < n_kept[r];
// rows of `words` 4-byte words. Threads stride over (row, word) pairs.
__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(
    GatherBatch b, const uint32_t* __restrict__ src, long long words, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ n_kept, uint32_t* __restrict__ dst) {
    const int r = blockIdx.y;
    const long long off = b.cu[r];
    const long long n = (long long)n_kept[b.first + r];
    const long long total = n * words;
    for (long long e = (long long)blockIdx.x * kGatherThreads + threadIdx.x; e < total;
         e += (long long)gridDim.x * kGatherThreads) {
        const long long o = e / words, wd = e - o * words;
        dst[(off + o) * words + wd] = src[(long long)kept[off + o] * words + wd];
    }
}

// Requests r < R with output offsets cu[r] (host) and at most max_rows kept rows each.
hipError_t launch_gather(const void* src, long long row_bytes, const int32_t* kept,
                         const int32_t* n_kept, int R, const int64_t* cu, long long max_rows,
                         void* dst, hipStream_t stream) {
    const long long words = row_bytes / 4;
    long long blocks = (max_rows * words + kGatherThreads - 1) / kGatherThreads;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    for (int r0 = 0; r0 < R; r0 += kGatherBatch) {
        const int nr = R - r0 < kGatherBatch ? R - r0 : kGatherBatch;
        GatherBatch b;
        for (int i = 0; i < nr; ++i) b.cu[i] = cu[r0 + i];
        b.first = r0;
        hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks, (unsigned)nr),
                           dim3(kGatherThreads), 0, stream, b, (const uint32_t*)src, words, kept,
                           n_kept, (uint32_t*)dst);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sp
