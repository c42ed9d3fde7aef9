// Measurement aid, not part of the scoring computation: a plain streaming read
// of a device buffer, to measure the HBM read rate the device sustains with a
// given number of workgroups (the practical ceiling the scoring kernel, which
// reads each key once, is compared against).
#include "sp_internal.h"

namespace sp {

typedef int probe_i4 __attribute__((ext_vector_type(4)));

// 16-byte loads, U of them in flight per thread; workgroup b reads the
// 512 * U * 16-byte chunks b, b + grid, b + 2 grid, ... The loaded words are
// folded with XOR into one value that is stored only if it equals a constant
// no real data produces by chance in practice (so the loads are kept and
// nothing is written).
template <int U>
__global__ __launch_bounds__(512) void read_probe_kernel(const probe_i4* __restrict__ p,
                                                        long long n16, int* __restrict__ out) {
    constexpr long long kChunk = 512ll * U;
    probe_i4 acc = {0, 0, 0, 0};
    for (long long c = blockIdx.x; c * kChunk < n16; c += gridDim.x) {
        const long long base = c * kChunk + threadIdx.x;
        probe_i4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long i = base + 512ll * u;
            v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : probe_i4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x5a17c0de) out[0] = 1;
}

}  // namespace sp

extern "C" sp_status sp_read_probe(const void* buf, size_t bytes, int32_t grid, int32_t depth,
                                   int32_t* flag, void* stream) {
    if (!buf || !flag || grid < 1 || bytes < 16 || (bytes % 16) != 0 || ((uintptr_t)buf % 16) != 0)
        return SP_EINVAL;
    if (depth != 4 && depth != 8 && depth != 16) return SP_EUNSUPPORTED;
    const long long n16 = (long long)(bytes / 16);
    hipStream_t s = (hipStream_t)stream;
    if (depth == 4)
        hipLaunchKernelGGL(sp::read_probe_kernel<4>, dim3(grid), dim3(512), 0, s, (const sp::probe_i4*)buf, n16, flag);
    else if (depth == 8)
        hipLaunchKernelGGL(sp::read_probe_kernel<8>, dim3(grid), dim3(512), 0, s, (const sp::probe_i4*)buf, n16, flag);
    else
        hipLaunchKernelGGL(sp::read_probe_kernel<16>, dim3(grid), dim3(512), 0, s, (const sp::probe_i4*)buf, n16, flag);
    return hipGetLastError() == hipSuccess ? SP_OK : SP_EDEVICE;
}
