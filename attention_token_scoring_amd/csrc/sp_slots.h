#pragma once
// Cross-workgroup slots of the kernels' exchanges: 8-byte words written and
// read at agent scope (every CU's view, across the XCDs' L2 caches), a 32-bit
// value in the low half and the epoch of the launch that wrote it in the
// high half, so a word left by an earlier launch is never taken for this
// one's and nothing is reset between launches.
#include <hip/hip_runtime.h>

namespace sp {

__device__ __forceinline__ unsigned long long ld64(const void* p) {
    return __hip_atomic_load((unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned ld32(const void* p) {
    return __hip_atomic_load((unsigned*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st64u(void* p, unsigned long long v) {
    __hip_atomic_store((unsigned long long*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A 32-bit value in the low half of a slot, the epoch of its launch in the high half.
__device__ __forceinline__ unsigned long long tagged(float v, unsigned epoch) {
    return (unsigned long long)__float_as_uint(v) | ((unsigned long long)epoch << 32);
}
__device__ __forceinline__ bool tag_is(unsigned long long v, unsigned epoch) {
    return (unsigned)(v >> 32) == epoch;
}
__device__ __forceinline__ float tag_value(unsigned long long v) { return __uint_as_float((unsigned)v); }

// A score range as published by a workgroup (min and max words): a range
// holding a non-finite score publishes this max.
constexpr unsigned kNonFiniteMark = 0xffffffffu;

}  // namespace sp
