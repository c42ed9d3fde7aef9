// Scoring: the small kernel before the scoring kernel (prep: per-unit
// synchronisation state and the look-ahead keys' statistics) and the launch
// sequence. The method and the scoring kernel are described in
// sp_score_kernel.h.
#include "sp_score_kernel.h"

namespace sp {

// Before the scoring kernel: reset its synchronisation state (every
// partial and log-sum-exp slot to the sentinel, the error word), and compute
// for every unit and query row the share of the look-ahead keys M..M+N-1 in the
// row's softmax denominator (row j sees look-ahead key t iff t <= j), as a raw
// max and a sum of exp2((x - max) * c). One 256-thread block per unit: one
// thread per (row, look-ahead key) dot product, 16-byte loads.
template <bool BF16>
__device__ __forceinline__ float dot16(uint4 q, uint4 k, float acc) {
    if constexpr (BF16) {
        const unsigned qa[4] = {q.x, q.y, q.z, q.w}, ka[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(__uint_as_float(qa[i] << 16), __uint_as_float(ka[i] << 16), acc);
            acc = fmaf(__uint_as_float(qa[i] & 0xffff0000u), __uint_as_float(ka[i] & 0xffff0000u), acc);
        }
    } else {
        acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
        acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
        acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
        acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    }
    return acc;
}

template <bool BF16, int D>
__global__ __launch_bounds__(256) void score_prep_kernel(ScoreArgs a, int rows) {
    __shared__ float logit[32][33];  // [row][look-ahead key]
    const int u = blockIdx.x, tid = threadIdx.x;
    if (u == 0 && tid == 0 && a.reset_err) *a.err = 0;
    if (u == 0)
        for (int x = tid; x < a.g; x += 256) a.done[x] = 0u;
    // this unit's g * rows partial slots, two per 16-byte store
    uint4* slots = (uint4*)(a.part + (size_t)u * a.g * rows);
    for (int x = tid; x < a.g * rows / 2; x += 256) slots[x] = make_uint4(~0u, ~0u, ~0u, ~0u);
    if (tid < rows) ((unsigned*)a.lse)[(size_t)u * rows + tid] = kSentinel32;

    const int l = u / a.Hkv, kvh = u % a.Hkv;
    constexpr int esz = BF16 ? 2 : 4;
    const char* kp = (const char*)a.K + ((long long)u * a.plane_stride + (long long)a.M * a.d) * esz;
    constexpr int n16 = D * esz / 16;  // (all of a row's loads in flight at once)
    for (int x = tid; x < rows * a.N; x += 256) {
        const int row = x / a.N, t = x % a.N;
        const int j = row / a.G, hl = row % a.G;
        if (j < a.N && t <= j && t < a.tail_n) {
            const long long qrow = ((long long)l * a.H + (long long)kvh * a.G + hl) * a.N + j;
            const uint4* q = (const uint4*)((const char*)a.Q + qrow * D * esz);
            const uint4* k = (const uint4*)(kp + (long long)t * D * esz);
            uint4 qv[n16], kv[n16];
#pragma unroll
            for (int e = 0; e < n16; ++e) {
                qv[e] = q[e];
                kv[e] = k[e];
            }
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < n16; ++e) acc = dot16<BF16>(qv[e], kv[e], acc);
            logit[row][t] = acc;
        }
    }
    __syncthreads();
    if (tid < rows) {
        const int j = tid / a.G;
        float m = -INFINITY, s = 0.f;
        const int nt = min(j + 1, a.tail_n);  // look-ahead keys row j sees
        if (j < a.N) {
            for (int t = 0; t < nt; ++t) m = fmaxf(m, logit[tid][t]);
            for (int t = 0; t < nt; ++t) s += exp2_hw(fmaf(logit[tid][t], a.c, -m * a.c));
        }
        a.tail[(size_t)u * rows + tid] = make_float2(m, s);
    }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static const void* pick_kernel(int dtype, int d, int rows, int G, int tpw, bool dma) {
    if (dtype == SP_BF16) {
        if (d == 128) return score_kernel_bf16_d128(rows, G, tpw, dma);
        if (d == 64) return score_kernel_bf16_d64(rows, G, tpw, dma);
    } else {
        if (d == 128) return score_kernel_f32_d128(rows, G, tpw, dma);
        if (d == 64) return score_kernel_f32_d64(rows, G, tpw, dma);
    }
    return nullptr;
}

static thread_local hipEvent_t t_ev_before = nullptr, t_ev_after = nullptr;
static thread_local unsigned long long t_wait_limit = 0;

void set_profile_events(hipEvent_t before, hipEvent_t after) {
    t_ev_before = before;
    t_ev_after = after;
}

void set_wait_limit(unsigned long long ticks) { t_wait_limit = ticks; }

// One request: prep (reset synchronisation state, look-ahead statistics; the
// error word only for the first request of a call, so that it reports a time-out
// in any request of the call),
// then the scoring kernel, which also writes the importance: an ordinary
// launch (every workgroup resident on an otherwise idle device) or, if the
// descriptor asks for it, a cooperative one.
hipError_t launch_score(const ScorePlan& p, const sp_score_desc& d, const void* Q, const void* K,
                        long long plane_stride, int M, int M_out, float* importance, void* ws,
                        bool first, int tail_n, int blend_n, hipStream_t stream) {
    char* base = (char*)ws;
    ScoreArgs a;
    a.Q = Q;
    a.K = K;
    a.plane_stride = plane_stride;
    a.err = (int*)(base + p.ws_err);
    a.done = (unsigned*)(base + p.ws_err + 128);
    a.importance = importance;
    a.M_out = M_out;
    a.part = (float2*)(base + p.ws_part);
    a.tail = (float2*)(base + p.ws_tail);
    a.lse = (float*)(base + p.ws_lse);
    a.Tg = (int*)(base + p.ws_tg);
    a.L = d.L;
    a.H = d.H;
    a.Hkv = d.Hkv;
    a.G = d.H / d.Hkv;
    a.N = d.N;
    a.M = M;
    a.d = d.d;
    a.g = p.g;
    a.ngroups = p.ngroups;
    a.KR = p.KR;
    a.units = p.units;
    a.defer = p.defer;
    a.nbk = p.defer + 1;
    a.lds = p.lds;
    const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.d);
    a.c = scale * 1.4426950408889634f;
    a.reset_err = first ? 1 : 0;
    a.tail_n = tail_n;
    a.blend_n = blend_n;
    a.spin_ticks = t_wait_limit > 0 ? t_wait_limit : kSpinTicks;

    const void* fn = pick_kernel(d.dtype, d.d, p.rows, a.G, p.tpw, p.dma);
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds.total);
    if (e != hipSuccess) return e;

    if (d.dtype == SP_BF16) {
        if (d.d == 128)
            hipLaunchKernelGGL((score_prep_kernel<true, 128>), dim3(p.units), dim3(256), 0, stream, a, p.rows);
        else
            hipLaunchKernelGGL((score_prep_kernel<true, 64>), dim3(p.units), dim3(256), 0, stream, a, p.rows);
    } else {
        if (d.d == 128)
            hipLaunchKernelGGL((score_prep_kernel<false, 128>), dim3(p.units), dim3(256), 0, stream, a, p.rows);
        else
            hipLaunchKernelGGL((score_prep_kernel<false, 64>), dim3(p.units), dim3(256), 0, stream, a, p.rows);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* args[] = {&a};
    if (t_ev_before) {
        e = hipEventRecord(t_ev_before, stream);
        if (e != hipSuccess) return e;
    }
    if (d.launch == SP_LAUNCH_COOPERATIVE) {
        e = hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(kThreads), args, (unsigned)p.lds.total, stream);
    } else {
        // every workgroup must fit on the device at once (one per unit here)
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, p.lds.total);
        if (e != hipSuccess) return e;
        if (per_cu < 1 || (long long)p.grid > (long long)per_cu * p.cus)
            return hipErrorCooperativeLaunchTooLarge;
        e = hipLaunchKernel(fn, dim3(p.grid), dim3(kThreads), args, (unsigned)p.lds.total, stream);
    }
    if (e != hipSuccess) return e;
    if (t_ev_after) {
        e = hipEventRecord(t_ev_after, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sp
