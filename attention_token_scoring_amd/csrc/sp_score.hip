// Scoring: the launch sequence (the method and the scoring kernel are
// described in sp_score_kernel.h).
#include <atomic>

#include "sp_score_kernel.h"

namespace sp {

// Under stream capture a launch's epoch is fixed into the graph, and every
// replay would reuse it: a small kernel captured before the scoring kernel
// clears the tagged words (counters, partial and log-sum-exp slots; the
// error word only before a call's first launch), so that each replay starts
// from slots that no epoch matches.
__global__ __launch_bounds__(256) void clear_tags_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
// The scoring kernel for a launch plan (sel: the fused launch that also selects).
static const void* pick_kernel(int dtype, int d, int rows, int G, int tpw, bool dma, bool sel) {
    if (dtype == SP_BF16) {
        if (d == 128)
            return sel ? score_select_kernel_bf16_d128(rows, G, tpw, dma) : score_kernel_bf16_d128(rows, G, tpw, dma);
        if (d == 64)
            return sel ? score_select_kernel_bf16_d64(rows, G, tpw, dma) : score_kernel_bf16_d64(rows, G, tpw, dma);
    } else {
        if (d == 128)
            return sel ? score_select_kernel_f32_d128(rows, G, tpw, dma) : score_kernel_f32_d128(rows, G, tpw, dma);
        if (d == 64)
            return sel ? score_select_kernel_f32_d64(rows, G, tpw, dma) : score_kernel_f32_d64(rows, G, tpw, dma);
    }
    return nullptr;
}

static thread_local hipEvent_t t_ev_before = nullptr, t_ev_after = nullptr;
static thread_local unsigned long long t_wait_limit = 0;

// The limit of a bounded wait, in ticks of the 100 MHz clock (the calling
// thread's test setting, else the default).
unsigned long long wait_limit_ticks() { return t_wait_limit > 0 ? t_wait_limit : kSpinTicks; }

void set_profile_events(hipEvent_t before, hipEvent_t after) {
    t_ev_before = before;
    t_ev_after = after;
}

void set_wait_limit(unsigned long long ticks) { t_wait_limit = ticks; }

// Epochs: a process-wide launch count passed through a bijective 32-bit
// integer mix (the "lowbias32" function of Wellons' hash-prospector), so that
// no two launches of the process share one, and leftover data in a workspace
// (small integers, a constant fill, earlier epochs) does not pass for the
// current one. 0 and ~0 are skipped.
static std::atomic<unsigned> g_launches{0};

unsigned next_epoch() {
    for (;;) {
        unsigned x = g_launches.fetch_add(1u, std::memory_order_relaxed) + 1u;
        x ^= x >> 16;
        x *= 0x7feb352du;
        x ^= x >> 15;
        x *= 0x846ca68bu;
        x ^= x >> 16;
        if (x != 0u && x != ~0u) return x;
    }
}

// One launch of the scoring kernel (which also writes the importance): an
// ordinary launch (every workgroup resident on an otherwise idle device) or,
// if the descriptor asks for it, a cooperative one. call_epoch tags the
// call's error word (shared by all its launches); first: the call's first
// launch.
hipError_t launch_score(const ScorePlan& p, const sp_score_desc& d, const void* Q, const void* K,
                        long long plane_stride, int M, int M_out, float* importance, void* ws,
                        unsigned call_epoch, bool first, int tail_n, int blend_n, const FusedSelect* fs,
                        hipStream_t stream) {
    char* base = (char*)ws;
    ScoreArgs a;
    a.Q = Q;
    a.K = K;
    a.plane_stride = plane_stride;
    a.err = (unsigned long long*)(base + p.ws_err);
    a.hdr = (unsigned*)(base + p.ws_err + 8);
    a.flags = (unsigned long long*)(base + p.ws_err + 128);
    a.importance = importance;
    a.M_out = M_out;
    a.part = (unsigned long long*)(base + p.ws_part);
    a.lse = (unsigned long long*)(base + p.ws_lse);
    a.Tg = (int*)(base + p.ws_tg);
    a.epoch = next_epoch();
    a.call_epoch = call_epoch;
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
    a.tail_n = tail_n;
    a.blend_n = blend_n;
    a.spin_ticks = wait_limit_ticks();
    a.done = (unsigned long long*)(base + p.ws_err + kDoneFlags);
    a.sel_sums = (unsigned long long*)(base + p.ws_sel);
    // The streaming workgroups sum the chunk masses (min-max normalisation)
    // for prompts of 16K tokens or more: below that the selecting workgroup
    // stages at most two tiles of scores itself, which measured faster than
    // the extra exchange (fused step at 4608 tokens 53.2 against 55.5 us;
    // at 32K 344.1 against 342.8, at 128K 1276 against 1254).
    a.sel_dist = fs && fs->p.norm == SP_NORM_MINMAX && M >= kSelDistMin ? 1 : 0;
    if (fs) {
        a.selp = fs->p;
        a.sel_pos_base = fs->pos_base;
        a.sel_kept = fs->kept;
        a.sel_pos = fs->pos;
        a.sel_n = fs->n_kept;
    }
    // (the fused selection reuses the combiner's LDS)
    size_t lds = p.lds.total;
    if (fs && lds < sizeof(SelectShared<kThreads>)) lds = sizeof(SelectShared<kThreads>);

    const void* fn = pick_kernel(d.dtype, d.d, p.rows, a.G, p.tpw, p.dma, fs != nullptr);
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;

    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
        const size_t lo = first ? 0 : 16;  // (keep the call's error word)
        const size_t n16 = (p.ws_tg - lo) / 16;
        hipLaunchKernelGGL(clear_tags_kernel, dim3((unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024)),
                           dim3(256), 0, stream, (uint4*)(base + lo), n16);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    void* args[] = {&a};
    if (t_ev_before) {
        e = hipEventRecord(t_ev_before, stream);
        if (e != hipSuccess) return e;
    }
    if (d.launch == SP_LAUNCH_COOPERATIVE) {
        e = hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(kThreads), args, (unsigned)lds, stream);
    } else {
        // every workgroup must fit on the device at once (one per unit here)
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds);
        if (e != hipSuccess) return e;
        if (per_cu < 1 || (long long)p.grid > (long long)per_cu * p.cus)
            return hipErrorCooperativeLaunchTooLarge;
        e = hipLaunchKernel(fn, dim3(p.grid), dim3(kThreads), args, (unsigned)lds, stream);
    }
    if (e != hipSuccess) return e;
    if (t_ev_after) {
        e = hipEventRecord(t_ev_after, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sp
