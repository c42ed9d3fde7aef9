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
// The scoring kernel for a launch plan and launch mode (kLaunchPlain,
// kLaunchFused: also selects, kLaunchPack: several requests).
static const void* pick_kernel(int dtype, int d, int rows, int G, int tpw, bool dma, int mode) {
    using Pick = const void* (*)(int, int, int, bool);
    static const Pick table[2][2][3] = {
        {{score_kernel_f32_d64, score_select_kernel_f32_d64, score_pack_kernel_f32_d64},
         {score_kernel_f32_d128, score_select_kernel_f32_d128, score_pack_kernel_f32_d128}},
        {{score_kernel_bf16_d64, score_select_kernel_bf16_d64, score_pack_kernel_bf16_d64},
         {score_kernel_bf16_d128, score_select_kernel_bf16_d128, score_pack_kernel_bf16_d128}}};
    if ((d != 64 && d != 128) || mode < kLaunchPlain || mode > kLaunchPack) return nullptr;
    return table[dtype == SP_BF16 ? 1 : 0][d == 128 ? 1 : 0][mode](rows, G, tpw, dma);
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
// The kernel arguments of one request whose workspace region starts at base;
// call_ws: the region of the call's error word and last epoch.
static void fill_args(const ScorePlan& p, const sp_score_desc& d, const void* Q, const void* K,
                      long long plane_stride, int M, int M_out, float* importance, char* base, char* call_ws,
                      unsigned call_epoch, int tail_n, int blend_n, const FusedSelect* fs, ScoreArgs& a) {
    a.Q = Q;
    a.K = K;
    a.plane_stride = plane_stride;
    a.err = (unsigned long long*)(call_ws + p.ws_err);
    a.hdr = (unsigned*)(call_ws + p.ws_err + 8);
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
}

// Under capture: the clearing of one workspace region's tagged words.
static hipError_t clear_region(const ScorePlan& p, char* base, bool first, hipStream_t stream) {
    const size_t lo = first ? 0 : 16;  // (keep the call's error word)
    const size_t n16 = (p.ws_tg - lo) / 16;
    hipLaunchKernelGGL(clear_tags_kernel, dim3((unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024)),
                       dim3(256), 0, stream, (uint4*)(base + lo), n16);
    return hipGetLastError();
}

// The launch itself (grid workgroups of kThreads threads, lds bytes of
// dynamic LDS), bracketed by the profiling events when they are set.
static hipError_t launch_grid(const sp_score_desc& d, const void* fn, void** args, int grid, int cus, size_t lds,
                              hipStream_t stream) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (t_ev_before) {
        e = hipEventRecord(t_ev_before, stream);
        if (e != hipSuccess) return e;
    }
    if (d.launch == SP_LAUNCH_COOPERATIVE) {
        e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, (unsigned)lds, stream);
    } else {
        // every workgroup must fit on the device at once (one per unit here)
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds);
        if (e != hipSuccess) return e;
        if (per_cu < 1 || (long long)grid > (long long)per_cu * cus) return hipErrorCooperativeLaunchTooLarge;
        e = hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, (unsigned)lds, stream);
    }
    if (e != hipSuccess) return e;
    if (t_ev_after) {
        e = hipEventRecord(t_ev_after, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_score(const ScorePlan& p, const sp_score_desc& d, const void* Q, const void* K,
                        long long plane_stride, int M, int M_out, float* importance, void* ws,
                        unsigned call_epoch, bool first, int tail_n, int blend_n, const FusedSelect* fs,
                        hipStream_t stream) {
    char* base = (char*)ws;
    ScoreArgs a;
    fill_args(p, d, Q, K, plane_stride, M, M_out, importance, base, base, call_epoch, tail_n, blend_n, fs, a);
    // (the fused selection reuses the combiner's LDS)
    size_t lds = p.lds.total;
    if (fs && lds < sizeof(SelectShared<kThreads>)) lds = sizeof(SelectShared<kThreads>);

    const void* fn = pick_kernel(d.dtype, d.d, p.rows, a.G, p.tpw, p.dma, fs ? kLaunchFused : kLaunchPlain);
    if (!fn) return hipErrorInvalidValue;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
        e = clear_region(p, base, first, stream);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&a};
    return launch_grid(d, fn, args, p.grid, p.cus, lds, stream);
}

// n requests in one launch: request r with plan pk[r].plan on its own share of
// the device's CUs and its own workspace region at pk[r].ws (all plans have
// the same tiles per wave and K path); the call's error word is in pk[0]'s
// region.
hipError_t launch_score_pack(const PackRequest* pk, int n, const sp_score_desc& d, long long plane_stride,
                             unsigned call_epoch, bool first, hipStream_t stream) {
    if (n < 1 || n > kMaxPack) return hipErrorInvalidValue;
    PackArgs m;
    m.n = n;
    m.first[0] = 0;
    size_t lds = 0;
    int cus = 0;
    for (int r = 0; r < n; ++r) {
        const ScorePlan& p = pk[r].plan;
        if (p.tpw != pk[0].plan.tpw || p.dma != pk[0].plan.dma || p.rows != pk[0].plan.rows)
            return hipErrorInvalidValue;
        fill_args(p, d, pk[r].Q, pk[r].K, plane_stride, pk[r].M, pk[r].M_out, pk[r].importance, (char*)pk[r].ws,
                  (char*)pk[0].ws, call_epoch, d.N, 0, nullptr, m.args[r]);
        m.first[r + 1] = m.first[r] + p.grid;
        if (p.lds.total > lds) lds = p.lds.total;
        cus += p.cus;
    }
    for (int r = n; r < kMaxPack; ++r) m.first[r + 1] = m.first[n];
    const ScorePlan& p0 = pk[0].plan;
    const void* fn = pick_kernel(d.dtype, d.d, p0.rows, d.H / d.Hkv, p0.tpw, p0.dma, kLaunchPack);
    if (!fn) return hipErrorInvalidValue;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
        for (int r = 0; r < n; ++r) {
            e = clear_region(pk[r].plan, (char*)pk[r].ws, first && r == 0, stream);
            if (e != hipSuccess) return e;
        }
    }
    void* args[] = {&m};
    return launch_grid(d, fn, args, m.first[n], cus, lds, stream);
}

}  // namespace sp
