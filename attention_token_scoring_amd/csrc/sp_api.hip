// C ABI of libspecprefill: argument validation, launch planning, dispatch.
// Every argument error is reported before anything is enqueued.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "sp_internal.h"

// Workspace of sp_score_noalloc: one copy per device, held until the process
// ends. In host code this name only stands for the array; kernels get the
// device address that hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) unsigned char scratch[SP_NOALLOC_SCRATCH_BYTES];

namespace sp {

hipError_t launch_score(const ScorePlan& p, const sp_score_desc& d, const void* Q, const void* K,
                        long long plane_stride, int M, int M_out, float* importance, void* ws,
                        unsigned call_epoch, bool first, int tail_n, int blend_n, const FusedSelect* fs,
                        hipStream_t stream);
hipError_t launch_score_pack(const PackRequest* pk, int n, const sp_score_desc& d, long long plane_stride,
                             unsigned call_epoch, bool first, hipStream_t stream);
unsigned next_epoch();
hipError_t launch_gather(const void* src, long long row_bytes, const int32_t* kept,
                         const int32_t* n_kept, int R, const int64_t* cu, long long max_rows,
                         void* dst, hipStream_t stream);
hipError_t launch_select(const SelectParamsDev& p, const int64_t* cu, const int32_t* pos_base,
                         int R, const float* importance, int32_t* kept_idx, int32_t* pos_ids,
                         int32_t* n_kept, hipStream_t stream);
hipError_t launch_select_dist(const SelectParamsDev& p, const float* importance, int M, int pos_base,
                              int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept, void* ws, unsigned epoch,
                              unsigned long long spin, int cus, hipStream_t stream);
unsigned long long wait_limit_ticks();

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxSelectChunks = 5120;   // top-K and mass modes
constexpr int kMaxThresholdChunks = 4096;
constexpr int kMaxSelectRequests = 1024;

int g_cus[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Device address of each device's copy of the scratch array of
// sp_score_noalloc (looked up once per device, that device current).
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Compute units of the current device (0 if there is no usable device).
int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(g_once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 0;
        g_cus[dev] = n;
    });
    return g_cus[dev];
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int esize(sp_dtype t) { return t == SP_BF16 ? 2 : 4; }

// Shape checks shared by every scoring entry point.
sp_status check_desc(const sp_score_desc* d) {
    if (!d) return SP_EINVAL;
    if (d->L < 1 || d->H < 1 || d->Hkv < 1 || d->d < 1 || d->N < 1) return SP_EINVAL;
    if (d->H % d->Hkv != 0) return SP_EINVAL;
    if (d->dtype != SP_F32 && d->dtype != SP_BF16) return SP_EINVAL;
    if (!(d->scale >= 0.f) || !isfinite(d->scale)) return SP_EINVAL;
    if (d->launch != SP_LAUNCH_RESIDENT && d->launch != SP_LAUNCH_COOPERATIVE) return SP_EINVAL;
    const int G = d->H / d->Hkv;
    if (d->d != 64 && d->d != 128) return SP_EUNSUPPORTED;
    if ((G & (G - 1)) != 0 || G * d->N > 32) return SP_EUNSUPPORTED;
    if ((long long)d->L * d->Hkv > (1 << 20)) return SP_EUNSUPPORTED;
    return SP_OK;
}

sp_status to_status(hipError_t e) { return e == hipSuccess ? SP_OK : SP_EDEVICE; }

sp_status check_select_params(const sp_select_params* p) {
    if (!p) return SP_EINVAL;
    if (p->chunk < 1 || p->pool_k < 1 || (p->pool_k % 2) == 0) return SP_EINVAL;
    if (p->mode == SP_SELECT_TOPK) {
        if (!(p->keep_rate > 0.f && p->keep_rate <= 1.f)) return SP_EINVAL;
    } else if (p->mode == SP_SELECT_MASS) {
        if (!(p->mass > 0.f && p->mass <= 1.f)) return SP_EINVAL;
    } else if (p->mode == SP_SELECT_THRESHOLD) {
        // raw scores: no pooling, no boosts
        if (!(p->keep_rate > 0.f && p->keep_rate <= 1.f)) return SP_EINVAL;
        if (p->pool_k != 1 || p->boost_first_n != 0 || p->boost_last_n != 0) return SP_EINVAL;
        if (p->min_tok < 0 || p->max_keep < 0) return SP_EINVAL;
    } else {
        return SP_EINVAL;
    }
    if (p->mode != SP_SELECT_THRESHOLD && (p->min_tok != 0 || p->max_keep != 0)) return SP_EINVAL;
    if (p->norm == SP_NORM_MINMAX) {
        if (p->norm_lo != 0.f || p->norm_hi != 0.f) return SP_EINVAL;
    } else if (p->norm == SP_NORM_PERCENTILE) {
        if (!(p->norm_lo >= 0.f && p->norm_lo < p->norm_hi && p->norm_hi <= 1.f)) return SP_EINVAL;
    } else if (p->norm == SP_NORM_ZSCORE) {
        if (p->norm_lo != 0.f || !(p->norm_hi > 0.f) || !isfinite(p->norm_hi)) return SP_EINVAL;
    } else {
        return SP_EINVAL;
    }
    if (p->mode == SP_SELECT_THRESHOLD && p->norm != SP_NORM_MINMAX) return SP_EINVAL;
    if (p->boost_first_n < 0 || p->boost_last_n < 0) return SP_EINVAL;
    if (!(p->boost_first_mult >= 0.f) || !(p->boost_last_mult >= 0.f) ||
        !isfinite(p->boost_first_mult) || !isfinite(p->boost_last_mult))
        return SP_EINVAL;
    return SP_OK;
}

// Per-prompt limits of the selection kernel (see the header).
sp_status check_select_prompt(const sp_select_params* p, long long M) {
    if (M < 1) return SP_EINVAL;
    if (M > (1ll << 24)) return SP_EUNSUPPORTED;
    const long long nc = (M + p->chunk - 1) / p->chunk;
    if (nc > kMaxSelectChunks) return SP_EUNSUPPORTED;
    if (p->mode == SP_SELECT_THRESHOLD) return nc > kMaxThresholdChunks ? SP_EUNSUPPORTED : SP_OK;
    double vmax = 1.0;
    const double a = p->boost_first_mult, b = p->boost_last_mult;
    if (a > vmax) vmax = a;
    if (b > vmax) vmax = b;
    if (a * b > vmax) vmax = a * b;
    const double win = (double)p->pool_k * (double)p->chunk;
    if (vmax * 4294967296.0 * 1.0000001 * win >= 9007199254740992.0) return SP_EUNSUPPORTED;
    if (vmax * 4294967296.0 * 1.0000001 * (double)M >= 1.8e19) return SP_EUNSUPPORTED;
    return SP_OK;
}

SelectParamsDev to_dev(const sp_select_params* p) {
    SelectParamsDev q;
    q.chunk = p->chunk;
    q.pool_k = p->pool_k;
    q.mode = p->mode;
    q.keep_rate = p->keep_rate;
    q.mass = p->mass;
    q.first_n = p->boost_first_n;
    q.first_mult = p->boost_first_mult;
    q.last_n = p->boost_last_n;
    q.last_mult = p->boost_last_mult;
    q.min_tok = p->min_tok;
    q.max_keep = p->max_keep;
    q.norm = p->norm;
    q.norm_lo = p->norm_lo;
    q.norm_hi = p->norm_hi;
    return q;
}

size_t round_up256(size_t x) { return (x + 255) / 256 * 256; }

// The per-launch time the planner's estimates leave out (launch, pipeline
// start, the end of the exchange; measured ~15-20 us on the MI355X), and the
// streaming workgroups at which the kernel reaches the full read rate (the
// planner's bandwidth model).
constexpr double kLaunchFixedS = 15e-6;
constexpr double kFullRateWgs = 200.0;
// Which requests share a launch (measured on the MI355X at the 8B shape).
// Packs of prompts of similar length gained 3-75 % (16 x 4K tokens 1.03 ->
// 0.75 ms, 4 x 1000 0.170 -> 0.096 ms, 4 of 15K-53K 1.34 -> 1.30 ms), and
// packs of up to 8 more than packs of up to 4 (32 x 1000 0.80 -> 0.50 ms,
// 16 x 2048 0.46 -> 0.42 ms, the ragged 16 prompts of 5K-61K 4.93 -> 4.86 ms;
// 16 x 4096 0.77 -> 0.78 ms); packs
// that mixed lengths 5 to 50 times apart lost 5-20 % against estimates of
// small gains (the smallest requests' few CUs, with one combining workgroup
// for every unit, fall behind the plans' estimates), so the longest prompt
// of a pack is at most kPackSpread times its shortest. The estimates also
// favoured the smaller tile count where the larger measured faster: packs
// are planned with the larger where the configuration has one. A pack must
// be estimated at least kPackMargin faster than its requests in turn.
constexpr long long kPackSpread = 4;
constexpr double kPackMargin = 0.01;
constexpr int kPackPasses = 4;

// One launch for requests [r0, r0 + n), each on its own share of the CUs and
// planned for that share with tpw tiles per wave (a launch runs one kernel
// configuration). The shares start proportional to the requests' keys; each
// further pass sets them in proportion to the last plans' estimated CU-time
// (estimate x share), which evens out their estimates. Returns the best
// pass's estimated time of the launch (plans and workspace offsets in pk), or
// a negative number where no pass has plans that fit ws_bytes.
double plan_one_pack(const sp_score_desc& d, const long long* Ms, int r0, int n, int cus, int tpw,
                     size_t ws_bytes, PackRequest* pk) {
    double w[kMaxPack], W = 0.0, best = -1.0;
    for (int i = 0; i < n; ++i) {
        w[i] = (double)(Ms[r0 + i] + d.N);
        W += w[i];
    }
    int last[kMaxPack] = {};
    PackRequest cand[kMaxPack];
    for (int pass = 0; pass < kPackPasses; ++pass) {
        // shares: at least 2 CUs (a streaming and a combining workgroup)
        int c[kMaxPack], used = 0;
        for (int i = 0; i < n; ++i) {
            c[i] = (int)(cus * w[i] / W);
            if (c[i] < 2) c[i] = 2;
            used += c[i];
        }
        while (used > cus) {  // (the floors of 2 overshot: take from the largest)
            int j = 0;
            for (int i = 1; i < n; ++i) j = c[i] > c[j] ? i : j;
            if (c[j] <= 2) return best;
            --c[j];
            --used;
        }
        for (; used < cus; ++used) {  // the rest to the largest weight per CU
            int j = 0;
            for (int i = 1; i < n; ++i) j = w[i] / c[i] > w[j] / c[j] ? i : j;
            ++c[j];
        }
        bool same = true;
        for (int i = 0; i < n; ++i) {
            same = same && c[i] == last[i];
            last[i] = c[i];
        }
        if (same) break;  // (the shares have settled)
        int S = 0;
        double worst = 0.0;
        size_t off = 0;
        for (int i = 0; i < n; ++i) {
            ScorePlan& p = cand[i].plan;
            if (make_plan(d, Ms[r0 + i], c[i], &p, tpw) != SP_OK || p.dma != cand[0].plan.dma)
                return best;
            S += p.g * p.ngroups;
            worst = p.cost > worst ? p.cost : worst;
            cand[i].ws = (void*)off;  // (an offset until the launch)
            off += round_up256(p.ws_total);
        }
        if (off > ws_bytes) return best;
        // (the plans model a request's bandwidth as its share of the full
        // rate: the device's total caps it)
        const double t = worst * (S > kFullRateWgs ? S / kFullRateWgs : 1.0) + kLaunchFixedS;
        if (best < 0.0 || t < best) {
            best = t;
            for (int i = 0; i < n; ++i) pk[i] = cand[i];
        }
        W = 0.0;
        for (int i = 0; i < n; ++i) {
            w[i] = cand[i].plan.cost * cand[i].plan.cus;
            W += w[i];
        }
    }
    return best;
}

// Packing from request r0 on of R requests of prompt lengths Ms: the n (1 ..
// kMaxPack) whose one launch (plan_one_pack) is estimated fastest per request
// against scoring them one after the other, with the plans and workspace
// offsets in pk (n = 1: no packing). full: each request's plan for the whole
// device.
int plan_pack(const sp_score_desc& d, const long long* Ms, int r0, int R, int cus, size_t ws_bytes,
              const ScorePlan* full, PackRequest* pk) {
    int best_n = 1;
    double best_gain = 0.0;
    PackRequest cand[kMaxPack];
    const int tpw0 = tiles_per_wave(d.dtype == SP_BF16, d.d);
    long long lo = Ms[r0], hi = lo;
    for (int n = 2; n <= kMaxPack && r0 + n <= R; ++n) {
        const long long M = Ms[r0 + n - 1];
        lo = M < lo ? M : lo;
        hi = M > hi ? M : hi;
        if (hi > kPackSpread * lo) break;
        double seq = 0.0;
        for (int i = 0; i < n; ++i) seq += full[r0 + i].cost + kLaunchFixedS;
        double t = plan_one_pack(d, Ms, r0, n, cus, tpw0 + 1, ws_bytes, cand);
        if (t < 0.0) t = plan_one_pack(d, Ms, r0, n, cus, tpw0, ws_bytes, cand);
        if (t < 0.0 || seq - t <= kPackMargin * seq) continue;
        if ((seq - t) / n > best_gain) {
            best_gain = (seq - t) / n;
            best_n = n;
            for (int i = 0; i < n; ++i) pk[i] = cand[i];
        }
    }
    return best_n;
}

// The launches of a ragged batch: the requests in order of prompt length
// (shortest first; launches are independent, and packs want lengths alike),
// consecutive ones packed where plan_pack finds it pays. A launch of n = 1
// scores request req[0] alone with its plan for the whole device.
struct BatchLaunch {
    int n;
    int req[kMaxPack];
    PackRequest pk[kMaxPack];  // (n > 1; ws holds the region's offset)
};

// A batch's launches, planned one at a time (so that a caller can enqueue each
// as soon as it is planned): init validates every request's plan for the
// whole device (full, by request) and orders the requests by length; next
// plans the launch from the next unscheduled request on.
struct BatchSchedule {
    const sp_score_desc* d = nullptr;
    int R = 0, cus = 0, done = 0;
    size_t ws_bytes = 0;
    std::vector<ScorePlan> full;
    std::vector<int> order;
    std::vector<long long> Ms;      // prompt lengths in order
    std::vector<ScorePlan> fs;      // full plans in order

    sp_status init(const sp_score_desc& desc, int nreq, const int64_t* cu, int ncus, size_t wsb) {
        d = &desc;
        R = nreq;
        cus = ncus;
        ws_bytes = wsb;
        done = 0;
        full.resize((size_t)R);
        for (int r = 0; r < R; ++r) {
            const sp_status s = make_plan(desc, cu[r + 1] - cu[r], cus, &full[r]);
            if (s != SP_OK) return s;
            if (ws_bytes < full[r].ws_total) return SP_EWORKSPACE;
        }
        order.resize((size_t)R);
        for (int r = 0; r < R; ++r) order[r] = r;
        std::stable_sort(order.begin(), order.end(),
                         [&](int a, int b) { return cu[a + 1] - cu[a] < cu[b + 1] - cu[b]; });
        Ms.resize((size_t)R);
        fs.resize((size_t)R);
        for (int i = 0; i < R; ++i) {
            Ms[i] = cu[order[i] + 1] - cu[order[i]];
            fs[i] = full[order[i]];
        }
        return SP_OK;
    }
    bool next(BatchLaunch& b) {
        if (done >= R) return false;
        b.n = plan_pack(*d, Ms.data(), done, R, cus, ws_bytes, fs.data(), b.pk);
        for (int j = 0; j < b.n; ++j) b.req[j] = order[done + j];
        done += b.n;
        return true;
    }
};

// Requests r in [0, R) of a ragged batch, scored in the launches BatchSchedule
// plans (alone, or several in one launch on shares of the device where the
// workspace holds their regions side by side); with keep, only the first
// keep[r] scores of request r are written, packed one request after the
// other in request order (else all M_r scores at offset cu[r]).
sp_status score_batch(const sp_score_desc* desc, int32_t R, const void* Q, const void* K,
                      const int64_t* cu, const int64_t* keep, float* importance, void* ws,
                      size_t ws_bytes, void* stream) {
    sp_status s = check_desc(desc);
    if (s != SP_OK) return s;
    if (R < 1 || !Q || !K || !cu || !importance) return SP_EINVAL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(importance, 4)) return SP_EINVAL;
    if (cu[0] != 0) return SP_EINVAL;
    for (int r = 0; r < R; ++r) {
        if (cu[r + 1] - cu[r] < 1) return SP_EINVAL;
        if (keep && (keep[r] < 1 || keep[r] > cu[r + 1] - cu[r])) return SP_EINVAL;
    }
    if (cu[R] + (long long)R * desc->N > (1ll << 40)) return SP_EUNSUPPORTED;
    const int cus = device_cus();
    if (cus < 1) return SP_EDEVICE;
    if (!ws || !aligned(ws, 256)) return SP_EWORKSPACE;
    // validate every request's plan before enqueueing anything (the packs are
    // planned launch by launch below: a pack that does not pay or fit falls
    // back to the request alone, so their planning fails nothing)
    BatchSchedule sched;
    s = sched.init(*desc, R, cu, cus, ws_bytes);
    if (s != SP_OK) return s;
    const int es = esize(desc->dtype);
    const long long T = cu[R] + (long long)R * desc->N;
    const long long qsz = (long long)desc->L * desc->H * desc->N * desc->d * es;
    std::vector<long long> out((size_t)R);  // where request r's scores go
    long long o = 0;
    for (int r = 0; r < R; ++r) {
        out[r] = keep ? o : cu[r];
        o += keep ? keep[r] : 0;
    }
    const unsigned call = next_epoch();
    bool first = true;
    BatchLaunch b;
    while (sched.next(b)) {
        for (int i = 0; i < b.n; ++i) {
            const int r = b.req[i];
            const long long M = cu[r + 1] - cu[r];
            PackRequest& q = b.pk[i];
            q.Q = (const char*)Q + r * qsz;
            q.K = (const char*)K + (cu[r] + (long long)r * desc->N) * desc->d * es;
            q.M = (int)M;
            q.M_out = (int)(keep ? keep[r] : M);
            q.importance = importance + out[r];
            if (b.n > 1) q.ws = (char*)ws + (size_t)q.ws;
        }
        if (b.n == 1) {
            const PackRequest& q = b.pk[0];
            s = to_status(launch_score(sched.full[b.req[0]], *desc, q.Q, q.K, T * desc->d, q.M, q.M_out,
                                       q.importance, ws, call, first, desc->N, 0, nullptr, (hipStream_t)stream));
        } else {
            s = to_status(launch_score_pack(b.pk, b.n, *desc, T * desc->d, call, first, (hipStream_t)stream));
        }
        if (s != SP_OK) return s;
        first = false;
    }
    return SP_OK;
}

// The workspace with which score_batch packs as its plans allow (at least
// what every request needs alone).
size_t batch_workspace(const sp_score_desc& d, int R, const int64_t* cu, int cus) {
    BatchSchedule sched;
    if (sched.init(d, R, cu, cus, (size_t)-1) != SP_OK) return 0;
    size_t need = 0;
    for (const ScorePlan& p : sched.full) need = p.ws_total > need ? p.ws_total : need;
    BatchLaunch b;
    while (sched.next(b)) {
        if (b.n == 1) continue;
        const size_t end = (size_t)b.pk[b.n - 1].ws + round_up256(b.pk[b.n - 1].plan.ws_total);
        need = end > need ? end : need;
    }
    return need;
}

}  // namespace
}  // namespace sp

using namespace sp;

extern "C" {

const char* sp_status_string(sp_status s) {
    switch (s) {
        case SP_OK: return "SP_OK";
        case SP_EINVAL: return "SP_EINVAL: invalid argument";
        case SP_EUNSUPPORTED: return "SP_EUNSUPPORTED: shape or parameter outside what the kernels implement";
        case SP_EWORKSPACE: return "SP_EWORKSPACE: workspace missing or too small";
        case SP_EDEVICE: return "SP_EDEVICE: kernel launch failed";
    }
    return "unknown sp_status";
}

size_t sp_score_workspace_bytes(const sp_score_desc* desc, int64_t max_prompt_len) {
    if (check_desc(desc) != SP_OK || max_prompt_len < 1) return 0;
    // (plans get harder as prompts grow: if the longest has none, 0). The
    // bound also covers the one-step plans of sp_score_lastrow's second pass.
    ScorePlan p;
    if (make_plan(*desc, max_prompt_len, device_cus(), &p) != SP_OK) return 0;
    sp_score_desc d1 = *desc;
    d1.N = 1;
    const size_t a = workspace_bound(*desc, max_prompt_len, device_cus());
    const size_t b = workspace_bound(d1, max_prompt_len, device_cus());
    return a > b ? a : b;
}

size_t sp_score_batch_workspace_bytes(const sp_score_desc* desc, int32_t R, const int64_t* cu) {
    if (check_desc(desc) != SP_OK || R < 1 || !cu || cu[0] != 0) return 0;
    long long maxM = 0;
    for (int r = 0; r < R; ++r) {
        const long long M = cu[r + 1] - cu[r];
        if (M < 1) return 0;
        maxM = M > maxM ? M : maxM;
    }
    const size_t one = sp_score_workspace_bytes(desc, maxM);
    if (one == 0) return 0;
    const size_t packed = batch_workspace(*desc, R, cu, device_cus() > 0 ? device_cus() : kDefaultCUs);
    if (packed == 0) return 0;
    return packed > one ? packed : one;
}

sp_status sp_score_batch_plan(const sp_score_desc* desc, int32_t R, const int64_t* cu, size_t ws_bytes,
                              int32_t* launch_of, int32_t* n_launches) {
    sp_status s = check_desc(desc);
    if (s != SP_OK) return s;
    if (R < 1 || !cu || cu[0] != 0 || !n_launches) return SP_EINVAL;
    for (int r = 0; r < R; ++r)
        if (cu[r + 1] - cu[r] < 1) return SP_EINVAL;
    const int cus = device_cus() > 0 ? device_cus() : kDefaultCUs;
    BatchSchedule sched;
    s = sched.init(*desc, R, cu, cus, ws_bytes);
    if (s != SP_OK) return s;
    int32_t l = 0;
    BatchLaunch b;
    for (; sched.next(b); ++l)
        for (int i = 0; i < b.n; ++i)
            if (launch_of) launch_of[b.req[i]] = l;
    *n_launches = l;
    return SP_OK;
}

sp_status sp_profile_score_kernel(void* before, void* after) {
    if ((before == nullptr) != (after == nullptr)) return SP_EINVAL;
    sp::set_profile_events((hipEvent_t)before, (hipEvent_t)after);
    return SP_OK;
}

sp_status sp_set_wait_limit(uint64_t ticks) {
    sp::set_wait_limit((unsigned long long)ticks);
    return SP_OK;
}

sp_status sp_score_status(const void* ws, void* stream, int32_t* timed_out) {
    if (!ws || !timed_out) return SP_EINVAL;
    // The workspace starts with the error word ((call epoch << 32) | 1 once a
    // wait timed out) and, at byte 8, the epoch of the last call.
    unsigned long long v[2] = {0ull, 0ull};
    if (hipMemcpyAsync(v, ws, sizeof(v), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
        return SP_EDEVICE;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SP_EDEVICE;
    *timed_out = (v[0] & 1ull) != 0ull && (unsigned)(v[0] >> 32) == (unsigned)v[1] ? 1 : 0;
    return SP_OK;
}

sp_status sp_score_plan(const sp_score_desc* desc, int32_t M, int32_t info[9]) {
    sp_status s = check_desc(desc);
    if (s != SP_OK) return s;
    if (!info) return SP_EINVAL;
    const int cus = device_cus();
    ScorePlan p;
    s = make_plan(*desc, M, cus, &p);
    if (s != SP_OK) return s;
    info[0] = p.grid;
    info[1] = p.g;
    info[2] = p.ngroups;
    info[3] = p.KR;
    info[4] = p.rows;
    info[5] = p.units;
    info[6] = cus > 0 ? cus : kDefaultCUs;
    info[7] = p.defer;
    info[8] = p.dma ? 1 : 0;
    return SP_OK;
}

sp_status sp_score(const sp_score_desc* desc, const void* Q, const void* K, int32_t M,
                   float* importance, void* ws, size_t ws_bytes, void* stream) {
    sp_status s = check_desc(desc);
    if (s != SP_OK) return s;
    if (!Q || !K || !importance || M < 1) return SP_EINVAL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(importance, 4)) return SP_EINVAL;
    const int cus = device_cus();
    if (cus < 1) return SP_EDEVICE;
    ScorePlan p;
    s = make_plan(*desc, M, cus, &p);
    if (s != SP_OK) return s;
    if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total) return SP_EWORKSPACE;
    const long long plane = (long long)(M + desc->N) * desc->d;
    return to_status(launch_score(p, *desc, Q, K, plane, M, M, importance, ws, next_epoch(), true,
                                  desc->N, 0, nullptr, (hipStream_t)stream));
}

sp_status sp_score_select(const sp_score_desc* desc, const void* Q, const void* K, int32_t M,
                          const sp_select_params* params, int32_t pos_base, float* importance,
                          int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept, void* ws,
                          size_t ws_bytes, void* stream) {
    sp_status s = check_desc(desc);
    if (s != SP_OK) return s;
    s = check_select_params(params);
    if (s != SP_OK) return s;
    if (params->mode == SP_SELECT_THRESHOLD) return SP_EUNSUPPORTED;
    if (!Q || !K || !importance || !kept_idx || !pos_ids || !n_kept || M < 1) return SP_EINVAL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(importance, 4)) return SP_EINVAL;
    s = check_select_prompt(params, M);
    if (s != SP_OK) return s;
    if ((long long)pos_base + M > 2147483647ll || (long long)pos_base < -2147483647ll) return SP_EINVAL;
    const int cus = device_cus();
    if (cus < 1) return SP_EDEVICE;
    ScorePlan p;
    s = make_plan(*desc, M, cus, &p);
    if (s != SP_OK) return s;
    if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total) return SP_EWORKSPACE;
    const FusedSelect fs{to_dev(params), pos_base, kept_idx, pos_ids, n_kept};
    const long long plane = (long long)(M + desc->N) * desc->d;
    return to_status(launch_score(p, *desc, Q, K, plane, M, M, importance, ws, next_epoch(), true,
                                  desc->N, 0, &fs, (hipStream_t)stream));
}

sp_status sp_score_noalloc(const sp_score_desc* desc, const void* Q, const void* K, int32_t M,
                           float* importance, void* stream) {
    sp_status s = check_desc(desc);
    if (s != SP_OK) return s;
    if (!Q || !K || !importance || M < 1) return SP_EINVAL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(importance, 4)) return SP_EINVAL;
    const int cus = device_cus();
    if (cus < 1) return SP_EDEVICE;
    ScorePlan p;
    s = make_plan(*desc, M, cus, &p);
    if (s != SP_OK) return s;
    if (p.ws_total > SP_NOALLOC_SCRATCH_BYTES) return SP_EWORKSPACE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SP_EDEVICE;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = ptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return SP_EDEVICE;
    const long long plane = (long long)(M + desc->N) * desc->d;
    return to_status(launch_score(p, *desc, Q, K, plane, M, M, importance, g_scratch_ptr[dev],
                                  next_epoch(), true, desc->N, 0, nullptr, (hipStream_t)stream));
}

sp_status sp_score_lastrow(const sp_score_desc* desc, const void* Q, const void* Q_last,
                           const void* K, int32_t M, float* importance, void* ws,
                           size_t ws_bytes, void* stream) {
    sp_status s = check_desc(desc);
    if (s != SP_OK) return s;
    if (!Q || !Q_last || !K || !importance || M < 1) return SP_EINVAL;
    if (!aligned(Q, 16) || !aligned(Q_last, 16) || !aligned(K, 16) || !aligned(importance, 4))
        return SP_EINVAL;
    const int cus = device_cus();
    if (cus < 1) return SP_EDEVICE;
    // pass 1: the N look-ahead rows; pass 2: the last prompt token's row (one
    // step, keys 0..M-1, no look-ahead keys), blended in as step N + 1
    sp_score_desc d1 = *desc;
    d1.N = 1;
    ScorePlan p, p1;
    s = make_plan(*desc, M, cus, &p);
    if (s != SP_OK) return s;
    s = make_plan(d1, M, cus, &p1);
    if (s != SP_OK) return s;
    if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total || ws_bytes < p1.ws_total)
        return SP_EWORKSPACE;
    const long long plane = (long long)(M + desc->N) * desc->d;
    const unsigned call = next_epoch();
    s = to_status(launch_score(p, *desc, Q, K, plane, M, M, importance, ws, call, true, desc->N, 0,
                               nullptr, (hipStream_t)stream));
    if (s != SP_OK) return s;
    return to_status(launch_score(p1, d1, Q_last, K, plane, M, M, importance, ws, call, false, 0,
                                  desc->N, nullptr, (hipStream_t)stream));
}

sp_status sp_score_varlen(const sp_score_desc* desc, int32_t R, const void* Q, const void* K,
                          const int64_t* cu, float* importance, void* ws, size_t ws_bytes,
                          void* stream) {
    return score_batch(desc, R, Q, K, cu, nullptr, importance, ws, ws_bytes, stream);
}

sp_status sp_score_windows(const sp_score_desc* desc, int32_t R, const void* Q, const void* K,
                           const int64_t* cu_window_host, const int64_t* keep_host,
                           float* importance, void* ws, size_t ws_bytes, void* stream) {
    if (!keep_host) return SP_EINVAL;
    return score_batch(desc, R, Q, K, cu_window_host, keep_host, importance, ws, ws_bytes, stream);
}

sp_status sp_window_layout(int64_t M, int32_t window, int32_t stride, int32_t* n_windows,
                           int64_t* starts, int64_t* lens, int64_t* keeps, int32_t capacity) {
    if (!n_windows || M < 1 || window < 1 || stride < 1 || stride > window || capacity < 0)
        return SP_EINVAL;
    // windows at 0, stride, 2 stride, ...; each keeps its first stride scores,
    // the one that reaches the prompt's end keeps all of its own and is last
    int32_t R = 0;
    for (int64_t pos = 0;; pos += stride) {
        const int64_t end = pos + window < M ? pos + window : M;
        const bool last = end >= M;
        if (starts && R < capacity) {
            starts[R] = pos;
            lens[R] = end - pos;
            keeps[R] = last ? end - pos : stride;
        }
        ++R;
        if (last) break;
    }
    *n_windows = R;
    if (starts && (!lens || !keeps || capacity < R)) return SP_EINVAL;
    return SP_OK;
}

sp_status sp_gather_rows(const void* src, int64_t row_bytes, const int32_t* kept_idx,
                         const int32_t* n_kept, int32_t R, const int64_t* cu_host, void* dst,
                         void* stream) {
    if (!src || !kept_idx || !n_kept || !cu_host || !dst || R < 1) return SP_EINVAL;
    if (row_bytes < 4 || row_bytes % 4 != 0) return SP_EUNSUPPORTED;
    if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(kept_idx, 4) || !aligned(n_kept, 4))
        return SP_EINVAL;
    if (cu_host[0] != 0) return SP_EINVAL;
    long long max_rows = 0;
    for (int r = 0; r < R; ++r) {
        const long long m = cu_host[r + 1] - cu_host[r];
        if (m < 1) return SP_EINVAL;
        if (m > max_rows) max_rows = m;
    }
    if (device_cus() < 1) return SP_EDEVICE;
    return to_status(launch_gather(src, row_bytes, kept_idx, n_kept, R, cu_host, max_rows, dst,
                                   (hipStream_t)stream));
}

sp_status sp_break_even(int64_t M, float keep_fraction, float spec_tps, float target_tps,
                        float safety, int32_t* run) {
    if (!run || M < 1 || !(keep_fraction >= 0.f && keep_fraction <= 1.f) || !(spec_tps > 0.f) ||
        !(target_tps > 0.f) || !(safety > 0.f))
        return SP_EINVAL;
    const double scoring = (double)M / spec_tps;
    const double saved = ((double)M - (double)keep_fraction * (double)M) / target_tps;
    *run = saved >= scoring * safety ? 1 : 0;
    return SP_OK;
}

// Whether sp_select may select one prompt of M tokens by several
// workgroups (given a workspace): min-max normalisation, top-K or mass,
// M >= kSelGridMin.
static bool select_dist_eligible(int64_t M, const sp_select_params* params) {
    return params->mode != SP_SELECT_THRESHOLD && params->norm == SP_NORM_MINMAX && M >= kSelGridMin;
}

size_t sp_select_workspace_bytes(int32_t R, int64_t total_prompt_len,
                                 const sp_select_params* params) {
    if (R < 1 || total_prompt_len < R || check_select_params(params) != SP_OK) return (size_t)-1;
    return R == 1 && select_dist_eligible(total_prompt_len, params) ? kSelDistBytes : 0;
}

sp_status sp_select(const float* importance, int32_t M, const sp_select_params* params,
                    int32_t pos_base, int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept,
                    void* ws, size_t ws_bytes, void* stream) {
    sp_status s = check_select_params(params);
    if (s != SP_OK) return s;
    if (!importance || !kept_idx || !pos_ids || !n_kept) return SP_EINVAL;
    s = check_select_prompt(params, M);
    if (s != SP_OK) return s;
    if ((long long)pos_base + M > 2147483647ll || (long long)pos_base < -2147483647ll)
        return SP_EINVAL;
    const int cus = device_cus();
    if (cus < 1) return SP_EDEVICE;
    const SelectParamsDev p = to_dev(params);
    if (select_dist_eligible(M, params) && ws && ws_bytes >= kSelDistBytes && aligned(ws, 16)) {
        // several workgroups, unless the stream is being captured (their
        // exchange slots carry a launch's epoch, which a graph would fix)
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing((hipStream_t)stream, &cap) != hipSuccess) return SP_EDEVICE;
        if (cap == hipStreamCaptureStatusNone)
            return to_status(launch_select_dist(p, importance, M, pos_base, kept_idx, pos_ids, n_kept, ws,
                                                next_epoch(), wait_limit_ticks(), cus, (hipStream_t)stream));
    }
    const int64_t cu[2] = {0, M};
    return to_status(launch_select(p, cu, &pos_base, 1, importance, kept_idx, pos_ids, n_kept,
                                   (hipStream_t)stream));
}

sp_status sp_select_varlen(const float* importance, int32_t R, const int64_t* cu,
                           const int32_t* pos_base_host, const sp_select_params* params,
                           int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept, void* ws,
                           size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    sp_status s = check_select_params(params);
    if (s != SP_OK) return s;
    if (R < 1 || !cu || !importance || !kept_idx || !pos_ids || !n_kept) return SP_EINVAL;
    if (R > kMaxSelectRequests) return SP_EUNSUPPORTED;
    if (cu[0] != 0) return SP_EINVAL;
    for (int r = 0; r < R; ++r) {
        if (cu[r + 1] - cu[r] < 1) return SP_EINVAL;
        s = check_select_prompt(params, cu[r + 1] - cu[r]);
        if (s != SP_OK) return s;
        const long long pb = pos_base_host ? pos_base_host[r] : 0;
        if (pb + (cu[r + 1] - cu[r]) > 2147483647ll) return SP_EINVAL;
    }
    if (cu[R] > 2147483647ll) return SP_EUNSUPPORTED;
    if (device_cus() < 1) return SP_EDEVICE;
    const SelectParamsDev p = to_dev(params);
    return to_status(launch_select(p, cu, pos_base_host, R, importance, kept_idx, pos_ids, n_kept,
                                   (hipStream_t)stream));
}

}  // extern "C"
