// Launch planning for the scoring kernel: the split of each (layer, kv-head)
// unit over workgroups, the LDS layout and the workspace.
#include <mutex>

#include "sp_internal.h"

namespace sp {

namespace {

constexpr int kMaxCombiners = 4;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int esize(sp_dtype t) { return t == SP_BF16 ? 2 : 4; }

}  // namespace

// Launch plan for one prompt of M keys: choose the number g of workgroups that
// share a (layer, kv-head) unit so that each slice fits what one workgroup can
// keep in flight and park (registers and LDS), the groups fill the device with
// at least one CU left for combining, and the per-unit exchanges stay few;
// then lay out LDS and the workspace.
static sp_status plan_uncached(const sp_score_desc& d, long long M, int cus, int only_tpw, ScorePlan* out) {
    ScorePlan p;
    const int G = d.H / d.Hkv;
    const bool bf = d.dtype == SP_BF16;
    p.rows = G * d.N <= 16 ? 16 : 32;
    const int tk = kTileKeys;
    const int row_bytes = d.d * esize(d.dtype);
    p.units = d.L * d.Hkv;
    if (M < 1) return SP_EINVAL;
    if ((unsigned long long)(M + d.N) * d.d * esize(d.dtype) >= (1ull << 31)) return SP_EUNSUPPORTED;
    if (cus < 1) cus = kDefaultCUs;
    if (cus < 2) return SP_EUNSUPPORTED;
    const double bytes_per_key = (double)row_bytes;
    // the slices cover the prompt and the look-ahead keys (the last slice
    // holds the latter too: they count in the rows' softmax denominators)
    const long long MK = M + d.N;
    // A step takes the longer of (a) the busiest streaming wave's work on its
    // tiles (measured on the MI355X: ~4.1 us for 4 tiles, ~5.7 us for 5 tiles
    // without the registers for the guard-free statistics), and (b) the
    // step's bytes at the HBM rate the kernel sustains (~6.2 TB/s).
    const double bw_total = 6.2e12;
    const double wave_base = 1.0e-6, wave_per_tile = 0.77e-6, wave_tight = 0.85e-6,
                 wave_partial = 0.1e-6;
    double best = 1e300;
    int bg = 0, bkr = 0, bng = 0, bdef = 0, btpw = 0;
    const int tpw0 = tiles_per_wave(bf, d.d);
    // (one head per step over two halves: the base tile count only)
    const int tpw1 = (G == 1 && p.rows == 32) ? tpw0 : tpw0 + 1;
    for (int tpw = tpw0; tpw <= tpw1; ++tpw) {
        if (only_tpw > 0 && tpw != only_tpw) continue;
        const int cap = kStreamWaves * tpw * kTileKeys;
        const long long gmin = (MK + cap - 1) / cap;
        const bool roomy = score_roomy(row_bytes, tpw, p.rows / 16);
        for (long long cand = 0; cand < 2 * (cus - gmin + 1); ++cand) {
            // each g with the smallest slice that covers M, then with a full one
            // (cap keys; the last workgroup takes the rest)
            const long long g = gmin + cand / 2;
            if (g > cus - 1 || g > kMaxRanks) break;
            long long kr = (MK + g - 1) / g;
            kr = (kr + tk - 1) / tk * tk;
            if (cand % 2 == 1) {
                if (kr == cap) continue;  // (already planned)
                kr = cap;
            }
            if (kr > cap) continue;
            const long long geff = (MK + kr - 1) / kr;
            if (geff != g) continue;  // the same slice with fewer workgroups is planned at geff
            int defer = 0;
            for (int D = kMaxDefer; D >= 1; --D)
                if (score_lds_layout(D + 1, tpw, p.rows, row_bytes, d.N, (int)kr).total <= kLdsBytes) {
                    defer = D;
                    break;
                }
            if (defer == 0) continue;
            long long ng = (cus - 1) / g;
            if (ng > p.units) ng = p.units;
            if (ng > kMaxFlags / g) ng = kMaxFlags / g;
            if (ng > kMaxDone / g) ng = kMaxDone / g;
            if (ng < 1) continue;
            const long long iters = (p.units + ng - 1) / ng;
            // where the kernel has a guard-free copy of the statistics for
            // waves whose tiles all lie inside the slice, a slice that leaves
            // some wave short puts the slower copy on every step's critical
            // path; a shallower deferral exposes more of each exchange's latency
            const long long busiest = (kr / tk + kStreamWaves - 1) / kStreamWaves;  // tiles of the busiest wave
            const double wave = wave_base + wave_per_tile * busiest + (roomy ? 0.0 : wave_tight) +
                                (roomy && kr < cap ? wave_partial : 0.0);
            const double hbm = (double)(g * ng) * kr * bytes_per_key / bw_total;
            const double sync = (kMaxDefer - defer) * 1.0e-6;
            double cost = iters * ((wave > hbm ? wave : hbm) + sync);
            if (bf && score_lds_layout(kMaxDefer + 1, tpw, p.rows, row_bytes, d.N, (int)kr, true).total +
                              dma_static_lds(p.rows, row_bytes) <= kLdsBytes) {
                // K by DMA (measured on the MI355X at the 8B shape): a step
                // streams at the full read rate (~7.1 TB/s once ~200 CUs
                // stream) plus ~0.28 us of per-step work that does not
                // overlap; waves with fewer tiles than the others (a slice
                // that is not a whole number of tiles per wave) add ~0.12 us
                const double bw = 7.1e12 * ((double)(g * ng) < 200.0 ? (double)(g * ng) / 200.0 : 1.0);
                const bool whole = kr % (kStreamWaves * kTileKeys) == 0 || g == 1;
                cost = iters * ((double)(g * ng) * kr * bytes_per_key / bw + 0.28e-6 + (whole ? 0.0 : 0.12e-6));
            }
            if (cost < best * 0.999) {
                best = cost;
                bg = (int)g;
                bkr = (int)kr;
                bng = (int)ng;
                bdef = defer;
                btpw = tpw;
            }
        }
    }
    if (bg == 0) return SP_EUNSUPPORTED;
    // bf16 streams K by DMA into LDS when its slots, with the full deferral,
    // fit
    p.dma = bf &&
            score_lds_layout(kMaxDefer + 1, btpw, p.rows, row_bytes, d.N, bkr, true).total +
                    dma_static_lds(p.rows, row_bytes) <= kLdsBytes;
    if (p.dma) bdef = kMaxDefer;
    p.tpw = btpw;
    p.cap = kStreamWaves * btpw * kTileKeys;
    p.g = bg;
    p.KR = bkr;
    p.ngroups = bng;
    p.defer = bdef;
    p.ncomb = cus - bg * bng;
    if (p.ncomb > kMaxCombiners) p.ncomb = kMaxCombiners;
    p.grid = bg * bng + p.ncomb;
    p.cus = cus;
    p.cost = best;
    p.lds = score_lds_layout(bdef + 1, btpw, p.rows, row_bytes, d.N, bkr, p.dma);
    // the header (error word, last epoch, the groups' flags, the fused
    // call's words per streaming workgroup), the tagged partials and
    // log-sum-exps, the fused call's chunk masses, the groups' running maxima
    p.ws_err = 0;
    p.ws_part = kHeaderBytes;
    p.ws_lse = p.ws_part + round_up((size_t)p.units * p.g * p.rows * 16, 256);
    p.ws_sel = p.ws_lse + round_up((size_t)p.units * p.rows * 16, 256);
    p.ws_tg = p.ws_sel + round_up((size_t)kSelMaxChunks * 16, 256);
    p.ws_total = p.ws_tg + round_up((size_t)p.ngroups * d.N * M * 4, 256);
    *out = p;
    return SP_OK;
}

// The search above costs microseconds of host time per call, as much as a
// small prompt's whole scoring kernel; a serving loop asks for the same few
// shapes over and over, so plans are kept in a small direct-mapped table
// keyed by everything the search reads.
namespace {

struct PlanKey {
    int L, H, Hkv, d, N, dtype, cus, tpw;
    long long M;
    bool operator==(const PlanKey& o) const {
        return L == o.L && H == o.H && Hkv == o.Hkv && d == o.d && N == o.N && dtype == o.dtype &&
               cus == o.cus && tpw == o.tpw && M == o.M;
    }
};

constexpr int kPlanSlots = 256;
struct PlanSlot {
    bool used = false;
    PlanKey key;
    ScorePlan plan;
};
PlanSlot g_plans[kPlanSlots];
std::mutex g_plans_mu;

unsigned plan_slot(const PlanKey& k) {
    unsigned long long h = 1469598103934665603ull;
    const long long f[9] = {k.L, k.H, k.Hkv, k.d, k.N, k.dtype, k.cus, k.tpw, k.M};
    for (long long v : f) h = (h ^ (unsigned long long)v) * 1099511628211ull;
    return (unsigned)(h ^ (h >> 29)) % kPlanSlots;
}

}  // namespace

sp_status make_plan(const sp_score_desc& d, long long M, int cus, ScorePlan* out, int only_tpw) {
    const PlanKey k{d.L, d.H, d.Hkv, d.d, d.N, (int)d.dtype, cus, only_tpw, M};
    const unsigned slot = plan_slot(k);
    {
        std::lock_guard<std::mutex> lk(g_plans_mu);
        if (g_plans[slot].used && g_plans[slot].key == k) {
            *out = g_plans[slot].plan;
            return SP_OK;
        }
    }
    ScorePlan p;
    const sp_status s = plan_uncached(d, M, cus, only_tpw, &p);
    if (s != SP_OK) return s;
    {
        std::lock_guard<std::mutex> lk(g_plans_mu);
        g_plans[slot].used = true;
        g_plans[slot].key = k;
        g_plans[slot].plan = p;
    }
    *out = p;
    return SP_OK;
}

// Workspace for any prompt of at most max_M keys (bounds that hold for every
// plan make_plan can choose for M <= max_M).
size_t workspace_bound(const sp_score_desc& d, long long max_M, int cus) {
    if (cus < 1) cus = kDefaultCUs;
    const int G = d.H / d.Hkv;
    const int rows = G * d.N <= 16 ? 16 : 32;
    const long long cap = (long long)kStreamWaves * (tiles_per_wave(d.dtype == SP_BF16, d.d) + 1) * kTileKeys;
    const long long units = (long long)d.L * d.Hkv;
    long long tg_elems = (long long)(units < cus ? units : cus) * max_M;
    if (tg_elems > (long long)cus * cap) tg_elems = (long long)cus * cap;
    tg_elems *= d.N;
    return kHeaderBytes + round_up((size_t)units * cus * rows * 16, 256) + round_up((size_t)units * rows * 16, 256) +
           round_up((size_t)kSelMaxChunks * 16, 256) + round_up((size_t)tg_elems * 4, 256);
}

}  // namespace sp
