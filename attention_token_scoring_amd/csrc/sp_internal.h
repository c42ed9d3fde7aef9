// Internal declarations shared by the library's host code and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/specprefill.h"

namespace sp {

// Scoring workgroups have 8 waves (two per SIMD, 256 registers each): 7 stream
// K, one synchronises. Keys are processed in tiles of 16 (the M dimension of
// the 16x16 MFMAs); query rows in 16-row halves (NH = 1 or 2 halves per
// kv-head). Each streaming wave owns TPW tiles of its workgroup's key slice
// in every unit and keeps two units of K tiles in flight.
constexpr int kWaves = 8;
constexpr int kStreamWaves = 7;
constexpr int kThreads = kWaves * 64;
constexpr int kTileKeys = 16;
// Ranks (partials) one combiner lane polls at once, and the workgroups that can
// share a unit: at most what a combiner workgroup gathers in one batch
// (8 waves x 2 lane groups x kCombinerBatch ranks at 32 query rows).
constexpr int kCombinerBatch = 16;
constexpr int kMaxRanks = kWaves * 2 * kCombinerBatch;
// The workspace header: the error word at byte 0, the last call's epoch at 8,
// from byte 128 one 8-byte flag per streaming workgroup (rank x group: its
// running maxima are in place), and from byte kDoneFlags two 8-byte words per
// streaming workgroup (the min and max of its scores once written; the fused
// selection waits for them).
constexpr int kHeaderBytes = 8192;
constexpr int kDoneFlags = 4096;
constexpr int kMaxFlags = (kDoneFlags - 128) / 8;
constexpr int kMaxDone = (kHeaderBytes - kDoneFlags) / 16;
// Per-prompt chunk limit of the selection (five per thread at 1024 threads:
// 5120 covers the longest prompt the scoring kernel takes, 142,792 tokens, at
// chunk 28 or more); the fused launch's chunk-mass slots are sized by it.
constexpr int kSelMaxChunks = 5120;
// Prompts of at least this many tokens (min-max normalisation) have their
// chunk masses summed by several workgroups: the fused launch's streaming
// workgroups (from kSelDistMin, below which its one 512-thread workgroup
// selects faster), or the selection kernel's grid when given a workspace
// (from kSelGridMin: measured on the MI355X, one 1024-thread workgroup
// selects 32K tokens in 17.1 us, a grid of 16 in 17.5 us; 128K tokens in
// 37.7 against 20.5 us).
constexpr int kSelDistMin = 16384;
constexpr int kSelGridMin = 49152;
// Workspace of the selection by several workgroups: 256 score ranges, then
// the chunk masses (two 8-byte words each).
constexpr size_t kSelDistBytes = (size_t)(2 * 256 + 2 * kSelMaxChunks) * 8;
constexpr int kMaxDefer = 3;          // units between streaming and finishing a unit
constexpr int kLdsBytes = 160 * 1024;  // LDS of one CU
constexpr int kDefaultCUs = 256;       // MI355X; used when no device can be queried
// Tiles per streaming wave and unit: the base value, or one more for long
// prompts (a deeper slice per workgroup).
constexpr int tiles_per_wave(bool bf16, int d) { return (!bf16 && d == 128) ? 2 : 4; }
// Whether a streaming wave's K ring (two units of tpw tiles, row_bytes / 64
// 16-byte loads each) and MFMA accumulators (tpw tiles x nh halves) leave
// registers for the scoring kernel's second copy of the row statistics
// (taken by waves whose tiles all lie inside the slice) and for per-row
// running maxima (the head max taken once, at the end).
constexpr bool score_roomy(int row_bytes, int tpw, int nh) {
    return 2 * tpw * (row_bytes / 64) * 4 + tpw * nh * 4 <= 160;
}
// Floats per look-ahead row of the LDS running maximum: rows start 16 banks
// apart.
constexpr int row_stride(int kr) { return (kr + 63) / 64 * 64 + 16; }

// K slots per streaming wave when K goes by DMA into LDS: one per tile of a
// unit, at most 4 for 256-byte key rows (the LDS holds 7 x 4 tiles of 4 KB
// besides the kernel's other regions). (Two units' worth for 128-byte rows,
// twice the bytes in flight, measured no faster at the 0.8B shape.)
constexpr int dma_slots(int row_bytes, int tpw) { return row_bytes >= 256 && tpw > 4 ? 4 : tpw; }
// LDS bytes of the DMA kernel's static region (Q, statistics, references,
// log-sum-exps), besides its dynamic K slots.
constexpr int dma_static_lds(int rows, int row_bytes, int N_unused = 0) {
    return 2 * rows * (row_bytes + 16) + 2 * kStreamWaves * rows * 8 + (kMaxDefer + 1) * kStreamWaves * rows * 4 +
           2 * rows * 4 + N_unused * 0;
}

// Byte offsets of the scoring kernel's LDS regions (all 16-byte aligned).
struct ScoreLds {
    int bank;   // [nbk][SW][TPW][64 lanes][NH][4]: parked logits, 16-bit codes
    int ref;    // [nbk][SW][rows] float: reference (log2 domain) of the parked logits
    int q;      // [2][rows][row bytes + 16]: Q of the current and the next unit
    int trun;   // [N][row_stride(KR)] int: running maxima in code steps, written at the end over the banks
    int red;    // [2][SW][rows] float2: per-wave (max, sum) of the unit just streamed
    int lse;    // [2][rows] float: log-sum-exp of the unit being finished
    int total;
};

// With dma, the first region holds the K tiles (one slot per tile of each
// streaming wave) instead of parked logits, which stay in registers.
inline ScoreLds score_lds_layout(int nbk, int tpw, int rows, int row_bytes, int N, int KR,
                                 bool dma = false) {
    auto up = [](int x) { return (x + 15) / 16 * 16; };
    const int nh = rows / 16;
    ScoreLds l;
    l.bank = 0;
    // the running maxima are written once, at the end, over the banks
    l.trun = 0;
    const int slots = dma_slots(row_bytes, tpw);
    const int banks = dma ? kStreamWaves * slots * kTileKeys * row_bytes
                          : nbk * kStreamWaves * tpw * 64 * nh * 8;
    if (dma) {
        // only the K slots (and, at the end, the running maxima over them) are
        // dynamic; the kernel's other regions are a static array of misc bytes
        const int trun = N * row_stride(KR) * 4;
        l.ref = l.q = l.red = l.lse = 0;
        l.total = up(banks > trun ? banks : trun);
        return l;
    }
    const int trun = N * row_stride(KR) * 4;
    l.ref = l.bank + up(banks > trun ? banks : trun);
    l.q = l.ref + up(nbk * kStreamWaves * rows * 4);
    l.red = l.q + up(2 * rows * (row_bytes + 16));
    l.lse = l.red + up(2 * kStreamWaves * rows * 8);
    l.total = l.lse + up(2 * rows * 4);
    return l;
}

struct SelectParamsDev {
    int chunk, pool_k, mode;
    float keep_rate, mass;
    int first_n;
    float first_mult;
    int last_n;
    float last_mult;
    int min_tok, max_keep;  // (threshold mode)
    int norm;               // SP_NORM_MINMAX / SP_NORM_PERCENTILE / SP_NORM_ZSCORE
    float norm_lo, norm_hi; // (percentile: the two quantiles; z-score: 0 and the clip c)
};

// The selection a fused scoring launch runs after its scores (sp_score_select).
struct FusedSelect {
    SelectParamsDev p;
    int pos_base;
    int32_t* kept;
    int32_t* pos;
    int32_t* n_kept;
};

// Everything the cooperative scoring kernel needs for one request.
struct ScoreArgs {
    const void* Q;             // [L][H][N][d] of this request
    const void* K;             // key row 0 of (layer 0, kv-head 0) of this request
    long long plane_stride;    // elements between consecutive (layer, kv-head) key planes
    int* Tg;                   // [ngroups][N][M]: per-group running max of log2 probabilities, in code steps
    // Synchronisation slots carry the epoch of the launch that wrote them in
    // the high 32 bits of each 8-byte word, so a slot left by an earlier
    // launch is never taken for this one's and nothing is reset in between
    // (epochs are distinct, non-zero and scattered over 32 bits; a slot counts
    // as written only when both of its words carry the epoch, so leftover
    // bytes pass for one with odds of about 2^-64).
    unsigned long long* part;  // [units][g][rows][2]: per-workgroup (row max | epoch), (row sum | epoch)
    unsigned long long* lse;   // [units][rows][2]: each row's (log2-sum-exp2 | epoch), twice
    unsigned long long* err;   // [1]: (call epoch << 32) | 1 once a wait of the call has timed out
    unsigned* hdr;             // [1]: the epoch of the last call (for sp_score_status)
    unsigned long long* flags; // [g][ngroups]: (epoch << 32) | epoch once a group's running maxima are in Tg
    unsigned epoch;            // this launch's tag
    unsigned call_epoch;       // the call's tag (shared by its launches: the error word spans the call)
    float* importance;         // [M]: the output
    int M_out;                 // only importance[0..M_out) is written (M_out <= M)
    int L, H, Hkv, G, N, M, d;
    int g;                     // workgroups cooperating on one unit
    int ngroups;               // groups working in parallel
    int KR;                    // prompt keys per workgroup (multiple of the tile width)
    int units;                 // L * Hkv
    int defer;                 // D: a unit is finished D units after it is streamed
    int nbk;                   // D + 1 banks of parked logits
    ScoreLds lds;
    float c;                   // scale * log2(e)
    int tail_n;                // look-ahead keys after the prompt, seen causally (N; 0: none)
    int blend_n;               // 0: write the scores; n > 0: importance = (n importance + score) / (n + 1)
    unsigned long long spin_ticks;  // limit of a bounded wait, in ticks of the 100 MHz clock
    // Fused selection (sp_score_select): once every streaming workgroup has
    // written its scores (flags in done), the last combiner workgroup selects
    // from importance[0..M).
    int sel_pos_base;
    SelectParamsDev selp;
    int32_t* sel_kept;         // [M]
    int32_t* sel_pos;          // [M]
    int32_t* sel_n;            // [1]
    unsigned long long* done;  // [streaming workgroups][2]: its scores' min | epoch, max | epoch, once written
    unsigned long long* sel_sums;  // [chunks][2]: a chunk's fixed-point mass, low | epoch, high | epoch
    int sel_dist;              // 1: the streaming workgroups sum the chunk masses
};

// Requests scored in one launch (sp_score_varlen): request r on blocks
// [first[r], first[r + 1]).
constexpr int kMaxPack = 8;
constexpr int kLaunchPlain = 0, kLaunchFused = 1, kLaunchPack = 2;
struct PackArgs {
    int n;
    int first[kMaxPack + 1];
    ScoreArgs args[kMaxPack];
};
static_assert(sizeof(PackArgs) <= 4096, "kernel arguments are limited to 4 KiB");

struct ScorePlan {
    int rows;      // 16 or 32
    int tpw;       // tiles per streaming wave and unit
    bool dma;      // K tiles by DMA into LDS (parked logits in registers)
    int cap;       // prompt keys one workgroup can hold
    int g, ngroups, KR, units;
    int ncomb;     // combiner workgroups (on CUs no group uses)
    int grid;      // g * ngroups + ncomb
    int defer;
    int cus;       // compute units of the device planned for
    double cost;   // the planner's estimate of the kernel's time (s) with cus CUs to itself
    ScoreLds lds;
    size_t ws_err, ws_part, ws_lse, ws_sel, ws_tg, ws_total;  // byte offsets / sizes in the workspace
};

// One request of a launch that scores several (launch_score_pack): its plan
// (for its share of the CUs), operands, output and workspace region.
struct PackRequest {
    ScorePlan plan;
    const void* Q;
    const void* K;
    int M, M_out;
    float* importance;
    void* ws;
};

// Launch plan for one prompt of M keys on a device with cus compute units
// (SP_EINVAL for M < 1, SP_EUNSUPPORTED where no split fits); only_tpw > 0
// restricts the plan to that many tiles per wave.
sp_status make_plan(const sp_score_desc& d, long long M, int cus, ScorePlan* out, int only_tpw = 0);

// Workspace bytes that cover every plan make_plan can choose for M <= max_M.
size_t workspace_bound(const sp_score_desc& d, long long max_M, int cus);

// Events the calling thread wants recorded around each scoring kernel launch
// (profiling aid; both null when unset).
void set_profile_events(hipEvent_t before, hipEvent_t after);

// Limit of the scoring kernel's bounded waits for the calling thread's later
// calls (0: the default of 2 s); a testing aid.
void set_wait_limit(unsigned long long ticks);

// Scoring kernels, one translation unit per operand type and head
// dimension: the instantiation for (rows, G, tiles per wave, K path), or nullptr.
const void* score_kernel_bf16_d128(int rows, int G, int tpw, bool dma);
const void* score_kernel_bf16_d64(int rows, int G, int tpw, bool dma);
const void* score_kernel_f32_d128(int rows, int G, int tpw, bool dma);
const void* score_kernel_f32_d64(int rows, int G, int tpw, bool dma);
const void* score_select_kernel_bf16_d128(int rows, int G, int tpw, bool dma);
const void* score_select_kernel_bf16_d64(int rows, int G, int tpw, bool dma);
const void* score_select_kernel_f32_d128(int rows, int G, int tpw, bool dma);
const void* score_select_kernel_f32_d64(int rows, int G, int tpw, bool dma);
const void* score_pack_kernel_bf16_d128(int rows, int G, int tpw, bool dma);
const void* score_pack_kernel_bf16_d64(int rows, int G, int tpw, bool dma);
const void* score_pack_kernel_f32_d128(int rows, int G, int tpw, bool dma);
const void* score_pack_kernel_f32_d64(int rows, int G, int tpw, bool dma);

}  // namespace sp
