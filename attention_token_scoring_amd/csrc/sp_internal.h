// Internal declarations shared by the library's host code and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/specprefill.h"

namespace sp {

// Scoring workgroups have 8 waves (two per SIMD, 256 registers each): 7 stream
// K, one synchronises. Keys are processed in tiles of 16 (the M dimension of
// the 16x16 MFMAs); query rows in 16-row halves (NH = 1 or 2 halves per
// kv-head). Each streaming wave keeps the logits of kBanks units in registers
// (a unit is finished kBanks-1 units after it is streamed).
constexpr int kWaves = 8;
constexpr int kStreamWaves = 7;
constexpr int kThreads = kWaves * 64;
constexpr int kTileKeys = 16;
constexpr int kBanks = 3;
constexpr int tiles_per_wave(bool bf16, int nh) { return (bf16 ? 4 : 2) * (nh == 1 ? 2 : 1); }
// Extra floats per look-ahead row of the LDS running maximum: rows start 16
// banks apart.
constexpr int row_stride(int kr) { return (kr + 63) / 64 * 64 + 16; }

// Everything the cooperative scoring kernel needs for one request.
struct ScoreArgs {
    const void* Q;             // [L][H][N][d] of this request
    const void* K;             // key row 0 of (layer 0, kv-head 0) of this request
    long long plane_stride;    // elements between consecutive (layer, kv-head) key planes
    float* Tg;                 // [ngroups][N][M]: per-group running max of log2 probabilities
    float2* part;              // [units][g][rows]: per-workgroup (row max, row sum) partials
    float2* tail;              // [units][rows]: the look-ahead keys' (row max, row sum)
    float* lse;                // [units][rows]: each row's log2-sum-exp2 (scaled logits)
    int* flag;                 // [units]: set once the unit's lse is published
    int* cnt;                  // [units]: arrival counters of the per-unit barriers
    int* err;                  // [1]: set when a barrier wait times out
    int L, H, Hkv, G, N, M, d;
    int g;                     // workgroups cooperating on one unit
    int ngroups;               // groups working in parallel
    int KR;                    // prompt keys per workgroup (multiple of the tile width)
    int units;                 // L * Hkv
    int xcd_local;             // 1: map groups onto the 8 XCDs (g divides 32)
    float c;                   // scale * log2(e)
};

struct ScorePlan {
    int rows;      // 16 or 32
    int cap;       // prompt keys one workgroup can hold
    int g, ngroups, KR, units, grid;
    int xcd_local;
    size_t ws_cnt, ws_part, ws_tail, ws_lse, ws_flag, ws_tg, ws_total;  // byte offsets / sizes in the workspace
};

// Selection of one request (one workgroup).
struct SelectReq {
    const float* x;       // importance of this request
    int32_t* kept;        // output region of this request
    int32_t* pos;
    int32_t* n_kept;      // one int
    int M;
    int pos_base;
    int base_index;       // added to kept indices (packed offset of the request)
};

struct SelectParamsDev {
    int chunk, pool_k, mode;
    float keep_rate, mass;
    int first_n;
    float first_mult;
    int last_n;
    float last_mult;
};

}  // namespace sp
