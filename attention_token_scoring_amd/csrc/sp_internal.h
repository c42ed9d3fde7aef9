// Internal declarations shared by the library's host code and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/specprefill.h"

namespace sp {

// Waves per scoring workgroup and logit tiles each wave keeps in registers.
// Query-row tiles are 16 or 32 rows (the MFMA N dimension); a tile covers as
// many keys as rows, so one workgroup holds the logits of 8*4*32 = 1024 keys
// (32-row tiles) or 8*16*16 = 2048 keys (16-row tiles) for one (layer,
// kv-head) unit.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTilesPerWave32 = 4;
constexpr int kTilesPerWave16 = 16;
// Padding (floats) between the look-ahead rows of the per-workgroup running
// maximum in LDS, to spread the rows over banks.
constexpr int kRowPad = 8;

// Everything the cooperative scoring kernel needs for one request.
struct ScoreArgs {
    const void* Q;             // [L][H][N][d] of this request
    const void* K;             // key row 0 of (layer 0, kv-head 0) of this request
    long long plane_stride;    // elements between consecutive (layer, kv-head) key planes
    float* Tg;                 // [ngroups][N][M]: per-group running max of log2 probabilities
    float2* part;              // [units][g][rows]: per-workgroup (row max, row sum) partials
    int* cnt;                  // [units]: arrival counters of the per-unit barriers
    int* err;                  // [1]: set when a barrier wait times out
    int L, H, Hkv, G, N, M;
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
    size_t ws_cnt, ws_part, ws_tg, ws_total;  // byte offsets / sizes in the workspace
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
