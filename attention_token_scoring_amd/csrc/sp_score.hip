// Look-ahead attention scoring on gfx950.
//
// What is computed ("Speculative Prefill" review page, Core formulas: attention
// score a_ij = Softmax(Q_{M+j} K^T)_i and the max-max-mean importance
// aggregation; "SpecPrefill - Implementation Guide", How It Works, token
// importance): for every layer l, query head h and look-ahead step j the softmax
// of the scaled logits of query M+j over the M+j+1 keys it sees, then
//   importance_i = (1/N) sum_j max_{l,h} p_{l,h,j,i},  i < M.
//
// How (K is read from HBM once):
//  * A unit is one (layer, kv-head) plane of K. The G query heads of the plane
//    and the N look-ahead steps give G*N query rows (row = j*G + h_local),
//    handled as one or two 16-row halves. Logits come from 16x16x32 bf16 (or
//    16x16x4 f32) MFMAs with keys as the M dimension: each lane ends up holding
//    one query row for 4 keys of a tile, so row statistics are lane-local, and
//    each load instruction reads 64 contiguous bytes of a key row.
//  * g workgroups (one per CU; launched cooperatively so all are resident)
//    share a unit, each owning a key slice whose logits stay in registers.
//    Seven waves stream K; the eighth does all synchronisation, because on
//    gfx950 a wave's vector-memory counter is in order: a barrier poll or a
//    release issued by a streaming wave would wait for all of that wave's
//    prefetches. Per unit the control wave publishes the workgroup's per-row
//    (max, sum) partial and arrives at the unit's counter; the last of the g
//    workgroups to arrive combines the partials into each row's log-sum-exp
//    and raises the unit's flag. A unit is finished (log2 probabilities,
//    without touching K again) a unit or two after it is streamed, so the
//    flag is normally up by then; register banks rotate. A ring of K tiles
//    per streaming wave keeps the next unit in flight.
//  * The look-ahead keys M..M+N-1 only enter denominators; a small prep
//    kernel computes their share of each row's statistics.
//  * The max over the G heads of a step is a DPP max across G adjacent lanes;
//    the max over kv-heads and layers is a running max in LDS, in the log2
//    domain (exp2 is monotone, so one exponential per (step, key) at the end).
//    Each group writes its running max; a small kernel takes the max over
//    groups, exponentiates and averages over the steps.
//  * Groups of g <= 32 workgroups sit on one XCD (blockIdx % 8 picks the XCD),
//    so a barrier's traffic stays within one L2.
#include <math.h>

#include <type_traits>

#include "sp_internal.h"

namespace sp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 2 s of the 100 MHz constant clock: a barrier wait longer than this is a bug;
// the kernel records it in the error word and moves on instead of hanging.
constexpr unsigned long long kSpinTicks = 200000000ull;
// Buffer offset that is always out of range: loads there return zeros.
constexpr uint32_t kOob = 0x7ffffff0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ i32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// (m, s) <- combination of two partial softmax statistics (raw-logit max m,
// sum of exp2((x - m) * c)).
__device__ __forceinline__ void combine(float& m, float& s, float m2, float s2, float c) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    s = s * exp2_hw((m - mn) * c) + s2 * exp2_hw((m2 - mn) * c);
    m = mn;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf,
                                                       false));
}

// Max over the G (<= 16) adjacent lanes that hold the G heads of one step.
template <int G>
__device__ __forceinline__ float group_max16(float v) {
    if constexpr (G >= 2) v = fmaxf(v, dpp<0xb1>(v));   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v = fmaxf(v, dpp<0x4e>(v));   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
    if constexpr (G >= 16) v = fmaxf(v, dpp<0x140>(v)); // row_mirror
    return v;
}

template <int G, int K>
__device__ __forceinline__ void group_max16_all(float (&v)[K]) {
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = group_max16<G>(v[i]);
}

// ---------------------------------------------------------------------------------------
// 16-key tiles. A = K tile (16 keys x d), B = Q^T (d x 16 rows), C[key][row].
// Lane L supplies key (and row) L % 16; its lane group g = L / 16 reads bytes
// [64 s + 16 g, 64 s + 16 g + 16) of the row for load s, i.e. the 4 lane groups
// of one load instruction read 64 contiguous bytes of each of 16 key rows. For
// bf16 one load is one 32-deep MFMA k-step (d = 32 s + 8 g + e); for f32 it is
// four 4-deep k-steps (d = 16 s + 4 g + e). Both operands use the same mapping.
// C layout: lane L holds rows L % 16 of keys 4 (L / 16) + r, r = 0..3.
// ---------------------------------------------------------------------------------------
template <int D_, bool BF16_, int NH_>
struct Cfg {
    static constexpr int D = D_, NH = NH_;
    static constexpr bool BF16 = BF16_;
    static constexpr int ESZ = BF16 ? 2 : 4;
    static constexpr int KB = D * ESZ;    // bytes per key row
    static constexpr int NLD = KB / 64;   // 16-byte loads per lane per tile
    static constexpr int TPW = tiles_per_wave(BF16, NH);
    // tiles in flight per wave; must divide TPW so that tile t of every unit
    // lands in ring slot t % NBUF
    static constexpr int NBUF = TPW <= 4 ? TPW : 4;
    static constexpr int NB = kBanks;
    static_assert(TPW % NBUF == 0, "ring depth must divide the tiles per wave");
    static constexpr int ROWS = 16 * NH;
};

template <class C>
struct Frag {
    i32x4 v[C::NLD];
};

template <class C>
__device__ __forceinline__ void mma(f32x4& acc, const i32x4& q, const i32x4& k) {
    if constexpr (C::BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                      __builtin_bit_cast(bf16x8, q), acc, 0, 0, 0);
    } else {
        const f32x4 kv = __builtin_bit_cast(f32x4, k);
        const f32x4 qv = __builtin_bit_cast(f32x4, q);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.x, qv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.y, qv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.z, qv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.w, qv.w, acc, 0, 0, 0);
    }
}

// K fragment of the 16-key tile starting at key0 (zeros when !valid; the
// buffer descriptor bounds the plane, so reads past its end are zeros too).
template <class C>
__device__ __forceinline__ void load_k(Frag<C>& f, __amdgpu_buffer_rsrc_t rs, int key0,
                                       bool valid, int lane) {
    const uint32_t off = valid ? (uint32_t)(key0 + (lane & 15)) * (uint32_t)C::KB +
                                     (uint32_t)(16 * (lane >> 4))
                               : kOob;
#pragma unroll
    for (int s = 0; s < C::NLD; ++s) f.v[s] = load16(rs, off + 64u * s);
}

// Per-unit geometry shared by the helpers below.
struct Unit {
    __amdgpu_buffer_rsrc_t rs;  // this unit's key plane
    int u;                      // unit index, or -1 when the group has no such unit
};

__device__ __forceinline__ Unit unit_at(const ScoreArgs& a, int group, int it, uint32_t plane_bytes,
                                        int esz) {
    Unit x;
    x.u = group + it * a.ngroups;
    if (it >= (1 << 27) || x.u >= a.units) x.u = -1;
    const int uu = x.u < 0 ? 0 : x.u;
    const char* plane = (const char*)a.K + (long long)uu * a.plane_stride * esz;
    x.rs = make_rsrc(plane, x.u < 0 ? 0u : plane_bytes);
    return x;
}

// Q fragments of unit u (both row halves): row = half*16 + lane%16 = j*G + hl.
template <class C>
__device__ __forceinline__ void load_q(Frag<C> (&qf)[C::NH], const ScoreArgs& a, int u, int lane) {
#pragma unroll
    for (int hf = 0; hf < C::NH; ++hf) {
        const int qr = hf * 16 + (lane & 15);
        const int j = qr / a.G, hl = qr - (qr / a.G) * a.G;
        if (u >= 0 && j < a.N) {
            const int l = u / a.Hkv, kvh = u - (u / a.Hkv) * a.Hkv;
            const long long row = ((long long)l * a.H + (long long)kvh * a.G + hl) * a.N + j;
            const char* p = (const char*)a.Q + row * C::KB + 16 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < C::NLD; ++s) qf[hf].v[s] = *(const i32x4*)(p + 64 * s);
        } else {
#pragma unroll
            for (int s = 0; s < C::NLD; ++s) qf[hf].v[s] = i32x4{0, 0, 0, 0};
        }
    }
}

template <class C>
__global__ __launch_bounds__(kThreads, 2) void score_kernel(ScoreArgs a) {
    constexpr int TPW = C::TPW, NH = C::NH, NBUF = C::NBUF, ROWS = C::ROWS, NB = C::NB;
    constexpr int SW = kStreamWaves;  // waves 0..SW-1 stream K; wave SW synchronises
    constexpr int D = NB - 1;         // a unit is finished D units after it is streamed
    extern __shared__ float Trun[];   // [N][row_stride(KR)], log2-domain running max
    __shared__ float2 red[2][SW][ROWS];
    __shared__ float lse_s[2][ROWS];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool ctrl = w == SW;
    int group, rank;
    if (a.xcd_local) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        group = xcd * (32 / a.g) + slot / a.g;
        rank = slot % a.g;
    } else {
        group = blockIdx.x / a.g;
        rank = blockIdx.x % a.g;
    }
    const int KRP = row_stride(a.KR);
    for (int x = tid; x < a.N * KRP; x += kThreads) Trun[x] = -INFINITY;

    const int r0 = rank * a.KR;
    const int r1 = min(r0 + a.KR, a.M);
    const int nkeys = max(r1 - r0, 0);
    const int ntiles = (nkeys + kTileKeys - 1) / kTileKeys;
    const uint32_t plane_bytes = (uint32_t)(a.M + a.N) * (uint32_t)C::KB;
    const float c = a.c;
    const int g4 = lane >> 4;  // lane group

    // Per-lane query rows of the halves, and whether the lane writes the
    // running max of its step (it holds the step's first head; for G = 32 both
    // halves hold one step and half 0 writes).
    int jrow[NH];
    bool own[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const int qr = hf * 16 + (lane & 15);
        jrow[hf] = qr / a.G;
        own[hf] = (qr - jrow[hf] * a.G) == 0 && jrow[hf] < a.N && !(NH == 2 && a.G == 32 && hf == 1);
    }

    f32x4 acc0[TPW][NH], acc1[TPW][NH], acc2[TPW][NH];
    Frag<C> qf[NH];
    Frag<C> fb[NBUF];

    const int n_units = group < a.units ? (a.units - group + a.ngroups - 1) / a.ngroups : 0;
    // prime the streaming waves: Q and the first NBUF tiles of the first unit
    if (!ctrl) {
        const Unit first = unit_at(a, group, 0, plane_bytes, C::ESZ);
        load_q<C>(qf, a, first.u, lane);
#pragma unroll
        for (int t = 0; t < NBUF; ++t) {
            const int tile = w + SW * t;
            load_k<C>(fb[t], first.rs, r0 + tile * kTileKeys, first.u >= 0 && tile < ntiles, lane);
        }
    }

    // [streaming waves] Stream unit `cur` into acc (the ring runs ahead into
    // `nxt`) and leave the slice's per-row statistics in red[pb].
    auto stream = [&](f32x4 (&acc)[TPW][NH], const Unit& cur, const Unit& nxt, int pb) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
                acc[t][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < C::NLD; ++s) mma<C>(acc[t][hf], qf[hf].v[s], fb[t % NBUF].v[s]);
            }
            const int tn = t + NBUF;  // refill the slot with the tile NBUF ahead
            if (tn < TPW) {
                const int tile = w + SW * tn;
                load_k<C>(fb[t % NBUF], cur.rs, r0 + tile * kTileKeys, tile < ntiles, lane);
            } else {
                const int tile = w + SW * (tn - TPW);
                load_k<C>(fb[t % NBUF], nxt.rs, r0 + tile * kTileKeys, nxt.u >= 0 && tile < ntiles,
                          lane);
            }
        }
        load_q<C>(qf, a, nxt.u, lane);  // the Q registers are free

        float m[NH], sm[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            m[hf] = -INFINITY;
            sm[hf] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int kt = (w + SW * t) * kTileKeys;  // first key of the tile in the slice
            if (kt + kTileKeys > nkeys) {             // partial or empty tile: mask
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int hf = 0; hf < NH; ++hf)
                        if (kt + 4 * g4 + r >= nkeys) acc[t][hf][r] = -INFINITY;
            }
#pragma unroll
            for (int hf = 0; hf < NH; ++hf)
#pragma unroll
                for (int r = 0; r < 4; ++r) m[hf] = fmaxf(m[hf], acc[t][hf][r]);
        }
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            if (m[hf] != -INFINITY) {
                const float mc = m[hf] * c;
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sm[hf] += exp2_hw(fmaf(acc[t][hf][r], c, -mc));
            }
            // lanes L, L^16, L^32, L^48 hold the same row
            combine(m[hf], sm[hf], __shfl_xor(m[hf], 16), __shfl_xor(sm[hf], 16), c);
            combine(m[hf], sm[hf], __shfl_xor(m[hf], 32), __shfl_xor(sm[hf], 32), c);
            if (g4 == 0) red[pb][w][hf * 16 + lane] = make_float2(m[hf], sm[hf]);
        }
    };

    // Cross-workgroup data (partials, counters, log-sum-exps, flags) moves
    // through agent-scope atomic loads and stores, which are coherent across
    // the XCDs' L2s; a producer waits for its stores to complete (vmcnt(0), this
    // wave's own operations only) before it signals, and a consumer issues its
    // loads only after it has seen the signal.
    auto st64 = [](void* p, float x, float y) {
        const unsigned long long bits =
            (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
        __hip_atomic_store((unsigned long long*)p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto ld64 = [](const void* p) -> float2 {
        const unsigned long long bits = __hip_atomic_load((unsigned long long*)p, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
        return make_float2(__uint_as_float((unsigned)bits), __uint_as_float((unsigned)(bits >> 32)));
    };

    // [control wave] Publish the workgroup's partial of unit u and arrive at
    // the unit's counter. The last of the g workgroups to arrive combines all
    // partials and the look-ahead keys' share into each row's log-sum-exp and
    // raises the unit's flag. Lane L handles row pair q = L % 16 (rows 2q,
    // 2q+1) for ranks L / 16, L / 16 + 4, ...
    auto arrive = [&](int u, int pb) {
        if (lane < ROWS) {
            float mm = red[pb][0][lane].x, ss = red[pb][0][lane].y;
            for (int x = 1; x < SW; ++x) combine(mm, ss, red[pb][x][lane].x, red[pb][x][lane].y, c);
            st64(a.part + ((size_t)u * a.g + rank) * ROWS + lane, mm, ss);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the partial is stored
        int old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(a.cnt + u, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        if (old != a.g - 1) return;
        const int q = lane & 15, sub = lane >> 4;
        const bool live = 2 * q < ROWS;
        float m0 = -INFINITY, s0 = 0.f, m1 = -INFINITY, s1 = 0.f;
        if (sub == 0 && live) {
            const float4 t = *(const float4*)(a.tail + (size_t)u * ROWS + 2 * q);
            m0 = t.x; s0 = t.y; m1 = t.z; s1 = t.w;
        }
        constexpr int B = 24;  // ranks in flight per lane
        for (int rr0 = sub; rr0 < a.g; rr0 += 4 * B) {
            float2 p0[B], p1[B];
#pragma unroll
            for (int x = 0; x < B; ++x) {
                const int rr = rr0 + 4 * x;
                if (live && rr < a.g) {
                    const float2* base = a.part + ((size_t)u * a.g + rr) * ROWS + 2 * q;
                    p0[x] = ld64(base);
                    p1[x] = ld64(base + 1);
                } else {
                    p0[x] = p1[x] = make_float2(-INFINITY, 0.f);
                }
            }
#pragma unroll
            for (int x = 0; x < B; ++x) {
                combine(m0, s0, p0[x].x, p0[x].y, c);
                combine(m1, s1, p1[x].x, p1[x].y, c);
            }
        }
        combine(m0, s0, __shfl_xor(m0, 16), __shfl_xor(s0, 16), c);
        combine(m1, s1, __shfl_xor(m1, 16), __shfl_xor(s1, 16), c);
        combine(m0, s0, __shfl_xor(m0, 32), __shfl_xor(s0, 32), c);
        combine(m1, s1, __shfl_xor(m1, 32), __shfl_xor(s1, 32), c);
        if (sub == 0 && live)
            st64(a.lse + (size_t)u * ROWS + 2 * q, m0 * c + log2_hw(s0), m1 * c + log2_hw(s1));
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the log-sum-exps are stored
        if (lane == 0) __hip_atomic_store(a.flag + u, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // [control wave] Wait for unit fu's flag, then put its log-sum-exps in
    // lse_s[pb].
    auto fetch_lse = [&](int fu, int pb) {
        if (lane == 0) {
            const unsigned long long t0 = wall_clock64();
            while (__hip_atomic_load(a.flag + fu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
                __builtin_amdgcn_s_sleep(1);
                if (wall_clock64() - t0 > kSpinTicks) {
                    __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < ROWS)
            lse_s[pb][lane] = __hip_atomic_load(a.lse + (size_t)fu * ROWS + lane, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    };

    // [streaming waves] Finish a unit: log2 probabilities, max over the G
    // heads of each step, running max over units in LDS.
    auto finish = [&](f32x4 (&acc)[TPW][NH], int pb) {
        float lse[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) lse[hf] = lse_s[pb][hf * 16 + (lane & 15)];
        const bool g32 = NH == 2 && a.G == 32;  // both halves hold the one step
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
                if (hf == 1 && g32) break;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = fmaf(acc[t][hf][r], c, -lse[hf]);
                    if (g32) v[r] = fmaxf(v[r], fmaf(acc[t][NH - 1][r], c, -lse[NH - 1]));
                }
                switch (a.G) {
                    case 1: break;
                    case 2: group_max16_all<2>(v); break;
                    case 4: group_max16_all<4>(v); break;
                    case 8: group_max16_all<8>(v); break;
                    default: group_max16_all<16>(v); break;
                }
                if (!own[hf]) continue;
                float* row = Trun + jrow[hf] * KRP + 4 * g4;
                const int kt = (w + SW * t) * kTileKeys;
                if (kt + kTileKeys <= nkeys) {  // full tile
                    float old[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) old[r] = row[kt + r];
#pragma unroll
                    for (int r = 0; r < 4; ++r) row[kt + r] = fmaxf(old[r], v[r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (kt + 4 * g4 + r < nkeys) row[kt + r] = fmaxf(row[kt + r], v[r]);
                }
            }
        }
    };

    // Unit `it` streams into acc0 and is finished D units later; the banks
    // rotate (acc0 -> acc1 -> acc2) after every step. The streaming waves and
    // the control wave run separate loops with one workgroup barrier per step
    // each: before it, streaming (red[pb]) and the control wave's combine
    // (lse_s[pb]); after it, finishing and arriving. The LDS buffers alternate
    // by step parity.
    if (!ctrl) {
        for (int it = 0; it < n_units + D; ++it) {
            const int pb = it & 1;
            const Unit cur = unit_at(a, group, it, plane_bytes, C::ESZ);
            const int fu = it >= D ? unit_at(a, group, it - D, plane_bytes, C::ESZ).u : -1;
            if (cur.u >= 0) stream(acc0, cur, unit_at(a, group, it + 1, plane_bytes, C::ESZ), pb);
            __syncthreads();
            if (fu >= 0) {
                if constexpr (NB == 3) finish(acc2, pb);
                else finish(acc1, pb);
            }
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    if constexpr (NB == 3) acc2[t][hf] = acc1[t][hf];
                    acc1[t][hf] = acc0[t][hf];
                }
        }
    } else {
        for (int it = 0; it < n_units + D; ++it) {
            const int pb = it & 1;
            const int cu = it < n_units ? group + it * a.ngroups : -1;
            const int fu = (it >= D && it - D < n_units) ? group + (it - D) * a.ngroups : -1;
            if (fu >= 0) fetch_lse(fu, pb);
            __syncthreads();
            if (cu >= 0) arrive(cu, pb);
        }
    }
    __syncthreads();
    for (int x = tid; x < a.N * nkeys; x += kThreads) {
        const int jj = x / nkeys, k = x - (x / nkeys) * nkeys;
        a.Tg[((size_t)group * a.N + jj) * a.M + r0 + k] = Trun[jj * KRP + k];
    }
}

// Before the cooperative kernel: zero its barrier counters, and compute for
// every unit and query row the share of the look-ahead keys M..M+N-1 in the
// row's softmax denominator (row j sees look-ahead key t iff t <= j), as a raw
// max and a sum of exp2((x - max) * c). One wave per unit, one lane per row.
template <bool BF16>
__global__ __launch_bounds__(64) void score_prep_kernel(ScoreArgs a, int rows) {
    const int u = blockIdx.x, lane = threadIdx.x;
    if (lane == 0) {
        a.cnt[u] = 0;
        a.flag[u] = 0;
    }
    if (u == 0 && lane == 0) *a.err = 0;
    if (lane >= rows) return;
    const int j = lane / a.G, hl = lane - (lane / a.G) * a.G;
    float m = -INFINITY, s = 0.f;
    if (j < a.N) {
        const int l = u / a.Hkv, kvh = u - (u / a.Hkv) * a.Hkv;
        const int esz = BF16 ? 2 : 4;
        const long long qrow = ((long long)l * a.H + (long long)kvh * a.G + hl) * a.N + j;
        const char* q = (const char*)a.Q + qrow * a.d * esz;
        const char* kp = (const char*)a.K + ((long long)u * a.plane_stride + (long long)a.M * a.d) * esz;
        float x[32];
        for (int t = 0; t <= j; ++t) {
            float acc = 0.f;
            for (int e = 0; e < a.d; ++e) {
                float qv, kv;
                if (BF16) {
                    qv = __uint_as_float((unsigned)((const unsigned short*)q)[e] << 16);
                    kv = __uint_as_float((unsigned)((const unsigned short*)kp)[(long long)t * a.d + e] << 16);
                } else {
                    qv = ((const float*)q)[e];
                    kv = ((const float*)kp)[(long long)t * a.d + e];
                }
                acc = fmaf(qv, kv, acc);
            }
            x[t] = acc;
            m = fmaxf(m, acc);
        }
        for (int t = 0; t <= j; ++t) s += exp2_hw(fmaf(x[t], a.c, -m * a.c));
    }
    a.tail[(size_t)u * rows + lane] = make_float2(m, s);
}

// importance_i = (1/N) sum_j exp2(max_group Tg[group][j][i])
__global__ void score_finalize_kernel(const float* __restrict__ Tg, int ngroups, int N, int M,
                                      float* __restrict__ importance) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M) return;
    float sum = 0.f;
    for (int jj = 0; jj < N; ++jj) {
        float mx = -INFINITY;
        for (int gr = 0; gr < ngroups; ++gr) mx = fmaxf(mx, Tg[((size_t)gr * N + jj) * M + i]);
        sum += exp2_hw(mx);
    }
    importance[i] = sum / (float)N;
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
template <class C>
static const void* kernel_ptr() {
    return (const void*)&score_kernel<C>;
}

static const void* pick_kernel(int dtype, int d, int rows) {
    const bool bf = dtype == SP_BF16;
    if (rows == 32) {
        if (d == 128) return bf ? kernel_ptr<Cfg<128, true, 2>>() : kernel_ptr<Cfg<128, false, 2>>();
        if (d == 64) return bf ? kernel_ptr<Cfg<64, true, 2>>() : kernel_ptr<Cfg<64, false, 2>>();
    } else {
        if (d == 128) return bf ? kernel_ptr<Cfg<128, true, 1>>() : kernel_ptr<Cfg<128, false, 1>>();
        if (d == 64) return bf ? kernel_ptr<Cfg<64, true, 1>>() : kernel_ptr<Cfg<64, false, 1>>();
    }
    return nullptr;
}

// One request: prep (zero barrier counters), cooperative scoring, finalize.
hipError_t launch_score(const ScorePlan& p, const sp_score_desc& d, const void* Q, const void* K,
                        long long plane_stride, int M, float* importance, void* ws,
                        hipStream_t stream) {
    char* base = (char*)ws;
    ScoreArgs a;
    a.Q = Q;
    a.K = K;
    a.plane_stride = plane_stride;
    a.cnt = (int*)(base + p.ws_cnt);
    a.err = (int*)(base + p.ws_cnt + 4 * (size_t)p.units);
    a.part = (float2*)(base + p.ws_part);
    a.tail = (float2*)(base + p.ws_tail);
    a.lse = (float*)(base + p.ws_lse);
    a.flag = (int*)(base + p.ws_flag);
    a.d = d.d;
    a.Tg = (float*)(base + p.ws_tg);
    a.L = d.L;
    a.H = d.H;
    a.Hkv = d.Hkv;
    a.G = d.H / d.Hkv;
    a.N = d.N;
    a.M = M;
    a.g = p.g;
    a.ngroups = p.ngroups;
    a.KR = p.KR;
    a.units = p.units;
    a.xcd_local = p.xcd_local;
    const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.d);
    a.c = scale * 1.4426950408889634f;

    const void* fn = pick_kernel(d.dtype, d.d, p.rows);
    if (!fn) return hipErrorInvalidValue;
    // Dynamic LDS: the running max, padded so that two workgroups never share a CU.
    size_t lds = (size_t)d.N * row_stride(p.KR) * sizeof(float);
    const size_t min_lds = 96 * 1024;
    if (lds < min_lds) lds = min_lds;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;

    if (d.dtype == SP_BF16)
        hipLaunchKernelGGL(score_prep_kernel<true>, dim3(p.units), dim3(64), 0, stream, a, p.rows);
    else
        hipLaunchKernelGGL(score_prep_kernel<false>, dim3(p.units), dim3(64), 0, stream, a, p.rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* args[] = {&a};
    e = hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(kThreads), args, (unsigned)lds, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(score_finalize_kernel, dim3((M + 255) / 256), dim3(256), 0, stream,
                       (const float*)a.Tg, p.ngroups, d.N, M, importance);
    return hipGetLastError();
}

}  // namespace sp
