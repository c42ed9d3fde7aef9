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
//    each load instruction reads 64 contiguous bytes of 16 key rows.
//  * g workgroups (one per CU, all resident at once: an ordinary launch no
//    larger than what the device holds at a time, or a cooperative launch)
//    share a unit, each owning a key slice; the slices cover the M prompt keys
//    and then the N look-ahead keys (look-ahead key M+i counts in the softmax
//    of steps j >= i only, a per-lane mask on the one tile per wave that
//    reaches past key M). Seven waves stream K: bf16 tiles travel HBM -> LDS
//    by DMA (buffer loads with the lds modifier) through a few slots per wave,
//    f32 tiles through a register ring two units deep, so HBM never waits for
//    the rest of the pipeline. A streamed unit's logits are parked as 16-bit
//    fixed-point log2 values relative to each wave-row's maximum (in
//    registers on the DMA path, in LDS otherwise), together with the wave's
//    (max, sum) per row.
//  * The eighth wave of each workgroup does the cross-workgroup exchange, off
//    the streaming waves' instruction stream (a wave's vector-memory counter is
//    in order on gfx950, so a poll issued by a streaming wave would wait for
//    all of its prefetches): it publishes the workgroup's per-row (max, sum) of
//    each unit, stages the next unit's Q in LDS, and fetches log-sum-exps one
//    step before they are needed.
//  * Combiner workgroups on CUs no group uses gather the g partials of each unit
//    (their loads do not queue behind any K stream; the eight waves of a
//    combiner split the ranks) and publish each row's log-sum-exp. Every
//    exchanged word carries the epoch of the launch that wrote it, so nothing
//    is reset between launches (and no counter is shared).
//  * D units after streaming a unit, its parked logits become log2
//    probabilities in whole code steps (integers; a probability p carries a
//    relative error of at most 3.4e-4); the max over the G heads of a step is
//    a DPP max across G adjacent lanes; the max over kv-heads and layers is a
//    running max kept in registers (log2 domain: exp2 is monotone, so one
//    exponential per (step, key) at the end).
//  * At the end the ngroups workgroups holding the same key slice (one per
//    group) leave their running maxima in memory and raise epoch-tagged
//    flags; then each takes the max over groups of its share of the slice's
//    keys, exponentiates and averages over the steps.
//  * The fused launch (sp_score_select, an instantiation of its own) then
//    selects: one combiner workgroup runs the chunk selection on the scores,
//    for long prompts on chunk masses the streaming workgroups have summed
//    between them.
//  * A packed launch (sp_score_varlen, also an instantiation of its own)
//    scores up to eight requests side by side: each workgroup finds its request
//    from its block index and runs the one-request code above on that
//    request's workgroups, plan and workspace region.
#pragma once

#include <math.h>

#include <type_traits>

#include "sp_internal.h"
#include "sp_select_core.h"

namespace sp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 2 s of the 100 MHz constant clock (the default limit of a bounded wait): a
// wait longer than this means a workgroup it waits for is not running (not
// resident, or a bug); the kernel records it in the error word and moves on
// instead of hanging. The host may lower the limit (a testing aid).
constexpr unsigned long long kSpinTicks = 200000000ull;
// After 100 us a wait also looks at the error word, so that once one wait of
// the launch has timed out the others end too and the launch drains in about
// one time-out.
constexpr unsigned long long kAbortTicks = 10000ull;
// Buffer offset that is always out of range: loads there return zeros.
constexpr uint32_t kOob = 0x7ffffff0u;

// Bits of the quiet NaN written in place of the scores of a call that timed out.
constexpr unsigned kNaNBits = 0x7fc00000u;

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

// Lane permutation within rows of 16 lanes. Every source lane exists, so
// bound_ctrl is irrelevant; setting it lets the compiler fold the move into
// the consuming v_max.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}

// Max over the G (<= 16) adjacent lanes that hold the G heads of one step.
template <int G>
__device__ __forceinline__ int group_max16(int v) {
    if constexpr (G >= 2) v = max(v, dpp_i<0xb1>(v));   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v = max(v, dpp_i<0x4e>(v));   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v = max(v, dpp_i<0x141>(v));  // row_half_mirror
    if constexpr (G >= 16) v = max(v, dpp_i<0x140>(v)); // row_mirror
    return v;
}

// Butterfly reductions across lanes L ^ 16 and L ^ 32: the swap instructions
// exchange rows (16 lanes) or halves (32 lanes) between two registers, so
// swapping a value with itself leaves each lane holding its own value and its
// partner's, one in each result register.
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void st64(void* p, float x, float y) {
    const unsigned long long bits =
        (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
    __hip_atomic_store((unsigned long long*)p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// The call's error word: set once a bounded wait of any of its launches has
// timed out.
template <class A>
__device__ __forceinline__ bool err_set(const A& a) {
    const unsigned long long v = ld64(a.err);
    return tag_is(v, a.call_epoch) && (v & 1ull) != 0ull;
}
template <class A>
__device__ __forceinline__ void set_err(const A& a) {
    st64u(a.err, ((unsigned long long)a.call_epoch << 32) | 1ull);
}

// A streaming wave's tiles are w, w + SW, ... (ntv of them in the slice).
// masked_tile: the one that needs per-key masks (its last, when that reaches
// past the nall keys every row sees), else -1. The keys past nall (at most
// N - 1 look-ahead keys and the slice's ragged end) span at most three
// consecutive tiles, so no wave has two of them.
__device__ __forceinline__ int masked_tile(int ntv, int w, int nall) {
    return ntv > 0 && (w + kStreamWaves * (ntv - 1) + 1) * kTileKeys > nall ? ntv - 1 : -1;
}
// Keys of tile `tile` (of the slice [r0, r1)) that step j sees, counted from
// this lane's first key in it (4 (lane / 16)); step j sees keys < M + j + 1.
__device__ __forceinline__ int visible_keys(const ScoreArgs& a, int r0, int r1, int j, int tile) {
    const int lane = (int)(threadIdx.x & 63);
    return min(r1, a.M + j + 1) - r0 - tile * kTileKeys - 4 * (lane >> 4);
}

// Whether a bounded wait that started at t0 should give up.
template <class A>
__device__ __forceinline__ bool wait_expired(unsigned long long t0, const A& a) {
    const unsigned long long dt = wall_clock64() - t0;
    return dt > a.spin_ticks || (dt > kAbortTicks && err_set(a));
}

// Parked logits: y = (log2-domain logit) - (row reference) <= 0 as a 16-bit
// unsigned-normalised code of -y / 32 (v_cvt_pknorm_u16_f32 rounds and clamps
// to [0, 65535]): a step of kStep = 32/65535 (about 2^-11) in log2 units over
// y in [-32, 0]. Two codes share one 32-bit word, which travels by value
// (bit-casting an element of a vector-typed value in place is not reliable
// with this compiler).
//
// Finishing works in whole steps: a row's offset (reference - log-sum-exp, in
// log2 units) is rounded to a whole number of steps, so a log2 probability is
// the integer (offset - code) times kStep, and the max over heads and units is
// an integer max. Both roundings are at most half a step, so the final
// p = exp2(kStep * v) carries a relative error of at most ln2 * kStep (3.4e-4)
// whenever y >= -32; below that p < 2^-32 and the clamp changes it by less.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
constexpr float kCodeRange = 32.f;
constexpr float kStep = kCodeRange / 65535.f;
constexpr int kNegInf = -2147483647 - 1;  // running-max start: below every value
// u = -y / kCodeRange, in [0, 1] for y in [-kCodeRange, 0]
__device__ __forceinline__ int pack_u2(float u_lo, float u_hi) {
    return __builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_u16(u_lo, u_hi));
}
// a row's offset in whole steps (clamped far below any probability that
// survives exp2 in fp32, so that offset - code cannot wrap)
__device__ __forceinline__ int offset_steps(float off) {
    return (int)rintf(fmaxf(off * (1.f / kStep), -1.0e9f));
}
// (lo, hi) codes of a word -> log2 probabilities in steps
__device__ __forceinline__ void unpack_v2(int word, int off, int& lo, int& hi) {
    const unsigned w = (unsigned)word;
    lo = off - (int)(w & 0xffffu);
    hi = off - (int)(w >> 16);
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
template <int D_, bool BF16_, int NH_, int G_, int TPW_, bool DMA_ = false>
struct Cfg {
    static constexpr int D = D_, NH = NH_, G = G_;
    static constexpr bool BF16 = BF16_;
    static constexpr bool DMA = DMA_;  // K tiles by DMA into LDS (else a register ring)
    static constexpr int ESZ = BF16 ? 2 : 4;
    static constexpr int KB = D * ESZ;    // bytes per key (and query) row
    static constexpr int QS = KB + 16;    // LDS bytes per staged query row
    static constexpr int NLD = KB / 64;   // 16-byte loads per lane per tile
    static constexpr int TPW = TPW_;     // tiles per wave and unit
    static constexpr int NBUF = 2 * TPW;  // ring: two units of this wave's tiles
    static constexpr int ROWS = 16 * NH;
    // Q loads of the control wave per unit: ROWS rows of KB bytes, 16 B per lane
    static constexpr int QLD = ROWS * KB / (64 * 16);
    // G = 32 (one step per unit) spans both halves; otherwise a step's heads
    // sit in G adjacent lanes of one half
    static_assert(G <= 16 || (G == 32 && NH == 2), "unsupported head grouping");
    static constexpr int GL = G == 32 ? 16 : G;  // heads of a step within one half
    // DMA slots per streaming wave (one per tile of a unit, at most 4 for
    // 256-byte key rows)
    static constexpr int S = !DMA ? 0 : dma_slots(KB, TPW);
};

// s_waitcnt operands (gfx9 encoding): vector memory count n, nothing else
// waited for; LDS / scalar count 0, nothing else waited for.
constexpr unsigned vm_wait(int n) { return (unsigned)((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8)); }
constexpr unsigned kLgkmWait0 = (15u) | (3u << 14) | (7u << 4);
// cache policy of the DMA loads: non-temporal (streamed once)
constexpr int kNonTemporal = 2;

// LDS stores the compiler does not order against the DMA writes in flight
// (it cannot tell that they go to other addresses, and would wait for every
// load before each store). LDS operations complete in issue order, so the
// waits the compiler computes for its own LDS accesses stay correct.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void lds_store_f2(void* p, float2 v) {
    asm volatile("ds_write_b64 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store_f1(void* p, float v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// One DMA load: 16 bytes per lane from the buffer at voffset + soffset into
// LDS at lds + 16 * lane (non-temporal). (A device function: the builtin
// cannot appear in a lambda, which is also compiled for the host.)
__device__ __forceinline__ void dma_load16(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t voffset,
                                           uint32_t soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset,
                                             soffset, 0, kNonTemporal);
}

// The per-step workgroup barrier. With K in flight by DMA it waits for the
// wave's LDS operations only (a full barrier would also wait for every load in
// flight); the compiler fences keep LDS accesses on their side of it.
template <class C>
__device__ __forceinline__ void step_barrier() {
    if constexpr (C::DMA) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(kLgkmWait0);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    } else {
        __syncthreads();
    }
}

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

// K fragment of a 16-key tile; off is the lane's byte offset of its first
// load in the plane (kOob for a tile past the slice: zeros; the buffer
// descriptor bounds the plane, so reads past its end are zeros too).
template <class C>
__device__ __forceinline__ void load_k(Frag<C>& f, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    // one offset register per tile; the 64-byte steps go in the instructions'
    // offset field (otherwise every (tile, step) offset is kept live)
    asm volatile("" : "+v"(off));
#pragma unroll
    for (int s = 0; s < C::NLD; ++s) f.v[s] = load16(rs, off + 64u * s);
}

// Key plane of unit u (an empty descriptor when u < 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const ScoreArgs& a, int u,
                                                             uint32_t plane_bytes, int esz) {
    const int uu = u < 0 ? 0 : u;
    const char* plane = (const char*)a.K + (long long)uu * a.plane_stride * esz;
    return make_rsrc(plane, u < 0 ? 0u : plane_bytes);
}

// The fused selection, a function of its own (not inlined: with the
// scoring kernel's register pressure the inlined selection does not compile),
// on the launch's dynamic LDS.
extern __shared__ __attribute__((aligned(16))) unsigned long long fused_lds[];
__device__ __attribute__((noinline)) inline void fused_select(SelectParamsDev p, const float* x, int M, int pb,
                                                              int32_t* kept, int32_t* pos, int32_t* n) {
    select_prompt<kThreads>(*reinterpret_cast<SelectShared<kThreads>*>(fused_lds), p, x, M, 0, pb, kept, pos, n);
}
// Steps 4-7 only, from chunk masses already in the LDS.
__device__ __attribute__((noinline)) inline void fused_select_ranked(SelectParamsDev p, int M, int pb, int32_t* kept,
                                                                     int32_t* pos, int32_t* n) {
    select_ranked<kThreads>(*reinterpret_cast<SelectShared<kThreads>*>(fused_lds), p, M, 0, pb, kept, pos, n);
}

// The streaming workgroups' end of a fused launch. Without sel_dist the
// workgroup raises a tagged flag once its scores are written. With it, the
// workgroup publishes the min and max of the scores it wrote (complete before
// the words), waits for every workgroup's, and sums the fixed-point masses of
// chunks sw, sw + nstream, ... (sw = its index) over the scores (every token's
// value and boosts as the selection computes them; the sums are exact, so the
// split does not change them), each chunk's mass stored as two tagged words.
__device__ __forceinline__ void fused_tail(const ScoreArgs& a, float smn, float smx, int snf, int nstream,
                                           const int bid) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    __shared__ float mm[2 * kWaves];
    __shared__ float gmm[2];
    __shared__ int gbad;
    const unsigned long long Et = (unsigned long long)a.epoch << 32;
    if (!a.sel_dist) {
        // (the selecting workgroup does every step: it only needs to know
        // that the scores are written)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) st64u(a.done + 2 * bid, Et | a.epoch);
        return;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        smn = fminf(smn, __shfl_xor(smn, o));
        smx = fmaxf(smx, __shfl_xor(smx, o));
    }
    if (lane == 0) {
        mm[w] = smn;
        mm[kWaves + w] = smx;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's scores are written
    const bool nf = __syncthreads_or(snf);
    if (tid == 0) {
        float m0 = mm[0], m1 = mm[kWaves];
        for (int x = 1; x < kWaves; ++x) {
            m0 = fminf(m0, mm[x]);
            m1 = fmaxf(m1, mm[kWaves + x]);
        }
        st64u(a.done + 2 * bid, Et | __float_as_uint(m0));
        st64u(a.done + 2 * bid + 1, Et | (nf ? kNonFiniteMark : __float_as_uint(m1)));
    }
    const int chunk = a.selp.chunk;
    const int nc = (a.M + chunk - 1) / chunk;
    const int sw = bid;
    const int nj = sw < nc ? (nc - sw + nstream - 1) / nstream : 0;  // this workgroup's chunks
    if (nj == 0) return;
    if (w == 0) {
        // every workgroup's min and max; lane x watches workgroups x, x + 64, ...
        float gmn = INFINITY, gmx = -INFINITY;
        bool bad = false;
        const unsigned long long t0 = wall_clock64();
        while (true) {
            bool miss = false, nfx = false;
            gmn = INFINITY;
            gmx = -INFINITY;
            for (int x = lane; x < nstream; x += 64) {
                const unsigned long long lo = ld64(a.done + 2 * x), hi = ld64(a.done + 2 * x + 1);
                miss |= !(tag_is(lo, a.epoch) && tag_is(hi, a.epoch));
                nfx |= (unsigned)hi == kNonFiniteMark;
                gmn = fminf(gmn, tag_value(lo));
                gmx = fmaxf(gmx, tag_value(hi));
            }
            if (__ballot(miss) == 0) {
                bad = __ballot(nfx) != 0;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            if (wait_expired(t0, a)) {
                if (lane == 0) set_err(a);
                bad = true;
                break;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            gmn = fminf(gmn, __shfl_xor(gmn, o));
            gmx = fmaxf(gmx, __shfl_xor(gmx, o));
        }
        if (lane == 0) {
            gmm[0] = gmn;
            gmm[1] = gmx;
            gbad = bad ? 1 : 0;
        }
    }
    __syncthreads();
    if (gbad) return;  // (the selecting workgroup reports it)
    MinMaxNorm nm;
    nm.init(gmm[0], gmm[1]);
    unsigned long long* sums = fused_lds;  // (the launch's dynamic LDS: its K slots are free now)
    constexpr int kB = 256;  // chunks per batch
    for (int jb = 0; jb < nj; jb += kB) {
        const int nb = min(kB, nj - jb);
        for (int t = tid; t < nb; t += kThreads) sums[t] = 0ull;
        __syncthreads();
        for (int f = tid; f < nb * chunk; f += kThreads) {
            const int j = f / chunk, e = f - j * chunk;
            const int i = (sw + (jb + j) * nstream) * chunk + e;
            // (agent-scope loads see the other workgroups' scores; an acquire
            // fence in every workgroup instead costs more than the loads)
            if (i < a.M)
                atomicAdd(&sums[j], token_mass(nm.value(__uint_as_float(ld32(a.importance + i))), i, a.M, a.selp));
        }
        __syncthreads();
        for (int t = tid; t < nb; t += kThreads) {
            const unsigned long long v = sums[t];
            unsigned long long* sl = a.sel_sums + 2 * (sw + (jb + t) * nstream);
            st64u(sl, Et | (unsigned)v);
            st64u(sl + 1, Et | (unsigned)(v >> 32));
        }
        __syncthreads();  // (sums is rewritten by the next batch)
    }
}

// SEL: the fused launch (sp_score_select), which also selects from the scores.
// A: ScoreArgs (one request per launch: workgroup b of the grid is the
// request's workgroup b) or PackArgs (several requests per launch, request r
// on blocks [first[r], first[r + 1]) with its own workgroups, combiners and
// workspace: the requests share nothing; not with SEL).
template <class C, bool SEL, class A>
__global__ __launch_bounds__(kThreads, 1) void score_kernel(A karg) {
    // this workgroup's request, its index among the request's workgroups, and
    // their count (-1: the whole grid, read where it is used rather than kept
    // live)
    int bid = (int)blockIdx.x, nblocks = -1;
    const ScoreArgs* ap;
    if constexpr (std::is_same<A, PackArgs>::value) {
        static_assert(!SEL, "the fused selection scores one request per launch");
        int r = 0;
        for (int i = 1; i < karg.n; ++i) r = bid >= karg.first[i] ? i : r;
        ap = &karg.args[r];
        nblocks = karg.first[r + 1] - karg.first[r];
        bid -= karg.first[r];
    } else {
        ap = &karg;
    }
    const ScoreArgs& a = *ap;
    constexpr int TPW = C::TPW, NH = C::NH, ROWS = C::ROWS, G = C::G, NLD = C::NLD;
    constexpr int SW = kStreamWaves;  // waves 0..SW-1 stream K; wave SW synchronises
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform across the wave: say so, so that everything
    // derived from it stays in scalar registers and branches
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;  // lane group
    const float c = a.c;
    const int nstream = a.g * a.ngroups;
    // (the workspace remembers the last call's epoch, for the status query)
    if (bid == 0 && tid == 0)
        __hip_atomic_store(a.hdr, a.call_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---------------------------------------------------------------------------
    // Combiner workgroups: for units cw, cw + ncw, ... wait until the g
    // partials of this launch are published (both words of a slot carry its
    // epoch), combine them (the last slice's partial includes the look-ahead
    // keys) and publish each row's log-sum-exp. Lane L handles row L % ROWS
    // for ranks L / ROWS, L / ROWS + SUBS, ... in batches of B.
    // ---------------------------------------------------------------------------
    if (bid >= nstream) {
        const int cg = bid - nstream, ncg = (nblocks < 0 ? (int)gridDim.x : nblocks) - nstream;
        float2* cred = (float2*)smem;  // [kWaves][ROWS]
        constexpr int SUBS = 64 / ROWS;
        constexpr int B = kCombinerBatch;  // ranks polled per lane at once
        const int row = lane % ROWS, sub = lane / ROWS;
        const unsigned E = a.epoch;
        // Teams of wpu waves share a unit: each wave gathers at most SUBS * B
        // ranks [k_lo, k_hi) in one batch, and the team's first wave combines
        // the team's results through LDS. wpu grows while enough units can
        // still be gathered at once (two steps' worth: 2 * ngroups).
        const int need_w = (a.g + SUBS * B - 1) / (SUBS * B);
        int wpu = 1;
        while (wpu < kWaves && (wpu < need_w || ncg * (kWaves / (2 * wpu)) >= 2 * a.ngroups)) wpu *= 2;
        const int teams = kWaves / wpu, team = w / wpu, wt = w % wpu;
        const int per = (a.g + wpu - 1) / wpu;
        const int k_lo = min(wt * per, a.g), k_hi = min(k_lo + per, a.g);
        for (int ub = cg * teams; ub < a.units; ub += ncg * teams) {
            const int u = ub + team;  // (past the last unit: barriers only)
            float m = -INFINITY, s = 0.f;
            // (row max, row sum) words of rank k at slot + 2 k ROWS, + 1
            const unsigned long long* slot = a.part + ((size_t)u * a.g * ROWS + row) * 2;
            const unsigned long long t0 = wall_clock64();
            if (u < a.units && k_lo < k_hi) {
                // Until this wave's partials start to appear, watch one slot
                // (the sum word of its last rank's first row) instead of
                // re-polling all of them: the combiner CUs' memory queues stay short.
                const unsigned long long* gate = a.part + (((size_t)u * a.g + k_hi - 1) * ROWS) * 2 + 1;
                while (!tag_is(ld64(gate), E)) {
                    __builtin_amdgcn_s_sleep(8);
                    if (wait_expired(t0, a)) {
                        if (lane == 0) set_err(a);
                        break;
                    }
                }
                const int k0 = k_lo + sub;
                unsigned long long vm[B], vs[B];
                unsigned long long pend = 0;  // bit x: rank k0 + SUBS x not seen yet
    #pragma unroll
                for (int x = 0; x < B; ++x) {
                    vm[x] = vs[x] = 0ull;
                    if (k0 + SUBS * x < k_hi) pend |= 1ull << x;
                }
                while (true) {
    #pragma unroll
                    for (int x = 0; x < B; ++x)
                        if ((pend >> x) & 1) {
                            const unsigned long long* sl = slot + (size_t)(k0 + SUBS * x) * ROWS * 2;
                            vm[x] = ld64(sl);
                            vs[x] = ld64(sl + 1);
                        }
                    unsigned long long np = 0;
    #pragma unroll
                    for (int x = 0; x < B; ++x)
                        if (((pend >> x) & 1) && !(tag_is(vm[x], E) && tag_is(vs[x], E))) np |= 1ull << x;
                    pend = np;
                    if (__ballot(pend != 0) == 0) break;
                    __builtin_amdgcn_s_sleep(2);
                    if (wait_expired(t0, a)) {
                        if (lane == 0) set_err(a);
                        break;
                    }
                }
                float mx = -INFINITY;
    #pragma unroll
                for (int x = 0; x < B; ++x)
                    if (k0 + SUBS * x < k_hi && !((pend >> x) & 1)) mx = fmaxf(mx, tag_value(vm[x]));
                if (mx != -INFINITY) {
                    float acc = 0.f;
    #pragma unroll
                    for (int x = 0; x < B; ++x)
                        if (k0 + SUBS * x < k_hi && !((pend >> x) & 1))
                            acc = fmaf(tag_value(vs[x]), exp2_hw((tag_value(vm[x]) - mx) * c), acc);
                    m = mx;
                    s = acc;
                }
                if constexpr (SUBS == 4) combine(m, s, __shfl_xor(m, 16), __shfl_xor(s, 16), c);
                combine(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32), c);
            }
            if (sub == 0) cred[w * ROWS + row] = make_float2(m, s);
            __syncthreads();
            if (u < a.units && wt == 0 && lane < ROWS) {
                float mm = -INFINITY, ss = 0.f;
                for (int x = 0; x < wpu; ++x)
                    combine(mm, ss, cred[(team * wpu + x) * ROWS + lane].x, cred[(team * wpu + x) * ROWS + lane].y, c);
                // (two tagged copies: a slot is taken only when both words carry the epoch)
                const unsigned long long v = tagged(mm * c + log2_hw(ss), E);
                st64u(a.lse + ((size_t)u * ROWS + lane) * 2, v);
                st64u(a.lse + ((size_t)u * ROWS + lane) * 2 + 1, v);
            }
            __syncthreads();  // (cred is rewritten for the next unit)
        }
        if (SEL && cg == ncg - 1) {
            // Fused selection, once every streaming workgroup has written its
            // scores (each raises a tagged flag). When the streaming
            // workgroups sum the chunks' fixed-point masses between them
            // (sel_dist: min-max normalisation, long prompts; exact integers,
            // so the split does not change them), the flag is the min and max
            // of the workgroup's scores (or a mark that one is not finite),
            // and this workgroup gathers the masses and ranks; otherwise it
            // runs every step itself on the scores (an agent-scope acquire
            // makes them visible to this CU's plain loads). Either way on the
            // LDS the combiner no longer needs.
            bool expired = false, nonfinite = false;
            if (w == 0) {
                const unsigned long long t0 = wall_clock64();
                while (true) {
                    bool miss = false, nf = false;
                    if (a.sel_dist) {
                        for (int x = lane; x < nstream; x += 64) {
                            const unsigned long long lo = ld64(a.done + 2 * x), hi = ld64(a.done + 2 * x + 1);
                            miss |= !(tag_is(lo, a.epoch) && tag_is(hi, a.epoch));
                            nf |= (unsigned)hi == kNonFiniteMark;
                        }
                    } else {
                        // (the scores' own check finds non-finite ones)
                        const unsigned long long mark = ((unsigned long long)a.epoch << 32) | a.epoch;
                        for (int x = lane; x < nstream; x += 64) miss |= ld64(a.done + 2 * x) != mark;
                    }
                    if (__ballot(miss) == 0) {
                        nonfinite = __ballot(nf) != 0;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    if (wait_expired(t0, a)) {
                        if (lane == 0) set_err(a);
                        expired = true;
                        break;
                    }
                }
            }
            if (__syncthreads_or(expired || nonfinite) || err_set(a)) {
                // (scores missing, poisoned or not finite: no selection)
                if (tid == 0) *a.sel_n = -1;
                return;
            }
            if (a.sel_dist) {
                SelectShared<kThreads>& sh = *reinterpret_cast<SelectShared<kThreads>*>(fused_lds);
                const int nc = (a.M + a.selp.chunk - 1) / a.selp.chunk;
                constexpr int P = kSelMaxChunks / kThreads;  // chunks per thread
                unsigned long long lo[P], hi[P];
                unsigned pend = 0;  // bit e: chunk tid + e * kThreads not seen yet
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    lo[e] = hi[e] = 0ull;
                    if (tid + e * kThreads < nc) pend |= 1u << e;
                }
                const unsigned long long t0 = wall_clock64();
                while (true) {
#pragma unroll
                    for (int e = 0; e < P; ++e)
                        if ((pend >> e) & 1) {
                            const unsigned long long* sl = a.sel_sums + 2 * (tid + e * kThreads);
                            lo[e] = ld64(sl);
                            hi[e] = ld64(sl + 1);
                        }
                    unsigned np = 0;
#pragma unroll
                    for (int e = 0; e < P; ++e)
                        if (((pend >> e) & 1) && !(tag_is(lo[e], a.epoch) && tag_is(hi[e], a.epoch))) np |= 1u << e;
                    pend = np;
                    if (__ballot(pend != 0) == 0) break;
                    __builtin_amdgcn_s_sleep(2);
                    if (wait_expired(t0, a)) {
                        if (lane == 0) set_err(a);
                        expired = true;
                        break;
                    }
                }
#pragma unroll
                for (int e = 0; e < P; ++e)
                    if (tid + e * kThreads < nc)
                        sh.C[tid + e * kThreads] = (unsigned long long)(unsigned)lo[e] | (hi[e] << 32);
                if (__syncthreads_or(expired) || err_set(a)) {
                    if (tid == 0) *a.sel_n = -1;
                    return;
                }
                fused_select_ranked(a.selp, a.M, a.sel_pos_base, a.sel_kept, a.sel_pos, a.sel_n);
            } else {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                fused_select(a.selp, a.importance, a.M, a.sel_pos_base, a.sel_kept, a.sel_pos, a.sel_n);
            }
        }
        return;
    }

    // ---------------------------------------------------------------------------
    // Streaming workgroups.
    // ---------------------------------------------------------------------------
    const int group = bid / a.g, rank = bid % a.g;
    const int KRP = row_stride(a.KR);
    // With K by DMA, the regions other than the K slots live in an array of
    // their own, so that the compiler can tell the waves' LDS stores there from
    // the DMA writes in flight (it would otherwise wait for every load before
    // each store).
    constexpr int kMiscQ = 0, kMiscRed = kMiscQ + 2 * ROWS * C::QS,
                  kMiscRef = kMiscRed + 2 * SW * ROWS * 8,
                  kMiscLse = kMiscRef + (kMaxDefer + 1) * SW * ROWS * 4,
                  kMiscBytes = kMiscLse + 2 * ROWS * 4;
    __shared__ __attribute__((aligned(16))) char misc_lds[C::DMA ? kMiscBytes : 16];
    int* Trun = (int*)(smem + a.lds.trun);  // running maxima at the end (over the parked banks)
    float2* red = (float2*)(C::DMA ? misc_lds + kMiscRed : smem + a.lds.red);   // [2][SW][ROWS]
    float* lse_s = (float*)(C::DMA ? misc_lds + kMiscLse : smem + a.lds.lse);   // [2][ROWS]
    float* refs = (float*)(C::DMA ? misc_lds + kMiscRef : smem + a.lds.ref);    // [nbk][SW][ROWS]
    char* qlds = C::DMA ? misc_lds + kMiscQ : smem + a.lds.q;                  // [2][ROWS][QS]
    char* banks = smem + a.lds.bank;                // [nbk][SW][TPW][64][NH][8 B]

    // The slices cover the prompt keys and then the tail_n look-ahead keys
    // (the last slice holds these): look-ahead key M + i counts in the
    // softmax of steps j >= i only. nall: keys of the slice every step sees;
    // nout: prompt keys of the slice (the ones that get scores).
    const int r0 = rank * a.KR;
    const int r1 = min(r0 + a.KR, a.M + a.tail_n);
    const int nkeys = max(r1 - r0, 0);
    const int nall = max(min(r1, a.M + 1) - r0, 0);
    const int nout = max(min(r1, a.M) - r0, 0);
    const int ntiles = (nkeys + kTileKeys - 1) / kTileKeys;
    const uint32_t plane_bytes = (uint32_t)(a.M + a.N) * (uint32_t)C::KB;
    const int D = a.defer, nbk = a.nbk;
    const int n_units = group < a.units ? (a.units - group + a.ngroups - 1) / a.ngroups : 0;
    // even: the register-ring loop is unrolled by 2; the DMA loop by its banks (4)
    const int n_steps = C::DMA ? (n_units + D + 3) & ~3 : (n_units + D + 1) & ~1;
    auto unit_of = [&](int it) __attribute__((always_inline)) { return it >= 0 && it < n_units ? group + it * a.ngroups : -1; };

    // Per-lane query rows of the halves: the look-ahead step of each
    int jrow[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) jrow[hf] = (hf * 16 + (lane & 15)) / G;

    if (w < SW) {
        if constexpr (C::DMA) {
        // ============= streaming waves: K tiles by DMA into LDS =============
        // The tiles of the next unit travel HBM -> LDS (buffer loads with the
        // lds modifier: no registers, non-temporal), each load instruction
        // covering whole 128-byte lines of consecutive key rows; a tile is
        // stored with its 16-byte chunks XOR-swizzled by row, so that the
        // MFMA-layout reads (16 rows x one chunk column) hit every bank once.
        // Each wave streams its tiles q = it * TPW + t through S LDS slots
        // (tile q in slot q % S); a slot is refilled with tile q + S as soon
        // as tile q's reads are done, so S - 1 tiles are always in flight and
        // the outstanding load count before every tile is the same. With the
        // step loop unrolled by NB (a multiple of S), slots and refills are
        // compile-time constants. Parked logits stay in registers (NB banks),
        // and the per-step barrier waits for LDS only, never for the loads in
        // flight.
        constexpr int TB = kTileKeys * C::KB;  // bytes of one 16-key tile
        constexpr int CPR = C::KB / 16;         // 16-byte chunks per key row
        constexpr int RPI = 64 / CPR;           // key rows one load instruction covers
        constexpr int SWZ = 16 / CPR;           // rows sharing one 64-bank line
        constexpr int NB = kMaxDefer + 1;       // register banks of parked logits
        constexpr int S = C::S;                 // LDS slots of this wave
        constexpr int VM_AHEAD = (S - 1) * NLD; // loads issued after a tile's own
        static_assert(RPI * NLD == kTileKeys, "tile load shape");
        static_assert((S <= TPW && NB % S == 0) || S == TPW, "slots must be static in the unrolled loop");
        char* ring = smem + a.lds.bank + (size_t)w * S * TB;
        const int ntv = min(max((ntiles - w + SW - 1) / SW, 0), TPW);
        const int tpart = masked_tile(ntv, w, nall);
        const int tile_p = w + SW * max(tpart, 0);  // (its index in the slice)
        const bool full = tpart < 0 && ntv == TPW;
        // DMA side: the lane's byte offset in a tile for load s (row RPI s + lane / CPR,
        // the chunk that lands in LDS column lane % CPR); read side: the LDS offset
        // of row lane % 16, k-step s (chunk 4 s + lane / 16)
        uint32_t loff[NLD];
        int roff[NLD];
#pragma unroll
        for (int s = 0; s < NLD; ++s) {
            const int row = RPI * s + lane / CPR, col = lane % CPR;
            loff[s] = (uint32_t)(row * C::KB + ((col ^ ((row / SWZ) % CPR)) * 16));
            const int r2 = lane & 15, ch = 4 * s + g4;
            roff[s] = r2 * C::KB + ((ch ^ ((r2 / SWZ) % CPR)) * 16);
        }
        uint32_t tbo[TPW];  // byte offset of tile t in the plane (past the slice: out of range, zeros)
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            tbo[t] = t < ntv ? (uint32_t)(r0 + (w + SW * t) * kTileKeys) * (uint32_t)C::KB : kOob;
        // tile t of a unit (plane rs) into LDS slot sl
        auto issue_tile = [&](__amdgpu_buffer_rsrc_t rs, int t, int sl) __attribute__((always_inline)) {
#pragma unroll
            for (int s = 0; s < NLD; ++s) dma_load16(rs, ring + sl * TB + s * 1024, loff[s], tbo[t]);
        };

        constexpr int NHF = G == 32 ? 1 : NH;
        constexpr bool kRoomy = NB * TPW * NH * 2 + NH * NLD * 4 + NLD * 4 + TPW * NH * 4 <= 176;
        constexpr int SGL = C::GL >= 2 && !kRoomy ? 2 : 1;
        constexpr int KEEP = 4 / SGL;
        int trun[TPW][NHF][KEEP];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
                for (int kk = 0; kk < KEEP; ++kk) trun[t][hf][kk] = kNegInf;
        const bool lb0 = (lane & 1) != 0;

        int park[NB][TPW][2 * NH];  // parked logits of the last NB units (16-bit codes, 2 per word)
        f32x4 acc[TPW][NH];
        {
            // tiles 0..S-1 (of unit 0) into slots 0..S-1
            const auto rs = plane_rsrc(a, unit_of(0), plane_bytes, C::ESZ);
#pragma unroll
            for (int t = 0; t < S; ++t) issue_tile(rs, t, t);
        }
        step_barrier<C>();  // Q of unit 0 is staged

        auto stream = [&](auto Pc, auto Bc, int it) __attribute__((always_inline)) {
            constexpr int P = decltype(Pc)::value, B = decltype(Bc)::value;
            i32x4 qf[NH][NLD];
#pragma unroll
            for (int hf = 0; hf < NH; ++hf)
#pragma unroll
                for (int s = 0; s < NLD; ++s)
                    qf[hf][s] = *(const i32x4*)(qlds + (P * ROWS + hf * 16 + (lane & 15)) * C::QS + 16 * g4 + 64 * s);
            const auto rs0 = plane_rsrc(a, unit_of(it), plane_bytes, C::ESZ);
            const auto rs1 = plane_rsrc(a, unit_of(it + 1), plane_bytes, C::ESZ);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                // tile q = it TPW + t sits in slot q % S; (it % NB = B is static)
                const int sl = (B * TPW + t) % S;
                __builtin_amdgcn_s_waitcnt(vm_wait(VM_AHEAD));  // this tile's loads have landed
                i32x4 kf[NLD];
#pragma unroll
                for (int s = 0; s < NLD; ++s) kf[s] = *(const i32x4*)(ring + sl * TB + roff[s]);
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) acc[t][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NLD; ++s)
#pragma unroll
                    for (int hf = 0; hf < NH; ++hf) mma<C>(acc[t][hf], qf[hf][s], kf[s]);
                // the slot's reads are done: refill it with tile q + S (tile
                // (t + S) % TPW of this unit or the next)
                __builtin_amdgcn_s_waitcnt(kLgkmWait0);
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                issue_tile(t + S < TPW ? rs0 : rs1, (t + S) % TPW, sl);
            }
            // per wave-row statistics over this wave's keys of the slice (as in
            // the register-ring variant) and the shifted log2 logits in acc
            auto stats = [&](auto FullC) __attribute__((always_inline)) {
                constexpr bool FULL = decltype(FullC)::value;
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    float m = -INFINITY;
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        float mt = fmaxf(fmaxf(acc[t][hf][0], acc[t][hf][1]), fmaxf(acc[t][hf][2], acc[t][hf][3]));
                        if constexpr (FULL) {
                            m = fmaxf(m, mt);
                        } else {
                            if (t == tpart) {
                                // keys of the tile this lane's rows see (4 g4 + r < lim)
                                int lim = visible_keys(a, r0, r1, (hf * 16 + (lane & 15)) / G, tile_p);
                                asm volatile("" : "+v"(lim));
                                mt = -INFINITY;
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (r < lim) mt = fmaxf(mt, acc[t][hf][r]);
                            }
                            if (t < ntv) m = fmaxf(m, mt);
                        }
                    }
                    m = xor16_max(m);
                    m = xor32_max(m);
                    const float cm = m == -INFINITY ? 0.f : m * c;
                    float s = 0.f;
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        float e[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float y = fmaf(acc[t][hf][r], c, -cm);
                            acc[t][hf][r] = y;
                            e[r] = exp2_hw(y);
                        }
                        float st = (e[0] + e[1]) + (e[2] + e[3]);
                        if constexpr (FULL) {
                            s += st;
                        } else {
                            if (t == tpart) {
                                // keys of the tile this lane's rows see (4 g4 + r < lim)
                                int lim = visible_keys(a, r0, r1, (hf * 16 + (lane & 15)) / G, tile_p);
                                asm volatile("" : "+v"(lim));
                                st = 0.f;
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (r < lim) st += e[r];
                            }
                            if (t < ntv) s += st;
                        }
                    }
                    s = xor16_sum(s);
                    s = xor32_sum(s);
                    if (g4 == 0) {
                        lds_store_f2(&red[(P * SW + w) * ROWS + hf * 16 + lane], make_float2(m, s));
                        lds_store_f1(&refs[(B * SW + w) * ROWS + hf * 16 + lane], cm);
                    }
                }
            };
            if (full) stats(std::true_type{});
            else stats(std::false_type{});
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    constexpr float k = -1.f / kCodeRange;
                    park[B][t][2 * hf] = pack_u2(acc[t][hf][0] * k, acc[t][hf][1] * k);
                    park[B][t][2 * hf + 1] = pack_u2(acc[t][hf][2] * k, acc[t][hf][3] * k);
                }
        };

        // finish the unit parked in register bank BF (log-sum-exps in lse_s[pb])
        auto finish = [&](auto BFc, int pb) __attribute__((always_inline)) {
            constexpr int BF = decltype(BFc)::value;
            int off[NH];
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
                const int row = hf * 16 + (lane & 15);
                off[hf] = offset_steps(refs[(BF * SW + w) * ROWS + row] - lse_s[pb * ROWS + row]);
            }
#pragma unroll
            for (int hf = 0; hf < NHF; ++hf) {
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    int y[4], y1[4];
                    unpack_v2(park[BF][t][2 * hf], off[hf], y[0], y[1]);
                    unpack_v2(park[BF][t][2 * hf + 1], off[hf], y[2], y[3]);
                    if constexpr (G == 32) {
                        unpack_v2(park[BF][t][2], off[1], y1[0], y1[1]);
                        unpack_v2(park[BF][t][3], off[1], y1[2], y1[3]);
                    }
                    int v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        int x = y[r];
                        if constexpr (G == 32) x = max(x, y1[r]);
                        v[r] = group_max16<SGL>(x);
                    }
                    if constexpr (KEEP == 2) {
                        trun[t][hf][0] = max(trun[t][hf][0], lb0 ? v[2] : v[0]);
                        trun[t][hf][1] = max(trun[t][hf][1], lb0 ? v[3] : v[1]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) trun[t][hf][r] = max(trun[t][hf][r], v[r]);
                    }
                }
            }
        };

        // step it: stream unit it into bank it % NB, then (after the barrier,
        // when the control wave has put unit it - 3's log-sum-exps in LDS)
        // finish unit it - 3, parked in bank (it + 1) % NB
        auto step = [&](auto Pc, auto Bc, int it) __attribute__((always_inline)) {
            constexpr int B = decltype(Bc)::value;
            if (it < n_units) stream(Pc, Bc, it);
            step_barrier<C>();
            const int fu = it - kMaxDefer;
            if (fu >= 0 && fu < n_units) finish(std::integral_constant<int, (B + 1) % NB>{}, it & 1);
        };
        for (int it = 0; it < n_steps; it += NB) {
            step(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, it);
            step(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, it + 1);
            step(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, it + 2);
            step(std::integral_constant<int, 1>{}, std::integral_constant<int, 3>{}, it + 3);
        }
        __builtin_amdgcn_s_waitcnt(vm_wait(0));  // the last (empty) refills have landed
        __syncthreads();  // every wave is done with its slots, which Trun overlays
#pragma unroll
        for (int m = SGL; m < C::GL; m <<= 1)
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
                    for (int kk = 0; kk < KEEP; ++kk)
                        trun[t][hf][kk] = max(trun[t][hf][kk], __shfl_xor(trun[t][hf][kk], m));
        const int kg = (lane & 15) % C::GL;
#pragma unroll
        for (int hf = 0; hf < NHF; ++hf)
            if (jrow[hf] < a.N && kg < SGL) {
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    if (t >= ntv) break;
                    int* rowp = Trun + jrow[hf] * KRP + (w + SW * t) * kTileKeys + 4 * g4;
                    if constexpr (KEEP == 2) {
                        rowp[2 * (lane & 1)] = trun[t][hf][0];
                        rowp[2 * (lane & 1) + 1] = trun[t][hf][1];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) rowp[r] = trun[t][hf][r];
                    }
                }
            }
        } else {
        // ======================= streaming waves =======================
        // This wave's tiles w, w + SW, ...: the first ntv hold keys of the
        // slice (the rest are read as zeros and masked); when the slice ends
        // inside tile tpart, that tile's keys past the end are masked too.
        const int ntv = min(max((ntiles - w + SW - 1) / SW, 0), TPW);
        const int tpart = masked_tile(ntv, w, nall);
        const int tile_p = w + SW * max(tpart, 0);  // (its index in the slice)
        const bool full = tpart < 0 && ntv == TPW;  // every tile of this wave inside the slice
        uint32_t koff[TPW];  // buffer offset of this lane's first load of tile t
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            koff[t] = t < ntv ? (uint32_t)(r0 + (w + SW * t) * kTileKeys + (lane & 15)) * (uint32_t)C::KB +
                                    (uint32_t)(16 * g4)
                              : kOob;
        // key plane of unit it + 2 for the refill in step it (advanced by one
        // group stride per step)
        const long long ustep = (long long)a.ngroups * a.plane_stride * C::ESZ;
        const char* kb2 = (const char*)a.K + ((long long)group + 2ll * a.ngroups) * a.plane_stride * C::ESZ;
        asm volatile("" : "+s"(kb2));  // a pointer of its own, not recomputed from a.K in the loop

        // Running max over units, in registers. The max over heads commutes
        // with the max over units, so it is taken once, at the end, where the
        // registers allow: each lane keeps the running maxima of its own query
        // row for its 4 keys (C rows r = 0..3). Where the ring and the
        // accumulators leave no room for that, each step takes the head max
        // over lane pairs (heads 2m, 2m + 1: one DPP max) and lane k keeps
        // keys 2 (k % 2) and 2 (k % 2) + 1 of its pair.
        constexpr int NHF = G == 32 ? 1 : NH;  // G = 32: both halves hold the one step
        constexpr bool kRoomy = score_roomy(C::KB, TPW, NH);  // registers left by K ring + accumulators
        constexpr int SGL = C::GL >= 2 && !kRoomy ? 2 : 1;
        constexpr int KEEP = 4 / SGL;
        int trun[TPW][NHF][KEEP];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
                for (int kk = 0; kk < KEEP; ++kk) trun[t][hf][kk] = kNegInf;
        const bool lb0 = (lane & 1) != 0;

        Frag<C> fb[C::NBUF];
        f32x4 acc[TPW][NH];
        // prime the ring with the first two units
#pragma unroll
        for (int P = 0; P < 2; ++P) {
            const auto rs = plane_rsrc(a, unit_of(P), plane_bytes, C::ESZ);
#pragma unroll
            for (int t = 0; t < TPW; ++t) load_k<C>(fb[P * TPW + t], rs, koff[t]);
        }
        __syncthreads();  // Q of unit 0 is staged

        // Stream unit `it` (ring slots of parity P), park its logits in bank
        // b and its per-row statistics in red[P].
        auto stream = [&](auto Pc, int it, int b) __attribute__((always_inline)) {
            constexpr int P = decltype(Pc)::value;
            // k-outer: for each 16-byte k-slice, this unit's Q fragments of both
            // halves come from LDS, then every tile's MFMAs consume them
            const auto rs2 = make_rsrc(kb2, it + 2 < n_units ? plane_bytes : 0u);
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) acc[t][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NLD; ++s) {
                i32x4 q[NH];
#pragma unroll
                for (int hf = 0; hf < NH; ++hf)
                    q[hf] = *(const i32x4*)(qlds + (P * ROWS + hf * 16 + (lane & 15)) * C::QS + 16 * g4 + 64 * s);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int hf = 0; hf < NH; ++hf) mma<C>(acc[t][hf], q[hf], fb[P * TPW + t].v[s]);
            }
            // refill the slots with the same tiles of the unit two ahead
#pragma unroll
            for (int t = 0; t < TPW; ++t) load_k<C>(fb[P * TPW + t], rs2, koff[t]);
            // Per wave-row statistics over this wave's keys of the slice (lanes
            // L, L^16, L^32, L^48 hold the same row): the max m, the shifted
            // log2 logits y = c x - c m (<= 0 on those keys) and their exp2
            // sum. When the slice does not fill this wave's tiles (!FULL),
            // tiles t >= ntv are left out by wave-uniform selects and the keys
            // of tile tpart past the slice's end by per-lane masks in a branch
            // only that tile's wave takes; waves whose tiles are all full take
            // a copy without either. The logits themselves are not masked:
            // what is parked for keys outside the slice is never written out.
            auto stats = [&](auto FullC) __attribute__((always_inline)) {
                constexpr bool FULL = decltype(FullC)::value;
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    float m = -INFINITY;
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        float mt = fmaxf(fmaxf(acc[t][hf][0], acc[t][hf][1]), fmaxf(acc[t][hf][2], acc[t][hf][3]));
                        if constexpr (FULL) {
                            m = fmaxf(m, mt);
                        } else {
                            if (t == tpart) {
                                // keys of the tile this lane's rows see (4 g4 + r < lim)
                                int lim = visible_keys(a, r0, r1, (hf * 16 + (lane & 15)) / G, tile_p);
                                asm volatile("" : "+v"(lim));  // keep the per-lane compares in this branch
                                mt = -INFINITY;
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (r < lim) mt = fmaxf(mt, acc[t][hf][r]);
                            }
                            if (t < ntv) m = fmaxf(m, mt);
                        }
                    }
                    m = xor16_max(m);
                    m = xor32_max(m);
                    const float cm = m == -INFINITY ? 0.f : m * c;
                    float s = 0.f;
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        float e[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float y = fmaf(acc[t][hf][r], c, -cm);
                            acc[t][hf][r] = y;
                            e[r] = exp2_hw(y);
                        }
                        float st = (e[0] + e[1]) + (e[2] + e[3]);
                        if constexpr (FULL) {
                            s += st;
                        } else {
                            if (t == tpart) {
                                // keys of the tile this lane's rows see (4 g4 + r < lim)
                                int lim = visible_keys(a, r0, r1, (hf * 16 + (lane & 15)) / G, tile_p);
                                asm volatile("" : "+v"(lim));
                                st = 0.f;
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (r < lim) st += e[r];
                            }
                            if (t < ntv) s += st;
                        }
                    }
                    s = xor16_sum(s);
                    s = xor32_sum(s);
                    if (g4 == 0) {
                        red[(P * SW + w) * ROWS + hf * 16 + lane] = make_float2(m, s);
                        refs[(b * SW + w) * ROWS + hf * 16 + lane] = cm;
                    }
                }
            };
            if constexpr (kRoomy) {
                if (full) stats(std::true_type{});
                else stats(std::false_type{});
            } else {
                stats(std::false_type{});  // (no registers for a second copy)
            }
            // park the shifted logits: 4 halves per (tile, half), NH*8 bytes per lane
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                int* dst = (int*)(banks + ((size_t)((b * SW + w) * TPW + t) * 64 + lane) * (NH * 8));
                int wd[2 * NH];
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    constexpr float k = -1.f / kCodeRange;
                    wd[2 * hf] = pack_u2(acc[t][hf][0] * k, acc[t][hf][1] * k);
                    wd[2 * hf + 1] = pack_u2(acc[t][hf][2] * k, acc[t][hf][3] * k);
                }
                if constexpr (NH == 2) *(int4*)dst = make_int4(wd[0], wd[1], wd[2], wd[3]);
                else *(int2*)dst = make_int2(wd[0], wd[1]);
            }
        };

        // Finish the unit parked in bank b (its log-sum-exps in lse_s[pb]):
        // log2 probabilities, max over the G heads of each step, running max
        // over units in LDS. Only this wave's first ntv tiles are updated; keys
        // of tile tpart past the slice's end land in columns that are never
        // written out.
        auto finish = [&](int b, int pb) __attribute__((always_inline)) {
            int off[NH];  // row offsets in whole steps
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
                const int row = hf * 16 + (lane & 15);
                off[hf] = offset_steps(refs[(b * SW + w) * ROWS + row] - lse_s[pb * ROWS + row]);
            }
            int wd[TPW][2 * NH];
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int* src = (const int*)(banks + ((size_t)((b * SW + w) * TPW + t) * 64 + lane) * (NH * 8));
                if constexpr (NH == 2) {
                    const int4 q4 = *(const int4*)src;
                    wd[t][0] = q4.x;
                    wd[t][1] = q4.y;
                    wd[t][2] = q4.z;
                    wd[t][3] = q4.w;
                } else {
                    const int2 q2 = *(const int2*)src;
                    wd[t][0] = q2.x;
                    wd[t][1] = q2.y;
                }
            }
#pragma unroll
            for (int hf = 0; hf < NHF; ++hf) {
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    int y[4], y1[4];  // log2 probabilities in steps (y1: the other half, G = 32)
                    unpack_v2(wd[t][2 * hf], off[hf], y[0], y[1]);
                    unpack_v2(wd[t][2 * hf + 1], off[hf], y[2], y[3]);
                    if constexpr (G == 32) {
                        unpack_v2(wd[t][2], off[1], y1[0], y1[1]);
                        unpack_v2(wd[t][3], off[1], y1[2], y1[3]);
                    }
                    int v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        int x = y[r];
                        if constexpr (G == 32) x = max(x, y1[r]);
                        v[r] = group_max16<SGL>(x);
                    }
                    if constexpr (KEEP == 2) {
                        trun[t][hf][0] = max(trun[t][hf][0], lb0 ? v[2] : v[0]);
                        trun[t][hf][1] = max(trun[t][hf][1], lb0 ? v[3] : v[1]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) trun[t][hf][r] = max(trun[t][hf][r], v[r]);
                    }
                }
            }
        };

        // Step `it`: stream unit it into bank b, then (after the workgroup
        // barrier, when the control wave has put unit it - D's log-sum-exps in
        // LDS) finish unit it - D, parked in bank (it - D) mod (D + 1), the
        // bank after b.
        int b = 0;
        auto step = [&](auto Pc, int it) __attribute__((always_inline)) {
            if (it < n_units) stream(Pc, it, b);
            kb2 += ustep;
            b = b + 1 == nbk ? 0 : b + 1;
            __syncthreads();
            const int fu = it - D;
            if (fu >= 0 && fu < n_units) finish(b, it & 1);
        };
        for (int it = 0; it < n_steps; it += 2) {
            step(std::integral_constant<int, 0>{}, it);
            step(std::integral_constant<int, 1>{}, it + 1);
        }
        __syncthreads();  // every wave is done with the banks, which Trun overlays
        // the rest of the head max (lanes k and k ^ m of a head group keep the
        // same keys for m >= SGL), then the first SGL lanes of each head group
        // write their kept maxima of the tiles in the slice: row jrow, column
        // tile + 4 g4 + r
#pragma unroll
        for (int m = SGL; m < C::GL; m <<= 1)
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
                    for (int kk = 0; kk < KEEP; ++kk)
                        trun[t][hf][kk] = max(trun[t][hf][kk], __shfl_xor(trun[t][hf][kk], m));
        const int kg = (lane & 15) % C::GL;
#pragma unroll
        for (int hf = 0; hf < NHF; ++hf)
            if (jrow[hf] < a.N && kg < SGL) {
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    if (t >= ntv) break;
                    int* rowp = Trun + jrow[hf] * KRP + (w + SW * t) * kTileKeys + 4 * g4;
                    if constexpr (KEEP == 2) {
                        rowp[2 * (lane & 1)] = trun[t][hf][0];
                        rowp[2 * (lane & 1) + 1] = trun[t][hf][1];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) rowp[r] = trun[t][hf][r];
                    }
                }
            }
        }
    } else {
        // ======================= control wave =======================
        // Its memory instructions are few and latency-critical: they are
        // issued at raised priority (ahead of the streaming waves' refills
        // when the memory pipeline is backed up), the rest of its work at the
        // normal one, so that the streaming wave sharing its SIMD is not held
        // back.
        // Q of one unit: ROWS rows of KB bytes, 16 bytes per lane and load.
        // Two register sets: Q of unit it+1 is stored to LDS at step it from
        // loads issued at step it-2 (the loads of this CU's control wave queue
        // behind its K stream, so they get two steps).
        i32x4 qc[2][C::QLD];
        auto q_issue = [&](auto Sc, int u) __attribute__((always_inline)) {
            constexpr int S = decltype(Sc)::value;
#pragma unroll
            for (int i = 0; i < C::QLD; ++i) {
                const int e = (i * 64 + lane) * 16;
                const int row = e / C::KB, col = e % C::KB;
                const int j = row / G, hl = row % G;
                if (u >= 0 && j < a.N) {
                    const int l = u / a.Hkv, kvh = u % a.Hkv;
                    const long long qrow = ((long long)l * a.H + (long long)kvh * G + hl) * a.N + j;
                    qc[S][i] = *(const i32x4*)((const char*)a.Q + qrow * C::KB + col);
                } else {
                    qc[S][i] = i32x4{0, 0, 0, 0};
                }
            }
        };
        auto q_store = [&](auto Sc, int buf) __attribute__((always_inline)) {
            constexpr int S = decltype(Sc)::value;
#pragma unroll
            for (int i = 0; i < C::QLD; ++i) {
                const int e = (i * 64 + lane) * 16;
                const int row = e / C::KB, col = e % C::KB;
                *(i32x4*)(qlds + (buf * ROWS + row) * C::QS + col) = qc[S][i];
            }
        };
        // log-sum-exps: loads issued kLseAhead steps before they are needed
        // (a unit's log-sum-exps appear a few microseconds after the last of
        // its g workgroups has published; one step later they are there)
        constexpr int kLseAhead = 1;
        unsigned long long lse_v[2][2] = {{0ull, 0ull}, {0ull, 0ull}};
        auto lse_load = [&](auto Sc, int u) __attribute__((always_inline)) {
            constexpr int S = decltype(Sc)::value;
            const unsigned long long* sl = a.lse + ((size_t)u * ROWS + lane) * 2;
            lse_v[S][0] = ld64(sl);
            lse_v[S][1] = ld64(sl + 1);
        };
        auto lse_issue = [&](auto Sc, int u) __attribute__((always_inline)) {
            if (u >= 0 && lane < ROWS) lse_load(Sc, u);
        };
        auto lse_take = [&](auto Sc, int u, int pb) __attribute__((always_inline)) {
            constexpr int S = decltype(Sc)::value;
            auto absent = [&]() __attribute__((always_inline)) {
                return lane < ROWS && !(tag_is(lse_v[S][0], a.epoch) && tag_is(lse_v[S][1], a.epoch));
            };
            bool miss = absent();
            if (__ballot(miss) != 0) {
                const unsigned long long t0 = wall_clock64();
                while (true) {
                    __builtin_amdgcn_s_sleep(2);
                    if (miss) lse_load(Sc, u);
                    miss = absent();
                    if (__ballot(miss) == 0) break;
                    if (wait_expired(t0, a)) {
                        if (lane == 0) set_err(a);
                        break;
                    }
                }
            }
            if (lane < ROWS) lse_s[pb * ROWS + lane] = tag_value(lse_v[S][0]);
        };
        // the workgroup's partial of unit u: combine the streaming waves' rows
        // and publish (row max, row sum), each word tagged with the epoch
        auto publish = [&](int u, int pb) __attribute__((always_inline)) {
            if (lane < ROWS) {
                float mm = red[(pb * SW + 0) * ROWS + lane].x, ss = red[(pb * SW + 0) * ROWS + lane].y;
                for (int x = 1; x < SW; ++x)
                    combine(mm, ss, red[(pb * SW + x) * ROWS + lane].x, red[(pb * SW + x) * ROWS + lane].y, c);
                unsigned long long* sl = a.part + (((size_t)u * a.g + rank) * ROWS + lane) * 2;
                st64u(sl, tagged(mm, a.epoch));
                st64u(sl + 1, tagged(ss, a.epoch));
            }
        };
        // Step it (parity P): take unit it-D's log-sum-exps (loaded kLseAhead
        // steps ago) into lse_s[P]; stage Q of unit it+1 and load Q of unit
        // it+3; after the barrier publish unit it's partial, then load unit
        // it+kLseAhead-D's log-sum-exps (as late as possible in the step, so
        // that they are more likely to be there).
        auto ctrl_step = [&](auto Pc, int it) __attribute__((always_inline)) {
            constexpr int P = decltype(Pc)::value;
            constexpr std::integral_constant<int, P> sp{};
            constexpr std::integral_constant<int, 1 - P> so{};
            constexpr std::integral_constant<int, (P + kLseAhead) & 1> sl{};
            const int fu = it - D;
            if (fu >= 0 && fu < n_units) lse_take(sp, unit_of(fu), P);
            q_store(so, 1 - P);             // Q of unit it+1 -> LDS buffer (it+1)&1
            __builtin_amdgcn_s_setprio(3);
            q_issue(so, unit_of(it + 3));
            __builtin_amdgcn_s_setprio(0);
            step_barrier<C>();
            __builtin_amdgcn_s_setprio(3);
            if (it < n_units) publish(unit_of(it), P);
            lse_issue(sl, unit_of(it + kLseAhead - D));
            __builtin_amdgcn_s_setprio(0);
        };

        // (Q of unit 1 is in flight while unit 0's lands; unit 2's loads are
        // issued after the first barrier, so that the streaming waves, whose
        // first K tiles are already on their way, do not wait for their issue)
        q_issue(std::integral_constant<int, 0>{}, unit_of(0));
        q_issue(std::integral_constant<int, 1>{}, unit_of(1));
        q_store(std::integral_constant<int, 0>{}, 0);
        lse_issue(std::integral_constant<int, 0>{}, unit_of(-D));
        if constexpr (kLseAhead == 2) lse_issue(std::integral_constant<int, 1>{}, unit_of(1 - D));
        step_barrier<C>();
        q_issue(std::integral_constant<int, 0>{}, unit_of(2));
        for (int it = 0; it < n_steps; it += 2) {
            ctrl_step(std::integral_constant<int, 0>{}, it);
            ctrl_step(std::integral_constant<int, 1>{}, it + 1);
        }
        __syncthreads();  // (the streaming waves' barrier before they write the running maxima)
    }
    __syncthreads();
    // The ngroups workgroups of this rank (one per group) hold the running
    // maxima of the same key slice. Each leaves its copy in Tg (agent-scope
    // stores, complete before its flag) and raises a flag tagged with the
    // epoch; once the slice's flags are all up, the workgroup of group q takes
    // the max over groups of its share of the slice's keys (keys [q s, q s + s),
    // s = ceil(nout / ngroups)), exponentiates and averages over the steps:
    // importance_i = (1/N) sum_j exp2(kStep * max v). (A shared counter would
    // let the last group to arrive do it alone, but a read-modify-write that
    // dozens of workgroups retry at once costs tens of microseconds, and one
    // workgroup merging all keys of 28 groups waits for four batches of loads.)
    int k_lo = 0, k_hi = nout;
    if (a.ngroups > 1) {
        unsigned long long* flags = a.flags + (size_t)rank * a.ngroups;
        const unsigned long long mark = ((unsigned long long)a.epoch << 32) | a.epoch;
        for (int x = tid; x < a.N * nout; x += kThreads) {
            const int jj = x / nout, k = x - jj * nout;
            __hip_atomic_store(&a.Tg[((size_t)group * a.N + jj) * a.M + r0 + k], Trun[jj * KRP + k],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) st64u(flags + group, mark);
        if (w == 0) {
            // lane x watches groups x, x + 64, ...
            const unsigned long long t0 = wall_clock64();
            while (true) {
                bool miss = false;
                for (int x = lane; x < a.ngroups; x += 64) miss |= x != group && ld64(flags + x) != mark;
                if (__ballot(miss) == 0) break;
                __builtin_amdgcn_s_sleep(2);
                if (wait_expired(t0, a)) {
                    if (lane == 0) set_err(a);
                    break;
                }
            }
        }
        __syncthreads();
        const int share = (nout + a.ngroups - 1) / a.ngroups;
        k_lo = min(group * share, nout);
        k_hi = min(k_lo + share, nout);
        // XB values per thread, the other groups' copies GB at a time: up to
        // XB * GB = 60 independent loads in flight (a wave can have 63)
        // instead of one round trip each, shaped to the merge (XB = 1 when
        // one pass covers the values, GB the smallest that covers the other
        // groups), since the issue of a wave's loads, not their latency, is
        // what a small merge waits for. Every load is issued unconditionally
        // from an address in bounds (lanes past the end read element 0,
        // batches past the last group re-read it; neither changes a max), so
        // that none waits for another.
        const int cnt = k_hi - k_lo;
        const int total = a.N * cnt;
        const size_t gstride = (size_t)a.N * a.M;
        const int last_other = a.ngroups - 2;  // the others, as 0 .. ngroups - 2
        auto merge = [&](auto XBc, auto GBc) __attribute__((always_inline)) {
            constexpr int XB = decltype(XBc)::value, GB = decltype(GBc)::value;
            for (int x0 = 0; x0 < total; x0 += kThreads * XB) {
                int v[XB], li[XB], go[XB];
#pragma unroll
                for (int i = 0; i < XB; ++i) {
                    const int x = x0 + i * kThreads + tid;
                    const int jj = x / cnt, k = k_lo + x - jj * cnt;
                    li[i] = x < total ? jj * KRP + k : -1;
                    go[i] = x < total ? jj * a.M + r0 + k : 0;
                    v[i] = x < total ? Trun[li[i]] : kNegInf;
                }
                for (int gb = 0; gb <= last_other; gb += GB) {
                    int t[GB][XB];
#pragma unroll
                    for (int y = 0; y < GB; ++y) {
                        const int o = min(gb + y, last_other);
                        const int* tg = a.Tg + (size_t)(o + (o >= group ? 1 : 0)) * gstride;
#pragma unroll
                        for (int i = 0; i < XB; ++i) t[y][i] = (int)ld32(tg + go[i]);
                    }
                    // (every load issued before the first max: the scheduler
                    // would otherwise interleave them, a wait between each)
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int y = 0; y < GB; ++y)
#pragma unroll
                        for (int i = 0; i < XB; ++i) v[i] = max(v[i], t[y][i]);
                }
#pragma unroll
                for (int i = 0; i < XB; ++i)
                    if (li[i] >= 0) Trun[li[i]] = v[i];
            }
        };
        using I = std::integral_constant<int, 1>;
        if (last_other < 3) merge(std::integral_constant<int, 4>{}, std::integral_constant<int, 3>{});
        else if (last_other < 7) merge(std::integral_constant<int, 4>{}, std::integral_constant<int, 7>{});
        else if (total > kThreads) merge(std::integral_constant<int, 4>{}, std::integral_constant<int, 15>{});
        else if (last_other < 30) merge(I{}, std::integral_constant<int, 30>{});
        else merge(I{}, std::integral_constant<int, 60>{});
        __syncthreads();
    }
    // A call in which some bounded wait gave up (here or in any workgroup
    // that got to it first) has scores built on missing statistics: they are
    // replaced by NaN bit patterns (stored as bits, no arithmetic on them), so
    // that the selection rejects them instead of returning a plausible set.
    // (With blend_n = n > 0 this call adds one more step to scores already
    // averaged over n steps: (n * importance + this step's score) / (n + 1).)
    const bool poisoned = err_set(a);
    float smn = INFINITY, smx = -INFINITY;  // (fused selection: this share's min and max)
    int snf = 0;                            //   and whether it holds a non-finite score
    for (int k = k_lo + tid; k < k_hi && r0 + k < a.M_out; k += kThreads) {
        float sum = 0.f;
        for (int jj = 0; jj < a.N; ++jj) sum += exp2_hw((float)Trun[jj * KRP + k] * kStep);
        float v = sum / (float)a.N;
        if (a.blend_n > 0) v = (a.importance[r0 + k] * (float)a.blend_n + v) / (float)(a.blend_n + 1);
        const unsigned bits = poisoned ? kNaNBits : __float_as_uint(v);
        __hip_atomic_store((unsigned*)a.importance + r0 + k, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (SEL) {
            snf |= (bits & 0x7f800000u) == 0x7f800000u;
            smn = fminf(smn, __uint_as_float(bits));
            smx = fmaxf(smx, __uint_as_float(bits));
        }
    }
    if constexpr (SEL)
        fused_tail(a, smn, smx, snf, nstream, bid);
}

// The kernels of one configuration: kLaunchPlain, kLaunchFused (with the
// selection) or kLaunchPack (several requests).
template <class C, int MODE>
const void* kernel_ptr() {
    if constexpr (MODE == kLaunchPack) return (const void*)&score_kernel<C, false, PackArgs>;
    else return (const void*)&score_kernel<C, MODE == kLaunchFused, ScoreArgs>;
}

// The instantiation for head-group size G (nullptr when unsupported).
template <int D, bool BF, int NH, int TPW, bool DMA, int MODE>
const void* pick_g(int G) {
    switch (G) {
        case 1:
            // (one head per step and two halves keep 32 running maxima per
            // lane: only the base tile count fits the registers)
            if constexpr (NH == 2 && TPW > tiles_per_wave(BF, D)) return nullptr;
            else return kernel_ptr<Cfg<D, BF, NH, 1, TPW, DMA>, MODE>();
        case 2: return kernel_ptr<Cfg<D, BF, NH, 2, TPW, DMA>, MODE>();
        case 4: return kernel_ptr<Cfg<D, BF, NH, 4, TPW, DMA>, MODE>();
        case 8: return kernel_ptr<Cfg<D, BF, NH, 8, TPW, DMA>, MODE>();
        case 16: return kernel_ptr<Cfg<D, BF, NH, 16, TPW, DMA>, MODE>();
        case 32:
            if constexpr (NH == 2) return kernel_ptr<Cfg<D, BF, 2, 32, TPW, DMA>, MODE>();
            return nullptr;
        default: return nullptr;
    }
}

// The instantiation for (rows, G, tiles per wave, K path) of one operand type
// and head dimension; TPW is tiles_per_wave(BF, D) or one more; the DMA path
// exists for bf16 at the base tile count.
template <int D, bool BF, int MODE>
const void* pick_kernel_for(int rows, int G, int tpw, bool dma) {
    constexpr int T0 = tiles_per_wave(BF, D);
    if (dma) {
        if constexpr (BF) {
            if (tpw == T0) return rows == 32 ? pick_g<D, BF, 2, T0, true, MODE>(G) : pick_g<D, BF, 1, T0, true, MODE>(G);
            if (tpw == T0 + 1)
                return rows == 32 ? pick_g<D, BF, 2, T0 + 1, true, MODE>(G) : pick_g<D, BF, 1, T0 + 1, true, MODE>(G);
        }
        return nullptr;
    }
    if (tpw == T0) return rows == 32 ? pick_g<D, BF, 2, T0, false, MODE>(G) : pick_g<D, BF, 1, T0, false, MODE>(G);
    if (tpw == T0 + 1)
        return rows == 32 ? pick_g<D, BF, 2, T0 + 1, false, MODE>(G) : pick_g<D, BF, 1, T0 + 1, false, MODE>(G);
    return nullptr;
}

}  // namespace sp
