// Look-ahead attention scoring on gfx950.
//
// What is computed ("Speculative Prefill" review page, Core formulas: attention
// score a_ij = Softmax(Q_{M+j} K^T)_i and the max-max-mean importance
// aggregation; "SpecPrefill - Implementation Guide", How It Works, token
// importance): for every layer l, query head h and look-ahead step j the softmax
// of the scaled logits of query M+j over the M+j+1 keys it sees, then
//   importance_i = (1/N) sum_j max_{l,h} p_{l,h,j,i},  i < M.
//
// How (one pass over K in HBM):
//  * A unit is one (layer, kv-head) plane of K. The G query heads of the plane
//    and the N look-ahead steps form G*N query rows, padded to a 16- or 32-row
//    MFMA tile (row = j*G + h_local), so one bf16 MFMA chain computes
//    K_tile x Q^T for all of them: keys are the MFMA M dimension, query rows
//    the N dimension, and each lane ends up holding one query row for several
//    keys, so row statistics are mostly lane-local.
//  * g workgroups (one per CU, launched cooperatively so all are resident)
//    share a unit, each holding the logits of its slice of <= 1024 (2048) keys
//    in registers. Each publishes its slice's (row max, row sum), waits at a
//    per-unit barrier for the other g-1, combines the g partials into the row
//    log-sum-exp, and turns its registers into log2 probabilities without
//    touching K again.
//  * The max over the G heads of a step is a DPP max across the G adjacent
//    lanes; the max over kv-heads and layers is a running max in LDS, kept in
//    the log2 domain (exp2 is monotone, so the exponential is taken once per
//    (step, key) at the end). Each group writes its running max; a small
//    kernel takes the max over groups, exponentiates and averages over steps.
//  * Groups of g <= 32 workgroups sit on one XCD (blockIdx % 8 picks the XCD),
//    so a barrier's atomics stay within one L2.
#include <math.h>

#include "sp_internal.h"

namespace sp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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

// ---------------------------------------------------------------------------------------
// MFMA tile engines. A = K tile (TK keys x d), B = Q^T (d x ROWS query rows),
// C[key][row]. Lane L supplies key/row L % TK and the contiguous d-range
// [lg * D/LG, (lg+1) * D/LG) with lg = L / TK for both operands, so A's and B's
// k-index maps to the same d.
// ---------------------------------------------------------------------------------------
template <int D_, bool BF16>
struct Eng32 {  // 32 rows x 32 keys
    static constexpr int D = D_, ROWS = 32, TK = 32, NACC = 16, LG = 2;
    static constexpr int ESZ = BF16 ? 2 : 4;
    static constexpr int DPL = D / LG;
    static constexpr int NLD = DPL * ESZ / 16;
    using Acc = f32x16;
    struct Frag {
        i32x4 v[NLD];
    };
    __device__ static int qrow(int lane) { return lane & 31; }
    __device__ static int lgrp(int lane) { return lane >> 5; }
    __device__ static int key_of(int lane, int r) {
        return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    __device__ static Acc mma(const Frag& q, const Frag& k) {
        Acc c = {};
        if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < NLD; ++s)
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k.v[s]),
                                                            __builtin_bit_cast(bf16x8, q.v[s]),
                                                            c, 0, 0, 0);
        } else {
#pragma unroll
            for (int s = 0; s < NLD; ++s) {
                const f32x4 kv = __builtin_bit_cast(f32x4, k.v[s]);
                const f32x4 qv = __builtin_bit_cast(f32x4, q.v[s]);
                c = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, qv.x, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, qv.y, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, qv.z, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, qv.w, c, 0, 0, 0);
            }
        }
        return c;
    }
};

template <int D_, bool BF16>
struct Eng16 {  // 16 rows x 16 keys
    static constexpr int D = D_, ROWS = 16, TK = 16, NACC = 4, LG = 4;
    static constexpr int ESZ = BF16 ? 2 : 4;
    static constexpr int DPL = D / LG;
    static constexpr int NLD = DPL * ESZ / 16;
    using Acc = f32x4;
    struct Frag {
        i32x4 v[NLD];
    };
    __device__ static int qrow(int lane) { return lane & 15; }
    __device__ static int lgrp(int lane) { return lane >> 4; }
    __device__ static int key_of(int lane, int r) { return 4 * (lane >> 4) + r; }
    __device__ static Acc mma(const Frag& q, const Frag& k) {
        Acc c = {};
        if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < NLD; ++s)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k.v[s]),
                                                            __builtin_bit_cast(bf16x8, q.v[s]),
                                                            c, 0, 0, 0);
        } else {
#pragma unroll
            for (int s = 0; s < NLD; ++s) {
                const f32x4 kv = __builtin_bit_cast(f32x4, k.v[s]);
                const f32x4 qv = __builtin_bit_cast(f32x4, q.v[s]);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.x, qv.x, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.y, qv.y, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.z, qv.z, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.w, qv.w, c, 0, 0, 0);
            }
        }
        return c;
    }
};

// K fragment of the tile whose first key is `key0` (zeros when !valid or past
// the end of the plane: the buffer descriptor bounds the plane).
template <class E>
__device__ __forceinline__ void load_k(typename E::Frag& f, __amdgpu_buffer_rsrc_t rs, int key0,
                                       bool valid, int lane) {
    const uint32_t off =
        valid ? (uint32_t)(key0 + (lane % E::TK)) * (uint32_t)(E::D * E::ESZ) +
                    (uint32_t)(E::lgrp(lane) * E::DPL * E::ESZ)
              : kOob;
#pragma unroll
    for (int s = 0; s < E::NLD; ++s) f.v[s] = load16(rs, off + 16u * s);
}

// Q fragment of query row (l, kvh*G + hl, j); zeros for padding rows.
template <class E>
__device__ __forceinline__ void load_q(typename E::Frag& f, const void* Q, int l, int kvh, int j,
                                       int hl, bool valid, int H, int G, int N, int lane) {
    if (valid) {
        const long long row = ((long long)l * H + (long long)kvh * G + hl) * N + j;
        const char* p = (const char*)Q + (row * E::D + E::lgrp(lane) * E::DPL) * E::ESZ;
#pragma unroll
        for (int s = 0; s < E::NLD; ++s) f.v[s] = *(const i32x4*)(p + 16 * s);
    } else {
#pragma unroll
        for (int s = 0; s < E::NLD; ++s) f.v[s] = i32x4{0, 0, 0, 0};
    }
}

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

// Max over the G adjacent lanes that hold the G heads of one look-ahead step.
__device__ __forceinline__ float group_max(float v, int G) {
    if (G >= 2) v = fmaxf(v, dpp<0xb1>(v));   // quad_perm [1,0,3,2]
    if (G >= 4) v = fmaxf(v, dpp<0x4e>(v));   // quad_perm [2,3,0,1]
    if (G >= 8) v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
    if (G >= 16) v = fmaxf(v, dpp<0x140>(v)); // row_mirror
    if (G >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    return v;
}

template <class E>
__device__ __forceinline__ void lane_combine(float& m, float& s, float c) {
    if constexpr (E::LG == 2) {
        combine(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32), c);
    } else {
        combine(m, s, __shfl_xor(m, 16), __shfl_xor(s, 16), c);
        combine(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32), c);
    }
}

template <class E, int TPW>
__global__ __launch_bounds__(kThreads, 2) void score_kernel(ScoreArgs a) {
    constexpr int ROWS = E::ROWS, TK = E::TK, NACC = E::NACC;
    constexpr int NSUB = kThreads / ROWS;
    extern __shared__ float Trun[];  // [N][KR + kRowPad], log2-domain running max
    __shared__ float2 red[kWaves][ROWS];
    __shared__ float2 red2[kThreads];
    __shared__ float lse_s[ROWS];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int group, rank;
    if (a.xcd_local) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        group = xcd * (32 / a.g) + slot / a.g;
        rank = slot % a.g;
    } else {
        group = blockIdx.x / a.g;
        rank = blockIdx.x % a.g;
    }
    const int KRP = a.KR + kRowPad;
    for (int x = tid; x < a.N * KRP; x += kThreads) Trun[x] = -INFINITY;

    const int r0 = rank * a.KR;
    const int r1 = min(r0 + a.KR, a.M);
    const int nkeys = max(r1 - r0, 0);
    const int ntiles = (nkeys + TK - 1) / TK;
    const bool tail_owner = (r0 < a.M) && (r1 == a.M);
    const int qr = E::qrow(lane);
    const int j = qr / a.G, hl = qr - (qr / a.G) * a.G;
    const bool qvalid = j < a.N;
    const uint32_t plane_bytes = (uint32_t)(a.M + a.N) * (uint32_t)(E::D * E::ESZ);
    const float c = a.c;

    for (int it = 0;; ++it) {
        const int u = group + it * a.ngroups;
        if (u >= a.units) break;
        const int l = u / a.Hkv, kvh = u - (u / a.Hkv) * a.Hkv;

        typename E::Frag qf;
        load_q<E>(qf, a.Q, l, kvh, j, hl, qvalid, a.H, a.G, a.N, lane);
        const char* plane =
            (const char*)a.K + (long long)(l * a.Hkv + kvh) * a.plane_stride * E::ESZ;
        const auto rs = make_rsrc(plane, plane_bytes);

        // logits of this workgroup's key slice, kept in registers
        typename E::Acc acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = w + t * kWaves;
            typename E::Frag kf;
            load_k<E>(kf, rs, r0 + tile * TK, tile < ntiles, lane);
            acc[t] = E::mma(qf, kf);
        }
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int r = 0; r < NACC; ++r) {
                const int key = r0 + (w + t * kWaves) * TK + E::key_of(lane, r);
                if (key >= r1) acc[t][r] = -INFINITY;
                m = fmaxf(m, acc[t][r]);
            }
        float s = 0.f;
        if (m != -INFINITY) {
            const float mc = m * c;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int r = 0; r < NACC; ++r) s += exp2_hw(fmaf(acc[t][r], c, -mc));
        }
        // look-ahead keys M..M+N-1: in the denominators of the rows that see them
        if (tail_owner && w == kWaves - 1) {
            typename E::Frag kf;
            load_k<E>(kf, rs, a.M, true, lane);
            typename E::Acc at = E::mma(qf, kf);
            float mt = -INFINITY;
#pragma unroll
            for (int r = 0; r < NACC; ++r) {
                const int tk = E::key_of(lane, r);
                if (!(tk < a.N && tk <= j)) at[r] = -INFINITY;
                mt = fmaxf(mt, at[r]);
            }
            if (mt != -INFINITY) {
                float st = 0.f;
#pragma unroll
                for (int r = 0; r < NACC; ++r) st += exp2_hw(fmaf(at[r], c, -mt * c));
                combine(m, s, mt, st, c);
            }
        }
        lane_combine<E>(m, s, c);
        if (E::lgrp(lane) == 0) red[w][qr] = make_float2(m, s);
        __syncthreads();
        if (tid < ROWS) {
            float mm = red[0][tid].x, ss = red[0][tid].y;
            for (int x = 1; x < kWaves; ++x) combine(mm, ss, red[x][tid].x, red[x][tid].y, c);
            a.part[((size_t)u * a.g + rank) * ROWS + tid] = make_float2(mm, ss);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        }
        __syncthreads();
        // per-unit barrier across the g workgroups of the group
        if (tid == 0) {
            __hip_atomic_fetch_add(a.cnt + u, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned long long t0 = wall_clock64();
            while (__hip_atomic_load(a.cnt + u, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < a.g) {
                __builtin_amdgcn_s_sleep(1);
                if (wall_clock64() - t0 > kSpinTicks) {
                    __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        {
            const int row = tid % ROWS, sub = tid / ROWS;
            float mm = -INFINITY, ss = 0.f;
            for (int rr = sub; rr < a.g; rr += NSUB) {
                float* src = (float*)(a.part + ((size_t)u * a.g + rr) * ROWS + row);
                const float pm = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const float ps =
                    __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                combine(mm, ss, pm, ps, c);
            }
            red2[tid] = make_float2(mm, ss);
        }
        __syncthreads();
        if (tid < ROWS) {
            float mm = red2[tid].x, ss = red2[tid].y;
            for (int x = 1; x < NSUB; ++x)
                combine(mm, ss, red2[tid + x * ROWS].x, red2[tid + x * ROWS].y, c);
            lse_s[tid] = mm * c + log2_hw(ss);
        }
        __syncthreads();
        // log2 probabilities; max over the G heads of a step; running max over units
        const float lse = lse_s[qr];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int r = 0; r < NACC; ++r) {
                const float v = group_max(fmaf(acc[t][r], c, -lse), a.G);
                const int lk = (w + t * kWaves) * TK + E::key_of(lane, r);
                if (hl == 0 && qvalid && lk < nkeys) {
                    float* p = &Trun[j * KRP + lk];
                    *p = fmaxf(*p, v);
                }
            }
    }
    __syncthreads();
    for (int x = tid; x < a.N * nkeys; x += kThreads) {
        const int jj = x / nkeys, k = x - (x / nkeys) * nkeys;
        a.Tg[((size_t)group * a.N + jj) * a.M + r0 + k] = Trun[jj * KRP + k];
    }
}

__global__ void score_prep_kernel(int* cnt, int units, int* err) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < units; i += gridDim.x * blockDim.x)
        cnt[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
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
typedef void (*KernelFn)(ScoreArgs);

template <class E, int TPW>
static const void* kernel_ptr() {
    return (const void*)&score_kernel<E, TPW>;
}

static const void* pick_kernel(int dtype, int d, int rows) {
    const bool bf = dtype == SP_BF16;
    if (rows == 32) {
        if (d == 128) return bf ? kernel_ptr<Eng32<128, true>, kTilesPerWave32>()
                                : kernel_ptr<Eng32<128, false>, kTilesPerWave32>();
        if (d == 64) return bf ? kernel_ptr<Eng32<64, true>, kTilesPerWave32>()
                               : kernel_ptr<Eng32<64, false>, kTilesPerWave32>();
    } else {
        if (d == 128) return bf ? kernel_ptr<Eng16<128, true>, kTilesPerWave16>()
                                : kernel_ptr<Eng16<128, false>, kTilesPerWave16>();
        if (d == 64) return bf ? kernel_ptr<Eng16<64, true>, kTilesPerWave16>()
                               : kernel_ptr<Eng16<64, false>, kTilesPerWave16>();
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
    size_t lds = (size_t)d.N * (p.KR + kRowPad) * sizeof(float);
    const size_t min_lds = 96 * 1024;
    if (lds < min_lds) lds = min_lds;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;

    hipLaunchKernelGGL(score_prep_kernel, dim3((p.units + 255) / 256), dim3(256), 0, stream,
                       a.cnt, p.units, a.err);
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
