/*
 * libspecprefill: SpecPrefill's token-importance estimator on one AMD Instinct
 * MI355X (gfx950), as a C ABI.
 *
 * The method (cited by web-page title and section):
 *   [SP-R] "Speculative Prefill: Turbocharging TTFT with Lightweight and
 *          Training-Free Token Importance Estimation" (paper review page),
 *          sections "Core algorithm" and "Core formulas".
 *   [SP-G] "SpecPrefill - Implementation Guide", sections "How It Works",
 *          "v3 Improvements", "v3.1 Optimizations & Bug Fixes" and
 *          "Configuration Reference".
 * A small speculator decodes N look-ahead tokens after an M-token prompt; the
 * softmax attention of those N queries over the prompt keys says which prompt
 * tokens matter. sp_score turns the queries and keys into one importance score
 * per prompt token; sp_select turns the scores into the list of prompt tokens a
 * large model should prefill, with their original position ids.
 *
 * Conventions for every call:
 *  - Pointers marked "device" are HIP device memory (hipMalloc / torch CUDA
 *    tensors); "host" pointers are ordinary CPU memory read during the call.
 *    The caller owns every buffer; the library allocates nothing. Between
 *    calls it keeps only host-side caches that do not change any result: each
 *    device's compute-unit count and the launch plans of recent (shape, M)
 *    pairs, guarded for concurrent callers. Tensors are dense, row-major,
 *    innermost index last.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *    asynchronous and stream-ordered: they enqueue kernels and return. No call
 *    synchronises the device.
 *  - Argument errors are reported synchronously, before anything is enqueued:
 *    SP_EINVAL (malformed arguments), SP_EUNSUPPORTED (well-formed but outside
 *    what the kernels implement), SP_EWORKSPACE (workspace missing or too
 *    small). SP_EDEVICE reports a failed kernel launch; faults during
 *    execution surface at the caller's next synchronisation, as usual in HIP.
 *  - Q or K containing NaN or Inf give unspecified (but memory-safe) scores;
 *    scores containing NaN or Inf make the selection report n_kept = -1.
 *  - Two calls may run concurrently only with distinct workspaces and outputs;
 *    concurrent scoring calls also compete for compute units, which an
 *    ordinary (SP_LAUNCH_RESIDENT) scoring launch needs all at once: see
 *    sp_launch below.
 */
#ifndef SPECPREFILL_H
#define SPECPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SP_OK = 0,
    SP_EINVAL = 1,
    SP_EUNSUPPORTED = 2,
    SP_EWORKSPACE = 3,
    SP_EDEVICE = 4
} sp_status;

typedef enum { SP_F32 = 0, SP_BF16 = 1 } sp_dtype;

typedef enum { SP_SELECT_TOPK = 0, SP_SELECT_MASS = 1, SP_SELECT_THRESHOLD = 2 } sp_select_mode;

/* How sp_select maps the scores to [0, 1] before boosting (step 1 of sp_select). */
typedef enum { SP_NORM_MINMAX = 0, SP_NORM_PERCENTILE = 1, SP_NORM_ZSCORE = 2 } sp_norm;

/* How sp_score launches its scoring kernel, whose workgroups wait on each
 * other and so must all be resident on the device at once.
 *   SP_LAUNCH_RESIDENT     (0, the default) an ordinary launch of no more
 *       workgroups than the device holds at a time (one per compute unit; the
 *       call returns SP_EDEVICE otherwise): on a device not otherwise busy,
 *       every workgroup is resident from the start. Kernels that occupy compute units for long
 *       on other streams (or processes) can keep some workgroups waiting for
 *       a unit; the others' waits are bounded, so the call then ends after at
 *       most about 2 s with its scores invalid and the time-out reported by
 *       sp_score_status.
 *   SP_LAUNCH_COOPERATIVE  (1) a cooperative launch (hipLaunchCooperativeKernel):
 *       the runtime guarantees co-residency whatever else runs, at a cost of
 *       about 20 us of device time per call. */
typedef enum { SP_LAUNCH_RESIDENT = 0, SP_LAUNCH_COOPERATIVE = 1 } sp_launch;

/* Shape of the speculator's attention: L attention layers, H query heads,
 * Hkv key/value heads (H % Hkv == 0; query head h reads kv-head h / (H/Hkv)),
 * head dimension d, N look-ahead steps. scale multiplies the logits; 0 selects
 * 1/sqrt(d). launch is an sp_launch (0 = SP_LAUNCH_RESIDENT). Supported:
 * d in {64, 128}; G = H/Hkv a power of two; G*N <= 32; and prompts whose
 * M + N keys are at most (compute units - 1) x 560 (x 336 for f32 at d = 128;
 * fewer for G = 1 with 32 query rows): M <= 142,792 at N = 8 on a 256-CU
 * MI355X, 85,672 for f32 at d = 128. sp_score_plan reports SP_EUNSUPPORTED
 * beyond. */
typedef struct {
    int32_t L, H, Hkv, d, N;
    sp_dtype dtype;
    float scale;
    sp_launch launch;
} sp_score_desc;

/* Selection parameters ([SP-G] Configuration Reference gives the pages'
 * defaults: chunk 32, keep rate 0.3, mass 0.85, boosts first 64 x1.5 and last
 * 128 x1.3, SP_MAX_KEEP 2000).
 *   chunk      tokens per chunk (>= 1)
 *   pool_k     odd width of the average pool over chunk scores (1 = none)
 *   mode       SP_SELECT_TOPK uses keep_rate in (0,1]; SP_SELECT_MASS uses mass in (0,1];
 *              SP_SELECT_THRESHOLD uses keep_rate in (0,1], min_tok and max_keep
 *   boost_*    multipliers >= 0 for the first / last n tokens (1.0 = off)
 *   min_tok    (threshold mode) >= 0; the fill target is min(min_tok, max(4, M/10))
 *              tokens (the Guide's program passes 128); 0 in the other modes
 *   max_keep   (threshold mode) >= 0; cap on kept tokens, 0 = none; 0 in the other modes
 *   norm       an sp_norm (0 = SP_NORM_MINMAX, the only one threshold mode takes);
 *              SP_NORM_PERCENTILE uses the quantiles 0 <= norm_lo < norm_hi <= 1;
 *              SP_NORM_ZSCORE uses norm_lo = 0 and the clip c = norm_hi > 0
 *              (in standard deviations); both 0 for SP_NORM_MINMAX */
typedef struct {
    int32_t chunk, pool_k;
    sp_select_mode mode;
    float keep_rate, mass;
    int32_t boost_first_n;
    float boost_first_mult;
    int32_t boost_last_n;
    float boost_last_mult;
    int32_t min_tok, max_keep;
    sp_norm norm;
    float norm_lo, norm_hi;
} sp_select_params;

/* Bytes of device workspace sp_score / sp_score_lastrow / sp_score_varlen /
 * sp_score_windows need for prompts of at most max_prompt_len tokens; 0 if the
 * shape is invalid or unsupported. */
size_t sp_score_workspace_bytes(const sp_score_desc* desc, int64_t max_prompt_len);

/*
 * Token importance of one prompt ([SP-R] Core formulas: attention score
 * a_ij = Softmax(Q_{M+j} K^T)_i and the importance aggregation; [SP-G] How It
 * Works, token importance):
 *   importance[i] = (1/N) * sum_{j<N} max_{l<L, h<H} softmax_j(s_{l,h,j,.})[i],
 *   s_{l,h,j,i} = scale * <Q[l][h][j][:], K[l][h/G][i][:]>,
 * where row j is the query at position M+j and its softmax runs over the
 * M+j+1 keys 0..M+j it can see (the look-ahead keys M..M+N-1 enter only the
 * denominators of the rows that see them); i < M.
 *   Q           device, [L][H][N][d] of desc->dtype (RoPE already applied)
 *   K           device, [L][Hkv][M+N][d] of desc->dtype
 *   M           prompt length, >= 1
 *   importance  device, [M] float32 (written)
 *   ws          device workspace of ws_bytes >= sp_score_workspace_bytes(desc, M);
 *               contents need no initialisation and are clobbered. Calls that
 *               overlap on one workspace (other streams or threads) race.
 * The call may be captured into a HIP graph (a small clearing kernel is then
 * captured before the scoring kernel, so that replays start afresh); eager
 * calls need nothing between them (what the kernel leaves in the workspace is
 * tagged with a per-launch number).
 */
sp_status sp_score(const sp_score_desc* desc, const void* Q, const void* K, int32_t M,
                   float* importance, void* ws, size_t ws_bytes, void* stream);

/*
 * sp_score for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels as sp_score, with the workspace in a static
 * device array of SP_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends (its address is looked up on the
 * first call on each device). The call allocates nothing. Every call on a
 * device shares that device's array: calls that overlap on one device (other
 * streams, other threads) race and must not be made; consecutive calls need
 * nothing in between.
 * A time-out of its bounded waits shows as NaN scores (sp_select then reports
 * n_kept = -1); sp_score_status does not apply.
 *   Arguments as for sp_score, without the workspace. SP_EWORKSPACE when the
 *   plan for (desc, M) needs more than SP_NOALLOC_SCRATCH_BYTES of workspace
 *   (the 8B shape needs about 12 MiB at 32K keys, 34 MiB at 128K keys).
 */
#define SP_NOALLOC_SCRATCH_BYTES (64u << 20)
sp_status sp_score_noalloc(const sp_score_desc* desc, const void* Q, const void* K, int32_t M,
                           float* importance, void* stream);

/*
 * sp_score with the query row of the last prompt token as one more step
 * ([SP-G] How It Works, Attention Capture (cb_eval): the attention of the last
 * query position is captured during the speculator's prefill, like each
 * look-ahead step's, and the importance averages over all captured steps).
 * That row, at position M-1, sees the M prompt keys 0..M-1 (none of the
 * look-ahead keys):
 *   importance[i] = (1/(N+1)) * (sum_{j<N} max_{l,h} a_{l,h,j,i} + max_{l,h} b_{l,h,i}),
 *   b_{l,h,.} = softmax over i < M of scale * <Q_last[l][h][:], K[l][h/G][i][:]>,
 * with a as for sp_score. Two passes over K: the look-ahead rows as sp_score
 * computes them, then the last row, whose finishing blends it in.
 *   Q_last  device, [L][H][d] of desc->dtype; the other arguments as for sp_score
 *           (the workspace bound of sp_score_workspace_bytes covers both passes)
 */
sp_status sp_score_lastrow(const sp_score_desc* desc, const void* Q, const void* Q_last,
                           const void* K, int32_t M, float* importance, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * sp_score for a ragged batch of R requests (R >= 1), each scored as sp_score
 * would score it alone (bit for bit where it has a launch to itself; a request
 * that shares a launch has its own split of the keys over workgroups, so its
 * scores can differ in rounding).
 *   Q              device, [R][L][H][N][d]
 *   K              device, [L][Hkv][T][d], T = sum_r (M_r + N); request r's
 *                  M_r prompt keys followed by its N look-ahead keys start at
 *                  key row cu_prompt_host[r] + r*N
 *   cu_prompt_host host, [R+1] prompt offsets: cu_prompt_host[0] = 0,
 *                  M_r = cu_prompt_host[r+1] - cu_prompt_host[r] >= 1
 *   importance     device, [cu_prompt_host[R]] float32; request r's scores at
 *                  offset cu_prompt_host[r]
 *   ws             as for sp_score with max_prompt_len = max_r M_r; with
 *                  ws_bytes >= sp_score_batch_workspace_bytes(desc, R,
 *                  cu_prompt_host), requests of similar length (up to 8, the
 *                  longest at most 4 times the shortest) whose one launch the
 *                  planner estimates faster than their launches in turn are
 *                  scored in one launch, each on its own share of the CUs and
 *                  its own part of the workspace (launches go in order of
 *                  prompt length; each request's scores are those sp_score
 *                  computes, up to rounding; a smaller workspace scores in
 *                  turn what does not fit)
 */
sp_status sp_score_varlen(const sp_score_desc* desc, int32_t R, const void* Q, const void* K,
                          const int64_t* cu_prompt_host, float* importance, void* ws,
                          size_t ws_bytes, void* stream);

/* Bytes of device workspace with which sp_score_varlen / sp_score_windows score
 * the batch cu_prompt_host[0..R] (host, as for sp_score_varlen) with every
 * launch that packs several requests (at least sp_score_workspace_bytes of the
 * longest request); 0 if the arguments are invalid or a request has no plan. */
size_t sp_score_batch_workspace_bytes(const sp_score_desc* desc, int32_t R,
                                      const int64_t* cu_prompt_host);

/* The launches sp_score_varlen / sp_score_windows would make for the batch
 * cu_prompt_host[0..R] with a workspace of ws_bytes (for reports and tests; no
 * device work): launch_of (host, [R], or NULL) gets each request's launch
 * index, requests with the same index sharing one launch; n_launches (host,
 * [1]) the number of launches. SP_EWORKSPACE if ws_bytes is below what a
 * request needs alone. */
sp_status sp_score_batch_plan(const sp_score_desc* desc, int32_t R, const int64_t* cu_prompt_host,
                              size_t ws_bytes, int32_t* launch_of, int32_t* n_launches);

/*
 * Sliding-window scoring ([SP-G] Sliding Window, "Sliding Window Solution";
 * Implementation Details, "Sliding Window Loop (v3.1)"): a prompt too long for
 * the speculator is scored in overlapping windows, each prefilled and decoded
 * by the speculator on its own (its cache cleared in between), so each window
 * brings its own look-ahead queries and keys.
 *
 * sp_window_layout: windows start at 0, stride, 2*stride, ...; window w covers
 * tokens [start_w, min(start_w + window, M)); the first window that reaches M
 * is the last and keeps the scores of all its tokens, every other window
 * keeps its first stride scores. With 1 <= stride <= window this covers every
 * token exactly once (the Guide's per-token count of scores is then 1).
 *   n_windows           host, [1] (written: the number of windows R)
 *   starts, lens, keeps host, [capacity] int64 each (written), or all NULL to
 *                       count only
 * Returns SP_EINVAL for M < 1, window < 1, stride < 1, stride > window, or
 * capacity < R with arrays given. Host only; no device work.
 *
 * sp_score_windows: sp_score_varlen over R windows (window r's prompt keys are
 * its cu_window_host[r+1] - cu_window_host[r] tokens, laid out as for
 * sp_score_varlen), writing only the first keep_host[r] scores of window r
 * (1 <= keep_host[r] <= its length), packed in window order. With the
 * layout above (cu from lens, keep from keeps), importance[i] is token i's
 * score from the window that keeps it, i < M.
 *   importance  device, [sum_r keep_host[r]] float32
 *   ws          as for sp_score_varlen
 */
sp_status sp_window_layout(int64_t M, int32_t window, int32_t stride, int32_t* n_windows,
                           int64_t* starts, int64_t* lens, int64_t* keeps, int32_t capacity);
sp_status sp_score_windows(const sp_score_desc* desc, int32_t R, const void* Q, const void* K,
                           const int64_t* cu_window_host, const int64_t* keep_host,
                           float* importance, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace sp_select / sp_select_varlen can use: for one
 * prompt (R = 1) of at least 49152 tokens with min-max normalisation in the
 * top-K or mass mode, 86016 (the exchange of selection by several
 * workgroups, see sp_select); otherwise 0. (size_t)-1 if the arguments are
 * invalid. */
size_t sp_select_workspace_bytes(int32_t R, int64_t total_prompt_len,
                                 const sp_select_params* params);

/*
 * Chunk selection and compaction for one prompt ([SP-G] How It Works and v3
 * Improvements; [SP-R] Core algorithm: chunk selection, pooling, position-ID
 * recovery). With x = importance:
 *  1. v_i = (x_i - min x) / (max x - min x) in float32 (all 1 if max == min);
 *     or, for the robust normalisations ([SP-G] Limitations item 5 names
 *     percentile-based and z-score normalisation as remedies for outliers):
 *     SP_NORM_PERCENTILE: lo = s[floor(norm_lo (M-1))], hi = s[ceil(norm_hi (M-1))]
 *       for s = x sorted ascending (indices in double); v_i = (x_i - lo) / (hi - lo)
 *       in float32 clamped to [0, 1] (x_i >= hi ? 1 : 0 when hi == lo);
 *     SP_NORM_ZSCORE: u_i the min-max values above, y_i = rint(u_i 2^16),
 *       S1 = sum y, S2 = sum y^2, D = M S2 - S1^2 (exact integers); v_i = 1 if
 *       D == 0, else z_i = (double)(M y_i - S1) / sqrt((double) D) clipped to
 *       [-c, c] (c = norm_hi) and v_i = (float)((z_i + c) / (2c)) in double;
 *  2. v_i *= first_mult for i < first_n, then v_i *= last_mult for i >= M - last_n;
 *  3. q_i = round_half_even(v_i * 2^32) as uint64;
 *  4. chunk c holds tokens [c*chunk, min((c+1)*chunk, M)); C_c = sum q_i;
 *  5. key_c = (double) sum_{c'} C_c' / (double) sum_{c'} len_c' over the pool
 *     window c' in [c - (pool_k-1)/2, c + (pool_k-1)/2] clipped to [0, nc);
 *  6. chunks ranked by key descending, ties by smaller index;
 *     top-K keeps the first K = min(nc, max(1, ceil((double)keep_rate * nc)));
 *     mass keeps ranked chunks until (double)(sum of their C) >=
 *     (double)mass * (double)(sum of all C), the crossing chunk included;
 *  7. every token i of every kept chunk, ascending:
 *     kept_idx[n] = i, pos_ids[n] = pos_base + i. The first decode position
 *     afterwards is pos_base + M.
 * SP_SELECT_THRESHOLD instead follows the Implementation Guide's own program
 * ([SP-G] Full Source Code, its chunk selection and the cap on sparse tokens;
 * How It Works, chunk selection; Configuration Reference, SP_MAX_KEEP) on the
 * raw scores (pool_k must be 1 and the boosts off):
 *  a. eff_min = min(min_tok, max(4, M/10)); keep_rate >= 1 or M <= eff_min
 *     keeps every token;
 *  b. chunk means a_c = (float)(double sum of the chunk's scores in index
 *     order / its token count);
 *  c. K = max(1, ceil((float)nc * keep_rate)) (single-precision product);
 *     every chunk whose mean is >= the K-th largest mean is kept (equal
 *     means may keep more than K chunks);
 *  d. tokens 0..3 and, when M > 4, M-2 and M-1 are kept;
 *  e. while fewer than eff_min tokens are kept, the tokens of the other
 *     chunks are added in index order;
 *  f. the kept tokens ascend; with max_keep > 0 and more than max_keep kept,
 *     only kept[0], kept[s], kept[2s], ... (s = n / max_keep, integer
 *     division; max_keep of them) remain, the last replaced by the last kept
 *     token.
 * The result is a pure function of the float32 scores: identical inputs give
 * identical outputs on every run.
 *   importance  device, [M] float32
 *   kept_idx, pos_ids  device, [M] int32 each (first *n_kept entries written)
 *   n_kept      device, [1] int32 (written): the kept count, or -1 if some score
 *               is NaN or infinite (kept_idx and pos_ids are then not written;
 *               a scoring call whose bounded waits timed out leaves NaN scores)
 *   ws, ws_bytes  device workspace, 16-byte aligned, or NULL / 0: with at
 *               least sp_select_workspace_bytes(1, M, params) bytes, a prompt
 *               of 49152 tokens or more with min-max normalisation is selected
 *               by several workgroups (up to 64; each sums the exact chunk
 *               masses of its share, one ranks), which must all be resident
 *               at once (an otherwise idle device; a wait that gives up leaves
 *               n_kept = -1); the outputs are the same as with one workgroup.
 *               Not used while the stream is being captured into a graph.
 * Supported: M <= 2^24, nc = ceil(M/chunk) <= 5120 (4096 in threshold mode:
 * with chunk 32 that is 163,840 tokens, more than the longest prompt sp_score
 * takes, and 131,072 in threshold mode), and boost multipliers
 * with max(1, first_mult, last_mult, first_mult*last_mult) * 2^32 * pool_k *
 * chunk < 2^53 (so the pooled sums stay exact in double).
 */
sp_status sp_select(const float* importance, int32_t M, const sp_select_params* params,
                    int32_t pos_base, int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * sp_select applied independently to each request of a ragged batch (one
 * workgroup per request; R <= 1024).
 *   importance      device, [cu_prompt_host[R]] float32
 *   cu_prompt_host  host, [R+1] prompt offsets (as for sp_score_varlen)
 *   pos_base_host   host, [R] position of each request's first prompt token,
 *                   or NULL for all 0
 *   kept_idx        device, [cu_prompt_host[R]] int32: request r writes its
 *                   kept tokens as packed indices cu_prompt_host[r] + i, from
 *                   offset cu_prompt_host[r]
 *   pos_ids         device, [cu_prompt_host[R]] int32: pos_base_r + i, same offsets
 *   n_kept          device, [R] int32 (-1 for a request with a non-finite score)
 */
sp_status sp_select_varlen(const float* importance, int32_t R, const int64_t* cu_prompt_host,
                           const int32_t* pos_base_host, const sp_select_params* params,
                           int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Sparse-prefill batch ([SP-G] Full Source Code: the target's batch holds,
 * for each kept index, the input token at that index and position): copies
 * the rows of the kept tokens in kept order. For request r (offsets
 * cu_host[r], as for sp_select_varlen; R = 1 and cu_host = {0, M} for
 * sp_select's output):
 *   dst row cu_host[r] + o = src row kept_idx[cu_host[r] + o], o < n_kept[r].
 *   src       device, rows of row_bytes (a multiple of 4), indexed by kept_idx
 *             (e.g. int32 token ids: row_bytes = 4; hidden states: d x 2 for bf16)
 *   kept_idx  device int32, n_kept device int32 [R]: as sp_select / sp_select_varlen
 *             write them (the counts are read on the device: no host synchronisation)
 *   dst       device, at least cu_host[R] rows; rows past each request's count
 *             are left as they are
 * Positions come with the selection (pos_ids). SP_EUNSUPPORTED for a row size
 * that is not a positive multiple of 4.
 */
sp_status sp_gather_rows(const void* src, int64_t row_bytes, const int32_t* kept_idx,
                         const int32_t* n_kept, int32_t R, const int64_t* cu_host, void* dst,
                         void* stream);

/*
 * Break-even gate ([SP-G] v3 Improvements, "Break-Even Detection";
 * Configuration Reference, SP_BREAK_EVEN, SP_SPEC_THROUGHPUT,
 * SP_BREAK_EVEN_SAFETY): scoring takes about M / spec_tps seconds, sparse
 * prefill saves about (M - keep_fraction * M) / target_tps; *run = 1 when the
 * saving is at least safety times the scoring time (the Guide's defaults:
 * 600 and 270 tokens/s, safety 1.2). Host only, in double precision.
 */
sp_status sp_break_even(int64_t M, float keep_fraction, float spec_tps, float target_tps,
                        float safety, int32_t* run);

/* Static, human-readable name of a status code. */
const char* sp_status_string(sp_status status);

/*
 * Launch plan sp_score would use for one prompt of M tokens (for reports and
 * tests): info[0] workgroups, info[1] workgroups per (layer, kv-head) unit,
 * info[2] groups working in parallel, info[3] prompt keys per workgroup,
 * info[4] query rows per tile (16 or 32), info[5] units, info[6] device
 * compute units, info[7] units between streaming a unit and finishing it,
 * info[8] 1 if K tiles travel by DMA into LDS (else a register ring).
 * Workgroups beyond info[1] * info[2] combine the per-unit statistics. No
 * device work is enqueued.
 */
sp_status sp_score_plan(const sp_score_desc* desc, int32_t M, int32_t info[9]);

/*
 * Profiling aid, not part of the scoring computation. While set, every
 * sp_score / sp_score_varlen call made by the calling thread records the HIP
 * events `before` and `after` (hipEvent_t handles created by the caller) on
 * its stream immediately before and after each launch of the
 * scoring kernel, so that hipEventElapsedTime gives that kernel's duration
 * apart from the small kernels around it (for sp_score_varlen the events end
 * up around its last launch). Pass NULL, NULL to stop. The setting
 * is per thread; the library never creates, waits on or destroys the events.
 * Returns SP_EINVAL if exactly one of the two is NULL.
 */
sp_status sp_profile_score_kernel(void* before, void* after);

/*
 * sp_score and sp_select of one prompt in one launch (the computation of
 * each as cited there): once every workgroup of the scoring kernel has
 * written its scores, one of its workgroups (512 threads) runs the
 * selection on them. For prompts of 16K tokens or more with min-max
 * normalisation, the scoring workgroups first sum the chunks' fixed-point
 * masses between them (exact integer sums), and that workgroup only pools,
 * ranks and emits. The outputs are those of sp_score followed by sp_select
 * with the same arguments, bit for bit.
 *   desc, Q, K, M, ws, ws_bytes, stream  as for sp_score (importance is
 *            written as well)
 *   params, pos_base, kept_idx, pos_ids, n_kept  as for sp_select; the
 *            top-K and mass modes only (SP_EUNSUPPORTED for the threshold mode)
 * A time-out of the scoring kernel's bounded waits leaves n_kept = -1.
 */
sp_status sp_score_select(const sp_score_desc* desc, const void* Q, const void* K, int32_t M,
                          const sp_select_params* params, int32_t pos_base, float* importance,
                          int32_t* kept_idx, int32_t* pos_ids, int32_t* n_kept, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Whether the last scoring call (sp_score, sp_score_lastrow, sp_score_select,
 * sp_score_varlen or sp_score_windows) that used workspace ws ran to
 * completion without any of its bounded
 * cross-workgroup waits running out (in any of its requests). The scoring
 * kernel never hangs: a wait that sees no progress for 2 s (which would take a
 * workgroup that never runs) gives up and marks the workspace; the
 * workgroups that finish after that write NaN in place of their scores (so
 * that sp_select reports n_kept = -1), and the call's importance is not valid.
 *   ws         device workspace passed to that call
 *   stream     the stream that call was enqueued on
 *   timed_out  host, written: 0 (complete) or 1 (a wait timed out)
 * This call waits for the stream (it copies 16 bytes back to the host).
 * SP_EINVAL for null pointers; SP_EDEVICE if the copy fails.
 */
sp_status sp_score_status(const void* ws, void* stream, int32_t* timed_out);

/*
 * Testing aid: the limit, in ticks of the device's 100 MHz constant clock, of
 * every bounded wait in the scoring calls, and in sp_select by several
 * workgroups, that the calling thread makes from now on (0 restores the
 * default, 2 s). A tiny limit makes those waits give up at
 * once, so that the time-out path (error word, NaN scores, n_kept = -1) can be
 * exercised with every kernel still ending normally. Always SP_OK.
 */
sp_status sp_set_wait_limit(uint64_t ticks);

/*
 * Measurement aid, not part of the scoring computation: enqueues one plain
 * streaming read of `bytes` bytes of device memory at buf by `grid`
 * workgroups of 512 threads, each thread keeping `depth` (4, 8 or 16) 16-byte
 * loads in flight (workgroup b reads the chunks b, b + grid, ... of
 * 512 x depth x 16 bytes). bytes divided by the launch's duration is the HBM
 * read rate the device sustains for that launch shape: the practical ceiling
 * of a kernel that reads its input once.
 *   buf     device, 16-byte aligned; bytes a positive multiple of 16
 *   flag    device, [1] int32: written (1) only if the XOR of all words read
 *           equals 0x5a17c0de (this keeps the loads; normally untouched)
 * SP_EINVAL for null pointers or bad sizes, SP_EUNSUPPORTED for another depth.
 */
sp_status sp_read_probe(const void* buf, size_t bytes, int32_t grid, int32_t depth, int32_t* flag,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECPREFILL_H */
