/*
 * retention.h - C ABI of the MI355X (gfx950) multi-scale retention library, libretention.so.
 *
 * Retention is the sequence mixer of RetNet: for each (batch b, head h) with a fixed decay gamma_h,
 *     S_n = gamma S_{n-1} + k_n^T v_n,   o_n = q_n S_n            (state S: d_k x d_v, S before token 0 given)
 * with q and k first rotated by their absolute position (xPos/rotary form). Sources: "Hybrid Architectures:
 * RetNet and the Three Computation Paradigms" (sections 2, 4, 6 and 7) and the RetNet paper summary
 * (Eq. 5 parallel, Eq. 6 recurrent, Eq. 7 chunkwise; the paper's ParallelRetention / RecurrentRetention /
 * ChunkwiseRetention interfaces, whose precomputed decay tensors are replaced here by gamma itself).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts (row-major, contiguous, device memory):
 *     q, k  [B, N, H, d_k]      v, o  [B, N, H, d_v]      state [B, H, d_k, d_v] (fp32, d_v fastest)
 *     decode step: q, k [B, H, d_k], v, o [B, H, d_v]
 * dtypes: q/k/v in `in_dt`, o in `out_dt`; supported pairs are (F32, F32), (BF16, BF16) and (BF16, F32).
 *     Products accumulate in fp32 and the state is always fp32. On the BF16 path the rotated q and k, the
 *     masked scores and the copy of the state used for q.S are rounded to bf16 (nearest-even) as MFMA
 *     operands; the carried state is never rounded.
 * gamma: HOST float[H], 0 < gamma <= 1 (per-head decay; multi-scale schedule 1 - 2^(-5-h) in the pages).
 * theta: HOST double[d_k/2] rotation frequencies, or NULL for no rotation. Pair (2i, 2i+1) of q and of k at
 *     absolute position p is turned by the angle +p*theta_i, so q'.k' depends on positions only through
 *     n - m (the conjugate-transpose reading of the paper summary's rotation; blog section 6.8).
 * pos0 / pos: absolute position of the first token (0 for a fresh sequence).
 * stream: a hipStream_t (NULL = the null stream). Every call only enqueues work and never synchronises.
 * Ownership: the caller owns every buffer. The library allocates no device memory; gamma/theta are read
 *     during the call and copied into kernel arguments.
 * Alignment: device pointers must be 16-byte aligned.
 * Errors: a non-zero status is returned before anything is enqueued, and ret_last_error() gives a detail
 *     string for the calling thread. RET_ERR_INVALID_ARG: null pointer, non-positive size, gamma outside
 *     (0, 1] or NaN, odd d_k with theta, misalignment, o aliasing an input, bad dtype pair.
 *     RET_ERR_UNSUPPORTED: a shape outside the kernels' tiling (listed per call). RET_ERR_HIP: a launch failed
 *     (device faults surface at the caller's next synchronisation). There is no fallback path.
 * NaN/Inf in inputs propagate into outputs; nothing traps.
 */
#ifndef RETENTION_H
#define RETENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RET_ABI_VERSION 7

typedef enum { RET_F32 = 0, RET_BF16 = 1 } ret_dtype_t;

typedef enum {
    RET_OK = 0,
    RET_ERR_INVALID_ARG = -1,
    RET_ERR_UNSUPPORTED = -2,
    RET_ERR_WORKSPACE = -3,
    RET_ERR_HIP = -4
} ret_status_t;

/* ABI version of the loaded library (RET_ABI_VERSION at build time). */
int ret_abi_version(void);

/* Digest of the sources the library was built from (for detecting a stale build). */
const char* ret_source_digest(void);

/* Static text for a status code. */
const char* ret_status_string(int status);

/* Detail for the last non-OK status returned on the calling thread ("" if none). */
const char* ret_last_error(void);

/*
 * Parallel form: O = (Q K^T (.) D) V, D[n][m] = gamma^(n-m) for n >= m and 0 otherwise, per (b, h), over the
 * whole sequence (blog sections 4.2-4.3; paper summary Eq. 5). No state in or out. Cost O(N^2 d).
 * Supported: F32 input: d_k in {16, 32, 64}, d_v a multiple of 16. BF16 input: d_k in {32, 64, 128, 256},
 * d_v a multiple of 64. N >= 1 (any length).
 */
ret_status_t ret_parallel_fwd(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                              int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                              const double* theta, int64_t pos0, void* stream);

/*
 * Workspace (device bytes) that ret_chunkwise_fwd can use, for the given shape and input dtype:
 *  - segment states: each sequence is split into segments that run in parallel, and the state entering a
 *    segment is built from the end states of the segments before it (a scan of the chunk state over
 *    segments; BF16 input: counters, flags and two d_k x 64 fp32 slots per segment and d_v tile of 64);
 *  - BF16 input with rotation and d_v >= 256: bf16 copies of q and k rotated once (2 * B*N*H*d_k*2 bytes),
 *    so the d_v tiles of a head do not each rotate the same rows. They start past the chain's first 64 KB
 *    (header, counters, flags), which are reserved even when the plan has a single segment.
 * 0 means the call runs one segment per (b, h) and needs none. A smaller workspace is allowed: the call then
 * first drops the rotated copies, then uses fewer segments; the results are the same up to rounding order.
 * The workspace must be zero-filled before its first use. Every call leaves it in a state the next call
 * accepts: the header (first 256 bytes) zero except a sticky error word, counters and flags zero (they occupy
 * the first 64 KB, ahead of every shape's state slots, while units x segments stays below about 16,000; beyond
 * that, zero-fill the workspace again before a call of another shape). Calls sharing a workspace must not
 * overlap in time (on one stream they do not). The library never frees it.
 */
size_t ret_chunkwise_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt);

/*
 * Synchronises `stream` and reports whether any call that used this workspace had to abandon a wait for
 * the state of an earlier segment (a sticky flag in the workspace). A wait gives up after about 0.17 s without
 * any progress of the segments it waits for (a flag rising resets the limit); the segment that gave up then
 * takes NaN for its entering state, so its outputs, and whatever is computed from its state (the final state,
 * later segments' entering states where its state enters them), come out NaN rather than silently wrong. RET_OK if no wait gave up (or workspace is NULL), RET_ERR_HIP with detail
 * otherwise.
 */
ret_status_t ret_chunkwise_check(const void* workspace, void* stream);

/*
 * Chunkwise recurrent form with chunk size `chunk` (blog section 7.2; paper summary Eq. 7). For chunk i of
 * length L (the last chunk may be shorter):
 *     O_[i] = (Q_[i] K_[i]^T (.) D) V_[i] + (Q_[i] R_{i-1}) (.) xi,   xi_j = gamma^(j+1)
 *     R_i   = gamma^L R_{i-1} + K_[i]^T (V_[i] (.) zeta),             zeta_j = gamma^(L-1-j)
 * with R_{-1} = state_in (NULL = zeros). state_out (may be NULL, may equal state_in) receives the state after
 * the last token, so a sequence can resume with pos0 = N and state_in = state_out, or hand over to
 * ret_recurrent_step. Results equal the recurrent and parallel forms up to rounding.
 * workspace: device memory of `workspace_bytes` (see ret_chunkwise_workspace_bytes), or NULL with 0.
 * Supported: F32 input: d_k in {16, 32, 64}, d_v a multiple of 16, chunk in {16, 32, 64}. BF16 input:
 * d_k in {32, 64, 128, 256}, d_v a multiple of 64, chunk in {32, 64, 128, 256, 512}. N >= 1. BF16 chunks
 * longer than 64 tokens are computed as runs of 64-token chunks, which the chunkwise form allows (any chunk
 * size gives the same result up to rounding). Kernels that read a chunk address it with 32-bit offsets:
 * chunk * H * max(d_k, d_v) * 4 must stay below 2^31 (RET_ERR_UNSUPPORTED otherwise).
 */
ret_status_t ret_chunkwise_fwd(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                               int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                               const double* theta, int64_t pos0, int chunk, const float* state_in,
                               float* state_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent (decode) step at absolute position `pos` (blog section 2.1; paper summary Eq. 6):
 *     S <- gamma S + k'^T v,   o = q' S      (update, then read; the token sees itself)
 * `state` [B, H, d_k, d_v] fp32 is updated in place. q, k [B, H, d_k], v, o [B, H, d_v].
 * Supported: d_k in {16, 32, 64, 128, 256}, d_v a multiple of 4 and <= 512.
 */
ret_status_t ret_recurrent_step(const void* q, const void* k, const void* v, void* o, float* state, int B, int H,
                                int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                const double* theta, int64_t pos, void* stream);

/*
 * The decode step of ret_recurrent_step with one position per sequence: sequence b is at absolute position
 * pos[b] (a batch of sequences at different lengths; the pages decode one token per step at its own position,
 * paper summary Eq. 6 and "Overall RetNet Architecture and Training/Inference Protocol"). pos: device int64[B],
 * 8-byte aligned, read by the kernel when it runs (a captured graph can advance it on the device); unused
 * without theta. The rotation factors are evaluated on the device (fp64 angle reduced by pi/2, fp32 sine and
 * cosine; angle error about pos * 2^-52 rad) rather than on the host, so results may differ from
 * ret_recurrent_step in the last bits. Otherwise as ret_recurrent_step.
 */
ret_status_t ret_recurrent_step_positions(const void* q, const void* k, const void* v, void* o, float* state, int B,
                                          int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                          const float* gamma, const double* theta, const int64_t* pos,
                                          void* stream);

/*
 * Multi-scale retention epilogue ("Hybrid Architectures: RetNet and the Three Computation Paradigms",
 * sections 8.4 and 9.1; paper summary, "Gating mechanism"):
 *     y = swish(gate) (.) GroupNorm_h(o),   swish(x) = x * sigmoid(x)
 * o, gate, y: [rows, H, d_v] device arrays, row-major (rows = B*N tokens of a chunkwise or parallel call, or B
 * for one decode step). GroupNorm has one group per head: each (row, head) vector of d_v values is
 * standardized by its own mean and biased variance, (x - mean) / sqrt(var + eps), then multiplied by
 * gn_weight[h * d_v + c] and shifted by gn_bias[h * d_v + c] (device float[H * d_v] each; NULL means 1 and 0).
 * gate: the gate projection X W_G, or NULL for no gate; the projections themselves are the caller's.
 * o_dt, gate_dt, y_dt: F32 or BF16 each. y may equal o or gate (in place); other overlaps are not allowed.
 * Every pointer 16-byte aligned. rows = 0 does nothing. Supported: d_v in {16, 32, 64, 128, 256, 512} and
 * rows * H < 2^31.
 * eps >= 0 and finite (RET_ERR_INVALID_ARG otherwise). Asynchronous on `stream`.
 */
ret_status_t ret_msr_epilogue(const void* o, const void* gate, const float* gn_weight, const float* gn_bias,
                              void* y, int64_t rows, int H, int dv, ret_dtype_t o_dt, ret_dtype_t gate_dt,
                              ret_dtype_t y_dt, float eps, void* stream);

/*
 * Chunkwise retention followed by the multi-scale retention epilogue, into y [B, N, H, d_v]:
 *     y = swish(gate) (.) GroupNorm_h(O),   O = ret_chunkwise_fwd's output, rounded to out_dt
 * Arguments as ret_chunkwise_fwd (with y in the place of o) and ret_msr_epilogue (gate [B, N, H, d_v] or
 * NULL, gate_dt, gn_weight, gn_bias, eps). Where the kernel holds whole head rows (bf16 input and output,
 * d_v = 64, the on-chip kernel: segments of at most 256 tokens) the epilogue is applied before the outputs are
 * stored, which saves writing and reading O; otherwise ret_msr_epilogue runs over y in place. Either way the
 * result equals the two calls in sequence up to rounding. gate must not alias q, k, v or y. Every check of
 * either call is made before anything is launched, except those of the chunkwise plan itself.
 */
ret_status_t ret_chunkwise_msr_fwd(const void* q, const void* k, const void* v, const void* gate, void* y, int B,
                                   int N, int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                   ret_dtype_t gate_dt, const float* gamma, const double* theta, int64_t pos0,
                                   int chunk, const float* state_in, float* state_out, const float* gn_weight,
                                   const float* gn_bias, float eps, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Gradients of chunkwise retention, for training with the chunkwise form (paper summary, "Overall RetNet
 * Architecture and Training/Inference Protocol"). With O the output of ret_chunkwise_fwd from a zero state
 * (state_in NULL) and dout = dL/dO [B, N, H, d_v], writes dq, dk [B, N, H, d_k] and dv [B, N, H, d_v]; the
 * gradients with respect to q and k are taken through their rotation. They follow from the parallel form
 * ("Hybrid Architectures: RetNet and the Three Computation Paradigms", section 4.3; paper summary Eq. 5):
 *     dq'_n = sum_{m<=n} gamma^(n-m) (dO_n . v_m) k'_m,    dk'_m = sum_{n>=m} gamma^(n-m) (dO_n . v_m) q'_n,
 *     dv_m  = sum_{n>=m} gamma^(n-m) (q'_n . k'_m) dO_n,   dq, dk = dq', dk' turned back by the rotation's
 *     transpose,
 * each a retention (the last two over the reversed sequence) that the chunkwise kernels compute.
 * in_dt: BF16 or F32 (q, k, v, dout); out_dt: F32 or BF16 (dq, dk, dv; F32 for F32 input). No gradient for a
 * state in or out.
 * workspace: device memory of ret_chunkwise_bwd_workspace_bytes for the input dtype (zero-filled once by the
 * caller, like the chunkwise workspace; every call leaves its chain part zeroed again; ret_chunkwise_check
 * accepts it and reports a segment-chain wait that gave up). dq, dk, dv must not alias the inputs or each
 * other. Errors: RET_ERR_INVALID_ARG (as ret_chunkwise_fwd, a null or aliased gradient), RET_ERR_UNSUPPORTED
 * (shape), RET_ERR_WORKSPACE (missing or smaller than the query). Supported wherever the forward supports
 * (d_k, d_v) and (w, d_k) for the input dtype, with w = d_v or, when d_v is too wide for a retention's d_k,
 * w = d_v / 2 (dq' and dk' are then sums of two retentions over the halves of d_v): BF16 d_k in {64, 128, 256}
 * and d_v in {64, 128, 256, 512} (the paper's d_k = 256, d_v = 512 included), every BF16 chunk size; F32 d_k in
 * {16, 32, 64}, d_v in {16, 32, 64, 128}, chunk in {16, 32, 64}. The workspace query returns 0 for other
 * shapes. Asynchronous on `stream`.
 */
size_t ret_chunkwise_bwd_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt);
ret_status_t ret_chunkwise_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk_out,
                               void* dv_out, int B, int N, int H, int dk, int dv, ret_dtype_t in_dt,
                               ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos0, int chunk,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel launch records for measurement tools: a caller-owned object, passed in ret_options_t.timer. While a
 * call holds one, every kernel it launches is bracketed by a pair of HIP events on the launch stream and
 * recorded in it (the library keeps no timing state of its own). ret_timer_query synchronises those events and
 * returns the total milliseconds and launch count recorded for kernels whose name equals `kernel` ("" or NULL =
 * all). Kernel names: "ret_chunk_seg", "ret_chunk_fused", "ret_chunk_fused_local", "ret_chunk_fused_scan",
 * "ret_chunk_wide", "ret_chunk_dma_local", "ret_chunk_dma_scan", "ret_chunk_dma" and "ret_rotate_qk" (bf16 input),
 * "ret_chunk_full", "ret_chunk_local", "ret_segment_scan" (fp32 input), "ret_parallel", "ret_recurrent_step",
 * "ret_msr_epilogue", "ret_permute_rotate" (gradients), "ret_norm_zseg", "ret_norm_rows", "ret_norm_scale",
 * "ret_norm_step" (score normalizations). A timer must not be attached to calls that are being captured into a
 * graph. One timer may be shared by calls on several threads.
 */
typedef struct ret_timer ret_timer_t;
ret_timer_t* ret_timer_create(void);   /* NULL if out of host memory */
void ret_timer_destroy(ret_timer_t* t);
int ret_timer_query(ret_timer_t* t, const char* kernel, double* total_ms, int64_t* launches);
void ret_timer_reset(ret_timer_t* t);

/*
 * Options of the *_ex entry points: the plan the library would otherwise choose, for measurements and for
 * tests that compare kernels and plans (every choice gives the result of the default plan up to rounding
 * order), and an optional timer. NULL options, or ret_options_default(), mean the library's own plan.
 *   segments     > 0: segments per sequence of the chained chunkwise kernels (capped at one per chunk); 0: planner
 *   target_wgs   > 0: workgroups the segment planner aims for; 0: the kernel's default
 *   prerotate    -1: planner; 0: q and k rotated while staging; 1: rotated once up front into the workspace
 *   onchip       -1 or 1: the on-chip segment kernel where segments fit (d_k <= 64, <= 256 tokens); 0: never
 *   variant      0: default kernel of the shape; d_v a multiple of 128: 3 = the wide-head kernel (32-token steps,
 *                q and k rotated once up front; the default for d_k = 256 where d_v is not a multiple of 256);
 *                d_k = 256: 5 = the LDS-loading wide-head kernels (d_v a multiple of 256, the default there:
 *                local passes, a scan, the full pass; gives way to 4 when q and k need rotating and the workspace
 *                has no room for rotated copies), 1 = 256 threads whose waves own 32 columns, 2 = 256 threads
 *                with d_v tiles of 64, 4 = 512 threads x 16 columns; d_k = 128: 4 = 512 threads x 16 columns
 *                (d_v tiles of 128, the default where d_v is a multiple of 128), 1 = 256 threads whose waves
 *                own 32 columns, 2 = 256 threads with d_v tiles of 64
 *   step_cw, step_wr, step_pairs   decode tile: columns per workgroup (16, 32, 64), rows per wave (16, 32, 64),
 *                pairs (0 planner, 1 one (b, h) per workgroup, 2 grouped); 0 = default
 *   bwd_direct   -1 or 1: gradients by the reversed traversal, with d_v blocks of dO and V read in place, where
 *                the kernels have them; 0: through reordered copies
 *   step_cache   0: the decode step streams the state (non-temporal loads and stores, one (b, h) per
 *                workgroup): right when each step's state has left the caches by the next step, as with a state
 *                per layer of a model; 1: the state's accesses may stay cached (grouped workgroups), faster when
 *                the same state is stepped again while it still fits the 256 MB Infinity Cache
 *   chain_spin   segment-chain wait limit in device clock ticks (100 MHz) without progress before a wait gives
 *                up; 0 = default (2^24 ticks, ~0.17 s); negative: every wait gives up at once (for testing the
 *                give-up path: the affected outputs become NaN and ret_chunkwise_check reports it)
 *   timer        launch records, or NULL
 */
typedef struct {
    int segments;
    int target_wgs;
    int prerotate;
    int onchip;
    int variant;
    int step_cw, step_wr, step_pairs;
    int bwd_direct;
    int step_cache;
    long long chain_spin;
    ret_timer_t* timer;
} ret_options_t;
void ret_options_default(ret_options_t* o);

/* ret_chunkwise_workspace_bytes, ret_chunkwise_bwd_workspace_bytes, ret_chunkwise_fwd, ret_chunkwise_msr_fwd,
 * ret_chunkwise_bwd, ret_recurrent_step and ret_recurrent_step_positions with options (NULL = defaults);
 * otherwise identical. A call planned with options wants the workspace its _ex query returns for them. */
size_t ret_chunkwise_workspace_bytes_ex(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt,
                                        const ret_options_t* opts);
size_t ret_chunkwise_bwd_workspace_bytes_ex(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt,
                                            const ret_options_t* opts);
ret_status_t ret_chunkwise_fwd_ex(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                                  int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                  const double* theta, int64_t pos0, int chunk, const float* state_in,
                                  float* state_out, void* workspace, size_t workspace_bytes, void* stream,
                                  const ret_options_t* opts);
ret_status_t ret_chunkwise_msr_fwd_ex(const void* q, const void* k, const void* v, const void* gate, void* y, int B,
                                      int N, int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                      ret_dtype_t gate_dt, const float* gamma, const double* theta, int64_t pos0,
                                      int chunk, const float* state_in, float* state_out, const float* gn_weight,
                                      const float* gn_bias, float eps, void* workspace, size_t workspace_bytes,
                                      void* stream, const ret_options_t* opts);
ret_status_t ret_chunkwise_bwd_ex(const void* q, const void* k, const void* v, const void* dout, void* dq,
                                  void* dk_out, void* dv_out, int B, int N, int H, int dk, int dv, ret_dtype_t in_dt,
                                  ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos0,
                                  int chunk, void* workspace, size_t workspace_bytes, void* stream,
                                  const ret_options_t* opts);
/*
 * ret_chunkwise_bwd after the forward, for a training step: fwd_workspace (fwd_workspace_bytes) is the workspace of
 * a ret_chunkwise_fwd call on the same q, k, v, gamma, theta, pos0 and chunk with no state_in (and the same
 * options), passed unchanged since that call. Where that call ran the LDS-loading d_k = 256 kernels (d_v a
 * multiple of 256, several segments, N a multiple of 32) it left there the rotated copies of q and k and the
 * state entering each segment, which the gradients need too: they are read instead of recomputed (the dq'
 * retentions enter their segments with those states, transposed); where it ran the streaming kernel's split
 * launches (d_k = d_v = 128, several segments) it left the states, read the same way. Otherwise, or with
 * fwd_workspace NULL, the call is ret_chunkwise_bwd_ex. Same results as ret_chunkwise_bwd_ex (bit for bit on the
 * LDS-loading kernels, whose forward ran the same products; to rounding on the streaming kernel, whose forward
 * formed the states in another order); a forward workspace from another call gives wrong gradients, which the
 * library cannot detect. fwd_workspace is only read.
 */
ret_status_t ret_chunkwise_bwd_saved_ex(const void* q, const void* k, const void* v, const void* dout, void* dq,
                                        void* dk_out, void* dv_out, int B, int N, int H, int dk, int dv,
                                        ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta,
                                        int64_t pos0, int chunk, const void* fwd_workspace, size_t fwd_workspace_bytes,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        const ret_options_t* opts);
ret_status_t ret_recurrent_step_ex(const void* q, const void* k, const void* v, void* o, float* state, int B, int H,
                                   int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                   const double* theta, int64_t pos, void* stream, const ret_options_t* opts);
ret_status_t ret_recurrent_step_positions_ex(const void* q, const void* k, const void* v, void* o, float* state,
                                             int B, int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                             const float* gamma, const double* theta, const int64_t* pos,
                                             void* stream, const ret_options_t* opts);

/*
 * Retention score normalizations ("Hybrid Architectures: RetNet and the Three Computation Paradigms", section
 * 8.5; RetNet paper summary, "Retention Score Normalization"), selected by `norm` (any combination, 0 = none):
 *   RET_NORM_SCALE   scores Q K^T divided by sqrt(d_k)
 *   RET_NORM_DECAY   each row of the decay matrix divided by the square root of its sum, sum_{i<=p} gamma^i
 *   RET_NORM_SCORES  each row of the (scaled) scores divided by max(|row sum|, 1)
 * The pages state them for the parallel form. Each is a positive factor per output row, so the normalized
 * output of the row at absolute position p is the plain one times c_p / den_p, with c_p the product of the
 * first two factors and den_p = max(|c_p q'_p . z_p|, 1) under RET_NORM_SCORES, where z_p = gamma z_{p-1} + k'_p
 * is the decayed sum of the rotated keys (q'_p . z_p is the row sum of the scores). Rows refer to the whole
 * sequence from its first token at position 0: a call that resumes at pos0 passes the key sum z [B, H, d_k]
 * (fp32) of the tokens before it, as it passes the state. GroupNorm cancels every factor (section 8.4).
 */
#define RET_NORM_SCALE 1
#define RET_NORM_DECAY 2
#define RET_NORM_SCORES 4

/*
 * Chunkwise form (as ret_chunkwise_fwd, options as the _ex calls) with the score normalizations. z_in: the key
 * sum before token 0 ([B, H, d_k] fp32 device, or NULL = zeros); z_out: the key sum after the last token (or
 * NULL; may equal z_in). pos0 >= 0. The workspace is required: ret_chunkwise_normalized_workspace_bytes (0 for
 * an unsupported shape) bytes, zero-filled before first use like the chunkwise workspace. Supported: as
 * ret_chunkwise_fwd. RET_ERR_INVALID_ARG also for norm outside 0..7 and misaligned z buffers,
 * RET_ERR_WORKSPACE for a missing or short workspace. Kernels: the chunkwise kernels, then "ret_norm_zseg",
 * "ret_segment_scan", "ret_norm_rows" and "ret_norm_scale" (the output scaled in place).
 */
size_t ret_chunkwise_normalized_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt,
                                                const ret_options_t* opts);
ret_status_t ret_chunkwise_normalized_fwd(const void* q, const void* k, const void* v, void* o, int B, int N, int H,
                                          int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                          const double* theta, int64_t pos0, int chunk, int norm,
                                          const float* state_in, float* state_out, const float* z_in, float* z_out,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          const ret_options_t* opts);

/*
 * One decode step (as ret_recurrent_step) with the score normalizations: the state S and the key sum z
 * ([B, H, d_k] fp32 device, required) are both updated in place, S <- gamma S + k'^T v, z <- gamma z + k', and
 * o = c_p (q' S) / den_p at position p = pos >= 0. Kernels: "ret_recurrent_step", then "ret_norm_step".
 */
ret_status_t ret_recurrent_step_normalized(const void* q, const void* k, const void* v, void* o, float* state,
                                           float* z, int B, int H, int dk, int dv, ret_dtype_t in_dt,
                                           ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos,
                                           int norm, void* stream, const ret_options_t* opts);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): ret_chunkwise_fwd (arguments as there, defaults for the options) with the workspace
 * taken from a device array the library owns, RET_NOALLOC_SCRATCH_BYTES on every GPU it runs on, held until the
 * process ends. The call allocates nothing; the first call on a device looks up the array's address and zeroes
 * its first 64 KB with a fill kernel on `stream`. The call uses the library's segment plan for the shape, with
 * the rotated copies of q and k only where they fit beside the chain (otherwise staging rotates: the same result
 * up to rounding). RET_ERR_WORKSPACE (before anything is enqueued) when the plan's segment chain needs more than
 * the array, or more counters and flags than its zeroed region holds. Every call on a GPU shares that GPU's
 * array and leaves its counters and flags zero: calls that overlap in time on one GPU (different streams or
 * threads) race and must not be made. The array is not visible to ret_chunkwise_check; a segment-chain wait
 * that gives up shows as NaN outputs.
 */
#define RET_NOALLOC_SCRATCH_BYTES (128u << 20)
ret_status_t ret_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int N, int H,
                                       int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                       const double* theta, int64_t pos0, int chunk, const float* state_in,
                                       float* state_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RETENTION_H */
