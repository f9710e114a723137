/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer-step library.
 *
 * The Muon step for one layer matrix is: momentum update, Newton-Schulz
 * orthogonalization of the whole momentum matrix, weight update with the
 * orthogonalized momentum. Sources are web reports of NVIDIA's blog post
 * "Advancing Emerging Optimizers for Accelerated LLM Training":
 *   [zh] wiki.whaty.org, "使用 NVIDIA Megatron 推进新兴优化器以加速 LLM 训练"
 *   [de] ki-news-radar.de news summary (running text)
 *   [pt] cafecomtech.com, "NVIDIA Megatron ganha suporte a Muon ..."
 *
 * Conventions for every entry point:
 *   - Matrices are row-major device buffers described by muon_mat. Element
 *     (r, c) lives at data + (r * ld + c) * sizeof(dtype).
 *   - All work is enqueued asynchronously on the calling thread's stream
 *     (muon_set_stream); validation runs synchronously on the host first.
 *   - Validation is all-or-nothing: on any error status nothing is enqueued
 *     and no buffer is touched. muon_last_error() then describes the problem.
 *   - The library never allocates or frees device memory. Scratch space is a
 *     caller-owned workspace (muon_set_workspace). The library keeps no
 *     pointer after return other than in work already enqueued; buffers must
 *     stay alive until that work has finished on the stream.
 *   - The precision path follows the dtype: all-float32 matrices run the
 *     float32 path (float32 arithmetic throughout); all-bfloat16 matrices run
 *     the bfloat16 matrix-core path (bf16 operands, fp32 accumulation, fp32
 *     epilogues, bf16 intermediates; A*A from bf16(A) by default, from A
 *     split into bf16 hi + lo with MUON_AA_SPLIT).
 *   - NaN and Inf in the inputs propagate; nothing is masked.
 *   - State set by muon_set_* is per host thread.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1, /* null pointer, bad count, bad option value  */
  MUON_ERR_SHAPE = 2,       /* rows/cols <= 0, ld < cols, bad col_blocks,
                               dimension beyond the supported maximum       */
  MUON_ERR_DTYPE = 3,       /* unknown dtype or a mix of dtypes             */
  MUON_ERR_ALIGN = 4,       /* data not aligned to its element size, or a
                               workspace not aligned to 256 bytes           */
  MUON_ERR_ALIAS = 5,       /* written matrices overlap other matrices, or
                               a matrix reaches into the workspace           */
  MUON_ERR_WORKSPACE = 6,   /* no workspace, or smaller than required       */
  MUON_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed   */
} muon_status;

typedef enum muon_dtype { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* One layer matrix: rows x cols, row pitch ld (elements, ld >= cols).
 * data must be aligned to its element size. Rows that start on 16-byte
 * boundaries (16-byte aligned data and ld * sizeof(dtype) a multiple of 16)
 * take the vectorized load/store path; any other pitch takes a slower
 * element-by-element path.
 * col_blocks is read only under MUON_NS_BLOCKWISE and MUON_NS_DISTRIBUTED
 * and ignored otherwise. Blockwise: the columns are split into col_blocks
 * equal blocks, each orthogonalized on its own. Distributed: col_blocks is
 * the number of column shards P (the same for every matrix of the call). In
 * both, col_blocks must divide cols; 0 or 1 means the whole matrix. */
typedef struct muon_mat {
  void *data;
  int64_t rows;
  int64_t cols;
  int64_t ld;
  int32_t dtype;      /* muon_dtype */
  int32_t col_blocks; /* >= 0 */
} muon_mat;

/* Mode bits. */
#define MUON_NS_FULL 0x000u      /* orthogonalize each whole matrix          */
#define MUON_NS_BLOCKWISE 0x001u /* orthogonalize col_blocks column blocks of
                                    each matrix independently                */
#define MUON_NS_DISTRIBUTED 0x002u /* the whole-matrix result, computed as
                                    col_blocks column shards that share one
                                    Gram per iteration (see below)           */
#define MUON_PACK_RR 0x000u      /* matrices enter the grouped launches in the
                                    order given (round robin)                */
#define MUON_PACK_COST 0x010u    /* ... in descending cost order             */
#define MUON_AA_PLAIN 0x000u     /* A*A and b A from bf16-rounded A
                                    (1 product); honoured up to 12
                                    iterations, above that the split form
                                    runs (the plain form's error nears the
                                    bf16 path's 2e-2 bound at ~20)          */
#define MUON_AA_SPLIT 0x100u     /* A*A and b A from A as bf16 hi + lo halves
                                    (3 products: hi hi + hi lo + lo hi);
                                    about 1.3x less error, 3x the A*A work   */

/* Limits: the smaller dimension of a matrix (or block) at most 32768, the
 * larger at most 4194304; iters at most 64; n_mats at most 1048576. */

/*
 * Newton-Schulz orthogonalization of n_mats matrices, in place.
 *
 * Defines: each whole matrix X (or, in blockwise mode, each column block) is
 * oriented wide (transposed when rows > cols), normalized to
 * X / (||X||_F + eps), then `iters` times: A = X X^T, B = b A + c A A,
 * X = a X + B X (three products per iteration, the first two symmetric, only
 * their upper-triangle tiles computed and mirrored), then oriented back.
 * Three matrix products per iteration: [zh] section "Distributed mode", [de];
 * the first two symmetric rank-k products computed as full mirrored matrices:
 * [zh] section "SYRK 和融合的 all-reduce"; usually five iterations: [zh]
 * section "Duplicated mode"; blockwise mode: [zh] section "Distributed mode"
 * (blockwise paragraph), [pt] section "2. Newton-Schulz distribuído".
 *
 *   descs   host array of n_mats descriptors (read during the call only);
 *           descs[i].data is overwritten with the result in its own dtype.
 *           All descriptors must share one dtype and must not overlap.
 *   iters   >= 0; 0 means normalize only.
 *   coeffs  host array {a, b, c}; NULL means {3.4445, -4.7750, 2.0315}.
 *           All finite, c != 0 and b / c finite (B is formed as
 *           c (A A + (b / c) A)); otherwise MUON_ERR_INVALID_ARG.
 *   mode    MUON_NS_* | MUON_PACK_* | MUON_AA_* bits.
 *
 * MUON_NS_DISTRIBUTED simulates, on one GPU, the pages' tensor-parallel
 * ("distributed") mode ([zh] section "Distributed mode"; [pt] section
 * "2. Newton-Schulz distribuído"): each matrix (rows <= cols; pass a tall
 * matrix transposed) is split into P = col_blocks column shards X_p, every
 * matrix of the call with the same P. Per iteration each shard forms its
 * partial Gram X_p X_p^T; the partials are exchanged as float32 upper
 * triangles ([zh] section "SYRK 和融合的 all-reduce") and summed in shard
 * order, standing in for the all-reduce; every shard then forms B from the
 * full A (redundantly, as every rank would) and updates its own columns. The
 * norm is the whole matrix's. The result is the full-matrix Newton-Schulz up
 * to rounding order. bf16: the Gram kernel writes each partial tile by tile,
 * straight from its accumulators, as the upper 256 x 256 tiles in float32
 * (tile-packed), and the sum, 16 bytes per access, leaves as the bf16 A that
 * every shard of the matrix reads; float32: packed rows (row i holding
 * columns i .. mp - 1, mp the padded row count).
 *   eps     taken from muon_set_step_options (default 1e-7).
 * n_mats == 0 is a no-op returning MUON_OK.
 */
muon_status muon_ns_batched(const muon_mat *descs, int32_t n_mats, int32_t iters,
                            const float coeffs[3], uint32_t mode);

/*
 * One Muon optimizer step for n_mats layer matrices.
 *
 * Per matrix: M <- beta * M + G (momentum buffer; [zh] section
 * "分布式 Newton-Schulz" names the whole momentum-buffer matrix as the input of
 * the orthogonalization), X = M (or G + beta * M with nesterov != 0),
 * O = NewtonSchulz(X) exactly as muon_ns_batched defines it, then
 * W <- W - lr * O (each GPU updates the weights it owns with the
 * orthogonalized momentum: [zh] section "Duplicated mode").
 *
 *   params  host array of n_mats descriptors of W (updated in place).
 *   grads   host array of n_mats descriptors of G (read only).
 *   moms    host array of n_mats descriptors of M (updated in place).
 *           params[i], grads[i], moms[i] must have the same rows, cols and
 *           dtype (pitches may differ). W and M of any matrix may not overlap
 *           any other buffer of the call. Blockwise splits use
 *           params[i].col_blocks.
 *   lr, beta   scalars (finite).
 *   nesterov   0 or 1.
 * iters, coeffs, eps and mode come from muon_set_step_options.
 */
muon_status muon_step(const muon_mat *params, const muon_mat *grads, const muon_mat *moms,
                      int32_t n_mats, float lr, float beta, int32_t nesterov);

/*
 * muon_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same step, with the same arguments, results and error codes, but with
 * scratch space taken from a device array inside the library instead of the
 * caller's workspace (muon_set_workspace is ignored). Nothing is allocated or
 * freed on the call path.
 *
 *   - The array holds MUON_NOALLOC_SCRATCH_BYTES; matrices are processed in
 *     consecutive groups that fit it. A matrix (or column block) that alone
 *     needs more returns MUON_ERR_WORKSPACE (a 2048 x 7168 bf16 matrix needs
 *     about 143 MB, so it fits, one at a time).
 *   - Each GPU holds its own copy of the array from the first call on it
 *     until the process ends; its address is looked up on that first call.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (two streams, two threads) race and must be serialized
 *     by the caller. The array needs no clearing between calls.
 *   - Phase timing (muon_set_phase_timing) is not recorded for these calls.
 */
#define MUON_NOALLOC_SCRATCH_BYTES (256u << 20)
muon_status muon_step_noalloc(const muon_mat *params, const muon_mat *grads, const muon_mat *moms,
                              int32_t n_mats, float lr, float beta, int32_t nesterov);

/* Stream for this thread's subsequent calls (a hipStream_t); NULL selects
 * the null stream. */
muon_status muon_set_stream(void *hip_stream);

/* Workspace bytes that let every matrix (or block) of the call be in flight
 * at once, for muon_ns_batched(descs, ...) or muon_step(descs=params, ...).
 * A smaller workspace still works down to muon_workspace_min_size: the
 * matrices are then processed in consecutive groups. */
muon_status muon_workspace_size(const muon_mat *descs, int32_t n_mats, uint32_t mode,
                                size_t *bytes);

/* Smallest workspace with which the call can run (the largest single matrix
 * or block). */
muon_status muon_workspace_min_size(const muon_mat *descs, int32_t n_mats, uint32_t mode,
                                    size_t *bytes);

/* Caller-owned device workspace for this thread's subsequent calls.
 * device_ptr must be 256-byte aligned; (NULL, 0) clears it. The contents
 * need no initialization. Two calls in flight on different streams must use
 * different workspaces. No matrix of a call may reach into
 * [device_ptr, device_ptr + bytes) (first to last byte of each matrix):
 * such a call returns MUON_ERR_ALIAS. */
muon_status muon_set_workspace(void *device_ptr, size_t bytes);

/* Options used by muon_step (and eps by muon_ns_batched) on this thread.
 * Defaults: iters 5, coeffs {3.4445, -4.7750, 2.0315}, eps 1e-7,
 * mode MUON_NS_FULL | MUON_PACK_COST | MUON_AA_PLAIN. coeffs NULL keeps the
 * current coefficients; non-NULL coefficients follow the rule of
 * muon_ns_batched (finite, c != 0, b / c finite). eps must be finite and
 * >= 0. */
muon_status muon_set_step_options(int32_t iters, const float coeffs[3], float eps,
                                  uint32_t mode);

/* Text of the last error on this thread ("" after success). The pointer is
 * valid until the next call on this thread. */
const char *muon_last_error(void);

/*
 * Per-kernel timing, for measurement. While enabled (enable != 0), every
 * kernel launch the library makes on this thread is bracketed by a pair of
 * HIP events recorded on the call's stream. muon_phase_times() waits for the
 * recorded events, writes each kernel kind's summed milliseconds and launch
 * count into ms[8] and launches[8] (order: prep, norm, gram, aa, bx, finish,
 * adamw, reduce; either pointer may be NULL) and clears the record. Events are created by
 * the library on first use and reused; no device memory is allocated.
 */
muon_status muon_set_phase_timing(int32_t enable);
muon_status muon_phase_times(double ms[8], int64_t launches[8]);

/*
 * Host-only description of how a call would be scheduled, as JSON written
 * into buf (NUL-terminated, truncated to len): the processing order of
 * matrices/blocks (orientation, padded shape, cost), the groups that fit the
 * given workspace size, and per group the uniform-shape segments and the
 * tile counts of each grouped launch. Launches nothing; needs no GPU.
 * *needed receives the full length including the NUL.
 */
muon_status muon_plan_info(const muon_mat *descs, int32_t n_mats, int32_t iters, uint32_t mode,
                           size_t workspace_bytes, char *buf, size_t len, size_t *needed);

/*
 * One AdamW step for n_mats matrices: the optimizer the pages measure Muon
 * against (Table 1 of the blog post: AdamW and Muon training throughput on
 * the same models), for a like-for-like optimizer-step time on one GPU. The
 * pages do not restate it; this is the published algorithm (Adam's
 * bias-corrected moments, Kingma and Ba, Algorithm 1; decoupled weight
 * decay, Loshchilov and Hutter, Algorithm 2), element by element:
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   W <- W (1 - lr weight_decay) - lr / (1 - beta1^step) * m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 * in float32 arithmetic.
 *   params      W, updated in place; all F32 or all BF16.
 *   grads       g, read only; the dtype of params.
 *   exp_avg     m, float32, updated in place.
 *   exp_avg_sq  v, float32, updated in place.
 *               The four descriptors of matrix i share rows and cols
 *               (pitches may differ); written buffers may not overlap any
 *               other buffer of the call.
 *   lr, weight_decay  finite;  beta1, beta2 in [0, 1);  eps finite, > 0;
 *   step        1-based count of this step (bias correction), >= 1.
 * Needs no workspace. n_mats == 0 is a no-op. Launches are timed under the
 * "adamw" kind of muon_phase_times.
 */
muon_status muon_adamw_step(const muon_mat *params, const muon_mat *grads, const muon_mat *exp_avg,
                            const muon_mat *exp_avg_sq, int32_t n_mats, float lr, float beta1,
                            float beta2, float eps, float weight_decay, int32_t step);

/*
 * Placement of whole matrices on `ranks` data-parallel ranks, each of which
 * would then run muon_step on its share (layer-wise distribution: [zh]
 * section "逐层分布式优化器"). Perfect balance is not reachable in general;
 * the pages place matrices round robin today and expect estimated costs to
 * do better ([zh] section "负载均衡"):
 *   MUON_PLACE_RR   matrix i goes to rank i mod ranks;
 *   MUON_PLACE_LPT  matrices in descending cost (ties: lower index first)
 *                   each go to the rank with the least cost so far (ties:
 *                   lower rank), the longest-processing-time-first rule.
 *   costs      host array of n_mats finite costs >= 0 (measured times, or the
 *              cost model of muon_plan_info), read only.
 *   ranks      1 .. 65536.
 *   owner      host array of n_mats, receives each matrix's rank.
 *   load       host array of `ranks` (or NULL), receives each rank's summed
 *              cost.
 *   imbalance  (or NULL) receives max(load) / mean(load); 1 when every cost
 *              is 0.
 * Host only; launches nothing. Invalid arguments: MUON_ERR_INVALID_ARG,
 * nothing written.
 */
#define MUON_PLACE_RR 0u
#define MUON_PLACE_LPT 1u
muon_status muon_place(const double *costs, int32_t n_mats, int32_t ranks, uint32_t policy,
                       int32_t *owner, double *load, double *imbalance);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */
