/*
 * meo.h -- C ABI of the fused optimizer-step library for AMD MI355X (gfx950).
 *
 * One call runs one optimizer step over a list of parameter tensors:
 *
 *   meo_adafactor_step  Adafactor with the factored second moment (row and column
 *                       statistics for tensors of two or more dims, a full
 *                       statistic for 1-D tensors), RMS clipping, relative step
 *                       size, parameter scaling, weight decay and an optional
 *                       first moment.
 *   meo_came_step       CAME: Adafactor's factored statistic plus a factored
 *                       confidence statistic of the update's instability.
 *   meo_lamb_step       LAMB: Adam moments with a per-tensor trust ratio.
 *
 * Source of the method: the Colossal-AI distributed-optimizers page
 * ("Colossal-AI 分布式优化器全解析", blog.gitcode.com): section "Step 3" (Adafactor
 * defaults, relative step and its errors, optional first moment, the factored
 * rule and the statistic shapes), the note after "Step 5" (beta2t schedule, RMS
 * clipping, scale_parameter), the "four optimizers" table (row * col
 * factorisation, CAME's confidence matrix, LAMB's layer-wise trust ratio), and
 * the DistributedLAMB / DistributedCAME paragraphs (defaults, validation).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor, state and workspace pointers are DEVICE pointers owned by the
 *   caller, in memory of the current device allocated through HIP (hipMalloc,
 *   hipMallocManaged, or an allocator built on them such as PyTorch's).
 *   Parameters and states (float32, or bf16 where noted) are updated in place;
 *   gradients are read only. Every buffer is contiguous and row-major (last dim
 *   innermost). Buffers must not alias one another. fp32 buffers need 4-byte
 *   alignment and bf16 ones 2-byte alignment; 16-byte alignment (and, for
 *   factored tensors, cols % 8 == 0) selects the vectorised path.
 * - `stream` is a hipStream_t (NULL = the default stream). The step is enqueued
 *   asynchronously on it and never synchronises the host; results are valid
 *   once the stream reaches that point. Calls that overlap on different streams
 *   must not share a workspace.
 * - `step` is the 1-based index of the step being taken (the caller increments
 *   its counter before the call); all tensors of one call share it.
 * - Every argument is validated on the host before anything is enqueued: a
 *   failing call leaves every tensor untouched. Besides values, shapes, dtypes
 *   and alignment, a step checks with the HIP runtime that the workspace
 *   (every call) and every tensor and state (when a launch table is built)
 *   lies inside one device allocation of the current device (MEO_EWORKSPACE,
 *   MEO_EMEMORY); meo_*_validate does not touch the device and skips this. Return value: MEO_OK, or a
 *   negative MEO_E* code with a message available from meo_last_error().
 * - Tensors with zero elements are skipped.
 * - `workspace` is device scratch of at least meo_*_workspace_size() bytes,
 *   256-byte aligned, valid only while the enqueued work runs; no value is kept
 *   in it between calls.
 * - The library keeps a cache of device-side launch tables keyed on the tensor
 *   list (shapes and pointers), up to 64 lists. A call over a list that is not
 *   cached allocates device memory for its tables (hipMalloc) and copies them
 *   synchronously; past 64 lists the least recently used table is freed
 *   (hipFree, which waits for the device). Calls over a cached list allocate
 *   nothing. meo_release_plans() frees the cache. meo_adafactor_step_noalloc
 *   never allocates.
 */
#ifndef MEO_H
#define MEO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEO_VERSION 8

/* Return codes. */
#define MEO_OK          0
#define MEO_EINVAL     (-1) /* hyperparameter or step out of range            */
#define MEO_ESHAPE     (-2) /* inconsistent batch/rows/cols/ndim or too large */
#define MEO_EDTYPE     (-3) /* unsupported dtype                              */
#define MEO_ENULL      (-4) /* required pointer is NULL                       */
#define MEO_EWORKSPACE (-5) /* workspace NULL, misaligned or too small        */
#define MEO_EALIGN     (-6) /* tensor pointer misaligned for its dtype        */
#define MEO_EHIP       (-7) /* HIP runtime error while enqueueing             */
#define MEO_EMEMORY    (-8) /* a tensor or state pointer is not device memory
                               of the current device, or the range it
                               describes passes the end of its allocation   */

/* Element types. */
#define MEO_F32  0
#define MEO_BF16 1
#define MEO_I8   2   /* state_dtype only: 8-bit group-quantized first moment */

/*
 * One parameter tensor and its gradient, viewed as [batch, rows, cols]:
 * ndim >= 2 -> rows = size of dim -2, cols = size of dim -1, batch = product of
 * the leading dims; the Adafactor/CAME statistics are factored per matrix
 * (page "Step 3": tensors of two or more dimensions keep factored statistics).
 * ndim 0 or 1 -> batch = rows = 1, cols = numel; full (unfactored) statistic.
 * LAMB ignores the view and treats the tensor as one flat layer.
 */
typedef struct meo_tensor {
    void*       param;       /* param_dtype [batch*rows*cols], updated in place */
    const void* grad;        /* grad_dtype [batch*rows*cols], read only        */
    int64_t     batch;
    int64_t     rows;
    int64_t     cols;
    int32_t     ndim;        /* the tensor's number of dims (0, 1, 2, ...)     */
    int32_t     param_dtype; /* MEO_F32 or MEO_BF16                            */
    int32_t     grad_dtype;  /* MEO_F32 or MEO_BF16                            */
    int32_t     state_dtype; /* element type of this tensor's exp_avg (first
                                moment): MEO_F32, MEO_BF16 or MEO_I8; every
                                other state array is float32                   */
} meo_tensor;

/*
 * 16-bit storage (the memory-saving 16-bit path that the page's DistributedCAME
 * paragraph says CAME supports). A bf16 parameter or first moment is widened to
 * float32 on load, every step computes in float32, and each new value is rounded
 * to the nearest bf16 (ties to even) when it is formed: later uses within the same
 * step (the update, CAME's instability, LAMB's direction) see the rounded first
 * moment, exactly what the next step will read back. Statistics, second moments
 * and the workspace stay float32. A bf16 pointer must be 2-byte aligned.
 *
 * 8-bit first moment (state_dtype MEO_I8): the GaLore section's 8-bit optimizer
 * base keeps its states block-wise quantized, and the ms-swift page's Q-GaLore
 * code quantizes in groups of 128 values with one absmax scale each. exp_avg
 * then holds int8 codes [numel] and exp_avg_scale one float32 scale per group of
 * 128 consecutive values (row-major order) [ceil(numel / 128)]; a last short
 * group stands alone. Each step dequantizes (code * scale), updates in float32,
 * and re-quantizes: scale = max|m| / 127 over the group, code = m / scale rounded
 * half to even (0 for a zero group). The rest of the step uses the dequantized
 * new value. A group holding a NaN or an infinity stores scale NaN and codes 0.
 * Factored tensors (Adafactor and CAME, ndim >= 2) need cols % 128 == 0, so that
 * no group crosses a row (MEO_ESHAPE otherwise). Both states start at zero.
 */

/* ------------------------------------------------------------------ Adafactor */

/* Hyperparameters. Defaults (meo_adafactor_defaults) are the page's, section
 * "Step 3": lr = None (has_lr = 0), eps = (1e-30, 1e-3), clip_threshold = 1.0,
 * decay_rate = -0.8, beta1 = None (has_beta1 = 0), weight_decay = 0.0,
 * scale_parameter = 1, relative_step = 1, warmup_init = 0.
 * The learning rate is min(1e-2, 1/sqrt(step)) with relative_step (1e-2 becomes
 * 1e-6*step with warmup_init), else lr; with scale_parameter it is multiplied by
 * max(eps2, RMS(param)). beta2t = 1 - step**decay_rate (note after "Step 5").
 * Errors (MEO_EINVAL): has_lr with relative_step ("Cannot combine manual lr and
 * relative_step=True options"), warmup_init without relative_step
 * ("warmup_init=True requires relative_step=True"), neither lr nor
 * relative_step, clip_threshold <= 0, negative eps, non-finite values. */
typedef struct meo_adafactor_hparams {
    double  lr;
    double  eps1;
    double  eps2;
    double  clip_threshold;
    double  decay_rate;
    double  beta1;
    double  weight_decay;
    int32_t has_lr;
    int32_t has_beta1;
    int32_t scale_parameter;
    int32_t relative_step;
    int32_t warmup_init;
    int32_t reserved;
} meo_adafactor_hparams;

/* Per-tensor state, caller-allocated, zero before the first step; float32 except
 * exp_avg, whose type is the tensor's state_dtype.
 * Names follow the page ("Step 3"). */
typedef struct meo_adafactor_state {
    void*  exp_avg;        /* state_dtype [numel]; required iff has_beta1       */
    float* exp_avg_sq_row; /* [batch*rows]; factored tensors only               */
    float* exp_avg_sq_col; /* [batch*cols]; factored tensors only               */
    float* exp_avg_sq;     /* [numel]; 1-D tensors only                          */
    float* exp_avg_scale;  /* [ceil(numel / 128)]; iff exp_avg is MEO_I8          */
    float* param_sumsq;    /* [1]; meo_adafactor_step_carry only (else ignored)  */
} meo_adafactor_state;

void   meo_adafactor_defaults(meo_adafactor_hparams* hp);
size_t meo_adafactor_workspace_size(int32_t n, const meo_tensor* tensors);
int    meo_adafactor_validate(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                              const meo_tensor* tensors, const meo_adafactor_state* states);
int    meo_adafactor_step(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                          const meo_tensor* tensors, const meo_adafactor_state* states,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The same step, carrying sum(X^2) from one step to the next.
 *
 * scale_parameter multiplies the step size by RMS(X) of the parameter before
 * the update (the note after "Step 5": the step size scales with the
 * parameter's RMS). That parameter is exactly what the previous step stored, so
 * this call sums the squares of the parameter it stores, in the same pass that
 * stores it, and leaves the sum in each tensor's param_sumsq[0] (float32, the
 * sum over the whole tensor of the stored values: bf16 parameters as rounded).
 * The next call can then take RMS(X) from it instead of reading the parameter
 * a second time, which saves 4 (fp32) or 2 (bf16) bytes per parameter of HBM
 * traffic per step.
 *
 * param_sumsq_valid (host flag, for the whole list):
 *   1  every tensor's param_sumsq holds the sum that the previous carry call
 *      left for it, and nothing has written the parameter since. RMS(X) comes
 *      from it; the parameter is read only by the apply pass.
 *   0  RMS(X) is taken from the parameter, as meo_adafactor_step does (the
 *      first step, or after anything else wrote a parameter, e.g. a checkpoint
 *      load). Use 0 whenever in doubt: a stale sum silently scales the step by
 *      the wrong RMS.
 * In both cases param_sumsq is rewritten with the new parameter's sum. Results
 * equal meo_adafactor_step's up to the order of the sum of squares (relative
 * difference of RMS(X) around 1e-7).
 *
 * Every tensor with elements needs param_sumsq (4-byte aligned device memory,
 * MEO_ENULL / MEO_EALIGN / MEO_EMEMORY otherwise); entries of tensors with zero
 * elements are not touched. With scale_parameter = 0 the step uses no RMS(X):
 * param_sumsq is neither read nor written and the call equals
 * meo_adafactor_step. Everything else (validation, workspace, stream, errors)
 * is as for meo_adafactor_step. */
int    meo_adafactor_step_carry(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                                const meo_tensor* tensors, const meo_adafactor_state* states,
                                int32_t param_sumsq_valid, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The Adafactor step (meo_adafactor_step) for callers that cannot allocate device
 * memory: code that runs under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. It takes no workspace and calls no hipMalloc, hipFree or
 * other allocating routine: the launch tables and the workspace of the call live
 * in a scratch array of MEO_NOALLOC_SCRATCH_BYTES that the library's code object
 * holds on each GPU it runs on (allocated when the code is loaded on that GPU and
 * kept until the process ends). The tables are built on the host (cached per
 * distinct list in host memory) and copied into the scratch on `stream` before the
 * passes; the same kernels then run in the same order, so the results are those
 * of meo_adafactor_step, bit for bit.
 *
 * Limits: a list whose launch tables and workspace need more than
 * MEO_NOALLOC_SCRATCH_BYTES is refused (MEO_EWORKSPACE) before anything runs; a
 * Llama-7B decoder layer needs about 22 MB, the whole 7B list about 0.7 GB (use
 * meo_adafactor_step for it). Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (on different streams, or from different threads
 * before the earlier one's work has run) race and must be serialised by the
 * caller. Nothing in the scratch is carried from one call to the next, and
 * nothing in it needs to start at zero (every pass writes what a later pass
 * reads). Arguments, validation, stream semantics and errors are otherwise as for
 * meo_adafactor_step.
 *
 * Graph capture: the call records no memset. The table upload is a
 * hipMemcpyAsync whose source is the library's host copy of that list's tables,
 * kept for the 16 distinct lists this entry point saw last (meo_release_plans
 * does not drop them). A captured call replays that copy from the same host
 * memory, so a graph may be replayed only while its list is among those 16.
 * Capture itself is not exercised by the tests. */
#define MEO_NOALLOC_SCRATCH_BYTES (64u << 20)
int    meo_adafactor_step_noalloc(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                                  const meo_tensor* tensors, const meo_adafactor_state* states, void* stream);

/* ----------------------------------------------------------------------- CAME */

/* Hyperparameters. Defaults (meo_came_defaults) are the page's DistributedCAME
 * paragraph: eps = (1e-30, 1e-16), clip_threshold = 1.0,
 * betas = (0.9, 0.999, 0.9999), weight_decay = 0.0. The page's lr default is
 * None, but CAME has no relative step, so lr must be given (has_lr = 1).
 * beta2 is constant (no decay schedule); no bias correction. Errors
 * (MEO_EINVAL): no lr, lr < 0, a beta outside [0, 1), clip_threshold <= 0,
 * negative eps, non-finite values. */
typedef struct meo_came_hparams {
    double  lr;
    double  eps1;
    double  eps2;
    double  clip_threshold;
    double  beta1;
    double  beta2;
    double  beta3;
    double  weight_decay;
    int32_t has_lr;
    int32_t reserved;
} meo_came_hparams;

/* Per-tensor state, zero before the first step; float32 except exp_avg
 * (state_dtype). The confidence statistic is factored like the squared-gradient
 * one. */
typedef struct meo_came_state {
    void*  exp_avg;         /* state_dtype [numel], always required              */
    float* exp_avg_sq_row;  /* [batch*rows]; factored only                       */
    float* exp_avg_sq_col;  /* [batch*cols]; factored only                       */
    float* exp_avg_res_row; /* [batch*rows]; factored only                       */
    float* exp_avg_res_col; /* [batch*cols]; factored only                       */
    float* exp_avg_sq;      /* [numel]; 1-D only                                  */
    float* exp_avg_scale;   /* [ceil(numel / 128)]; iff exp_avg is MEO_I8         */
} meo_came_state;

void   meo_came_defaults(meo_came_hparams* hp);
size_t meo_came_workspace_size(int32_t n, const meo_tensor* tensors);
int    meo_came_validate(const meo_came_hparams* hp, int64_t step, int32_t n,
                         const meo_tensor* tensors, const meo_came_state* states);
int    meo_came_step(const meo_came_hparams* hp, int64_t step, int32_t n,
                     const meo_tensor* tensors, const meo_came_state* states,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------- LAMB */

/* Hyperparameters. Defaults (meo_lamb_defaults) are the page's DistributedLAMB
 * paragraph: lr = 1e-3, betas = (0.9, 0.999), eps = 1e-6, weight_decay = 0,
 * bias_correction = 1. The page says lr, eps and betas are validated: MEO_EINVAL
 * for lr < 0, eps < 0, a beta outside [0, 1), or non-finite values.
 * Per tensor: m, v Adam moments (bias-corrected if asked), direction
 * d = m_hat / (sqrt(v_hat) + eps) + weight_decay * param, trust ratio
 * ||param|| / ||d|| (1 when either is 0), param -= lr * ratio * d. */
typedef struct meo_lamb_hparams {
    double  lr;
    double  beta1;
    double  beta2;
    double  eps;
    double  weight_decay;
    int32_t bias_correction;
    int32_t reserved;
} meo_lamb_hparams;

/* Per-tensor state, zero before the first step; exp_avg is state_dtype,
 * exp_avg_sq float32. */
typedef struct meo_lamb_state {
    void*  exp_avg;       /* state_dtype [numel] */
    float* exp_avg_sq;    /* [numel] */
    float* exp_avg_scale; /* [ceil(numel / 128)]; iff exp_avg is MEO_I8 */
} meo_lamb_state;

void   meo_lamb_defaults(meo_lamb_hparams* hp);
size_t meo_lamb_workspace_size(int32_t n, const meo_tensor* tensors);
int    meo_lamb_validate(const meo_lamb_hparams* hp, int64_t step, int32_t n,
                         const meo_tensor* tensors, const meo_lamb_state* states);
int    meo_lamb_step(const meo_lamb_hparams* hp, int64_t step, int32_t n,
                     const meo_tensor* tensors, const meo_lamb_state* states,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------- row-sharded steps */

/*
 * One rank's share of a step whose tensors are split by rows across ranks, the
 * layout of the page's tensor-parallel and ZeRO versions ([CAI] "Step 4":
 * setup_distributed; row statistics reduced within the group, column statistics
 * gathered). Each rank holds whole rows of every factored tensor (rows
 * [r0, r0 + rows) of dim -2, all columns) and a contiguous element range of every
 * 1-D tensor (LAMB: of every tensor). A factored tensor stays factored whatever its
 * share: a shard of one row is still one row of a factored matrix (the page makes
 * CAME's H = 1 shards factored for the same reason).
 *
 * A step is three stages:
 *   1. meo_*_shard_stats: the shard's own statistics (Adafactor: its row statistic
 *      and, for 1-D tensors, its full second moment; LAMB: its moments) plus a
 *      record of partial sums in `partials`;
 *   2. the caller sums `partials` over all ranks (an all-reduce with SUM of one flat
 *      float32 buffer, e.g. RCCL over xGMI); the library does no communication;
 *   3. meo_*_shard_apply with the reduced `partials`: the replicated statistics
 *      (Adafactor's column statistic, kept whole on every rank and updated
 *      identically), the per-tensor scalars and the update of the shard.
 * The same hparams, step, tensors, shards and states go to both calls.
 *
 * `partials` (float32, meo_*_partials_size() floats, contiguous; every entry is a
 * sum, so summing the ranks' buffers gives the whole tensor's values), per tensor
 * in list order:
 *   Adafactor, factored: [B][W] sum of G^2 + eps1 over the shard's rows, [B][W] sum
 *     of G^2 / R_i (R_i the new row statistic), [B] sum of the new R_i, [1] sum of
 *     X^2 of the shard;
 *   Adafactor, 1-D: [1] sum of U^2 = G^2 / V, [1] sum of X^2;
 *   LAMB: [1] sum of X^2, [1] sum of d^2 (the update direction).
 * Every tensor has its record, also where the rank holds none of it (rows = 0 or
 * an empty range): the stats call writes zeros there, so all ranks' buffers line
 * up; such a rank neither uses nor updates that tensor's column statistic.
 * Factored Adafactor shards need row-complete rows (cols % 8 == 0, cols <= 12288,
 * param and grad 16-byte aligned; MEO_ESHAPE otherwise). The workspace is scratch
 * for each call; nothing in it is carried from the stats call to the apply call.
 * Errors as for the whole-tensor step, plus MEO_ENULL for NULL shards or partials,
 * MEO_ESHAPE for rows_total below the shard's size, and MEO_EMEMORY when partials
 * is not device memory of the record's size.
 */
typedef struct meo_shard {
    int64_t rows_total;  /* rows of the whole matrix (dim -2) for a factored tensor;
                            elements of the whole tensor for a 1-D one (LAMB: for
                            every tensor); >= the shard's own                       */
} meo_shard;

size_t meo_adafactor_partials_size(int32_t n, const meo_tensor* tensors);
int    meo_adafactor_shard_stats(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                                 const meo_tensor* tensors, const meo_shard* shards,
                                 const meo_adafactor_state* states, float* partials,
                                 void* workspace, size_t workspace_bytes, void* stream);
int    meo_adafactor_shard_apply(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                                 const meo_tensor* tensors, const meo_shard* shards,
                                 const meo_adafactor_state* states, const float* partials,
                                 void* workspace, size_t workspace_bytes, void* stream);
/* The row-sharded Adafactor step with the carried sum(X^2) of
 * meo_adafactor_step_carry. Each rank's param_sumsq holds the sum of squares of
 * its own shard: meo_adafactor_shard_apply_carry leaves it (the sum over the rows
 * the rank stored), and meo_adafactor_shard_stats_carry with
 * param_sumsq_valid = 1 puts it into the record's sum of X^2 instead of reading the
 * shard's parameter, so the all-reduce still yields the whole tensor's sum.
 * param_sumsq_valid = 0 reads the parameter as meo_adafactor_shard_stats does.
 * The flag must be the same on every rank (it selects what the record holds, not
 * how it is summed). param_sumsq requirements and the scale_parameter = 0 case are
 * as for meo_adafactor_step_carry; everything else as for the plain shard calls. */
int    meo_adafactor_shard_stats_carry(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                                       const meo_tensor* tensors, const meo_shard* shards,
                                       const meo_adafactor_state* states, int32_t param_sumsq_valid,
                                       float* partials, void* workspace, size_t workspace_bytes,
                                       void* stream);
int    meo_adafactor_shard_apply_carry(const meo_adafactor_hparams* hp, int64_t step, int32_t n,
                                       const meo_tensor* tensors, const meo_shard* shards,
                                       const meo_adafactor_state* states, const float* partials,
                                       void* workspace, size_t workspace_bytes, void* stream);
/* CAME takes two exchanges. meo_came_shard_stats writes `partials` (the Adafactor
 * record above; its sum of X^2 is 0); after the all-reduce, meo_came_shard_moment
 * folds it (column statistic, clip divisor), updates the first moment of the shard
 * (1-D tensors finish their step here), finishes the confidence row statistic
 * (whole rows) and writes `confidence`: per factored tensor [B][W] sums of the
 * instability E = (U - M)^2 + eps2 over the shard's rows and [B] sums of the new
 * confidence row statistic; 1-D tensors have no entry. After its all-reduce,
 * meo_came_shard_apply folds it into the replicated confidence column statistic
 * and applies the step to the shard. */
size_t meo_came_partials_size(int32_t n, const meo_tensor* tensors);
size_t meo_came_confidence_size(int32_t n, const meo_tensor* tensors);
int    meo_came_shard_stats(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* tensors,
                            const meo_shard* shards, const meo_came_state* states, float* partials,
                            void* workspace, size_t workspace_bytes, void* stream);
int    meo_came_shard_moment(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* tensors,
                             const meo_shard* shards, const meo_came_state* states, const float* partials,
                             float* confidence, void* workspace, size_t workspace_bytes, void* stream);
int    meo_came_shard_apply(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* tensors,
                            const meo_shard* shards, const meo_came_state* states, const float* confidence,
                            void* workspace, size_t workspace_bytes, void* stream);
size_t meo_lamb_partials_size(int32_t n, const meo_tensor* tensors);
int    meo_lamb_shard_stats(const meo_lamb_hparams* hp, int64_t step, int32_t n,
                            const meo_tensor* tensors, const meo_shard* shards,
                            const meo_lamb_state* states, float* partials,
                            void* workspace, size_t workspace_bytes, void* stream);
int    meo_lamb_shard_apply(const meo_lamb_hparams* hp, int64_t step, int32_t n,
                            const meo_tensor* tensors, const meo_shard* shards,
                            const meo_lamb_state* states, const float* partials,
                            void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------------- GaLore */

/* GaLore: AdamW on a low-rank projection of each 2-D gradient (Colossal-AI
 * distributed-optimizers page, section on GaLore's special configuration, with
 * its table of group fields; ms-swift page, section on low-rank projection).
 *
 * A tensor with ndim == 2 (batch 1) is projected. With m = rows, n = cols and
 * r = min(rank, min(m, n)) (the effective rank), the projection takes one side of
 * the matrix: proj_type MEO_GALORE_STD takes the shorter one (m >= n: the right
 * side, else the left), MEO_GALORE_REVERSE_STD the longer one (the page's table
 * names "std" and "reverse_std"). On the right side d = n and D = m, on the left
 * d = m and D = n:
 *   - every update_proj_gap steps, at steps t with (t - 1) % update_proj_gap == 0,
 *     the projector U (d x r, orthonormal columns) is recomputed from the current
 *     gradient: the leading r right singular vectors of G (right side) or left
 *     singular vectors (left side), each signed so that its entry of largest
 *     magnitude is positive;
 *   - project(): R = G U (right) or R = G^T U (left), D x r;
 *   - AdamW on R: exp_avg <- b1 exp_avg + (1 - b1) R, exp_avg_sq <- b2 exp_avg_sq
 *     + (1 - b2) R^2, N = (exp_avg / (1 - b1^t)) / (sqrt(exp_avg_sq / (1 - b2^t)) + eps);
 *   - project_back() and update: X <- X (1 - lr wd) - lr scale (N U^T) (right),
 *     X <- X (1 - lr wd) - lr scale (U N^T) (left).
 * Every other tensor takes the same AdamW update on its elements, without scale.
 * The moments persist across projector refreshes.
 *
 * Storage of a projected tensor: grad bf16 (MEO_EDTYPE otherwise; the products
 * run on bf16 matrix cores with fp32 accumulation), param fp32 or bf16,
 * state_dtype MEO_F32; exp_avg and exp_avg_sq float32 [D][r]; the projector in
 * bf16 (rounded to nearest even) twice, as `projector` [d][r] and as its
 * transpose `projector_t` [r][d], both written by the refresh and read by every
 * step. N is split into two bf16 planes (its nearest bf16 and the bf16 of the
 * remainder) for the back-projection. r must not exceed 256 (MEO_EINVAL).
 * Non-projected tensors: param and grad fp32 or bf16, exp_avg and exp_avg_sq
 * float32 [numel], projector pointers NULL. All states start at zero.
 *
 * Defaults (meo_galore_defaults): rank 256, update_proj_gap 200, scale 0.25,
 * proj_type std (the page's table); lr 1e-3, betas (0.9, 0.999), eps 1e-8,
 * weight_decay 0 (the pages name these fields without values). Errors
 * (MEO_EINVAL): lr < 0, a beta outside [0, 1), eps < 0, rank < 1,
 * update_proj_gap < 1, an unknown proj_type, non-finite values.
 */
#define MEO_GALORE_STD          0
#define MEO_GALORE_REVERSE_STD  1
typedef struct meo_galore_hparams {
    double  lr;
    double  beta1, beta2;
    double  eps;
    double  weight_decay;
    int32_t rank;
    int32_t update_proj_gap;
    double  scale;
    int32_t proj_type;   /* MEO_GALORE_STD or MEO_GALORE_REVERSE_STD */
    int32_t reserved;    /* 0 */
} meo_galore_hparams;

typedef struct meo_galore_state {
    float* exp_avg;      /* [D][r] projected, [numel] otherwise                */
    float* exp_avg_sq;   /* [D][r] projected, [numel] otherwise                */
    void*  projector;    /* bf16 [d][r]; NULL for tensors that are not 2-D      */
    void*  projector_t;  /* bf16 [r][d]; NULL for tensors that are not 2-D      */
} meo_galore_state;

void    meo_galore_defaults(meo_galore_hparams* hp);
/* Effective rank r of a tensor (0 when it is not projected). */
int32_t meo_galore_rank(const meo_galore_hparams* hp, const meo_tensor* tensor);
size_t  meo_galore_workspace_size(const meo_galore_hparams* hp, int32_t n, const meo_tensor* tensors);
int     meo_galore_validate(const meo_galore_hparams* hp, int64_t step, int32_t n, const meo_tensor* tensors,
                            const meo_galore_state* states);
/* One step of the list; refreshes the projectors first when the step is due. */
int     meo_galore_step(const meo_galore_hparams* hp, int64_t step, int32_t n, const meo_tensor* tensors,
                        const meo_galore_state* states, void* workspace, size_t workspace_bytes, void* stream);
/* Recomputes the projectors of the list's 2-D tensors from their gradients, as a
 * due step does before projecting, and changes nothing else. */
int     meo_galore_refresh(const meo_galore_hparams* hp, int32_t n, const meo_tensor* tensors,
                           const meo_galore_state* states, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------- per-tensor scalars */

/*
 * For tests and diagnostics. A step call over a list leaves, for every tensor
 * with elements, 8 float32 per-tensor scalars in the workspace; they can be read
 * back once the call's work on the stream has completed and before the
 * workspace is used again (the next call overwrites them). meo_*_scalar_offsets
 * writes, for each of the n tensors, the offset in floats from the workspace's
 * start of that tensor's 8 slots, or -1 for a tensor with zero elements; the
 * offsets depend on the list (shapes and the 16-byte alignment of param and
 * grad), exactly as the step call lays the workspace out. Host only; MEO_OK,
 * MEO_ENULL (tensors or offsets NULL with n > 0) or MEO_ESHAPE.
 *
 * Slots (from the note after "Step 5" of the Colossal-AI distributed-optimizers
 * page: RMS clipping and scale_parameter; the "four optimizers" table and the
 * DistributedLAMB paragraph: the layer-wise trust ratio):
 *   [0] Adafactor: alpha, the step size rho times max(eps2, RMS(param)) with
 *       scale_parameter (else rho); CAME: 1
 *   [1] alpha / kappa (Adafactor, CAME)
 *   [2] decoupled weight-decay factor: weight_decay * alpha (Adafactor),
 *       weight_decay * lr (CAME)
 *   [3] RMS of the unclipped update U = G / sqrt(V_hat) (Adafactor, CAME)
 *   [4] RMS(param) before the update (Adafactor; written with scale_parameter);
 *       LAMB: ||param||_2
 *   [5] LAMB: ||d||_2 of the update direction
 *   [6] kappa = max(1, RMS(U) / clip_threshold), the clip divisor (Adafactor, CAME)
 *   [7] LAMB: the trust ratio ||param|| / ||d|| (1 when either norm is 0)
 * Slots an optimizer does not name hold unspecified values. The row-sharded
 * calls use the same slots (their values then come from the reduced sums).
 */
int meo_adafactor_scalar_offsets(int32_t n, const meo_tensor* tensors, int64_t* offsets);
int meo_came_scalar_offsets(int32_t n, const meo_tensor* tensors, int64_t* offsets);
int meo_lamb_scalar_offsets(int32_t n, const meo_tensor* tensors, int64_t* offsets);

/* ----------------------------------------------------------------- utilities */

/* Message of the last failing call on this thread ("" if none). The pointer
 * stays valid until the next call on the same thread. */
const char* meo_last_error(void);

/* Frees the cached launch tables. Waits for the device first. */
void meo_release_plans(void);

/* MEO_VERSION of the built library. */
int meo_version(void);

/* ----------------------------------------------------------- pass timing
 * For measurement only. While enabled (meo_profile_enable(1)), every step call
 * also records a hipEvent on its stream before its first pass and after each
 * pass, so that the time of each pass can be read back. The events sit between
 * the passes' launches; they add no device work to the passes themselves.
 * Pass ids are 0 .. MEO_NUM_PASSES-1, named by meo_pass_name().
 * meo_profile_collect() waits for the recorded events, adds each pass's
 * elapsed milliseconds into total_ms[id] and its launch count into
 * launches[id] (both arrays of MEO_NUM_PASSES entries, caller-owned host
 * memory, zeroed by the caller), and forgets the events. Returns MEO_OK or
 * MEO_EHIP. Not for use under graph capture. */
#define MEO_NUM_PASSES 17
int         meo_profile_enable(int on);
const char* meo_pass_name(int id);
int         meo_profile_collect(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MEO_H */
