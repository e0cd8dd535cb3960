/*
 * zero_shard.h -- C ABI of libzeroshard.so: the owner-rank step of ZeRO-DP
 * optimizer-state and gradient partitioning (P_os / P_os+g) on one gfx950 GPU.
 *
 * The method (pages cited by title and section):
 *  - "ZeRO：大模型训练的内存优化革命", 3.1.1: with P_os each of the Nd
 *    data-parallel processes keeps and updates only 1/Nd of the optimizer
 *    state; at the end of the step the updated parameters are all-gathered.
 *  - same page, 3.1.2: with P_os+g the gradients are reduced only on the process
 *    that owns the partition (a reduce-scatter in place of the all-reduce).
 *  - same page, 3.2.2, and the "SC-2020 ZeRO" notes, "C_B: Constant Size
 *    Buffers": the reduce works through constant-size fused buffers.
 *  - "AI论文陪读·ZeRO" section 01 and the blog.vllbc.top ZeRO/DeepSpeed page
 *    (ledger and stage formulas): 2-byte params and grads, 12 bytes of fp32
 *    master / momentum / variance per parameter, 16 Psi in total, 16 Psi/Nd per
 *    rank when everything is partitioned.
 *  - "SC-2020 ZeRO" notes, "Where Did All the Memory Go?": the update runs on the
 *    fp32 master weights, which are then cast back to the 2-byte format.
 *
 * One call sequence per training step, on one handle:
 *     zero_bucket_reduce   x nbuckets  (ascending, contiguous, covering [0, S))
 *     zero_overflow_check            (synchronises the stream once)
 *     zero_adam_step                 (skipped when the check found inf/nan)
 * or the device-gated form (zero_adam_step_gated + zero_step_resolve), or the
 * device-resident form, whose whole step is one enqueue that a caller may
 * capture in a HIP graph (zero_device_begin, zero_step_device per step,
 * zero_device_end).
 *
 * Conventions for every function:
 *  - Returns a zero_status.  Arguments are validated before anything is
 *    launched; on any error nothing is launched and no handle state changes.
 *    zero_last_error() then holds a one-line explanation (thread-local).
 *  - No exceptions, aborts or prints cross this boundary.
 *  - "Device pointer" means memory of the device that was current when the
 *    handle was created.  Any 2-byte-aligned address is accepted for 2-byte
 *    arrays and any 4-byte-aligned address for fp32 arrays; the kernels peel
 *    unaligned heads and tails.  Performance: arrays whose offsets from a
 *    16-byte boundary differ in element count (for example a param slice one
 *    element off the master's phase) leave no common vector layout, and the
 *    update then runs element-wise, measured 12-23% slower for an offset
 *    2-byte array on MI355X.  A bucket reduce whose contributions do not
 *    share the output's phase modulo 16 bytes cuts each contribution's runs
 *    out of aligned 16-byte loads (any phase, 2-byte or fp32), measured 1-5%
 *    slower than aligned contributions.  Before any launch the library asks
 *    the HIP runtime about every array and contribution and refuses (INVALID_ARG)
 *    pageable host memory, another device's memory, and a range that runs
 *    past the end of its allocation; this is best effort (the runtime sees
 *    allocations, not the caller's tensors inside them), not a guarantee.
 *  - Every call that enqueues work must be made with the handle's device
 *    current (else ZERO_ERR_STATE) and, for a non-NULL stream, with a stream
 *    of that device (else ZERO_ERR_INVALID_ARG).
 *  - A handle is not thread-safe.  Separate handles are independent.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_SHARD_ABI_VERSION 1
/* Largest number of contributions one bucket reduce accepts. */
#define ZERO_MAX_CONTRIB 64

typedef enum {
    ZERO_OK = 0,
    ZERO_ERR_INVALID_ARG = 1, /* NULL pointer, value out of range, misaligned */
    ZERO_ERR_STATE = 2,       /* call out of order, bad coverage, dead handle */
    ZERO_ERR_HIP = 3,         /* the HIP runtime reported an error            */
    ZERO_ERR_OOM = 4,         /* workspace allocation failed                  */
    ZERO_ERR_UNSUPPORTED = 5  /* valid request the library does not implement */
} zero_status;

/* Storage format of grads, contributions and params: the 2-byte formats of
 * mixed precision (IEEE binary16 or bfloat16; an fp32 master copy is updated
 * and cast back), or ZERO_FP32, 4-byte storage (the pages' b = 4 case of the
 * (2b+K) Psi ledger): fp32 grads and contributions, and `master` is the fp32
 * parameter itself (param_shard must then be NULL). */
typedef enum { ZERO_FP16 = 1, ZERO_BF16 = 2, ZERO_FP32 = 3 } zero_lp_dtype;

/* Weight decay: decoupled (AdamW form, u += wd * p before p -= lr * u) or L2
 * (g += wd * p before the moments). */
typedef enum { ZERO_WD_DECOUPLED = 0, ZERO_WD_L2 = 1 } zero_wd_mode;

typedef struct zero_shard_s* zero_shard_t; /* opaque */

/*
 * The owner's shard.  Rank `rank` of `nd` owns elements [rank*S, (rank+1)*S) of
 * the flat Psi-element parameter space, S = ceil(psi / nd) (the last shard is
 * zero-padded).  All arrays hold S elements, are caller-owned device memory,
 * must not overlap, and must outlive the handle:
 *   master      : fp32 master weights (with ZERO_FP32 storage: the parameters)
 *   exp_avg     : Adam first moment; SGD momentum buffer (NULL: plain SGD)
 *   exp_avg_sq  : Adam second moment (NULL for SGD)
 *   grad_shard  : reduced gradient in the storage format (written by the reduce)
 *   param_shard : 2-byte params: the owner's slice of the parameter all-gather
 *                 buffer (written by the update); NULL with ZERO_FP32 storage
 * bucket_elems is C_B: every bucket but the last of a step holds exactly C_B
 * elements.
 */
typedef struct {
    int64_t psi;
    int32_t nd;
    int32_t rank;
    int64_t bucket_elems;
    zero_lp_dtype lp;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    void* grad_shard;
    void* param_shard;
} zero_shard_desc;

/* Textbook Adam (Kingma & Ba 2015, Algorithm 1); the pages give no formula.
 * Ranges: lr >= 0, 0 <= beta1 < 1, 0 <= beta2 < 1 (also after rounding to
 * fp32: a beta within 3e-8 of 1 is refused), eps > 0, weight_decay >= 0,
 * initial_step >= 0 (number of steps already applied). */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int32_t bias_correction; /* 0 or 1 */
    zero_wd_mode wd_mode;
    int64_t initial_step;
} zero_adam_hparams;

/* SGD, the K = 4 (with momentum) and K = 0 (plain) optimizers of the
 * blog.vllbc.top page's (2b+K) Psi extension; the pages give no formula.
 * Textbook heavy-ball SGD with L2 weight decay, per element (fp32, each
 * operation rounded to nearest even, no fused multiply-add):
 *     g = f32(grad) * fp32(1/scale) ;  g = g * coef   [clipping, else 1]
 *                                        [wd != 0: g = g + wd*p]
 *     with a momentum buffer: buf = mu*buf + g ; p = p - lr*buf
 *     plain:                  p = p - lr*g
 *     2-byte storage:         param = rne_2byte(p)
 * lr, mu, wd are the fp32 roundings of the values.  Ranges: lr >= 0,
 * 0 <= momentum < 1 (0 without a buffer), weight_decay >= 0,
 * initial_step >= 0. */
typedef struct {
    double lr, momentum, weight_decay;
    int64_t initial_step;
} zero_sgd_hparams;

/* Loss scaling (not on the pages).  dynamic = 1: an overflowing step halves
 * the scale (not below min_scale); growth_interval clean steps in a row double
 * it.  dynamic = 0: the scale stays at init_scale; an overflowing step is still
 * skipped.  The check unscales first: a step overflows when any unscaled
 * gradient f32(grad) * fp32(1/scale) is not finite, which includes a finite
 * stored value that a scale below 1 unscales past the fp32 range.
 * init_scale > 0 and min_scale > 0, each with a finite, non-zero fp32
 * reciprocal (about 3e-39 < scale < 1.4e45); growth_interval >= 1. */
typedef struct {
    double init_scale;
    int32_t dynamic;
    int32_t growth_interval;
    double min_scale;
} zero_loss_scale_cfg;

/* Result of a check or a step.  grad_norm is the L2 norm of the unscaled
 * shard gradient (fp64 accumulation; inf or nan when the step overflows).
 * step_t counts applied steps.  scale_used is the loss scale the gradients of
 * this step carry; scale_next the one the next step's gradients must carry. */
typedef struct {
    int32_t overflow;
    int32_t skipped;
    int64_t step_t;
    double grad_norm;
    double scale_used;
    double scale_next;
} zero_step_info;

/* Per-rank ledger.  Allocation of this library's shard, and the analytic per-rank
 * model-state bytes of stages 0..3 with their components (params, grads,
 * optimizer state) and the per-step communication volume in bytes, from the
 * blog.vllbc.top ZeRO/DeepSpeed page (stage formulas, Table 1, worked examples,
 * communication ledger):
 *   Stage 0 = (2b+K) Psi, Stage 1 = 2b Psi + K Psi/Nd,
 *   Stage 2 = b Psi + (b+K) Psi/Nd, Stage 3 = (2b+K) Psi/Nd,
 *   communication 2 b Psi for stages 0-2 and 3 b Psi for stage 3 (stage 1 with
 *   the step-end parameter gather: 3 b Psi). */
typedef struct {
    int64_t shard_elems;
    int64_t bytes_master, bytes_m, bytes_v, bytes_grad, bytes_param;
    int64_t bytes_shard_total; /* = 16 * S for an Adam shard of either storage */
    int64_t bytes_staging;     /* = n_contrib * C_B * (2 or 4): one bucket of contributions */
    double per_rank_stage[4];
    double comm_bytes_stage[4];
    double comm_bytes_stage1_with_gather;
    double comp_params[4], comp_grads[4], comp_optim[4];
} zero_state_bytes_t;

/*
 * Ledger for mixed-precision Adam (b = 2, K = 12).  Pure host arithmetic, no
 * device access.  psi >= 1, nd >= 1, n_contrib in [1, ZERO_MAX_CONTRIB],
 * bucket_elems >= 1, lp a zero_lp_dtype, out non-NULL.  The allocation fields
 * describe an Adam shard of storage format lp (with ZERO_FP32: 4-byte grads,
 * no param_shard).
 */
zero_status zero_state_bytes(int64_t psi, int32_t nd, int32_t n_contrib,
                             int64_t bucket_elems, zero_lp_dtype lp,
                             zero_state_bytes_t* out);

/*
 * Same ledger with the parameter byte width b (2 or 4) and optimizer multiplier
 * K (12 mixed-precision Adam, 8 fp32 Adam, 4 SGD with momentum, 0 SGD) of the
 * page's (2b+K) Psi extension (its group C examples).  The allocation fields
 * describe the shard a handle of storage lp and optimizer K holds: the fp32
 * master, fp32 optimizer arrays for K - 4 bytes (2-byte storage, where K counts
 * the master copy) or K bytes (ZERO_FP32 storage, where the master is the
 * parameter), the stored gradient and the 2-byte parameter.  With b matching lp
 * and Nd dividing psi, bytes_shard_total equals per_rank_stage[3].
 */
zero_status zero_state_bytes_ex(int64_t psi, int32_t nd, int32_t n_contrib,
                                int64_t bucket_elems, zero_lp_dtype lp,
                                int32_t param_bytes, int32_t k_optim,
                                zero_state_bytes_t* out);

/*
 * Create a handle bound to the current device.  Copies *desc, *hp and *ls.
 * Allocates a device workspace for the check's per-workgroup partials and the
 * device-resident step state, 8 bytes per 512 shard elements (per 256 with
 * ZERO_FP32 storage) plus 16 bytes per bucket plus 8.2 KiB (31.3 MB for a
 * 2e9-element 2-byte shard), and 256 bytes of
 * pinned host memory; touches none of the caller's arrays.
 * Errors: INVALID_ARG (NULL argument or pointer in desc, psi < 1, nd < 1, rank
 * outside [0, nd), bucket_elems < 1, unknown lp, misaligned or overlapping
 * arrays, hp or ls out of range), UNSUPPORTED (buckets so small that the
 * partials would need more than 2^25 slots), OOM, HIP.
 */
zero_status zero_shard_init(const zero_shard_desc* desc, const zero_adam_hparams* hp,
                            const zero_loss_scale_cfg* ls, zero_shard_t* out);

/*
 * Create a handle whose update rule is SGD (zero_sgd_step /
 * zero_sgd_step_gated) instead of Adam.  desc as for zero_shard_init, with
 * exp_avg the momentum buffer (NULL for plain SGD, which then needs
 * momentum == 0) and exp_avg_sq NULL.  The bucket reduce, the check, the merge
 * and zero_step_resolve are shared with Adam handles; the Adam step calls
 * refuse an SGD handle and the SGD step calls an Adam handle (ZERO_ERR_STATE).
 * Errors as zero_shard_init.
 */
zero_status zero_shard_init_sgd(const zero_shard_desc* desc, const zero_sgd_hparams* hp,
                                const zero_loss_scale_cfg* ls, zero_shard_t* out);

/*
 * Reduce one C_B bucket of the owner's shard from n_contrib contributions
 * ("ZeRO：大模型训练的内存优化革命" 3.1.2: gradients reduced on the owner).
 * contribs: host array of n_contrib device pointers, each to bucket_len
 * gradients in the storage format (contribution r, elements
 * [bucket_off, bucket_off+len) of the shard).  Per element: fp32 sum over
 * r = 0..R-1 in that order starting from +0, times fp32(1/R), stored in the
 * storage format (rounded to nearest even for the 2-byte formats) into
 * grad_shard[bucket_off + i].  The same pass records the overflow flag and the
 * squared norm of the unscaled values for zero_overflow_check.
 * Asynchronous on `stream`; contribution memory must stay valid until the
 * kernel has run.  Buckets of one step must be submitted in ascending,
 * contiguous order starting at 0; bucket_len must equal bucket_elems except
 * for the last bucket, which ends at S.  A contribution may be the bucket's
 * own slice of grad_shard (&grad_shard[bucket_off], an in-place reduce: each
 * element is read before it is written); otherwise contributions must not
 * overlap grad_shard, and none may overlap master, exp_avg, exp_avg_sq or
 * param_shard.
 * Performance: contributions whose base addresses lie exactly 512 MiB, 1 GiB
 * or 2 GiB apart hit the same DRAM banks in step and were measured 10-15%
 * slower on MI355X than ones at unrelated distances; a skew of 2-8 KiB
 * between them avoids it.  Eight fp16 contributions 360 MiB apart ran 4-8%
 * slower than the same eight 90 MiB or 358 MiB apart.
 * Errors: INVALID_ARG (NULL, n_contrib outside [1, 64], bucket outside [0, S),
 * bucket_len < 1 or > bucket_elems, pointer not aligned to its element size,
 * a contribution overlapping a shard array as above), STATE (dead handle,
 * bucket not the next one, step already checked, device-resident flow
 * active), HIP.
 */
zero_status zero_bucket_reduce(zero_shard_t h, const void* const* contribs, int32_t n_contrib,
                               int64_t bucket_off, int64_t bucket_len, void* stream);

/*
 * Finish the overflow check of the step: OR of "not finite" over the unscaled
 * gradient shard (f32(grad) * fp32(1/scale)) and its squared norm, summed over per-block
 * partials in a fixed order (bitwise reproducible).  If no bucket was reduced
 * this step, the stored grad_shard is scanned instead (for callers that fill
 * it themselves).  With clipping on, the same fold computes the step's
 * clipping coefficient.  Synchronises `stream` and fills *out (skipped =
 * overflow; step_t is the count before this step).  Calling it again before
 * the step call returns the same result.
 * Errors: INVALID_ARG (NULL out), STATE (dead handle, buckets cover only part
 * of the shard, device-resident flow active), HIP.
 */
zero_status zero_overflow_check(zero_shard_t h, void* stream, zero_step_info* out);

/*
 * Apply the step decided by zero_overflow_check.  On overflow: nothing is
 * launched, the states are unchanged, t is unchanged, and with dynamic scaling
 * the scale halves.  Otherwise t += 1 and, per element (fp32, every operation
 * rounded to nearest even, no fused multiply-add):
 *     g = f32(grad) * fp32(1/scale) ;  g = g * coef   [coef: clipping, else 1]
 *                                              [L2 mode: g = g + wd*p]
 *     m = b1*m + (1-b1)*g ;  v = b2*v + (1-b2)*(g*g)
 *     u = (m/bc1) / (sqrt(v/bc2) + eps)         [decoupled: u = u + wd*p]
 *     p = p - lr*u ;  param = rne_2byte(p)      [no param with fp32 storage]
 * with b1, b2, lr, eps, wd the fp32 roundings of the hyper-parameters,
 * bc_k = fp32(1 - b_k^t) (b_k^t a product of t fp64 factors; 1 when bias
 * correction is off).  hp = NULL uses the values given at init; otherwise *hp
 * is used for this step only (its initial_step is ignored).  Asynchronous on
 * `stream`; *out (may be NULL) gets the step's result.
 * Errors: STATE (dead handle, an SGD handle, no completed check this step),
 * INVALID_ARG (hp out of range), HIP.
 */
zero_status zero_adam_step(zero_shard_t h, const zero_adam_hparams* hp, void* stream,
                           zero_step_info* out);

/*
 * The SGD update of a checked step, as zero_adam_step is for Adam: skipped on
 * overflow, else t += 1 and the update of zero_sgd_hparams.  hp = NULL uses the
 * values given at init; otherwise *hp is used for this step only.
 * Errors: STATE (dead handle, not an SGD handle, no completed check this step),
 * INVALID_ARG (hp out of range), HIP.
 */
zero_status zero_sgd_step(zero_shard_t h, const zero_sgd_hparams* hp, void* stream,
                          zero_step_info* out);

/*
 * Device-gated check + SGD update, as zero_adam_step_gated is for Adam; finish
 * with zero_step_resolve.  Errors: STATE (also: not an SGD handle), INVALID_ARG,
 * HIP.
 */
zero_status zero_sgd_step_gated(zero_shard_t h, const zero_sgd_hparams* hp, void* stream);

/*
 * Global-norm clipping (not on the pages; the textbook rule, as PyTorch's
 * clip_grad_norm_): with max_grad_norm > 0, every later step multiplies the
 * unscaled gradient by coef = min(1, max_grad_norm / (norm + 1e-6)), norm the
 * step's gradient norm (grad_norm of zero_step_info), coef computed in fp64
 * and rounded to fp32, before weight decay and the moments:
 *     g = f32(grad) * fp32(1/scale) ;  g = g * coef ;  ...
 * A coefficient of 1 leaves the update bitwise unchanged.  The check computes
 * coef on the device from its own norm; after zero_overflow_merge it comes from
 * the merged global norm.  max_grad_norm = 0 turns clipping off (the default).
 * Errors: STATE (dead handle, a step in progress, device-resident flow
 * active), INVALID_ARG (negative or not finite).
 */
zero_status zero_shard_set_clip(zero_shard_t h, double max_grad_norm);

/*
 * Install the step's global check result on every rank before zero_adam_step,
 * for data parallelism across Nd processes: each rank runs
 * zero_overflow_check on its own partition, the caller all-reduces the
 * overflow flags (MAX) and the squared norms (SUM, from grad_norm^2) over the
 * ranks, and passes the outcome here, so that all ranks skip or apply the
 * step together ("ZeRO：大模型训练的内存优化革命" 3.1.1 and 3.1.2: every process
 * updates only its partition, so the decision must be shared).  Phase must be
 * CHECKED.  global_overflow must be 0 or 1 and not below this rank's own flag;
 * global_grad_norm is reported as the step's norm and, with clipping on, sets
 * the coefficient.  With global_overflow = 0 it must be finite and not below
 * this rank's own norm (relative slack 1e-9); with 1 it is only reported.
 * *out (may be NULL) gets the merged result.  Errors: STATE (dead handle, not
 * checked), INVALID_ARG (the handle is left unchanged).
 */
zero_status zero_overflow_merge(zero_shard_t h, int32_t global_overflow, double global_grad_norm,
                                zero_step_info* out);

/*
 * Device-gated check + Adam: the same step as zero_overflow_check followed by
 * zero_adam_step, without the stream stall between them.  After the buckets
 * of a step (or with none, scanning a caller-filled grad_shard), this
 * enqueues the check, an asynchronous copy of its result to pinned host
 * memory, and the Adam update for step t + 1; every Adam workgroup reads the
 * check's device result first and returns at once when it reports a
 * non-finite gradient, so a skipped step still changes no state.  The host
 * then calls zero_step_resolve, which waits only for the result copy (not for
 * the update) and commits t and the loss scale.  Callers that hold a stream
 * of steps in flight keep the GPU busy across the decision.  hp as in
 * zero_adam_step.
 * Errors: STATE (dead handle, an SGD handle, partial coverage, step already
 * checked or pending, device-resident flow active), INVALID_ARG (hp out of
 * range), HIP.
 */
zero_status zero_adam_step_gated(zero_shard_t h, const zero_adam_hparams* hp, void* stream);

/*
 * Finish a gated step: wait for its check result, fill *out (may be NULL) as
 * zero_adam_step would, advance t when the step was applied and update the
 * loss scale.  The update itself may still be running on the stream.  Until
 * this call, every other step call on the handle returns ZERO_ERR_STATE.
 * Errors: STATE (dead handle, no gated step pending), HIP.
 */
zero_status zero_step_resolve(zero_shard_t h, zero_step_info* out);

/*
 * Device-resident flow, for shards whose step is short enough that launches
 * and host round trips dominate.  zero_device_begin copies t, the loss scale
 * and the clean-step count into device memory (one kernel on `stream`); from
 * then on each zero_step_device enqueues a whole step on `stream`, with no
 * host synchronisation and no host-side state change:
 *   - the reduce of every C_B bucket of the shard from n_contrib contributions
 *     (contribs: host array of device pointers, each to S elements of the
 *     storage format; element i of contribution r is its value for shard
 *     element i; a contribution may be grad_shard itself, none may overlap
 *     it otherwise or overlap another shard array), or, with contribs = NULL
 *     and n_contrib = 0, the scan of a caller-filled grad_shard;
 *   - the fixed-order fold (norm, overflow, clipping coefficient), whose last
 *     lane then decides the step exactly as the host flows do (skip on
 *     overflow; otherwise t += 1 and the bias corrections of step t; the
 *     loss-scale rule) and advances the device copy of the counters;
 *   - the update (Adam or SGD with the init hyper-parameters), which reads
 *     the decision and the step's scalars from device memory and writes
 *     nothing on a skipped step.
 * When the step has at most 1024 per-workgroup partials and the update covers
 * the shard in one vector launch (every array 16-byte aligned, S a multiple of
 * 4), the update itself folds the partials in the same fixed order and takes
 * the same decision, and its workgroup 0 advances the counters: one launch
 * fewer, bitwise the same results (see zero_shard_inline_folds).
 * Because every launch argument is fixed for fixed contribution pointers,
 * the enqueue of zero_step_device may be captured in a HIP graph and
 * replayed; each replay is one step.  The loss scale the next step's
 * gradients must carry is only known on the device (or after
 * zero_device_end).  zero_device_end synchronises `stream`, copies the
 * counters back to the handle and leaves the flow; *out (may be NULL) gets the
 * last step's result (step_t and scale_next are the current values; with no
 * step run, overflow = 0 and grad_norm = 0).  While the flow is active every
 * other step, check, merge, counter and clipping call returns ZERO_ERR_STATE.
 * Errors: STATE (dead handle, flow not / already active, a step in progress),
 * INVALID_ARG (contribution pointers as for zero_bucket_reduce), HIP.
 */
zero_status zero_device_begin(zero_shard_t h, void* stream);
zero_status zero_step_device(zero_shard_t h, const void* const* contribs, int32_t n_contrib,
                             void* stream);
zero_status zero_device_end(zero_shard_t h, void* stream, zero_step_info* out);

/*
 * For callers that cannot allocate device memory (code that may not call
 * hipMalloc: serving loops and harnesses that forbid allocation): one whole
 * synchronous Adam step on a shard with no handle and no allocation.  The
 * result equals that of a handle created over the same desc, hp and ls, with
 * its counters set to *step_t, *scale and *good_steps and its clipping limit
 * to max_grad_norm, running zero_bucket_reduce over every C_B bucket (or, with
 * contribs = NULL and n_contrib = 0, the scan of a caller-filled grad_shard),
 * zero_overflow_check and zero_adam_step.  contribs as for zero_step_device
 * (n_contrib device pointers, each to S elements).  *step_t, *scale and
 * *good_steps are the counters before the step (as zero_shard_get_counters
 * returns them) and are updated in place; hp->initial_step and
 * ls->init_scale are not used.  *out (may be NULL) gets the step's result.
 * The check's partials, its fold and its result live in a 4 MiB static array
 * of device memory, one per GPU, held until the process ends: a shard whose
 * check needs more than 523,232 partial slots is refused (about 267M 2-byte
 * elements with 8 or more contributions, up to 800M with fewer and buckets of
 * at least 3.9M elements, 134M fp32 elements with 8 or more).  Every call on
 * a GPU shares that GPU's array, so calls that overlap on one GPU (other
 * threads, or other streams before this call's update has run) race; calls in
 * order on one stream do not.  Synchronises
 * `stream` once (for the check); the update stays asynchronous on it.
 * Errors: INVALID_ARG (as zero_shard_init and zero_step_device, counters out
 * of range, max_grad_norm negative or not finite, a shard too large for the
 * scratch), STATE (another device current than the stream's), UNSUPPORTED
 * (device ordinal 64 or above), HIP.
 */
zero_status zero_adam_step_noalloc(const zero_shard_desc* desc, const zero_adam_hparams* hp,
                                   const zero_loss_scale_cfg* ls, double max_grad_norm,
                                   const void* const* contribs, int32_t n_contrib,
                                   int64_t* step_t, double* scale, int64_t* good_steps,
                                   void* stream, zero_step_info* out);

/* Diagnostic: *count = the zero_step_device calls on this handle, since init,
 * that enqueued the fold inside the update instead of a fold launch.
 * Errors: STATE (dead handle), INVALID_ARG (count NULL). */
zero_status zero_shard_inline_folds(zero_shard_t h, int64_t* count);

/* Step counter, current loss scale and clean-step count (for checkpoints).
 * STATE while the device-resident flow is active (the values live on the
 * device until zero_device_end). */
zero_status zero_shard_get_counters(zero_shard_t h, int64_t* step_t, double* scale,
                                    int64_t* good_steps);
/* Restore them between steps (phase must be idle, device-resident flow not
 * active).  step_t >= 0, good_steps >= 0, scale as init_scale of
 * zero_loss_scale_cfg. */
zero_status zero_shard_set_counters(zero_shard_t h, int64_t step_t, double scale,
                                    int64_t good_steps);

/* Release the workspace.  The caller's arrays are untouched.  The handle is
 * dead afterwards; a second destroy returns ZERO_ERR_STATE. */
zero_status zero_shard_destroy(zero_shard_t h);

const char* zero_status_str(zero_status s);
const char* zero_last_error(void);
int zero_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
