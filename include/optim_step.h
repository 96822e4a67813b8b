/*
 * optim_step.h -- C ABI of the fused, multi-tensor AdamW-family optimizer
 * step for AMD Instinct MI355X (gfx950).
 *
 * Sources for the operations (web pages, cited by title and section):
 *  [BNB]  "Fix decoupled weight decay ordering in the CUDA Adam/AdEMAMix
 *         kernels" (bitsandbytes PR #2040)
 *  [AO]   "4 bit Adam should support non constant lr" (pytorch/ao #730)
 *  [MINI] "Adam-mini <> DTensor" (Adam-mini issue #14)
 *  [LTN]  "FusedAdam & PyTorch Lightning AMP" (Lightning issue #15501)
 *  [TE]   "Support store_param_remainders feature from Apex in TE Fused
 *         Adam" (TransformerEngine PR #1408)
 *
 * Conventions for every entry point:
 *  - Returns OPTIM_OK (0) or a positive OPTIM_E* code; optim_last_error()
 *    then holds a message for the calling thread.  Nothing aborts, throws or
 *    blocks the host; a failed call has launched nothing.
 *  - "dev" pointers are device (HBM) pointers owned by the caller; "host"
 *    pointers are host memory owned by the caller.  The library allocates no
 *    device memory: plan metadata, per-step scalars and reduction partials
 *    live in a caller-owned workspace (or, for optim_plan_create_static, in
 *    the library's static device workspace).  The only host allocation is
 *    the plan object itself.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *    device-side effect is enqueued on it, in order; nothing reads device
 *    memory back to the host, so a whole step can be captured in a HIP graph.
 *  - Updates are in place.  Gradients are read only and must not alias any
 *    buffer the step writes.
 */
#ifndef OPTIM_STEP_H
#define OPTIM_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define OPTIM_OK 0
#define OPTIM_EINVAL 1       /* bad argument or hyperparameter             */
#define OPTIM_EALIGN 2       /* pointer not aligned to its element size    */
#define OPTIM_EDTYPE 3       /* dtype combination not supported            */
#define OPTIM_EWORKSPACE 4   /* workspace missing, misaligned or too small */
#define OPTIM_EUNSUPPORTED 5 /* valid request this library does not do    */
#define OPTIM_EHIP 6         /* a HIP runtime call failed                  */

/* ---- enumerations ------------------------------------------------------ */
enum { OPTIM_F32 = 0, OPTIM_BF16 = 1, OPTIM_F16 = 2 };
/* state layouts (optim_plan_opts.state_layout)                            */
enum { OPTIM_LAYOUT_SEPARATE = 0, OPTIM_LAYOUT_INTERLEAVED = 1 };
enum {
    OPTIM_ALGO_ADAMW = 0,
    OPTIM_ALGO_ADEMAMIX = 1,
    OPTIM_ALGO_ADAM_MINI = 2,
    OPTIM_ALGO_BLOCKWISE = 3,
    OPTIM_ALGO_BLOCKWISE_ADEMAMIX = 4,
    OPTIM_ALGO_LION = 5,
    OPTIM_ALGO_LAMB = 6
};
/* Adam-mini partition of a tensor ([MINI], AdamWMini constructor/step). */
enum { OPTIM_MINI_FULL_V = 0, OPTIM_MINI_HEAD = 1, OPTIM_MINI_SCALAR = 2 };
enum { OPTIM_SCHED_NONE = 0, OPTIM_SCHED_COSINE = 1 };

/* ---- tensor list -------------------------------------------------------
 * n tensors; every array below is a host array of length n (or NULL where
 * the algorithm does not use it) whose entries are device pointers.
 *
 *  numel        elements per tensor, 0 .. 2^48 (0: an empty tensor, skipped)
 *  param        F32: float[numel]; BF16: uint16 bf16 patterns[numel];
 *               F16 (with master only): uint16 fp16 patterns[numel]
 *  grad         F32 float[numel] or BF16 uint16[numel] (grad_dtype)
 *  m, v         float[numel] first / second moment (AdamW, AdEMAMix, LAMB,
 *               Adam-mini FULL_V).  Adam-mini HEAD/SCALAR: m float[numel]
 *               and v float[numel/head_numel] (one shared v per block).
 *               Lion: m only (v NULL).  AdamW / AdEMAMix in the
 *               interleaved moment layout (opts->state_layout): m holds all
 *               of a tensor's moments, v and m2 are NULL.
 *  m2           float[numel] AdEMAMix slow EMA; NULL otherwise
 *  remainder    int16[numel] low halves of the fp32 master ([TE]); required
 *               when param_dtype is BF16, NULL otherwise
 *  qm, qv       blockwise codes: 8-bit one byte per element; 4-bit two per
 *               byte (element 2i in the low nibble); m signed, v unsigned
 *  absmax_m/_v  float[ceil(numel/block)] per-block scale of qm / qv
 *  qm2,         blockwise AdEMAMix only: codes of the slow EMA m2 (signed,
 *  absmax_m2    layout as qm) and their per-block scale; NULL otherwise
 *  scale_m,     AdamW plans with 16-bit states (opts->state_dtype): one
 *  scale_v      device float per tensor, the scale of its stored m / v
 *               (1.0 for a fresh state); m and v are then uint16 patterns
 *  master       float[numel] fp32 master weights of a BF16 or F16 model
 *               param ([TE] review: master weights beside a low-precision
 *               model param), AdamW and AdEMAMix only: the step updates the
 *               master and rewrites param as the master rounded to nearest
 *               even.  remainder must be NULL then.  NULL otherwise.
 *  weight_decay per-tensor decoupled decay (>= 0)
 *  mini_kind    Adam-mini only: OPTIM_MINI_*
 *  head_numel   Adam-mini only: block length for HEAD (must divide numel);
 *               ignored otherwise
 * All device arrays must be aligned to their element size; 16-byte aligned
 * tensors take the vector path, others a per-element path.                */
typedef struct optim_tensor_list {
    int32_t n;
    const int64_t *numel;
    void *const *param;
    const void *const *grad;
    void *const *m;
    void *const *v;
    void *const *m2;
    void *const *remainder;
    void *const *qm;
    void *const *qv;
    float *const *absmax_m;
    float *const *absmax_v;
    const double *weight_decay;
    const int32_t *mini_kind;
    const int64_t *head_numel;
    int32_t param_dtype;
    int32_t grad_dtype;
    void *const *qm2;
    float *const *absmax_m2;
    float *const *master;
    float *const *scale_m;
    float *const *scale_v;
} optim_tensor_list;

/* Plan options (NULL = all defaults).
 *  bits/block  blockwise algorithms only (8-bit: block 64, 128 or 256;
 *              4-bit: block 128, 256 or 512)
 *  grid        0 (default): one workgroup per work unit; > 0: a persistent
 *              grid of that many workgroups walking the units grid-stride
 *  tile        elements per work unit, a power of two in [1024, 2^24]
 *              (blockwise: at least 2048); 0 = 2048 (AdamW, AdEMAMix
 *              with fp32 moments and Lion on lists of more than 2^20 and at
 *              most 2^24 elements 4096; Adam-mini, LAMB and fp16 states 4096;
 *              blockwise 8-bit 4096 in the separate state layout, 8192 in
 *              the interleaved one, 4-bit 8192, and blockwise AdEMAMix
 *              8-bit 8192, 4-bit 16384).  AdamW, AdEMAMix and Lion lay
 *              runs of tensors of at most min(tile, 2048) / 2 elements end
 *              to end in shared units of up to min(tile, 2048) elements
 *  state_dtype AdamW only: OPTIM_F32 (0, default) fp32 moments; OPTIM_F16
 *              or OPTIM_BF16 16-bit moments with a per-tensor scale
 *              ([TE] review: state scaling), see optim_step_adamw
 *  segment_bytes  Adam-mini only: the step runs its block-sum, finalize
 *              and update kernels once per segment, a run of consecutive
 *              whole tensors with shared v holding at most this many
 *              gradient bytes (a larger tensor forms a segment alone), or a
 *              run of full-v tensors; 0 = 384 MiB (the gradients are read
 *              twice, the second time mostly from the Infinity Cache).  Results
 *              do not depend on it.  Negative: OPTIM_EINVAL.
 *  state_layout  OPTIM_LAYOUT_SEPARATE (0, default): every state is an
 *              array of its own.  OPTIM_LAYOUT_INTERLEAVED (1), for
 *              OPTIM_ALGO_ADAMW and OPTIM_ALGO_ADEMAMIX with fp32 moments:
 *              the moments of a tensor share its m array, in blocks of 1024
 *              elements -- block b holds m, then v (then AdEMAMix's m2) of
 *              elements [1024 b, 1024 b + 1024), 1024 floats each, the last
 *              block whole too -- so m holds K * 1024 * ceil(numel / 1024)
 *              floats (K = 2 AdamW, 3 AdEMAMix); v and m2 must be NULL.
 *              Element e's m sits at m[K * 1024 * (e / 1024) + e % 1024], its
 *              v 1024 floats further, its m2 2048.  The values are those of
 *              separate arrays, bit for bit; the step streams one (AdamW) or
 *              two (AdEMAMix) arrays fewer.  (A storage choice of this
 *              library, not of the pages, which keep each state a tensor of
 *              its own.)  Lion, LAMB, Adam-mini, blockwise AdEMAMix and
 *              16-bit moments refuse the interleaved layout
 *              (OPTIM_EUNSUPPORTED).
 *              For OPTIM_ALGO_BLOCKWISE, OPTIM_LAYOUT_SEPARATE: qm / qv and
 *              absmax_m / absmax_v are four arrays.
 *              OPTIM_LAYOUT_INTERLEAVED (1): each element's m and v codes
 *              sit side by side in qm -- 8-bit: 2 bytes per element, m
 *              first; 4-bit: 1 byte per element, m in the low nibble, v in
 *              the high one -- and absmax_m holds (absmax of m, absmax of v)
 *              per block (8-byte aligned); qv and absmax_v must be NULL.
 *              The values are those of the separate layout, bit for bit; the
 *              step streams two arrays fewer.  The quantize / dequantize
 *              helpers below work on separate arrays.                     */
typedef struct optim_plan_opts {
    int32_t bits;
    int32_t block;
    int32_t grid;
    int32_t tile;
    int32_t state_dtype;
    int64_t segment_bytes;
    int32_t state_layout;
} optim_plan_opts;

/* Hyperparameters, validated as in [MINI] AdamWMini's constructor:
 * 0 <= beta < 1, eps >= 0.  The learning rate is a device scalar.        */
typedef struct optim_adamw_hp {
    double beta1, beta2, eps;
} optim_adamw_hp;

typedef struct optim_ademamix_hp {
    double beta1, beta2, beta3, alpha, eps;
} optim_ademamix_hp;

/* Lion: beta1 interpolates the sign argument, beta2 the momentum.        */
typedef struct optim_lion_hp {
    double beta1, beta2;
} optim_lion_hp;

typedef struct optim_plan optim_plan;

/* Message for the last failed call on this thread ("" if none).          */
const char *optim_last_error(void);

/* ---- plans --------------------------------------------------------------
 * A plan fixes a tensor list and algorithm: it validates them, splits every
 * tensor into work units and lays out the device-side tables (tensor
 * descriptors, unit spans, weight-decay groups, quantization tables) in the
 * workspace.  This size query is host-only and touches no device.        */
int optim_plan_workspace_size(const optim_tensor_list *list, int32_t algo,
                              const optim_plan_opts *opts, size_t *bytes);

/* Builds the plan, copies its tables into `workspace` (device, >= the size
 * above, 256-byte aligned) on `stream` and waits for that one copy (plan
 * creation is set-up, not part of a step).  The workspace must stay
 * allocated and untouched while the plan lives; steps of one plan must not
 * overlap each other (they share its workspace).  The host arrays of `list`
 * may be freed after return.  Queries the current device's compute-unit
 * count.                                                                  */
int optim_plan_create(const optim_tensor_list *list, int32_t algo,
                      const optim_plan_opts *opts, void *workspace,
                      size_t workspace_bytes, void *stream, optim_plan **out);

/* Frees the host plan object.  Work already enqueued is unaffected.      */
int optim_plan_destroy(optim_plan *plan);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * plan as optim_plan_create, built on a workspace the library holds in
 * static device memory -- OPTIM_STATIC_WORKSPACE_BYTES per device, held by
 * every device the library runs on until the process ends -- instead of a
 * caller buffer.  It calls no device allocator (the host plan object is
 * malloc'd as with optim_plan_create; free it with optim_plan_destroy).
 * A plan needing more workspace than that (Adam-mini lists of more than
 * ~8.5 billion elements, LAMB lists of more than ~4.2 billion, lists of more
 * than ~90,000 tensors, or ~71,000 tensors small enough to share packs) is
 * refused with OPTIM_EWORKSPACE before anything is touched.
 * One static workspace per device, shared by every call on that device: a
 * call overwrites the tables of the previous static plan of the current
 * device, which from then on fails (OPTIM_EINVAL) in every entry point.
 * Creating a static plan while a step of the previous one may still run on
 * the device (another stream, not yet synchronised) races with that step;
 * so do steps of one static plan that overlap each other.  The commit
 * counters (and the maxima slots of fp16 states) are cleared by the call.
 * Validation, stream semantics and errors as optim_plan_create; the device
 * is the current one.                                                      */
#define OPTIM_STATIC_WORKSPACE_BYTES ((size_t)16 << 20)
int optim_plan_create_static(const optim_tensor_list *list, int32_t algo,
                             const optim_plan_opts *opts, void *stream,
                             optim_plan **out);

/* ---- kernel trace (measurement) -----------------------------------------
 * The device duration of every kernel a plan's calls launch, for measuring
 * a step kernel by kernel (the multi-kernel steps -- Adam-mini's block sums,
 * finalize and update per segment, LAMB's passes, the gradient norm's
 * stages -- are otherwise timed only as a whole).
 * optim_plan_trace(plan, capacity > 0): from now on each of the next
 * `capacity` kernel launches of the plan's step, check and norm calls
 * carries a pair of HIP events that the kernel's own dispatch stamps at its
 * start and end (hipExtLaunchKernel); nothing else is added to the stream.
 * Launches beyond the capacity run untraced and are counted.  Creates
 * 2*capacity HIP events (host resources, no device memory); not meant for
 * graph capture.  capacity 0 ends the trace and frees the events (also done
 * by optim_plan_destroy); a new call restarts it.
 * optim_plan_trace_read: blocks the host until the traced launches have
 * finished (the one other blocking call, with optim_plan_create), writes
 * min(count, max) records in launch order to out[], the number of traced
 * launches to *count and of untraced ones to *dropped (may be NULL), and
 * empties the trace for the next launches.  kernel names are the kernels'
 * function names, valid until the trace is freed.                          */
typedef struct optim_kernel_time {
    const char *kernel;   /* e.g. "mini_update_kernel"                      */
    int64_t workgroups;   /* grid size of the launch                        */
    double ms;            /* from the kernel's start to its end             */
} optim_kernel_time;

int optim_plan_trace(optim_plan *plan, int32_t capacity);
int optim_plan_trace_read(optim_plan *plan, optim_kernel_time *out,
                          int32_t max, int32_t *count, int64_t *dropped);

/* Device learning-rate schedule ([AO]: the lr changes every step and must
 * stay a device scalar updated in place, with no per-step allocation).
 * OPTIM_SCHED_COSINE: at each step call the library reads k = *iter_dev,
 * writes *lr_dev = fl32(lr_min + (lr_max - lr_min)*(1 + cos(pi*min(k,K)/K))/2)
 * (evaluated in fp64) and stores k + 1 into *iter_dev -- also on a skipped
 * step, since k counts loop iterations.  OPTIM_SCHED_NONE: *lr_dev is read
 * as given.  iter_dev: device int32, caller-owned.                        */
int optim_plan_set_schedule(optim_plan *plan, int32_t kind, double lr_max,
                            double lr_min, int32_t K, int32_t *iter_dev);

/* ---- steps --------------------------------------------------------------
 * Common arguments:
 *  lr_dev        device float learning rate (read; written when a schedule
 *                is set)
 *  inv_scale_dev device float; gradients are multiplied by it exactly once
 *                ([LTN] analysis: the fused step does the unscale, so the
 *                caller must not unscale first).  NULL = 1.
 *  found_inf_dev device float; non-zero means skip: no parameter, state,
 *                remainder, code or absmax byte is written and *step_dev is
 *                not advanced.  NULL = never skip.
 *  step_dev      device int32 count of applied steps; the step uses
 *                t = *step_dev + 1 for bias correction and stores t.
 * Per element (t-th applied step, g = grad * inv_scale):
 *  m <- beta1 m + (1-beta1) g;  v <- beta2 v + (1-beta2) g^2
 *  p <- p (1 - lr wd) - (lr / (1-beta1^t)) m / (sqrt(v)/sqrt(1-beta2^t) + eps)
 * the decay taken from the previous p, in Loshchilov & Hutter Algorithm 2
 * order ([BNB] PR description; [MINI] AdamWMini for bias correction and
 * eps placement).  Bias corrections are evaluated in fp64 on the device and
 * rounded once to fp32; the element math is fp32, with the decay and the
 * update applied as p - fma(fl32(lr wd), p, update), so each step rounds once
 * at the parameter's scale (no fl32(1 - lr wd) factor whose rounding would
 * bias every step the same way).  With BF16 params the
 * fp32 master is rebuilt from (param, remainder), updated, and split back
 * ([TE] description).
 *
 * With 16-bit states (plan opts state_dtype OPTIM_F16 / OPTIM_BF16; [TE]
 * review: a scaled low-precision state, its fp32 value being stored * scale,
 * a new state being value * rscale copied into the 16-bit tensor): per
 * tensor m~ = fl32(h(m) * scale_m) (likewise v), the moments follow the
 * fp32 recipe m = fl32(fl32(b1 m~) + fl32(c1 g)), v = fl32(fl32(b2 v~) +
 * fl32(c2 fl32(g g))), p is updated from these fp32 moments, and the stored
 * moments become rne16(fl32(m * fl32(1/scale'))) with, for fp16, scale' =
 * fl32(max|m| / 65504) over the tensor (1 if zero) and, for bf16, 1.  bf16
 * states take one kernel; fp16 states two (p and the new maxima, then the
 * stored moments recomputed from the old stored ones), and the new scales
 * are written at the end of the step.  A skipped step changes no scale.    */
int optim_step_adamw(optim_plan *plan, const optim_adamw_hp *hp, float *lr_dev,
                     const float *inv_scale_dev, const float *found_inf_dev,
                     int32_t *step_dev, void *stream);

/* AdEMAMix ([BNB] PR description and PR body): adds the slow EMA
 *  m2 <- beta3 m2 + (1-beta3) g (no bias correction) and uses
 *  p <- p (1 - lr wd) - lr (m/(1-beta1^t) + alpha m2) / (sqrt(v)/sqrt(1-beta2^t) + eps).
 * alpha and beta3 are constants.                                          */
int optim_step_ademamix(optim_plan *plan, const optim_ademamix_hp *hp,
                        float *lr_dev, const float *inv_scale_dev,
                        const float *found_inf_dev, int32_t *step_dev,
                        void *stream);

/* Adam-mini ([MINI] AdamWMini.step): FULL_V tensors take the AdamW step;
 * HEAD tensors share one v per block of head_numel consecutive elements and
 * SCALAR tensors one v for the whole tensor:
 *  V_b <- beta2 V_b + (1-beta2) mean_{i in b}(g_i^2)
 *  p <- p (1 - lr wd) - lr (m/(1-beta1^t)) / (sqrt(V_b)/sqrt(1-beta2^t) + eps).
 * Block sums are reduced in a fixed order (deterministic).                */
int optim_step_adam_mini(optim_plan *plan, const optim_adamw_hp *hp,
                         float *lr_dev, const float *inv_scale_dev,
                         const float *found_inf_dev, int32_t *step_dev,
                         void *stream);

/* Blockwise-quantized 2-state AdamW ([BNB]: the 2-state branch of the
 * blockwise 8-bit kernel, same decay ordering; [AO]: 4-bit states).
 * bits/block must equal the plan's.  Per block: dequantize m, v
 * (x = fl32(+-M[idx] * absmax)), update them in fp32 without contraction
 *  m = fl32(fl32(b1 m) + fl32(c1 g)), v = fl32(fl32(b2 v) + fl32(c2 fl32(g g)))
 * with b1 = fl32(beta1), c1 = fl32(1-beta1) (likewise beta2), update p as
 * in optim_step_adamw, then requantize: absmax A = max|x| over the block,
 * a = fl32(|x| * fl32(1/A)), code = largest j with T[j] <= a (sign in the
 * top bit for m; 0 if A = 0).  M and T are the tables optim_quant_codebook
 * returns.                                                                */
int optim_step_8bit_blockwise(optim_plan *plan, const optim_adamw_hp *hp,
                              int32_t bits, int32_t block, float *lr_dev,
                              const float *inv_scale_dev,
                              const float *found_inf_dev, int32_t *step_dev,
                              void *stream);

/* Lion ([BNB] PR review: Lion applies decoupled decay to the parameter
 * before its sign update; update rule of Chen et al., arXiv:2302.06675).
 * Per element, in fp32 without contraction:
 *   c = fl32(fl32(b1 m) + fl32(c1 g)),  p <- p (1 - lr wd) - lr sign(c),
 *   m <- fl32(fl32(b2 m) + fl32(c2 g)),  sign(0) = 0,
 * b1 = fl32(beta1), c1 = fl32(1-beta1) (likewise beta2), g = G * inv_scale.
 * Plan algorithm OPTIM_ALGO_LION (param, grad, m).  The step counter
 * advances as for the other steps.                                          */
int optim_step_lion(optim_plan *plan, const optim_lion_hp *hp, float *lr_dev,
                    const float *inv_scale_dev, const float *found_inf_dev,
                    int32_t *step_dev, void *stream);

/* LAMB, trust ratio per tensor ([BNB] PR description: LAMB shares the Adam
 * kernels' decay ordering; update of You et al., arXiv:1904.00962, Alg. 2):
 *   m, v as optim_step_adamw;  r = (m/bc1) / (sqrt(v)/sqrt(bc2) + eps)
 *   u = r + wd p;  p <- p - lr (|p| / |u|) u   (norms over each tensor,
 *   from the previous p; the ratio is 1 when either norm is 0).
 * Plan algorithm OPTIM_ALGO_LAMB (param, grad, m, v).  Three kernels: moments
 * and per-unit sums of p^2 and u^2, per-tensor ratios (fixed-order fp64
 * sums), update.                                                             */
int optim_step_lamb(optim_plan *plan, const optim_adamw_hp *hp, float *lr_dev,
                    const float *inv_scale_dev, const float *found_inf_dev,
                    int32_t *step_dev, void *stream);

/* Blockwise-quantized AdEMAMix ([BNB]: the blockwise 8-bit kernel's
 * AdEMAMix branch, same decay ordering; the fresh step mixes in
 * alpha*(1-beta3)*g).  Plan algorithm OPTIM_ALGO_BLOCKWISE_ADEMAMIX, with
 * qm, qm2, qv and their absmax in the tensor list.  As
 * optim_step_8bit_blockwise with a third state: m2 uses the signed map and
 *  m2 = fl32(fl32(b3 m2) + fl32(c3 g)), b3 = fl32(beta3), c3 = fl32(1-beta3),
 * and the update is p <- p (1 - lr wd) - lr (m/bc1 + alpha m2) / h (m2 not
 * bias-corrected), as optim_step_ademamix.                                  */
int optim_step_8bit_blockwise_ademamix(optim_plan *plan,
                                       const optim_ademamix_hp *hp,
                                       int32_t bits, int32_t block,
                                       float *lr_dev, const float *inv_scale_dev,
                                       const float *found_inf_dev,
                                       int32_t *step_dev, void *stream);

/* ---- helpers ------------------------------------------------------------ */

/* Sets *found_inf_dev = 1.0f if any gradient element of the plan is NaN or
 * +-Inf ([LTN] analysis: the fused step consumes found_inf); otherwise
 * leaves it unchanged, so the caller zeroes it first.                     */
int optim_check_finite(optim_plan *plan, float *found_inf_dev, void *stream);

/* Gradient clipping folded into the fused step ([LTN] analysis: unscale_
 * before step exists so that gradients can be clipped, and a fused step
 * that unscales inside must not receive already-unscaled gradients).  One
 * read of every gradient of the plan: as optim_check_finite it ORs 1.0f
 * into *found_inf_dev on a NaN / +-Inf, and it sums G^2 (the stored, scaled
 * gradients; each square exact in fp64, summed in fp64 per lane, per
 * workgroup and across workgroups in a fixed order, so a finite gradient
 * list always has a finite norm).  Then, with s = *inv_scale_dev (NULL: 1):
 *   *norm_dev           = sqrt(sum G^2) * s, the global L2 norm of the
 *                         unscaled gradients (norm_dev may be NULL);
 *   *clip_inv_scale_dev = s * min(1, max_norm / (norm + 1e-6)),
 * to be passed as the inv_scale of the step that follows.  max_norm <= 0
 * or +inf means no clipping (clip = s); NaN is EINVAL.  The norm is not
 * finite only when an element is NaN / +-Inf: then clip = s, found_inf is
 * set and the step skips.  Uses the
 * plan's workspace (partial sums): do not overlap it with a step of the
 * same plan on another stream.                                             */
int optim_grad_norm(optim_plan *plan, const float *inv_scale_dev,
                    double max_norm, float *found_inf_dev, float *norm_dev,
                    float *clip_inv_scale_dev, void *stream);

/* Dynamic loss scale, once per loop iteration after the step ([LTN]: the
 * loop ends with the scaler's update; rule as GradScaler documents it).
 * If *found_inf_dev != 0: scale *= backoff_factor, tracker = 0.  Else
 * tracker += 1, and when it reaches growth_interval: scale *= growth_factor
 * (kept only if finite) and tracker = 0.  Products in double, rounded once
 * to the stored float.  If inv_scale_dev is not NULL it receives
 * fl32(1/scale) (exact for power-of-two scales), ready for the next step.
 * growth_factor > 1 (finite), 0 < backoff_factor < 1, growth_interval >= 1,
 * else EINVAL.                                                              */
int optim_scaler_update(float *scale_dev, float *inv_scale_dev,
                        int32_t *growth_tracker_dev,
                        const float *found_inf_dev, double growth_factor,
                        double backoff_factor, int32_t growth_interval,
                        void *stream);

/* Blockwise quantize / dequantize of a plain fp32 device array with the
 * codebook, bits and block of a blockwise `plan`, by the same device code as
 * optim_step_8bit_blockwise: for importing fp32 optimizer state into codes
 * and exporting it back (checkpoints).  is_signed: the signed map (used for
 * m) or the unsigned map (for v).  codes: (n*bits+7)/8 bytes (4-bit: element
 * 2i in the low nibble); absmax: ceil(n/block) floats; blocks start at
 * element 0.  Quantize: A = max|x| per block, a = fl32(|x| * fl32(1/A)),
 * code = largest j with T[j] <= a (sign above the magnitude bits for the
 * signed map, 0 if A = 0).  Dequantize: x = fl32(+-M[idx] * A).          */
int optim_quantize_blockwise(optim_plan *plan, int32_t is_signed,
                             const float *x_dev, int64_t n, uint8_t *codes_dev,
                             float *absmax_dev, void *stream);
int optim_dequantize_blockwise(optim_plan *plan, int32_t is_signed,
                               const uint8_t *codes_dev,
                               const float *absmax_dev, int64_t n,
                               float *x_dev, void *stream);

/* [TE] description: fp32 master <-> (bf16 param, int16 remainder).  For the
 * 32-bit pattern u of x: r = low 16 bits of u as int16, b = (high 16 bits of
 * u) + (r < 0) mod 2^16, i.e. x rounded to bf16, nearest, ties away from
 * zero.  reconstruct(split(x)) == x for every pattern.  n >= 0 elements;
 * device arrays.                                                          */
int optim_remainder_split(const float *master_dev, uint16_t *bf16_dev,
                          int16_t *rem_dev, int64_t n, void *stream);
int optim_remainder_reconstruct(const uint16_t *bf16_dev,
                                const int16_t *rem_dev, float *master_dev,
                                int64_t n, void *stream);

/* Host: the dynamic quantization map the blockwise step uses.  bits 8 or
 * 4; is_signed selects the map for m (sign bit + bits-1 magnitude bits) or
 * for v (bits magnitude bits).  Writes the 2^mb sorted magnitudes
 *  {0} U {10^-e (0.1 + 0.9 (k+1)/2^(mb-1-e)) : e < mb, k < 2^(mb-1-e)}
 * (each evaluated in fp64, rounded to fp32) to values[2^mb] and the decision
 * thresholds T[j] = fl32((M[j-1]+M[j])/2), T[0] = 0, to thresholds[2^mb].
 * The map follows the dynamic (exponent + linear fraction) quantization of
 * Dettmers et al., arXiv:2110.02861; the pages give no values.           */
int optim_quant_codebook(int32_t bits, int32_t is_signed, float *values,
                         float *thresholds);

#ifdef __cplusplus
}
#endif
#endif /* OPTIM_STEP_H */
