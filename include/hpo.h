/*
 * hpo.h -- C ABI of libhpo: the mixed-precision AdamW optimizer step on one
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages):
 *   [OPT-INFRA]  "02 · Optimizer：算法与 infra" (llm-infra-atlas, train/02_optimizer)
 *   [HANDBOOK]   "优化器：AdamW、Muon 与分布式优化器" (ai-infra-handbooks, train/algo/optimizer)
 *   [FP32-RFC]   "支持FP32优化器" / "AutoModels Trainer 支持 FP32 main_param 优化器"
 *                (hyper-parallel issue)
 *
 * One optimizer step, in the order the pages give it ([OPT-INFRA] §10.2,
 * §11.1, §9.2; [FP32-RFC] §8.2):
 *   1. unscale the fp32 main grads by the loss scale and look for inf/NaN;
 *      if any is found the whole step is skipped (no clip, no update, the
 *      applied-step count does not move);
 *   2. take the global L2 norm of the unscaled grads and clip them to
 *      max_norm;
 *   3. run Adam / AdamW on the fp32 master, exp_avg and exp_avg_sq;
 *   4. write the master back to the 16-bit model params (bf16, round to
 *      nearest even).
 *
 * Conventions shared by every call:
 *   - Every pointer argument marked "device" is a device address on the
 *     device that was current when the set was created; that device must be
 *     current for every later call on the set (HPO_EDEVICE otherwise).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call that launches work is asynchronous on that stream and
 *     returns as soon as the work is enqueued; host-side argument errors are
 *     detected before anything is enqueued, and then nothing is.
 *   - The caller owns (allocates, frees) every tensor and every device
 *     result buffer.  The library never frees or resizes them.  A set holds
 *     only its own small device tables (one 64-byte descriptor per tensor,
 *     16 bytes per chunk, 20 bytes per grad-pass workgroup of reduction
 *     partials); it never allocates per-element memory.
 *   - The tensors of a set must stay allocated while the set exists and must
 *     not overlap one another.  All element counts are int64.
 *   - Return value: HPO_OK or a negative hpo_status; hpo_last_error() then
 *     returns a message (thread-local).  No call throws or aborts.
 *   - Two calls on the same set that run concurrently on different streams
 *     race on the set's reduction partials; order them on one stream.
 */
#ifndef HPO_H
#define HPO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 5: the device step state (64 bytes) reports the grads' zero count and the
 *    scale the step unscaled with; the norm calls report the zero count. */
#define HPO_ABI_VERSION 5
/* Most parameter groups one step can take (per-group lr / weight decay). */
#define HPO_MAX_GROUPS 16

typedef enum {
    HPO_OK = 0,
    HPO_EINVAL = -1,  /* bad argument (null pointer, negative size, range, ...) */
    HPO_EDTYPE = -2,  /* unsupported param dtype ([FP32-RFC] §7.2: anything but the
                         supported float types is an error, never a silent cast) */
    HPO_ENOMEM = -3,  /* the set's small device tables could not be allocated */
    HPO_EHIP = -4,    /* a HIP runtime call or launch failed; message has the HIP error */
    HPO_EDEVICE = -5  /* the current device is not the set's device */
} hpo_status;

/* dtype of the model params a set writes back to ([OPT-INFRA] §9.2: the
 * wrapper keeps an fp32 master for fp16 and bf16 params).
 * HPO_PARAM_BF16: bf16 params, each with its own fp32 master.
 * HPO_PARAM_FP32: fp32 params are their own master ([FP32-RFC] §7.2, native
 *                 fp32 params): param must be NULL or equal to main_param, and
 *                 no write-back happens.
 * HPO_PARAM_FP16: fp16 params (IEEE round-to-nearest-even write-back, fp16
 *                 subnormals kept, overflow to infinity); fp16 training is
 *                 what the dynamic loss scaler below is for.
 * Optionally OR-ed with HPO_STATE_BF16: exp_avg and exp_avg_sq are then bf16
 * arrays (the exp_avg / exp_avg_sq pointers point at 2-byte elements), read
 * exactly and written back rounded to nearest even ([OPT-INFRA] §16, the
 * precision-aware optimizer's lower-precision moments); the update itself
 * still runs in fp32.  Any other value is rejected with HPO_EDTYPE, never
 * silently cast ([FP32-RFC] §7.2). */
typedef enum { HPO_PARAM_BF16 = 0, HPO_PARAM_FP32 = 1, HPO_PARAM_FP16 = 2 } hpo_param_dtype;
#define HPO_STATE_BF16 0x100
/* fp16 moments are refused (HPO_EDTYPE).  [OPT-INFRA] §16 lets
 * exp_avg_dtype / exp_avg_sq_dtype go below fp32 without fixing a format or a
 * scale.  Without a per-tensor scale, fp16 cannot hold the second moment at
 * ordinary grad magnitudes: (1 - beta2) g^2 falls below half fp16's smallest
 * subnormal (2^-25) once |g| is under about 1.7e-4 and is stored as 0, and the
 * first moment runs subnormal (few bits) below |g| of about 6e-4, so the
 * update stops being Adam's.  bf16 has fp32's range and keeps both. */
#define HPO_STATE_FP16 0x800

/* The main grads and the master may be stored below fp32 as well ([OPT-INFRA]
 * §16 lists main_grads and main_params among the precision-aware optimizer's
 * lower-precision fields).  OR-ed into param_dtype like HPO_STATE_BF16:
 * HPO_GRAD_BF16: main_grad points at bf16 elements (2 bytes), read exactly;
 *     the norm, the check and the update see their fp32 values.
 *     hpo_unscale_check_inf stores bf16(fp32(G * inv_scale)), rounded to
 *     nearest even.
 * HPO_MASTER_FP16: main_param points at fp16 elements.  Only with
 *     HPO_PARAM_BF16 (under fp16 params an fp16 master would be the params
 *     themselves; fp32 params are their own master).  The update widens the
 *     master exactly, runs in fp32 as for an fp32 master, stores the master
 *     rounded to nearest even (fp16 subnormals kept, overflow to infinity), and
 *     writes the bf16 param as the bf16 rounding of the stored fp16 master, as
 *     hpo_copy_main_to_model does.  An update below half an fp16 ulp of the
 *     master is lost: that is the format's.
 * Both are AdamW-set options: Muon sets reject them (HPO_EDTYPE). */
#define HPO_GRAD_BF16 0x200
#define HPO_MASTER_FP16 0x400

/* Weight-decay form ([OPT-INFRA] §3): decoupled (AdamW, the default there) or
 * an L2 term added to the gradient before the moments (Adam + L2). */
typedef enum { HPO_ADAMW = 0, HPO_ADAM_L2 = 1 } hpo_mode;

/* Adam hyperparameters ([OPT-INFRA] §2: defaults beta1 0.9, beta2 0.999,
 * eps 1e-8; §17 config fields).  0 <= beta < 1, eps >= 0. */
typedef struct {
    double beta1;
    double beta2;
    double eps;
    int32_t mode; /* hpo_mode */
} hpo_adam_cfg;

/* One parameter group: learning rate and weight decay.  The usual no-decay
 * group (norm gains, biases: [HANDBOOK] AdamW section) is a group with
 * weight_decay = 0. */
typedef struct {
    double lr;
    double weight_decay;
} hpo_group;

/* Opaque handle on a set of parameters stepped together. */
typedef struct hpo_set_* hpo_set;

/* A set whose arrays take at most 192 MiB in all stays in the GPU's on-die
 * cache between steps; its update then reads and writes through the caches
 * (the same results), while larger sets use streaming accesses that go
 * around them. */
typedef struct {
    int32_t n_tensors;
    int32_t param_dtype;
    int32_t is_flat;
    int32_t chunk_elems;   /* elements per work chunk (one workgroup each) */
    int64_t numel;         /* total elements over all tensors */
    int64_t n_chunks;
    int64_t device_bytes;  /* bytes of device memory the set itself holds */
    int32_t device;        /* HIP device ordinal of the set */
    int32_t n_vector;      /* tensors (ranges) whose body takes the 16-byte vector path */
    int32_t grad_group;    /* consecutive chunks per grad-pass workgroup */
    int32_t kind;          /* HPO_SET_ADAM or HPO_SET_MUON */
    int64_t n_grad_parts;  /* grad-pass workgroups = binary64 partials per norm */
} hpo_set_info_t;

/* What a set is stepped with: AdamW (the list and flat sets) or Muon (the
 * matrix sets of hpo_muon_set_create). */
typedef enum { HPO_SET_ADAM = 0, HPO_SET_MUON = 1 } hpo_set_kind;

/* ---------------------------------------------------------------------- */
/* Sets                                                                    */
/* ---------------------------------------------------------------------- */

/* A set over a list of n_tensors parameters ([OPT-INFRA] §9.2: the wrapper
 * keeps the model params, their fp32 masters and the fp32 main grads side by
 * side).  Tensor i is the contiguous 1-D range of numel[i] elements at each
 * of the five device pointers:
 *   param[i]      bf16 model param (HPO_PARAM_BF16), or NULL / main_param[i]
 *                 for HPO_PARAM_FP32;
 *   main_param[i] fp32 master, main_grad[i] fp32 main grad (stored, i.e. still
 *                 multiplied by the loss scale), exp_avg[i], exp_avg_sq[i] fp32.
 * group_index[i] in [0, HPO_MAX_GROUPS) selects the tensor's hpo_group in
 * hpo_adamw_step (NULL: every tensor is in group 0).  numel[i] may be 0;
 * n_tensors may be 0 (then every call is a no-op and the norm is 0).
 * Pointers need 4-byte (fp32) and 2-byte (16-bit) alignment.  Tensors whose
 * pointers are 16-byte aligned (8-byte for 16-bit arrays) take vector
 * accesses of 4 elements; a tensor whose five pointers sit at the same
 * element offset inside their aligned 4-element lines (a view a few elements
 * into a flat buffer) has its first 1..3 elements stepped one at a time and the rest vectorized; any
 * other tensor is stepped one element at a time.  Results are the same bits
 * on every path.
 * The host arrays are read during the call only.  The device tables are
 * uploaded on `stream`, and the call waits for that upload to finish. */
hpo_status hpo_set_create_list(hpo_set* out, int32_t n_tensors, int32_t param_dtype,
                               void* const* param, float* const* main_param,
                               float* const* main_grad, float* const* exp_avg,
                               float* const* exp_avg_sq, const int64_t* numel,
                               const int32_t* group_index, void* stream);

/* A set over one flat, contiguous range of numel elements: the ZeRO-1 shard
 * layout of [OPT-INFRA] §12.1 (each data-parallel rank owns one contiguous
 * slice of the flat grad/param buffers, param boundaries ignored).  One group
 * (group 0).  Same pointer rules as one tensor of a list set. */
hpo_status hpo_set_create_flat(hpo_set* out, int64_t numel, int32_t param_dtype, void* param,
                               float* main_param, float* main_grad, float* exp_avg,
                               float* exp_avg_sq, void* stream);

/* A flat ZeRO-1 shard whose elements belong to several parameter groups.
 * The shard is cut without regard to param boundaries ([OPT-INFRA] §12.1), so
 * one rank's slice mixes decaying weights with norm gains and biases that
 * take no weight decay ([HANDBOOK] AdamW section).  Range k covers elements
 * [range_start[k], range_start[k+1]) (the last one ends at numel) and uses
 * group range_group[k] in hpo_adamw_step.  range_start[0] must be 0 and the
 * starts strictly increasing (no empty ranges).  Pointers follow the flat
 * set's rules; a range that does not start on a 4-element line has its first
 * 1..3 elements stepped one at a time and the rest vectorized. */
hpo_status hpo_set_create_flat_ranges(hpo_set* out, int64_t numel, int32_t param_dtype, void* param,
                                      float* main_param, float* main_grad, float* exp_avg,
                                      float* exp_avg_sq, int32_t n_ranges, const int64_t* range_start,
                                      const int32_t* range_group, void* stream);

/* Frees the set's device tables after waiting for the device to go idle.
 * NULL is accepted. */
hpo_status hpo_set_destroy(hpo_set s);

hpo_status hpo_set_info(hpo_set s, hpo_set_info_t* out);

/* ---------------------------------------------------------------------- */
/* The step                                                               */
/* ---------------------------------------------------------------------- */

/* Unscale and check, the pages' in-place form ([OPT-INFRA] §9.2 table, unscale
 * row; §10.2): every main grad element G becomes fp32(G * inv_scale) in place,
 * and *d_found_inf (device int32) is set to 1 when any stored element was inf
 * or NaN; it is never cleared, so zero it before the first call of a step.
 * With inv_scale == 1 the grads are only read (multiplying by 1 changes no
 * finite value).  After this call pass inv_scale = 1 to the two calls below. */
hpo_status hpo_unscale_check_inf(hpo_set s, float inv_scale, int32_t* d_found_inf, void* stream);

/* Global grad norm ([OPT-INFRA] §11.1): *d_norm (device fp32) receives
 * fp32(sqrt(sum over all elements of g^2)) with g = fp32(G * inv_scale), the
 * squares and the sum in binary64 (per-workgroup partials, then one fixed-order
 * sum, so the result is deterministic).  The grads are not written.
 * d_found_inf (device int32, nullable) is set to 1 when any stored element is
 * inf or NaN (same rule as above) -- the same read serves both.  When a
 * non-finite value is present the norm is inf or NaN.
 * d_num_zeros (device int64, nullable) receives the number of elements whose
 * g is zero, +0 or -0: the step's num_zeros ([OPT-INFRA] §10.2, an applied
 * step returns (success, grad_norm, num_zeros); §17 log_num_zeros_in_grad),
 * counted on the unscaled grads whose norm is taken, before the clip.  A
 * stored value that the unscale rounds to zero counts; NaN and inf do not. */
hpo_status hpo_grad_global_norm(hpo_set s, float inv_scale, float* d_norm, int32_t* d_found_inf,
                                int64_t* d_num_zeros, void* stream);

/* Clip + Adam/AdamW update + bf16 write-back, one fused pass
 * ([OPT-INFRA] §11.1, §2, §3, §9.2).  For every element, with fp32 arithmetic
 * in the order written and no fused multiply-add:
 *   g  = G * inv_scale;  if clipping: g = g * C
 *   Adam + L2 only:  g = g + wd * theta
 *   m  = b1 * m + (1 - b1) * g;      v = b2 * v + (1 - b2) * (g * g)
 *   u  = (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 *   AdamW: theta = theta - lr * (u + wd * theta);  Adam + L2: theta = theta - lr * u
 *   bf16 sets: param = bf16_rne(theta)
 * b1, b2, 1-b1, 1-b2, 1-b^t, eps, lr and wd are formed in binary64 on the host
 * and rounded to fp32 once.  Clipping: when max_norm > 0, c = max_norm /
 * ((double)*d_norm + 1e-6) is formed in binary64 on the device; it applies
 * when c < 1, as C = fp32(c).  max_norm <= 0 turns clipping off (d_norm may
 * then be NULL).
 * t is the 1-based count of applied steps including this one; a skipped step
 * must not advance it ([OPT-INFRA] §10.2).  groups[k] holds group k's lr and
 * weight decay; n_groups must cover every group index of the set.
 * d_found_inf (device int32, nullable): when it is non-zero at run time the
 * whole launch does nothing (device-side skip), so the step can be enqueued
 * before the flag is read back. */
hpo_status hpo_adamw_step(hpo_set s, const hpo_adam_cfg* cfg, const hpo_group* groups,
                          int32_t n_groups, int64_t t, float inv_scale, double max_norm,
                          const float* d_norm, const int32_t* d_found_inf, void* stream);

/* ---------------------------------------------------------------------- */
/* Device-resident step: loss scaler, skip decision and step counter on the */
/* device, so steps can be enqueued without a host synchronisation.         */
/* ---------------------------------------------------------------------- */

/* Most values of t one device-resident call holds bias corrections for (see
 * hpo_step_device): the steps that can be enqueued, or replayed from one
 * captured call (a HIP graph), between two reads of the state.  The fp32
 * tables travel in the kernel arguments (2 KB at 256). */
#define HPO_MAX_WINDOW 256

/* Loss-scaler and step state kept in device memory (64 bytes, caller-owned,
 * 8-byte aligned).  The caller multiplies its loss by loss_scale before
 * backward ([OPT-INFRA] §10.2: the loss is scaled, the grads are unscaled
 * before the step) and may read the struct back at any time after a sync.
 * After a step, loss_scale / inv_scale hold the scale for the next step
 * and step_inv_scale the one this step's grads were unscaled with. */
typedef struct {
    float loss_scale;           /* S */
    float inv_scale;            /* fp32(1 / S), formed in binary64; what the next step multiplies by */
    int32_t growth_tracker;     /* clean steps since the last growth or non-finite step */
    int32_t hysteresis_tracker; /* non-finite steps still tolerated before a back-off */
    int64_t applied_steps;      /* steps applied so far = t of the last applied step */
    int64_t skipped_steps;      /* steps skipped (non-finite grads or norm over the threshold) */
    float grad_norm;            /* norm of the last step's unscaled grads (inf/NaN if non-finite) */
    int32_t found_inf;          /* the last step saw an inf/NaN grad */
    int32_t applied;            /* the last step was applied */
    int32_t error;              /* sticky: a step's t fell outside the window it was given */
    int64_t num_zeros;          /* zeros among the last step's unscaled grads (as hpo_grad_global_norm) */
    float step_inv_scale;       /* the inv_scale the last step's grads were unscaled with */
    int32_t reserved;           /* 0 */
} hpo_scaler_state;

/* Scaler and skip policy ([OPT-INFRA] §10.1 scaler rules and defaults; §11.4
 * and §17 grad_norm_skip_threshold, default off).
 *   dynamic = 0: constant scale, never changed (an explicit loss scale).
 *   dynamic = 1: on a step with non-finite grads the growth tracker resets and
 *     the hysteresis tracker drops by one; once it is <= 0 the scale becomes
 *     max(scale * backoff_factor, min_scale) (so a single spike is tolerated
 *     when hysteresis > 1).  After growth_interval clean steps in a row the
 *     scale is multiplied by growth_factor and both trackers reset.  The
 *     pages' defaults: initial scale 2^32, growth 2.0, backoff 0.5, interval
 *     1000, hysteresis 2, min scale 1.0.
 *   A step whose grad norm exceeds grad_norm_skip_threshold is skipped too (no
 *   update, t unchanged); it still counts as clean for the scaler, which the
 *   pages update before the norm is taken. */
typedef struct {
    int32_t dynamic;
    int32_t growth_interval;
    int32_t hysteresis;
    float growth_factor;
    float backoff_factor;
    float min_scale;
    double grad_norm_skip_threshold; /* +inf: never */
} hpo_scaler_cfg;

/* Writes a fresh state: loss_scale, inv_scale = fp32(1/loss_scale),
 * hysteresis_tracker = hysteresis, applied_steps as given (a resumed run),
 * every other field 0.  Enqueued on stream (a one-lane kernel). */
hpo_status hpo_scaler_state_init(hpo_scaler_state* d_state, float loss_scale, int32_t hysteresis,
                                 int64_t applied_steps, void* stream);

/* One whole step with everything decided on the device: the grad pass (check
 * + norm + zero count, multiplying by d_state->inv_scale), the finalize
 * (norm, found_inf, the skip decision, then the counters and the scaler
 * rule), and the fused clip + update + write-back, run only when the step is
 * applied, with t = the new applied_steps and the step's inv_scale.
 * Nothing is read back.
 * The bias corrections 1 - beta^t are formed on the host in binary64 and
 * rounded to fp32 for t = t_first .. t_first + window - 1, where t_first is
 * applied_steps + 1 as of the caller's last read of the state and window
 * (1..HPO_MAX_WINDOW) counts the steps enqueued since that read, this one
 * included; if the device's t falls outside, the step is not applied and
 * d_state->error is set.  Same arithmetic, bit for bit, as the three calls
 * above with the same scale.  The call enqueues kernels only (no allocation,
 * no copy, no synchronisation), so it can be captured in a HIP graph; a
 * replay of the graph is one more step of this window. */
hpo_status hpo_step_device(hpo_set s, const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                           double max_norm, const hpo_scaler_cfg* scfg, hpo_scaler_state* d_state,
                           int64_t t_first, int32_t window, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * device-resident step of one flat shard with no set, so no call, first or
 * later, allocates, copies or frees anything.  It computes exactly what
 * hpo_set_create_flat over the same arrays followed by hpo_step_device with
 * the one group *group (n_groups = 1) computes, bit for bit, with the same
 * argument rules (pointers as for one tensor of a list set; the state,
 * t_first and window as for hpo_step_device).  A shard whose pointers are
 * not on their 4-element vector lines steps element by element (same bits,
 * slower): there is no table to peel its head into.
 * The grad pass's reduction partials live in a static device array of
 * HPO_STATIC_MAX_PARTS entries (20 bytes each, about 5 MiB) that each GPU the
 * library runs on holds until the process ends; a shard whose plan needs
 * more partials (more than about HPO_STATIC_MAX_PARTS * 65536, i.e. 1.7e10
 * elements) is refused with HPO_EINVAL before anything is enqueued.  All
 * calls on one GPU share that array: calls that overlap on one GPU (two
 * streams or two threads at once) race on it and must be ordered by the
 * caller. */
#define HPO_STATIC_MAX_PARTS (1 << 18)
hpo_status hpo_step_device_flat_static(int64_t numel, int32_t param_dtype, void* param, float* main_param,
                                       float* main_grad, void* exp_avg, void* exp_avg_sq, const hpo_adam_cfg* cfg,
                                       const hpo_group* group, double max_norm, const hpo_scaler_cfg* scfg,
                                       hpo_scaler_state* d_state, int64_t t_first, int32_t window, void* stream);

/* Master -> model copy alone: param = bf16_rne(main_param) for every element
 * of a bf16 set ([OPT-INFRA] §9.2, the write-back row; the same conversion the
 * step fuses).  A no-op for fp32 sets. */
hpo_status hpo_copy_main_to_model(hpo_set s, void* stream);

/* ---------------------------------------------------------------------- */
/* Muon, chained with AdamW                                                */
/* ---------------------------------------------------------------------- */
/* Muon ([HANDBOOK] "优化器：AdamW、Muon 与分布式优化器", Muon section;
 * [OPT-INFRA] §5) steps the hidden 2-D weight matrices; embeddings, the
 * output head and every 1-D parameter stay on AdamW ([OPT-INFRA] §5.5,
 * §14.2).  Per matrix W (rows x cols) with fp32 master, fp32 main grad G and
 * fp32 momentum M, each applied step computes, with g = G * inv_scale
 * (times the clip coefficient C when clipping, the same global norm and rule
 * as the AdamW step):
 *   momentum   HPO_MUON_MOMENTUM_SUM ([HANDBOOK]):  M = mu M + g,          g~ = g + mu M
 *              HPO_MUON_MOMENTUM_EMA ([OPT-INFRA] §1): M = mu M + (1-mu) g, g~ = (1-mu) g + mu M
 *              (without Nesterov g~ = M); fp32, one rounding per operation;
 *   NS         X = g~ / (||g~||_F + eps) (the sum of squares in binary64, the
 *              norm and the guard in fp32), transposed when rows > cols; then
 *              ns_steps times: A = X X^T, B = b A + c A A, X = a X + B X, with
 *              (a, b, c) of each step; O = X, transposed back.  The matmuls
 *              run on the bf16 matrix cores ([OPT-INFRA] §5.2, §5.4): X, A
 *              and B are rounded to bf16 (nearest even) as operands, products
 *              accumulate in fp32, the last X stays fp32;
 *   update     W = fp32(W * fp32(1 - lr*wd)); W = fp32(W - fp32(lr*scale) * O)
 *              (decay first, as the handbook listing does), scale =
 *              base * extra_scale with base sqrt(max(rows, cols)) (spectral;
 *              extra 0.2 is Moonlight's RMS match, [OPT-INFRA] §5.4),
 *              sqrt(max(1, rows/cols)) (shape) or sqrt(rows/cols) (unit RMS)
 *              ([OPT-INFRA] §14.6); then param = bf16_rne(W).
 * The momentum and the param / master of skipped steps are bit-unchanged. */
typedef enum { HPO_MUON_MOMENTUM_SUM = 0, HPO_MUON_MOMENTUM_EMA = 1 } hpo_muon_momentum;
typedef enum { HPO_MUON_SCALE_SPECTRAL = 0, HPO_MUON_SCALE_SHAPE = 1, HPO_MUON_SCALE_UNIT_RMS = 2 } hpo_muon_scale;
#define HPO_NS_MAX_STEPS 16

/* Muon hyperparameters.  Defaults (the handbook's Muon): momentum 0.95,
 * nesterov 1, HPO_MUON_MOMENTUM_SUM, 5 NS steps with (a, b, c) =
 * (3.4445, -4.7750, 2.0315), eps 1e-7, spectral scale with extra 0.2. */
typedef struct {
    double momentum;          /* mu, in [0, 1) */
    int32_t nesterov;         /* 0 or 1 */
    int32_t momentum_form;    /* hpo_muon_momentum */
    int32_t ns_steps;         /* 1 .. HPO_NS_MAX_STEPS */
    int32_t scale_mode;       /* hpo_muon_scale */
    double extra_scale;       /* finite, >= 0 */
    double ns_eps;            /* finite, >= 0 */
    const double* ns_coeffs;  /* host array of 3 * ns_steps (a, b, c per step, rounded to fp32),
                                 or NULL for the original set at every step */
} hpo_muon_cfg;

/* Default workspace cap of a Muon set (see hpo_muon_set_create). */
#define HPO_MUON_DEFAULT_WORKSPACE (((int64_t)16) << 30)

/* Largest rows or cols of a Muon matrix (and of hpo_newton_schulz): the
 * matrix-core kernels address one 256-row operand panel with 32-bit byte
 * offsets. */
#define HPO_MUON_MAX_DIM (((int64_t)1) << 21)

/* A Muon set over n_matrices row-major matrices: matrix i has rows[i] x
 * cols[i] elements at param[i] (bf16 model param, or NULL / main_param[i]
 * for HPO_PARAM_FP32), main_param[i] (fp32 master), main_grad[i] (fp32 main
 * grad, as stored) and momentum[i] (fp32).  Every pointer must be 16-byte
 * aligned.  param_dtype: HPO_PARAM_BF16 or HPO_PARAM_FP32; fp16 params with
 * Muon are an error ([OPT-INFRA] §14.3), as is HPO_STATE_BF16 (HPO_EDTYPE).
 * group_index[i] selects the matrix's hpo_group in hpo_muon_step (NULL:
 * group 0).  Matrices with rows or cols 0 are allowed and never touched;
 * rows or cols above HPO_MUON_MAX_DIM are an error (HPO_EINVAL).
 * The set plans batches of same-shape matrices and allocates one device
 * workspace for the largest batch: per matrix 4 B per element (the Nesterov
 * gradient) plus bf16 X, two X^T and the two Gram-sized matrices of NS, with
 * both dimensions padded to multiples of 256.  workspace_bytes caps the
 * batch size (0: HPO_MUON_DEFAULT_WORKSPACE); a shape class is split into
 * equal batches under the cap (and of at most 65535 matrices, the launch
 * grid's z limit), and a matrix that alone needs more gets a batch of its
 * own.  Larger batches keep more of the GPU busy in the NS launches (16 GiB
 * holds 24 of Llama-8B's 4096 x 14336 matrices).  hpo_set_info reports the
 * total in device_bytes.
 * hpo_unscale_check_inf, hpo_grad_global_norm, hpo_grad_global_norm_sets and
 * hpo_copy_main_to_model accept Muon sets; hpo_adamw_step and
 * hpo_step_device do not (HPO_EINVAL). */
hpo_status hpo_muon_set_create(hpo_set* out, int32_t n_matrices, int32_t param_dtype, void* const* param,
                               float* const* main_param, float* const* main_grad, float* const* momentum,
                               const int64_t* rows, const int64_t* cols, const int32_t* group_index,
                               int64_t workspace_bytes, void* stream);

/* One Muon update of every matrix of the set, host-driven like
 * hpo_adamw_step: inv_scale, the clip from max_norm and *d_norm (device fp32,
 * read when max_norm > 0), and the device-side skip on *d_found_inf (nullable).
 * groups[k] = lr / weight decay of group k. */
hpo_status hpo_muon_step(hpo_set s, const hpo_muon_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                         float inv_scale, double max_norm, const float* d_norm, const int32_t* d_found_inf,
                         void* stream);

/* The global norm over several sets at once ([OPT-INFRA] §11.4: a chain of
 * optimizers takes one norm over all of its grads): *d_norm receives
 * fp32(sqrt(sum over every element of every set of (G * inv_scale)^2)), the
 * sum in binary64, the sets' partial sums added in array order; d_found_inf
 * and d_num_zeros as in hpo_grad_global_norm, over all the sets.
 * 1 <= n_sets <= 4, all on one device. */
hpo_status hpo_grad_global_norm_sets(const hpo_set* sets, int32_t n_sets, float inv_scale, float* d_norm,
                                     int32_t* d_found_inf, int64_t* d_num_zeros, void* stream);

/* hpo_step_device for an AdamW set and a Muon set stepped as one chain
 * ([OPT-INFRA] §11.4): one grad pass over both, one norm (AdamW grads
 * first), one found_inf and one skip decision; then the AdamW update, the
 * Muon update and the counters / scaler.  Either set may be NULL (not both). */
hpo_status hpo_step_device_chain(hpo_set adam_set, const hpo_adam_cfg* cfg, const hpo_group* groups,
                                 int32_t n_groups, hpo_set muon_set, const hpo_muon_cfg* mcfg,
                                 const hpo_group* muon_groups, int32_t n_muon_groups, double max_norm,
                                 const hpo_scaler_cfg* scfg, hpo_scaler_state* d_state, int64_t t_first,
                                 int32_t window, void* stream);

/* Newton-Schulz alone ([HANDBOOK] Muon listing, the NS function): O (fp32,
 * rows x cols, row-major, device) from G (fp32, same shape, device), with
 * cfg's ns_steps, ns_coeffs and ns_eps (the momentum and scale fields are not
 * read) and the same bf16 matrix-core arithmetic as hpo_muon_step.  The
 * caller provides a device workspace of at least
 * hpo_newton_schulz_workspace(rows, cols) bytes, 256-byte aligned.  rows and
 * cols lie in [0, HPO_MUON_MAX_DIM] (else HPO_EINVAL from both calls). */
hpo_status hpo_newton_schulz(const float* d_G, int64_t rows, int64_t cols, const hpo_muon_cfg* cfg, float* d_out,
                             void* d_workspace, int64_t workspace_bytes, void* stream);
hpo_status hpo_newton_schulz_workspace(int64_t rows, int64_t cols, int64_t* out_bytes);

/* Measurement only, not part of a step: the fused update's memory traffic
 * with none of its arithmetic, on a flat set of fp32 grads, master and
 * moments with 16-bit params whose pointers are on their 4-element vector
 * lines (else HPO_EINVAL).  Each chunk's grad, master, exp_avg and
 * exp_avg_sq are read (16 bytes per element) and master, exp_avg, exp_avg_sq
 * written back unchanged and the param written as the 16-bit rounding of
 * the master (14 bytes), with the update's launch shape and streaming
 * accesses; chunk tails that are not whole vectors are skipped.  The
 * state is left as it was wherever param already equals the rounding of the
 * master, which every step keeps.  Timing it gives the practical HBM
 * ceiling of the update's read/write mix, which the roofline of the update
 * is reported against besides the published peak. */
hpo_status hpo_stream_probe(hpo_set s, void* stream);

/* Opt-in timing of a Muon set's launches (for measurement, not for the
 * hot loop): while enabled, every Muon update of the set (hpo_muon_step,
 * hpo_step_device_chain) records HIP events on its stream around each launch
 * and notes the launch's algorithmic work.  hpo_muon_profile_read waits for
 * the recorded events, returns the totals since the last read (or since
 * enabling) and clears them.  Categories: */
typedef enum {
    HPO_MUON_PROF_MOMENTUM = 0,  /* momentum + Nesterov gradient pass and the per-matrix norms */
    HPO_MUON_PROF_INPUT = 1,     /* X0 = bf16(g~ / (norm + eps)) and its transpose */
    HPO_MUON_PROF_GRAM = 2,      /* A = X X^T (symmetric: upper-triangle tiles, mirrored) */
    HPO_MUON_PROF_POLY = 3,      /* B = b A + c A A^T (symmetric) */
    HPO_MUON_PROF_STEP = 4,      /* X' = a X + B X, steps before the last */
    HPO_MUON_PROF_UPDATE = 5,    /* the last step's X' = a X + B X fused with the master update */
    HPO_MUON_PROF_N = 6
} hpo_muon_prof_kind;

typedef struct {
    double ms[HPO_MUON_PROF_N];        /* summed launch time (event to event) */
    int64_t launches[HPO_MUON_PROF_N];
    double flops[HPO_MUON_PROF_N];     /* algorithmic: m(m+1)n for a Gram matrix of an m x n X (one
                                          triangle), m^2(m+1) for A A^T, 2 m^2 n for B X; 0 for the
                                          elementwise passes */
    double bytes[HPO_MUON_PROF_N];     /* algorithmic HBM bytes of the elementwise passes: momentum
                                          16 per element (read G, M; write M, g~), input 8 (read g~,
                                          write X and X^T in bf16) */
} hpo_muon_profile;

/* enable != 0 starts recording (host memory only); enable == 0 waits for the
 * device to go idle, then drops the events and any unread totals.  Both
 * take Muon sets only (HPO_EINVAL otherwise); hpo_muon_profile_read is
 * HPO_EINVAL while timing is off. */
hpo_status hpo_muon_profile_enable(hpo_set s, int32_t enable);
hpo_status hpo_muon_profile_read(hpo_set s, hpo_muon_profile* out);

/* ---------------------------------------------------------------------- */
/* Host-only queries (no device needed)                                   */
/* ---------------------------------------------------------------------- */

/* The work split a list set over these sizes would use, for tensors whose
 * pointers are 16-byte aligned: chunk size, number of chunks (workgroups of
 * the update pass) and the set's own device bytes.  Writes only the outputs
 * given (each may be NULL). */
hpo_status hpo_plan(int32_t n_tensors, const int64_t* numel, int32_t* out_chunk_elems,
                    int64_t* out_n_chunks, int64_t* out_device_bytes);

/* The chunk table such a list set would build: for chunk c, tensor index,
 * first element and element count.  Each array must hold n_chunks entries
 * as returned by hpo_plan. */
hpo_status hpo_plan_chunks(int32_t n_tensors, const int64_t* numel, int64_t n_chunks,
                           int32_t* out_tensor, int64_t* out_start, int32_t* out_len);

const char* hpo_last_error(void);
const char* hpo_status_string(int32_t status);
int32_t hpo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HPO_H */
