/*
 * hpo_impl.h -- layouts shared by libhpo's host planner (hpo_api.cpp) and its
 * gfx950 kernels (hpo_kernels.hip).  Not part of the public ABI.
 */
#ifndef HPO_IMPL_H
#define HPO_IMPL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "hpo.h"

namespace hpo {

/* Workgroup size of every streaming kernel (default: 4 wavefronts of 64). */
#ifndef HPO_BLOCK
#define HPO_BLOCK 256
#endif
constexpr int kBlock = HPO_BLOCK;
/* Elements one lane handles per vector access (one 16-byte fp32 load). */
constexpr int kVec = 4;
/* Chunk sizes the planner chooses from (powers of two, multiples of
 * kBlock * kVec so that every chunk start keeps 16-byte alignment). */
#ifndef HPO_MAX_CHUNK_LOG2
#define HPO_MAX_CHUNK_LOG2 14
#endif
constexpr int kMinChunk = 1 << 12;
constexpr int kMaxChunk = 1 << HPO_MAX_CHUNK_LOG2;
/* Aim for at least this many workgroups per pass: 256 CUs x 8. */
constexpr int64_t kTargetChunks = 2048;
/* Workgroup size of the grad pass (read-only streaming; 16 wavefronts). */
#ifndef HPO_GRAD_BLOCK
#define HPO_GRAD_BLOCK 1024
#endif
constexpr int kGradBlock = HPO_GRAD_BLOCK;
/* One grad-pass workgroup covers this many elements' worth of consecutive
 * chunks, so the number of reduction partials stays near numel / 64K. */
#ifndef HPO_GRAD_SPAN_LOG2
#define HPO_GRAD_SPAN_LOG2 16
#endif
constexpr int64_t kGradSpan = int64_t(1) << HPO_GRAD_SPAN_LOG2;
/* Workgroup size of the reduction finalizer, and the partials one
 * workgroup folds per stage (sets with more partials reduce in two stages). */
constexpr int kFinalBlock = 1024;
constexpr int64_t kFinalSpan = 8192;
/* Second-stage partials a set needs for n first-stage partials. */
constexpr int64_t stage_parts(int64_t n) { return n > kFinalSpan ? (n + kFinalSpan - 1) / kFinalSpan : 0; }

/* One tensor of a set, as the kernels see it (64 bytes). */
struct TensorDesc {
    void* param;       /* 16-bit model param; == master for fp32 sets */
    float* master;     /* fp32, or fp16 elements in an HPO_MASTER_FP16 set */
    float* grad;       /* fp32, or bf16 elements in an HPO_GRAD_BF16 set */
    void* exp_avg;     /* fp32 or bf16 elements, per the set's state dtype */
    void* exp_avg_sq;
    int64_t numel;
    int32_t group;
    int32_t vec_ok;    /* every array allows a 4-element vector access (16 B fp32, 8 B 16-bit) */
    int64_t reserved;  /* pads the descriptor to 64 bytes */
};
static_assert(sizeof(TensorDesc) == 64, "TensorDesc layout");

/* One chunk: a contiguous range of one tensor, processed by one workgroup. */
struct Chunk {
    int32_t tensor;
    int32_t len;       /* <= chunk_elems */
    int64_t start;     /* first element, a multiple of chunk_elems */
};
static_assert(sizeof(Chunk) == 16, "Chunk layout");

/* Where a pass finds its tensors: a flat set carries its one descriptor by
 * value and computes chunk ranges from blockIdx; a list set reads both
 * tables from device memory. */
struct SetView {
    TensorDesc flat;            /* flat sets only */
    const TensorDesc* tensors;  /* list sets only */
    const Chunk* chunks;        /* list sets only */
    int64_t chunk_elems;
    int32_t is_flat;
    int32_t param_dtype;  /* HPO_PARAM_BF16 / FP32 / FP16 */
    int32_t state_store;  /* exp_avg / exp_avg_sq storage: 0 fp32, 1 bf16, 2 fp16 */
    int16_t grad_bf16;    /* main grads held as bf16 */
    int16_t master_fp16;  /* master held as fp16 (bf16 params) */
    int32_t cached;       /* the update takes cached (not streaming) accesses: the set fits the on-die cache */
};
/* A set whose five arrays take at most this many bytes stays in MI355X's
 * 256 MB on-die cache from one step to the next, so its update reads and
 * writes through the caches; larger sets stream around them. */
constexpr int64_t kCachedMaxBytes = int64_t(192) << 20;

/* Per-step scalars of the update, all formed on the host in binary64 and
 * rounded to fp32 once. */
struct AdamScalars {
    float inv_scale;
    float b1, b2, c1, c2;   /* beta1, beta2, 1 - beta1, 1 - beta2 */
    float bc1, bc2;         /* 1 - beta1^t, 1 - beta2^t */
    float eps;
    double max_norm;        /* <= 0: no clipping */
    const float* d_norm;    /* device fp32 norm (read when max_norm > 0) */
    const int32_t* d_found; /* device skip flag, nullable */
    float lr[HPO_MAX_GROUPS];
    float wd[HPO_MAX_GROUPS];
    /* device-resident step only: t, inv_scale, norm and the apply decision
     * come from the state; bias corrections from the table for t_first + j */
    const hpo_scaler_state* d_state;
    int64_t t_first;
    int32_t window;
    float bc1_tab[HPO_MAX_WINDOW];
    float bc2_tab[HPO_MAX_WINDOW];
};

static_assert(sizeof(hpo_scaler_state) == 64, "hpo_scaler_state layout");
static_assert(offsetof(hpo_scaler_state, step_inv_scale) == 56, "hpo_scaler_state layout");
static_assert(offsetof(hpo_scaler_state, applied_steps) == 16, "hpo_scaler_state layout");
static_assert(offsetof(hpo_scaler_state, num_zeros) == 48, "hpo_scaler_state layout");

/* Scaler rule constants for the end of a device-resident step. */
struct ScalerRule {
    int32_t dynamic;
    int32_t growth_interval;
    int32_t hysteresis;
    float growth_factor;
    float backoff_factor;
    float min_scale;
};

enum class GradPass : int { kNorm = 0, kCheck = 1, kUnscale = 2 };

/* The reduction partials of one set: one entry per grad-pass workgroup (its
 * binary64 sum of squares, non-finite flag and zero count), and the
 * second-stage entries of sets with more than kFinalSpan of them.  The
 * finalizers fold the partials of several sets (an AdamW set and a Muon set
 * stepped together share one norm, one found_inf and one zero count). */
struct Partials {
    double* sum;
    int32_t* flag;
    int64_t* zeros;
    int64_t n;
    double* stage_sum;    /* stage_parts(n) entries */
    int32_t* stage_flag;
    int64_t* stage_zeros;
};
constexpr int kMaxFoldSets = 4;
/* Device bytes of the partials of a pass with n workgroups (at least one
 * entry, so an empty set still has a place for its finalize to read). */
constexpr int64_t kPartialBytes = sizeof(double) + sizeof(int32_t) + sizeof(int64_t);
constexpr int64_t partial_entries(int64_t n) { return (n > 0 ? n : 1) + stage_parts(n); }
/* Carves the partials of an n-workgroup pass out of one buffer of
 * partial_entries(n) * kPartialBytes bytes, 8-byte aligned. */
inline Partials carve_partials(void* base, int64_t n)
{
    const int64_t first = n > 0 ? n : 1;
    const int64_t e = partial_entries(n);
    char* b = static_cast<char*>(base);
    Partials p;
    p.sum = reinterpret_cast<double*>(b);
    p.zeros = reinterpret_cast<int64_t*>(b + e * sizeof(double));
    p.flag = reinterpret_cast<int32_t*>(b + e * (sizeof(double) + sizeof(int64_t)));
    p.n = n;
    p.stage_sum = p.sum + first;
    p.stage_zeros = p.zeros + first;
    p.stage_flag = p.flag + first;
    return p;
}

/* Where the finalize of a grad pass writes (both nullable per field):
 * host-driven calls get the norm, found_inf and the zero count; the
 * device-resident step gets the state and the end-of-step rule. */
struct FinalOut {
    float* d_norm;
    int32_t* d_found;
    int64_t* d_zeros;
    hpo_scaler_state* st;
    double threshold;
    ScalerRule rule;
    int64_t t_first;
    int32_t window;
};


/* Launchers (hpo_kernels.hip).  Each enqueues on `stream` and returns the
 * launch status. */
/* The grad pass runs one workgroup per group of `grad_group` consecutive
 * chunks (n_parts = ceil(n_chunks / grad_group) workgroups and partials,
 * written to p's first-stage entries). */
hipError_t launch_grad_pass(const SetView& sv, int64_t n_chunks, int32_t grad_group, GradPass pass,
                            float inv_scale, const float* d_inv, const Partials& p, hipStream_t stream);
/* The grad pass followed by its finalize kernels (one stage, or two for
 * sets with more than kFinalSpan partials).  out.st set: the
 * device-resident step's finalize (state, skip decision, counters, scaler);
 * else the norm (when out.d_norm is set), found_inf and the zero count. */
hipError_t launch_grad_pass_final(const SetView& sv, int64_t n_chunks, int32_t grad_group, GradPass pass,
                                  float inv_scale, const float* d_inv, const Partials& p, const FinalOut& out,
                                  hipStream_t stream);
hipError_t launch_adam(const SetView& sv, int64_t n_chunks, int32_t mode, const AdamScalars& sc,
                       hipStream_t stream);
hipError_t launch_scaler_init(hpo_scaler_state* st, float loss_scale, int32_t hysteresis, int64_t applied,
                              hipStream_t stream);
hipError_t launch_copy_main_to_model(const SetView& sv, int64_t n_chunks, hipStream_t stream);
/* The update's memory traffic with no arithmetic (fp32 flat sets with 16-bit params). */
hipError_t launch_stream_probe(const SetView& sv, int64_t n_chunks, hipStream_t stream);
/* Folds the partials of n_sets sets (in order) into *d_norm =
 * fp32(sqrt(sum)) and the zero count *d_zeros (both skipped when d_norm is
 * null: the sums and counts are then not read; d_zeros is nullable) and
 * *d_found |= any flag.  Sets with more than kFinalSpan partials go through
 * their second-stage entries first. */
hipError_t launch_finalize_sets(const Partials* p, int n_sets, float* d_norm, int32_t* d_found, int64_t* d_zeros,
                                hipStream_t stream);
/* Same folding, then the device step state: the norm, the zero count,
 * found_inf, the apply decision (finite, norm <= threshold and t in the
 * window), the counters and the scaler rule, and the step's inv_scale. */
hipError_t launch_finalize_state_sets(const Partials* p, int n_sets, const FinalOut& out, hipStream_t stream);

}  // namespace hpo

#endif /* HPO_IMPL_H */
