/*
 * hpo_muon_impl.h -- layouts shared by the Muon host code (hpo_muon_api.cpp)
 * and the Muon kernels (hpo_muon.hip).  Not part of the public ABI.
 */
#ifndef HPO_MUON_IMPL_H
#define HPO_MUON_IMPL_H

#include "hpo_impl.h"

namespace hpo {

/* ---------------------------------------------------------------------- */
/* Muon                                                                    */
/* ---------------------------------------------------------------------- */
/* Newton-Schulz matrices are zero-padded to multiples of this in both
 * dimensions (the largest GEMM tile), so the GEMMs need no edge handling:
 * zero rows and columns stay zero through every iteration. */
constexpr int64_t kNsPad = 256;
constexpr __host__ __device__ int64_t ns_pad(int64_t x) { return (x + kNsPad - 1) / kNsPad * kNsPad; }

/* Per-matrix facts the Muon kernels need beyond the TensorDesc pointers
 * (param, master, grad, exp_avg = momentum). */
struct MuonInfo {
    int64_t rows, cols;   /* natural shape, row-major */
    int64_t first_chunk;  /* chunks of this matrix: [first_chunk, first_chunk + n_chunks) */
    int32_t n_chunks;
    int32_t transposed;   /* rows > cols: NS works on the transpose */
    int32_t group;
    int32_t reserved;
};
static_assert(sizeof(MuonInfo) == 40, "MuonInfo layout");

/* When a Muon launch runs: host-driven steps read the found_inf flag, the
 * device-resident step reads the state's decision and step window. */
struct MuonGate {
    const int32_t* d_found;       /* host-driven: skip when non-zero (nullable) */
    const hpo_scaler_state* st;   /* device-resident: skip unless applied and in window */
    int64_t t_first;
    int32_t window;
    int32_t dev;
};

/* Scalars of the momentum pass. */
struct MuonScalars {
    float inv_scale;      /* host-driven only */
    float mu, omu;        /* mu and 1 - mu, rounded from binary64 */
    float eps;            /* NS guard added to the fp32 norm */
    double max_norm;
    const float* d_norm;  /* host-driven: the global norm (max_norm > 0) */
    MuonGate gate;
    int32_t form;         /* HPO_MUON_MOMENTUM_SUM / _EMA */
    int32_t nesterov;
};

/* One batch of same-shape matrices stepped together: the matrices
 * [first, first + count) of the set, in the wide orientation m <= n, padded
 * to mp x np, with their chunks [c0, c1). */
struct MuonBatch {
    int32_t first, count;
    int64_t m, n, mp, np;
    int64_t c0, c1;
    int64_t gt_stride;    /* elements between slots of MuonWork::gt (m * n rounded up to 64) */
    int32_t transposed;   /* the natural shape is n x m (rows > cols) */
    int32_t reserved;
};

/* Device workspace of one batch (slot z holds matrix first + z). */
struct MuonWork {
    float* gt;        /* [count][m * n] fp32 Nesterov gradient, natural layout */
    float* dnorm;     /* [n_matrices] fp32(norm(g~)) + eps, indexed by matrix */
    double* part;     /* [n_chunks] per-chunk sum of squares of g~ */
    uint16_t* X;      /* [count][mp][np] bf16 */
    uint16_t* XT[2];  /* [count][np][mp] bf16, ping-pong */
    uint16_t* A;      /* [count][mp][mp] bf16 */
    uint16_t* B;      /* [count][mp][mp] bf16 */
};

/* The update of one Muon step: per-group lr / weight decay (binary64; each
 * matrix forms fp32(1 - lr*wd) and fp32(lr*scale) from them). */
struct MuonUpdate {
    double lr[HPO_MAX_GROUPS];
    double wd[HPO_MAX_GROUPS];
    double extra_scale;   /* the update scale is base(rows, cols) * extra_scale */
    int32_t scale_mode;   /* hpo_muon_scale: which base */
    int32_t param_dtype;  /* HPO_PARAM_BF16 or HPO_PARAM_FP32 */
};

/* Muon launchers (hpo_muon.hip). */
/* Momentum + Nesterov gradient of batch b's matrices into w.gt, with the
 * per-chunk sums of squares, then each matrix's fp32 norm + eps. */
hipError_t launch_muon_momentum(const SetView& sv, const MuonInfo* d_info, const MuonBatch& b, const MuonScalars& sc,
                                const MuonWork& w, hipStream_t stream);
/* bf16 X0 = g~ / (norm + eps) in the wide orientation, and its transpose. */
hipError_t launch_muon_ns_input(const MuonBatch& b, const MuonWork& w, const MuonGate& gate, hipStream_t stream);
/* steps Newton-Schulz iterations on the batch; the last one either updates
 * the masters / params (out == nullptr) or writes O (fp32, natural layout,
 * one matrix: batch count 1) to out.  coeffs: host array of 3 * steps. */
/* Optional callback around each NS launch (timing): kind is a
 * hpo_muon_prof_kind, after = 0 before the launch and 1 after it, flops the
 * launch's algorithmic work. */
struct NsHook {
    void (*fn)(void* ctx, int kind, int after, double flops);
    void* ctx;
};
hipError_t launch_muon_ns(const TensorDesc* d_desc, const MuonInfo* d_info, const MuonBatch& b, const MuonWork& w,
                          const MuonGate& gate, int32_t steps, const float* coeffs, const MuonUpdate& up, float* out,
                          hipStream_t stream, const NsHook* hook = nullptr);
/* Standalone NS input: fp32 G (natural layout, batch count 1) -> its norm
 * into w.dnorm[0], then X0 / XT0. */
hipError_t launch_ns_input_from(const float* G, float eps, const MuonBatch& b, const MuonWork& w, hipStream_t stream);

}  // namespace hpo

#endif /* HPO_MUON_IMPL_H */
