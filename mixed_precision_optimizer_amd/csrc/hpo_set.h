/*
 * hpo_set.h -- the set object and the host helpers shared by libhpo's two
 * host files (hpo_api.cpp: sets and the AdamW step; hpo_muon_api.cpp: Muon
 * sets, NS and the chained step).  Not part of the public ABI.
 */
#ifndef HPO_SET_H
#define HPO_SET_H

#include <string>
#include <vector>

#include "hpo_muon_impl.h"

/* Event-pair timing of Muon launches (hpo_muon_profile_enable). */
struct hpo_muon_prof {
    std::vector<hipEvent_t> pool;  /* created on demand, reused after each read */
    size_t used = 0;               /* events recorded since the last read */
    struct Rec { int kind; size_t ev0, ev1; double flops, bytes; };
    std::vector<Rec> recs;
};

/* Muon-only part of a set: per-matrix facts, the batch plan and the
 * workspace (one device allocation sized for the largest batch). */
struct hpo_muon_part {
    hpo_muon_prof* prof = nullptr;     /* non-NULL while timing is enabled */
    std::vector<hpo::MuonInfo> info;       /* internal (batched) order */
    std::vector<hpo::MuonBatch> batches;
    hpo::MuonInfo* d_info = nullptr;
    char* d_ws = nullptr;                  /* batch buffers, see muon_work() */
    int64_t ws_bytes = 0;
    float* d_dnorm = nullptr;              /* one per matrix */
    double* d_part = nullptr;              /* one per chunk */
};

struct hpo_set_ {
    hpo::SetView view{};
    int32_t kind = HPO_SET_ADAM;
    int32_t n_tensors = 0;
    int32_t param_dtype = 0;
    int32_t is_flat = 0;
    int32_t device = 0;
    int32_t max_group = 0;   /* largest group index in the set */
    int32_t n_vector = 0;
    int64_t numel = 0;
    int64_t n_chunks = 0;
    int32_t grad_group = 1;  /* chunks per grad-pass workgroup */
    int64_t n_parts = 0;     /* grad-pass workgroups = reduction partials */
    int64_t device_bytes = 0;
    hpo::TensorDesc* d_tensors = nullptr;
    hpo::Chunk* d_chunks = nullptr;
    void* d_parts = nullptr;  /* the grad pass's reduction partials (hpo::carve_partials) */
    hpo::Partials parts{};
    hpo_muon_part* muon = nullptr;
};

namespace hpo_host {

/* What a set stores: the model-param dtype and the widths of the moments,
 * the main grads and the master. */
struct Layout {
    int32_t pdt;         /* HPO_PARAM_BF16 / FP32 / FP16 */
    int32_t state_bf16;  /* exp_avg / exp_avg_sq are bf16 */
    int32_t state_fp16;  /* exp_avg / exp_avg_sq are fp16 (refused by decode_dtype) */
    int32_t grad_bf16;   /* main grads are bf16 */
    int32_t master_fp16; /* the master is fp16 (bf16 params only) */
    int64_t mom_bytes() const { return (state_bf16 || state_fp16) ? 2 : 4; }
    int32_t state_store() const { return state_fp16 ? 2 : (state_bf16 ? 1 : 0); }
    int64_t grad_bytes() const { return grad_bf16 ? 2 : 4; }
    int64_t master_bytes() const { return master_fp16 ? 2 : 4; }
    /* bytes of the five arrays per element (the param's none for fp32 params) */
    int64_t elem_bytes() const
    {
        return (pdt == HPO_PARAM_FP32 ? 0 : 2) + master_bytes() + grad_bytes() + 2 * mom_bytes();
    }
    /* whether a set of numel elements takes the update's cached accesses */
    int32_t cached(int64_t numel) const { return numel * elem_bytes() <= hpo::kCachedMaxBytes ? 1 : 0; }
};

hpo_status fail(hpo_status st, const char* fmt, ...);
hpo_status hip_fail(hipError_t e, const char* what);
hpo_status ok();
bool aligned(const void* p, uintptr_t a);
bool is_finite(double x);
int64_t count_chunks(const int64_t* numel, int32_t n, int64_t ch);
int32_t choose_chunk(const int64_t* numel, int32_t n);
void build_chunks(const int64_t* numel, int32_t n, int64_t ch, std::vector<hpo::Chunk>& out);
/* Chunks per grad-pass workgroup, and the workgroups (= partials) of a pass. */
int32_t grad_group_of(int32_t chunk_elems, int64_t n_chunks);
int64_t parts_of(int64_t n_chunks, int32_t group);
int64_t partial_bytes(int64_t n_parts);
hpo_status decode_dtype(int32_t param_dtype, Layout& lay);
/* Pointer rules for one tensor (hpo.h, hpo_set_create_list). */
hpo_status check_tensor(int32_t i, const Layout& lay, void* param, float* master, float* grad, void* m, void* v,
                        int64_t numel);
hpo::TensorDesc make_desc(const Layout& lay, void* param, float* master, float* grad, void* m, void* v,
                          int64_t numel, int32_t group);
/* Argument rules of the step calls (the configuration and the groups). */
hpo_status check_step_args(const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups, int32_t max_group,
                           double max_norm);
hpo_status check_scaler_args(const hpo_scaler_cfg* scfg, const hpo_scaler_state* d_state, int64_t t_first,
                             int32_t window);
/* The update's scalars for a device-resident step over t_first .. t_first + window - 1. */
hpo::AdamScalars device_scalars(const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                                double max_norm, hpo_scaler_state* d_state, int64_t t_first, int32_t window);
hpo::ScalerRule rule_of(const hpo_scaler_cfg* scfg);
/* The finalize outputs of a device-resident step: the state and its end-of-step rule. */
hpo::FinalOut state_out(const hpo_scaler_cfg* scfg, hpo_scaler_state* d_state, int64_t t_first, int32_t window);
hpo_status alloc_partials(hpo_set s);
void free_set(hpo_set s);
hpo_status check_set(hpo_set s);
hipStream_t as_stream(void* stream);
hpo::Partials partials_of(hpo_set s);

/* hpo_muon_api.cpp */
void free_muon(hpo_muon_part* m);
/* Validates a Muon configuration and the groups against a Muon set. */
hpo_status check_muon_step(hpo_set s, const hpo_muon_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                           double max_norm);
/* Enqueues the Muon update of every batch of s behind `gate`. */
hpo_status muon_enqueue(hpo_set s, const hpo_muon_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                        const hpo::MuonGate& gate, float inv_scale, double max_norm, const float* d_norm,
                        hipStream_t stream);

}  // namespace hpo_host

#endif /* HPO_SET_H */
