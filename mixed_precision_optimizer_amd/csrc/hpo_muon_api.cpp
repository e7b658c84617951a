/*
 * hpo_muon_api.cpp -- host side of the Muon step: Muon sets (batch plan,
 * workspace), hpo_muon_step, the standalone Newton-Schulz call, and the Muon
 * half of the chained device-resident step.
 * Host code only (compiled as plain C++ against the HIP runtime API).
 *
 * Sources (web pages):
 *   [HANDBOOK]   "优化器：AdamW、Muon 与分布式优化器" (ai-infra-handbooks,
 *                train/algo/optimizer), Muon section
 *   [OPT-INFRA]  "02 · Optimizer：算法与 infra" (llm-infra-atlas, train/02_optimizer),
 *                §5 (Muon, NS, Moonlight), §11.4 (one norm for a chain),
 *                §14.3 (no fp16 with Muon), §14.6 (update scales)
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <new>
#include <utility>
#include <vector>

#include "hpo_set.h"

using namespace hpo_host;

namespace {

/* (a, b, c) of the quintic the pages print, applied at every step unless
 * the caller gives a schedule. */
constexpr double kNsA = 3.4445, kNsB = -4.7750, kNsC = 2.0315;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

/* Bytes of one batch slot: g~ (fp32), X, two X^T (bf16, padded), A, B (bf16). */
int64_t slot_bytes(const hpo::MuonBatch& b)
{
    return 4 * b.gt_stride + 2 * (3 * b.mp * b.np + 2 * b.mp * b.mp);
}

/* The batch's buffers inside the set's workspace. */
hpo::MuonWork muon_work(const hpo_muon_part& m, const hpo::MuonBatch& b)
{
    hpo::MuonWork w{};
    char* p = m.d_ws;
    const int64_t c = b.count;
    w.gt = reinterpret_cast<float*>(p);
    p += 4 * c * b.gt_stride;
    w.X = reinterpret_cast<uint16_t*>(p);
    p += 2 * c * b.mp * b.np;
    w.XT[0] = reinterpret_cast<uint16_t*>(p);
    p += 2 * c * b.mp * b.np;
    w.XT[1] = reinterpret_cast<uint16_t*>(p);
    p += 2 * c * b.mp * b.np;
    w.A = reinterpret_cast<uint16_t*>(p);
    p += 2 * c * b.mp * b.mp;
    w.B = reinterpret_cast<uint16_t*>(p);
    w.dnorm = m.d_dnorm;
    w.part = m.d_part;
    return w;
}

hpo::MuonBatch shape_batch(int64_t rows, int64_t cols)
{
    hpo::MuonBatch b{};
    b.transposed = rows > cols ? 1 : 0;
    b.m = b.transposed ? cols : rows;
    b.n = b.transposed ? rows : cols;
    b.mp = hpo::ns_pad(b.m);
    b.np = hpo::ns_pad(b.n);
    b.gt_stride = align_up(b.m * b.n, 64);
    return b;
}

/* The NS coefficients of a step as fp32 (rounded once from binary64). */
void ns_coeffs(const hpo_muon_cfg* cfg, float* out)
{
    for (int32_t s = 0; s < cfg->ns_steps; ++s) {
        const double* c = cfg->ns_coeffs ? cfg->ns_coeffs + 3 * s : nullptr;
        out[3 * s + 0] = static_cast<float>(c ? c[0] : kNsA);
        out[3 * s + 1] = static_cast<float>(c ? c[1] : kNsB);
        out[3 * s + 2] = static_cast<float>(c ? c[2] : kNsC);
    }
}

hpo_status check_muon_cfg(const hpo_muon_cfg* cfg, bool ns_only)
{
    if (!cfg)
        return fail(HPO_EINVAL, "cfg is NULL");
    if (cfg->ns_steps < 1 || cfg->ns_steps > HPO_NS_MAX_STEPS)
        return fail(HPO_EINVAL, "ns_steps must be in [1, %d] (got %d)", HPO_NS_MAX_STEPS, cfg->ns_steps);
    if (!(cfg->ns_eps >= 0.0) || !is_finite(cfg->ns_eps))
        return fail(HPO_EINVAL, "ns_eps must be finite and >= 0 (got %g)", cfg->ns_eps);
    if (cfg->ns_coeffs)
        for (int32_t k = 0; k < 3 * cfg->ns_steps; ++k)
            if (!is_finite(cfg->ns_coeffs[k]))
                return fail(HPO_EINVAL, "ns_coeffs[%d] is not finite", k);
    if (ns_only)
        return HPO_OK;
    if (!(cfg->momentum >= 0.0 && cfg->momentum < 1.0))
        return fail(HPO_EINVAL, "momentum must lie in [0, 1) (got %g)", cfg->momentum);
    if (cfg->nesterov != 0 && cfg->nesterov != 1)
        return fail(HPO_EINVAL, "nesterov must be 0 or 1 (got %d)", cfg->nesterov);
    if (cfg->momentum_form != HPO_MUON_MOMENTUM_SUM && cfg->momentum_form != HPO_MUON_MOMENTUM_EMA)
        return fail(HPO_EINVAL, "momentum_form %d is not a hpo_muon_momentum", cfg->momentum_form);
    if (cfg->scale_mode < HPO_MUON_SCALE_SPECTRAL || cfg->scale_mode > HPO_MUON_SCALE_UNIT_RMS)
        return fail(HPO_EINVAL, "scale_mode %d is not a hpo_muon_scale", cfg->scale_mode);
    if (!(cfg->extra_scale >= 0.0) || !is_finite(cfg->extra_scale))
        return fail(HPO_EINVAL, "extra_scale must be finite and >= 0 (got %g)", cfg->extra_scale);
    return HPO_OK;
}

/* Records one event of the profile pool on `stream`; returns its index. */
size_t prof_mark(hpo_muon_prof& p, hipStream_t stream)
{
    if (p.used == p.pool.size()) {
        hipEvent_t ev = nullptr;
        if (hipEventCreate(&ev) != hipSuccess)
            return SIZE_MAX;
        p.pool.push_back(ev);
    }
    const size_t k = p.used++;
    if (hipEventRecord(p.pool[k], stream) != hipSuccess)
        return SIZE_MAX;
    return k;
}

struct ProfCtx {
    hpo_muon_prof* p;
    hipStream_t stream;
    size_t ev0;
};

void prof_hook(void* ctx, int kind, int after, double flops)
{
    ProfCtx* c = static_cast<ProfCtx*>(ctx);
    if (!after) {
        c->ev0 = prof_mark(*c->p, c->stream);
        return;
    }
    const size_t ev1 = prof_mark(*c->p, c->stream);
    if (c->ev0 != SIZE_MAX && ev1 != SIZE_MAX)
        c->p->recs.push_back({kind, c->ev0, ev1, flops, 0.0});
}

void free_prof(hpo_muon_prof* p)
{
    if (!p)
        return;
    for (hipEvent_t ev : p->pool)
        (void)hipEventDestroy(ev);
    delete p;
}

}  // namespace

namespace hpo_host {

void free_muon(hpo_muon_part* m)
{
    if (!m)
        return;
    free_prof(m->prof);
    if (m->d_info) (void)hipFree(m->d_info);
    if (m->d_ws) (void)hipFree(m->d_ws);
    if (m->d_dnorm) (void)hipFree(m->d_dnorm);
    if (m->d_part) (void)hipFree(m->d_part);
    delete m;
}

hpo_status check_muon_step(hpo_set s, const hpo_muon_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                           double max_norm)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    if (s->kind != HPO_SET_MUON || !s->muon)
        return fail(HPO_EINVAL, "not a Muon set (create it with hpo_muon_set_create)");
    st = check_muon_cfg(cfg, false);
    if (st != HPO_OK)
        return st;
    if (n_groups < 1 || n_groups > HPO_MAX_GROUPS)
        return fail(HPO_EINVAL, "n_groups must be in [1, %d] (got %d)", HPO_MAX_GROUPS, n_groups);
    if (!groups)
        return fail(HPO_EINVAL, "groups is NULL");
    if (s->max_group >= n_groups)
        return fail(HPO_EINVAL, "the set uses group %d but only %d groups were given", s->max_group, n_groups);
    for (int32_t k = 0; k < n_groups; ++k)
        if (!is_finite(groups[k].lr) || !is_finite(groups[k].weight_decay))
            return fail(HPO_EINVAL, "group %d: lr and weight_decay must be finite", k);
    if (std::isnan(max_norm))
        return fail(HPO_EINVAL, "max_norm is NaN");
    return HPO_OK;
}

hpo_status muon_enqueue(hpo_set s, const hpo_muon_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                        const hpo::MuonGate& gate, float inv_scale, double max_norm, const float* d_norm,
                        hipStream_t stream)
{
    hpo::MuonScalars sc{};
    sc.inv_scale = inv_scale;
    sc.mu = static_cast<float>(cfg->momentum);
    sc.omu = static_cast<float>(1.0 - cfg->momentum);
    sc.eps = static_cast<float>(cfg->ns_eps);
    sc.max_norm = max_norm;
    sc.d_norm = d_norm;
    sc.gate = gate;
    sc.form = cfg->momentum_form;
    sc.nesterov = cfg->nesterov;
    hpo::MuonUpdate up{};
    for (int32_t k = 0; k < n_groups; ++k) {
        up.lr[k] = groups[k].lr;
        up.wd[k] = groups[k].weight_decay;
    }
    up.extra_scale = cfg->extra_scale;
    up.scale_mode = cfg->scale_mode;
    up.param_dtype = s->view.param_dtype;
    float coeffs[3 * HPO_NS_MAX_STEPS];
    ns_coeffs(cfg, coeffs);
    const hpo_muon_part& m = *s->muon;
    ProfCtx pc{m.prof, stream, SIZE_MAX};
    const hpo::NsHook hook{prof_hook, &pc};
    const hpo::NsHook* hk = m.prof ? &hook : nullptr;
    for (const hpo::MuonBatch& b : m.batches) {
        const hpo::MuonWork w = muon_work(m, b);
        const double elems = static_cast<double>(b.count) * static_cast<double>(b.m * b.n);
        size_t ev0 = m.prof ? prof_mark(*m.prof, stream) : 0;
        hipError_t e = hpo::launch_muon_momentum(s->view, m.d_info, b, sc, w, stream);
        if (e != hipSuccess)
            return hip_fail(e, "launch Muon momentum");
        if (m.prof) {
            const size_t ev1 = prof_mark(*m.prof, stream);
            if (ev0 != SIZE_MAX && ev1 != SIZE_MAX)
                m.prof->recs.push_back({HPO_MUON_PROF_MOMENTUM, ev0, ev1, 0.0, 16.0 * elems});
            ev0 = ev1;
        }
        e = hpo::launch_muon_ns_input(b, w, gate, stream);
        if (e != hipSuccess)
            return hip_fail(e, "launch Newton-Schulz input");
        if (m.prof) {
            const size_t ev1 = prof_mark(*m.prof, stream);
            if (ev0 != SIZE_MAX && ev1 != SIZE_MAX)
                m.prof->recs.push_back({HPO_MUON_PROF_INPUT, ev0, ev1, 0.0, 8.0 * elems});
        }
        e = hpo::launch_muon_ns(s->d_tensors, m.d_info, b, w, gate, cfg->ns_steps, coeffs, up, nullptr, stream, hk);
        if (e != hipSuccess)
            return hip_fail(e, "launch Newton-Schulz");
    }
    return HPO_OK;
}

}  // namespace hpo_host

extern "C" {

hpo_status hpo_muon_set_create(hpo_set* out, int32_t n_matrices, int32_t param_dtype, void* const* param,
                               float* const* main_param, float* const* main_grad, float* const* momentum,
                               const int64_t* rows, const int64_t* cols, const int32_t* group_index,
                               int64_t workspace_bytes, void* stream)
{
    if (!out)
        return fail(HPO_EINVAL, "out is NULL");
    *out = nullptr;
    if (param_dtype == HPO_PARAM_FP16)
        return fail(HPO_EDTYPE, "fp16 params cannot take Muon (bf16 or fp32 only)");
    if (param_dtype != HPO_PARAM_BF16 && param_dtype != HPO_PARAM_FP32)
        return fail(HPO_EDTYPE, "param dtype %d is not supported by Muon sets (bf16 = 0, fp32 = 1)", param_dtype);
    if (n_matrices < 0)
        return fail(HPO_EINVAL, "n_matrices must be >= 0 (got %d)", n_matrices);
    if (workspace_bytes < 0)
        return fail(HPO_EINVAL, "workspace_bytes must be >= 0");
    if (n_matrices > 0 && (!main_param || !main_grad || !momentum || !rows || !cols))
        return fail(HPO_EINVAL, "pointer and shape arrays must be non-NULL");
    if (n_matrices > 0 && param_dtype == HPO_PARAM_BF16 && !param)
        return fail(HPO_EINVAL, "param array is NULL for a bf16 set");
    const bool bf16 = param_dtype == HPO_PARAM_BF16;
    int32_t max_group = 0;
    for (int32_t i = 0; i < n_matrices; ++i) {
        if (rows[i] < 0 || cols[i] < 0)
            return fail(HPO_EINVAL, "matrix %d: negative shape %lld x %lld", i, (long long)rows[i], (long long)cols[i]);
        if (rows[i] > HPO_MUON_MAX_DIM || cols[i] > HPO_MUON_MAX_DIM ||
            (rows[i] > 0 && cols[i] > (int64_t(1) << 40) / rows[i]))
            return fail(HPO_EINVAL, "matrix %d: %lld x %lld is too large (each side at most %lld, 2^40 elements)", i,
                        (long long)rows[i], (long long)cols[i], (long long)HPO_MUON_MAX_DIM);
        const int32_t g = group_index ? group_index[i] : 0;
        if (g < 0 || g >= HPO_MAX_GROUPS)
            return fail(HPO_EINVAL, "group_index[%d] = %d is outside [0, %d)", i, g, HPO_MAX_GROUPS);
        max_group = std::max(max_group, g);
        if (rows[i] * cols[i] == 0)
            continue;
        void* p = param ? param[i] : nullptr;
        if (!main_param[i] || !main_grad[i] || !momentum[i] || (bf16 && !p))
            return fail(HPO_EINVAL, "matrix %d: a pointer is NULL", i);
        if (!bf16 && p != nullptr && p != static_cast<void*>(main_param[i]))
            return fail(HPO_EINVAL, "matrix %d: an fp32 param is its own master (param must be NULL or main_param)",
                        i);
        if (!aligned(main_param[i], 16) || !aligned(main_grad[i], 16) || !aligned(momentum[i], 16) ||
            (bf16 && !aligned(p, 16)))
            return fail(HPO_EINVAL, "matrix %d: every pointer of a Muon matrix must be 16-byte aligned", i);
    }

    /* internal order: shape classes in order of first appearance, each in
     * input order; empty matrices last (no batch) */
    std::vector<std::pair<int64_t, int64_t>> shapes;
    std::map<std::pair<int64_t, int64_t>, std::vector<int32_t>> members;
    std::vector<int32_t> empty;
    for (int32_t i = 0; i < n_matrices; ++i) {
        if (rows[i] * cols[i] == 0) {
            empty.push_back(i);
            continue;
        }
        const auto key = std::make_pair(rows[i], cols[i]);
        if (!members.count(key))
            shapes.push_back(key);
        members[key].push_back(i);
    }
    std::vector<int32_t> order;
    for (const auto& k : shapes)
        for (int32_t i : members[k])
            order.push_back(i);
    for (int32_t i : empty)
        order.push_back(i);

    std::vector<hpo::TensorDesc> descs(order.size());
    std::vector<int64_t> sizes(order.size());
    for (size_t k = 0; k < order.size(); ++k) {
        const int32_t i = order[k];
        hpo::TensorDesc& d = descs[k];
        d.master = main_param[i];
        d.param = bf16 ? param[i] : static_cast<void*>(main_param[i]);
        d.grad = main_grad[i];
        d.exp_avg = momentum[i];
        d.exp_avg_sq = nullptr;
        d.numel = rows[i] * cols[i];
        d.group = group_index ? group_index[i] : 0;
        d.vec_ok = d.numel > 0 ? 1 : 0;
        sizes[k] = d.numel;
    }
    const int32_t n = static_cast<int32_t>(order.size());
    const int32_t ch = choose_chunk(sizes.data(), n);
    const int64_t nc = count_chunks(sizes.data(), n, ch);
    if (nc > 0x7FFFFFFFLL)
        return fail(HPO_EINVAL, "set needs %lld chunks, more than one launch can hold", (long long)nc);
    std::vector<hpo::Chunk> chunks;
    chunks.reserve(static_cast<size_t>(nc));
    build_chunks(sizes.data(), n, ch, chunks);

    hpo_muon_part* m = new (std::nothrow) hpo_muon_part;
    if (!m)
        return fail(HPO_ENOMEM, "host allocation failed");
    m->info.resize(order.size());
    int64_t c = 0;
    for (size_t k = 0; k < order.size(); ++k) {
        const int32_t i = order[k];
        hpo::MuonInfo& in = m->info[k];
        in.rows = rows[i];
        in.cols = cols[i];
        in.first_chunk = c;
        in.n_chunks = static_cast<int32_t>((sizes[k] + ch - 1) / ch);
        in.transposed = rows[i] > cols[i] ? 1 : 0;
        in.group = descs[k].group;
        c += in.n_chunks;
    }
    /* batches: runs of one shape class, as many matrices as the cap allows */
    const int64_t cap = workspace_bytes > 0 ? workspace_bytes : HPO_MUON_DEFAULT_WORKSPACE;
    int64_t ws = 0;
    int32_t k0 = 0;
    for (const auto& key : shapes) {
        const int32_t cnt = static_cast<int32_t>(members[key].size());
        hpo::MuonBatch proto = shape_batch(key.first, key.second);
        const int64_t per = slot_bytes(proto);
        /* as many matrices per batch as the cap allows, then the class
         * split into equal batches (no small remainder batch) */
        /* a batch's matrices are the z dimension of its launches (at most 65535) */
        constexpr int64_t kMaxBatch = 65535;
        const int64_t fit_cap = std::min<int64_t>(cap / per, kMaxBatch);
        const int32_t most = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(cnt, fit_cap)));
        const int32_t n_batches = (cnt + most - 1) / most;
        const int32_t fit = (cnt + n_batches - 1) / n_batches;
        for (int32_t a = 0; a < cnt; a += fit) {
            hpo::MuonBatch b = proto;
            b.first = k0 + a;
            b.count = std::min(fit, cnt - a);
            b.c0 = m->info[b.first].first_chunk;
            const hpo::MuonInfo& last = m->info[b.first + b.count - 1];
            b.c1 = last.first_chunk + last.n_chunks;
            m->batches.push_back(b);
            ws = std::max(ws, per * b.count);
        }
        k0 += cnt;
    }

    hpo_set s = new (std::nothrow) hpo_set_;
    if (!s) {
        free_muon(m);
        return fail(HPO_ENOMEM, "host allocation failed");
    }
    s->muon = m;
    s->kind = HPO_SET_MUON;
    hipError_t e = hipGetDevice(&s->device);
    if (e != hipSuccess) {
        free_set(s);
        return hip_fail(e, "hipGetDevice");
    }
    s->n_tensors = n_matrices;
    s->param_dtype = param_dtype;
    s->max_group = max_group;
    s->n_chunks = nc;
    s->n_vector = n;
    for (int64_t z : sizes)
        s->numel += z;
    const size_t td_bytes = descs.size() * sizeof(hpo::TensorDesc);
    const size_t ck_bytes = chunks.size() * sizeof(hpo::Chunk);
    const size_t in_bytes = m->info.size() * sizeof(hpo::MuonInfo);
    auto dmalloc = [&](void** p, size_t bytes, const char* what) -> hpo_status {
        if (bytes == 0)
            return HPO_OK;
        hipError_t err = hipMalloc(p, bytes);
        if (err != hipSuccess)
            return fail(HPO_ENOMEM, "hipMalloc of %s (%zu bytes): %s", what, bytes, hipGetErrorString(err));
        s->device_bytes += static_cast<int64_t>(bytes);
        return HPO_OK;
    };
    hpo_status st = dmalloc(reinterpret_cast<void**>(&s->d_tensors), td_bytes, "tensor table");
    if (st == HPO_OK) st = dmalloc(reinterpret_cast<void**>(&s->d_chunks), ck_bytes, "chunk table");
    if (st == HPO_OK) st = dmalloc(reinterpret_cast<void**>(&m->d_info), in_bytes, "matrix table");
    if (st == HPO_OK) st = dmalloc(reinterpret_cast<void**>(&m->d_dnorm), 4 * std::max<size_t>(1, order.size()),
                                   "matrix norms");
    if (st == HPO_OK) st = dmalloc(reinterpret_cast<void**>(&m->d_part), 8 * std::max<int64_t>(1, nc),
                                   "chunk sums");
    if (st == HPO_OK) st = dmalloc(reinterpret_cast<void**>(&m->d_ws), static_cast<size_t>(ws), "NS workspace");
    m->ws_bytes = ws;
    if (st != HPO_OK) {
        free_set(s);
        return st;
    }
    s->view.chunk_elems = ch;
    st = alloc_partials(s);
    if (st != HPO_OK) {
        free_set(s);
        return st;
    }
    hipStream_t strm = as_stream(stream);
    struct Up { void* dst; const void* src; size_t bytes; } ups[] = {
        {s->d_tensors, descs.data(), td_bytes}, {s->d_chunks, chunks.data(), ck_bytes},
        {m->d_info, m->info.data(), in_bytes}};
    for (const Up& u : ups) {
        if (!u.bytes)
            continue;
        e = hipMemcpyAsync(u.dst, u.src, u.bytes, hipMemcpyHostToDevice, strm);
        if (e != hipSuccess) {
            free_set(s);
            return hip_fail(e, "upload Muon tables");
        }
    }
    e = hipStreamSynchronize(strm);
    if (e != hipSuccess) {
        free_set(s);
        return hip_fail(e, "hipStreamSynchronize after table upload");
    }
    s->view.tensors = s->d_tensors;
    s->view.chunks = s->d_chunks;
    s->view.is_flat = 0;
    s->view.param_dtype = param_dtype;
    s->view.state_store = 0;
    *out = s;
    return ok();
}

hpo_status hpo_muon_step(hpo_set s, const hpo_muon_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                         float inv_scale, double max_norm, const float* d_norm, const int32_t* d_found_inf,
                         void* stream)
{
    hpo_status st = check_muon_step(s, cfg, groups, n_groups, max_norm);
    if (st != HPO_OK)
        return st;
    if (!std::isfinite(inv_scale))
        return fail(HPO_EINVAL, "inv_scale must be finite");
    if (max_norm > 0.0 && !d_norm)
        return fail(HPO_EINVAL, "clipping (max_norm > 0) needs d_norm");
    hpo::MuonGate gate{};
    gate.d_found = d_found_inf;
    st = muon_enqueue(s, cfg, groups, n_groups, gate, inv_scale, max_norm, d_norm, as_stream(stream));
    if (st != HPO_OK)
        return st;
    return ok();
}

hpo_status hpo_newton_schulz_workspace(int64_t rows, int64_t cols, int64_t* out_bytes)
{
    if (!out_bytes)
        return fail(HPO_EINVAL, "out_bytes is NULL");
    if (rows < 0 || cols < 0 || rows > HPO_MUON_MAX_DIM || cols > HPO_MUON_MAX_DIM ||
        (rows > 0 && cols > (int64_t(1) << 40) / rows))
        return fail(HPO_EINVAL, "bad shape %lld x %lld (each side in [0, %lld])", (long long)rows, (long long)cols,
                    (long long)HPO_MUON_MAX_DIM);
    if (rows * cols == 0) {
        *out_bytes = 0;
        return ok();
    }
    const hpo::MuonBatch b = shape_batch(rows, cols);
    const int64_t blocks = (rows * cols + 65535) / 65536;
    *out_bytes = align_up(8 * blocks, 256) + 256 + 2 * (3 * b.mp * b.np + 2 * b.mp * b.mp);
    return ok();
}

hpo_status hpo_newton_schulz(const float* d_G, int64_t rows, int64_t cols, const hpo_muon_cfg* cfg, float* d_out,
                             void* d_workspace, int64_t workspace_bytes, void* stream)
{
    hpo_status st = check_muon_cfg(cfg, true);
    if (st != HPO_OK)
        return st;
    int64_t need = 0;
    st = hpo_newton_schulz_workspace(rows, cols, &need);
    if (st != HPO_OK)
        return st;
    if (need == 0)
        return ok();
    if (!d_G || !d_out || !aligned(d_G, 4) || !aligned(d_out, 4))
        return fail(HPO_EINVAL, "d_G and d_out must be non-NULL, 4-byte aligned device pointers");
    if (!d_workspace || !aligned(d_workspace, 256))
        return fail(HPO_EINVAL, "d_workspace must be a non-NULL, 256-byte aligned device pointer");
    if (workspace_bytes < need)
        return fail(HPO_EINVAL, "workspace of %lld bytes is below the %lld this shape needs",
                    (long long)workspace_bytes, (long long)need);
    hpo::MuonBatch b = shape_batch(rows, cols);
    b.first = 0;
    b.count = 1;
    const int64_t blocks = (rows * cols + 65535) / 65536;
    char* p = static_cast<char*>(d_workspace);
    hpo::MuonWork w{};
    w.part = reinterpret_cast<double*>(p);
    p += align_up(8 * blocks, 256);
    w.dnorm = reinterpret_cast<float*>(p);
    p += 256;
    w.X = reinterpret_cast<uint16_t*>(p);
    p += 2 * b.mp * b.np;
    w.XT[0] = reinterpret_cast<uint16_t*>(p);
    p += 2 * b.mp * b.np;
    w.XT[1] = reinterpret_cast<uint16_t*>(p);
    p += 2 * b.mp * b.np;
    w.A = reinterpret_cast<uint16_t*>(p);
    p += 2 * b.mp * b.mp;
    w.B = reinterpret_cast<uint16_t*>(p);
    hipStream_t strm = as_stream(stream);
    hipError_t e = hpo::launch_ns_input_from(d_G, static_cast<float>(cfg->ns_eps), b, w, strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch Newton-Schulz input");
    float coeffs[3 * HPO_NS_MAX_STEPS];
    ns_coeffs(cfg, coeffs);
    hpo::MuonUpdate up{};
    hpo::MuonGate open{};
    e = hpo::launch_muon_ns(nullptr, nullptr, b, w, open, cfg->ns_steps, coeffs, up, d_out, strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch Newton-Schulz");
    return ok();
}

hpo_status hpo_muon_profile_enable(hpo_set s, int32_t enable)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    if (s->kind != HPO_SET_MUON || !s->muon)
        return fail(HPO_EINVAL, "not a Muon set");
    if (enable && !s->muon->prof) {
        s->muon->prof = new (std::nothrow) hpo_muon_prof;
        if (!s->muon->prof)
            return fail(HPO_ENOMEM, "host allocation failed");
    } else if (!enable && s->muon->prof) {
        hipError_t e = hipDeviceSynchronize();
        free_prof(s->muon->prof);
        s->muon->prof = nullptr;
        if (e != hipSuccess)
            return hip_fail(e, "hipDeviceSynchronize before dropping the profile events");
    }
    return ok();
}

hpo_status hpo_muon_profile_read(hpo_set s, hpo_muon_profile* out)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    if (!out)
        return fail(HPO_EINVAL, "out is NULL");
    if (s->kind != HPO_SET_MUON || !s->muon || !s->muon->prof)
        return fail(HPO_EINVAL, "timing is not enabled on this set (hpo_muon_profile_enable)");
    hpo_muon_prof& p = *s->muon->prof;
    *out = hpo_muon_profile{};
    for (const auto& r : p.recs) {
        hipError_t e = hipEventSynchronize(p.pool[r.ev1]);
        if (e != hipSuccess)
            return hip_fail(e, "hipEventSynchronize");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, p.pool[r.ev0], p.pool[r.ev1]);
        if (e != hipSuccess)
            return hip_fail(e, "hipEventElapsedTime");
        out->ms[r.kind] += ms;
        out->launches[r.kind] += 1;
        out->flops[r.kind] += r.flops;
        out->bytes[r.kind] += r.bytes;
    }
    p.recs.clear();
    p.used = 0;
    return ok();
}

}  // extern "C"
