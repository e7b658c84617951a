/*
 * hpo_api.cpp -- host side of libhpo: argument validation, the chunk planner,
 * set lifecycle, the per-step scalars and the C entry points of hpo.h.
 * Host code only (compiled as plain C++ against the HIP runtime API).
 *
 * Sources (web pages):
 *   [OPT-INFRA]  "02 · Optimizer：算法与 infra" (llm-infra-atlas, train/02_optimizer)
 *   [FP32-RFC]   "支持FP32优化器" (hyper-parallel issue)
 */
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "hpo_set.h"

namespace hpo_host {

thread_local std::string g_last_error;

hpo_status fail(hpo_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

hpo_status hip_fail(hipError_t e, const char* what)
{
    return fail(HPO_EHIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

hpo_status ok()
{
    g_last_error.clear();
    return HPO_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t count_chunks(const int64_t* numel, int32_t n, int64_t ch)
{
    int64_t c = 0;
    for (int32_t i = 0; i < n; ++i)
        c += (numel[i] + ch - 1) / ch;
    return c;
}

/* Largest power-of-two chunk in [kMinChunk, kMaxChunk] that still gives at
 * least kTargetChunks workgroups per pass; small sets get the smallest. */
int32_t choose_chunk(const int64_t* numel, int32_t n)
{
    for (int64_t ch = hpo::kMaxChunk; ch >= hpo::kMinChunk; ch >>= 1)
        if (count_chunks(numel, n, ch) >= hpo::kTargetChunks)
            return static_cast<int32_t>(ch);
    return hpo::kMinChunk;
}

/* A grad pass keeps at least this many workgroups (four per CU of a 256-CU
 * chip) when the set has the chunks for it, so that small sets are still
 * read by the whole chip. */
constexpr int64_t kGradMinParts = 1024;

/* Chunks per grad-pass workgroup: enough to cover kGradSpan elements, fewer
 * where that would leave under kGradMinParts workgroups. */
int32_t grad_group_of(int32_t chunk_elems, int64_t n_chunks)
{
    int64_t g = hpo::kGradSpan / chunk_elems;
    const int64_t cap = n_chunks / kGradMinParts;
    if (g > cap)
        g = cap;
    return static_cast<int32_t>(g > 1 ? g : 1);
}

int64_t parts_of(int64_t n_chunks, int32_t group) { return (n_chunks + group - 1) / group; }

/* First-stage partials plus the second-stage ones of large sets. */
int64_t partial_bytes(int64_t n_parts) { return hpo::partial_entries(n_parts) * hpo::kPartialBytes; }

hpo_status check_sizes(int32_t n_tensors, const int64_t* numel)
{
    if (n_tensors < 0)
        return fail(HPO_EINVAL, "n_tensors must be >= 0 (got %d)", n_tensors);
    if (n_tensors > 0 && numel == nullptr)
        return fail(HPO_EINVAL, "numel is NULL");
    for (int32_t i = 0; i < n_tensors; ++i)
        if (numel[i] < 0)
            return fail(HPO_EINVAL, "numel[%d] = %lld is negative", i, (long long)numel[i]);
    return HPO_OK;
}

hpo_status decode_dtype(int32_t param_dtype, Layout& lay)
{
    constexpr int32_t kFlags = HPO_STATE_BF16 | HPO_STATE_FP16 | HPO_GRAD_BF16 | HPO_MASTER_FP16;
    lay.pdt = param_dtype & 0xFF;
    lay.state_bf16 = (param_dtype & HPO_STATE_BF16) ? 1 : 0;
    lay.state_fp16 = (param_dtype & HPO_STATE_FP16) ? 1 : 0;
    lay.grad_bf16 = (param_dtype & HPO_GRAD_BF16) ? 1 : 0;
    lay.master_fp16 = (param_dtype & HPO_MASTER_FP16) ? 1 : 0;
    const bool pdt_ok = lay.pdt == HPO_PARAM_BF16 || lay.pdt == HPO_PARAM_FP32 || lay.pdt == HPO_PARAM_FP16;
    if (!pdt_ok || (param_dtype & ~(0xFF | kFlags)) != 0)
        return fail(HPO_EDTYPE,
                    "param dtype %d is not supported (bf16 = 0, fp32 = 1, fp16 = 2, optionally | HPO_STATE_BF16 "
                    "or HPO_STATE_FP16, | HPO_GRAD_BF16, | HPO_MASTER_FP16)",
                    param_dtype);
    if (lay.state_fp16)
        return fail(HPO_EDTYPE,
                    "fp16 moments (HPO_STATE_FP16) are not supported: with no per-tensor scale fp16 stores "
                    "exp_avg_sq = (1 - beta2) g^2 as 0 below |g| ~ 1.7e-4; use bf16 moments (HPO_STATE_BF16)");
    if (lay.master_fp16 && lay.pdt != HPO_PARAM_BF16)
        return fail(HPO_EDTYPE, "HPO_MASTER_FP16 needs bf16 params (param dtype %d)", param_dtype);
    return HPO_OK;
}

void* advance(void* p, int64_t elems, int64_t bytes)
{
    return p ? static_cast<void*>(static_cast<char*>(p) + elems * bytes) : nullptr;
}

/* Pointer rules for one tensor (see hpo.h). */
hpo_status check_tensor(int32_t i, const Layout& lay, void* param, float* master, float* grad, void* m, void* v,
                        int64_t numel)
{
    if (numel == 0)
        return HPO_OK;
    if (!master || !grad || !m || !v)
        return fail(HPO_EINVAL, "tensor %d: main_param, main_grad, exp_avg and exp_avg_sq must be non-NULL", i);
    if (!aligned(master, static_cast<uintptr_t>(lay.master_bytes())))
        return fail(HPO_EINVAL, "tensor %d: main_param must be %lld-byte aligned", i, (long long)lay.master_bytes());
    if (!aligned(grad, static_cast<uintptr_t>(lay.grad_bytes())))
        return fail(HPO_EINVAL, "tensor %d: main_grad must be %lld-byte aligned", i, (long long)lay.grad_bytes());
    if (!aligned(m, static_cast<uintptr_t>(lay.mom_bytes())) || !aligned(v, static_cast<uintptr_t>(lay.mom_bytes())))
        return fail(HPO_EINVAL, "tensor %d: exp_avg / exp_avg_sq must be %lld-byte aligned", i,
                    (long long)lay.mom_bytes());
    if (lay.pdt != HPO_PARAM_FP32) {
        if (!param)
            return fail(HPO_EINVAL, "tensor %d: 16-bit param pointer is NULL", i);
        if (!aligned(param, 2))
            return fail(HPO_EINVAL, "tensor %d: 16-bit param pointer must be 2-byte aligned", i);
    } else if (param != nullptr && param != static_cast<void*>(master)) {
        return fail(HPO_EINVAL,
                    "tensor %d: an fp32 param is its own master, so param must be NULL or equal main_param", i);
    }
    return HPO_OK;
}

hpo::TensorDesc make_desc(const Layout& lay, void* param, float* master, float* grad, void* m, void* v,
                          int64_t numel, int32_t group)
{
    hpo::TensorDesc d{};
    d.param = (lay.pdt == HPO_PARAM_FP32) ? static_cast<void*>(master) : param;
    d.master = master;
    d.grad = grad;
    d.exp_avg = m;
    d.exp_avg_sq = v;
    d.numel = numel;
    d.group = group;
    const bool p_ok = (lay.pdt == HPO_PARAM_FP32) || aligned(d.param, 8);
    /* 4 elements of each array */
    const uintptr_t mv = static_cast<uintptr_t>(4 * lay.mom_bytes());
    const uintptr_t tv = static_cast<uintptr_t>(4 * lay.master_bytes());
    const uintptr_t gv = static_cast<uintptr_t>(4 * lay.grad_bytes());
    d.vec_ok = (aligned(master, tv) && aligned(grad, gv) && aligned(m, mv) && aligned(v, mv) && p_ok) ? 1 : 0;
    return d;
}

/* Position of a pointer inside the aligned line that holds 4 of its
 * elements, in elements: 0..3 (16-byte lines for fp32, 8-byte lines for
 * 16-bit data). */
int32_t phase_of(const void* p, int64_t bytes)
{
    return static_cast<int32_t>((reinterpret_cast<uintptr_t>(p) / static_cast<uintptr_t>(bytes)) % 4);
}

float* advance_f(float* p, int64_t elems, int64_t bytes) { return static_cast<float*>(advance(p, elems, bytes)); }

/* Appends the descriptor piece(s) of one tensor.  A tensor whose pointers all
 * sit at the same element phase of their 4-element lines (views that start
 * a few elements into a flat buffer, shard ranges) is split into a head of
 * fewer than 4 elements on the element-at-a-time path and a body whose
 * pointers all allow vector access.  Returns whether the tensor's body takes
 * the vector path. */
bool add_pieces(std::vector<hpo::TensorDesc>& out, const Layout& lay, void* param, float* master, float* grad,
                void* m, void* v, int64_t numel, int32_t group)
{
    if (numel == 0) {
        out.push_back(make_desc(lay, param, master, grad, m, v, 0, group));
        return false;
    }
    hpo::TensorDesc d = make_desc(lay, param, master, grad, m, v, numel, group);
    if (d.vec_ok) {
        out.push_back(d);
        return true;
    }
    const int32_t ph = phase_of(master, lay.master_bytes());
    const bool same = phase_of(grad, lay.grad_bytes()) == ph && phase_of(m, lay.mom_bytes()) == ph &&
                      phase_of(v, lay.mom_bytes()) == ph && (lay.pdt == HPO_PARAM_FP32 || phase_of(param, 2) == ph);
    if (!same) {
        out.push_back(d);
        return false;
    }
    const int64_t head = std::min<int64_t>((4 - ph) % 4, numel);
    out.push_back(make_desc(lay, param, master, grad, m, v, head, group));
    if (numel == head)
        return false;
    void* p2 = (lay.pdt == HPO_PARAM_FP32) ? nullptr : advance(param, head, 2);
    hpo::TensorDesc body = make_desc(lay, p2, advance_f(master, head, lay.master_bytes()),
                                     advance_f(grad, head, lay.grad_bytes()), advance(m, head, lay.mom_bytes()),
                                     advance(v, head, lay.mom_bytes()), numel - head, group);
    out.push_back(body);
    return body.vec_ok != 0;
}

void piece_sizes(const std::vector<hpo::TensorDesc>& descs, std::vector<int64_t>& sizes)
{
    sizes.resize(descs.size());
    for (size_t i = 0; i < descs.size(); ++i)
        sizes[i] = descs[i].numel;
}

void build_chunks(const int64_t* numel, int32_t n, int64_t ch, std::vector<hpo::Chunk>& out)
{
    for (int32_t i = 0; i < n; ++i)
        for (int64_t s = 0; s < numel[i]; s += ch) {
            hpo::Chunk c;
            c.tensor = i;
            c.start = s;
            c.len = static_cast<int32_t>(numel[i] - s < ch ? numel[i] - s : ch);
            out.push_back(c);
        }
}

void free_set(hpo_set s)
{
    if (!s)
        return;
    if (s->d_tensors) (void)hipFree(s->d_tensors);
    if (s->d_chunks) (void)hipFree(s->d_chunks);
    if (s->d_parts) (void)hipFree(s->d_parts);
    free_muon(s->muon);
    delete s;
}

hpo_status alloc_partials(hpo_set s)
{
    s->grad_group = grad_group_of(static_cast<int32_t>(s->view.chunk_elems), s->n_chunks);
    s->n_parts = parts_of(s->n_chunks, s->grad_group);
    const int64_t bytes = partial_bytes(s->n_parts);
    hipError_t e = hipMalloc(&s->d_parts, static_cast<size_t>(bytes));
    if (e != hipSuccess)
        return fail(HPO_ENOMEM, "hipMalloc of %lld reduction partials: %s", (long long)hpo::partial_entries(s->n_parts),
                    hipGetErrorString(e));
    s->parts = hpo::carve_partials(s->d_parts, s->n_parts);
    s->device_bytes += bytes;
    return HPO_OK;
}

hpo_status check_set(hpo_set s)
{
    if (!s)
        return fail(HPO_EINVAL, "set is NULL");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev != s->device)
        return fail(HPO_EDEVICE, "current device %d is not the set's device %d", dev, s->device);
    return HPO_OK;
}

hipStream_t as_stream(void* stream) { return static_cast<hipStream_t>(stream); }

bool is_finite(double x) { return std::isfinite(x); }

hpo::Partials partials_of(hpo_set s) { return s->parts; }

}  // namespace hpo_host

using namespace hpo_host;

extern "C" {

int32_t hpo_abi_version(void) { return HPO_ABI_VERSION; }

const char* hpo_last_error(void) { return g_last_error.c_str(); }

const char* hpo_status_string(int32_t status)
{
    switch (status) {
    case HPO_OK: return "HPO_OK";
    case HPO_EINVAL: return "HPO_EINVAL";
    case HPO_EDTYPE: return "HPO_EDTYPE";
    case HPO_ENOMEM: return "HPO_ENOMEM";
    case HPO_EHIP: return "HPO_EHIP";
    case HPO_EDEVICE: return "HPO_EDEVICE";
    default: return "unknown hpo_status";
    }
}

hpo_status hpo_plan(int32_t n_tensors, const int64_t* numel, int32_t* out_chunk_elems,
                    int64_t* out_n_chunks, int64_t* out_device_bytes)
{
    hpo_status st = check_sizes(n_tensors, numel);
    if (st != HPO_OK)
        return st;
    const int32_t ch = choose_chunk(numel, n_tensors);
    const int64_t nc = count_chunks(numel, n_tensors, ch);
    if (out_chunk_elems) *out_chunk_elems = ch;
    if (out_n_chunks) *out_n_chunks = nc;
    if (out_device_bytes)
        *out_device_bytes = static_cast<int64_t>(n_tensors) * sizeof(hpo::TensorDesc) +
                            nc * static_cast<int64_t>(sizeof(hpo::Chunk)) +
                            partial_bytes(parts_of(nc, grad_group_of(ch, nc)));
    return ok();
}

hpo_status hpo_plan_chunks(int32_t n_tensors, const int64_t* numel, int64_t n_chunks,
                           int32_t* out_tensor, int64_t* out_start, int32_t* out_len)
{
    hpo_status st = check_sizes(n_tensors, numel);
    if (st != HPO_OK)
        return st;
    const int32_t ch = choose_chunk(numel, n_tensors);
    std::vector<hpo::Chunk> chunks;
    build_chunks(numel, n_tensors, ch, chunks);
    if (static_cast<int64_t>(chunks.size()) != n_chunks)
        return fail(HPO_EINVAL, "n_chunks %lld does not match the plan (%zu)", (long long)n_chunks, chunks.size());
    if (n_chunks > 0 && (!out_tensor || !out_start || !out_len))
        return fail(HPO_EINVAL, "output arrays must be non-NULL");
    for (size_t c = 0; c < chunks.size(); ++c) {
        out_tensor[c] = chunks[c].tensor;
        out_start[c] = chunks[c].start;
        out_len[c] = chunks[c].len;
    }
    return ok();
}

}  // extern "C"

namespace {

/* Builds a table-driven set from descriptor pieces (see add_pieces). */
hpo_status create_from_pieces(hpo_set* out, int32_t param_dtype, const Layout& lay,
                              std::vector<hpo::TensorDesc>& descs, int32_t n_tensors, int32_t n_vector,
                              int32_t max_group, void* stream)
{
    if (descs.size() > 0x7FFFFFFFu)
        return fail(HPO_EINVAL, "too many tensor pieces");
    std::vector<int64_t> sizes;
    piece_sizes(descs, sizes);
    const int32_t n_pieces = static_cast<int32_t>(descs.size());
    const int32_t ch = choose_chunk(sizes.data(), n_pieces);
    const int64_t nc = count_chunks(sizes.data(), n_pieces, ch);
    if (nc > 0x7FFFFFFFLL)
        return fail(HPO_EINVAL, "set needs %lld chunks, more than one launch can hold", (long long)nc);

    hpo_set s = new (std::nothrow) hpo_set_;
    if (!s)
        return fail(HPO_ENOMEM, "host allocation failed");
    hipError_t e = hipGetDevice(&s->device);
    if (e != hipSuccess) {
        free_set(s);
        return hip_fail(e, "hipGetDevice");
    }
    s->n_tensors = n_tensors;
    s->param_dtype = param_dtype;
    s->is_flat = 0;
    s->max_group = max_group;
    s->n_chunks = nc;
    s->n_vector = n_vector;
    for (const auto& d : descs)
        s->numel += d.numel;

    std::vector<hpo::Chunk> chunks;
    chunks.reserve(static_cast<size_t>(nc));
    build_chunks(sizes.data(), n_pieces, ch, chunks);

    const size_t td_bytes = descs.size() * sizeof(hpo::TensorDesc);
    const size_t ck_bytes = chunks.size() * sizeof(hpo::Chunk);
    if (td_bytes) {
        e = hipMalloc(reinterpret_cast<void**>(&s->d_tensors), td_bytes);
        if (e != hipSuccess) { free_set(s); return fail(HPO_ENOMEM, "hipMalloc tensor table: %s", hipGetErrorString(e)); }
    }
    if (ck_bytes) {
        e = hipMalloc(reinterpret_cast<void**>(&s->d_chunks), ck_bytes);
        if (e != hipSuccess) { free_set(s); return fail(HPO_ENOMEM, "hipMalloc chunk table: %s", hipGetErrorString(e)); }
    }
    s->device_bytes = static_cast<int64_t>(td_bytes + ck_bytes);
    s->view.chunk_elems = ch;
    hpo_status st = alloc_partials(s);
    if (st != HPO_OK) { free_set(s); return st; }
    if (td_bytes) {
        e = hipMemcpyAsync(s->d_tensors, descs.data(), td_bytes, hipMemcpyHostToDevice, as_stream(stream));
        if (e != hipSuccess) { free_set(s); return hip_fail(e, "upload tensor table"); }
    }
    if (ck_bytes) {
        e = hipMemcpyAsync(s->d_chunks, chunks.data(), ck_bytes, hipMemcpyHostToDevice, as_stream(stream));
        if (e != hipSuccess) { free_set(s); return hip_fail(e, "upload chunk table"); }
    }
    e = hipStreamSynchronize(as_stream(stream));
    if (e != hipSuccess) { free_set(s); return hip_fail(e, "hipStreamSynchronize after table upload"); }

    s->view.tensors = s->d_tensors;
    s->view.chunks = s->d_chunks;
    s->view.is_flat = 0;
    s->view.param_dtype = lay.pdt;
    s->view.state_store = lay.state_store();
    s->view.grad_bf16 = static_cast<int16_t>(lay.grad_bf16);
    s->view.master_fp16 = static_cast<int16_t>(lay.master_fp16);
    s->view.cached = lay.cached(s->numel);
    *out = s;
    return ok();
}

}  // namespace

extern "C" {

hpo_status hpo_set_create_list(hpo_set* out, int32_t n_tensors, int32_t param_dtype,
                               void* const* param, float* const* main_param,
                               float* const* main_grad, float* const* exp_avg,
                               float* const* exp_avg_sq, const int64_t* numel,
                               const int32_t* group_index, void* stream)
{
    if (!out)
        return fail(HPO_EINVAL, "out is NULL");
    *out = nullptr;
    Layout lay{};
    hpo_status st = decode_dtype(param_dtype, lay);
    if (st != HPO_OK)
        return st;
    st = check_sizes(n_tensors, numel);
    if (st != HPO_OK)
        return st;
    if (n_tensors > 0 && (!main_param || !main_grad || !exp_avg || !exp_avg_sq))
        return fail(HPO_EINVAL, "pointer arrays must be non-NULL");
    if (n_tensors > 0 && lay.pdt != HPO_PARAM_FP32 && !param)
        return fail(HPO_EINVAL, "param array is NULL for a 16-bit-param set");
    int32_t max_group = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        void* p = param ? param[i] : nullptr;
        st = check_tensor(i, lay, p, main_param[i], main_grad[i], exp_avg[i], exp_avg_sq[i], numel[i]);
        if (st != HPO_OK)
            return st;
        const int32_t g = group_index ? group_index[i] : 0;
        if (g < 0 || g >= HPO_MAX_GROUPS)
            return fail(HPO_EINVAL, "group_index[%d] = %d is outside [0, %d)", i, g, HPO_MAX_GROUPS);
        if (g > max_group)
            max_group = g;
    }
    std::vector<hpo::TensorDesc> descs;
    descs.reserve(static_cast<size_t>(n_tensors));
    int32_t n_vector = 0;
    for (int32_t i = 0; i < n_tensors; ++i)
        n_vector += add_pieces(descs, lay, param ? param[i] : nullptr, main_param[i], main_grad[i],
                               exp_avg[i], exp_avg_sq[i], numel[i], group_index ? group_index[i] : 0);
    return create_from_pieces(out, param_dtype, lay, descs, n_tensors, n_vector, max_group, stream);
}

hpo_status hpo_set_create_flat_ranges(hpo_set* out, int64_t numel, int32_t param_dtype, void* param,
                                      float* main_param, float* main_grad, float* exp_avg,
                                      float* exp_avg_sq, int32_t n_ranges, const int64_t* range_start,
                                      const int32_t* range_group, void* stream)
{
    if (!out)
        return fail(HPO_EINVAL, "out is NULL");
    *out = nullptr;
    Layout lay{};
    hpo_status st = decode_dtype(param_dtype, lay);
    if (st != HPO_OK)
        return st;
    st = check_sizes(1, &numel);
    if (st != HPO_OK)
        return st;
    st = check_tensor(0, lay, param, main_param, main_grad, exp_avg, exp_avg_sq, numel);
    if (st != HPO_OK)
        return st;
    if (n_ranges < 1 || !range_start || !range_group)
        return fail(HPO_EINVAL, "a flat shard with ranges needs n_ranges >= 1 and both range arrays");
    if (range_start[0] != 0)
        return fail(HPO_EINVAL, "range_start[0] must be 0 (got %lld)", (long long)range_start[0]);
    int32_t max_group = 0;
    for (int32_t k = 0; k < n_ranges; ++k) {
        const int64_t end = k + 1 < n_ranges ? range_start[k + 1] : numel;
        if (end <= range_start[k] || end > numel)
            return fail(HPO_EINVAL, "range %d [%lld, %lld) is empty, unordered or past numel %lld", k,
                        (long long)range_start[k], (long long)end, (long long)numel);
        if (range_group[k] < 0 || range_group[k] >= HPO_MAX_GROUPS)
            return fail(HPO_EINVAL, "range_group[%d] = %d is outside [0, %d)", k, range_group[k], HPO_MAX_GROUPS);
        max_group = std::max(max_group, range_group[k]);
    }
    std::vector<hpo::TensorDesc> descs;
    descs.reserve(static_cast<size_t>(n_ranges) + 1);
    int32_t n_vector = 0;
    for (int32_t k = 0; k < n_ranges; ++k) {
        const int64_t a = range_start[k];
        const int64_t len = (k + 1 < n_ranges ? range_start[k + 1] : numel) - a;
        void* p = (lay.pdt == HPO_PARAM_FP32) ? param : advance(param, a, 2);
        n_vector += add_pieces(descs, lay, p, advance_f(main_param, a, lay.master_bytes()),
                               advance_f(main_grad, a, lay.grad_bytes()), advance(exp_avg, a, lay.mom_bytes()),
                               advance(exp_avg_sq, a, lay.mom_bytes()), len, range_group[k]);
    }
    return create_from_pieces(out, param_dtype, lay, descs, n_ranges, n_vector, max_group, stream);
}

hpo_status hpo_set_create_flat(hpo_set* out, int64_t numel, int32_t param_dtype, void* param,
                               float* main_param, float* main_grad, float* exp_avg,
                               float* exp_avg_sq, void* stream)
{
    if (!out)
        return fail(HPO_EINVAL, "out is NULL");
    *out = nullptr;
    Layout lay{};
    hpo_status st = decode_dtype(param_dtype, lay);
    if (st != HPO_OK)
        return st;
    st = check_sizes(1, &numel);
    if (st != HPO_OK)
        return st;
    st = check_tensor(0, lay, param, main_param, main_grad, exp_avg, exp_avg_sq, numel);
    if (st != HPO_OK)
        return st;
    if (numel > 0 && !make_desc(lay, param, main_param, main_grad, exp_avg, exp_avg_sq, numel, 0).vec_ok) {
        /* a flat range that does not start on a vector line: table-driven,
         * with the head peeled off (same results, vector body) */
        std::vector<hpo::TensorDesc> descs;
        const int32_t nv = add_pieces(descs, lay, param, main_param, main_grad, exp_avg, exp_avg_sq, numel, 0);
        st = create_from_pieces(out, param_dtype, lay, descs, 1, nv, 0, stream);
        if (st == HPO_OK)
            (*out)->is_flat = 1;
        return st;
    }
    const int32_t ch = choose_chunk(&numel, 1);
    const int64_t nc = count_chunks(&numel, 1, ch);
    if (nc > 0x7FFFFFFFLL)
        return fail(HPO_EINVAL, "set needs %lld chunks, more than one launch can hold", (long long)nc);

    hpo_set s = new (std::nothrow) hpo_set_;
    if (!s)
        return fail(HPO_ENOMEM, "host allocation failed");
    hipError_t e = hipGetDevice(&s->device);
    if (e != hipSuccess) {
        free_set(s);
        return hip_fail(e, "hipGetDevice");
    }
    s->n_tensors = 1;
    s->param_dtype = param_dtype;
    s->is_flat = 1;
    s->numel = numel;
    s->n_chunks = nc;
    s->view.flat = make_desc(lay, param, main_param, main_grad, exp_avg, exp_avg_sq, numel, 0);
    s->n_vector = s->view.flat.vec_ok;
    s->view.chunk_elems = ch;
    s->view.is_flat = 1;
    s->view.param_dtype = lay.pdt;
    s->view.state_store = lay.state_store();
    s->view.grad_bf16 = static_cast<int16_t>(lay.grad_bf16);
    s->view.master_fp16 = static_cast<int16_t>(lay.master_fp16);
    s->view.cached = lay.cached(numel);
    st = alloc_partials(s);
    if (st != HPO_OK) { free_set(s); return st; }
    *out = s;
    return ok();
}

hpo_status hpo_set_destroy(hpo_set s)
{
    if (!s)
        return ok();
    hipError_t e = hipDeviceSynchronize();
    free_set(s);
    if (e != hipSuccess)
        return hip_fail(e, "hipDeviceSynchronize before freeing the set");
    return ok();
}

hpo_status hpo_set_info(hpo_set s, hpo_set_info_t* out)
{
    if (!s || !out)
        return fail(HPO_EINVAL, "set and out must be non-NULL");
    out->n_tensors = s->n_tensors;
    out->param_dtype = s->param_dtype;
    out->is_flat = s->is_flat;
    out->chunk_elems = static_cast<int32_t>(s->view.chunk_elems);
    out->numel = s->numel;
    out->n_chunks = s->n_chunks;
    out->device_bytes = s->device_bytes;
    out->device = s->device;
    out->n_vector = s->n_vector;
    out->grad_group = s->grad_group;
    out->kind = s->kind;
    out->n_grad_parts = s->n_parts;
    return ok();
}

hpo_status hpo_unscale_check_inf(hpo_set s, float inv_scale, int32_t* d_found_inf, void* stream)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    if (!d_found_inf)
        return fail(HPO_EINVAL, "d_found_inf is NULL");
    if (!std::isfinite(inv_scale))
        return fail(HPO_EINVAL, "inv_scale must be finite");
    const hpo::GradPass pass = (inv_scale == 1.0f) ? hpo::GradPass::kCheck : hpo::GradPass::kUnscale;
    hpo::FinalOut out{};
    out.d_found = d_found_inf;
    hipError_t e = hpo::launch_grad_pass_final(s->view, s->n_chunks, s->grad_group, pass, inv_scale, nullptr,
                                               s->parts, out, as_stream(stream));
    if (e != hipSuccess)
        return hip_fail(e, "launch unscale/check pass");
    return ok();
}

hpo_status hpo_grad_global_norm(hpo_set s, float inv_scale, float* d_norm, int32_t* d_found_inf,
                                int64_t* d_num_zeros, void* stream)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    if (!d_norm)
        return fail(HPO_EINVAL, "d_norm is NULL");
    if (!std::isfinite(inv_scale))
        return fail(HPO_EINVAL, "inv_scale must be finite");
    if (d_num_zeros && !aligned(d_num_zeros, 8))
        return fail(HPO_EINVAL, "d_num_zeros must be 8-byte aligned");
    hpo::FinalOut out{};
    out.d_norm = d_norm;
    out.d_found = d_found_inf;
    out.d_zeros = d_num_zeros;
    hipError_t e = hpo::launch_grad_pass_final(s->view, s->n_chunks, s->grad_group, hpo::GradPass::kNorm,
                                               inv_scale, nullptr, s->parts, out, as_stream(stream));
    if (e != hipSuccess)
        return hip_fail(e, "launch norm pass and finalize");
    return ok();
}

}  // extern "C"

namespace hpo_host {

/* Argument rules shared by the step calls: the configuration and the groups
 * (max_group: the largest group index the stepped tensors use). */
hpo_status check_step_args(const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups, int32_t max_group,
                           double max_norm)
{
    if (!cfg)
        return fail(HPO_EINVAL, "cfg is NULL");
    if (cfg->mode != HPO_ADAMW && cfg->mode != HPO_ADAM_L2)
        return fail(HPO_EINVAL, "mode %d is neither HPO_ADAMW (0) nor HPO_ADAM_L2 (1)", cfg->mode);
    if (!(cfg->beta1 >= 0.0 && cfg->beta1 < 1.0) || !(cfg->beta2 >= 0.0 && cfg->beta2 < 1.0))
        return fail(HPO_EINVAL, "betas must lie in [0, 1) (got %g, %g)", cfg->beta1, cfg->beta2);
    if (!(cfg->eps >= 0.0) || !is_finite(cfg->eps))
        return fail(HPO_EINVAL, "eps must be finite and >= 0 (got %g)", cfg->eps);
    if (n_groups < 1 || n_groups > HPO_MAX_GROUPS)
        return fail(HPO_EINVAL, "n_groups must be in [1, %d] (got %d)", HPO_MAX_GROUPS, n_groups);
    if (!groups)
        return fail(HPO_EINVAL, "groups is NULL");
    if (max_group >= n_groups)
        return fail(HPO_EINVAL, "the set uses group %d but only %d groups were given", max_group, n_groups);
    for (int32_t k = 0; k < n_groups; ++k)
        if (!is_finite(groups[k].lr) || !is_finite(groups[k].weight_decay))
            return fail(HPO_EINVAL, "group %d: lr and weight_decay must be finite", k);
    if (std::isnan(max_norm))
        return fail(HPO_EINVAL, "max_norm is NaN");
    return HPO_OK;
}

hpo_status check_step(hpo_set s, const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                      double max_norm)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    if (s->kind != HPO_SET_ADAM)
        return fail(HPO_EINVAL, "a Muon set takes hpo_muon_step / hpo_step_device_chain, not the AdamW step");
    return check_step_args(cfg, groups, n_groups, s->max_group, max_norm);
}

/* 1 - beta^t, formed in binary64 and rounded once to fp32. */
float bias_correction(double beta, int64_t t) { return static_cast<float>(1.0 - std::pow(beta, static_cast<double>(t))); }

/* Per-step scalars other than t: binary64 once, rounded to fp32 once. */
hpo::AdamScalars base_scalars(const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups, double max_norm)
{
    hpo::AdamScalars sc{};
    sc.b1 = static_cast<float>(cfg->beta1);
    sc.b2 = static_cast<float>(cfg->beta2);
    sc.c1 = static_cast<float>(1.0 - cfg->beta1);
    sc.c2 = static_cast<float>(1.0 - cfg->beta2);
    sc.eps = static_cast<float>(cfg->eps);
    sc.max_norm = max_norm;
    for (int32_t k = 0; k < n_groups; ++k) {
        sc.lr[k] = static_cast<float>(groups[k].lr);
        sc.wd[k] = static_cast<float>(groups[k].weight_decay);
    }
    return sc;
}

}  // namespace hpo_host

extern "C" {

hpo_status hpo_adamw_step(hpo_set s, const hpo_adam_cfg* cfg, const hpo_group* groups,
                          int32_t n_groups, int64_t t, float inv_scale, double max_norm,
                          const float* d_norm, const int32_t* d_found_inf, void* stream)
{
    hpo_status st = check_step(s, cfg, groups, n_groups, max_norm);
    if (st != HPO_OK)
        return st;
    if (t < 1)
        return fail(HPO_EINVAL, "t is the 1-based count of applied steps, must be >= 1 (got %lld)", (long long)t);
    if (!std::isfinite(inv_scale))
        return fail(HPO_EINVAL, "inv_scale must be finite");
    if (max_norm > 0.0 && !d_norm)
        return fail(HPO_EINVAL, "clipping (max_norm > 0) needs d_norm");
    hpo::AdamScalars sc = base_scalars(cfg, groups, n_groups, max_norm);
    sc.inv_scale = inv_scale;
    sc.bc1 = bias_correction(cfg->beta1, t);
    sc.bc2 = bias_correction(cfg->beta2, t);
    sc.d_norm = d_norm;
    sc.d_found = d_found_inf;
    hipError_t e = hpo::launch_adam(s->view, s->n_chunks, cfg->mode, sc, as_stream(stream));
    if (e != hipSuccess)
        return hip_fail(e, "launch adam update");
    return ok();
}

hpo_status hpo_scaler_state_init(hpo_scaler_state* d_state, float loss_scale, int32_t hysteresis,
                                 int64_t applied_steps, void* stream)
{
    if (!d_state || !aligned(d_state, 8))
        return fail(HPO_EINVAL, "d_state must be a non-NULL, 8-byte aligned device pointer");
    if (!(loss_scale > 0.0f) || !std::isfinite(loss_scale))
        return fail(HPO_EINVAL, "loss_scale must be finite and > 0 (got %g)", (double)loss_scale);
    if (hysteresis < 1 || applied_steps < 0)
        return fail(HPO_EINVAL, "hysteresis must be >= 1 and applied_steps >= 0");
    hipError_t e = hpo::launch_scaler_init(d_state, loss_scale, hysteresis, applied_steps, as_stream(stream));
    if (e != hipSuccess)
        return hip_fail(e, "launch scaler init");
    return ok();
}

}  // extern "C"

namespace hpo_host {

hpo_status check_scaler_args(const hpo_scaler_cfg* scfg, const hpo_scaler_state* d_state, int64_t t_first,
                             int32_t window)
{
    if (!scfg)
        return fail(HPO_EINVAL, "scfg is NULL");
    if (!d_state || !aligned(d_state, 8))
        return fail(HPO_EINVAL, "d_state must be a non-NULL, 8-byte aligned device pointer");
    if (t_first < 1)
        return fail(HPO_EINVAL, "t_first must be >= 1 (got %lld)", (long long)t_first);
    if (window < 1 || window > HPO_MAX_WINDOW)
        return fail(HPO_EINVAL, "window must be in [1, %d] (got %d)", HPO_MAX_WINDOW, window);
    if (std::isnan(scfg->grad_norm_skip_threshold))
        return fail(HPO_EINVAL, "grad_norm_skip_threshold is NaN");
    if (scfg->dynamic) {
        if (scfg->growth_interval < 1 || scfg->hysteresis < 1)
            return fail(HPO_EINVAL, "growth_interval and hysteresis must be >= 1");
        if (!(scfg->growth_factor > 0.0f) || !(scfg->backoff_factor > 0.0f) || !(scfg->min_scale > 0.0f) ||
            !std::isfinite(scfg->growth_factor) || !std::isfinite(scfg->backoff_factor) ||
            !std::isfinite(scfg->min_scale))
            return fail(HPO_EINVAL, "growth_factor, backoff_factor and min_scale must be finite and > 0");
    }
    return HPO_OK;
}

hpo::AdamScalars device_scalars(const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                                double max_norm, hpo_scaler_state* d_state, int64_t t_first, int32_t window)
{
    hpo::AdamScalars sc = base_scalars(cfg, groups, n_groups, max_norm);
    sc.d_state = d_state;
    sc.t_first = t_first;
    sc.window = window;
    for (int32_t j = 0; j < window; ++j) {
        sc.bc1_tab[j] = bias_correction(cfg->beta1, t_first + j);
        sc.bc2_tab[j] = bias_correction(cfg->beta2, t_first + j);
    }
    return sc;
}

hpo::FinalOut state_out(const hpo_scaler_cfg* scfg, hpo_scaler_state* d_state, int64_t t_first, int32_t window)
{
    hpo::FinalOut o{};
    o.st = d_state;
    o.threshold = scfg->grad_norm_skip_threshold;
    o.rule = rule_of(scfg);
    o.t_first = t_first;
    o.window = window;
    return o;
}

hpo::ScalerRule rule_of(const hpo_scaler_cfg* scfg)
{
    hpo::ScalerRule rule{};
    rule.dynamic = scfg->dynamic ? 1 : 0;
    rule.growth_interval = scfg->growth_interval;
    rule.hysteresis = scfg->hysteresis;
    rule.growth_factor = scfg->growth_factor;
    rule.backoff_factor = scfg->backoff_factor;
    rule.min_scale = scfg->min_scale;
    return rule;
}

}  // namespace hpo_host

extern "C" {

hpo_status hpo_step_device(hpo_set s, const hpo_adam_cfg* cfg, const hpo_group* groups, int32_t n_groups,
                           double max_norm, const hpo_scaler_cfg* scfg, hpo_scaler_state* d_state,
                           int64_t t_first, int32_t window, void* stream)
{
    hpo_status st = check_step(s, cfg, groups, n_groups, max_norm);
    if (st != HPO_OK)
        return st;
    st = check_scaler_args(scfg, d_state, t_first, window);
    if (st != HPO_OK)
        return st;
    const hpo::AdamScalars sc = device_scalars(cfg, groups, n_groups, max_norm, d_state, t_first, window);
    hipStream_t strm = as_stream(stream);
    const hpo::FinalOut out = state_out(scfg, d_state, t_first, window);
    hipError_t e = hpo::launch_grad_pass_final(s->view, s->n_chunks, s->grad_group, hpo::GradPass::kNorm, 1.0f,
                                               &d_state->inv_scale, s->parts, out, strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch norm pass and finalize");
    e = hpo::launch_adam(s->view, s->n_chunks, cfg->mode, sc, strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch adam update");
    return ok();
}

hpo_status hpo_stream_probe(hpo_set s, void* stream)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    const hpo::SetView& v = s->view;
    if (!v.is_flat || !v.flat.vec_ok || v.param_dtype == HPO_PARAM_FP32 || v.state_store != 0 || v.grad_bf16 ||
        v.master_fp16 || s->kind != HPO_SET_ADAM)
        return fail(HPO_EINVAL, "the probe takes flat sets with fp32 grads, master and moments, 16-bit params and "
                                "pointers on their vector lines");
    hipError_t e = hpo::launch_stream_probe(v, s->n_chunks, as_stream(stream));
    if (e != hipSuccess)
        return hip_fail(e, "launch stream probe");
    return ok();
}

hpo_status hpo_copy_main_to_model(hpo_set s, void* stream)
{
    hpo_status st = check_set(s);
    if (st != HPO_OK)
        return st;
    if (s->view.param_dtype == HPO_PARAM_FP32)
        return ok();
    hipError_t e = hpo::launch_copy_main_to_model(s->view, s->n_chunks, as_stream(stream));
    if (e != hipSuccess)
        return hip_fail(e, "launch master->model copy");
    return ok();
}

hpo_status hpo_grad_global_norm_sets(const hpo_set* sets, int32_t n_sets, float inv_scale, float* d_norm,
                                     int32_t* d_found_inf, int64_t* d_num_zeros, void* stream)
{
    if (!sets || n_sets < 1 || n_sets > hpo::kMaxFoldSets)
        return fail(HPO_EINVAL, "sets must be an array of 1..%d sets (got %d)", hpo::kMaxFoldSets, n_sets);
    if (!d_norm)
        return fail(HPO_EINVAL, "d_norm is NULL");
    if (!std::isfinite(inv_scale))
        return fail(HPO_EINVAL, "inv_scale must be finite");
    if (d_num_zeros && !aligned(d_num_zeros, 8))
        return fail(HPO_EINVAL, "d_num_zeros must be 8-byte aligned");
    hpo::Partials p[hpo::kMaxFoldSets];
    for (int32_t k = 0; k < n_sets; ++k) {
        hpo_status st = check_set(sets[k]);
        if (st != HPO_OK)
            return st;
        for (int32_t j = 0; j < k; ++j)
            if (sets[j] == sets[k])
                return fail(HPO_EINVAL, "set %d appears twice", k);
        p[k] = partials_of(sets[k]);
    }
    hipStream_t strm = as_stream(stream);
    for (int32_t k = 0; k < n_sets; ++k) {
        hpo_set s = sets[k];
        hipError_t e = hpo::launch_grad_pass(s->view, s->n_chunks, s->grad_group, hpo::GradPass::kNorm, inv_scale,
                                             nullptr, s->parts, strm);
        if (e != hipSuccess)
            return hip_fail(e, "launch norm pass");
    }
    hipError_t e = hpo::launch_finalize_sets(p, n_sets, d_norm, d_found_inf, d_num_zeros, strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch norm finalize");
    return ok();
}

hpo_status hpo_step_device_chain(hpo_set adam_set, const hpo_adam_cfg* cfg, const hpo_group* groups,
                                 int32_t n_groups, hpo_set muon_set, const hpo_muon_cfg* mcfg,
                                 const hpo_group* muon_groups, int32_t n_muon_groups, double max_norm,
                                 const hpo_scaler_cfg* scfg, hpo_scaler_state* d_state, int64_t t_first,
                                 int32_t window, void* stream)
{
    if (!adam_set && !muon_set)
        return fail(HPO_EINVAL, "the chain needs at least one set");
    hpo_status st = HPO_OK;
    if (adam_set) {
        st = check_step(adam_set, cfg, groups, n_groups, max_norm);
        if (st != HPO_OK)
            return st;
    }
    if (muon_set) {
        st = check_muon_step(muon_set, mcfg, muon_groups, n_muon_groups, max_norm);
        if (st != HPO_OK)
            return st;
    }
    if (adam_set && muon_set && adam_set->device != muon_set->device)
        return fail(HPO_EDEVICE, "the two sets live on different devices");
    st = check_scaler_args(scfg, d_state, t_first, window);
    if (st != HPO_OK)
        return st;
    hipStream_t strm = as_stream(stream);
    hpo::Partials p[2];
    int n_sets = 0;
    for (hpo_set s : {adam_set, muon_set}) {
        if (!s)
            continue;
        hipError_t e = hpo::launch_grad_pass(s->view, s->n_chunks, s->grad_group, hpo::GradPass::kNorm, 1.0f,
                                             &d_state->inv_scale, s->parts, strm);
        if (e != hipSuccess)
            return hip_fail(e, "launch norm pass");
        p[n_sets++] = partials_of(s);
    }
    hipError_t e = hpo::launch_finalize_state_sets(p, n_sets, state_out(scfg, d_state, t_first, window), strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch norm finalize");
    if (adam_set) {
        const hpo::AdamScalars sc = device_scalars(cfg, groups, n_groups, max_norm, d_state, t_first, window);
        e = hpo::launch_adam(adam_set->view, adam_set->n_chunks, cfg->mode, sc, strm);
        if (e != hipSuccess)
            return hip_fail(e, "launch adam update");
    }
    if (muon_set) {
        hpo::MuonGate gate{};
        gate.st = d_state;
        gate.t_first = t_first;
        gate.window = window;
        gate.dev = 1;
        st = muon_enqueue(muon_set, mcfg, muon_groups, n_muon_groups, gate, 1.0f, max_norm, nullptr, strm);
        if (st != HPO_OK)
            return st;
    }
    return ok();
}

}  // extern "C"
