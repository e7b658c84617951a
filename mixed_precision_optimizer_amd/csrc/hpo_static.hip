/*
 * hpo_static.hip -- the device-resident step of a flat shard with no set and
 * no allocation: hpo_step_device_flat_static (include/hpo.h).
 *
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  It runs the same
 * kernels as hpo_set_create_flat + hpo_step_device, but the grad pass's
 * reduction partials live in one file-scope device array, `scratch`, instead
 * of a set's allocation, and the flat descriptor travels by value in the
 * kernel arguments, so nothing is allocated, copied or freed per call.
 *
 * Each GPU the library runs on holds its own copy of `scratch` until the
 * process ends.  Host code never passes the array's name to a kernel (in host
 * code it is only a stand-in for the symbol): the first call on a device,
 * with that device current, asks the runtime for the array's device address
 * with hipGetSymbolAddress and keeps it per device; every launch then takes
 * that address.  Every call on one device shares that device's array and
 * leaves its partials there; each call writes every partial it reads before
 * reading it, so nothing needs clearing.  Calls that overlap on one device
 * (two streams, two threads) race on the array.
 */
#include <mutex>

#include <hip/hip_runtime.h>

#include "hpo_set.h"

namespace {

/* Grad-pass partials (binary64 sum, flag, zero count: 20 bytes each) for up
 * to HPO_STATIC_MAX_PARTS workgroups plus their second-stage entries. */
constexpr size_t kScratchBytes =
    static_cast<size_t>(HPO_STATIC_MAX_PARTS + hpo::stage_parts(HPO_STATIC_MAX_PARTS)) * hpo::kPartialBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static_assert(hpo::partial_entries(HPO_STATIC_MAX_PARTS) * hpo::kPartialBytes <= static_cast<int64_t>(kScratchBytes),
              "the largest plan's partials fit");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

/* Device address of `scratch` on the current device (looked up once per
 * device, with that device current). */
hpo_status scratch_on_device(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return hpo_host::fail(HPO_EDEVICE, "device ordinal %d is outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hpo_host::hip_fail(e, "hipGetSymbolAddress of the static scratch array");
        if (ptr == nullptr)
            return hpo_host::fail(HPO_EHIP, "hipGetSymbolAddress returned NULL for the static scratch array");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return HPO_OK;
}

}  // namespace

using namespace hpo_host;

extern "C" hpo_status hpo_step_device_flat_static(int64_t numel, int32_t param_dtype, void* param, float* main_param,
                                                  float* main_grad, void* exp_avg, void* exp_avg_sq,
                                                  const hpo_adam_cfg* cfg, const hpo_group* group, double max_norm,
                                                  const hpo_scaler_cfg* scfg, hpo_scaler_state* d_state,
                                                  int64_t t_first, int32_t window, void* stream)
{
    /* every argument is checked on the host before the device is touched */
    Layout lay{};
    hpo_status st = decode_dtype(param_dtype, lay);
    if (st != HPO_OK)
        return st;
    if (numel < 0)
        return fail(HPO_EINVAL, "numel = %lld is negative", (long long)numel);
    st = check_tensor(0, lay, param, main_param, main_grad, exp_avg, exp_avg_sq, numel);
    if (st != HPO_OK)
        return st;
    st = check_step_args(cfg, group, 1, 0, max_norm);
    if (st != HPO_OK)
        return st;
    st = check_scaler_args(scfg, d_state, t_first, window);
    if (st != HPO_OK)
        return st;
    /* the flat set's plan (hpo_set_create_flat) */
    const int32_t ch = choose_chunk(&numel, 1);
    const int64_t n_chunks = count_chunks(&numel, 1, ch);
    const int32_t gg = grad_group_of(ch, n_chunks);
    const int64_t n_parts = parts_of(n_chunks, gg);
    if (n_parts > HPO_STATIC_MAX_PARTS || n_chunks > 0x7FFFFFFFLL)
        return fail(HPO_EINVAL,
                    "numel %lld needs %lld grad-pass partials; the static scratch holds at most %d "
                    "(about %lld elements)",
                    (long long)numel, (long long)n_parts, HPO_STATIC_MAX_PARTS,
                    (long long)HPO_STATIC_MAX_PARTS * hpo::kGradSpan);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    void* base = nullptr;
    st = scratch_on_device(dev, &base);
    if (st != HPO_OK)
        return st;

    hpo::SetView sv{};
    /* a range off the vector lines steps element by element (a set would peel
     * its head into a table piece; here there is no table) */
    sv.flat = make_desc(lay, param, main_param, main_grad, exp_avg, exp_avg_sq, numel, 0);
    sv.chunk_elems = ch;
    sv.is_flat = 1;
    sv.param_dtype = lay.pdt;
    sv.state_store = lay.state_store();
    sv.grad_bf16 = static_cast<int16_t>(lay.grad_bf16);
    sv.master_fp16 = static_cast<int16_t>(lay.master_fp16);
    sv.cached = lay.cached(numel);
    const hpo::Partials parts = hpo::carve_partials(base, n_parts);

    const hpo::AdamScalars sc = device_scalars(cfg, group, 1, max_norm, d_state, t_first, window);
    hipStream_t strm = as_stream(stream);
    e = hpo::launch_grad_pass_final(sv, n_chunks, gg, hpo::GradPass::kNorm, 1.0f, &d_state->inv_scale, parts,
                                    state_out(scfg, d_state, t_first, window), strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch norm pass and finalize");
    e = hpo::launch_adam(sv, n_chunks, cfg->mode, sc, strm);
    if (e != hipSuccess)
        return hip_fail(e, "launch adam update");
    return ok();
}
