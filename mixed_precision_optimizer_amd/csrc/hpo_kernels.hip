/*
 * hpo_kernels.hip -- gfx950 kernels of the mixed-precision AdamW step.
 *
 * Sources (web pages):
 *   [OPT-INFRA]  "02 · Optimizer：算法与 infra" (llm-infra-atlas, train/02_optimizer)
 *   [FP32-RFC]   "支持FP32优化器" (hyper-parallel issue)
 *
 * The whole path is elementwise plus one global sum, so it is bound by HBM
 * bandwidth, not by the matrix cores: no MFMA here.  The update walks the
 * set's chunk table with one 256-lane workgroup (4 wavefronts of 64) per
 * chunk of 4096..16384 contiguous elements of one tensor; the read-only grad
 * pass runs 1024-lane workgroups over groups of consecutive chunks (~64K
 * elements each), so it leaves few reduction partials.  On tensors whose
 * pointers are 16-byte aligned each lane moves 16 bytes per fp32 array per
 * access (global_load_dwordx4), a wavefront 1 KB contiguous, and the bf16
 * write-back is 8 bytes per lane (512 B per wavefront), so every access
 * covers whole cache lines.  Chunk tails and unaligned tensors take an
 * element-at-a-time path.
 *
 * Passes:
 *   grad pass   one read of the stored grads: non-finite flag and binary64
 *               sum of squares of the unscaled grads per workgroup
 *               (wavefront shuffles, then LDS across the 4 wavefronts);
 *               or the pages' in-place unscale.             4 or 8 B/elem
 *   finalize    one workgroup: fixed-order sum of the partials, sqrt, flag.
 *   adam        clip + Adam/AdamW + bf16 RNE write-back in registers:
 *               read grad, master, m, v (16 B), write master, m, v (12 B)
 *               and the bf16 param (2 B).                  30 B/elem
 *   copy        master -> bf16 param alone.                 6 B/elem
 *
 * Floating point: the library is built with -ffp-contract=off, so every
 * multiply and add below rounds on its own, in the order written; fp32
 * division and sqrtf are HIP's correctly rounded ones and fp32 denormals are
 * kept.  This reproduces, operation for operation, the formulas of
 * [OPT-INFRA] §2 (moments, bias correction, eps outside the root) and §3
 * (decoupled decay or the L2 term), with the clip of §11.1 in front.
 */
#include <hip/hip_runtime.h>

#include "hpo_impl.h"
#include "hpo_device.h"

/* Tuning knobs (compile time), defaults chosen by measurement on MI355X at
 * 8.75e9 elements.  UNROLL: 16-byte vectors per lane per array in flight in
 * one loop trip.  NT: streaming (nontemporal) loads / stores for data that is
 * touched exactly once per pass -- worth about +5% on the update and +12% on
 * the read-only grad pass, since nothing here is ever re-read from cache. */
#ifndef HPO_ADAM_UNROLL
#define HPO_ADAM_UNROLL 2
#endif
#ifndef HPO_GRAD_UNROLL
#define HPO_GRAD_UNROLL 1
#endif
#ifndef HPO_NT_LOADS
#define HPO_NT_LOADS 1
#endif
#ifndef HPO_NT_STORES
#define HPO_NT_STORES 1
#endif
/* XCD_REMAP: workgroups are handed to the 8 XCDs round-robin by index; with
 * the remap, XCD x works through one contiguous eighth of the chunks.
 * ADAM_MIN_BLOCKS: second __launch_bounds__ argument of the update (0: none). */
#ifndef HPO_XCD_REMAP
#define HPO_XCD_REMAP 0
#endif
#ifndef HPO_ADAM_MIN_BLOCKS
#define HPO_ADAM_MIN_BLOCKS 0
#endif

namespace hpo {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

/* 16-, 8- and 16-byte accesses, nontemporal (streaming) when NT: data that
 * is touched once per pass goes around the caches.  Sets small enough to sit
 * in the on-die cache from one step to the next take cached accesses in the
 * update instead (SetView::cached). */
template <bool NT = HPO_NT_LOADS>
__device__ __forceinline__ float4 ld_stream(const float4* p)
{
    if constexpr (NT) {
        const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <bool NT = HPO_NT_LOADS>
__device__ __forceinline__ uint2 ld_stream(const uint2* p)
{
    if constexpr (NT) {
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        return make_uint2(v.x, v.y);
    } else {
        return *p;
    }
}

template <bool NT = HPO_NT_LOADS>
__device__ __forceinline__ uint4 ld_stream(const uint4* p)
{
    if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <bool NT = HPO_NT_STORES>
__device__ __forceinline__ void st_stream(uint4* p, uint4 v)
{
    if constexpr (NT) {
        u32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    } else {
        *p = v;
    }
}

template <bool NT = HPO_NT_STORES>
__device__ __forceinline__ void st_stream(float4* p, float4 v)
{
    if constexpr (NT) {
        f32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t*>(p));
    } else {
        *p = v;
    }
}

template <bool NT = HPO_NT_STORES>
__device__ __forceinline__ void st_stream(uint2* p, uint2 v)
{
    if constexpr (NT) {
        u32x2_t w = {v.x, v.y};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
    } else {
        *p = v;
    }
}

/* Chunk handled by this workgroup of an n-workgroup update launch. */
__device__ __forceinline__ int64_t update_chunk(int64_t n)
{
#if HPO_XCD_REMAP
    constexpr int64_t kXcd = 8;
    const int64_t b = blockIdx.x;
    const int64_t x = b % kXcd, k = b / kXcd;
    const int64_t q = n / kXcd, r = n % kXcd;
    const int64_t first = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    return first + k;
#else
    (void)n;
    return blockIdx.x;
#endif
}

struct Range {
    TensorDesc d;
    int64_t start;
    int64_t len;
};

template <bool FLAT>
__device__ __forceinline__ Range chunk_range(const SetView& sv, int64_t chunk)
{
    Range r;
    if constexpr (FLAT) {
        r.d = sv.flat;
        r.start = chunk * sv.chunk_elems;
        const int64_t rem = r.d.numel - r.start;
        r.len = rem < sv.chunk_elems ? rem : sv.chunk_elems;
    } else {
        const Chunk c = sv.chunks[chunk];
        r.d = sv.tensors[c.tensor];
        r.start = c.start;
        r.len = c.len;
    }
    return r;
}

/* fp32 -> fp16 bits for fp16 model params ([OPT-INFRA] §9.2 write-back):
 * the hardware conversion, which rounds to nearest even under the default
 * mode and keeps fp16 subnormals. */
__device__ __forceinline__ uint32_t fp16_rne_bits(float x)
{
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

/* 16-bit model param bits of a master value, by param dtype. */
template <int PDT>
__device__ __forceinline__ uint32_t param_bits(float x)
{
    if constexpr (PDT == HPO_PARAM_FP16)
        return fp16_rne_bits(x);
    else
        return bf16_rne_bits(x);
}

template <int PDT>
__device__ __forceinline__ uint2 pack_param4(float4 t)
{
    return make_uint2(param_bits<PDT>(t.x) | (param_bits<PDT>(t.y) << 16),
                      param_bits<PDT>(t.z) | (param_bits<PDT>(t.w) << 16));
}

/* Storage of the moments, main grads and master ([OPT-INFRA] §16: the
 * precision-aware optimizer may keep each below fp32): fp32, or a 16-bit
 * format widened exactly on load and rounded to nearest even on store.  The
 * arithmetic is fp32 either way. */
enum Store : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

template <int S>
constexpr int64_t store_bytes() { return S == kF32 ? 4 : 2; }

template <int S>
__device__ __forceinline__ float widen16(uint32_t b)
{
    if constexpr (S == kF16)
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
    else
        return bf16_to_f32(b);
}

template <int S>
__device__ __forceinline__ uint32_t narrow16(float x)
{
    if constexpr (S == kF16)
        return fp16_rne_bits(x);
    else
        return bf16_rne_bits(x);
}

/* The value a store of x keeps (x itself for fp32). */
template <int S>
__device__ __forceinline__ float stored(float x)
{
    if constexpr (S == kF32)
        return x;
    else
        return widen16<S>(narrow16<S>(x));
}

/* 4 consecutive elements at 4-element index i of base. */
template <int S, bool NT = HPO_NT_LOADS>
__device__ __forceinline__ float4 ld4(const void* base, int64_t i)
{
    if constexpr (S == kF32) {
        return ld_stream<NT>(static_cast<const float4*>(base) + i);
    } else {
        const uint2 w = ld_stream<NT>(static_cast<const uint2*>(base) + i);
        return make_float4(widen16<S>(w.x & 0xFFFFu), widen16<S>(w.x >> 16), widen16<S>(w.y & 0xFFFFu),
                           widen16<S>(w.y >> 16));
    }
}

template <int S, bool NT = HPO_NT_STORES>
__device__ __forceinline__ void st4(void* base, int64_t i, float4 x)
{
    if constexpr (S == kF32)
        st_stream<NT>(static_cast<float4*>(base) + i, x);
    else
        st_stream<NT>(static_cast<uint2*>(base) + i, make_uint2(narrow16<S>(x.x) | (narrow16<S>(x.y) << 16),
                                                            narrow16<S>(x.z) | (narrow16<S>(x.w) << 16)));
}

/* Element e of base. */
template <int S>
__device__ __forceinline__ float ld1(const void* base, int64_t e)
{
    if constexpr (S == kF32)
        return static_cast<const float*>(base)[e];
    else
        return widen16<S>(static_cast<const uint16_t*>(base)[e]);
}

template <int S>
__device__ __forceinline__ void st1(void* base, int64_t e, float x)
{
    if constexpr (S == kF32)
        static_cast<float*>(base)[e] = x;
    else
        static_cast<uint16_t*>(base)[e] = static_cast<uint16_t>(narrow16<S>(x));
}

/* 8 consecutive 16-bit elements at 8-element index i: one 16-byte access. */
template <int S>
__device__ __forceinline__ void ld8(const void* base, int64_t i, float (&x)[8])
{
    const uint4 w = ld_stream(static_cast<const uint4*>(base) + i);
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = widen16<S>(q[j] & 0xFFFFu);
        x[2 * j + 1] = widen16<S>(q[j] >> 16);
    }
}

template <int S>
__device__ __forceinline__ void st8(void* base, int64_t i, const float (&x)[8])
{
    uint32_t q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        q[j] = narrow16<S>(x[2 * j]) | (narrow16<S>(x[2 * j + 1]) << 16);
    st_stream(static_cast<uint4*>(base) + i, make_uint4(q[0], q[1], q[2], q[3]));
}

/* Element `start` of an array of S elements. */
template <int S>
__device__ __forceinline__ void* at(void* base, int64_t start)
{
    return static_cast<char*>(base) + start * store_bytes<S>();
}

/* ---------------------------------------------------------------------- */
/* grad pass: non-finite flag + sum of squares, or in-place unscale        */
/* ---------------------------------------------------------------------- */
/* The norm pass also counts the unscaled grads that are zero (either sign):
 * the step's num_zeros ([OPT-INFRA] §10.2 return value, §17
 * log_num_zeros_in_grad), taken on the same values as the norm. */
template <GradPass PASS>
__device__ __forceinline__ void grad_elem(float& G, float inv, double& acc, int& bad, int& zeros)
{
    bad |= !__builtin_isfinite(G);
    if constexpr (PASS == GradPass::kNorm) {
        const float g = G * inv;
        zeros += g == 0.0f ? 1 : 0;
        const double gd = static_cast<double>(g);
        acc = __builtin_fma(gd, gd, acc); /* gd*gd is exact in binary64, so this is one rounding of acc + g^2 */
    } else if constexpr (PASS == GradPass::kUnscale) {
        G = G * inv;
    }
}

/* The body of a 16-bit grad range whose start is 16-byte aligned: 8
 * elements per lane access, so that each access moves as many bytes as an
 * fp32 one.  Returns the elements it covered. */
template <GradPass PASS, int GDT>
__device__ __forceinline__ int64_t grad_body16(void* __restrict__ G, int64_t len, float inv, double& acc, int& bad,
                                               int& zeros)
{
    constexpr int U = HPO_GRAD_UNROLL;
    const int tid = threadIdx.x;
    const int64_t nv = len / 8;
    for (int64_t base = tid; base < nv; base += kGradBlock * U) {
        float x[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kGradBlock;
            if (i < nv)
                ld8<GDT>(G, i, x[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kGradBlock;
            if (i < nv) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    grad_elem<PASS>(x[u][j], inv, acc, bad, zeros);
                if constexpr (PASS == GradPass::kUnscale)
                    st8<GDT>(G, i, x[u]);
            }
        }
    }
    return nv * 8;
}

template <GradPass PASS, int GDT>
__device__ __forceinline__ void grad_range(const Range& r, float inv, double& acc, int& bad, int& zeros)
{
    void* __restrict__ G = at<GDT>(r.d.grad, r.start);
    const int tid = threadIdx.x;
    int64_t done = 0;
    if (GDT != kF32 && r.d.vec_ok && reinterpret_cast<uintptr_t>(G) % 16 == 0) {
        done = grad_body16<PASS, GDT>(G, r.len, inv, acc, bad, zeros);
    } else if (r.d.vec_ok) {
        constexpr int U = HPO_GRAD_UNROLL;
        const int64_t nv = r.len / kVec;
        for (int64_t base = tid; base < nv; base += kGradBlock * U) {
            float4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + static_cast<int64_t>(u) * kGradBlock;
                if (i < nv)
                    x[u] = ld4<GDT>(G, i);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + static_cast<int64_t>(u) * kGradBlock;
                if (i < nv) {
                    grad_elem<PASS>(x[u].x, inv, acc, bad, zeros);
                    grad_elem<PASS>(x[u].y, inv, acc, bad, zeros);
                    grad_elem<PASS>(x[u].z, inv, acc, bad, zeros);
                    grad_elem<PASS>(x[u].w, inv, acc, bad, zeros);
                    if constexpr (PASS == GradPass::kUnscale)
                        st4<GDT>(G, i, x[u]);
                }
            }
        }
        done = nv * kVec;
    }
    for (int64_t i = done + tid; i < r.len; i += kGradBlock) {
        float x = ld1<GDT>(G, i);
        grad_elem<PASS>(x, inv, acc, bad, zeros);
        if constexpr (PASS == GradPass::kUnscale)
            st1<GDT>(G, i, x);
    }
}

/* ---------------------------------------------------------------------- */
/* finalize: one workgroup, fixed-order sum of the per-chunk partials       */
/* ---------------------------------------------------------------------- */
/* Sum of partials [lo, hi) by one workgroup: each lane keeps kAcc
 * independent accumulators so that kAcc loads are in flight at once; partial
 * i always lands in the same accumulator and the accumulators and lanes are
 * combined in a fixed tree, so the result is reproducible.  Valid in lane 0. */
/* The zero counts are integers, so their order does not matter.
 * want_sum == false: flags only (the check pass leaves no sums or counts). */
__device__ __forceinline__ double reduce_partials(const double* part_sum, const int32_t* part_flag,
                                                  const int64_t* part_zeros, int64_t lo, int64_t hi,
                                                  bool want_sum, int& any_bad, int64_t& zeros)
{
    constexpr int kAcc = 8;
    double acc[kAcc];
#pragma unroll
    for (int k = 0; k < kAcc; ++k)
        acc[k] = 0.0;
    int bad = 0;
    int64_t nz = 0;
    for (int64_t base = lo + threadIdx.x; base < hi; base += static_cast<int64_t>(kFinalBlock) * kAcc) {
#pragma unroll
        for (int k = 0; k < kAcc; ++k) {
            const int64_t i = base + static_cast<int64_t>(k) * kFinalBlock;
            if (i < hi) {
                if (want_sum) {
                    acc[k] += part_sum[i];
                    nz += part_zeros[i];
                }
                bad |= part_flag[i];
            }
        }
    }
    const double mine = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    any_bad = __syncthreads_or(bad);
    const double tot = block_sum<kFinalBlock>(mine);
    zeros = block_sum<kFinalBlock, int64_t>(nz);
    return tot;
}

/* First of two reduction stages for large sets: workgroup b folds partials
 * [b * kFinalSpan, (b + 1) * kFinalSpan) into one. */
__global__ __launch_bounds__(kFinalBlock) void k_reduce_stage(Partials in, int32_t want_sum)
{
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kFinalSpan;
    const int64_t hi = lo + kFinalSpan < in.n ? lo + kFinalSpan : in.n;
    int any_bad = 0;
    int64_t zeros = 0;
    const double tot = reduce_partials(in.sum, in.flag, in.zeros, lo, hi, want_sum != 0, any_bad, zeros);
    if (threadIdx.x == 0) {
        if (want_sum) {
            in.stage_sum[blockIdx.x] = tot;
            in.stage_zeros[blockIdx.x] = zeros;
        }
        in.stage_flag[blockIdx.x] = any_bad ? 1 : 0;
    }
}

/* The last-stage inputs of up to kMaxFoldSets sets, folded in order. */
struct Fold {
    const double* sum[kMaxFoldSets];
    const int32_t* flag[kMaxFoldSets];
    const int64_t* zeros[kMaxFoldSets];
    int64_t n[kMaxFoldSets];
    int32_t count;
};

__device__ __forceinline__ double fold_sets(const Fold& f, bool want_sum, int& any_bad, int64_t& zeros)
{
    double tot = 0.0;
    any_bad = 0;
    zeros = 0;
    for (int k = 0; k < f.count; ++k) {
        int bad = 0;
        int64_t nz = 0;
        const double s = reduce_partials(f.sum[k], f.flag[k], f.zeros[k], 0, f.n[k], want_sum, bad, nz);
        tot = k == 0 ? s : tot + s;
        any_bad |= bad;
        zeros += nz;
    }
    return tot;
}

/* Host-driven outputs of a finalize (thread 0): the norm and the zero count
 * when the sums were folded, found_inf or-ed in. */
__device__ __forceinline__ void write_norm_outputs(const FinalOut& o, double tot, int any_bad, int64_t zeros)
{
    if (o.d_norm != nullptr) {
        *o.d_norm = static_cast<float>(sqrt(tot));
        if (o.d_zeros != nullptr)
            *o.d_zeros = zeros;
    }
    if (o.d_found != nullptr && any_bad)
        *o.d_found = 1;
}

/* The end of a device-resident step (thread 0), once the partials are
 * folded: the norm, the zero count and found_inf; the step is applied when
 * the grads are finite, the norm is not above the skip threshold and its t
 * (applied_steps + 1) lies in the window of bias corrections it was given
 * (a t outside sets the sticky error instead); then the counters and the
 * loss-scale rule of [OPT-INFRA] §10.1.  step_inv_scale keeps the scale this
 * step's grads were unscaled with, for the update that follows; inv_scale
 * becomes the next step's. */
__device__ __forceinline__ void write_step_state(const FinalOut& o, double tot, int any_bad, int64_t zeros)
{
    hpo_scaler_state s = *o.st;
    const float norm = static_cast<float>(sqrt(tot));
    s.grad_norm = norm;
    s.num_zeros = zeros;
    s.found_inf = any_bad ? 1 : 0;
    s.step_inv_scale = s.inv_scale;
    /* the threshold test fails for a NaN norm, so "not above" is spelled out */
    const bool ok = !any_bad && !(static_cast<double>(norm) > o.threshold);
    const int64_t j = s.applied_steps + 1 - o.t_first;
    const bool in_window = j >= 0 && j < o.window;
    if (ok && !in_window)
        s.error = 1;
    s.applied = (ok && in_window) ? 1 : 0;
    if (s.applied)
        s.applied_steps += 1;
    else
        s.skipped_steps += 1;
    const ScalerRule& rule = o.rule;
    if (rule.dynamic) {
        if (s.found_inf) {
            s.growth_tracker = 0;
            s.hysteresis_tracker -= 1;
            if (s.hysteresis_tracker <= 0) {
                const float backed = s.loss_scale * rule.backoff_factor;
                s.loss_scale = backed > rule.min_scale ? backed : rule.min_scale;
            }
        } else {
            s.growth_tracker += 1;
            if (s.growth_tracker == rule.growth_interval) {
                s.growth_tracker = 0;
                s.hysteresis_tracker = rule.hysteresis;
                s.loss_scale = s.loss_scale * rule.growth_factor;
            }
        }
        s.inv_scale = static_cast<float>(1.0 / static_cast<double>(s.loss_scale));
    }
    *o.st = s;
}

/* Last stage: one workgroup over all remaining partials, then the outputs.
 * d_norm == nullptr: flag only (the sums are not read). */
__global__ __launch_bounds__(kFinalBlock) void k_finalize(Fold f, FinalOut o)
{
    int any_bad = 0;
    int64_t zeros = 0;
    const double tot = fold_sets(f, o.d_norm != nullptr, any_bad, zeros);
    if (threadIdx.x == 0)
        write_norm_outputs(o, tot, any_bad, zeros);
}

/* Last stage of the device-resident step. */
__global__ __launch_bounds__(kFinalBlock) void k_finalize_state(Fold f, FinalOut o)
{
    int any_bad = 0;
    int64_t zeros = 0;
    const double tot = fold_sets(f, true, any_bad, zeros);
    if (threadIdx.x == 0)
        write_step_state(o, tot, any_bad, zeros);
}

/* One workgroup per group of consecutive chunks; one partial per workgroup:
 * the flag, and for the norm pass the binary64 sum and the zero count. */
template <bool FLAT, GradPass PASS, int GDT>
__global__ __launch_bounds__(kGradBlock) void k_grad_pass(SetView sv, int64_t n_chunks, int32_t group,
                                                          float inv_arg, const float* d_inv, Partials p)
{
    const float inv = d_inv != nullptr ? *d_inv : inv_arg;
    double acc = 0.0;
    int bad = 0;
    int zeros = 0;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * group;
    const int64_t c1 = c0 + group < n_chunks ? c0 + group : n_chunks;
    for (int64_t c = c0; c < c1; ++c)
        grad_range<PASS, GDT>(chunk_range<FLAT>(sv, c), inv, acc, bad, zeros);
    const int any_bad = __syncthreads_or(bad);
    if constexpr (PASS == GradPass::kNorm) {
        const double tot = block_sum<kGradBlock>(acc);
        const int nz = block_sum<kGradBlock, int>(zeros);
        if (threadIdx.x == 0) {
            p.sum[blockIdx.x] = tot;
            p.zeros[blockIdx.x] = nz;
        }
    }
    if (threadIdx.x == 0)
        p.flag[blockIdx.x] = any_bad ? 1 : 0;
}

/* ---------------------------------------------------------------------- */
/* adam: clip + Adam/AdamW + bf16 write-back                              */
/* ---------------------------------------------------------------------- */
/* Per-step values that differ between the host-driven and the device-resident
 * step; everything else comes straight from the (read-only) kernel arguments. */
struct StepVals {
    float inv_scale;
    float bc1, bc2;  /* 1 - beta1^t, 1 - beta2^t */
    float C;         /* clip coefficient when clip is set */
    bool clip;
};

template <int MODE>
__device__ __forceinline__ void adam_elem(float G, float& th, float& m, float& v,
                                          const AdamScalars& sc, const StepVals& k, float lr, float wd)
{
    float g = G * k.inv_scale;           /* unscale ([OPT-INFRA] §10.2) */
    if (k.clip)
        g = g * k.C;                     /* clip ([OPT-INFRA] §11.1) */
    if constexpr (MODE == HPO_ADAM_L2)
        g = g + wd * th;                 /* L2 term joins the gradient ([OPT-INFRA] §3) */
    m = sc.b1 * m + sc.c1 * g;           /* first moment ([OPT-INFRA] §2) */
    v = sc.b2 * v + sc.c2 * (g * g);     /* raw second moment */
    const float mh = m / k.bc1;          /* bias corrections */
    const float vh = v / k.bc2;
    const float u = mh / (sqrtf(vh) + sc.eps); /* eps outside the root */
    if constexpr (MODE == HPO_ADAMW)
        th = th - lr * (u + wd * th);    /* decoupled decay ([OPT-INFRA] §3) */
    else
        th = th - lr * u;
}

#if HPO_ADAM_MIN_BLOCKS
#define HPO_ADAM_BOUNDS __launch_bounds__(kBlock, HPO_ADAM_MIN_BLOCKS)
#else
#define HPO_ADAM_BOUNDS __launch_bounds__(kBlock)
#endif

/* SDT, GDT, MST: storage (Store) of the moments, the main grads and the
 * master.  The param written back is the 16-bit rounding of the master as
 * stored, so an fp16 master and its bf16 param agree with a later copy. */
template <bool FLAT, int PDT, int MODE, bool DEV, int SDT, int GDT, int MST, bool NT>
__global__ HPO_ADAM_BOUNDS void k_adam(SetView sv, AdamScalars sc, int64_t n_chunks)
{
    StepVals k;
    float norm = 0.0f;
    if constexpr (DEV) {
        /* device-resident step: t, inv_scale, norm and the decision come
         * from the state; the bias corrections from the host's table */
        const hpo_scaler_state* st = sc.d_state;
        if (!st->applied)
            return;
        /* the finalize has counted this step: t = applied_steps, in the window */
        const int64_t j = st->applied_steps - sc.t_first;
        if (j < 0 || j >= sc.window)
            return;
        k.bc1 = sc.bc1_tab[j];
        k.bc2 = sc.bc2_tab[j];
        k.inv_scale = st->step_inv_scale;
        norm = st->grad_norm;
    } else {
        if (sc.d_found != nullptr && *sc.d_found != 0)
            return; /* found_inf: the whole step is skipped ([OPT-INFRA] §10.2) */
        k.bc1 = sc.bc1;
        k.bc2 = sc.bc2;
        k.inv_scale = sc.inv_scale;
        if (sc.max_norm > 0.0)
            norm = *sc.d_norm;
    }
    k.clip = false;
    k.C = 1.0f;
    if (sc.max_norm > 0.0) {
        const double c = sc.max_norm / (static_cast<double>(norm) + 1e-6);
        if (c < 1.0) {
            k.clip = true;
            k.C = static_cast<float>(c);
        }
    }
    const Range r = chunk_range<FLAT>(sv, update_chunk(n_chunks));
    const float lr = sc.lr[r.d.group];
    const float wd = sc.wd[r.d.group];
    const void* __restrict__ G = at<GDT>(r.d.grad, r.start);
    void* __restrict__ T = at<MST>(r.d.master, r.start);
    void* __restrict__ M = at<SDT>(r.d.exp_avg, r.start);
    void* __restrict__ V = at<SDT>(r.d.exp_avg_sq, r.start);
    uint16_t* __restrict__ P = static_cast<uint16_t*>(r.d.param) + r.start;
    const int tid = threadIdx.x;
    int64_t done = 0;
    if (r.d.vec_ok) {
        const int64_t nv = r.len / kVec;
        uint2* __restrict__ P4 = reinterpret_cast<uint2*>(P);
        constexpr int U = HPO_ADAM_UNROLL;
        for (int64_t base = tid; base < nv; base += kBlock * U) {
            float4 g[U], th[U], m[U], v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + static_cast<int64_t>(u) * kBlock;
                if (i < nv) {
                    g[u] = ld4<GDT, NT>(G, i);
                    th[u] = ld4<MST, NT>(T, i);
                    m[u] = ld4<SDT, NT>(M, i);
                    v[u] = ld4<SDT, NT>(V, i);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + static_cast<int64_t>(u) * kBlock;
                if (i < nv) {
                    adam_elem<MODE>(g[u].x, th[u].x, m[u].x, v[u].x, sc, k, lr, wd);
                    adam_elem<MODE>(g[u].y, th[u].y, m[u].y, v[u].y, sc, k, lr, wd);
                    adam_elem<MODE>(g[u].z, th[u].z, m[u].z, v[u].z, sc, k, lr, wd);
                    adam_elem<MODE>(g[u].w, th[u].w, m[u].w, v[u].w, sc, k, lr, wd);
                    th[u] = make_float4(stored<MST>(th[u].x), stored<MST>(th[u].y), stored<MST>(th[u].z),
                                        stored<MST>(th[u].w));
                    st4<MST, NT>(T, i, th[u]);
                    st4<SDT, NT>(M, i, m[u]);
                    st4<SDT, NT>(V, i, v[u]);
                    if constexpr (PDT != HPO_PARAM_FP32)
                        st_stream<NT>(P4 + i, pack_param4<PDT>(th[u]));
                }
            }
        }
        done = nv * kVec;
    }
    for (int64_t i = done + tid; i < r.len; i += kBlock) {
        float th = ld1<MST>(T, i), m = ld1<SDT>(M, i), v = ld1<SDT>(V, i);
        adam_elem<MODE>(ld1<GDT>(G, i), th, m, v, sc, k, lr, wd);
        th = stored<MST>(th);
        st1<MST>(T, i, th);
        st1<SDT>(M, i, m);
        st1<SDT>(V, i, v);
        if constexpr (PDT != HPO_PARAM_FP32)
            P[i] = static_cast<uint16_t>(param_bits<PDT>(th));
    }
}

/* ---------------------------------------------------------------------- */
/* bandwidth probe (measurement only)                                     */
/* ---------------------------------------------------------------------- */
/* The update's access pattern on an fp32 flat shard with a 16-bit param --
 * the same chunks, workgroups, unroll and streaming accesses -- with none of
 * its arithmetic: grad, master, exp_avg, exp_avg_sq read, the three state
 * arrays written back as read and the param written as the RNE of the
 * master.  The state is left as it was (param == bf16 / fp16 of the master
 * holds after every step), so this times the practical ceiling of the
 * update's 16-byte-read / 14-byte-write mix on the very buffers it steps.
 * The empty asm statements keep the grad loads and the stores from being
 * optimized away. */
template <int PDT>
__global__ HPO_ADAM_BOUNDS void k_stream_probe(SetView sv, int64_t n_chunks)
{
    const Range r = chunk_range<true>(sv, update_chunk(n_chunks));
    const float4* __restrict__ G = reinterpret_cast<const float4*>(r.d.grad + r.start);
    float4* __restrict__ T = reinterpret_cast<float4*>(r.d.master + r.start);
    float4* __restrict__ M = static_cast<float4*>(r.d.exp_avg) + r.start / kVec;
    float4* __restrict__ V = static_cast<float4*>(r.d.exp_avg_sq) + r.start / kVec;
    uint2* __restrict__ P = reinterpret_cast<uint2*>(static_cast<uint16_t*>(r.d.param) + r.start);
    const int64_t nv = r.len / kVec;  /* flat chunks start on vector lines; the tail is not probed */
    constexpr int U = HPO_ADAM_UNROLL;
    for (int64_t base = threadIdx.x; base < nv; base += kBlock * U) {
        float4 g[U], th[U], m[U], v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kBlock;
            if (i < nv) {
                g[u] = ld_stream(G + i);
                th[u] = ld_stream(T + i);
                m[u] = ld_stream(M + i);
                v[u] = ld_stream(V + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kBlock;
            if (i < nv) {
                asm volatile("" : "+v"(g[u].x), "+v"(g[u].y), "+v"(g[u].z), "+v"(g[u].w));
                asm volatile("" : "+v"(th[u].x), "+v"(th[u].y), "+v"(th[u].z), "+v"(th[u].w));
                asm volatile("" : "+v"(m[u].x), "+v"(m[u].y), "+v"(m[u].z), "+v"(m[u].w));
                asm volatile("" : "+v"(v[u].x), "+v"(v[u].y), "+v"(v[u].z), "+v"(v[u].w));
                st_stream(T + i, th[u]);
                st_stream(M + i, m[u]);
                st_stream(V + i, v[u]);
                st_stream(P + i, pack_param4<PDT>(th[u]));
            }
        }
    }
}

/* ---------------------------------------------------------------------- */
/* master -> model copy                                                   */
/* ---------------------------------------------------------------------- */
template <bool FLAT, int PDT, int MST>
__global__ __launch_bounds__(kBlock) void k_copy_main_to_model(SetView sv)
{
    const Range r = chunk_range<FLAT>(sv, blockIdx.x);
    const void* __restrict__ T = at<MST>(r.d.master, r.start);
    uint16_t* __restrict__ P = static_cast<uint16_t*>(r.d.param) + r.start;
    const int tid = threadIdx.x;
    int64_t done = 0;
    if (r.d.vec_ok) {
        const int64_t nv = r.len / kVec;
        uint2* __restrict__ P4 = reinterpret_cast<uint2*>(P);
        for (int64_t i = tid; i < nv; i += kBlock)
            P4[i] = pack_param4<PDT>(ld4<MST>(T, i));
        done = nv * kVec;
    }
    for (int64_t i = done + tid; i < r.len; i += kBlock)
        P[i] = static_cast<uint16_t>(param_bits<PDT>(ld1<MST>(T, i)));
}

/* ---------------------------------------------------------------------- */
/* device-resident step: state init and end-of-step bookkeeping            */
/* ---------------------------------------------------------------------- */
__global__ __launch_bounds__(64) void k_scaler_init(hpo_scaler_state* st, float loss_scale, int32_t hysteresis,
                                                    int64_t applied)
{
    if (threadIdx.x == 0) {
        hpo_scaler_state s{};
        s.loss_scale = loss_scale;
        s.inv_scale = static_cast<float>(1.0 / static_cast<double>(loss_scale));
        s.hysteresis_tracker = hysteresis;
        s.applied_steps = applied;
        s.step_inv_scale = s.inv_scale;
        *st = s;
    }
}

template <typename... Args>
hipError_t launch(void (*kernel)(Args...), int64_t grid, int block, hipStream_t stream,
                  Args... args)
{
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<uint32_t>(grid)),
                           dim3(block), argv, 0, stream);
}

}  // namespace

hipError_t launch_grad_pass(const SetView& sv, int64_t n_chunks, int32_t grad_group, GradPass pass,
                            float inv_scale, const float* d_inv, const Partials& p, hipStream_t stream)
{
    if (n_chunks == 0)
        return hipSuccess;
    const int64_t grid = (n_chunks + grad_group - 1) / grad_group;
    const bool flat = sv.is_flat != 0;
#define HPO_GRAD_LAUNCH_G(F, P, G) \
    launch(k_grad_pass<F, P, G>, grid, kGradBlock, stream, sv, n_chunks, grad_group, inv_scale, d_inv, p)
#define HPO_GRAD_LAUNCH(F, P) (sv.grad_bf16 ? HPO_GRAD_LAUNCH_G(F, P, kBF16) : HPO_GRAD_LAUNCH_G(F, P, kF32))
    switch (pass) {
    case GradPass::kNorm:
        return flat ? HPO_GRAD_LAUNCH(true, GradPass::kNorm) : HPO_GRAD_LAUNCH(false, GradPass::kNorm);
    case GradPass::kCheck:
        return flat ? HPO_GRAD_LAUNCH(true, GradPass::kCheck) : HPO_GRAD_LAUNCH(false, GradPass::kCheck);
    case GradPass::kUnscale:
        return flat ? HPO_GRAD_LAUNCH(true, GradPass::kUnscale) : HPO_GRAD_LAUNCH(false, GradPass::kUnscale);
    }
#undef HPO_GRAD_LAUNCH
#undef HPO_GRAD_LAUNCH_G
    return hipErrorInvalidValue;
}

template <bool DEV, int SDT, int GDT, int PDT, int MST, bool NT>
hipError_t launch_adam_n(const SetView& sv, int64_t n_chunks, int32_t mode, const AdamScalars& sc,
                         hipStream_t stream)
{
    const bool flat = sv.is_flat != 0;
    if (mode == HPO_ADAMW)
        return flat ? launch(k_adam<true, PDT, HPO_ADAMW, DEV, SDT, GDT, MST, NT>, n_chunks, kBlock, stream, sv, sc,
                             n_chunks)
                    : launch(k_adam<false, PDT, HPO_ADAMW, DEV, SDT, GDT, MST, NT>, n_chunks, kBlock, stream, sv, sc,
                             n_chunks);
    return flat ? launch(k_adam<true, PDT, HPO_ADAM_L2, DEV, SDT, GDT, MST, NT>, n_chunks, kBlock, stream, sv, sc,
                         n_chunks)
                : launch(k_adam<false, PDT, HPO_ADAM_L2, DEV, SDT, GDT, MST, NT>, n_chunks, kBlock, stream, sv, sc,
                         n_chunks);
}

template <bool DEV, int SDT, int GDT, int PDT, int MST>
hipError_t launch_adam_p(const SetView& sv, int64_t n_chunks, int32_t mode, const AdamScalars& sc,
                         hipStream_t stream)
{
    return sv.cached ? launch_adam_n<DEV, SDT, GDT, PDT, MST, false>(sv, n_chunks, mode, sc, stream)
                     : launch_adam_n<DEV, SDT, GDT, PDT, MST, true>(sv, n_chunks, mode, sc, stream);
}

template <bool DEV, int SDT, int GDT>
hipError_t launch_adam_s(const SetView& sv, int64_t n_chunks, int32_t mode, const AdamScalars& sc,
                         hipStream_t stream)
{
    switch (sv.param_dtype) {
    case HPO_PARAM_BF16:
        return sv.master_fp16 ? launch_adam_p<DEV, SDT, GDT, HPO_PARAM_BF16, kF16>(sv, n_chunks, mode, sc, stream)
                              : launch_adam_p<DEV, SDT, GDT, HPO_PARAM_BF16, kF32>(sv, n_chunks, mode, sc, stream);
    case HPO_PARAM_FP16: return launch_adam_p<DEV, SDT, GDT, HPO_PARAM_FP16, kF32>(sv, n_chunks, mode, sc, stream);
    default: return launch_adam_p<DEV, SDT, GDT, HPO_PARAM_FP32, kF32>(sv, n_chunks, mode, sc, stream);
    }
}

template <bool DEV, int SDT>
hipError_t launch_adam_g(const SetView& sv, int64_t n_chunks, int32_t mode, const AdamScalars& sc,
                         hipStream_t stream)
{
    return sv.grad_bf16 ? launch_adam_s<DEV, SDT, kBF16>(sv, n_chunks, mode, sc, stream)
                        : launch_adam_s<DEV, SDT, kF32>(sv, n_chunks, mode, sc, stream);
}

template <bool DEV>
hipError_t launch_adam_t(const SetView& sv, int64_t n_chunks, int32_t mode, const AdamScalars& sc,
                         hipStream_t stream)
{
    /* fp32 or bf16 moments (the host refuses fp16 ones) */
    return sv.state_store == kBF16 ? launch_adam_g<DEV, kBF16>(sv, n_chunks, mode, sc, stream)
                                   : launch_adam_g<DEV, kF32>(sv, n_chunks, mode, sc, stream);
}

hipError_t launch_adam(const SetView& sv, int64_t n_chunks, int32_t mode, const AdamScalars& sc,
                       hipStream_t stream)
{
    if (n_chunks == 0)
        return hipSuccess;
    return sc.d_state != nullptr ? launch_adam_t<true>(sv, n_chunks, mode, sc, stream)
                                 : launch_adam_t<false>(sv, n_chunks, mode, sc, stream);
}


namespace {

/* First stage for the sets with many partials, then the last-stage inputs. */
hipError_t fold_inputs(const Partials* p, int n_sets, bool want_sum, Fold& f, hipStream_t stream)
{
    if (n_sets < 1 || n_sets > kMaxFoldSets)
        return hipErrorInvalidValue;
    f.count = n_sets;
    for (int k = 0; k < n_sets; ++k) {
        const double* ps = p[k].sum;
        const int32_t* pf = p[k].flag;
        const int64_t* pz = p[k].zeros;
        int64_t n = p[k].n;
        if (n > kFinalSpan) {
            const int64_t n_stage = (n + kFinalSpan - 1) / kFinalSpan;
            hipError_t e = launch(k_reduce_stage, n_stage, kFinalBlock, stream, p[k], want_sum ? 1 : 0);
            if (e != hipSuccess)
                return e;
            ps = p[k].stage_sum;
            pf = p[k].stage_flag;
            pz = p[k].stage_zeros;
            n = n_stage;
        }
        f.sum[k] = ps;
        f.flag[k] = pf;
        f.zeros[k] = pz;
        f.n[k] = n;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_finalize_sets(const Partials* p, int n_sets, float* d_norm, int32_t* d_found, int64_t* d_zeros,
                                hipStream_t stream)
{
    Fold f{};
    hipError_t e = fold_inputs(p, n_sets, d_norm != nullptr, f, stream);
    if (e != hipSuccess)
        return e;
    FinalOut o{};
    o.d_norm = d_norm;
    o.d_found = d_found;
    o.d_zeros = d_zeros;
    return launch(k_finalize, 1, kFinalBlock, stream, f, o);
}

hipError_t launch_finalize_state_sets(const Partials* p, int n_sets, const FinalOut& out, hipStream_t stream)
{
    Fold f{};
    hipError_t e = fold_inputs(p, n_sets, true, f, stream);
    if (e != hipSuccess)
        return e;
    return launch(k_finalize_state, 1, kFinalBlock, stream, f, out);
}

hipError_t launch_grad_pass_final(const SetView& sv, int64_t n_chunks, int32_t grad_group, GradPass pass,
                                  float inv_scale, const float* d_inv, const Partials& p, const FinalOut& out,
                                  hipStream_t stream)
{
    hipError_t e = launch_grad_pass(sv, n_chunks, grad_group, pass, inv_scale, d_inv, p, stream);
    if (e != hipSuccess)
        return e;
    /* an empty set still finalizes, so the norm and the count read 0 */
    return out.st != nullptr ? launch_finalize_state_sets(&p, 1, out, stream)
                             : launch_finalize_sets(&p, 1, out.d_norm, out.d_found, out.d_zeros, stream);
}

hipError_t launch_scaler_init(hpo_scaler_state* st, float loss_scale, int32_t hysteresis, int64_t applied,
                              hipStream_t stream)
{
    return launch(k_scaler_init, 1, 64, stream, st, loss_scale, hysteresis, applied);
}

hipError_t launch_stream_probe(const SetView& sv, int64_t n_chunks, hipStream_t stream)
{
    if (n_chunks == 0)
        return hipSuccess;
    return sv.param_dtype == HPO_PARAM_FP16 ? launch(k_stream_probe<HPO_PARAM_FP16>, n_chunks, kBlock, stream, sv, n_chunks)
                                            : launch(k_stream_probe<HPO_PARAM_BF16>, n_chunks, kBlock, stream, sv, n_chunks);
}

hipError_t launch_copy_main_to_model(const SetView& sv, int64_t n_chunks, hipStream_t stream)
{
    if (n_chunks == 0 || sv.param_dtype == HPO_PARAM_FP32)
        return hipSuccess;
    if (sv.param_dtype == HPO_PARAM_FP16)
        return sv.is_flat ? launch(k_copy_main_to_model<true, HPO_PARAM_FP16, kF32>, n_chunks, kBlock, stream, sv)
                          : launch(k_copy_main_to_model<false, HPO_PARAM_FP16, kF32>, n_chunks, kBlock, stream, sv);
    if (sv.master_fp16)
        return sv.is_flat ? launch(k_copy_main_to_model<true, HPO_PARAM_BF16, kF16>, n_chunks, kBlock, stream, sv)
                          : launch(k_copy_main_to_model<false, HPO_PARAM_BF16, kF16>, n_chunks, kBlock, stream, sv);
    return sv.is_flat ? launch(k_copy_main_to_model<true, HPO_PARAM_BF16, kF32>, n_chunks, kBlock, stream, sv)
                      : launch(k_copy_main_to_model<false, HPO_PARAM_BF16, kF32>, n_chunks, kBlock, stream, sv);
}

}  // namespace hpo
