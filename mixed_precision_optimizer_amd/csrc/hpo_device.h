/*
 * hpo_device.h -- device helpers shared by libhpo's kernel files
 * (hpo_kernels.hip, hpo_muon.hip).  Not part of the public ABI.
 */
#ifndef HPO_DEVICE_H
#define HPO_DEVICE_H

#include <hip/hip_runtime.h>

namespace hpo {
namespace {

/* fp32 -> bf16 bits, IEEE round to nearest, ties to even ([OPT-INFRA] §9.2
 * write-back; [FP32-RFC] case 1: the model param equals the bf16 image of the
 * master after every step).  Adding 0x7FFF plus the kept part's lowest bit to
 * the fp32 bits and dropping the low half rounds up exactly when the dropped
 * half exceeds 0x8000, or equals it with an odd kept part; a carry ripples
 * into the exponent (up to infinity).  NaN becomes the quiet NaN 0x7FC0 with
 * the input's sign. */
__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return ((u >> 16) & 0x8000u) | 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

/* Sum of one value per lane over an NT-lane workgroup: wavefront shuffles,
 * then the wavefront sums through LDS in a fixed order (T = double for the
 * norm's partials, integers for counts). */
template <int NT, typename T = double>
__device__ __forceinline__ T block_sum(T x)
{
    constexpr int kWaves = NT / 64;
    __shared__ T wsum[kWaves];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_down(x, off, 64);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (lane == 0)
        wsum[wave] = x;
    __syncthreads();
    T tot = 0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            tot += wsum[w];
    }
    return tot; /* valid in thread 0 */
}

}  // namespace
}  // namespace hpo

#endif /* HPO_DEVICE_H */
