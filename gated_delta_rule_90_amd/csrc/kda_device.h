// kda_device.h - device helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;
constexpr float kNormEps = 1e-6f;  // x / sqrt(sum x^2 + eps): the pages give no epsilon
constexpr float kLog2e = 1.4426950408889634f;

struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x)
{
    // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    __bf16 b = (__bf16)x;
    return bf16_t{__builtin_bit_cast(uint16_t, b)};
}

// Numerically safe logistic: 1 / (1 + e^-x); exp overflow gives 0, underflow 1.
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

template <int W = kWave>
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Workgroup barrier that orders LDS traffic only: it waits for this wave's
// LDS operations and then for every wave of the workgroup.  Unlike
// __syncthreads() it does not drain the vector memory counter, so global loads
// issued ahead (prefetch) and global stores stay in flight across it.  Only
// valid where no wave reads global memory written by another wave of the
// same workgroup before the kernel ends.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float4 fma4(float a, float4 b, float4 c)
{
    return make_float4(fmaf(a, b.x, c.x), fmaf(a, b.y, c.y), fmaf(a, b.z, c.z), fmaf(a, b.w, c.w));
}

}  // namespace kda
