// kda_device.h - device helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
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

// ---- buffer resources: 32-bit byte offsets with a range check.  A load at an
// offset past the resource reads zero and a store there is dropped.  Only the
// lane's offset register and the instruction's immediate offset enter the
// check (the scalar offset field does not), so every offset that must be
// checked goes in the lane's offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// A pointer that is the same in every lane, moved to scalar registers (a
// pointer chosen by a select, or carried through divergent control flow, can
// otherwise land in vector registers, and a resource built from it then needs
// a per-lane loop).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Rows r .. nr - 1 of a block whose rows are `stride` bytes apart and `width`
// bytes wide (an empty resource when r >= nr): a lane then addresses its row
// relative to row r, and rows from nr on fall past the end.  Every argument
// is the same in every lane of the wave (the resource is built in scalar
// registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int r, int nr, uint32_t stride,
                                                            uint32_t width)
{
    const int n = nr - r;
    const uint32_t bytes = n > 0 ? (uint32_t)(n - 1) * stride + width : 0u;
    return buf_rsrc(uniform_ptr(static_cast<const char*>(base) + (size_t)r * stride),
                    __builtin_amdgcn_readfirstlane(bytes));
}

template <typename T>
__device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (sizeof(T) == 2)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
    else if constexpr (sizeof(T) == 4)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <typename T>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, T v)
{
    typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
    if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, 0);
    else if constexpr (sizeof(T) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
    else if constexpr (sizeof(T) == 8)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_v, v), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_v, v), r, off, 0, 0);
}

// Numerically safe logistic: 1 / (1 + e^-x); exp overflow gives 0, underflow 1.
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// Cross-lane sums on VALU data paths instead of LDS permutes (ds_bpermute, one
// LDS round trip per step): DPP within quads and 16-lane rows, ds_swizzle for
// the xor-4/8 partners, and gfx950's v_permlane16/32_swap between rows and
// halves.
//
// swap_rows16(x, y): rows are the four 16-lane groups; afterwards
//     x = (x.row0, y.row0, x.row2, y.row2),  y = (x.row1, y.row1, x.row3, y.row3).
// swap_halves32(x, y): afterwards x = (x.lo, y.lo), y = (x.hi, y.hi).
// So x + y holds, in the lanes of the first row (half) of each pair, the sum of
// x over the pair and, in the second, the sum of y: a transposing reduction
// step.  For y = x, x + y = x + partner(x) in every lane.
// The swaps are inline assembly: the compiler's builtins for them return the
// first result twice.  The s_nop covers the hazard of a VALU write read by the
// permlane two instructions later.
__device__ __forceinline__ void swap_rows16(float& x, float& y)
{
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap_halves32(float& x, float& y)
{
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ float swap_add16(float x)
{
    float y = x;
    swap_rows16(x, y);
    return x + y;
}
__device__ __forceinline__ float swap_add32(float x)
{
    float y = x;
    swap_halves32(x, y);
    return x + y;
}

template <int OFF>
__device__ __forceinline__ float xor_add(float x)
{
    static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "power of two < 64");
    const int xi = __builtin_bit_cast(int, x);
    if constexpr (OFF == 1) {
        return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    } else if constexpr (OFF == 2) {
        return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    } else if constexpr (OFF == 4 || OFF == 8) {
        return x + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(xi, 0x1F | (OFF << 10)));   // lane ^ OFF
    } else if constexpr (OFF == 16) {
        return swap_add16(x);
    } else {
        return swap_add32(x);
    }
}

// x summed over the lanes that agree with this one outside bits [log2 FROM, 6):
// lanes l and l ^ OFF for every OFF = FROM, 2 FROM, ..., 32.  The whole wave must be active.
template <int FROM>
__device__ __forceinline__ float xor_sum_from(float x)
{
    if constexpr (FROM <= 1) x = xor_add<1>(x);
    if constexpr (FROM <= 2) x = xor_add<2>(x);
    if constexpr (FROM <= 4) x = xor_add<4>(x);
    if constexpr (FROM <= 8) x = xor_add<8>(x);
    if constexpr (FROM <= 16) x = xor_add<16>(x);
    if constexpr (FROM <= 32) x = xor_add<32>(x);
    return x;
}

// Sum over each aligned group of N lanes (N = 16, 32 or 64), in every lane of
// the group: quads and rows by DPP (the row mirrors pair lanes whose partial
// sums are already equal within their quad and half row), then rows and halves
// by permlane swaps.  The whole wave must be active.  The DPP moves request
// bound_ctrl, which lets the compiler fold each into its add; every source
// lane of these patterns exists, so it does not change the result.
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(N == 16 || N == 32 || N == 64, "group of 16, 32 or 64 lanes");
    auto dpp_add = [](float v, auto ctrl) {
        return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value, 0xF, 0xF, true));
    };
    x = dpp_add(x, std::integral_constant<int, 0xB1>{});    // quad_perm 1,0,3,2
    x = dpp_add(x, std::integral_constant<int, 0x4E>{});    // quad_perm 2,3,0,1
    x = dpp_add(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
    x = dpp_add(x, std::integral_constant<int, 0x140>{});   // row_mirror
    if constexpr (N >= 32) x = swap_add16(x);
    if constexpr (N >= 64) x = swap_add32(x);
    return x;
}

// Sum over the 64 lanes of a wave, in every lane.  The whole wave must be active.
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

// A zero held in a vector register that the compiler cannot see through.
// Added to a uniform index it turns the load into a per-lane (vector) load.
// That matters for prefetches: scalar loads share the lgkm counter with LDS
// operations, so the next LDS barrier would wait for a scalar prefetch to
// arrive from memory.
__device__ __forceinline__ int vector_zero()
{
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
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

// An empty use of a loaded value: the compiler waits for its load here, and
// cannot sink the load into a branch that alone uses it (where it would be
// waited for at once, with every other load in flight).  Vectors are settled
// as one register tuple: split into scalars, they would have to be gathered
// into a tuple again for 16-byte LDS stores.
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(uint16_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(bf16_t& x) { asm volatile("" : "+v"(x.bits)); }
__device__ __forceinline__ void settle(float4& x)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 t = {x.x, x.y, x.z, x.w};
    asm volatile("" : "+v"(t));
    x = make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void settle(uint2& x)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 t = {x.x, x.y};
    asm volatile("" : "+v"(t));
    x = make_uint2(t[0], t[1]);
}

__device__ __forceinline__ float4 fma4(float a, float4 b, float4 c)
{
    return make_float4(fmaf(a, b.x, c.x), fmaf(a, b.y, c.y), fmaf(a, b.z, c.z), fmaf(a, b.w, c.w));
}

}  // namespace kda
