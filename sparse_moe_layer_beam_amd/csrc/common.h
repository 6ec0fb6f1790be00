// Device-side helpers shared by the HIP kernels of the MoE layer (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte load of data that one call reads once (the expert weights the decode kernels
// stream), with the non-temporal hint. Measured on MI355X, streams of 1 KB per load
// instruction read ~6.7-7.0 TB/s with it and ~6.1 TB/s without.
__device__ __forceinline__ u32x4 ld_once(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u16)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// double -> bf16 with a single rounding (to nearest even): round to float with
// round-to-odd (truncate, then force the last bit if anything was cut), which keeps
// enough information for the final float -> bf16 rounding to be exact.
__device__ __forceinline__ u16 f64_to_bf16(double v) {
    float t = __double2float_rz(v);
    uint32_t u = __float_as_uint(t);
    if ((double)t != v) u |= 1u;
    return (u16)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// silu(g) * u in FP32 with the hardware exponential and reciprocal (about 1 ulp each): against
// the IEEE division and the library expf, the prefill gate/up GEMM at T=8192 ran 3.54-3.57 ->
// 3.50-3.51 ms on MI355X. g -> -inf gives -0 (exp overflows, the reciprocal is 0), g -> +inf g * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = __shfl_xor(v, m, kWave);
        v = o > v ? o : v;
    }
    return v;
}

}  // namespace beam
