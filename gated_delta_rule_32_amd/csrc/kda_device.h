// kda_device.h -- small device-side helpers shared by the libkda kernels
// (element loads and stores for fp32 / bf16, the exp used for the gates, and
// the MFMA operand vector types).  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// exp(x) through the hardware base-2 exponential: exp(x) = 2^(x * log2(e)).
__device__ __forceinline__ float exp_fast(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950).
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

// Load 4 consecutive elements as fp32 (16-byte aligned for fp32, 8 for bf16).
__device__ __forceinline__ f32x4 load4(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ f32x4 load4(const bf16_t* p) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    f32x4 r;
    r[0] = (float)v[0]; r[1] = (float)v[1]; r[2] = (float)v[2]; r[3] = (float)v[3];
    return r;
}
__device__ __forceinline__ void store4(float* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
}
__device__ __forceinline__ void store4(bf16_t* p, f32x4 x) {
    bf16x4 v;
    v[0] = (bf16_t)x[0]; v[1] = (bf16_t)x[1]; v[2] = (bf16_t)x[2]; v[3] = (bf16_t)x[3];
    *reinterpret_cast<bf16x4*>(p) = v;
}

}  // namespace kda
