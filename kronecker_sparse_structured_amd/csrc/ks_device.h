// ks_device.h -- small device helpers shared by the libks kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace ks {

// bf16 values travel as their raw 16 bits: the upper half of an fp32 word.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// Low / high bf16 of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four consecutive elements (16-byte aligned for fp32, 8-byte for bf16),
// widened to fp32, in one load.
__device__ __forceinline__ void load4_f32(const float* p, float (&v)[4]) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 w = *reinterpret_cast<const f32x4*>(p);
    v[0] = w[0];
    v[1] = w[1];
    v[2] = w[2];
    v[3] = w[3];
}
__device__ __forceinline__ void load4_f32(const bf16_t* p, float (&v)[4]) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    v[0] = bf16_lo(w[0]);
    v[1] = bf16_hi(w[0]);
    v[2] = bf16_lo(w[1]);
    v[3] = bf16_hi(w[1]);
}

template <int N>
__device__ __forceinline__ void zero(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = 0.0f;
}

}  // namespace ks
