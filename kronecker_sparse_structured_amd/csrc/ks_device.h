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

template <int N>
__device__ __forceinline__ void zero(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = 0.0f;
}

}  // namespace ks
