// Device helpers shared by the gfx950 kernels of the rotated W4A4 path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rw4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// the two bf16 halves of a 32-bit word -> fp32 (element 0 = low half)
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// max over aligned groups of W lanes (W a power of two <= 64)
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// symmetric absmax INT4 code of v with step s (s > 0): clamp(rint(v / s), -8, 7).
// The quotient is the correctly rounded fp32 division, rounded half-to-even.
__device__ __forceinline__ int quant4(float v, float s) {
  float q = rintf(v / s);
  q = fminf(fmaxf(q, -8.0f), 7.0f);
  return static_cast<int>(q);
}

__device__ __forceinline__ uint32_t nib(int q) { return static_cast<uint32_t>(q) & 0xFu; }

}  // namespace rw4
