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

// ----------------------------------------------------------------------------
// FP6 operand tiles of the matrix-core GEMM.
//
// An INT4 code q in [-7, 7] is stored as the FP6 E2M3 number equal to q (sign
// bit 5, exponent bits 4..3 with bias 1, mantissa bits 2..0); every such
// integer is exact in E2M3, so the f8f6f4 matrix instruction multiplies the
// codes exactly. A matrix [R][K] (K % 64 == 0) is stored as tiles of 32 rows x
// 64 codes, 1536 bytes each, tile (R/32 index rt, K/64 index kt) at byte
// (rt * K/64 + kt) * 1536. Inside a tile, lane l of the consuming wave owns row
// l % 32 and codes 32 * (l / 32) + e, e = 0..31, as 32 six-bit fields (field e
// at bit 6e of 192 little-endian bits = six 32-bit words). Words 0..3 of lane l
// are the 16 bytes at l * 16 (plane 0, 1 KiB); words 4..5 are the 8 bytes at
// 1024 + l * 8 (plane 1, 512 bytes), so a wave reads a tile with one 16-byte
// and one 8-byte load per lane, both contiguous across the wave.
constexpr int kTileBytes = 1536;
constexpr int kPlane1 = 1024;

// E2M3 encoding of an integer in [-7, 7]
__device__ __forceinline__ uint32_t e2m3(int q) {
  constexpr uint64_t kMag = (8ull << 6) | (16ull << 12) | (20ull << 18) | (24ull << 24) |
                            (26ull << 30) | (28ull << 36) | (30ull << 42);
  const uint32_t a = static_cast<uint32_t>(q < 0 ? -q : q);
  return static_cast<uint32_t>((kMag >> (6 * a)) & 63u) | (q < 0 ? 32u : 0u);
}

// 16 six-bit fields packed into three words, field e at bit 6e
struct Field12 { uint32_t w0, w1, w2; };
__device__ __forceinline__ Field12 pack_fields16(const uint32_t (&f)[16]) {
  uint64_t a = 0, b = 0;
#pragma unroll
  for (int e = 0; e < 10; ++e) a |= static_cast<uint64_t>(f[e]) << (6 * e);
#pragma unroll
  for (int e = 10; e < 16; ++e) b |= static_cast<uint64_t>(f[e]) << (6 * (e - 10));
  return Field12{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) | static_cast<uint32_t>(b << 28),
                 static_cast<uint32_t>(b >> 4)};
}

// store the 16 fields of codes [k0, k0 + 16) of row t (k0 % 16 == 0) into a
// tiled matrix with K columns: they are words 0..2 (k0 % 32 == 0) or words
// 3..5 of the owning lane
__device__ __forceinline__ void store_fields16(uint8_t* tiles, int64_t t, int64_t k0, int64_t K,
                                               Field12 v) {
  const int64_t tile = (t >> 5) * (K >> 6) + (k0 >> 6);
  const int lane = static_cast<int>(((k0 >> 5) & 1) * 32 + (t & 31));
  uint8_t* base = tiles + tile * kTileBytes;
  uint32_t* p0 = reinterpret_cast<uint32_t*>(base + lane * 16);
  if (((k0 >> 4) & 1) == 0) {
    p0[0] = v.w0; p0[1] = v.w1; p0[2] = v.w2;
  } else {
    p0[3] = v.w0;
    *reinterpret_cast<uint2*>(base + kPlane1 + lane * 8) = make_uint2(v.w1, v.w2);
  }
}

}  // namespace rw4
