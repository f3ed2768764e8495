// Device helpers shared by the gfx950 kernels of the rotated W4A4 path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rw4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8bf ld8(const uint16_t* p) { return *reinterpret_cast<const v8bf*>(p); }
__device__ __forceinline__ v8bf as8(uint4 u) { return __builtin_bit_cast(v8bf, u); }

// D (16 x 16, fp32) += A (16 x 32, bf16) B (32 x 16, bf16). Lane l holds
// A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16] and
// D[4 (l / 16) + 0..3][l % 16].
__device__ __forceinline__ v4f mfma(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float v16f __attribute__((ext_vector_type(16)));

// Let the last matrix-core results land before anything else reads them: no
// instruction may be scheduled across, and the wave sleeps ~64 cycles (longer
// than the instruction's pipeline) in between.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_sched_barrier(0);
}

// this wave's LDS accesses have completed, then a workgroup barrier that the
// compiler may not move memory accesses across; global loads and stores in
// flight stay in flight
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Streaming 16-byte store (the non-temporal hint) for outputs of tens of MiB
// that the same XCD does not read back soon: the line goes out toward memory
// instead of staying dirty in the XCD's L2, where the next kernel's loads
// would wait behind its write-back. Measured on MI355X at D = 4096,
// T = 2048, 4096 -> 4096 (graph-replayed): projection + fused prologue + GEMM
// 48.6 instead of 51.5 us with the GEMM's bf16 output written this way, the
// standalone alignment 18.2 instead of 22.6 us with its fp32 output. Not for
// the FP6 tiles and codes that the GEMM reads next: streamed, they cost the
// pass 59 instead of 51.5 us.
__device__ __forceinline__ void store_stream16(void* p, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_stream16(void* p, float4 v) {
  store_stream16(p, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                               __float_as_uint(v.w)));
}

// Streaming 16-byte load (the non-temporal hint) for a row's last read: the
// line is not kept in L2 at the expense of lines that are still to be used.
// In the wave-per-row kernel (fp32 rows of 2048-8192 values), cold rows at
// D = 4096, T = 2048: transform in place 17.1 -> 12.3 us, quantizer
// 10.3 -> 9.3 us. Not in the workgroup-per-row kernel (its row kernel in the
// D = 8192 unit lost 15-30 us of 1260 with it) nor on the fused prologue's
// second read of x (slower).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ float4 load_stream16f(const void* p) {
  const uint4 u = load_stream16(p);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                     __uint_as_float(u.w));
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even: the gfx950 conversion
// instruction (v_cvt_pk_bf16_f32), one instruction where the integer
// rounding (add the rounding bias and the tie bit, shift) took three; the
// same bits for every finite input
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// the two bf16 halves of a 32-bit word -> fp32 (element 0 = low half)
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// SiLU(g) * u in fp32 (the gate of the SiLU-gated FFN), with the hardware
// base-2 exponential and reciprocal, each within 1 ulp: e = 2^(-g log2 e),
// then g / (1 + e) * u. The rounding of the exponent's argument adds up to
// |g| 2^-24 relative, so for every bf16 g >= -20 the gate is within 1.2e-6 of
// g / (1 + e^-g) (worked out over all of them against float64, with one ulp
// allowed per hardware operation); below -20 the gate itself is under
// 3e-9 |g|. Infinite and NaN inputs give what the quotient gives.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

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

// ----------------------------------------------------------------------------
// Cross-lane butterflies of the register-resident Walsh-Hadamard transforms.
// A butterfly on index bit b pairs values whose indices differ only in b; when
// b is a lane bit the partner value sits in another lane of the wave.
// butterfly with the lane whose index differs in one bit, partner read by a
// DPP move: the lower lane gets a + b, the upper b' - a' = a - b
template <int CTRL>
__device__ __forceinline__ float dpp_bfly(float v, float sgn) {
  const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
  return fmaf(sgn, v, p);
}
// lane bit 2 inside a 16-lane row: banks 0 and 2 (bit clear) read lane + 4
// (row_ror:12), banks 1 and 3 read lane - 4 (row_ror:4)
__device__ __forceinline__ float bfly_x4(float v, float sgn) {
  int p = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x12C, 0xF, 0x5, true);
  p = __builtin_amdgcn_update_dpp(p, __float_as_int(v), 0x124, 0xF, 0xA, false);
  return fmaf(sgn, v, __int_as_float(p));
}
// lane bit 4 (permlane16 swap) or 5 (permlane32 swap) for two values a, b at
// once: the swap moves the partner half-row of a next to a's own half and b's
// lower half next to b's upper half, the butterfly runs in-lane, and a second
// swap restores the layout
template <int BIT>
__device__ __forceinline__ void bfly_swap(float& a, float& b) {
  const unsigned ua = __float_as_uint(a), ub = __float_as_uint(b);
  auto p = BIT == 4 ? __builtin_amdgcn_permlane16_swap(ua, ub, false, false)
                    : __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
  const float A = __uint_as_float(p[0]), B = __uint_as_float(p[1]);
  const unsigned us = __float_as_uint(A + B), ud = __float_as_uint(A - B);
  auto q = BIT == 4 ? __builtin_amdgcn_permlane16_swap(us, ud, false, false)
                    : __builtin_amdgcn_permlane32_swap(us, ud, false, false);
  a = __uint_as_float(q[0]);
  b = __uint_as_float(q[1]);
}

// all butterflies of the six lane bits of a wave, for NV values per lane
// (sg1.. are +1 on lanes whose bit is clear, -1 where it is set); one lane bit
// at a time over every value, so that independent moves issue back to back
template <int NV, int LB>
__device__ __forceinline__ void lane_butterflies(float (&v)[NV], int lane) {
  static_assert(NV % 32 == 0 || LB <= 4, "swap butterflies pair values j and j + 16 of 32");
  const float sg1 = (lane & 1) ? -1.0f : 1.0f;
  const float sg2 = (lane & 2) ? -1.0f : 1.0f;
  const float sg4 = (lane & 4) ? -1.0f : 1.0f;
  const float sg8 = (lane & 8) ? -1.0f : 1.0f;
  if constexpr (LB > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = dpp_bfly<0xB1>(v[j], sg1);  // quad_perm 1,0,3,2
  }
  if constexpr (LB > 1) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = dpp_bfly<0x4E>(v[j], sg2);  // quad_perm 2,3,0,1
  }
  if constexpr (LB > 2) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = bfly_x4(v[j], sg4);
  }
  if constexpr (LB > 3) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = dpp_bfly<0x128>(v[j], sg8);  // row_ror:8
  }
  if constexpr (LB > 4) {
#pragma unroll
    for (int j0 = 0; j0 < NV; j0 += 32)
#pragma unroll
      for (int j = 0; j < 16; ++j) bfly_swap<4>(v[j0 + j], v[j0 + j + 16]);
  }
  if constexpr (LB > 5) {
#pragma unroll
    for (int j0 = 0; j0 < NV; j0 += 32)
#pragma unroll
      for (int j = 0; j < 16; ++j) bfly_swap<5>(v[j0 + j], v[j0 + j + 16]);
  }
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

// 16 six-bit fields packed into three words, field e at bit 6e
struct Field12 { uint32_t w0, w1, w2; };

// store the 16 fields of codes [k0, k0 + 16) of row t (k0 % 16 == 0) into a
// tiled matrix with K columns: they are words 0..2 (k0 % 32 == 0) or words
// 3..5 of the owning lane
// store the 32 fields of codes [k0, k0 + 32) of row t (k0 % 32 == 0): the six
// words of the owning lane, as one 16-byte and one 8-byte store
__device__ __forceinline__ void store_fields32(uint8_t* tiles, int64_t t, int64_t k0, int64_t K,
                                               Field12 a, Field12 b) {
  const int64_t tile = (t >> 5) * (K >> 6) + (k0 >> 6);
  const int lane = static_cast<int>(((k0 >> 5) & 1) * 32 + (t & 31));
  uint8_t* base = tiles + tile * kTileBytes;
  *reinterpret_cast<uint4*>(base + lane * 16) = make_uint4(a.w0, a.w1, a.w2, b.w0);
  *reinterpret_cast<uint2*>(base + kPlane1 + lane * 8) = make_uint2(b.w1, b.w2);
}

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

// Per-row quantizer with the step's reciprocal. For a row with step s
// (s = fl32(absmax / qmax), normal; qmax <= 7) and y = fl32(1 / s) (correctly
// rounded), t = fl32(v * y) differs from v / s by at most
// 2^-23 |v / s| <= 8.4e-7 and fl32(v / s) from v / s by at most 4.2e-7. So when t is at least 2^-18 away
// from every half-integer, fl32(v / s) lies strictly between the same two
// half-integers as t and rint(fl32(v / s)) == rint(t); otherwise the exact
// quotient decides. Codes equal quant4(v, s) for every v.
struct RowQuant {
  float s, y;
  bool fast;  // s normal: y finite and the bound above holds
  __device__ __forceinline__ explicit RowQuant(float step)
      : s(step), y(step > 0.0f ? 1.0f / step : 0.0f), fast(step >= 1.17549435e-38f) {}
  // integer-valued code in [-8, 7]; zero is +0 (never -0)
  __device__ __forceinline__ float code(float v) const {
    if (!(s > 0.0f)) return 0.0f;
    if (fast) {
      const float t = v * y;               // |t| <= qmax + 8.4e-7, so |rint(t)| <= qmax
      const float q = rintf(t);
      if (0.5f - fabsf(t - q) >= 3.814697265625e-06f)  // 2^-18
        return q + 0.0f;
    }
    return static_cast<float>(quant4(v, s));
  }
  // codes of v[0..NV) from the reciprocal, with one check for all of them:
  // true when every value is at least 2^-18 from a half-integer (then each
  // q[e] equals code(v[e])); false when the caller must use code()
  template <int NV>
  __device__ __forceinline__ bool fast_codes(const float (&v)[NV], float (&q)[NV]) const {
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const float t = v[e] * y;
      const float r = rintf(t);
      q[e] = r + 0.0f;
      mx = fmaxf(mx, fabsf(t - r));
    }
    return fast && 0.5f - mx >= 3.814697265625e-06f;
  }
};

// Packed E2M3 fields from integer-valued floats in [-7, 7] (no -0) with the
// gfx950 conversion instruction: with scale 1.0 it converts exactly, and it
// places element i of its first source in field 2i and element i of its
// second source in field 2i + 1 of a 192-bit result (field e at bit 6e).
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef uint32_t v6u_t __attribute__((ext_vector_type(6)));

// fields 0..31 = q[0..31]: the six words of one lane
__device__ __forceinline__ v6u_t pack_fp6_32(const float (&q)[32]) {
  v16f_t a, b;
#pragma unroll
  for (int i = 0; i < 16; ++i) { a[i] = q[2 * i]; b[i] = q[2 * i + 1]; }
  return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
}

// fields 0..15 = q[0..15]: three words
__device__ __forceinline__ Field12 pack_fp6_16(const float (&q)[16]) {
  v16f_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) { a[i] = q[2 * i]; b[i] = q[2 * i + 1]; }
#pragma unroll
  for (int i = 8; i < 16; ++i) { a[i] = 0.0f; b[i] = 0.0f; }
  const v6u_t w = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
  return Field12{w[0], w[1], w[2]};
}

}  // namespace rw4
