// W4A4 GEMM on gfx950 int8 MFMA ("Infra Quant II", QuaRot Method: INT4 x INT4
// products accumulated in INT32, then scaled by the activation row scale and
// the weight column scale).
//
// gfx950 has no INT4 matrix instruction, so the packed nibbles are widened to
// int8 in registers and fed to v_mfma_i32_32x32x32_i8. The widening keeps each
// nibble in the HIGH half of its byte ((w << 4) & 0xF0F0F0F0 for the even
// elements, w & 0xF0F0F0F0 for the odd ones): each int8 then equals 16 * code,
// every product carries a factor 256, and the int32 sum is shifted right by 8
// at the end (exact: |sum| <= 64 K * 256 < 2^31 for K <= 131072). The widened
// bytes of a lane are in the order 0,2,4,6,1,3,5,7,... of its codes; both
// operands use the same order, so each MFMA still pairs equal k.
//
// Tile: 128 tokens x 128 weight rows per workgroup, 4 waves (2 x 2), each wave
// 64 x 64 = 2 x 2 MFMA blocks of 32 x 32. K advances 128 codes (64 bytes) per
// step through double-buffered LDS (row pitch 80 bytes). MFMA A = weight rows,
// B = token rows, so each lane's accumulators hold 4 consecutive output
// columns of one token (8-byte bf16 stores).
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

constexpr int BM = 128;     // tokens per tile
constexpr int BN = 128;     // weight rows per tile
constexpr int BKB = 64;     // packed bytes per k-step (128 codes)
constexpr int PITCH = 80;   // LDS row pitch (bytes)

__device__ __forceinline__ void widen(const uint4 p, v4i& m0, v4i& m1) {
  const uint32_t H = 0xF0F0F0F0u;
  m0[0] = static_cast<int>((p.x << 4) & H); m0[1] = static_cast<int>(p.x & H);
  m0[2] = static_cast<int>((p.y << 4) & H); m0[3] = static_cast<int>(p.y & H);
  m1[0] = static_cast<int>((p.z << 4) & H); m1[1] = static_cast<int>(p.z & H);
  m1[2] = static_cast<int>((p.w << 4) & H); m1[3] = static_cast<int>(p.w & H);
}

template <bool I32OUT>
__global__ void __launch_bounds__(256)
gemm_kernel(const uint8_t* __restrict__ a, const float* __restrict__ s_a,
            const uint8_t* __restrict__ w, const float* __restrict__ s_w, void* __restrict__ y,
            int T, int K, int N) {
  __shared__ __attribute__((aligned(16))) uint8_t la[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t lw[2][BN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;          // token half of the tile
  const int wn = wave & 1;           // weight half of the tile
  const int n0 = blockIdx.x * BN;
  const int t0 = blockIdx.y * BM;
  const int KB = K / 2;
  const int nk = (KB + BKB - 1) / BKB;

  uint4 ra[2], rw[2];
  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 2;
      const int kb = ks * BKB + (c & 3) * 16;
      const int ta = min(t0 + row, T - 1);
      const int tn = min(n0 + row, N - 1);
      if (kb < KB) {
        ra[i] = *reinterpret_cast<const uint4*>(a + static_cast<int64_t>(ta) * KB + kb);
        rw[i] = *reinterpret_cast<const uint4*>(w + static_cast<int64_t>(tn) * KB + kb);
      } else {
        ra[i] = make_uint4(0, 0, 0, 0);
        rw[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 2;
      const int col = (c & 3) * 16;
      *reinterpret_cast<uint4*>(&la[st][row * PITCH + col]) = ra[i];
      *reinterpret_cast<uint4*>(&lw[st][row * PITCH + col]) = rw[i];
    }
  };

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  gload(0);
  lstore(0);
  __syncthreads();
  const int lrow = lane & 31;
  const int lgrp = (lane >> 5) * 16;
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v4i w0[2], w1[2], a0[2], a1[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint4 pw = *reinterpret_cast<const uint4*>(
            &lw[st][(wn * 64 + b * 32 + lrow) * PITCH + kk * 32 + lgrp]);
        const uint4 pa = *reinterpret_cast<const uint4*>(
            &la[st][(wm * 64 + b * 32 + lrow) * PITCH + kk * 32 + lgrp]);
        widen(pw, w0[b], w1[b]);
        widen(pa, a0[b], a1[b]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0[i], a0[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1[i], a1[j], acc[i][j], 0, 0, 0);
        }
    }
    if (ks + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds, for token t = .. + (lane & 31), output columns
  // n = .. + 8*(v/4) + 4*(lane/32) + v%4, v = 0..15
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + wm * 64 + j * 32 + (lane & 31);
    if (t >= T) continue;
    const float sa = I32OUT ? 0.0f : s_a[t];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + i * 32 + 8 * q + 4 * (lane >> 5);
        int vals[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vals[c] = acc[i][j][4 * q + c] >> 8;
        const int64_t off = static_cast<int64_t>(t) * N + n;
        if constexpr (I32OUT) {
          int* yp = static_cast<int*>(y) + off;
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<int4*>(yp) = make_int4(vals[0], vals[1], vals[2], vals[3]);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (n + c < N) yp[c] = vals[c];
          }
        } else {
          uint16_t* yp = static_cast<uint16_t*>(y) + off;
          uint16_t o[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float sw = (n + c < N) ? s_w[n + c] : 0.0f;
            o[c] = f32_to_bf16((static_cast<float>(vals[c]) * sa) * sw);
          }
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<uint2*>(yp) =
                make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                           o[2] | (static_cast<uint32_t>(o[3]) << 16));
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (n + c < N) yp[c] = o[c];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                       void* y, bool i32_out, int64_t T, int64_t K, int64_t N, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((T + BM - 1) / BM));
  if (i32_out)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(256), 0, s, a, s_a, w, s_w, y,
                       static_cast<int>(T), static_cast<int>(K), static_cast<int>(N));
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(256), 0, s, a, s_a, w, s_w, y,
                       static_cast<int>(T), static_cast<int>(K), static_cast<int>(N));
  return hipGetLastError();
}

}  // namespace rw4
