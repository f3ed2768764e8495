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
// Tile: NWW x NWT waves, each wave BW x BT blocks of 32 x 32 outputs (BW along
// the weight rows, BT along the tokens). K advances 128 codes (64 bytes) per
// step through double-buffered LDS holding the packed codes (row pitch 80
// bytes). MFMA A = weight rows, B = token rows, so each lane's accumulators
// hold 4 consecutive output columns of one token (8-byte bf16 stores).
// Workgroups are renumbered so that the eight XCDs (which receive workgroups
// round-robin) each work on a contiguous band of weight tiles.
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace gemm {

constexpr int BKB = 64;     // packed bytes per k-step (128 codes)
constexpr int PITCH = 80;   // LDS row pitch (bytes)

__device__ __forceinline__ void widen(const uint4 p, v4i& m0, v4i& m1) {
  const uint32_t H = 0xF0F0F0F0u;
  m0[0] = static_cast<int>((p.x << 4) & H); m0[1] = static_cast<int>(p.x & H);
  m0[2] = static_cast<int>((p.y << 4) & H); m0[3] = static_cast<int>(p.y & H);
  m1[0] = static_cast<int>((p.z << 4) & H); m1[1] = static_cast<int>(p.z & H);
  m1[2] = static_cast<int>((p.w << 4) & H); m1[3] = static_cast<int>(p.w & H);
}

template <int NWW, int NWT, int BW, int BT>
struct Cfg {
  static constexpr int TW = NWW * BW * 32;        // weight rows per tile
  static constexpr int TT = NWT * BT * 32;        // tokens per tile
  static constexpr int NTH = 64 * NWW * NWT;
  static constexpr int LW = TW * 4 / NTH;         // 16-byte chunks per thread per k-step
  static constexpr int LA = TT * 4 / NTH;
  static_assert(LW >= 1 && LA >= 1 && TW * 4 % NTH == 0 && TT * 4 % NTH == 0, "tile/threads");
};

template <int NWW, int NWT, int BW, int BT, bool I32OUT>
__global__ void __launch_bounds__(64 * NWW * NWT)
gemm_kernel(const uint8_t* __restrict__ a, const float* __restrict__ s_a,
            const uint8_t* __restrict__ w, const float* __restrict__ s_w, void* __restrict__ y,
            int T, int K, int N) {
  using C = Cfg<NWW, NWT, BW, BT>;
  __shared__ __attribute__((aligned(16))) uint8_t lw[2][C::TW * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t la[2][C::TT * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ww = wave % NWW;
  const int wt = wave / NWW;

  // XCD-aware renumbering: workgroup b lands on XCD b % 8; give XCD k the
  // contiguous range [k * nb / 8, (k + 1) * nb / 8) of the tile order below.
  const int nwt = (N + C::TW - 1) / C::TW;
  const int ntt = (T + C::TT - 1) / C::TT;
  const int nb = nwt * ntt;
  int b = blockIdx.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  // tile order: token tiles fastest, so a band shares few weight tiles
  const int n0 = (b / ntt) * C::TW;
  const int t0 = (b % ntt) * C::TT;

  const int KB = K / 2;
  const int nk = (KB + BKB - 1) / BKB;

  uint4 rw_[C::LW], ra_[C::LA];
  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int c = tid + C::NTH * i;
      const int row = c >> 2;
      const int kb = ks * BKB + (c & 3) * 16;
      const int tn = min(n0 + row, N - 1);
      rw_[i] = kb < KB ? *reinterpret_cast<const uint4*>(w + static_cast<int64_t>(tn) * KB + kb)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::LA; ++i) {
      const int c = tid + C::NTH * i;
      const int row = c >> 2;
      const int kb = ks * BKB + (c & 3) * 16;
      const int ta = min(t0 + row, T - 1);
      ra_[i] = kb < KB ? *reinterpret_cast<const uint4*>(a + static_cast<int64_t>(ta) * KB + kb)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int c = tid + C::NTH * i;
      *reinterpret_cast<uint4*>(&lw[st][(c >> 2) * PITCH + (c & 3) * 16]) = rw_[i];
    }
#pragma unroll
    for (int i = 0; i < C::LA; ++i) {
      const int c = tid + C::NTH * i;
      *reinterpret_cast<uint4*>(&la[st][(c >> 2) * PITCH + (c & 3) * 16]) = ra_[i];
    }
  };

  v16i acc[BW][BT];
#pragma unroll
  for (int i = 0; i < BW; ++i)
#pragma unroll
    for (int j = 0; j < BT; ++j)
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
      v4i w0[BW], w1[BW], a0[BT], a1[BT];
#pragma unroll
      for (int i = 0; i < BW; ++i) {
        const uint4 p = *reinterpret_cast<const uint4*>(
            &lw[st][((ww * BW + i) * 32 + lrow) * PITCH + kk * 32 + lgrp]);
        widen(p, w0[i], w1[i]);
      }
#pragma unroll
      for (int j = 0; j < BT; ++j) {
        const uint4 p = *reinterpret_cast<const uint4*>(
            &la[st][((wt * BT + j) * 32 + lrow) * PITCH + kk * 32 + lgrp]);
        widen(p, a0[j], a1[j]);
      }
#pragma unroll
      for (int i = 0; i < BW; ++i)
#pragma unroll
        for (int j = 0; j < BT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0[i], a0[j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < BW; ++i)
#pragma unroll
        for (int j = 0; j < BT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1[i], a1[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds, for token t = .. + (lane & 31), output columns
  // n = .. + 8*(v/4) + 4*(lane/32) + v%4, v = 0..15
#pragma unroll
  for (int j = 0; j < BT; ++j) {
    const int t = t0 + (wt * BT + j) * 32 + (lane & 31);
    if (t >= T) continue;
    const float sa = I32OUT ? 0.0f : s_a[t];
#pragma unroll
    for (int i = 0; i < BW; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + (ww * BW + i) * 32 + 8 * q + 4 * (lane >> 5);
        int vals[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vals[c] = acc[i][j][4 * q + c] >> 8;
        const int64_t off = static_cast<int64_t>(t) * N + n;
        const bool full = n + 3 < N && (N & 3) == 0;
        if constexpr (I32OUT) {
          int* yp = static_cast<int*>(y) + off;
          if (full) {
            *reinterpret_cast<int4*>(yp) = make_int4(vals[0], vals[1], vals[2], vals[3]);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (n + c < N) yp[c] = vals[c];
          }
        } else {
          uint16_t* yp = static_cast<uint16_t*>(y) + off;
          uint16_t o[4];
          if (full) {
            const float4 sw = *reinterpret_cast<const float4*>(s_w + n);
            o[0] = f32_to_bf16((static_cast<float>(vals[0]) * sa) * sw.x);
            o[1] = f32_to_bf16((static_cast<float>(vals[1]) * sa) * sw.y);
            o[2] = f32_to_bf16((static_cast<float>(vals[2]) * sa) * sw.z);
            o[3] = f32_to_bf16((static_cast<float>(vals[3]) * sa) * sw.w);
            *reinterpret_cast<uint2*>(yp) =
                make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                           o[2] | (static_cast<uint32_t>(o[3]) << 16));
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (n + c < N) yp[c] = f32_to_bf16((static_cast<float>(vals[c]) * sa) * s_w[n + c]);
          }
        }
      }
    }
  }
}

template <int NWW, int NWT, int BW, int BT>
hipError_t launch_cfg(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                      void* y, bool i32_out, int64_t T, int64_t K, int64_t N, hipStream_t s) {
  using C = Cfg<NWW, NWT, BW, BT>;
  const int64_t nb = ((N + C::TW - 1) / C::TW) * ((T + C::TT - 1) / C::TT);
  if (i32_out)
    hipLaunchKernelGGL((gemm_kernel<NWW, NWT, BW, BT, true>), dim3(static_cast<unsigned>(nb)),
                       dim3(C::NTH), 0, s, a, s_a, w, s_w, y, static_cast<int>(T),
                       static_cast<int>(K), static_cast<int>(N));
  else
    hipLaunchKernelGGL((gemm_kernel<NWW, NWT, BW, BT, false>), dim3(static_cast<unsigned>(nb)),
                       dim3(C::NTH), 0, s, a, s_a, w, s_w, y, static_cast<int>(T),
                       static_cast<int>(K), static_cast<int>(N));
  return hipGetLastError();
}

}  // namespace gemm

hipError_t launch_gemm(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                       void* y, bool i32_out, int64_t T, int64_t K, int64_t N, hipStream_t s) {
  if (T == 0) return hipSuccess;
  return gemm::launch_cfg<2, 2, 2, 2>(a, s_a, w, s_w, y, i32_out, T, K, N, s);
}

}  // namespace rw4
