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
// the weight rows, BT along the tokens). K advances 256 codes (128 bytes) per
// step through double-buffered LDS holding the packed codes (row pitch 144
// bytes), global loads running two steps ahead and each 64-code fragment read
// from LDS one sub-step before its MFMAs. MFMA A = weight rows, B = token rows, so each lane's accumulators
// hold 4 consecutive output columns of one token (8-byte bf16 stores).
// Workgroups are renumbered so that the eight XCDs (which receive workgroups
// round-robin) each work on a contiguous band of weight tiles.
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace gemm {

constexpr int BKB = 128;    // packed bytes per k-step (256 codes), one barrier each
constexpr int PITCH = 144;  // LDS row pitch (bytes): 128 + 16 keeps 16-lane b128 reads conflict-free
constexpr int KSUB = BKB / 32;  // 64-code sub-steps per k-step (two MFMAs each)

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
  static constexpr int CPR = BKB / 16;            // 16-byte chunks per row per k-step
  static constexpr int LW = TW * CPR / NTH;       // chunks per thread per k-step
  static constexpr int LA = TT * CPR / NTH;
  static_assert(LW >= 1 && LA >= 1 && TW * CPR % NTH == 0 && TT * CPR % NTH == 0, "tile/threads");
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

  // per-thread global source rows (clamped: rows past T or N load valid
  // memory and only feed outputs that are never stored)
  const uint8_t* gw[C::LW];
  const uint8_t* ga[C::LA];
  int cw[C::LW], ca[C::LA];
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int c = tid + C::NTH * i;
    cw[i] = (c % C::CPR) * 16;
    gw[i] = w + static_cast<int64_t>(min(n0 + c / C::CPR, N - 1)) * KB + cw[i];
  }
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int c = tid + C::NTH * i;
    ca[i] = (c % C::CPR) * 16;
    ga[i] = a + static_cast<int64_t>(min(t0 + c / C::CPR, T - 1)) * KB + ca[i];
  }
  uint4 rw_[C::LW], ra_[C::LA];
  // loads are unconditional (no exec-masked branches around them): chunks
  // past the end of K read the row's first chunk and are zeroed by a mask
  auto gload = [&](int ks) {
    const int kb = ks * BKB;
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const bool ok = kb + cw[i] < KB;
      uint4 v = *reinterpret_cast<const uint4*>(gw[i] + (ok ? kb : -cw[i]));
      const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
      v.x &= m; v.y &= m; v.z &= m; v.w &= m;
      rw_[i] = v;
    }
#pragma unroll
    for (int i = 0; i < C::LA; ++i) {
      const bool ok = kb + ca[i] < KB;
      uint4 v = *reinterpret_cast<const uint4*>(ga[i] + (ok ? kb : -ca[i]));
      const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
      v.x &= m; v.y &= m; v.z &= m; v.w &= m;
      ra_[i] = v;
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int c = tid + C::NTH * i;
      *reinterpret_cast<uint4*>(&lw[st][(c / C::CPR) * PITCH + cw[i]]) = rw_[i];
    }
#pragma unroll
    for (int i = 0; i < C::LA; ++i) {
      const int c = tid + C::NTH * i;
      *reinterpret_cast<uint4*>(&la[st][(c / C::CPR) * PITCH + ca[i]]) = ra_[i];
    }
  };

  v16i acc[BW][BT];
#pragma unroll
  for (int i = 0; i < BW; ++i)
#pragma unroll
    for (int j = 0; j < BT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  const int lrow = lane & 31;
  const int lgrp = (lane >> 5) * 16;
  const int wofs = ((ww * BW) * 32 + lrow) * PITCH + lgrp;
  const int aofs = ((wt * BT) * 32 + lrow) * PITCH + lgrp;
  auto frags = [&](int st, int kk, uint4 (&pw)[BW], uint4 (&pa)[BT]) {
#pragma unroll
    for (int i = 0; i < BW; ++i)
      pw[i] = *reinterpret_cast<const uint4*>(&lw[st][wofs + i * 32 * PITCH + kk * 32]);
#pragma unroll
    for (int j = 0; j < BT; ++j)
      pa[j] = *reinterpret_cast<const uint4*>(&la[st][aofs + j * 32 * PITCH + kk * 32]);
  };

  gload(0);
  lstore(0);
  if (nk > 1) gload(1);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    uint4 pw[BW], pa[BT];
    frags(st, 0, pw, pa);
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      uint4 qw[BW], qa[BT];
      if (kk + 1 < KSUB) frags(st, kk + 1, qw, qa);
      v4i w0[BW], w1[BW], a0[BT], a1[BT];
#pragma unroll
      for (int i = 0; i < BW; ++i) widen(pw[i], w0[i], w1[i]);
#pragma unroll
      for (int j = 0; j < BT; ++j) widen(pa[j], a0[j], a1[j]);
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
      if (kk + 1 < KSUB) {
#pragma unroll
        for (int i = 0; i < BW; ++i) pw[i] = qw[i];
#pragma unroll
        for (int j = 0; j < BT; ++j) pa[j] = qa[j];
      }
    }
    if (ks + 1 < nk) lstore(st ^ 1);
    __syncthreads();
    if (ks + 2 < nk) gload(ks + 2);
  }

  // epilogue: lane holds, for token t = .. + (lane & 31), output columns
  // n = .. + 8*(v/4) + 4*(lane/32) + v%4, v = 0..15
  if constexpr (!I32OUT) {
    // bf16 results go through LDS (the k-loop buffers are free now) so that the
    // tile is written as whole contiguous row segments: 16 lanes per 256 bytes
    constexpr int SP = C::TW + 8;                       // staging row pitch (bf16)
    static_assert(C::TT * SP * 2 <= 2 * (C::TW + C::TT) * PITCH, "staging fits the k-loop LDS");
    uint16_t* stage = reinterpret_cast<uint16_t*>(&lw[0][0]);
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      const int tt = (wt * BT + j) * 32 + (lane & 31);
      const float sa = s_a[min(t0 + tt, T - 1)];
#pragma unroll
      for (int i = 0; i < BW; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nn = (ww * BW + i) * 32 + 8 * q + 4 * (lane >> 5);
          // clamped, unconditional scale loads (columns past N are never stored)
          float swv[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) swv[c] = s_w[min(n0 + nn + c, N - 1)];
          uint16_t o[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            o[c] = f32_to_bf16((static_cast<float>(acc[i][j][4 * q + c] >> 8) * sa) * swv[c]);
          *reinterpret_cast<uint2*>(&stage[tt * SP + nn]) =
              make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
        }
      }
    }
    __syncthreads();
    constexpr int CPRW = C::TW / 8;                     // 16-byte chunks per staged row
    uint16_t* yb = static_cast<uint16_t*>(y);
    for (int c = tid; c < C::TT * CPRW; c += C::NTH) {
      const int tt = c / CPRW;
      const int nn = (c % CPRW) * 8;
      const int t = t0 + tt;
      const int n = n0 + nn;
      if (t >= T) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(&stage[tt * SP + nn]);
      uint16_t* yp = yb + static_cast<int64_t>(t) * N + n;
      if (n + 7 < N && (N & 7) == 0) {
        *reinterpret_cast<uint4*>(yp) = v;
      } else {
        const uint16_t e[8] = {static_cast<uint16_t>(v.x), static_cast<uint16_t>(v.x >> 16),
                               static_cast<uint16_t>(v.y), static_cast<uint16_t>(v.y >> 16),
                               static_cast<uint16_t>(v.z), static_cast<uint16_t>(v.z >> 16),
                               static_cast<uint16_t>(v.w), static_cast<uint16_t>(v.w >> 16)};
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (n + k < N) yp[k] = e[k];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      const int t = t0 + (wt * BT + j) * 32 + (lane & 31);
      if (t >= T) continue;
#pragma unroll
      for (int i = 0; i < BW; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (ww * BW + i) * 32 + 8 * q + 4 * (lane >> 5);
          int vals[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) vals[c] = acc[i][j][4 * q + c] >> 8;
          int* yp = static_cast<int*>(y) + static_cast<int64_t>(t) * N + n;
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<int4*>(yp) = make_int4(vals[0], vals[1], vals[2], vals[3]);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (n + c < N) yp[c] = vals[c];
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
