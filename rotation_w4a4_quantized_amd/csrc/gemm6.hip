// W4A4 GEMM on the gfx950 FP6 matrix cores ("Infra Quant II", QuaRot Method:
// INT4 x INT4 products accumulated exactly, then scaled by the activation row
// scale and the weight column scale).
//
// gfx950 has no INT4 matrix instruction. Its f8f6f4 instruction multiplies FP6
// E2M3 operands, and E2M3 holds every integer in [-7, 7] exactly, which is the
// whole range a symmetric absmax INT4 quantizer produces (step absmax / 7). So
// the codes are stored as E2M3 tiles (layout in common.hpp) and the products
// run on v_mfma_scale_f32_32x32x64_f8f6f4 with both block scales 1.0. Every
// product is an integer of magnitude <= 49 and every partial sum an integer of
// magnitude <= 49 K < 2^24 for K <= 131072, so the fp32 accumulation is exact
// and equals the INT32 accumulator. No VALU widening of nibbles is needed, and
// the FP6 rate is twice the int8 rate on this chip.
//
// Each workgroup is one wave computing BW x BT blocks of 32 x 32 outputs (BW
// along the weight rows, BT along the tokens). A fragment (32 rows x 64 codes)
// is one 1536-byte tile, read straight from global memory into registers with
// a 16-byte and an 8-byte load per lane (no LDS in the k-loop); PD tiles per operand are
// in flight. Workgroups are renumbered so that each XCD works on a contiguous
// band of weight tiles. The bf16 epilogue is staged in LDS for 16-byte stores.
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace g6 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// MFMA operand from a lane's two plane loads (elements 6, 7 are not read for FP6)
__device__ __forceinline__ v8i opnd(const uint4& a, const uint2& b) {
  return v8i{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
             static_cast<int>(a.w), static_cast<int>(b.x), static_cast<int>(b.y), 0, 0};
}

template <int BW, int BT, int PD, bool I32OUT>
__global__ void __launch_bounds__(64)
gemm6_kernel(const uint8_t* __restrict__ at, const float* __restrict__ s_a,
             const uint8_t* __restrict__ wt, const float* __restrict__ s_w, void* __restrict__ y,
             int T, int K, int N) {
  constexpr int TW = BW * 32, TT = BT * 32, NF = BW + BT;
  constexpr int SP = TW + 8;  // bf16 stage pitch
  __shared__ __attribute__((aligned(16))) uint16_t stage[I32OUT ? 1 : TT * SP];
  const int lane = threadIdx.x;

  const int nwt = (N + TW - 1) / TW;
  const int ntt = (T + TT - 1) / TT;
  const int nb = nwt * ntt;
  int b = blockIdx.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int n0 = (b / ntt) * TW;
  const int t0 = (b % ntt) * TT;
  const int KT = K >> 6;

  // operand tiles exist for every row of the padded row range (see the
  // tile-size rule of the ABI), so these pointers stay in bounds
  const uint8_t* pf[NF];
#pragma unroll
  for (int i = 0; i < BW; ++i)
    pf[i] = wt + static_cast<int64_t>((n0 >> 5) + i) * KT * kTileBytes;
#pragma unroll
  for (int j = 0; j < BT; ++j)
    pf[BW + j] = at + static_cast<int64_t>((t0 >> 5) + j) * KT * kTileBytes;

  // PD stages of raw fragments per operand, kept as the two planes and
  // assembled into MFMA operands at use
  uint4 r0[PD][NF];
  uint2 r1[PD][NF];
  v16f acc[BW][BT];
#pragma unroll
  for (int i = 0; i < BW; ++i)
#pragma unroll
    for (int j = 0; j < BT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto load = [&](int s, int k) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint8_t* p = pf[f] + static_cast<int64_t>(k) * kTileBytes;
      r0[s][f] = *reinterpret_cast<const uint4*>(p + lane * 16);
      r1[s][f] = *reinterpret_cast<const uint2*>(p + kPlane1 + lane * 8);
    }
  };
  auto mfmas = [&](int s) {
    v8i op[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) op[f] = opnd(r0[s][f], r1[s][f]);
#pragma unroll
    for (int i = 0; i < BW; ++i)
#pragma unroll
      for (int j = 0; j < BT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op[i], op[BW + j], acc[i][j], 2,
                                                                    2, 0, 127, 0, 127);
  };

#pragma unroll
  for (int s = 0; s < PD; ++s) load(s, s < KT ? s : KT - 1);
  // full groups of PD sub-steps: MFMAs on stage s, then refill stage s
  int kt = 0;
  for (; kt + PD <= KT; kt += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s);
      load(s, kt + s + PD < KT ? kt + s + PD : KT - 1);
    }
  }
  // the last KT % PD sub-steps: stage s already holds k-tile kt + s
  const int rem = KT - kt;
#pragma unroll
  for (int s = 0; s < PD - 1; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    if (s < rem) mfmas(s);  // uniform; no load inside
  }
  // results of the last MFMAs are read by plain VALU code below
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_sched_barrier(0);

  // accumulator element (i, j, v): weight row n0 + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4,
  // token t0 + 32 j + lane % 32
  if constexpr (I32OUT) {
    int32_t* yo = static_cast<int32_t*>(y);
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      const int t = t0 + 32 * j + (lane & 31);
      if (t >= T) continue;
#pragma unroll
      for (int i = 0; i < BW; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + 32 * i + 8 * q + 4 * (lane >> 5);
          int32_t* o = yo + static_cast<int64_t>(t) * N + n;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (n + c < N) o[c] = static_cast<int32_t>(acc[i][j][4 * q + c]);
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      const int tl = 32 * j + (lane & 31);
      const float sa = s_a[min(t0 + tl, T - 1)];
#pragma unroll
      for (int i = 0; i < BW; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = 32 * i + 8 * q + 4 * (lane >> 5);
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = (acc[i][j][4 * q + c] * sa) * s_w[min(n0 + nl + c, N - 1)];
          *reinterpret_cast<uint2*>(&stage[tl * SP + nl]) =
              make_uint2(f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
                         f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16));
        }
    }
    __syncthreads();
    uint16_t* yo = static_cast<uint16_t*>(y);
    constexpr int CPR = TW / 8;
    for (int c = lane; c < TT * CPR; c += 64) {
      const int row = c / CPR, col = (c % CPR) * 8;
      const int t = t0 + row, n = n0 + col;
      if (t >= T || n >= N) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(&stage[row * SP + col]);
      uint16_t* o = yo + static_cast<int64_t>(t) * N + n;
      if (n + 8 <= N && (N & 7) == 0) {
        *reinterpret_cast<uint4*>(o) = v;
      } else {
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&stage[row * SP + col]);
        for (int k = 0; k < 8 && n + k < N; ++k) o[k] = e[k];
      }
    }
  }
}

// INT4 rows [R][K/2] -> FP6 tiles of Rp rows (rows >= R get code 0); one
// thread per 12-byte field group. A code of -8 (not representable) is stored
// as 0 and raises *bad.
__global__ void __launch_bounds__(256)
tile_kernel(const uint8_t* __restrict__ codes, int64_t R, int64_t Rp, int64_t K,
            uint8_t* __restrict__ tiles, int* __restrict__ bad) {
  const int64_t groups = Rp * (K / 16);
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= groups) return;
  const int64_t row = g / (K / 16);
  const int64_t k0 = (g % (K / 16)) * 16;
  // unconditional load (row clamped), masked afterwards
  const bool live = row < R;
  const uint2 p = *reinterpret_cast<const uint2*>(codes + (live ? row : R - 1) * (K / 2) + k0 / 2);
  float f[16];
  bool neg8 = false;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t w = e < 8 ? p.x : p.y;
    int q = static_cast<int>((w >> (4 * (e & 7))) & 15u);
    q = live ? (q >= 8 ? q - 16 : q) : 0;
    neg8 |= q == -8;
    f[e] = q == -8 ? 0.0f : static_cast<float>(q);
  }
  store_fields16(tiles, row, k0, K, pack_fp6_16(f));
  if (neg8 && bad) atomicOr(bad, 1);
}

template <int BW, int BT, int PD, bool I32>
hipError_t launch_cfg(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                      void* y, int64_t T, int64_t K, int64_t N, hipStream_t s) {
  const int64_t nb = ((N + BW * 32 - 1) / (BW * 32)) * ((T + BT * 32 - 1) / (BT * 32));
  if (nb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gemm6_kernel<BW, BT, PD, I32>), dim3(static_cast<unsigned>(nb)), dim3(64), 0,
                     s, a, s_a, w, s_w, y, static_cast<int>(T), static_cast<int>(K),
                     static_cast<int>(N));
  return hipGetLastError();
}

}  // namespace g6

int64_t tiles_rows(int64_t R) { return (R + 255) / 256 * 256; }

size_t tiles_bytes(int64_t R, int64_t K) {
  return static_cast<size_t>(tiles_rows(R)) * static_cast<size_t>(K) * 3 / 4;
}

hipError_t launch_tile_codes(const uint8_t* codes, int64_t R, int64_t K, uint8_t* tiles, int* bad,
                             hipStream_t s) {
  const int64_t Rp = tiles_rows(R);
  const int64_t groups = Rp * (K / 16);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(g6::tile_kernel, dim3(static_cast<unsigned>((groups + 255) / 256)), dim3(256),
                     0, s, codes, R, Rp, K, tiles, bad);
  return hipGetLastError();
}

hipError_t launch_gemm_tiles(const uint8_t* a, const float* s_a, const uint8_t* w,
                             const float* s_w, void* y, bool i32_out, int64_t T, int64_t K,
                             int64_t N, hipStream_t s) {
  if (T == 0 || N == 0) return hipSuccess;
  const bool big = T >= 4096 && N >= 4096;
  if (i32_out)
    return big ? g6::launch_cfg<4, 4, 2, true>(a, s_a, w, s_w, y, T, K, N, s)
               : g6::launch_cfg<4, 2, 4, true>(a, s_a, w, s_w, y, T, K, N, s);
  return big ? g6::launch_cfg<4, 4, 2, false>(a, s_a, w, s_w, y, T, K, N, s)
             : g6::launch_cfg<4, 2, 4, false>(a, s_a, w, s_w, y, T, K, N, s);
}

}  // namespace rw4
