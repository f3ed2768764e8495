// Short-batch alignment projection, shared by the alignment's own launch and
// by the quantizer that runs it beside its rows ("ReSpinQuant" paper notes,
// key design 3: z = (M - I) Q^T x, here per 256-column chunk of D).
#pragma once
#include "common.hpp"

namespace rw4 {

constexpr int kSmallT = 16;       // tokens of a short batch at most
constexpr int kSmallChunk = 256;  // columns per projection workgroup

// One workgroup of 256 threads per 256-column chunk c: Zs[c][t][i] = sum over
// the chunk of Q'[i][d] x[t][d], Q' = Q'h + Q'l (exact in fp32), fp32 FMA in
// column order; x and 32-row blocks of Q' are staged in LDS. Every thread of
// the workgroup must call it (it has workgroup barriers).
__device__ __forceinline__ void asmall_proj_body(int c, const uint16_t* __restrict__ x, int T, int D,
                                                 int RP, int RK, const uint16_t* __restrict__ QtH,
                                                 const uint16_t* __restrict__ QtL,
                                                 float* __restrict__ Zs) {
  __shared__ __attribute__((aligned(16))) float xs[kSmallT][kSmallChunk + 4];
  __shared__ __attribute__((aligned(16))) float qs[32][kSmallChunk + 4];
  const int tid = threadIdx.x;
  const int d0 = c * kSmallChunk;
  const int nd = min(kSmallChunk, D - d0);           // a multiple of 64
  const bool col = tid < nd;
  const int dc = d0 + (col ? tid : nd - 1);
  // thread tid stages column d0 + tid of every token; the loads are
  // unconditional (clamped token and column, masked values), so that they
  // are all in flight before the first use
  // rows i0 .. i0 + 31 of Q' for this chunk, one column per thread; the first
  // block's loads go out ahead of x's, so that the thread waits for memory once
  uint16_t hr[32], lr[32];
  auto loadq = [&](int i0) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int64_t o = static_cast<int64_t>(min(i0 + k, RP - 1)) * D + dc;
      hr[k] = QtH[o];
      lr[k] = QtL[o];
    }
  };
  loadq(0);
  uint16_t xr[kSmallT];
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) xr[t] = x[static_cast<int64_t>(min(t, T - 1)) * D + dc];
  for (int i0 = 0; i0 < RK; i0 += 32) {
    if (i0 > 0) loadq(i0);
    float qv[32];
#pragma unroll
    for (int k = 0; k < 32; ++k)
      qv[k] = col && i0 + k < RP ? bf16_to_f32(hr[k]) + bf16_to_f32(lr[k]) : 0.0f;
    if (i0 == 0) {
      // x goes to LDS only now, so that no use of it comes before the Q' loads
#pragma unroll
      for (int t = 0; t < kSmallT; ++t) xs[t][tid] = col && t < T ? bf16_to_f32(xr[t]) : 0.0f;
    }
    __syncthreads();                                 // previous block's readers are done
#pragma unroll
    for (int k = 0; k < 32; ++k) qs[k][tid] = qv[k];
    __syncthreads();
    for (int o = tid; o < T * 32; o += 256) {
      const int t = o >> 5, k = o & 31;
      float acc = 0.0f;
#pragma unroll 4
      for (int d = 0; d < kSmallChunk; d += 4) {
        const float4 q4 = *reinterpret_cast<const float4*>(&qs[k][d]);
        const float4 x4 = *reinterpret_cast<const float4*>(&xs[t][d]);
        acc = fmaf(q4.x, x4.x, acc);
        acc = fmaf(q4.y, x4.y, acc);
        acc = fmaf(q4.z, x4.z, acc);
        acc = fmaf(q4.w, x4.w, acc);
      }
      Zs[(static_cast<int64_t>(c) * T + t) * RK + i0 + k] = acc;
    }
  }
}


}  // namespace rw4
