// Low-rank residual alignment ("ReSpinQuant" paper notes, key designs 2 and 3):
//   out[t] = x[t] + Q ((M - I) (Q^T x[t]))  (+ addend[t])
// three steps, no D x D product: project to r dims, apply the small matrix,
// lift and add.
//
// One workgroup (256 threads) aligns a block of TB tokens so that every Q row
// it streams from L2 is used TB times.
//   A: y = Q^T x. Thread (jq, dq) owns 4 columns of Q (float4) and every
//      ndq-th row of the current D chunk; the token chunk is staged in LDS as
//      fp32. Partial sums over dq are reduced through LDS.
//   B: z = (M - I) y, the identity subtracted from M's diagonal as it is read.
//   C: thread per output element d: out[t][d] = x[t][d] + Q[d,:] . z[t]; Q's row
//      is read once for all TB tokens.
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

constexpr int TB = 8;        // tokens per workgroup
constexpr int NT = 256;      // threads
constexpr int CH = 512;      // D-chunk staged in LDS
constexpr int RMAX = 128;

template <bool XF32, bool OF32, bool ADD>
__global__ void __launch_bounds__(NT)
align_kernel(const void* __restrict__ x, void* __restrict__ out, const float* __restrict__ Q,
             const float* __restrict__ M, const void* __restrict__ addend, int64_t T, int D,
             int r) {
  __shared__ float xs[TB][CH];
  __shared__ float part[8192];                 // ndq * TB * r <= 8192
  __shared__ float ys[TB][RMAX];
  __shared__ float zs[TB][RMAX];

  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int nt = static_cast<int>(T - t0 < TB ? T - t0 : TB);

  auto xval = [&](int tt, int d) -> float {
    const int64_t o = (t0 + tt) * static_cast<int64_t>(D) + d;
    if constexpr (XF32) return static_cast<const float*>(x)[o];
    else return bf16_to_f32(static_cast<const uint16_t*>(x)[o]);
  };

  if (r > 0) {
    const int RQ = r / 4;
    const int ndq = NT / RQ;
    const int jq = tid % RQ;
    const int dq = tid / RQ;
    float acc[TB][4];
#pragma unroll
    for (int i = 0; i < TB; ++i) acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.0f;

    for (int d0 = 0; d0 < D; d0 += CH) {
      const int cl = D - d0 < CH ? D - d0 : CH;
      // stage x[t0 .. t0+TB)[d0 .. d0+cl) as fp32 (8 values per step)
      for (int e = tid; e < TB * (cl / 8); e += NT) {
        const int tt = e / (cl / 8);
        const int c8 = (e % (cl / 8)) * 8;
        float vv[8];
        if (tt < nt) {
          const int64_t o = (t0 + tt) * static_cast<int64_t>(D) + d0 + c8;
          if constexpr (XF32) {
            const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + o);
            const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + o + 4);
            vv[0] = a.x; vv[1] = a.y; vv[2] = a.z; vv[3] = a.w;
            vv[4] = b.x; vv[5] = b.y; vv[6] = b.z; vv[7] = b.w;
          } else {
            const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + o);
            vv[0] = bf16lo(q.x); vv[1] = bf16hi(q.x); vv[2] = bf16lo(q.y); vv[3] = bf16hi(q.y);
            vv[4] = bf16lo(q.z); vv[5] = bf16hi(q.z); vv[6] = bf16lo(q.w); vv[7] = bf16hi(q.w);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) vv[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) xs[tt][c8 + i] = vv[i];
      }
      __syncthreads();
      if (dq < ndq) {
        for (int dd = dq; dd < cl; dd += ndq) {
          const float4 q = *reinterpret_cast<const float4*>(Q + static_cast<int64_t>(d0 + dd) * r + 4 * jq);
#pragma unroll
          for (int tt = 0; tt < TB; ++tt) {
            const float xv = xs[tt][dd];
            acc[tt][0] = fmaf(xv, q.x, acc[tt][0]);
            acc[tt][1] = fmaf(xv, q.y, acc[tt][1]);
            acc[tt][2] = fmaf(xv, q.z, acc[tt][2]);
            acc[tt][3] = fmaf(xv, q.w, acc[tt][3]);
          }
        }
      }
      __syncthreads();
    }
    if (dq < ndq) {
#pragma unroll
      for (int tt = 0; tt < TB; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) part[(dq * TB + tt) * r + 4 * jq + c] = acc[tt][c];
    }
    __syncthreads();
    for (int o = tid; o < TB * r; o += NT) {
      const int tt = o / r;
      const int j = o % r;
      float s = 0.0f;
      for (int k = 0; k < ndq; ++k) s += part[(k * TB + tt) * r + j];
      ys[tt][j] = s;
    }
    __syncthreads();
    for (int o = tid; o < TB * r; o += NT) {
      const int tt = o / r;
      const int i = o % r;
      float s = 0.0f;
      for (int j = 0; j < r; ++j) {
        float mij = M[i * r + j];
        if (i == j) mij -= 1.0f;
        s = fmaf(mij, ys[tt][j], s);
      }
      zs[tt][i] = s;
    }
    __syncthreads();
  }

  for (int d = tid; d < D; d += NT) {
    float corr[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) corr[tt] = 0.0f;
    for (int j = 0; j < r; j += 4) {
      const float4 q = *reinterpret_cast<const float4*>(Q + static_cast<int64_t>(d) * r + j);
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        float c = corr[tt];
        c = fmaf(q.x, zs[tt][j], c);
        c = fmaf(q.y, zs[tt][j + 1], c);
        c = fmaf(q.z, zs[tt][j + 2], c);
        c = fmaf(q.w, zs[tt][j + 3], c);
        corr[tt] = c;
      }
    }
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      if (tt >= nt) break;
      float o = xval(tt, d) + corr[tt];
      const int64_t off = (t0 + tt) * static_cast<int64_t>(D) + d;
      if constexpr (ADD) {
        if constexpr (OF32) o += static_cast<const float*>(addend)[off];
        else o += bf16_to_f32(static_cast<const uint16_t*>(addend)[off]);
      }
      if constexpr (OF32) static_cast<float*>(out)[off] = o;
      else static_cast<uint16_t*>(out)[off] = f32_to_bf16(o);
    }
  }
}

template <bool XF32, bool OF32, bool ADD>
hipError_t go(const void* x, void* out, const float* Q, const float* M, const void* addend,
              int64_t T, int64_t D, int64_t r, hipStream_t s) {
  const int64_t blocks = (T + TB - 1) / TB;
  hipLaunchKernelGGL((align_kernel<XF32, OF32, ADD>), dim3(static_cast<unsigned>(blocks)), dim3(NT),
                     0, s, x, out, Q, M, addend, T, static_cast<int>(D), static_cast<int>(r));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_align(const void* x, int x_f32, void* out, int out_f32, const float* Q,
                        const float* M, const void* addend, int64_t T, int64_t D, int64_t r,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool add = addend != nullptr;
#define RW4_AL(XF, OF, AD) \
  if (!!x_f32 == XF && !!out_f32 == OF && add == AD) return go<XF, OF, AD>(x, out, Q, M, addend, T, D, r, s);
  RW4_AL(false, false, false) RW4_AL(false, false, true) RW4_AL(false, true, false)
  RW4_AL(false, true, true) RW4_AL(true, false, false) RW4_AL(true, false, true)
  RW4_AL(true, true, false) RW4_AL(true, true, true)
#undef RW4_AL
  return hipErrorInvalidValue;
}

}  // namespace rw4
