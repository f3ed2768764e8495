// Low-rank residual alignment on bf16 matrix cores ("ReSpinQuant" paper notes,
// key design 3: y = Q^T x, z = (M - I) y, out = x + Q z).
//
// The activations are bf16, so x is exact as an MFMA operand. Q is split once
// per call into two bf16 terms, Q = Qh + Ql + O(2^-17 |Q|), and z likewise:
//   y   = x.Qh + x.Ql                      (two bf16 products, fp32 accumulate)
//   out = x + Qh.zh + Ql.zh + Qh.zl        (the dropped Ql.zl is ~2^-17 relative)
// which keeps the fp32 alignment well inside a 1e-5 normwise error while
// running on v_mfma_f32_16x16x32_bf16 instead of fp32 FMAs. With M = I, z is
// exactly zero and the output equals the input.
//
// Three launches, each over (token block of 16) x (D part of <= 512):
//   prep : Qh/Ql in both orientations ([r][D] for the projection, [D][r] for
//          the lift), zero-padded in r; M - I in fp32.
//   yproj: partial y over one D part (four waves split the part's 32-wide
//          k-steps, reduced through LDS) -> Ypart[part][t][j].
//   lift : sums the parts, forms z = (M - I) y and its bf16 split in LDS, then
//          out = x + Q z for its D part. The MFMA's row order is permuted so a
//          lane's accumulator covers the same 8 consecutive columns of one
//          token that its 16-byte x load holds: the accumulator starts as x.
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int TB = 16;          // tokens per workgroup (MFMA rows)
constexpr int NW = 4;           // waves per workgroup

__device__ __forceinline__ v8bf ld8(const uint16_t* p) { return *reinterpret_cast<const v8bf*>(p); }

__device__ __forceinline__ v4f mfma(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ void __launch_bounds__(256)
basis_prep_kernel(const float* __restrict__ Q, const float* __restrict__ M, int D, int r, int RP,
                  int RK, uint16_t* __restrict__ QtH, uint16_t* __restrict__ QtL,
                  uint16_t* __restrict__ QH, uint16_t* __restrict__ QL, float* __restrict__ Mm) {
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = tid; i < static_cast<int64_t>(D) * RK; i += nthreads) {
    const int d = static_cast<int>(i / RK);
    const int j = static_cast<int>(i % RK);
    const float q = j < r ? Q[static_cast<int64_t>(d) * r + j] : 0.0f;
    const uint16_t h = f32_to_bf16(q);
    QH[i] = h;
    QL[i] = f32_to_bf16(q - bf16_to_f32(h));
  }
  for (int64_t i = tid; i < static_cast<int64_t>(D) * RP; i += nthreads) {
    const int j = static_cast<int>(i / D);
    const int d = static_cast<int>(i % D);
    const float q = j < r ? Q[static_cast<int64_t>(d) * r + j] : 0.0f;
    const uint16_t h = f32_to_bf16(q);
    QtH[i] = h;
    QtL[i] = f32_to_bf16(q - bf16_to_f32(h));
  }
  for (int64_t i = tid; i < static_cast<int64_t>(r) * r; i += nthreads) {
    const int a = static_cast<int>(i / r);
    const int b = static_cast<int>(i % r);
    Mm[i] = a == b ? M[i] - 1.0f : M[i];
  }
}

template <int RP>
__global__ void __launch_bounds__(256)
yproj_kernel(const uint16_t* __restrict__ x, int64_t T, int D, int P,
             const uint16_t* __restrict__ QtH, const uint16_t* __restrict__ QtL,
             float* __restrict__ Ypart) {
  __shared__ float red[NW][TB][RP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int part = blockIdx.y;
  const int dbeg = part * P;
  const int dend = min(D, dbeg + P);
  const int nks = (dend - dbeg) / 32;
  const int g = lane >> 4;
  const int tl = lane & 15;
  const int64_t trow = min(t0 + tl, T - 1);
  const uint16_t* xrow = x + trow * D + 8 * g;

  v4f acc[RP / 16];
#pragma unroll
  for (int nb = 0; nb < RP / 16; ++nb) acc[nb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int ks = wave; ks < nks; ks += NW) {
    const int d0 = dbeg + 32 * ks;
    const v8bf a = ld8(xrow + d0);
#pragma unroll
    for (int nb = 0; nb < RP / 16; ++nb) {
      const int64_t qo = static_cast<int64_t>(16 * nb + tl) * D + d0 + 8 * g;
      acc[nb] = mfma(a, ld8(QtH + qo), acc[nb]);
      acc[nb] = mfma(a, ld8(QtL + qo), acc[nb]);
    }
  }
  // C layout: lane holds rows 4g + v (tokens), column tl (basis index in the block)
#pragma unroll
  for (int nb = 0; nb < RP / 16; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * g + v][16 * nb + tl] = acc[nb][v];
  __syncthreads();
  for (int o = tid; o < TB * RP; o += 256) {
    const int t = o / RP;
    const int j = o % RP;
    if (t0 + t < T) {
      const float s = (red[0][t][j] + red[1][t][j]) + (red[2][t][j] + red[3][t][j]);
      Ypart[(static_cast<int64_t>(part) * T + t0 + t) * RP + j] = s;
    }
  }
}

template <int RP, int RK, bool OF32, bool ADD>
__global__ void __launch_bounds__(256)
lift_kernel(const uint16_t* __restrict__ x, int64_t T, int D, int P, int S, int r,
            const float* __restrict__ Ypart, const float* __restrict__ Mm,
            const uint16_t* __restrict__ QH, const uint16_t* __restrict__ QL,
            const void* __restrict__ addend, void* __restrict__ out) {
  __shared__ float ys[TB][RP];
  __shared__ __attribute__((aligned(16))) uint16_t zh[TB][RK];
  __shared__ __attribute__((aligned(16))) uint16_t zl[TB][RK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int part = blockIdx.y;
  const int dbeg = part * P;
  const int dend = min(D, dbeg + P);
  const int nks = (dend - dbeg) / 32;

  for (int o = tid; o < TB * RP; o += 256) {
    const int t = o / RP;
    const int j = o % RP;
    float s = 0.0f;
    if (t0 + t < T)
      for (int p = 0; p < S; ++p) s += Ypart[(static_cast<int64_t>(p) * T + t0 + t) * RP + j];
    ys[t][j] = s;
  }
  __syncthreads();
  for (int o = tid; o < TB * RK; o += 256) {
    const int t = o / RK;
    const int i = o % RK;
    float z = 0.0f;
    if (i < r)
      for (int j = 0; j < r; ++j) z = fmaf(Mm[i * r + j], ys[t][j], z);
    const uint16_t h = f32_to_bf16(z);
    zh[t][i] = h;
    zl[t][i] = f32_to_bf16(z - bf16_to_f32(h));
  }
  __syncthreads();

  const int g = lane >> 4;
  const int tl = lane & 15;
  const int64_t t = t0 + tl;
  const int64_t trow = min(t, T - 1);
  const uint16_t* xrow = x + trow * D + 8 * g;
  for (int ks = wave; ks < nks; ks += NW) {
    const int d0 = dbeg + 32 * ks;
    const uint4 xv = *reinterpret_cast<const uint4*>(xrow + d0);
    v4f acc[2];
    acc[0] = v4f{bf16lo(xv.x), bf16hi(xv.x), bf16lo(xv.y), bf16hi(xv.y)};
    acc[1] = v4f{bf16lo(xv.z), bf16hi(xv.z), bf16lo(xv.w), bf16hi(xv.w)};
#pragma unroll
    for (int kk = 0; kk < RK / 32; ++kk) {
      const v8bf bh = *reinterpret_cast<const v8bf*>(&zh[tl][32 * kk + 8 * g]);
      const v8bf bl = *reinterpret_cast<const v8bf*>(&zl[tl][32 * kk + 8 * g]);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int drow = d0 + 8 * (tl >> 2) + 4 * b + (tl & 3);
        const int64_t qo = static_cast<int64_t>(drow) * RK + 32 * kk + 8 * g;
        const v8bf ah = ld8(QH + qo);
        const v8bf al = ld8(QL + qo);
        acc[b] = mfma(ah, bh, acc[b]);
        acc[b] = mfma(al, bh, acc[b]);
        acc[b] = mfma(ah, bl, acc[b]);
      }
    }
    if (t < T) {
      const int64_t off = t * D + d0 + 8 * g;
      float o[8] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3],
                    acc[1][0], acc[1][1], acc[1][2], acc[1][3]};
      if constexpr (ADD) {
        if constexpr (OF32) {
          const float4 a0 = *reinterpret_cast<const float4*>(static_cast<const float*>(addend) + off);
          const float4 a1 = *reinterpret_cast<const float4*>(static_cast<const float*>(addend) + off + 4);
          o[0] += a0.x; o[1] += a0.y; o[2] += a0.z; o[3] += a0.w;
          o[4] += a1.x; o[5] += a1.y; o[6] += a1.z; o[7] += a1.w;
        } else {
          const uint4 av = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(addend) + off);
          o[0] += bf16lo(av.x); o[1] += bf16hi(av.x); o[2] += bf16lo(av.y); o[3] += bf16hi(av.y);
          o[4] += bf16lo(av.z); o[5] += bf16hi(av.z); o[6] += bf16lo(av.w); o[7] += bf16hi(av.w);
        }
      }
      if constexpr (OF32) {
        float* op = static_cast<float*>(out) + off;
        reinterpret_cast<float4*>(op)[0] = make_float4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<float4*>(op)[1] = make_float4(o[4], o[5], o[6], o[7]);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = f32_to_bf16(o[2 * i]) | (static_cast<uint32_t>(f32_to_bf16(o[2 * i + 1])) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + off) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

inline int rp_of(int64_t r) { return static_cast<int>((r + 15) / 16 * 16); }
inline int rk_of(int64_t r) { return static_cast<int>((r + 31) / 32 * 32); }
inline size_t a256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }
constexpr int kPart = 512;

template <int RP>
hipError_t run_yproj(const uint16_t* x, int64_t T, int D, int P, int S, const uint16_t* QtH,
                     const uint16_t* QtL, float* Ypart, hipStream_t s) {
  hipLaunchKernelGGL(yproj_kernel<RP>, dim3(static_cast<unsigned>((T + TB - 1) / TB), S), dim3(256),
                     0, s, x, T, D, P, QtH, QtL, Ypart);
  return hipGetLastError();
}

template <int RP, int RK>
hipError_t run_lift(const uint16_t* x, int64_t T, int D, int P, int S, int r, const float* Ypart,
                    const float* Mm, const uint16_t* QH, const uint16_t* QL, const void* addend,
                    void* out, bool of32, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T + TB - 1) / TB), S);
#define RW4_LIFT(OF, AD)                                                                         \
  if (of32 == OF && (addend != nullptr) == AD) {                                                 \
    hipLaunchKernelGGL((lift_kernel<RP, RK, OF, AD>), grid, dim3(256), 0, s, x, T, D, P, S, r,   \
                       Ypart, Mm, QH, QL, addend, out);                                          \
    return hipGetLastError();                                                                    \
  }
  RW4_LIFT(true, false) RW4_LIFT(true, true) RW4_LIFT(false, false) RW4_LIFT(false, true)
#undef RW4_LIFT
  return hipErrorInvalidValue;
}

}  // namespace

bool align_mfma_supported(int64_t D, int64_t r) { return r > 0 && r <= 128 && D % 32 == 0; }

size_t align_mfma_workspace(int64_t T, int64_t D, int64_t r) {
  const int RP = rp_of(r), RK = rk_of(r);
  const int64_t S = (D + kPart - 1) / kPart;
  return 2 * a256(static_cast<size_t>(RP) * D * 2) + 2 * a256(static_cast<size_t>(D) * RK * 2) +
         a256(static_cast<size_t>(r) * r * 4) + a256(static_cast<size_t>(S) * T * RP * 4);
}

hipError_t launch_align_mfma(const uint16_t* x, void* out, int out_f32, const float* Q,
                             const float* M, const void* addend, int64_t T, int64_t D, int64_t r,
                             void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int RP = rp_of(r), RK = rk_of(r);
  const int P = static_cast<int>(D < kPart ? D : kPart);
  const int S = static_cast<int>((D + P - 1) / P);
  uint8_t* p = static_cast<uint8_t*>(ws);
  uint16_t* QtH = reinterpret_cast<uint16_t*>(p); p += a256(static_cast<size_t>(RP) * D * 2);
  uint16_t* QtL = reinterpret_cast<uint16_t*>(p); p += a256(static_cast<size_t>(RP) * D * 2);
  uint16_t* QH = reinterpret_cast<uint16_t*>(p);  p += a256(static_cast<size_t>(D) * RK * 2);
  uint16_t* QL = reinterpret_cast<uint16_t*>(p);  p += a256(static_cast<size_t>(D) * RK * 2);
  float* Mm = reinterpret_cast<float*>(p);        p += a256(static_cast<size_t>(r) * r * 4);
  float* Ypart = reinterpret_cast<float*>(p);

  const int64_t work = D * RK;
  const unsigned pblocks = static_cast<unsigned>(work / 256 < 1024 ? (work + 255) / 256 : 1024);
  hipLaunchKernelGGL(basis_prep_kernel, dim3(pblocks), dim3(256), 0, s, Q, M, static_cast<int>(D),
                     static_cast<int>(r), RP, RK, QtH, QtL, QH, QL, Mm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int Di = static_cast<int>(D);
  const int ri = static_cast<int>(r);
  switch (RP) {
#define RW4_Y(V) case V: e = run_yproj<V>(x, T, Di, P, S, QtH, QtL, Ypart, s); break;
    RW4_Y(16) RW4_Y(32) RW4_Y(48) RW4_Y(64) RW4_Y(80) RW4_Y(96) RW4_Y(112) RW4_Y(128)
#undef RW4_Y
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const bool of32 = out_f32 != 0;
  switch (RP) {
#define RW4_L(V, K) case V: return run_lift<V, K>(x, T, Di, P, S, ri, Ypart, Mm, QH, QL, addend, out, of32, s);
    RW4_L(16, 32) RW4_L(32, 32) RW4_L(48, 64) RW4_L(64, 64) RW4_L(80, 96) RW4_L(96, 96)
    RW4_L(112, 128) RW4_L(128, 128)
#undef RW4_L
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rw4
