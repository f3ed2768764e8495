// Structured Hadamard transforms of rows ("Infra Quant II", QuaRot Background
// and Method):
//   y = (H_A (x) K_B) diag(s) x / c,  D = A B, index f = i B + j (i < A, j < B)
// with A a power of two (H_A the Sylvester matrix, natural order) and K_B
// either a Hadamard matrix of non-power-of-two order B = m (the pages' H_d =
// H_{2^n} (x) H_m for d = 2^n m; H_m by Paley's construction, since the pages
// print none; c = sqrt(D)) or the identity (the transform across attention
// heads, H_{n_h} (x) I_{d_h}; c = sqrt(n_h)). s is an optional +-1 vector (the
// randomized H diag(s)), applied as the row is loaded.
//
// One workgroup of 512 threads per row, the row staged in LDS (fp32,
// D <= 16384):
//   1. load (bf16, fp32, or the SiLU-gated front of a gate|up row), coalesced,
//      with every load of the thread's share issued before the first use,
//      times s, into LDS; then for K_B = H_m the m-point product of every
//      group of m consecutive values, read back into registers (the +-1 table
//      is a compile-time constant, so the product is straight-line adds and
//      subtracts);
//   2. H_A along i (stride B) in LDS passes of radix 8 (the last one 2, 4 or
//      8), one barrier per pass, on 4-column groups when B % 4 == 0;
//   3. u = c^-1 x (the transform's scale), then fp32 rows, or the row's absmax
//      step and its codes (packed INT4 rows or FP6 operand tiles), from
//      32-value chunks of LDS.
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

constexpr int kKronThreads = 512;

constexpr bool kron_prime(int q) {
  if (q < 2) return false;
  for (int d = 2; d * d <= q; ++d)
    if (q % d == 0) return false;
  return true;
}

// Legendre symbol of a modulo the odd prime q: 0, +1 (nonzero square) or -1
constexpr int legendre(int a, int q) {
  a %= q;
  if (a < 0) a += q;
  if (a == 0) return 0;
  for (int y = 1; y < q; ++y)
    if ((y * y) % q == a) return 1;
  return -1;
}

// +-1 Hadamard matrix of order M by Paley's construction, rows and columns
// ordered as the point at infinity first, then the integers 0..q-1 mod q:
//   type I  (q = M - 1 prime, q = 3 mod 4): H = I + [[0, 1^T], [-1, J]],
//   type II (q = M/2 - 1 prime, q = 1 mod 4): H = C (x) [[1, 1], [1, -1]] +
//           I (x) [[1, -1], [-1, -1]], C = [[0, 1^T], [1, J]],
// where J[a][b] = legendre(a - b) is the Jacobsthal matrix of q.
template <int M>
struct Paley {
  signed char h[M][M];
  constexpr Paley() : h{} {
    if (kron_prime(M - 1) && (M - 1) % 4 == 3) {
      const int q = M - 1;
      for (int r = 0; r < M; ++r)
        for (int c = 0; c < M; ++c) {
          int v;
          if (r == 0) v = 1;
          else if (c == 0) v = -1;
          else v = legendre(r - c, q) + (r == c ? 1 : 0);
          h[r][c] = static_cast<signed char>(v);
        }
    } else {
      const int q = M / 2 - 1;
      for (int r = 0; r < M; ++r)
        for (int c = 0; c < M; ++c) {
          const int u = r / 2, w = c / 2, rr = r % 2, cc = c % 2;
          const int cv = u == w ? 0 : (u == 0 || w == 0) ? 1 : legendre(u - w, q);
          const int a = (rr == 1 && cc == 1) ? -1 : 1;
          const int b = (rr == 0 && cc == 0) ? 1 : -1;
          h[r][c] = static_cast<signed char>(cv * a + (u == w ? b : 0));
        }
    }
  }
};

template <int M>
constexpr bool paley_order() {
  return (kron_prime(M - 1) && (M - 1) % 4 == 3) ||
         (M % 2 == 0 && kron_prime(M / 2 - 1) && (M / 2 - 1) % 4 == 1);
}

// o = H_M v. With S = sum of v, row r of a +-1 matrix gives
// 2 (sum of v over the row's +1 entries) - S, or S - 2 (sum over its -1
// entries): about M / 2 adds per output instead of M - 1, over whichever set
// is smaller (the table is a compile-time constant).
template <int M>
__device__ __forceinline__ void paley_apply(const float (&v)[M], float (&o)[M]) {
  static_assert(paley_order<M>(), "Paley order");
  constexpr Paley<M> P{};
  float S = v[0];
#pragma unroll
  for (int c = 1; c < M; ++c) S += v[c];
#pragma unroll
  for (int r = 0; r < M; ++r) {
    int npos = 0;
#pragma unroll
    for (int c = 0; c < M; ++c) npos += P.h[r][c] > 0 ? 1 : 0;
    const signed char want = 2 * npos <= M ? 1 : -1;   // the smaller set
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < M; ++c)
      if (P.h[r][c] == want) acc += v[c];
    o[r] = want > 0 ? fmaf(2.0f, acc, -S) : fmaf(-2.0f, acc, S);
  }
}

// Raw bits of four consecutive input values at element offset off of a row
// (16-byte aligned for fp32, 8-byte for bf16; gate|up rows also hold the up
// half). Every load of a row is issued before the first value is used, so a
// thread waits for memory once per row.
template <int IN>
struct Raw4 {
  uint4 a;  // fp32: four values; bf16: .x, .y; gate|up: gate in .x, .y, up in .z, .w
};

template <int IN>
__device__ __forceinline__ void fetch4(Raw4<IN>& r, const void* x, int64_t off, int D) {
  if constexpr (IN == IN_F32) {
    r.a = *reinterpret_cast<const uint4*>(static_cast<const float*>(x) + off);
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(x) + off;
    const uint2 g = *reinterpret_cast<const uint2*>(p);
    r.a.x = g.x; r.a.y = g.y;
    if constexpr (IN == IN_SWIGLU) {
      const uint2 u = *reinterpret_cast<const uint2*>(p + D);
      r.a.z = u.x; r.a.w = u.y;
    }
  }
}

// the four fp32 values (SiLU(g) * u for gate|up rows), times the signs if any
template <int IN>
__device__ __forceinline__ void unpack4(float (&q)[4], const Raw4<IN>& r, bool use_signs,
                                        const float4& sg) {
  if constexpr (IN == IN_F32) {
    q[0] = __uint_as_float(r.a.x); q[1] = __uint_as_float(r.a.y);
    q[2] = __uint_as_float(r.a.z); q[3] = __uint_as_float(r.a.w);
  } else {
    q[0] = bf16lo(r.a.x); q[1] = bf16hi(r.a.x); q[2] = bf16lo(r.a.y); q[3] = bf16hi(r.a.y);
    if constexpr (IN == IN_SWIGLU) {
      const float u[4] = {bf16lo(r.a.z), bf16hi(r.a.z), bf16lo(r.a.w), bf16hi(r.a.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = silu_mul(q[e], u[e]);
    }
  }
  if (use_signs) {
    q[0] *= sg.x; q[1] *= sg.y; q[2] *= sg.z; q[3] *= sg.w;
  }
}

// natural-order R-point transform of the values (float) or 4-value columns
// (float4) at buf[base + r st], r < R
template <int R, typename V>
__device__ __forceinline__ void radix_pass(float* buf, int base, int st) {
  V v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = *reinterpret_cast<const V*>(buf + base + r * st);
#pragma unroll
  for (int h = 1; h < R; h <<= 1)
#pragma unroll
    for (int r = 0; r < R; ++r)
      if ((r & h) == 0) {
        const V a = v[r], b = v[r + h];
        v[r] = a + b;
        v[r + h] = a - b;
      }
#pragma unroll
  for (int r = 0; r < R; ++r) *reinterpret_cast<V*>(buf + base + r * st) = v[r];
}

// H_A along i (stride B) over the row in LDS: passes over three bits of i at
// a time, one barrier each. With V = float4 a work item is four adjacent
// columns j (B % 4 == 0), a quarter of the LDS instructions.
template <typename V>
__device__ __forceinline__ void h_a_passes(float* buf, int A, int B, int logA, int tid) {
  constexpr int L = sizeof(V) / sizeof(float);
  const int BL = B / L;
  const int D = A * B;
  for (int b0 = 0; b0 < logA; b0 += 3) {
    const int rb = min(3, logA - b0);
    const int items = (D >> rb) / L;
    const int st = B << b0;
    const int lomask = (1 << b0) - 1;
    for (int w = tid; w < items; w += kKronThreads) {
      const int jl = w % BL;
      const int t = w / BL;
      const int base = (((t >> b0) << (b0 + rb)) + (t & lomask)) * B + L * jl;
      if (rb == 3) radix_pass<8, V>(buf, base, st);
      else if (rb == 2) radix_pass<4, V>(buf, base, st);
      else radix_pass<2, V>(buf, base, st);
    }
    __syncthreads();
  }
}

enum KronOut { KRON_F32 = 0, KRON_PACKED = 1, KRON_TILES = 2 };

template <int IN, int M, int OUT>
__global__ void __launch_bounds__(kKronThreads)
kron_row_kernel(const void* __restrict__ x, int64_t ldx, int A, int B, int logA,
                const float* __restrict__ signs, float norm, float* __restrict__ y,
                uint8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ dbg,
                float qmax) {
  extern __shared__ __attribute__((aligned(16))) float buf[];  // D floats
  __shared__ float red[kKronThreads / 64];
  const int D = A * B;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;

  // 1. the row (all of the thread's loads issued before the first use; 4-value
  // chunks f = 4 (tid + k kKronThreads), coalesced), times s, into LDS
  constexpr int NC = kKronMaxD / (4 * kKronThreads);
  Raw4<IN> raw[NC];
  float4 sg[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int f = 4 * (tid + k * kKronThreads);
    if (f < D) {
      fetch4<IN>(raw[k], x, row * ldx + f, D);
      sg[k] = signs ? *reinterpret_cast<const float4*>(signs + f) : make_float4(1.f, 1.f, 1.f, 1.f);
    }
  }
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int f = 4 * (tid + k * kKronThreads);
    if (f < D) {
      float q[4];
      unpack4<IN>(q, raw[k], signs != nullptr, sg[k]);
      *reinterpret_cast<float4*>(buf + f) = make_float4(q[0], q[1], q[2], q[3]);
    }
  }
  __syncthreads();

  // the inner factor H_m on every group of m consecutive values, in place
  // (a group's float4 reads are m / 4 apart: no bank conflicts for m = 12,
  // 20, 28)
  if constexpr (M != 0) {
    static_assert(M % 4 == 0, "m is a multiple of 4");
    for (int i = tid; i < A; i += kKronThreads) {
      float v[M];
#pragma unroll
      for (int c = 0; c < M / 4; ++c) {
        const float4 q = *reinterpret_cast<const float4*>(buf + i * M + 4 * c);
        v[4 * c] = q.x; v[4 * c + 1] = q.y; v[4 * c + 2] = q.z; v[4 * c + 3] = q.w;
      }
      float o[M];
      paley_apply<M>(v, o);
#pragma unroll
      for (int c = 0; c < M / 4; ++c)
        *reinterpret_cast<float4*>(buf + i * M + 4 * c) =
            make_float4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    }
    __syncthreads();
  }

  // 2. H_A along i
  if (B % 4 == 0) h_a_passes<float4>(buf, A, B, logA, tid);
  else h_a_passes<float>(buf, A, B, logA, tid);

  // 3. output: u = norm * buf
  if constexpr (OUT == KRON_F32) {
    for (int f = 4 * tid; f < D; f += 4 * kKronThreads) {
      const float4 v = *reinterpret_cast<const float4*>(buf + f);
      store_stream16(y + row * D + f, make_float4(v.x * norm, v.y * norm, v.z * norm, v.w * norm));
    }
  } else {
    float m = 0.0f;
    for (int f = tid; f < D; f += kKronThreads) m = fmaxf(m, fabsf(buf[f] * norm));
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int k = 1; k < kKronThreads / 64; ++k) m = fmaxf(m, red[k]);
    const float stp = m / qmax;
    if (tid == 0) scales[row] = stp;
    const RowQuant rq(stp);
    for (int c = tid; c < D / 32; c += kKronThreads) {
      float u[32], q[32];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 v = *reinterpret_cast<const float4*>(buf + 32 * c + 4 * k);
        u[4 * k] = v.x * norm; u[4 * k + 1] = v.y * norm;
        u[4 * k + 2] = v.z * norm; u[4 * k + 3] = v.w * norm;
      }
      if (!rq.fast_codes(u, q)) {
#pragma unroll
        for (int e = 0; e < 32; ++e) q[e] = rq.code(u[e]);
      }
      if constexpr (OUT == KRON_TILES) {
        const v6u_t w = pack_fp6_32(q);
        store_fields32(codes, row, 32 * c, D, Field12{w[0], w[1], w[2]}, Field12{w[3], w[4], w[5]});
      } else {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t acc = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc |= nib(static_cast<int>(q[8 * k + e])) << (4 * e);
          wd[k] = acc;
        }
        *reinterpret_cast<uint4*>(codes + row * (D / 2) + 16 * c) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
      if (dbg) {
        float4* o = reinterpret_cast<float4*>(dbg + row * D + 32 * c);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = make_float4(u[4 * k], u[4 * k + 1], u[4 * k + 2], u[4 * k + 3]);
      }
    }
  }
}

template <int IN, int M, int OUT>
hipError_t launch_kron_out(const void* x, int64_t ldx, int64_t T, int A, int B, int logA,
                           const float* signs, float norm, float* y, uint8_t* codes,
                           float* scales, float* dbg, float qmax, hipStream_t s) {
  const size_t lds = static_cast<size_t>(A) * B * sizeof(float);
  hipLaunchKernelGGL((kron_row_kernel<IN, M, OUT>), dim3(static_cast<unsigned>(T)),
                     dim3(kKronThreads), lds, s, x, ldx, A, B, logA, signs, norm, y, codes,
                     scales, dbg, qmax);
  return hipGetLastError();
}

template <int IN, int M>
hipError_t launch_kron_m(const void* x, int64_t ldx, int64_t T, int A, int B, int logA,
                         const float* signs, float norm, float* y, uint8_t* codes, bool tiled,
                         float* scales, float* dbg, float qmax, hipStream_t s) {
  if (y)
    return launch_kron_out<IN, M, KRON_F32>(x, ldx, T, A, B, logA, signs, norm, y, codes, scales,
                                            dbg, qmax, s);
  if (tiled)
    return launch_kron_out<IN, M, KRON_TILES>(x, ldx, T, A, B, logA, signs, norm, y, codes,
                                              scales, dbg, qmax, s);
  return launch_kron_out<IN, M, KRON_PACKED>(x, ldx, T, A, B, logA, signs, norm, y, codes, scales,
                                             dbg, qmax, s);
}

template <int IN>
hipError_t launch_kron_in(int m, const void* x, int64_t ldx, int64_t T, int A, int B, int logA,
                          const float* signs, float norm, float* y, uint8_t* codes, bool tiled,
                          float* scales, float* dbg, float qmax, hipStream_t s) {
  switch (m) {
    case 0: return launch_kron_m<IN, 0>(x, ldx, T, A, B, logA, signs, norm, y, codes, tiled, scales, dbg, qmax, s);
    case 12: return launch_kron_m<IN, 12>(x, ldx, T, A, B, logA, signs, norm, y, codes, tiled, scales, dbg, qmax, s);
    case 20: return launch_kron_m<IN, 20>(x, ldx, T, A, B, logA, signs, norm, y, codes, tiled, scales, dbg, qmax, s);
    case 28: return launch_kron_m<IN, 28>(x, ldx, T, A, B, logA, signs, norm, y, codes, tiled, scales, dbg, qmax, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool kron_order_supported(int64_t m) { return m == 12 || m == 20 || m == 28; }

hipError_t launch_kron(const void* x, int in_mode, int64_t ldx, int64_t T, int64_t A, int64_t B,
                       int m, const float* signs, float norm, float* y, uint8_t* codes,
                       bool tiled, float* scales, float* dbg, int bits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (A < 1 || (A & (A - 1)) != 0 || B < 1 || A * B > kKronMaxD || (A * B) % 4 != 0)
    return hipErrorInvalidValue;
  if (m != 0 && (m != B || !kron_order_supported(m))) return hipErrorInvalidValue;
  if (!y && ((A * B) % 32 != 0 || (tiled && (A * B) % 64 != 0) || bits < 2 || bits > 4))
    return hipErrorInvalidValue;
  int logA = 0;
  while ((int64_t(1) << logA) < A) ++logA;
  const float qmax = static_cast<float>((1 << (bits - 1)) - 1);
  const int Ai = static_cast<int>(A), Bi = static_cast<int>(B);
  switch (in_mode) {
    case IN_BF16: return launch_kron_in<IN_BF16>(m, x, ldx, T, Ai, Bi, logA, signs, norm, y, codes, tiled, scales, dbg, qmax, s);
    case IN_F32: return launch_kron_in<IN_F32>(m, x, ldx, T, Ai, Bi, logA, signs, norm, y, codes, tiled, scales, dbg, qmax, s);
    case IN_SWIGLU: return launch_kron_in<IN_SWIGLU>(m, x, ldx, T, Ai, Bi, logA, signs, norm, y, codes, tiled, scales, dbg, qmax, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rw4
