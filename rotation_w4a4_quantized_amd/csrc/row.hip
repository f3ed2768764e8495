// Per-token row kernels: gated front, Walsh-Hadamard transform, INT4 quantization.
//
// Walsh-Hadamard transform ("QuaRot 与 SpinQuant" §2.2; "Infra Quant II",
// QuaRot Background): H_D = H_2 (x) ... (x) H_2, so the transform is one
// butterfly stage per index bit and the stages commute. A row of D = 2^N fp32
// values is split over P = D / EPT threads (EPT = 2^E values each). Pass 0
// butterflies the low E index bits in registers right after a contiguous
// vector load; every further pass takes the next group of at most E bits: the
// row goes through LDS (padded one word per 16 to spread banks), each thread
// reads the values whose indices differ only in that group, butterflies them
// in registers and writes them back. The 1/sqrt(D) scale is one multiply after
// the last stage.
//
// Quantization ("Infra Quant II", QuaRot Method; SpinQuant MOTIVATION): for
// b-bit codes (b = 4, or 3 and 2 for the lower settings of the ReSpinQuant
// notes' experiments), per row step = fl32(absmax / (2^(b-1) - 1)) and
// code = clamp(rint(fl32(v / step)), -2^(b-1), 2^(b-1) - 1); symmetric absmax
// keeps every code in [-(2^(b-1) - 1), 2^(b-1) - 1]. Codes are stored as INT4
// nibbles (element 2j in the low nibble) or FP6 tile fields, whatever b.
#include "align_small.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

__device__ __forceinline__ int padi(int i) { return i + (i >> 4); }

template <int N, int E>
struct Sched {
  static constexpr int REM = N - E;
  static constexpr int NP = REM > 0 ? (REM + E - 1) / E : 0;
  static constexpr int gsize(int p) { return REM / NP + (p < REM % NP ? 1 : 0); }
  static constexpr int gbase(int p) {
    int b = E;
    for (int i = 0; i < p; ++i) b += gsize(i);
    return b;
  }
};

// butterflies over G index bits for each of the 2^(E-G) sub-vectors held in v
template <int E, int G>
__device__ __forceinline__ void butterflies(float (&v)[1 << E]) {
  constexpr int SV = 1 << G;
#pragma unroll
  for (int s = 0; s < (1 << (E - G)); ++s) {
#pragma unroll
    for (int h = 1; h < SV; h <<= 1) {
#pragma unroll
      for (int j = 0; j < SV; ++j) {
        if ((j & h) == 0) {
          const float a = v[s * SV + j];
          const float b = v[s * SV + j + h];
          v[s * SV + j] = a + b;
          v[s * SV + j + h] = a - b;
        }
      }
    }
  }
}

// element index of entry j of the group [b, b+G) for free index f
__device__ __forceinline__ int gidx(int f, int j, int b, int G) {
  return (f & ((1 << b) - 1)) | (j << b) | ((f >> b) << (b + G));
}

template <int E, int G, int B>
__device__ __forceinline__ void lds_pass(float (&v)[1 << E], float* rowlds, int t, bool last,
                                         float norm) {
  constexpr int SV = 1 << G;
  constexpr int NS = 1 << (E - G);
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < SV; ++j) v[s * SV + j] = rowlds[padi(gidx(t * NS + s, j, B, G))];
  butterflies<E, G>(v);
  if (last) {
#pragma unroll
    for (int i = 0; i < (1 << E); ++i) v[i] *= norm;
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < SV; ++j) rowlds[padi(gidx(t * NS + s, j, B, G))] = v[s * SV + j];
}

template <int N, int E, int P>
__device__ __forceinline__ void run_passes(float (&v)[1 << E], float* rowlds, int t, float norm) {
  using S = Sched<N, E>;
  if constexpr (S::NP >= 1) {
    lds_pass<E, S::gsize(0), S::gbase(0)>(v, rowlds, t, S::NP == 1, norm);
    __syncthreads();
  }
  if constexpr (S::NP >= 2) {
    lds_pass<E, S::gsize(1), S::gbase(1)>(v, rowlds, t, S::NP == 2, norm);
    __syncthreads();
  }
  if constexpr (S::NP >= 3) {
    lds_pass<E, S::gsize(2), S::gbase(2)>(v, rowlds, t, S::NP == 3, norm);
    __syncthreads();
  }
  static_assert(S::NP <= 3, "at most three LDS passes");
}

// load EPT contiguous inputs of a row starting at element e0 as fp32
// Loads are unconditional: a row past T reads the last row (rowoff is
// clamped by the caller) and its values are zeroed afterwards, so no load sits
// inside a branch whose result is used after the branch.
template <int IN, int EPT>
__device__ __forceinline__ void load_row_raw(float (&v)[EPT], const void* x, int64_t rowoff, int e0,
                                             int D);

template <int IN, int EPT>
__device__ __forceinline__ void load_row(float (&v)[EPT], const void* x, int64_t rowoff, int e0,
                                         int D, bool active) {
  load_row_raw<IN, EPT>(v, x, rowoff, e0, D);
#pragma unroll
  for (int i = 0; i < EPT; ++i) v[i] = active ? v[i] : 0.0f;
}

template <int IN, int EPT>
__device__ __forceinline__ void load_row_raw(float (&v)[EPT], const void* x, int64_t rowoff, int e0,
                                             int D) {
  if constexpr (IN == IN_F32) {
    const float* p = static_cast<const float*>(x) + rowoff + e0;
    if constexpr (EPT >= 4) {
#pragma unroll
      for (int i = 0; i < EPT / 4; ++i) {
        const float4 q = reinterpret_cast<const float4*>(p)[i];
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPT; ++i) v[i] = p[i];
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(x) + rowoff + e0;
    float g[EPT];
    if constexpr (EPT >= 8) {
#pragma unroll
      for (int i = 0; i < EPT / 8; ++i) {
        const uint4 q = reinterpret_cast<const uint4*>(p)[i];
        g[8 * i + 0] = bf16lo(q.x); g[8 * i + 1] = bf16hi(q.x);
        g[8 * i + 2] = bf16lo(q.y); g[8 * i + 3] = bf16hi(q.y);
        g[8 * i + 4] = bf16lo(q.z); g[8 * i + 5] = bf16hi(q.z);
        g[8 * i + 6] = bf16lo(q.w); g[8 * i + 7] = bf16hi(q.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPT; ++i) g[i] = bf16_to_f32(p[i]);
    }
    if constexpr (IN == IN_SWIGLU) {
      // gate = first D values of the row, up = next D values
      const uint16_t* pu = p + D;
      float u[EPT];
      if constexpr (EPT >= 8) {
#pragma unroll
        for (int i = 0; i < EPT / 8; ++i) {
          const uint4 q = reinterpret_cast<const uint4*>(pu)[i];
          u[8 * i + 0] = bf16lo(q.x); u[8 * i + 1] = bf16hi(q.x);
          u[8 * i + 2] = bf16lo(q.y); u[8 * i + 3] = bf16hi(q.y);
          u[8 * i + 4] = bf16lo(q.z); u[8 * i + 5] = bf16hi(q.z);
          u[8 * i + 6] = bf16lo(q.w); u[8 * i + 7] = bf16hi(q.w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < EPT; ++i) u[i] = bf16_to_f32(pu[i]);
      }
#pragma unroll
      for (int i = 0; i < EPT; ++i) v[i] = silu_mul(g[i], u[i]);
    } else {
#pragma unroll
      for (int i = 0; i < EPT; ++i) v[i] = g[i];
    }
  }
}

template <int EPT>
__device__ __forceinline__ void store_f32(float* p, const float (&v)[EPT]) {
  if constexpr (EPT >= 4) {
#pragma unroll
    for (int i = 0; i < EPT / 4; ++i)
      store_stream16(reinterpret_cast<float4*>(p) + i,
                     make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]));
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) p[i] = v[i];
  }
}

template <int EPT>
__device__ __forceinline__ void store_codes(uint8_t* p, const float (&v)[EPT], float s) {
  uint32_t wds[(EPT + 7) / 8];
#pragma unroll
  for (int i = 0; i < (EPT + 7) / 8; ++i) wds[i] = 0;
  const RowQuant rq(s);
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int q = static_cast<int>(rq.code(v[i]));
    wds[i / 8] |= nib(q) << (4 * (i % 8));
  }
  if constexpr (EPT == 32) {
    reinterpret_cast<uint4*>(p)[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  } else if constexpr (EPT == 16) {
    reinterpret_cast<uint2*>(p)[0] = make_uint2(wds[0], wds[1]);
  } else if constexpr (EPT == 8) {
    reinterpret_cast<uint32_t*>(p)[0] = wds[0];
  } else if constexpr (EPT == 4) {
    reinterpret_cast<uint16_t*>(p)[0] = static_cast<uint16_t>(wds[0]);
  } else {
    p[0] = static_cast<uint8_t>(wds[0]);
  }
}

constexpr int kRowThreads = 256;

// codes of EPT (a multiple of 16) consecutive values starting at column k0 of
// row `row`, written as FP6 E2M3 fields into the tiled layout (common.hpp)
template <int EPT>
__device__ __forceinline__ void store_tiled(uint8_t* tiles, int64_t row, int64_t k0, int64_t K,
                                            const float (&v)[EPT], float s) {
  static_assert(EPT % 16 == 0, "tiled output needs 16-value groups");
  const RowQuant rq(s);
#pragma unroll
  for (int h = 0; h < EPT / 16; ++h) {
    float q[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) q[e] = rq.code(v[16 * h + e]);
    store_fields16(tiles, row, k0 + 16 * h, K, pack_fp6_16(q));
  }
}

// one row block (ROWS rows) of row_kernel, block index blk
template <int N, int E, int IN, bool FW, bool QOUT, bool TILED>
__device__ __forceinline__ void row_body(int64_t blk, const void* __restrict__ x, int64_t ldx,
                                         int64_t T, float* __restrict__ yf,
                                         uint8_t* __restrict__ codes, float* __restrict__ scales,
                                         float* __restrict__ dbg, float norm, float qmax) {
  constexpr int D = 1 << N;
  constexpr int EPT = 1 << E;
  constexpr int P = D >> E;                         // threads per row
  constexpr int ROWS = P >= kRowThreads ? 1 : kRowThreads / P;
  constexpr int PADD = D + (D >> 4);
  constexpr int WPR = P > 64 ? P / 64 : 1;          // waves per row
  __shared__ float lds[FW ? ROWS * PADD : 1];
  __shared__ float red[ROWS * WPR];

  const int tid = threadIdx.x;
  const int rl = tid / P;
  const int t = tid % P;
  const int64_t row = blk * ROWS + rl;
  const bool active = row < T;

  float v[EPT];
  load_row<IN, EPT>(v, x, (active ? row : T - 1) * ldx, t * EPT, D, active);

  if constexpr (FW) {
    float* rowlds = lds + rl * PADD;
    butterflies<E, E>(v);
    if constexpr (Sched<N, E>::NP == 0) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) v[i] *= norm;
    } else {
#pragma unroll
      for (int j = 0; j < EPT; ++j) rowlds[padi(t * EPT + j)] = v[j];
      __syncthreads();
      run_passes<N, E, P>(v, rowlds, t, norm);
      // back to the contiguous layout for the output phase
#pragma unroll
      for (int j = 0; j < EPT; ++j) v[j] = rowlds[padi(t * EPT + j)];
    }
  }

  if constexpr (!QOUT) {
    if (active) store_f32<EPT>(yf + row * D + t * EPT, v);
    return;
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) m = fmaxf(m, fabsf(v[i]));
    if constexpr (P <= 64) {
      m = group_max<P>(m);
    } else {
      m = wave_max(m);
      if ((tid & 63) == 0) red[rl * WPR + t / 64] = m;
      __syncthreads();
      m = red[rl * WPR];
#pragma unroll
      for (int i = 1; i < WPR; ++i) m = fmaxf(m, red[rl * WPR + i]);
    }
    if (!active) return;
    const float s = m / qmax;
    if (t == 0) scales[row] = s;
    if constexpr (TILED)
      store_tiled<EPT>(codes, row, static_cast<int64_t>(t) * EPT, D, v, s);
    else
      store_codes<EPT>(codes + row * (D / 2) + t * (EPT / 2), v, s);
    if (dbg) store_f32<EPT>(dbg + row * D + t * EPT, v);
  }
}

template <int N, int E, int IN, bool FW, bool QOUT, bool TILED>
__global__ void __launch_bounds__(1024)
row_kernel(const void* __restrict__ x, int64_t ldx, int64_t T, float* __restrict__ yf,
           uint8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ dbg,
           float norm, float qmax) {
  // tiled output: give each XCD (workgroups go to XCDs round-robin) a
  // contiguous band of rows, so a tile's 32 rows are written through one L2
  int64_t blk = blockIdx.x;
  if (TILED && (gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
  row_body<N, E, IN, FW, QOUT, TILED>(blk, x, ldx, T, yf, codes, scales, dbg, norm, qmax);
}

// The quantizer of a short batch (one 256-thread workgroup per row, D = 4096:
// 16 values per thread) and, beside it in the same launch, the short-batch
// alignment projection of the same rows for another basis (one 256-thread
// workgroup per 256-column chunk): workgroups 0 .. nq - 1 quantize, the rest
// project. Neither waits for the other; one launch instead of two.
template <bool FW, bool TILED>
__global__ void __launch_bounds__(256)
quant_proj_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t T, uint8_t* __restrict__ codes,
                  float* __restrict__ scales, float* __restrict__ dbg, float norm, float qmax,
                  int nq, int RP, int RK, const uint16_t* __restrict__ QtH,
                  const uint16_t* __restrict__ QtL, float* __restrict__ Zs) {
  if (static_cast<int>(blockIdx.x) < nq)
    row_body<12, 4, IN_BF16, FW, true, TILED>(blockIdx.x, x, ldx, T, nullptr, codes, scales, dbg,
                                             norm, qmax);
  else
    asmall_proj_body(static_cast<int>(blockIdx.x) - nq, x, static_cast<int>(T), 4096, RP, RK, QtH,
                     QtL, Zs);
}

// ---------------------------------------------------------------- one wave per row
// For D = 2^N with N in [11, 13] a row fits one wave's registers, and every
// wave streams its own row: no LDS, no barriers, many rows' loads in flight
// per CU. Two register layouts:
//   * coalesced (fp32 or packed-code output): lane L holds the 4 consecutive
//     values 256 c + 4 L + e (c < D / 256), so each load and store
//     instruction of the wave covers one contiguous 1 KiB (fp32) piece;
//   * tiled output: lane L holds 16 consecutive values 1024 k + 16 L + e, the
//     unit of a tile field group.
// Either way some index bits are register bits (butterflies in registers)
// and six are lane bits (the cross-lane moves of common.hpp); the absmax is a
// wave reduction.
constexpr int kWaveRows = 4;                        // rows (waves) per workgroup

// One wave per row (rowwave_kernel) or a workgroup per row (row_kernel) for
// rows of 2048..8192 values. Measured on MI355X (graph-replayed calls): the
// workgroup kernel is as fast or faster for FP6-tile outputs at every T
// (D = 8192, T = 4096 unit prologue: 49 against 89 us), for packed codes at
// D = 8192, and below 1024 rows for everything (T = 8: 3.4 against 7.8 us);
// one wave per row keeps the fp32 transform of many rows (T = 2048, D = 4096:
// 13.5 against 18.1 us) and packed codes at D <= 4096 (6.0 against 7.4 us).
template <int N, bool QOUT, bool TILED>
inline bool row_per_wave(int64_t T) {
  if (TILED || T < 1024) return false;
  return !QOUT || N <= 12;
}

template <int IN, int G>
__device__ __forceinline__ void load_group(float (&q)[G], const void* x, int64_t off, int D) {
  static_assert(G == 4 || G == 16, "groups of 4 or 16 values");
  if constexpr (IN == IN_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
      const float4 a = load_stream16f(p + i);
      q[4 * i] = a.x; q[4 * i + 1] = a.y; q[4 * i + 2] = a.z; q[4 * i + 3] = a.w;
    }
  } else {
    auto unpack = [](const uint16_t* p, float (&o)[G]) {
#pragma unroll
      for (int i = 0; i < G / 4; ++i) {
        const uint2 a = reinterpret_cast<const uint2*>(p)[i];
        o[4 * i] = bf16lo(a.x); o[4 * i + 1] = bf16hi(a.x);
        o[4 * i + 2] = bf16lo(a.y); o[4 * i + 3] = bf16hi(a.y);
      }
    };
    const uint16_t* p = static_cast<const uint16_t*>(x) + off;
    unpack(p, q);
    if constexpr (IN == IN_SWIGLU) {
      // gate = first D values of the row, up = next D values; fp32 SiLU(g) * u
      float u[G];
      unpack(p + D, u);
#pragma unroll
      for (int i = 0; i < G; ++i) q[i] = silu_mul(q[i], u[i]);
    }
  }
}

template <int N, int IN, bool FW, bool QOUT, bool TILED>
__global__ void __launch_bounds__(64 * kWaveRows)
rowwave_kernel(const void* __restrict__ x, int64_t ldx, int64_t T, float* __restrict__ yf,
               uint8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ dbg,
               float norm, float qmax) {
  constexpr int D = 1 << N;
  constexpr int G = TILED ? 16 : 4;                 // consecutive values per group
  constexpr int NG = D / (64 * G);                  // groups per lane
  constexpr int NV = D / 64;
  static_assert(N >= 11 && N <= 13, "D in [2048, 8192]");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int64_t blk = blockIdx.x;
  if (TILED && (gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
  const int64_t row = blk * kWaveRows + wave;
  const bool active = row < T;
  const int64_t rowoff = (active ? row : T - 1) * ldx;  // rows past T re-read the last row
  auto col = [&](int c) { return static_cast<int64_t>(64 * G) * c + G * lane; };

  float v[NV];
#pragma unroll
  for (int c = 0; c < NG; ++c) {
    float q[G];
    load_group<IN, G>(q, x, rowoff + col(c), D);
#pragma unroll
    for (int e = 0; e < G; ++e) v[G * c + e] = active ? q[e] : 0.0f;
  }
  if constexpr (FW) {
    // register bits: butterflies on v[j], v[j + h]
#pragma unroll
    for (int h = 1; h < NV; h <<= 1)
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if ((j & h) == 0) {
          const float a = v[j], b = v[j + h];
          v[j] = a + b;
          v[j + h] = a - b;
        }
    lane_butterflies<NV, 6>(v, lane);
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] *= norm;
  }
  auto put_f32 = [&](float* base) {
#pragma unroll
    for (int c = 0; c < NG; ++c) {
      float q[G];
#pragma unroll
      for (int e = 0; e < G; ++e) q[e] = v[G * c + e];
      store_f32<G>(base + row * D + col(c), q);
    }
  };
  if constexpr (!QOUT) {
    if (active) put_f32(yf);
  } else {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) m = fmaxf(m, fabsf(v[j]));
    m = wave_max(m);
    if (!active) return;
    const float st = m / qmax;
    if (lane == 0) scales[row] = st;
    const RowQuant rq(st);
    // codes per group of G values from the reciprocal, checked once per group
    // (RowQuant::fast_codes); a group with a value too close to a half-integer
    // takes the exact quotient
#pragma unroll
    for (int c = 0; c < NG; ++c) {
      float u[G], f[G];
#pragma unroll
      for (int e = 0; e < G; ++e) u[e] = v[G * c + e];
      if (!rq.fast_codes(u, f)) {
#pragma unroll
        for (int e = 0; e < G; ++e) f[e] = rq.code(u[e]);
      }
      if constexpr (TILED) {
        store_fields16(codes, row, col(c), D, pack_fp6_16(f));
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= nib(static_cast<int>(f[e])) << (4 * e);
        *reinterpret_cast<uint16_t*>(codes + row * (D / 2) + col(c) / 2) = static_cast<uint16_t>(w);
      }
    }
    if (dbg) put_f32(dbg);
  }
}

template <int N, int IN, bool FW, bool QOUT, bool TILED>
hipError_t launch_row_n(const void* x, int64_t ldx, int64_t T, float* yf, uint8_t* codes,
                        float* scales, float* dbg, float qmax, hipStream_t s) {
  constexpr int E = N >= 15 ? 5 : (N < 4 ? N : 4);
  constexpr int P = (1 << N) >> E;
  constexpr int ROWS = P >= kRowThreads ? 1 : kRowThreads / P;
  const float norm = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(1 << N)));
  if constexpr (N >= 11 && N <= 13) {
    if (row_per_wave<N, QOUT, TILED>(T)) {
      const int64_t wblocks = (T + kWaveRows - 1) / kWaveRows;
      hipLaunchKernelGGL((rowwave_kernel<N, IN, FW, QOUT, TILED>),
                         dim3(static_cast<unsigned>(wblocks)), dim3(64 * kWaveRows), 0, s, x, ldx,
                         T, yf, codes, scales, dbg, norm, qmax);
      return hipGetLastError();
    }
  }
  const int64_t blocks = (T + ROWS - 1) / ROWS;
  if constexpr (TILED && (1 << E) < 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL((row_kernel<N, E, IN, FW, QOUT, TILED && (1 << E) >= 16>),
                     dim3(static_cast<unsigned>(blocks)),
                     dim3(P * ROWS), 0, s, x, ldx, T, yf, codes, scales, dbg, norm, qmax);
  return hipGetLastError();
}

template <int IN, bool FW, bool QOUT, bool TILED>
hipError_t dispatch_n(int n, const void* x, int64_t ldx, int64_t T, float* yf, uint8_t* codes,
                      float* scales, float* dbg, float qmax, hipStream_t s) {
  switch (n) {
#define RW4_CASE(k) \
  case k: return launch_row_n<k, IN, FW, QOUT, TILED>(x, ldx, T, yf, codes, scales, dbg, qmax, s);
    RW4_CASE(1) RW4_CASE(2) RW4_CASE(3) RW4_CASE(4) RW4_CASE(5) RW4_CASE(6) RW4_CASE(7)
    RW4_CASE(8) RW4_CASE(9) RW4_CASE(10) RW4_CASE(11) RW4_CASE(12) RW4_CASE(13) RW4_CASE(14)
    RW4_CASE(15)
#undef RW4_CASE
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- any even D
template <int IN>
__global__ void __launch_bounds__(256)
quant_generic_kernel(const void* __restrict__ x, int64_t ldx, int64_t D,
                     uint8_t* __restrict__ codes, float* __restrict__ scales, float qmax) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  auto val = [&](int64_t i) -> float {
    if constexpr (IN == IN_F32) return static_cast<const float*>(x)[row * ldx + i];
    else return bf16_to_f32(static_cast<const uint16_t*>(x)[row * ldx + i]);
  };
  float m = 0.0f;
  for (int64_t i = tid; i < D; i += 256) m = fmaxf(m, fabsf(val(i)));
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m / qmax;
  if (tid == 0) scales[row] = s;
  for (int64_t j = tid; j < D / 2; j += 256) {
    const int q0 = s > 0.0f ? quant4(val(2 * j), s) : 0;
    const int q1 = s > 0.0f ? quant4(val(2 * j + 1), s) : 0;
    codes[row * (D / 2) + j] = static_cast<uint8_t>(nib(q0) | (nib(q1) << 4));
  }
}

}  // namespace

hipError_t launch_row(const void* x, int in_mode, int64_t ldx, int64_t T, int64_t D, bool do_fwht,
                      float* yf, uint8_t* codes, bool tiled, float* scales, float* dbg,
                      hipStream_t s, int bits) {
  if (T == 0) return hipSuccess;
  if (bits < 2 || bits > 4) return hipErrorInvalidValue;
  const float qmax = static_cast<float>((1 << (bits - 1)) - 1);
  int n = 0;
  while ((int64_t(1) << n) < D) ++n;
  const bool q = codes != nullptr;
  if (tiled && (!q || D < 64)) return hipErrorInvalidValue;
#define RW4_SEL(INM, FW, Q, TL) \
  if (in_mode == INM && do_fwht == FW && q == Q && tiled == TL) \
    return dispatch_n<INM, FW, Q, TL>(n, x, ldx, T, yf, codes, scales, dbg, qmax, s);
  RW4_SEL(IN_BF16, true, true, false) RW4_SEL(IN_BF16, true, false, false)
  RW4_SEL(IN_F32, true, true, false) RW4_SEL(IN_F32, true, false, false)
  RW4_SEL(IN_SWIGLU, true, true, false) RW4_SEL(IN_SWIGLU, false, true, false)
  RW4_SEL(IN_BF16, false, true, false) RW4_SEL(IN_F32, false, true, false)
  RW4_SEL(IN_BF16, true, true, true) RW4_SEL(IN_F32, true, true, true)
  RW4_SEL(IN_SWIGLU, true, true, true) RW4_SEL(IN_SWIGLU, false, true, true)
  RW4_SEL(IN_BF16, false, true, true) RW4_SEL(IN_F32, false, true, true)
#undef RW4_SEL
  return hipErrorInvalidValue;
}

bool quant_project_fused(int64_t T, int64_t D) { return T >= 1 && T <= kSmallT && D == 4096; }

hipError_t launch_quant_project(const uint16_t* x, int64_t ldx, int64_t T, int64_t D,
                                bool do_fwht, uint8_t* codes, bool tiled, float* scales,
                                float* dbg, int bits, const AlignBasis& pb, float* Zs,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!quant_project_fused(T, D) || bits < 2 || bits > 4) return hipErrorInvalidValue;
  const float qmax = static_cast<float>((1 << (bits - 1)) - 1);
  const float norm = static_cast<float>(1.0 / 64.0);   // 1 / sqrt(4096)
  const dim3 grid(static_cast<unsigned>(T + D / kSmallChunk));
#define RW4_QP(FW, TL)                                                                           \
  if (do_fwht == FW && tiled == TL) {                                                            \
    hipLaunchKernelGGL((quant_proj_kernel<FW, TL>), grid, dim3(256), 0, s, x, ldx, T, codes,    \
                       scales, dbg, norm, qmax, static_cast<int>(T), pb.RP, pb.RK, pb.QtH,      \
                       pb.QtL, Zs);                                                             \
    return hipGetLastError();                                                                    \
  }
  RW4_QP(false, false) RW4_QP(false, true) RW4_QP(true, false) RW4_QP(true, true)
#undef RW4_QP
  return hipErrorInvalidValue;
}

hipError_t launch_quant_generic(const void* x, int in_mode, int64_t ldx, int64_t T, int64_t D,
                                uint8_t* codes, float* scales, hipStream_t s, int bits) {
  if (T == 0) return hipSuccess;
  if (bits < 2 || bits > 4) return hipErrorInvalidValue;
  const float qmax = static_cast<float>((1 << (bits - 1)) - 1);
  if (in_mode == IN_F32)
    hipLaunchKernelGGL(quant_generic_kernel<IN_F32>, dim3(static_cast<unsigned>(T)), dim3(256), 0,
                       s, x, ldx, D, codes, scales, qmax);
  else
    hipLaunchKernelGGL(quant_generic_kernel<IN_BF16>, dim3(static_cast<unsigned>(T)), dim3(256), 0,
                       s, x, ldx, D, codes, scales, qmax);
  return hipGetLastError();
}

}  // namespace rw4
