// Fused prologue of the rotated linear: alignment lift + Walsh-Hadamard
// transform + per-token INT4 quantization, written as FP6 operand tiles.
//
// Per token (ReSpinQuant paper notes, key design 3; "QuaRot 与 SpinQuant"
// §2.2; "Infra Quant II", QuaRot Method):
//   v = x + Q z          (z = (M - I) Q^T x, summed from the projection's parts)
//   v = H_D v / sqrt(D)  (optional)
//   step = fl32(max |v| / 7), code = clamp(rint(fl32(v / step)), -8, 7)
// The unfused path writes v in fp32 to global memory and reads it back for
// the transform; here a workgroup of 16 waves keeps 8 aligned token rows in
// LDS (fp32, one pad word per 64 values) and runs every step on chip:
//   1. z of the 8 tokens (fixed summation order over the parts), split into
//      bf16 hi/lo in LDS; the 8 bf16 x rows read with coalesced 16-byte loads
//      (two waves per row) and widened into the LDS rows;
//   2. lift on bf16 matrix cores: each wave owns D/16 columns in 16-column
//      blocks, A = Q rows (bf16 hi and lo), B = z (hi and lo), the
//      accumulator starts as x read from LDS, and the sum Qh.zh + Ql.zh +
//      Qh.zl goes back into LDS (tokens are MFMA columns 0..7, 8..15 unused);
//      the Q fragments of the next group of blocks are in flight meanwhile;
//   3. transform of a row by its two waves (lanes L = 0..127): pass 1
//      butterflies index bits 7..N-1 in registers with lane L holding
//      L + 128 j; pass 2 holds the 32 contiguous values 32 L + j, butterflies
//      bits 0..4 in registers and bits 5, 6 (lane bits 0, 1) with DPP quad
//      permutes (stages commute), then the 1/sqrt(D) multiply;
//   4. absmax (wave reduction, then across the row's two waves), codes from
//      the step's reciprocal with an exact fallback near half-integers
//      (RowQuant), packed to E2M3 by the conversion instruction and stored
//      as one lane's six tile words; optional fp32 dump of v.
// The per-workgroup cost is D x RK x 4 bytes of Q read from L2 for 8 tokens,
// which is what bounds the shapes this kernel takes (lfq_supported).
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

constexpr int kTok = 8;            // tokens per workgroup
constexpr int kThreads = 1024;     // 16 waves; two per token row in the transform

__device__ __forceinline__ int padc(int i) { return i + (i >> 5); }

// butterfly with the lane whose index differs in bit 0 (XOR1) or bit 1 of the
// quad: the lower lane keeps a + b, the upper gets a - b
template <int CTRL>
__device__ __forceinline__ float dpp_butterfly(float v, float sgn) {
  const float p = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  return fmaf(sgn, v, p);                    // sgn = +1 on the lower lane, -1 on the upper
}

template <int N, int RK, bool FW, bool DBG>
__global__ void __launch_bounds__(kThreads)
lfq_kernel(const uint16_t* __restrict__ x, int64_t T, const float* __restrict__ Zpart, int S,
           const uint16_t* __restrict__ QH, const uint16_t* __restrict__ QL,
           uint8_t* __restrict__ tiles, float* __restrict__ s_a, float* __restrict__ dbg,
           float norm) {
  constexpr int D = 1 << N;
  constexpr int PW = D + D / 32 + 3;         // row pitch (words); 3 mod 32 keeps the lift's 16 rows on distinct banks
  constexpr int KK = RK / 32;
  constexpr int NB = D / 256;                // 16-column lift blocks per wave (16 waves)
  constexpr int QB = (NB < 4 / KK) ? NB : 4 / KK;   // blocks per group
  constexpr int NG = NB / QB;
  constexpr int J1 = D / 128;                // pass 1: values per lane (index L + 128 j)
  constexpr int NL2 = D / 32;                // pass 2: active lanes of a row (index 32 L + j)
  static_assert(N >= 8 && N <= 12, "D in [256, 4096]");
  static_assert(NB % QB == 0, "groups");
  __shared__ __attribute__((aligned(16))) float rows[kTok * PW];
  __shared__ __attribute__((aligned(16))) uint16_t zh[16][RK + 8];
  __shared__ __attribute__((aligned(16))) uint16_t zl[16][RK + 8];
  __shared__ float rmax[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = wave & 7;                  // token row of this wave in phases 1b, 3, 4
  const int half = wave >> 3;
  const int L = 64 * half + lane;            // lane index within the row's 128
  // give each XCD (workgroups go to XCDs round-robin) a contiguous band of
  // token blocks, so a tile's 32 rows are written through one L2
  int64_t blk = blockIdx.x;
  if ((gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
  const int64_t t0 = blk * kTok;

  // lift geometry; the first group of Q fragments is requested before the x
  // and z loads so that their latencies overlap
  const int i16 = lane & 15;                  // A row (column d0 + i16) / B, C column (token)
  const int g = lane >> 4;
  const int dw = wave * (D / 16);
  v8bf qa[2][QB][KK], qb[2][QB][KK];
  auto loadq = [&](int buf, int grp) {
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int64_t qo = static_cast<int64_t>(dw + 16 * (grp * QB + b) + i16) * RK + 32 * kk + 8 * g;
        qa[buf][b][kk] = ld8(QH + qo);
        qb[buf][b][kk] = ld8(QL + qo);
      }
  };
  loadq(0, 0);

  // ---- 1a. z = sum over the parts; MFMA columns 8..15 get zero
  for (int c = tid; c < 16 * RK; c += kThreads) {
    const int tt = c / RK;
    const int i = c % RK;
    const int64_t trow = min(t0 + (tt & 7), T - 1);
    float z = 0.0f;
    for (int p = 0; p < S; ++p) z += Zpart[(static_cast<int64_t>(p) * T + trow) * RK + i];
    z = tt < kTok ? z : 0.0f;
    const uint16_t h = f32_to_bf16(z);
    zh[tt][i] = h;
    zl[tt][i] = f32_to_bf16(z - bf16_to_f32(h));
  }
  // ---- 1b. x row -> LDS fp32, two waves per row (rows past T: last row, zeroed)
  {
    const int64_t trow = min(t0 + row, T - 1);  // rows past T repeat the last one; never stored
    const uint16_t* px = x + trow * D;
    float* rw = rows + row * PW;
    constexpr int NCH = D / 8;               // 16-byte chunks per row
#pragma unroll
    for (int it = 0; it < (NCH + 127) / 128; ++it) {
      const int c = it * 128 + L;
      const int cc = c < NCH ? c : NCH - 1;  // unconditional load, clamped
      const uint4 v = *reinterpret_cast<const uint4*>(px + 8 * cc);
      if (c < NCH) {
        float* dst = rw + padc(8 * c);       // 8 columns inside one 32-column group
        dst[0] = bf16lo(v.x); dst[1] = bf16hi(v.x);
        dst[2] = bf16lo(v.y); dst[3] = bf16hi(v.y);
        dst[4] = bf16lo(v.z); dst[5] = bf16hi(v.z);
        dst[6] = bf16lo(v.w); dst[7] = bf16hi(v.w);
      }
    }
  }
  __syncthreads();

  // ---- 2. lift: out[d][j] = x[j][d] + sum_k Q[d][k] z[j][k] for this wave's columns
  {
    const int jt = i16 & 7;                   // token row read for the accumulator start
    v8bf bh[KK], bl[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bh[kk] = *reinterpret_cast<const v8bf*>(&zh[i16][32 * kk + 8 * g]);
      bl[kk] = *reinterpret_cast<const v8bf*>(&zl[i16][32 * kk + 8 * g]);
    }
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      const int buf = grp & 1;
      if (grp + 1 < NG) loadq(buf ^ 1, grp + 1);   // compile-time condition (unrolled)
      v4f acc[QB];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int d = dw + 16 * (grp * QB + b) + 4 * g;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[b][v] = rows[jt * PW + padc(d + v)];
      }
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          acc[b] = mfma(qa[buf][b][kk], bh[kk], acc[b]);
          acc[b] = mfma(qb[buf][b][kk], bh[kk], acc[b]);
          acc[b] = mfma(qa[buf][b][kk], bl[kk], acc[b]);
        }
      mfma_drain();
      if (i16 < kTok) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          const int d = dw + 16 * (grp * QB + b) + 4 * g;
#pragma unroll
          for (int v = 0; v < 4; ++v) rows[i16 * PW + padc(d + v)] = acc[b][v];
        }
      }
    }
  }
  __syncthreads();

  // ---- 3. transform of row `row`, lanes L = 0..127 of its two waves
  float* rw = rows + row * PW;
  if constexpr (FW) {
    // pass 1: index bits 7..N-1, lane L holds L + 128 j (padc = L + L/32 + 132 j)
    float va[J1];
#pragma unroll
    for (int j = 0; j < J1; ++j) va[j] = rw[L + (L >> 5) + 132 * j];
#pragma unroll
    for (int h = 1; h < J1; h <<= 1)
#pragma unroll
      for (int j = 0; j < J1; ++j)
        if ((j & h) == 0) {
          const float a = va[j], b = va[j + h];
          va[j] = a + b;
          va[j + h] = a - b;
        }
#pragma unroll
    for (int j = 0; j < J1; ++j) rw[L + (L >> 5) + 132 * j] = va[j];
  }
  __syncthreads();
  // pass 2: lane L (< D / 32) holds the 32 values 32 L + j (padc = 33 L + j);
  // bits 0..4 in registers, bits 5 and 6 are bits 0 and 1 of the lane
  const bool act = L < NL2;
  const int Lc = act ? L : NL2 - 1;          // inactive lanes repeat a valid group, ignored
  float u[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) u[j] = rw[33 * Lc + j];
  if constexpr (FW) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if ((j & h) == 0) {
          const float a = u[j], b = u[j + h];
          u[j] = a + b;
          u[j + h] = a - b;
        }
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) u[j] = dpp_butterfly<0xB1>(u[j], sg1);
#pragma unroll
    for (int j = 0; j < 32; ++j) u[j] = dpp_butterfly<0x4E>(u[j], sg2);
#pragma unroll
    for (int j = 0; j < 32; ++j) u[j] *= norm;
  }

  // ---- 4. absmax over the row's two waves, codes, tiles
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(u[j]));
  m = act ? m : 0.0f;
  m = wave_max(m);
  if (lane == 0) rmax[wave] = m;
  __syncthreads();
  m = fmaxf(rmax[row], rmax[row + 8]);
  const int64_t t = t0 + row;
  if (t < T && act) {
    const float s = m / 7.0f;
    if (L == 0) s_a[t] = s;
    const RowQuant rq(s);
    float q[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) q[e] = rq.code(u[e]);
    const v6u_t w = pack_fp6_32(q);
    store_fields32(tiles, t, 32 * L, D, Field12{w[0], w[1], w[2]}, Field12{w[3], w[4], w[5]});
    if constexpr (DBG) {
      float4* o = reinterpret_cast<float4*>(dbg + t * D + 32 * L);
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = make_float4(u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]);
    }
  }
}

template <int N, int RK>
hipError_t launch_n(const uint16_t* x, int64_t T, const AlignParts& a, bool fw, uint8_t* tiles,
                    float* s_a, float* dbg, hipStream_t s) {
  const float norm = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(1 << N)));
  const dim3 grid(static_cast<unsigned>((T + kTok - 1) / kTok));
#define RW4_LFQ(F, G)                                                                            \
  if (fw == F && (dbg != nullptr) == G) {                                                        \
    hipLaunchKernelGGL((lfq_kernel<N, RK, F, G>), grid, dim3(kThreads), 0, s, x, T, a.Zpart, a.S, \
                       a.QH, a.QL, tiles, s_a, dbg, norm);                                       \
    return hipGetLastError();                                                                    \
  }
  RW4_LFQ(true, false) RW4_LFQ(true, true) RW4_LFQ(false, false) RW4_LFQ(false, true)
#undef RW4_LFQ
  return hipErrorInvalidValue;
}

template <int RK>
hipError_t launch_rk(int n, const uint16_t* x, int64_t T, const AlignParts& a, bool fw,
                     uint8_t* tiles, float* s_a, float* dbg, hipStream_t s) {
  switch (n) {
    case 8: return launch_n<8, RK>(x, T, a, fw, tiles, s_a, dbg, s);
    case 9: return launch_n<9, RK>(x, T, a, fw, tiles, s_a, dbg, s);
    case 10: return launch_n<10, RK>(x, T, a, fw, tiles, s_a, dbg, s);
    case 11: return launch_n<11, RK>(x, T, a, fw, tiles, s_a, dbg, s);
    case 12: return launch_n<12, RK>(x, T, a, fw, tiles, s_a, dbg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// D a power of two in [256, 4096] and r <= 64: Q costs D x RK x 4 bytes of L2
// reads per 8 tokens, below the 32 bytes per value of an fp32 round trip
bool lfq_supported(int64_t D, int64_t r) {
  return r > 0 && r <= 64 && D >= 256 && D <= 4096 && (D & (D - 1)) == 0;
}

hipError_t launch_lift_fwht_quant(const uint16_t* x, int64_t T, int64_t D, int64_t r, void* ws,
                                  bool do_fwht, uint8_t* tiles, float* s_a, float* dbg,
                                  hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!lfq_supported(D, r)) return hipErrorInvalidValue;
  const AlignParts a = align_parts(ws, T, D, r);
  int n = 0;
  while ((int64_t(1) << n) < D) ++n;
  if (a.RK == 32) return launch_rk<32>(n, x, T, a, do_fwht, tiles, s_a, dbg, s);
  if (a.RK == 64) return launch_rk<64>(n, x, T, a, do_fwht, tiles, s_a, dbg, s);
  return hipErrorInvalidValue;
}

}  // namespace rw4
