// Fused prologue of the rotated linear: alignment lift + Walsh-Hadamard
// transform + per-token INT4 quantization, written as FP6 operand tiles (or as
// packed INT4 rows for the packed-weight GEMM).
//
// Per token (ReSpinQuant paper notes, key design 3; "QuaRot 与 SpinQuant"
// §2.2; "Infra Quant II", QuaRot Method):
//   v = x + Q z          (z = (M - I) Q^T x, summed from the projection's parts)
//   u = H_D v / sqrt(D)  (optional)
//   step = fl32(max |u| / qmax), code = rint(fl32(u / step)) (qmax = 2^(b-1) - 1
//   for b-bit codes, 7 for INT4; |code| <= qmax by construction)
// H_D / sqrt(D) is symmetric and orthogonal, so H v / sqrt(D) =
// H x / sqrt(D) + P z with P = H Q / sqrt(D), prepared once with the basis
// (without the transform P is Q itself). The two terms are computed at the
// same time by different waves of one workgroup of 16 waves and 8 tokens:
//   * waves 0..7 ("row waves") each hold one token row in registers: lane L
//     holds the chunks c = L + 64 s (s < D / 2048) of 32 consecutive values
//     32 c + j. The transform butterflies index bits 0..4 and bit 11 in
//     registers, and the lane bits with cross-lane moves: DPP quad permutes
//     (lane bits 0, 1), DPP row rotations with bank masks (bits 2, 3), and
//     the gfx950 permlane16/permlane32 swaps (bits 4, 5), which exchange a
//     lane bit with a register index so that the butterfly runs in-lane;
//   * waves 8..15 ("lift waves") stream P (bf16 hi/lo, D x RK x 4 bytes per
//     workgroup) and compute P z on bf16 matrix cores, Ph.zh + Pl.zh + Ph.zl
//     (the dropped Pl.zl is ~2^-17 relative), into an LDS buffer laid out
//     like the row waves' registers. They run at a raised wave priority: the
//     P stream is the long pole, and the row waves' VALU work fills the gaps.
// After a workgroup barrier each row wave adds its lift, takes the absmax
// with a wave reduction, and quantizes: codes from the step's reciprocal,
// checked in bulk against the distance to the nearest half-integer, with the
// exact IEEE quotient as the (rare) fallback for the whole lane; packed to
// E2M3 by the conversion instruction and stored as the owning lane's six tile
// words per 32-value chunk (optional fp32 dump of u).
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

constexpr int kTok = 8;              // tokens per workgroup
constexpr int kThreads = 1024;       // 8 row waves + 8 lift waves
constexpr int kChunkPitch = 144;     // bytes per 32-value chunk in the lift buffer (16-byte pad)

// byte offset of 32-value chunk c in a token's lift buffer
__device__ __forceinline__ int lift_off(int c) { return c * kChunkPitch; }

// The lift waves of a 16-wave workgroup of kTok tokens (waves 8..15, lw =
// wave - 8): z of the tokens from the projection's parts (summed in a fixed
// order, bf16 hi/lo split into zh/zl), then A z on bf16 matrix cores for
// A = P (or Q), streamed from L2 in double-buffered groups of 16-row blocks;
// put(token, d, v) receives A z at columns d .. d + 3. Runs the workgroup's
// two barriers (z in LDS; results in LDS) at raised wave priority; the row
// waves meet the first as soon as their row loads are issued.
template <int D, int RK, typename Put>
__device__ __forceinline__ void lift_waves(int lw, int lane, int64_t t0, int64_t T,
                                           const float* __restrict__ Zpart, int S,
                                           const uint16_t* __restrict__ AH,
                                           const uint16_t* __restrict__ AL,
                                           uint16_t (&zh)[16][RK + 8], uint16_t (&zl)[16][RK + 8],
                                           Put put) {
  constexpr int KK = RK / 32;
  constexpr int NB = D / 128;                   // 16-column blocks per lift wave
  constexpr int QB = NB < 8 / KK ? NB : 8 / KK; // blocks per load group
  constexpr int NG = NB / QB;
  static_assert(NB % QB == 0, "groups");
  __builtin_amdgcn_s_setprio(3);
  const int i16 = lane & 15;                    // A row (column d0 + i16); B, C column (token)
  const int g = lane >> 4;
  // the wave's eighth of the columns, rotated by workgroup so that the
  // workgroups of an XCD do not all stream the same lines of A at once
  const int dw = ((lw + static_cast<int>(blockIdx.x)) & 7) * (D / 8);
  v8bf qa[2][QB][KK], qb[2][QB][KK];
  auto loadq = [&](int buf, int grp) {
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int64_t qo = static_cast<int64_t>(dw + 16 * (grp * QB + b) + i16) * RK + 32 * kk + 8 * g;
        qa[buf][b][kk] = ld8(AH + qo);
        qb[buf][b][kk] = ld8(AL + qo);
      }
  };
  loadq(0, 0);
  // z of the workgroup's tokens into LDS (MFMA columns 8..15 get zero): the
  // parts' loads are all issued before the first add, and the sum runs in
  // part order from zero
  constexpr int SP = (D + 511) / 512;           // D parts of the projection
  for (int c = lw * 64 + lane; c < 16 * RK; c += 512) {
    const int tt = c / RK;
    const int i = c % RK;
    const int64_t trow = min(t0 + (tt & 7), T - 1);
    float zp[SP];
#pragma unroll
    for (int p = 0; p < SP; ++p) zp[p] = Zpart[(static_cast<int64_t>(p) * T + trow) * RK + i];
    float z = 0.0f;
#pragma unroll
    for (int p = 0; p < SP; ++p) z += zp[p];
    z = tt < kTok ? z : 0.0f;
    const uint16_t h = f32_to_bf16(z);
    zh[tt][i] = h;
    zl[tt][i] = f32_to_bf16(z - bf16_to_f32(h));
  }
  lds_barrier();  // 1: z in LDS
  v8bf bh[KK], bl[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    bh[kk] = *reinterpret_cast<const v8bf*>(&zh[i16][32 * kk + 8 * g]);
    bl[kk] = *reinterpret_cast<const v8bf*>(&zl[i16][32 * kk + 8 * g]);
  }
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    const int buf = grp & 1;
    if (grp + 1 < NG) loadq(buf ^ 1, grp + 1);  // compile-time condition (unrolled)
    v4f acc[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      acc[b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        acc[b] = mfma(qa[buf][b][kk], bh[kk], acc[b]);
        acc[b] = mfma(qb[buf][b][kk], bh[kk], acc[b]);
        acc[b] = mfma(qa[buf][b][kk], bl[kk], acc[b]);
      }
    }
    mfma_drain();
    // C: lane holds token i16, columns d .. d + 3 of this block
    if (i16 < kTok) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
        put(i16, dw + 16 * (grp * QB + b) + 4 * g, make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]));
    }
  }
  lds_barrier();  // 2: A z in LDS
}

template <int N, int RK, bool FW, bool DBG, bool PK>
__global__ void __launch_bounds__(kThreads)
lfq_kernel(const uint16_t* __restrict__ x, int64_t T, const float* __restrict__ Zpart, int S,
           const uint16_t* __restrict__ PH, const uint16_t* __restrict__ PL,
           uint8_t* __restrict__ tiles, float* __restrict__ s_a, float* __restrict__ dbg,
           float norm, float qmax, const uint8_t* __restrict__ pre, int64_t pre_lines) {
  constexpr int D = 1 << N;
  constexpr int NCH = D / 32;                   // 32-value chunks per row
  constexpr int NS = NCH > 64 ? NCH / 64 : 1;   // chunks per lane
  constexpr int NA = NCH < 64 ? NCH : 64;       // lanes holding chunks
  constexpr int LB = N - 5 - (NS == 2 ? 1 : 0); // lane bits of the index
  constexpr int LPITCH = NCH * kChunkPitch + 64;  // bytes per token in the lift buffer
  static_assert(N >= 8 && N <= 12, "D in [256, 4096]");
  static_assert(NS <= 2, "geometry");
  __shared__ __attribute__((aligned(16))) uint8_t lift[kTok * LPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t zh[16][RK + 8];
  __shared__ __attribute__((aligned(16))) uint16_t zl[16][RK + 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // give each XCD (workgroups go to XCDs round-robin) a contiguous band of
  // token blocks, so a tile's 32 rows are written through one L2
  int64_t blk = blockIdx.x;
  if ((gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
  const int64_t t0 = blk * kTok;

  if (wave >= 8) {
    lift_waves<D, RK>(wave - 8, lane, t0, T, Zpart, S, PH, PL, zh, zl,
                      [&](int tok, int d, float4 v) {
                        *reinterpret_cast<float4*>(lift + tok * LPITCH + lift_off(d >> 5) +
                                                   (d & 31) * 4) = v;
                      });
    return;
  }

  // --------------------------------------------------------------- row waves
  const int tok = wave;
  const int64_t t = t0 + tok;
  const int64_t trow = t < T ? t : T - 1;   // rows past T repeat the last one; never stored
  const bool act = lane < NA;
  float u[NS][32];
  float m = 0.0f;
  uint4 raw[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = act ? 64 * s + lane : NCH - 1;  // unconditional load, clamped
    const uint4* p = reinterpret_cast<const uint4*>(x + trow * D + 32 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[s][q] = p[q];
  }
  // one word of a 128-byte line of the next product's weights per lane (the
  // lanes of the grid wrap over the lines), read behind the row: HBM is
  // otherwise idle while the lift streams from L2, and the product then finds
  // these lines in the caches. The value is consumed only under a condition
  // that never holds (pre_lines >= 1), so no wait for it is ever executed.
  const int64_t pl = ((static_cast<int64_t>(blockIdx.x) * 8 + tok) * 64 + lane) % pre_lines;
  const uint32_t pfv = *reinterpret_cast<const uint32_t*>(pre + pl * 128);
  lds_barrier();  // 1 (the row is still in flight)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 v = raw[s][q];
      asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
      u[s][8 * q + 0] = bf16lo(v.x); u[s][8 * q + 1] = bf16hi(v.x);
      u[s][8 * q + 2] = bf16lo(v.y); u[s][8 * q + 3] = bf16hi(v.y);
      u[s][8 * q + 4] = bf16lo(v.z); u[s][8 * q + 5] = bf16hi(v.z);
      u[s][8 * q + 6] = bf16lo(v.w); u[s][8 * q + 7] = bf16hi(v.w);
    }
  }
  if constexpr (FW) {
    // index i = 2048 s + 32 lane + j; every butterfly stage commutes with the others
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if ((j & h) == 0) {
            const float a = u[s][j], b = u[s][j + h];
            u[s][j] = a + b;
            u[s][j + h] = a - b;
          }
    if constexpr (NS == 2) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float a = u[0][j], b = u[1][j];
        u[0][j] = a + b;
        u[1][j] = a - b;
      }
    }
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg4 = (lane & 4) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
    // one lane bit at a time over every value, so that independent moves issue back to back
    if constexpr (LB > 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 32; ++j) u[s][j] = dpp_bfly<0xB1>(u[s][j], sg1);  // quad_perm 1,0,3,2
    }
    if constexpr (LB > 1) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 32; ++j) u[s][j] = dpp_bfly<0x4E>(u[s][j], sg2);  // quad_perm 2,3,0,1
    }
    if constexpr (LB > 2) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 32; ++j) u[s][j] = bfly_x4(u[s][j], sg4);
    }
    if constexpr (LB > 3) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 32; ++j) u[s][j] = dpp_bfly<0x128>(u[s][j], sg8);  // row_ror:8
    }
    if constexpr (LB > 4) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j) bfly_swap<4>(u[s][j], u[s][j + 16]);
    }
    if constexpr (LB > 5) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j) bfly_swap<5>(u[s][j], u[s][j + 16]);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < 32; ++j) u[s][j] *= norm;
  }
  // the transform has no memory accesses, so only this keeps the compiler
  // from sinking it below the barrier (behind the lift waves' work)
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < 32; ++j) asm volatile("" : "+v"(u[s][j]));
  lds_barrier();  // 2: lift in LDS
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = act ? 64 * s + lane : NCH - 1;
    const float4* p = reinterpret_cast<const float4*>(lift + tok * LPITCH + lift_off(c));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = p[q];
      u[s][4 * q + 0] += v.x; u[s][4 * q + 1] += v.y; u[s][4 * q + 2] += v.z; u[s][4 * q + 3] += v.w;
    }
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(u[s][j]));
  m = act ? m : 0.0f;
  m = wave_max(m);
  if (t < T && act) {
    const float st = m / qmax;
    if (lane == 0) s_a[t] = st;
    const RowQuant rq(st);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = 64 * s + lane;
      float q[32];
      if (!rq.fast_codes(u[s], q)) {
#pragma unroll
        for (int e = 0; e < 32; ++e) q[e] = rq.code(u[s][e]);
      }
      if constexpr (PK) {
        // packed INT4 row: element 2j in the low nibble of byte j
        uint32_t wd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wd[j] = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) wd[j] |= nib(static_cast<int>(q[8 * j + e])) << (4 * e);
        }
        *reinterpret_cast<uint4*>(tiles + t * (D / 2) + 16 * c) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      } else {
        const v6u_t w = pack_fp6_32(q);
        store_fields32(tiles, t, 32 * c, D, Field12{w[0], w[1], w[2]}, Field12{w[3], w[4], w[5]});
      }
      if constexpr (DBG) {
        float4* o = reinterpret_cast<float4*>(dbg + t * D + 32 * c);
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4)
          o[q4] = make_float4(u[s][4 * q4], u[s][4 * q4 + 1], u[s][4 * q4 + 2], u[s][4 * q4 + 3]);
      }
    }
  }
  if (pre_lines < 1) s_a[0] = __uint_as_float(pfv);
}

template <int N, int RK>
hipError_t launch_n(const uint16_t* x, int64_t T, const float* Zpart, int S, const uint16_t* PH,
                    const uint16_t* PL, bool fw, bool pk, uint8_t* tiles, float* s_a, float* dbg,
                    float qmax, hipStream_t s, const uint8_t* pre, int64_t pre_lines) {
  const float norm = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(1 << N)));
  const dim3 grid(static_cast<unsigned>((T + kTok - 1) / kTok));
#define RW4_LFQ(F, G, K)                                                                          \
  if (fw == F && (dbg != nullptr) == G && pk == K) {                                              \
    hipLaunchKernelGGL((lfq_kernel<N, RK, F, G, K>), grid, dim3(kThreads), 0, s, x, T, Zpart, S,  \
                       PH, PL, tiles, s_a, dbg, norm, qmax, pre, pre_lines);                      \
    return hipGetLastError();                                                                     \
  }
  RW4_LFQ(true, false, false) RW4_LFQ(true, true, false) RW4_LFQ(false, false, false)
  RW4_LFQ(false, true, false) RW4_LFQ(true, false, true) RW4_LFQ(true, true, true)
  RW4_LFQ(false, false, true) RW4_LFQ(false, true, true)
#undef RW4_LFQ
  return hipErrorInvalidValue;
}

template <int RK>
hipError_t launch_rk(int n, const uint16_t* x, int64_t T, const float* Zpart, int S,
                     const uint16_t* PH, const uint16_t* PL, bool fw, bool pk, uint8_t* tiles,
                     float* s_a, float* dbg, float qmax, hipStream_t s, const uint8_t* pre,
                     int64_t pl) {
  switch (n) {
    case 8: return launch_n<8, RK>(x, T, Zpart, S, PH, PL, fw, pk, tiles, s_a, dbg, qmax, s, pre, pl);
    case 9: return launch_n<9, RK>(x, T, Zpart, S, PH, PL, fw, pk, tiles, s_a, dbg, qmax, s, pre, pl);
    case 10: return launch_n<10, RK>(x, T, Zpart, S, PH, PL, fw, pk, tiles, s_a, dbg, qmax, s, pre, pl);
    case 11: return launch_n<11, RK>(x, T, Zpart, S, PH, PL, fw, pk, tiles, s_a, dbg, qmax, s, pre, pl);
    case 12: return launch_n<12, RK>(x, T, Zpart, S, PH, PL, fw, pk, tiles, s_a, dbg, qmax, s, pre, pl);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// D a power of two in [256, 4096] and r <= 64: a workgroup streams D x RK x 4
// bytes of P from L2 for 8 tokens, below the 32 bytes per value of an fp32
// round trip through memory, and the lift buffer fits LDS
bool lfq_supported(int64_t D, int64_t r) {
  return r > 0 && r <= 64 && D >= 256 && D <= 4096 && (D & (D - 1)) == 0;
}

hipError_t launch_lift_fwht_quant(const uint16_t* x, int64_t T, int64_t D, int64_t r,
                                  const void* basis, const float* Zpart, bool do_fwht,
                                  uint8_t* tiles, float* s_a, float* dbg, hipStream_t s,
                                  int bits, bool packed, const void* pre, size_t pre_bytes) {
  if (T == 0) return hipSuccess;
  if (!lfq_supported(D, r) || bits < 2 || bits > 4) return hipErrorInvalidValue;
  const float qmax = static_cast<float>((1 << (bits - 1)) - 1);
  const AlignBasis a = align_basis(basis, D, r, true);
  // without the transform the lift operand is Q itself
  const uint16_t* PH = do_fwht ? a.PH : a.QH;
  const uint16_t* PL = do_fwht ? a.PL : a.QL;
  const int S = align_parts_count(D);
  if (S != (D + 511) / 512) return hipErrorInvalidValue;  // the lift waves' part count
  int n = 0;
  while ((int64_t(1) << n) < D) ++n;
  // the read-ahead's lines; without weights, the one line read is x's first
  const bool ra = pre != nullptr && pre_bytes >= 128;
  const uint8_t* pb = ra ? static_cast<const uint8_t*>(pre) : reinterpret_cast<const uint8_t*>(x);
  const int64_t pl = ra ? static_cast<int64_t>(pre_bytes / 128) : 1;
  if (a.RK == 32)
    return launch_rk<32>(n, x, T, Zpart, S, PH, PL, do_fwht, packed, tiles, s_a, dbg, qmax, s,
                         pb, pl);
  if (a.RK == 64)
    return launch_rk<64>(n, x, T, Zpart, S, PH, PL, do_fwht, packed, tiles, s_a, dbg, qmax, s,
                         pb, pl);
  return hipErrorInvalidValue;
}

}  // namespace rw4
