// W4A4 GEMM on gfx950 int8 MFMA ("Infra Quant II", QuaRot Method: INT4 x INT4
// products accumulated in INT32, then scaled by the activation row scale and
// the weight column scale).
//
// gfx950 has no INT4 matrix instruction, so the packed nibbles are widened to
// int8 in registers and fed to v_mfma_i32_32x32x32_i8. The widening keeps each
// nibble in the HIGH half of its byte ((w << 4) & 0xF0F0F0F0 for the even
// elements, w & 0xF0F0F0F0 for the odd ones): each int8 then equals 16 * code,
// every product carries a factor 256, and the int32 sum S' = 256 S is shifted
// right by 8 at the end. Each product of two codes lies in [-56, 64] (-8 * -8
// is the only one above 49), so S lies in [-56 K, 64 K]. For K < 131072, 256 S
// stays inside int32; at K = 131072 the single value S = 64 K = 2^23 (every
// code -8 in both rows) gives 256 S = 2^31, which int32 cannot hold: the
// accumulator then reads -2^31 (wrapped) or 2^31 - 1 (saturated). Neither can
// be 256 S for an S in range (-2^23 is below -56 K, and 2^31 - 1 is no
// multiple of 256), so unscale() maps both to 2^23 and every result is exact
// for K <= 131072. The widened
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

// the integer sum S from the accumulator of 256 S (the header comment above)
__device__ __forceinline__ int unscale(int acc) {
  return (acc == INT32_MIN || acc == INT32_MAX) ? (1 << 23) : (acc >> 8);
}

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
            o[c] = f32_to_bf16((static_cast<float>(unscale(acc[i][j][4 * q + c])) * sa) * swv[c]);
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
        store_stream16(yp, v);
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
          for (int c = 0; c < 4; ++c) vals[c] = unscale(acc[i][j][4 * q + c]);
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

// ----------------------------------------------------------------------------
// Decode products (T <= 16 tokens): the weights stream once from HBM as packed
// INT4 rows (0.5 bytes per code), so the kernel is bound by that stream. A
// workgroup owns 16 weight rows; its NWV waves split K into steps of 256 codes
// (128 bytes of every row, whole cache lines), wave w taking steps w, w + NWV,
// ..., and issues the loads of SPW of its steps at once (a round), none past
// the end of K. Lane l holds row l % 16 and the 32-byte quarter l / 16 of each
// step as two 16-byte loads. When the T activation rows fit (ALDS bytes), the
// workgroup copies them into LDS once, while its first weight round is in
// flight, instead of every wave loading them from L2 for every step (measured
// at T = 8, 4096 -> 32768: 15.0 against 20.1 us). Each 16-byte load widens
// (16 * code, as above) into the operands of two v_mfma_i32_16x16x64_i8 with
// weight rows as the A operand and tokens as the B operand; token rows past T
// hold zero. The waves' partial sums (all of the form 256 S, added modulo 2^32)
// are summed through LDS in wave order, then unscaled.
constexpr int kDecRows = 16;
constexpr int kDecLds = 32768;  // activation bytes (T * K / 2) staged in LDS at most

constexpr int kResRmax = 128;   // basis width (RK) a residual epilogue takes at most

template <int NWV, int SPW, bool ALDS, bool I32OUT, bool RES>
__global__ void __launch_bounds__(64 * NWV)
gemm_decode_kernel(const uint8_t* __restrict__ a, const float* __restrict__ s_a,
                   const uint8_t* __restrict__ w, const float* __restrict__ s_w,
                   void* __restrict__ y, int T, int K, int N, GemmResidual res) {
  __shared__ uint32_t red[NWV][4][64];
  __shared__ __attribute__((aligned(16))) uint8_t al[ALDS ? kDecLds : 16];
  __shared__ float zsm[RES ? kDecRows : 1][RES ? kResRmax + 1 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * kDecRows;
  const int KB = K / 2;                       // bytes per row
  const int nstep = (KB + 127) / 128;         // 128-byte steps (the last may be partial)
  const int i = lane & 15, g = lane >> 4;
  // rows past N re-read the last row (their sums are never stored); token rows
  // past T read the last token and are zeroed
  const uint8_t* wrow = w + static_cast<int64_t>(min(n0 + i, N - 1)) * KB;
  const int arow = min(i, T - 1) * KB;
  const uint32_t mtok = i < T ? 0xFFFFFFFFu : 0u;
  uint4 wv[SPW][2];
  // lane's 16 bytes of step st, half h; quarters past the end of K read the
  // row's first 16 bytes (K >= 32) and are masked to zero
  auto offs = [&](int st, int h, uint32_t& m) {
    const int off = st * 128 + 64 * h + 16 * g;
    const bool ok = off + 16 <= KB;
    m = ok ? 0xFFFFFFFFu : 0u;
    return ok ? off : 0;
  };
  auto load = [&](int s0) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int st = s0 + wave + NWV * u;
      if (st < nstep) {  // uniform
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t m;
          const int o = offs(st, h, m);
          wv[u][h] = *reinterpret_cast<const uint4*>(wrow + o);
        }
      }
    }
  };
  load(0);
  // an epilogue thread's output (token et, row en) is known now: its skip
  // value and the first 32 values of its basis row load with the weights
  const int ev = threadIdx.x >> 6, el = threadIdx.x & 63;
  const int et = el & 15, en = n0 + 4 * (el >> 4) + ev;
  const bool eact = RES && threadIdx.x < 256 && et < T && en < N;
  uint4 eqh[4], eql[4];
  uint16_t exr = 0;
  if constexpr (RES) {
    const int64_t row = static_cast<int64_t>(eact ? en : 0) * res.RK;
    const uint4* qh = reinterpret_cast<const uint4*>(res.QH + row);
    const uint4* ql = reinterpret_cast<const uint4*>(res.QL + row);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      eqh[j] = qh[j];
      eql[j] = ql[j];
    }
    exr = res.x[static_cast<int64_t>(eact ? et : 0) * N + (eact ? en : 0)];
  }
  if constexpr (RES) {
    // z of the T tokens: the projection's chunk partials summed in chunk
    // order from zero, as the short-batch lift sums them
    for (int o = threadIdx.x; o < T * res.RK; o += 64 * NWV) {
      const int t = o / res.RK, i = o % res.RK;
      float z = 0.0f;
      for (int c0 = 0; c0 < res.C; c0 += 16) {
        float zp[16];
#pragma unroll
        for (int c = 0; c < 16; ++c)
          zp[c] = res.Zs[(static_cast<int64_t>(min(c0 + c, res.C - 1)) * T + t) * res.RK + i];
#pragma unroll
        for (int c = 0; c < 16; ++c) z += c0 + c < res.C ? zp[c] : 0.0f;
      }
      zsm[t][i] = z;
    }
  }
  if constexpr (ALDS) {
    const int nbytes = T * KB;  // a multiple of 16 (K % 32 == 0)
    for (int o = threadIdx.x * 16; o < nbytes; o += 64 * NWV * 16)
      *reinterpret_cast<uint4*>(al + o) = *reinterpret_cast<const uint4*>(a + o);
    __syncthreads();
  }
  v4i acc = {0, 0, 0, 0};
  for (int s0 = 0; s0 < nstep; s0 += NWV * SPW) {
    if (s0 > 0) load(s0);
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int st = s0 + wave + NWV * u;
      if (st < nstep) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t m;
          const int o = offs(st, h, m);
          uint4 va = ALDS ? *reinterpret_cast<const uint4*>(al + arow + o)
                          : *reinterpret_cast<const uint4*>(a + arow + o);
          uint4 vw = wv[u][h];
          const uint32_t ma = m & mtok;
          vw.x &= m; vw.y &= m; vw.z &= m; vw.w &= m;
          va.x &= ma; va.y &= ma; va.z &= ma; va.w &= ma;
          v4i w0, w1, a0, a1;
          widen(vw, w0, w1);
          widen(va, a0, a1);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w0, a0, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w1, a1, acc, 0, 0, 0);
        }
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][v][lane] = static_cast<uint32_t>(acc[v]);
  __syncthreads();
  if (threadIdx.x >= 256) return;
  // thread (v, l): weight row 4 (l / 16) + v of the block, token l % 16
  const int v = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = l & 15;
  const int n = n0 + 4 * (l >> 4) + v;
  if (t >= T || n >= N) return;
  uint32_t sum = 0;
#pragma unroll
  for (int ww = 0; ww < NWV; ++ww) sum += red[ww][v][l];
  const int S = unscale(static_cast<int>(sum));
  const int64_t off = static_cast<int64_t>(t) * N + n;
  if constexpr (I32OUT) {
    static_cast<int32_t*>(y)[off] = S;
  } else {
    const uint16_t yb = f32_to_bf16((static_cast<float>(S) * s_a[t]) * s_w[n]);
    static_cast<uint16_t*>(y)[off] = yb;
    if constexpr (RES) {
      // x + Q z with Q = Qh + Ql in fp32 and the FMAs in basis order (the
      // short-batch lift's arithmetic), then the block output, one rounding
      const uint4* qh = reinterpret_cast<const uint4*>(res.QH + static_cast<int64_t>(n) * res.RK);
      const uint4* ql = reinterpret_cast<const uint4*>(res.QL + static_cast<int64_t>(n) * res.RK);
      float corr = 0.0f;
      // basis values i0 .. i0 + 31 in fp32 (hi + lo), FMAs in basis order; the
      // first 32 come from the registers loaded at the start
      auto chunk = [&](const uint4 (&hv)[4], const uint4 (&lv)[4], int i0) {
        float q[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t hw[4] = {hv[j].x, hv[j].y, hv[j].z, hv[j].w};
          const uint32_t lw[4] = {lv[j].x, lv[j].y, lv[j].z, lv[j].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            q[8 * j + 2 * e] = bf16lo(hw[e]) + bf16lo(lw[e]);
            q[8 * j + 2 * e + 1] = bf16hi(hw[e]) + bf16hi(lw[e]);
          }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) corr = fmaf(q[i], zsm[t][i0 + i], corr);
      };
      chunk(eqh, eql, 0);
      for (int i0 = 32; i0 < res.RK; i0 += 32) {
        uint4 hv[4], lv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hv[j] = qh[i0 / 8 + j];
          lv[j] = ql[i0 / 8 + j];
        }
        chunk(hv, lv, i0);
      }
      float acc = bf16_to_f32(exr) + corr;
      acc += bf16_to_f32(yb);
      res.out[off] = f32_to_bf16(acc);
    }
  }
}

template <int NWV, int SPW, bool RES = false>
hipError_t launch_decode(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                         void* y, bool i32_out, int64_t T, int64_t K, int64_t N, hipStream_t s,
                         const GemmResidual& res = GemmResidual{}) {
  const int64_t nb = (N + kDecRows - 1) / kDecRows;
  if (nb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (RES && (i32_out || res.RK > kResRmax || res.RK % 32 != 0)) return hipErrorInvalidValue;
  const bool alds = T * (K / 2) <= kDecLds;
#define RW4_DEC(AL, I)                                                                           \
  if (alds == AL && i32_out == I) {                                                              \
    hipLaunchKernelGGL((gemm_decode_kernel<NWV, SPW, AL, I, RES>),                                \
                       dim3(static_cast<unsigned>(nb)), dim3(64 * NWV), 0, s, a, s_a, w, s_w, y,  \
                       static_cast<int>(T), static_cast<int>(K), static_cast<int>(N), res);      \
    return hipGetLastError();                                                                    \
  }
  RW4_DEC(true, false) RW4_DEC(false, false)
  if constexpr (!RES) {
    RW4_DEC(true, true) RW4_DEC(false, true)
  }
#undef RW4_DEC
  return hipErrorInvalidValue;
}

// the decode shapes of launch_gemm, with the residual epilogue
template <bool RES>
hipError_t launch_decode_any(const uint8_t* a, const float* s_a, const uint8_t* w,
                             const float* s_w, void* y, bool i32_out, int64_t T, int64_t K,
                             int64_t N, hipStream_t s, const GemmResidual& res) {
  // weight streaming. Measured at T = 8 (weights rotated past the last-level
  // cache): up to 256 workgroups (N <= 4096), 16 waves with one step each
  // per round (4096 x 4096: 4.0 us); K beyond 4096 codes, 16 waves with four
  // steps each (16384 x 4096: 9.8 us); otherwise 8 waves with two steps each
  // (4096 x 12288: 7.7 us; 4096 x 32768: 15.0 us).
  const int64_t nb = (N + kDecRows - 1) / kDecRows;
  if (K > 4096) return launch_decode<16, 4, RES>(a, s_a, w, s_w, y, i32_out, T, K, N, s, res);
  if (nb <= 256) return launch_decode<16, 1, RES>(a, s_a, w, s_w, y, i32_out, T, K, N, s, res);
  return launch_decode<8, 2, RES>(a, s_a, w, s_w, y, i32_out, T, K, N, s, res);
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
  if (T <= gemm::kDecRows)
    return gemm::launch_decode_any<false>(a, s_a, w, s_w, y, i32_out, T, K, N, s, GemmResidual{});
  return gemm::launch_cfg<2, 2, 2, 2>(a, s_a, w, s_w, y, i32_out, T, K, N, s);
}

hipError_t launch_gemm_residual(const uint8_t* a, const float* s_a, const uint8_t* w,
                                const float* s_w, uint16_t* y, const GemmResidual& res, int64_t T,
                                int64_t K, int64_t N, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > gemm::kDecRows) return hipErrorInvalidValue;
  return gemm::launch_decode_any<true>(a, s_a, w, s_w, y, false, T, K, N, s, res);
}

}  // namespace rw4
