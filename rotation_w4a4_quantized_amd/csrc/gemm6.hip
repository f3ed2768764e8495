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
// Four kernels:
//
// * gemm6_lds_kernel (K % 128 == 0, T >= 128): a workgroup of WW x WT waves
//   computes a (WW FW 32) x (WT FT 32) output block; each wave owns FW x FT
//   32 x 32 fragments. Operand tiles for two k-tiles (128 k) at a time are
//   copied straight from global memory into LDS with the gfx950 global->LDS
//   loads (no VGPR staging), into a ring of S stage buffers, and every wave
//   reads its fragments from LDS. Sharing the block's tiles among its waves
//   cuts the L2 traffic per MFMA by the wave-grid factor, which is what bounds
//   a one-wave-per-tile kernel on this chip.
// * gemm6_kernel (any K % 64 == 0, and small T): one wave per workgroup,
//   BW x BT fragments, tiles read straight into registers, PD k-tiles in
//   flight.
// * gemm6_decode16_kernel (T <= 16, N <= 16384) and gemm6_decode_kernel
//   (T <= 32): 16 or 32 weight rows per workgroup whose waves split K, for the
//   weight-streaming decode products.
//
// In both, workgroups are renumbered so that each XCD works on a contiguous
// band of weight tiles, and the bf16 epilogue is staged in LDS so that rows
// are written with 16-byte stores.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace g6 {

typedef int v8i __attribute__((ext_vector_type(8)));

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
        store_stream16(o, v);
      } else {
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&stage[row * SP + col]);
        for (int k = 0; k < 8 && n + k < N; ++k) o[k] = e[k];
      }
    }
  }
}

// ---------------------------------------------------------------- LDS-staged kernel
//
// The copies are written as inline assembly on purpose. The compiler's own
// global->LDS builtin makes its wait-count pass drain every copy in flight
// before each LDS read that it cannot prove disjoint from them, which turns
// the S-stage ring into a fully serialized one. Here the compiler does not see
// the LDS writes, and the kernel orders them itself:
//   * a copy into stage buffer b is issued only after a workgroup barrier that
//     every wave reaches after its LDS reads of b completed (lgkmcnt(0));
//   * a wave reads stage i only after waiting until at most (S-2) stages of
//     its own copies are in flight (vmcnt, in issue order) and a barrier, so
//     every wave's copies of stage i have landed.
// The copy instruction takes its LDS base from m0, which it sets itself; no
// other code in these kernels uses m0.
typedef const __attribute__((address_space(3))) uint8_t* lds_cptr;
// wave-uniform LDS byte address of a pointer into a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cptr)p)));
}
// 16 bytes per lane: lds + 16 lane <- base + off (wave-uniform base, per-lane
// 32-bit offset)
__device__ __forceinline__ void lds_copy16(const void* base, uint32_t off, const void* lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "s"(lds_addr(lds))
               : "memory");
}
// 4 bytes per lane: lds + 4 lane <- g (per-lane address)
__device__ __forceinline__ void lds_copy4(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr(lds))
               : "memory");
}
// workgroup barrier that the compiler may not move memory accesses across
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// wait until this wave's LDS reads are done and at most N of its vector
// memory loads (here: copies) are in flight
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

template <int FW, int FT, int WW, int WT, int S, bool I32OUT>
__global__ void __launch_bounds__(64 * WW * WT)
gemm6_lds_kernel(const uint8_t* __restrict__ at, const float* __restrict__ s_a,
                 const uint8_t* __restrict__ wt, const float* __restrict__ s_w,
                 void* __restrict__ y, int T, int K, int N, int rt, int st_t,
                 int st_n) {
  constexpr int NW = WW * WT;
  constexpr int TW = WW * FW * 32, TT = WT * FT * 32;
  constexpr int NRB = WW * FW + WT * FT;      // 32-row blocks of the workgroup (W, then A)
  constexpr int STAGE = NRB * 2 * kTileBytes;  // two k-tiles of each row block
  constexpr int NI = STAGE / 1024;             // 1 KiB copies per stage
  constexpr int LPW = (NI + NW - 1) / NW;      // copies per wave; the last round may repeat one
  constexpr int SPW = FW * 32 + 8;             // bf16 pitch of a wave's staged rows
  static_assert(S == 3 || S == 4, "stages");
  static_assert(TW <= 256 && TT <= 256, "blocks stay inside the 256-row padding");
  static_assert(NW * 32 * SPW * 2 <= STAGE, "epilogue staging fits one stage buffer");
  static_assert((S - 2) * LPW < 64, "vmcnt range");
  // one LDS object per stage, so that each is addressed with constants
  __shared__ __attribute__((aligned(16))) uint8_t L0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t L1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t L2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t L3[S > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) float sc[I32OUT ? 4 : TW + TT];  // s_w block | s_a block

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ww = wave % WW, wq = wave / WW;
  const int nwt = (N + TW - 1) / TW, ntt = (T + TT - 1) / TT, nb = nwt * ntt;
  // Workgroups are dispatched to the 8 XCDs round robin (b mod 8). With rt > 0
  // the tile grid is cut into 8 rectangles, rt along T by 8 / rt along N, and
  // XCD x takes rectangle x, so its L2 fetches only that rectangle's A and W
  // rows; rt = 0 gives each XCD a run of consecutive tiles instead. Inside
  // its rectangle an XCD takes super-tiles of st_t x st_n tiles (dividing the
  // rectangle's sides), T-fastest within and between them, so that the tiles
  // resident at once share few rows.
  int tb, nbk;
  {
    int b = blockIdx.x;
    if (rt > 0) {
      const int x = b & 7, l = b >> 3, rtt = ntt / rt, rnn = nwt / (8 / rt);
      const int per = st_t * st_n;
      const int sblk = l / per, w = l % per, nst = rtt / st_t;
      tb = (x % rt) * rtt + (sblk % nst) * st_t + w % st_t;
      nbk = (x / rt) * rnn + (sblk / nst) * st_n + w / st_t;
    } else {
      if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
      tb = b % ntt;
      nbk = b / ntt;
    }
  }
  const int n0 = nbk * TW, t0 = tb * TT;
  const int KT = K >> 6, KS = KT >> 1;  // k-tiles, stages

  // Copy i of a stage moves bytes [1024 i, 1024 i + 1024) of the stage: row
  // block i / 3, third i % 3 of its two consecutive k-tiles (3072 contiguous
  // bytes in the tile layout). The stage buffer keeps that order.
  // The copies address the block's first W and A rows (wave-uniform bases) plus
  // a per-lane 32-bit offset: at most 8 row blocks of K / 64 tiles, which for
  // K <= 131072 stays below 2^25.
  const uint8_t* const wb = wt + static_cast<int64_t>(n0 >> 5) * KT * kTileBytes;
  const uint8_t* const ab = at + static_cast<int64_t>(t0 >> 5) * KT * kTileBytes;
  bool isw[LPW];
  uint32_t src[LPW];
  int dst[LPW];
#pragma unroll
  for (int m = 0; m < LPW; ++m) {
    int i = wave + NW * m;
    if (i >= NI) i -= NW;
    const int rb = i / 3;
    isw[m] = rb < WW * FW;
    src[m] = static_cast<uint32_t>(isw[m] ? rb : rb - WW * FW) * KT * kTileBytes +
             (i % 3) * 1024 + lane * 16;
    dst[m] = i * 1024;
  }
  auto fetch = [&](uint8_t* L, int st) {
    const int64_t so = static_cast<int64_t>(st) * (2 * kTileBytes);
#pragma unroll
    for (int m = 0; m < LPW; ++m) lds_copy16(isw[m] ? wb + so : ab + so, src[m], L + dst[m]);
  };
  // the block's scales go first, so the first stage wait covers them
  if constexpr (!I32OUT) {
    static_assert((TW + TT) % 64 == 0, "scale copies");
    for (int m = wave; m < (TW + TT) / 64; m += NW) {
      const int e = m * 64 + lane;
      const float* p = e < TW ? s_w + min(n0 + e, N - 1) : s_a + min(t0 + e - TW, T - 1);
      lds_copy4(p, sc + m * 64);
    }
  }

  v16f acc[FW][FT];
#pragma unroll
  for (int i = 0; i < FW; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto compute = [&](const uint8_t* L) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i ow[FW], oa[FT];
#pragma unroll
      for (int i = 0; i < FW; ++i) {
        const uint8_t* q = L + (ww * FW + i) * (2 * kTileBytes) + h * kTileBytes;
        ow[i] = opnd(*reinterpret_cast<const uint4*>(q + lane * 16),
                     *reinterpret_cast<const uint2*>(q + kPlane1 + lane * 8));
      }
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const uint8_t* q = L + (WW * FW + wq * FT + j) * (2 * kTileBytes) + h * kTileBytes;
        oa[j] = opnd(*reinterpret_cast<const uint4*>(q + lane * 16),
                     *reinterpret_cast<const uint2*>(q + kPlane1 + lane * 8));
      }
#pragma unroll
      for (int i = 0; i < FW; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ow[i], oa[j], acc[i][j], 2,
                                                                      2, 0, 127, 0, 127);
    }
  };
  // stage i lives in buffer i % S; step i refills the buffer read in step i - 1
  auto step = [&](int i, const uint8_t* cur, uint8_t* nxt) {
    wait_copies<(S - 2) * LPW>();
    block_barrier();
    fetch(nxt, i + S - 1 < KS ? i + S - 1 : KS - 1);  // clamped copies are harmless repeats
    compute(cur);
  };
  fetch(L0, 0);
  fetch(L1, 1 < KS ? 1 : KS - 1);
  if constexpr (S > 3) fetch(L2, 2 < KS ? 2 : KS - 1);
  int i = 0;
  for (; i + S <= KS; i += S) {
    if constexpr (S == 3) {
      step(i, L0, L2);
      step(i + 1, L1, L0);
      step(i + 2, L2, L1);
    } else {
      step(i, L0, L3);
      step(i + 1, L1, L0);
      step(i + 2, L2, L1);
      step(i + 3, L3, L2);
    }
  }
  const int rem = KS - i;  // uniform
  if (rem > 0) step(i, L0, S == 3 ? L2 : L3);
  if (rem > 1) step(i + 1, L1, L0);
  if constexpr (S > 3)
    if (rem > 2) step(i + 2, L2, L1);
  // all copies (the repeats included) have landed and every wave is done with
  // the stage buffers before L0 is reused for the epilogue
  __builtin_amdgcn_s_waitcnt(0);
  block_barrier();
  // results of the last MFMAs are read by plain VALU code below
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_sched_barrier(0);

  // accumulator element (i, j, v): weight row wn0 + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4,
  // token wt0 + 32 j + lane % 32
  const int wn0 = n0 + ww * FW * 32, wt0 = t0 + wq * FT * 32;
  if constexpr (I32OUT) {
    int32_t* yo = static_cast<int32_t*>(y);
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int t = wt0 + 32 * j + (lane & 31);
      if (t >= T) continue;
#pragma unroll
      for (int ii = 0; ii < FW; ++ii)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = wn0 + 32 * ii + 8 * q + 4 * (lane >> 5);
          int32_t* o = yo + static_cast<int64_t>(t) * N + n;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (n + c < N) o[c] = static_cast<int32_t>(acc[ii][j][4 * q + c]);
        }
    }
  } else {
    // each wave stages 32 tokens x FW * 32 columns at a time in its own part of L0
    uint16_t* st = reinterpret_cast<uint16_t*>(L0) + wave * 32 * SPW;
    uint16_t* yo = static_cast<uint16_t*>(y);
    const int tl = lane & 31;
    // every scale this lane needs, read from LDS together (one wait instead
    // of one per fragment)
    float4 swv[FW][4];
    float sav[FT];
#pragma unroll
    for (int ii = 0; ii < FW; ++ii)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        swv[ii][q] = *reinterpret_cast<const float4*>(
            &sc[ww * FW * 32 + 32 * ii + 8 * q + 4 * (lane >> 5)]);
#pragma unroll
    for (int j = 0; j < FT; ++j) sav[j] = sc[TW + wq * FT * 32 + 32 * j + tl];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const float sa = sav[j];
#pragma unroll
      for (int ii = 0; ii < FW; ++ii)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = 32 * ii + 8 * q + 4 * (lane >> 5);
          const float4 sw = swv[ii][q];
          const float v0 = (acc[ii][j][4 * q + 0] * sa) * sw.x;
          const float v1 = (acc[ii][j][4 * q + 1] * sa) * sw.y;
          const float v2 = (acc[ii][j][4 * q + 2] * sa) * sw.z;
          const float v3 = (acc[ii][j][4 * q + 3] * sa) * sw.w;
          *reinterpret_cast<uint2*>(&st[tl * SPW + nl]) =
              make_uint2(f32_to_bf16(v0) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16),
                         f32_to_bf16(v2) | (static_cast<uint32_t>(f32_to_bf16(v3)) << 16));
        }
      // the wave reads back only what it wrote (LDS accesses of a wave are in
      // order): all of this row group's chunks first, then their stores
      constexpr int CPR = FW * 4;          // 16-byte chunks per staged row
      constexpr int RPJ = 32 * CPR / 64;   // chunks per lane
      uint4 cv[RPJ];
#pragma unroll
      for (int k = 0; k < RPJ; ++k) {
        const int c = lane + 64 * k;
        cv[k] = *reinterpret_cast<const uint4*>(&st[(c / CPR) * SPW + (c % CPR) * 8]);
      }
#pragma unroll
      for (int k = 0; k < RPJ; ++k) {
        const int c = lane + 64 * k;
        const int row = c / CPR, col = (c % CPR) * 8;
        const int t = wt0 + 32 * j + row, n = wn0 + col;
        if (t < T && n < N) {
          uint16_t* o = yo + static_cast<int64_t>(t) * N + n;
          if (n + 8 <= N && (N & 7) == 0) {
            store_stream16(o, cv[k]);
          } else {
            const uint32_t wv[4] = {cv[k].x, cv[k].y, cv[k].z, cv[k].w};
            for (int e = 0; e < 8 && n + e < N; ++e)
              o[e] = static_cast<uint16_t>(wv[e >> 1] >> (16 * (e & 1)));
          }
        }
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

// Decode products (T <= 32: one token tile). A workgroup of 16 waves owns 32
// weight rows; wave w takes the k-tiles w, w + 16, ... of the whole K, and
// the 16 partial 32 x 32 accumulators are then summed through LDS in wave
// order (deterministic) before the epilogue writes the T valid token columns.
// Lanes whose token row is past T load nothing and hold zeros: those rows
// only reach output columns that are never written, and at T = 8 this drops
// three quarters of the activation loads, which at K = 4096 are as many as the
// weight loads. One k-tile in flight per wave streams the weights as fast as
// four did: the chip-wide stream, not the per-wave depth, is the limit.
constexpr int kDecWaves = 16;
constexpr int kDecPD = 1;   // k-tiles a wave has in flight

template <bool I32OUT>
__global__ void __launch_bounds__(64 * kDecWaves)
gemm6_decode_kernel(const uint8_t* __restrict__ at, const float* __restrict__ s_a,
                    const uint8_t* __restrict__ wt, const float* __restrict__ s_w,
                    void* __restrict__ y, int T, int K, int N) {
  __shared__ float red[kDecWaves][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = (N + 31) / 32;
  int b = blockIdx.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int n0 = b * 32;
  const int KT = K >> 6;
  const uint8_t* wrow = wt + static_cast<int64_t>(n0 >> 5) * KT * kTileBytes;
  const uint8_t* arow = at;                      // token tile 0
  v16f acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  // rounds of kDecPD k-tiles: every load of a round is issued before its MFMAs
  for (int k0 = wave; k0 < KT; k0 += kDecWaves * kDecPD) {
    uint4 w0[kDecPD], a0[kDecPD];
    uint2 w1[kDecPD], a1[kDecPD];
#pragma unroll
    for (int u = 0; u < kDecPD; ++u) {
      const int kt = k0 + u * kDecWaves;
      const int kc = kt < KT ? kt : k0;          // past the end: a harmless repeat, not used
      const uint8_t* pw = wrow + static_cast<int64_t>(kc) * kTileBytes;
      const uint8_t* pa = arow + static_cast<int64_t>(kc) * kTileBytes;
      w0[u] = *reinterpret_cast<const uint4*>(pw + lane * 16);
      w1[u] = *reinterpret_cast<const uint2*>(pw + kPlane1 + lane * 8);
      if ((lane & 31) < T) {
        a0[u] = *reinterpret_cast<const uint4*>(pa + lane * 16);
        a1[u] = *reinterpret_cast<const uint2*>(pa + kPlane1 + lane * 8);
      } else {
        a0[u] = make_uint4(0, 0, 0, 0);
        a1[u] = make_uint2(0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kDecPD; ++u)
      if (k0 + u * kDecWaves < KT)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opnd(w0[u], w1[u]), opnd(a0[u], a1[u]),
                                                              acc, 2, 2, 0, 127, 0, 127);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int v = 0; v < 16; ++v) red[wave][v][lane] = acc[v];
  __syncthreads();
  // thread (v, l): weight row 8 (v / 4) + 4 (l / 32) + v % 4, token l % 32
  const int v = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = l & 31;
  const int n = n0 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
  if (t >= T || n >= N) return;
  float sum = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) sum += red[w][v][l];
  if constexpr (I32OUT) {
    static_cast<int32_t*>(y)[static_cast<int64_t>(t) * N + n] = static_cast<int32_t>(sum);
  } else {
    static_cast<uint16_t*>(y)[static_cast<int64_t>(t) * N + n] = f32_to_bf16((sum * s_a[t]) * s_w[n]);
  }
}

// Decode products with at most 16 tokens on 16 x 16 x 128 MFMAs: 16 weight
// rows per workgroup, twice the workgroups of the 32-row kernel, which leaves
// half of the CUs idle at N = 4096. The operands come straight from the
// 32-row tiles: operand lane l holds row l % 16 and K values 32 (l / 16) ..
// + 31 of a 128-wide step, which is lane slot 32 ((l / 16) % 2) + row of
// k-tile 2 kp + l / 32 (the 32 x 32 x 64 layout's K halves). NWV waves split
// the k-pairs; the partial 16 x 16 sums are added through LDS in wave order.
template <int NWV, bool I32OUT>
__global__ void __launch_bounds__(64 * NWV)
gemm6_decode16_kernel(const uint8_t* __restrict__ at, const float* __restrict__ s_a,
                      const uint8_t* __restrict__ wt, const float* __restrict__ s_w,
                      void* __restrict__ y, int T, int K, int N) {
  __shared__ float red[NWV][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = (N + 15) / 16;
  int b = blockIdx.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int n0 = b * 16;
  const int KT = K >> 6, KP = (KT + 1) >> 1;  // k-tiles, 128-wide steps (the last may be half)
  const uint8_t* wrow = wt + static_cast<int64_t>(n0 >> 5) * KT * kTileBytes;
  const int c = lane >> 4;
  const int tsub = c >> 1;
  const int wslot = (c & 1) * 32 + (n0 & 16) + (lane & 15);
  const int aslot = (c & 1) * 32 + (lane & 15);
  const bool aload = (lane & 15) < T;  // token rows past T hold zeros
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int kp = wave; kp < KP; kp += NWV) {
    const int kt = 2 * kp + tsub;
    uint4 w0 = make_uint4(0, 0, 0, 0), a0 = make_uint4(0, 0, 0, 0);
    uint2 w1 = make_uint2(0, 0), a1 = make_uint2(0, 0);
    if (kt < KT) {
      const uint8_t* pw = wrow + static_cast<int64_t>(kt) * kTileBytes;
      w0 = *reinterpret_cast<const uint4*>(pw + wslot * 16);
      w1 = *reinterpret_cast<const uint2*>(pw + kPlane1 + wslot * 8);
      if (aload) {
        const uint8_t* pa = at + static_cast<int64_t>(kt) * kTileBytes;
        a0 = *reinterpret_cast<const uint4*>(pa + aslot * 16);
        a1 = *reinterpret_cast<const uint2*>(pa + kPlane1 + aslot * 8);
      }
    }
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(opnd(w0, w1), opnd(a0, a1), acc, 2, 2,
                                                           0, 127, 0, 127);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (threadIdx.x >= 256) return;
  // thread (i, l): weight row 4 (l / 16) + i, token l % 16
  const int i = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = l & 15;
  const int n = n0 + 4 * (l >> 4) + i;
  if (t >= T || n >= N) return;
  float sum = 0.0f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) sum += red[w][i][l];
  if constexpr (I32OUT) {
    static_cast<int32_t*>(y)[static_cast<int64_t>(t) * N + n] = static_cast<int32_t>(sum);
  } else {
    static_cast<uint16_t*>(y)[static_cast<int64_t>(t) * N + n] = f32_to_bf16((sum * s_a[t]) * s_w[n]);
  }
}

template <int NWV>
hipError_t launch_decode16(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                           void* y, bool i32_out, int64_t T, int64_t K, int64_t N, hipStream_t s) {
  const unsigned nb = static_cast<unsigned>((N + 15) / 16);
  if (i32_out)
    hipLaunchKernelGGL((gemm6_decode16_kernel<NWV, true>), dim3(nb), dim3(64 * NWV), 0, s, a, s_a,
                       w, s_w, y, static_cast<int>(T), static_cast<int>(K), static_cast<int>(N));
  else
    hipLaunchKernelGGL((gemm6_decode16_kernel<NWV, false>), dim3(nb), dim3(64 * NWV), 0, s, a, s_a,
                       w, s_w, y, static_cast<int>(T), static_cast<int>(K), static_cast<int>(N));
  return hipGetLastError();
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

// rt for gemm6_lds_kernel: the split of the tile grid into 8 XCD rectangles
// (rt along T, 8 / rt along N) with the fewest A and W rows per XCD, or 0
// when no split divides the grid evenly
inline int xcd_regions(int64_t ntt, int64_t nwt, int64_t TT, int64_t TW) {
  int best = 0;
  int64_t cost = 0;
  for (int rt = 1; rt <= 8; rt *= 2) {
    const int rn = 8 / rt;
    if (ntt % rt || nwt % rn) continue;
    const int64_t c = (ntt / rt) * TT + (nwt / rn) * TW;
    if (best == 0 || c < cost) best = rt, cost = c;
  }
  return best;
}

// The super-tile {st_t, st_n} an XCD walks its rtt x rnn rectangle in: when
// the rectangle holds more tiles than the XCD runs at once (its CUs' resident
// workgroups), the st_t x st_n tiles resident together (st_t dividing rtt,
// st_n = resident / st_t dividing rnn) with the fewest A and W rows;
// otherwise, or when none divides, the whole T side (the rectangle's tiles
// T-fastest). On 256 x 256 tiles at 4096 -> 32768, T = 4096 (a 16 x 16
// rectangle, 32 resident) this takes 4 x 8 super-tiles: 9 instead of
// 13.5 MiB of operand rows per resident set. Measured on MI355X: prefill
// layer (T = 4096) 936 -> 910 us, 70B-shaped linear 1279 -> 1253 us.
struct SuperTile { int t, n; };
inline SuperTile xcd_supertile(int64_t rtt, int64_t rnn, int64_t TT, int64_t TW,
                               int64_t resident) {
  SuperTile best{static_cast<int>(rtt), 1};
  if (rtt * rnn <= resident || resident < 1) return best;
  int64_t cost = -1;
  for (int64_t st = 1; st <= rtt && st <= resident; st *= 2) {
    if (rtt % st || resident % st) continue;
    const int64_t sn = resident / st;
    if (rnn % sn) continue;
    const int64_t c = st * TT + sn * TW;
    if (cost < 0 || c < cost) cost = c, best = SuperTile{static_cast<int>(st), static_cast<int>(sn)};
  }
  return best;
}

template <int FW, int FT, int WW, int WT, int S, bool I32>
hipError_t launch_lds(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                      void* y, int64_t T, int64_t K, int64_t N, hipStream_t s) {
  constexpr int64_t TW = WW * FW * 32, TT = WT * FT * 32;
  const int64_t nwt = (N + TW - 1) / TW, ntt = (T + TT - 1) / TT, nb = nwt * ntt;
  if (nb > 0x7FFFFFFF || K < 128 || K % 128) return hipErrorInvalidConfiguration;
  const int rt = xcd_regions(ntt, nwt, TT, TW);
  // workgroups resident per CU: the 4-wave blocks take 74 KiB of LDS (two per
  // CU), the 8-wave ones 110-146 KiB (one)
  const int64_t resident = device_cus() / 8 * (WW * WT <= 4 ? 2 : 1);
  const SuperTile st = rt > 0 ? xcd_supertile(ntt / rt, nwt / (8 / rt), TT, TW, resident)
                              : SuperTile{1, 1};
  hipLaunchKernelGGL((gemm6_lds_kernel<FW, FT, WW, WT, S, I32>), dim3(static_cast<unsigned>(nb)),
                     dim3(64 * WW * WT), 0, s, a, s_a, w, s_w, y, static_cast<int>(T),
                     static_cast<int>(K), static_cast<int>(N), rt, st.t, st.n);
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
  if (K % 128 == 0 && T >= 128) {
    // Eight-wave blocks of 256 x 256 or 256 x 128 outputs (one workgroup per
    // CU) for large products, four-wave 128 x 128 blocks (two per CU)
    // otherwise. A 256 x 256 block moves two thirds of the operand bytes per
    // MFMA of a 256 x 128 one, and a full wave of them (one per CU) takes
    // about 16/9 of the time of a full wave of 256 x 128 blocks (K = 4096:
    // 48.4 us against 27.2); the shape with fewer such weighted waves is
    // taken, which picks 256 x 128 for 2048 x 4096 outputs (one wave against
    // one of 256 x 256 blocks on half the CUs) and 256 x 256 from 3072 x 4096
    // or 2048 x 8192 up.
    const bool big = T >= 2048 && N >= 4096;
    const int64_t cus = device_cus();
    const int64_t w2 = ((T + 255) / 256 * ((N + 255) / 256) + cus - 1) / cus;
    const int64_t w1 = ((T + 255) / 256 * ((N + 127) / 128) + cus - 1) / cus;
    const bool huge = big && 16 * w2 < 9 * w1;
    if (i32_out)
      return huge  ? g6::launch_lds<2, 4, 4, 2, 3, true>(a, s_a, w, s_w, y, T, K, N, s)
             : big ? g6::launch_lds<2, 2, 4, 2, 3, true>(a, s_a, w, s_w, y, T, K, N, s)
                   : g6::launch_lds<2, 2, 2, 2, 3, true>(a, s_a, w, s_w, y, T, K, N, s);
    return huge  ? g6::launch_lds<2, 4, 4, 2, 3, false>(a, s_a, w, s_w, y, T, K, N, s)
           : big ? g6::launch_lds<2, 2, 4, 2, 3, false>(a, s_a, w, s_w, y, T, K, N, s)
                 : g6::launch_lds<2, 2, 2, 2, 3, false>(a, s_a, w, s_w, y, T, K, N, s);
  }
  // decode products: up to 16 tokens and N <= 16384 on 16-row workgroups,
  // with fewer waves per workgroup as their number grows (measured at T = 8:
  // 16 waves for N = 4096, 4 for N = 12288); otherwise 32-row workgroups
  if (T <= 16 && N <= 16384) {
    const int64_t nb = (N + 15) / 16;
    if (nb <= 256) return g6::launch_decode16<16>(a, s_a, w, s_w, y, i32_out, T, K, N, s);
    if (nb <= 512) return g6::launch_decode16<8>(a, s_a, w, s_w, y, i32_out, T, K, N, s);
    return g6::launch_decode16<4>(a, s_a, w, s_w, y, i32_out, T, K, N, s);
  }
  if (T <= 32) {
    const unsigned nb = static_cast<unsigned>((N + 31) / 32);
    if (i32_out)
      hipLaunchKernelGGL((g6::gemm6_decode_kernel<true>), dim3(nb), dim3(64 * g6::kDecWaves), 0, s,
                         a, s_a, w, s_w, y, static_cast<int>(T), static_cast<int>(K), static_cast<int>(N));
    else
      hipLaunchKernelGGL((g6::gemm6_decode_kernel<false>), dim3(nb), dim3(64 * g6::kDecWaves), 0, s,
                         a, s_a, w, s_w, y, static_cast<int>(T), static_cast<int>(K), static_cast<int>(N));
    return hipGetLastError();
  }
  if (i32_out) return g6::launch_cfg<4, 2, 4, true>(a, s_a, w, s_w, y, T, K, N, s);
  return g6::launch_cfg<4, 2, 4, false>(a, s_a, w, s_w, y, T, K, N, s);
}

}  // namespace rw4
