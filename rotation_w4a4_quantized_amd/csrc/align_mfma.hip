// Low-rank residual alignment on bf16 matrix cores ("ReSpinQuant" paper notes,
// key design 3: y = Q^T x, z = (M - I) y, out = x + Q z).
//
// The activations are bf16, so x is exact as an MFMA operand. The basis is
// split into two bf16 terms, A = Ah + Al + O(2^-17 |A|), and z likewise:
//   z   = x.Q'h + x.Q'l                    (Q' = Q (M - I)^T; two bf16 products,
//                                           fp32 accumulate: z = (M - I) Q^T x)
//   out = x + Qh.zh + Ql.zh + Qh.zl        (the dropped Ql.zl is ~2^-17 relative)
// which keeps the fp32 alignment well inside a 1e-5 normwise error while
// running on v_mfma_f32_16x16x32_bf16 instead of fp32 FMAs. With M = I, Q' and
// z are exactly zero and the output equals the input.
//
// The basis (everything that depends on Q and M only) is prepared once and
// can be kept with the layer's weights; then two launches per call:
//   prep : Q'h/Q'l as [r][D] rows for the projection, Qh/Ql as [D][r] rows for
//          the lift, zero-padded in r; and, for the fused prologue, the
//          Hadamard image P = H Q / sqrt(D) split the same way.
//   yproj: per (64 tokens, 512-column D part): the part's share of z on the
//          matrix cores, reduced over the eight waves in LDS ->
//          Zpart[part][t][i] (z is the sum of the parts).
//   lift : per (64 tokens, D part): z = sum of the parts in a fixed order
//          (deterministic), its bf16 split in LDS, then out = x + Q z. The
//          MFMA's row order is permuted so a lane's accumulator covers the same
//          16 consecutive columns of one token that its x load holds: the
//          accumulator starts as x. Results go out through LDS as whole rows.
// Every global load is unconditional (clamped indices, masked values): loads
// inside branches whose values are used after the join read stale registers
// with this toolchain, and a short drain separates the last MFMA from the
// first non-MFMA read of its result.
#include <algorithm>

#include "align_small.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

constexpr int TB = 16;          // tokens per workgroup (MFMA rows)
constexpr int NW = 4;           // waves per workgroup

// One workgroup per 64 (d) x 32 (j) tile: the lift operand Q (bf16 hi/lo,
// [D][RK] rows written directly) and the projection operand Q' = Q (M - I)^T
// ([RP][D] rows of the same split, through an LDS transpose). With Q' the
// projection yields z = (M - I) Q^T x directly: Q'^T x = (M - I) Q^T x. The
// entries of M - I are exact in fp32 (M's diagonal lies well inside [0.5, 2]
// for the sub-rotations of the pages, so M_ii - 1 is exact by Sterbenz), and
// Q' is summed in fp32. Columns j >= r are zero padding.
// Q' is also written in the order the projection's waves read it (QtF): 1 KiB
// chunks, one per (64-column double step dg, 16-row block c, hi/lo, half h),
// lane 16 g + t holding Q'[16 c + t][64 dg + 16 g + 8 h .. + 8]. A wave then
// loads each operand fragment as one contiguous 1 KiB (from L2 a row-major
// fragment, 16 rows of 64 bytes, reads at about a third of that rate). Same
// values as Q'h/Q'l, so the same products. (A separate reordering launch
// cost ~4 us of the basis preparation.)
constexpr int kPrepRmax = 128;

__device__ __forceinline__ void basis_prep_tile(int bx, int by, const float* __restrict__ Q,
                                                const float* __restrict__ M, int D, int r, int RP,
                                                int RK, uint16_t* __restrict__ QtH,
                                                uint16_t* __restrict__ QtL,
                                                uint16_t* __restrict__ QH,
                                                uint16_t* __restrict__ QL,
                                                uint16_t* __restrict__ QtF) {
  __shared__ uint16_t th[32][64 + 2];
  __shared__ uint16_t tlo[32][64 + 2];
  __shared__ float qrow[64][kPrepRmax + 1];     // Q rows d0 .. d0 + 63
  __shared__ float mi[32][kPrepRmax + 1];       // (M - I) rows j0 .. j0 + 31
  const int tid = threadIdx.x;
  const int d0 = bx * 64;
  const int j0 = by * 32;
  for (int c = tid; c < 64 * r; c += 256) {
    const int dd = c / r, k = c % r;
    qrow[dd][k] = d0 + dd < D ? Q[static_cast<int64_t>(d0 + dd) * r + k] : 0.0f;
  }
  for (int c = tid; c < 32 * r; c += 256) {
    const int i = c / r, k = c % r;
    const int row = j0 + i;
    mi[i][k] = row < r ? (row == k ? M[row * r + k] - 1.0f : M[row * r + k]) : 0.0f;
  }
  __syncthreads();
  // 64 x 32 tile: thread -> (row dd = tid / 4, 8 columns jb + 0..7)
  const int dd = tid >> 2;
  const int jb = (tid & 3) * 8;
  const int d = d0 + dd;
  uint16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = j0 + jb + e;
    const float q = j < r ? qrow[dd][j] : 0.0f;
    h[e] = f32_to_bf16(q);
    l[e] = f32_to_bf16(q - bf16_to_f32(h[e]));
  }
  if (d < D && j0 + jb < RK) {
    uint4 vh, vl;
    vh.x = h[0] | (uint32_t(h[1]) << 16); vh.y = h[2] | (uint32_t(h[3]) << 16);
    vh.z = h[4] | (uint32_t(h[5]) << 16); vh.w = h[6] | (uint32_t(h[7]) << 16);
    vl.x = l[0] | (uint32_t(l[1]) << 16); vl.y = l[2] | (uint32_t(l[3]) << 16);
    vl.z = l[4] | (uint32_t(l[5]) << 16); vl.w = l[6] | (uint32_t(l[7]) << 16);
    *reinterpret_cast<uint4*>(QH + static_cast<int64_t>(d) * RK + j0 + jb) = vh;
    *reinterpret_cast<uint4*>(QL + static_cast<int64_t>(d) * RK + j0 + jb) = vl;
  }
  // Q'[d][j] = sum_k Q[d][k] (M - I)[j][k] (zero for j >= r), split the same way
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < r; ++k) {
    const float q = qrow[dd][k];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(q, mi[jb + e][k], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t hh = f32_to_bf16(acc[e]);
    th[jb + e][dd] = hh;
    tlo[jb + e][dd] = f32_to_bf16(acc[e] - bf16_to_f32(hh));
  }
  __syncthreads();
  // transposed rows: thread -> (row j = tid / 8, 8 consecutive d)
  const int jr = tid >> 3;
  const int db = (tid & 7) * 8;
  const int j = j0 + jr;
  if (j < RP && d0 + db < D) {
    uint4 vh, vl;
    vh.x = th[jr][db] | (uint32_t(th[jr][db + 1]) << 16); vh.y = th[jr][db + 2] | (uint32_t(th[jr][db + 3]) << 16);
    vh.z = th[jr][db + 4] | (uint32_t(th[jr][db + 5]) << 16); vh.w = th[jr][db + 6] | (uint32_t(th[jr][db + 7]) << 16);
    vl.x = tlo[jr][db] | (uint32_t(tlo[jr][db + 1]) << 16); vl.y = tlo[jr][db + 2] | (uint32_t(tlo[jr][db + 3]) << 16);
    vl.z = tlo[jr][db + 4] | (uint32_t(tlo[jr][db + 5]) << 16); vl.w = tlo[jr][db + 6] | (uint32_t(tlo[jr][db + 7]) << 16);
    *reinterpret_cast<uint4*>(QtH + static_cast<int64_t>(j) * D + d0 + db) = vh;
    *reinterpret_cast<uint4*>(QtL + static_cast<int64_t>(j) * D + d0 + db) = vl;
    if (d0 + 64 <= D) {  // whole double steps (the projection's parts)
      const int64_t q = ((static_cast<int64_t>(bx) * (RP / 16) + (j >> 4)) * 2) * 2 +
                        ((db >> 3) & 1);                      // hi; lo is chunk q + 2
      const int ln = 16 * (db >> 4) + (j & 15);
      *reinterpret_cast<uint4*>(QtF + (q * 64 + ln) * 8) = vh;
      *reinterpret_cast<uint4*>(QtF + ((q + 2) * 64 + ln) * 8) = vl;
    }
  }
}

__global__ void __launch_bounds__(256)
basis_prep_kernel(const float* __restrict__ Q, const float* __restrict__ M, int D, int r, int RP,
                  int RK, uint16_t* __restrict__ QtH, uint16_t* __restrict__ QtL,
                  uint16_t* __restrict__ QH, uint16_t* __restrict__ QL,
                  uint16_t* __restrict__ QtF) {
  basis_prep_tile(blockIdx.x, blockIdx.y, Q, M, D, r, RP, RK, QtH, QtL, QH, QL, QtF);
}

// Hadamard image of the basis for the fused prologue: P = H_D Q / sqrt(D),
// bf16 hi/lo split like Q, [D][RK] (columns j >= r are zero). One workgroup
// per column; the column is transformed in LDS with the butterfly order of
// the FWHT (h = 1, 2, ..., D/2) in fp32. Since H_D / sqrt(D) is symmetric and
// orthogonal, H (x + Q z) / sqrt(D) = H x / sqrt(D) + P z.
constexpr int kBasisFwhtMax = 4096;

__global__ void __launch_bounds__(1024)
basis_fwht_kernel(const float* __restrict__ Q, int D, int r, int RK, float norm,
                  uint16_t* __restrict__ PH, uint16_t* __restrict__ PL) {
  __shared__ float col[kBasisFwhtMax];
  const int tid = threadIdx.x;
  const int j = blockIdx.x;
  for (int d = tid; d < D; d += 1024) col[d] = j < r ? Q[static_cast<int64_t>(d) * r + j] : 0.0f;
  __syncthreads();
  for (int lh = 0; (1 << lh) < D; ++lh) {
    const int h = 1 << lh;
    for (int i = tid; i < D / 2; i += 1024) {
      const int lo = ((i >> lh) << (lh + 1)) + (i & (h - 1));
      const float a = col[lo], b = col[lo + h];
      col[lo] = a + b;
      col[lo + h] = a - b;
    }
    __syncthreads();
  }
  for (int d = tid; d < D; d += 1024) {
    const float v = col[d] * norm;
    const uint16_t hi = f32_to_bf16(v);
    PH[static_cast<int64_t>(d) * RK + j] = hi;
    PL[static_cast<int64_t>(d) * RK + j] = f32_to_bf16(v - bf16_to_f32(hi));
  }
}

// The same transform at D = 4096 with 256 threads of 16 values: the twelve
// butterfly levels run in registers in three phases of four (index bits 0-3,
// 4-7, 8-11), with the column exchanged through LDS between them (two
// barriers instead of one per level). Each level pairs the same elements in
// the same order as above (h = 1, 2, ..., 2048), so the results are the same
// bits. One workgroup per column, as above.
constexpr int kBasisFwhtFast = 4096;
__device__ __forceinline__ void basis_fwht4096_col(int j, const float* __restrict__ Q, int r,
                                                   int RK, float norm, uint16_t* __restrict__ PH,
                                                   uint16_t* __restrict__ PL) {
  constexpr int D = kBasisFwhtFast;
  __shared__ float col[D + D / 16];             // one pad word per 16 (conflict-free phase 1)
  const int t = threadIdx.x;
  auto at = [](int d) { return d + (d >> 4); };
  auto levels = [](float (&v)[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if ((k & h) == 0) {
          const float a = v[k], b = v[k + h];
          v[k] = a + b;
          v[k + h] = a - b;
        }
  };
  float v[16];
  // phase 1: bits 0-3, element k of thread t is d = 16 t + k
  const int jj = j < r ? j : 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = Q[static_cast<int64_t>(16 * t + k) * r + jj];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = j < r ? v[k] : 0.0f;
  levels(v);
#pragma unroll
  for (int k = 0; k < 16; ++k) col[at(16 * t + k)] = v[k];
  __syncthreads();
  // phase 2: bits 4-7, d = (t & 15) + 16 k + 256 (t >> 4)
  const int b2 = (t & 15) + 256 * (t >> 4);
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = col[at(b2 + 16 * k)];
  levels(v);
#pragma unroll
  for (int k = 0; k < 16; ++k) col[at(b2 + 16 * k)] = v[k];
  __syncthreads();
  // phase 3: bits 8-11, d = t + 256 k
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = col[at(t + 256 * k)];
  levels(v);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int d = t + 256 * k;
    const float w = v[k] * norm;
    const uint16_t hi = f32_to_bf16(w);
    PH[static_cast<int64_t>(d) * RK + j] = hi;
    PL[static_cast<int64_t>(d) * RK + j] = f32_to_bf16(w - bf16_to_f32(hi));
  }
}

// The basis preparation at D = 4096 in one launch: workgroups below the tile
// count run basis_prep_tile (tile b % gx, b / gx), the rest the Hadamard image
// of column b - tiles; neither reads what the other writes.
__global__ void __launch_bounds__(256)
basis_prep_p4096_kernel(const float* __restrict__ Q, const float* __restrict__ M, int r, int RP,
                        int RK, int gx, uint16_t* __restrict__ QtH, uint16_t* __restrict__ QtL,
                        uint16_t* __restrict__ QH, uint16_t* __restrict__ QL,
                        uint16_t* __restrict__ QtF, float norm, uint16_t* __restrict__ PH,
                        uint16_t* __restrict__ PL) {
  const int b = blockIdx.x;
  const int tiles = gx * (RK / 32);
  if (b < tiles)
    basis_prep_tile(b % gx, b / gx, Q, M, kBasisFwhtFast, r, RP, RK, QtH, QtL, QH, QL, QtF);
  else
    basis_fwht4096_col(b - tiles, Q, r, RK, norm, PH, PL);
}

// A D part of 512 columns is 8 double steps of 64 columns; each of the 8
// waves takes 1. Inside a double step lane group g (lane / 16) owns the 16
// contiguous columns [16g, 16g + 16): its first 8 feed one MFMA, the next 8 a
// second one. The k order of a dot product is free, so both operands use this
// same order, and every lane reads 32 contiguous bytes per row.
// A lift workgroup aligns TBW blocks of 16 tokens: every Q fragment it loads
// is used by TBW MFMA blocks, which keeps the L2 traffic for Q at 1/TBW of
// the token count; the projection uses the same 64-token blocks (16-token
// blocks measured slower: four times the Q traffic outweighs the overlap).
constexpr int YNW = 8;                    // projection waves per workgroup
constexpr int DPW = 1;                    // double steps per wave
constexpr int kPart = YNW * DPW * 64;
constexpr int TBW = 4;                    // 16-token blocks per lift workgroup
constexpr int TPW = TBW * TB;             // tokens per lift workgroup
constexpr int YTBW = 4;                   // 16-token blocks per projection workgroup
constexpr int YTPW = YTBW * TB;

// The projection's reduction over its 8 waves and the partial stores, shared by
// both projection kernels. Wave w holds, for its 64 columns, the block's
// partials acc[tb][c][v] = z-part of token 16 tb + 4 g + v, basis index
// 16 c + t. Waves 4..7 park theirs in red[w - 4], waves 0..3 add theirs
// (slot = own + parked), and z = (slot 0 + slot 1) + (slot 2 + slot 3).
// red[w][i][t] holds basis index i, token t (rows padded to 68 words): a lane's
// four tokens are one 16-byte access, and the 16 lanes of a row group fall on
// distinct banks. Each thread then forms four consecutive tokens of one
// basis index (i < RP; zero padding up to RK) and stores them, 4 per group
// (rows past T rewrite row T - 1 with the same bits).
constexpr int kRedPitch = YTPW + 4;

template <int RP, bool LB>
__device__ __forceinline__ void yproj_reduce_store(const v4f (&acc)[YTBW][RP / 16],
                                                   float (&red)[4][RP][kRedPitch], int wave,
                                                   int g, int tl, int tid, int part, int64_t T,
                                                   int64_t t0, float* __restrict__ Zpart) {
  constexpr int RK = (RP + 31) / 32 * 32;
  constexpr int NT = YNW * 64;
  constexpr int NQ = YTPW / 4;                        // token quads of the block
  static_assert(NQ * RK % NT == 0, "quads per thread");
  auto bar = [] {
    if constexpr (LB)
      lds_barrier();
    else
      __syncthreads();
  };
  if (wave >= 4) {
#pragma unroll
    for (int tb = 0; tb < YTBW; ++tb)
#pragma unroll
      for (int c = 0; c < RP / 16; ++c)
        *reinterpret_cast<v4f*>(&red[wave - 4][16 * c + tl][16 * tb + 4 * g]) = acc[tb][c];
  }
  bar();
  if (wave < 4) {
#pragma unroll
    for (int tb = 0; tb < YTBW; ++tb)
#pragma unroll
      for (int c = 0; c < RP / 16; ++c) {
        v4f& slot = *reinterpret_cast<v4f*>(&red[wave][16 * c + tl][16 * tb + 4 * g]);
        slot = acc[tb][c] + slot;
      }
  }
  bar();
#pragma unroll
  for (int k = 0; k < NQ * RK / NT; ++k) {
    const int o = tid + k * NT;
    const int i = o % RK;
    const int q = o / RK;
    v4f z = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    if (i < RP) {
      const v4f r0 = *reinterpret_cast<const v4f*>(&red[0][i][4 * q]);
      const v4f r1 = *reinterpret_cast<const v4f*>(&red[1][i][4 * q]);
      const v4f r2 = *reinterpret_cast<const v4f*>(&red[2][i][4 * q]);
      const v4f r3 = *reinterpret_cast<const v4f*>(&red[3][i][4 * q]);
      z = (r0 + r1) + (r2 + r3);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Zpart[(static_cast<int64_t>(part) * T + min(t0 + 4 * q + e, T - 1)) * RK + i] = z[e];
  }
}

template <int RP>
__global__ void __launch_bounds__(YNW * 64)
yproj_kernel(const uint16_t* __restrict__ x, int64_t T, int D, int P, int r,
             const uint16_t* __restrict__ QtF, float* __restrict__ Zpart) {
  constexpr int RK = (RP + 31) / 32 * 32;
  __shared__ __attribute__((aligned(16))) float red[4][RP][kRedPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // workgroups go to the XCDs round robin in launch order (x fastest). From
  // 16 D parts on (when the grid divides by 8), XCD k takes a contiguous run
  // of (token block, part) pairs in part-major order, so its L2 fetches only
  // a few parts of Q^T instead of all of it (2 MiB at D = 8192, r = 64)
  int64_t bx = blockIdx.x;
  int part = blockIdx.y;
  {
    const int64_t nb = static_cast<int64_t>(gridDim.x) * gridDim.y;
    const int64_t b = blockIdx.x + static_cast<int64_t>(gridDim.x) * blockIdx.y;
    if ((nb & 7) == 0 && gridDim.y >= 16) {
      const int64_t q = (b & 7) * (nb >> 3) + (b >> 3);
      bx = q % gridDim.x;
      part = static_cast<int>(q / gridDim.x);
    } else if ((gridDim.x & 7) == 0) {
      // fewer parts: XCD k takes the k-th eighth of the token blocks, every
      // part of them, the band of tokens the fused prologue that follows
      // gives the same XCD, which then finds those rows of x in its L2
      const int64_t per = gridDim.x >> 3;
      const int64_t j = b >> 3;
      bx = (b & 7) * per + j % per;
      part = static_cast<int>(j / per);
    }
  }
  const int64_t t0 = bx * YTPW;
  const int dbeg = part * P;
  const int dend = min(D, dbeg + P);
  const int nds = (dend - dbeg) / 64;                 // whole double steps in this part
  const int g = lane >> 4;
  const int tl = lane & 15;
  // basis blocks per load batch (divides RP/16): all of them up to RP = 64, so
  // that the whole projection waits for memory once
  constexpr int NBC = RP <= 64 ? RP / 16 : ((RP / 16) % 2 == 0 ? 2 : 1);

  // loads are unconditional: double steps past the part's end re-read its last
  // one and their x is zeroed; tokens past T re-read the last token
  v8bf xa[YTBW][DPW][2];
#pragma unroll
  for (int b = 0; b < YTBW; ++b) {
    const int64_t trow = min(t0 + 16 * b + tl, T - 1);
    const uint16_t* xrow = x + trow * D + 16 * g;
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int ds = wave * DPW + u;
      const int dsc = ds < nds ? ds : nds - 1;
      const uint4* px = reinterpret_cast<const uint4*>(xrow + dbeg + 64 * dsc);
      uint4 a0 = px[0], a1 = px[1];
      const uint32_t keep = ds < nds ? 0xFFFFFFFFu : 0u;
      a0.x &= keep; a0.y &= keep; a0.z &= keep; a0.w &= keep;
      a1.x &= keep; a1.y &= keep; a1.z &= keep; a1.w &= keep;
      xa[b][u][0] = as8(a0);
      xa[b][u][1] = as8(a1);
    }
  }
  v4f acc[YTBW][RP / 16];
#pragma unroll
  for (int b = 0; b < YTBW; ++b)
#pragma unroll
    for (int nb = 0; nb < RP / 16; ++nb) acc[b][nb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int nb0 = 0; nb0 < RP / 16; nb0 += NBC) {
    v8bf bh[DPW][NBC][2], bl[DPW][NBC][2];
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int ds = wave * DPW + u;
      const int dsc = ds < nds ? ds : nds - 1;
      const int64_t dg = dbeg / 64 + dsc;
#pragma unroll
      for (int c = 0; c < NBC; ++c) {
        const uint16_t* f = QtF + (dg * (RP / 16) + nb0 + c) * 4 * 512 + lane * 8;
        bh[u][c][0] = ld8(f);
        bh[u][c][1] = ld8(f + 512);
        bl[u][c][0] = ld8(f + 1024);
        bl[u][c][1] = ld8(f + 1536);
      }
    }
    // every load of the batch (and, in the first, of x) is issued before the
    // first product: left alone, the scheduler interleaves them with the
    // MFMAs to save registers and the wave waits for memory once per pair
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < DPW; ++u)
#pragma unroll
      for (int c = 0; c < NBC; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int b = 0; b < YTBW; ++b) {
            acc[b][nb0 + c] = mfma(xa[b][u][h], bh[u][c][h], acc[b][nb0 + c]);
            acc[b][nb0 + c] = mfma(xa[b][u][h], bl[u][c][h], acc[b][nb0 + c]);
          }
  }
  mfma_drain();
  yproj_reduce_store<RP, false>(acc, red, wave, g, tl, tid, part, T, t0, Zpart);
}

// The projection as a loop over 64-token blocks from 16 D parts on (RP <= 64):
// a grid of G x S workgroups, about one per CU; the workgroup of D part p
// takes the blocks b, b + G, b + 2G, ... Its block of Q' (RP rows of the
// part, bf16 hi/lo) is loaded once and stays in registers, and the next
// block's x is loaded while the current one is multiplied, reduced and
// stored. The products, their order and the reduction are those of
// yproj_kernel, so both give the same partials. Tokens past T re-read the
// last token and rewrite its partials with the same bits; every thread
// issues a fixed number of stores, so the wait for the next block's x leaves
// them in flight.
template <int RP>
__global__ void __launch_bounds__(YNW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
yproj_loop_kernel(const uint16_t* __restrict__ x, int64_t T, int D, int P,
                  const uint16_t* __restrict__ QtF, float* __restrict__ Zpart) {
  static_assert(RP <= 64 && DPW == 1, "the basis block is held in registers");
  constexpr int RK = (RP + 31) / 32 * 32;
  constexpr int NT = YNW * 64;
  constexpr int NBC = RP / 16;
  __shared__ __attribute__((aligned(16))) float red[4][RP][kRedPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int part = blockIdx.y;
  const int dbeg = part * P;
  const int dend = min(D, dbeg + P);
  const int nds = (dend - dbeg) / 64;
  const int g = lane >> 4;
  const int tl = lane & 15;
  const int dsc = wave < nds ? wave : nds - 1;
  const uint32_t keep = wave < nds ? 0xFFFFFFFFu : 0u;  // a double step past the part is zero
  const int64_t nb = (T + YTPW - 1) / YTPW;
  const int64_t G = gridDim.x;
  int64_t blk = blockIdx.x;
  if (blk >= nb) return;

  v8bf bh[NBC][2], bl[NBC][2];
  const int64_t dg = dbeg / 64 + dsc;
#pragma unroll
  for (int c = 0; c < NBC; ++c) {
    const uint16_t* f = QtF + (dg * NBC + c) * 4 * 512 + lane * 8;
    bh[c][0] = ld8(f);
    bh[c][1] = ld8(f + 512);
    bl[c][0] = ld8(f + 1024);
    bl[c][1] = ld8(f + 1536);
  }
  uint4 xn[YTBW][2];
  auto load_x = [&](int64_t b) {
#pragma unroll
    for (int tb = 0; tb < YTBW; ++tb) {
      const int64_t trow = min(b * YTPW + 16 * tb + tl, T - 1);
      const uint4* px = reinterpret_cast<const uint4*>(x + trow * D + 16 * g + dbeg + 64 * dsc);
      xn[tb][0] = px[0];
      xn[tb][1] = px[1];
    }
  };
  v8bf xa[YTBW][2];
  auto take_x = [&]() {
#pragma unroll
    for (int tb = 0; tb < YTBW; ++tb) {
      uint4 a0 = xn[tb][0], a1 = xn[tb][1];
      a0.x &= keep; a0.y &= keep; a0.z &= keep; a0.w &= keep;
      a1.x &= keep; a1.y &= keep; a1.z &= keep; a1.w &= keep;
      xa[tb][0] = as8(a0);
      xa[tb][1] = as8(a1);
    }
  };
  load_x(blk);
  take_x();
  // the basis block has arrived too (an explicit vmcnt(0)): otherwise its
  // waits land inside the loop, where they also drain the previous round's
  // stores
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (;;) {
    const int64_t t0 = blk * YTPW;
    const bool more = blk + G < nb;
    load_x(more ? blk + G : blk);
    __builtin_amdgcn_sched_barrier(0);
    v4f acc[YTBW][NBC];
#pragma unroll
    for (int tb = 0; tb < YTBW; ++tb)
#pragma unroll
      for (int c = 0; c < NBC; ++c) acc[tb][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < NBC; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tb = 0; tb < YTBW; ++tb) {
          acc[tb][c] = mfma(xa[tb][h], bh[c][h], acc[tb][c]);
          acc[tb][c] = mfma(xa[tb][h], bl[c][h], acc[tb][c]);
        }
    mfma_drain();
    yproj_reduce_store<RP, true>(acc, red, wave, g, tl, tid, part, T, t0, Zpart);
    // every read of red is done before the next block's writes
    lds_barrier();
    if (!more) break;
    // the next block's x, taken here at the end of the round so that the only
    // path to this wait is the one through this round's stores
    take_x();
    blk += G;
  }
}

// The lift runs 8 waves per workgroup, one 64-column double step each, so a
// 512-column part of 64 tokens keeps two waves per SIMD busy.
constexpr int LNW = 8;

// All of Q's k-chunks are loaded up front for RK <= 64 (with RK = 64 the
// second chunk used to be reloaded for every token block, each load waited
// for in turn: 169.7 us at T = D = 8192); that needs more than the 128
// registers of four waves per SIMD, so RK = 64 runs with two.
template <int RP, int RK, bool OF32, bool ADD>
__global__ void __launch_bounds__(LNW * 64) __attribute__((amdgpu_waves_per_eu(RK > 32 ? 2 : 4, 8)))
lift_kernel(const uint16_t* __restrict__ x, int64_t T, int D, int P, int S, int r,
            const float* __restrict__ Zpart, const uint16_t* __restrict__ QH,
            const uint16_t* __restrict__ QL, const void* __restrict__ addend,
            void* __restrict__ out) {
  constexpr int NT = LNW * 64;
  __shared__ __attribute__((aligned(16))) uint16_t zh[TPW][RK + 8];
  __shared__ __attribute__((aligned(16))) uint16_t zl[TPW][RK + 8];
  // one 16-token block of results, written out as whole row segments
  __shared__ __attribute__((aligned(16))) float stage[TB][kPart + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TPW;
  const int part = blockIdx.y;
  const int dbeg = part * P;
  const int dend = min(D, dbeg + P);
  const int nds = (dend - dbeg) / 64;
  const int g = lane >> 4;
  const int tl = lane & 15;
  constexpr int KQ = RK <= 64 ? RK / 32 : 1;          // Q k-chunks loaded up front
  const bool live = wave < nds;                       // this wave's double step exists
  const int d0 = dbeg + 64 * (live ? wave : nds - 1);
  static_assert(TPW * RK % (4 * NT) == 0 || TPW * RK < 4 * NT, "z chunks");

  // 1. every load of the lift, issued up front and unconditional (a wave past
  // the part's end re-reads its last double step and stores nothing; tokens
  // past T re-read the last token). With one z chunk per thread (RK = 32),
  // each thread fetches 4 consecutive z entries of the first eight D parts
  // (TPW * RK / 4 float4 chunks over the workgroup) first, then its Q and x. Block b of the double step covers
  // columns 16g + 4b + v for lane group g, so A's row i = 4g' + v of block b is
  // column 16g' + 4b + v.
  constexpr int ZC = TPW * RK / 4;                     // float4 chunks of z
  constexpr int ZPT = (ZC + NT - 1) / NT;              // chunks per thread
  // with more than one chunk per thread the early z loads cost more registers
  // than the round trip they save (the compiler then serializes single loads)
  constexpr bool ZPRE = ZPT == 1;
  float4 zp0[8];
  if constexpr (ZPRE) {
    const int c = min(tid, ZC - 1);
    const int64_t trow = min(t0 + (4 * c) / RK, T - 1);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      zp0[q] = *reinterpret_cast<const float4*>(
          Zpart + (static_cast<int64_t>(min(q, S - 1)) * T + trow) * RK + (4 * c) % RK);
  }
  v8bf qh[4][KQ], ql[4][KQ];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int drow = d0 + 16 * (tl >> 2) + 4 * b + (tl & 3);
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const int64_t qo = static_cast<int64_t>(drow) * RK + 32 * kk + 8 * g;
      qh[b][kk] = ld8(QH + qo);
      ql[b][kk] = ld8(QL + qo);
    }
  }
  uint4 xv[TBW][2];
#pragma unroll
  for (int tb = 0; tb < TBW; ++tb) {
    const int64_t trow = min(t0 + 16 * tb + tl, T - 1);
    const uint4* px = reinterpret_cast<const uint4*>(x + trow * D + d0 + 16 * g);
    xv[tb][0] = px[0];
    xv[tb][1] = px[1];
  }
  // the scheduler keeps every load above ahead of the first use (left alone,
  // it waits for the Q and x loads before issuing the z loads)
  if constexpr (ZPRE) __builtin_amdgcn_sched_barrier(0);
  // 2. z = sum over D parts (fixed order), its bf16 split into LDS
#pragma unroll
  for (int u = 0; u < ZPT; ++u) {
    const int c = tid + u * NT;
    if (c >= ZC) break;
    const int tt = (4 * c) / RK;
    const int i = (4 * c) % RK;
    const int64_t trow = min(t0 + tt, T - 1);
    // the parts in blocks of 8 (the first loaded above), each block's loads
    // issued together (unconditional, clamped, masked) and added in part order
    float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if constexpr (ZPRE) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < S) {
          z.x += zp0[q].x; z.y += zp0[q].y; z.z += zp0[q].z; z.w += zp0[q].w;
        }
    }
    for (int p0 = ZPRE ? 8 : 0; p0 < S; p0 += 8) {
      float4 zp[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        zp[q] = *reinterpret_cast<const float4*>(
            Zpart + (static_cast<int64_t>(min(p0 + q, S - 1)) * T + trow) * RK + i);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (p0 + q < S) {
          z.x += zp[q].x; z.y += zp[q].y; z.z += zp[q].z; z.w += zp[q].w;
        }
    }
    const float zz[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t h = f32_to_bf16(zz[e]);
      zh[tt][i + e] = h;
      zl[tt][i + e] = f32_to_bf16(zz[e] - bf16_to_f32(h));
    }
  }
  __syncthreads();

  // 4. out = x + Q z per token block; the accumulators start at x. Each block's
  // results are staged in LDS, then all threads write them as contiguous row
  // segments (the MFMA layout would scatter 16-byte pieces over 16 rows).
  const int ncols = dend - dbeg;
  // unrolled, so that xv[tb] stays in registers (a runtime index would move
  // the array to scratch memory)
#pragma unroll
  for (int tb = 0; tb < TBW; ++tb) {
    if (live) {
      v4f acc[4];
      acc[0] = v4f{bf16lo(xv[tb][0].x), bf16hi(xv[tb][0].x), bf16lo(xv[tb][0].y), bf16hi(xv[tb][0].y)};
      acc[1] = v4f{bf16lo(xv[tb][0].z), bf16hi(xv[tb][0].z), bf16lo(xv[tb][0].w), bf16hi(xv[tb][0].w)};
      acc[2] = v4f{bf16lo(xv[tb][1].x), bf16hi(xv[tb][1].x), bf16lo(xv[tb][1].y), bf16hi(xv[tb][1].y)};
      acc[3] = v4f{bf16lo(xv[tb][1].z), bf16hi(xv[tb][1].z), bf16lo(xv[tb][1].w), bf16hi(xv[tb][1].w)};
#pragma unroll
      for (int kk = 0; kk < RK / 32; ++kk) {
        const v8bf bh = *reinterpret_cast<const v8bf*>(&zh[16 * tb + tl][32 * kk + 8 * g]);
        const v8bf bl = *reinterpret_cast<const v8bf*>(&zl[16 * tb + tl][32 * kk + 8 * g]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          v8bf ah, al;
          if (kk < KQ) {
            ah = qh[b][kk < KQ ? kk : 0];
            al = ql[b][kk < KQ ? kk : 0];
          } else {
            const int drow = d0 + 16 * (tl >> 2) + 4 * b + (tl & 3);
            const int64_t qo = static_cast<int64_t>(drow) * RK + 32 * kk + 8 * g;
            ah = ld8(QH + qo);
            al = ld8(QL + qo);
          }
          acc[b] = mfma(ah, bh, acc[b]);
          acc[b] = mfma(al, bh, acc[b]);
          acc[b] = mfma(ah, bl, acc[b]);
        }
      }
      mfma_drain();
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<float4*>(&stage[tl][64 * wave + 16 * g + 4 * b]) =
            make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    }
    __syncthreads();
    // one 16-byte store per thread and chunk, so that every store instruction
    // of a wave covers 1 KiB of one row segment
    constexpr int CW = OF32 ? 4 : 8;
    for (int c = tid; c < TB * (ncols / CW); c += NT) {
      const int row = c / (ncols / CW);
      const int col = (c % (ncols / CW)) * CW;
      const int64_t t = t0 + 16 * tb + row;
      if (t >= T) continue;
      const int64_t off = t * D + dbeg + col;
      if constexpr (OF32) {
        float4 o = *reinterpret_cast<const float4*>(&stage[row][col]);
        if constexpr (ADD) {
          const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(addend) + off);
          o.x += a.x; o.y += a.y; o.z += a.z; o.w += a.w;
        }
        store_stream16(static_cast<float*>(out) + off, o);
      } else {
        const float4 s0 = *reinterpret_cast<const float4*>(&stage[row][col]);
        const float4 s1 = *reinterpret_cast<const float4*>(&stage[row][col + 4]);
        float o[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        if constexpr (ADD) {
          const uint4 av = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(addend) + off);
          o[0] += bf16lo(av.x); o[1] += bf16hi(av.x); o[2] += bf16lo(av.y); o[3] += bf16hi(av.y);
          o[4] += bf16lo(av.z); o[5] += bf16hi(av.z); o[6] += bf16lo(av.w); o[7] += bf16hi(av.w);
        }
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = f32_to_bf16(o[2 * i]) | (static_cast<uint32_t>(f32_to_bf16(o[2 * i + 1])) << 16);
        store_stream16(static_cast<uint16_t*>(out) + off, make_uint4(w[0], w[1], w[2], w[3]));
      }
    }
    __syncthreads();
  }
}

// The lift as a loop over 64-token blocks (RK <= 64, z already summed over
// the D parts). A grid of G x S workgroups, about one per CU: the workgroup of
// D part p takes the blocks b, b + G, b + 2G, ... Its slice of Q (the part's
// 512 rows, bf16 hi/lo) is loaded once and stays in registers, and the next
// block's z, x and addend are loaded while the current block is multiplied
// and written, so a CU keeps a block of loads in flight behind its stores
// instead of waiting for memory once per block (one workgroup per CU fits
// the registers this takes). z goes through a double-buffered LDS split and
// the results through the stage above; the arithmetic per output is the
// lift kernel's, in the same order (the addend joins the fp32 accumulator
// before the bf16 rounding, as there), so both give the same bits.
template <int RK, bool OF32, bool ADD>
__global__ void __launch_bounds__(LNW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
lift_loop_kernel(const uint16_t* __restrict__ x, int64_t T, int D, int P,
                 const float* __restrict__ Z, const uint16_t* __restrict__ QH,
                 const uint16_t* __restrict__ QL, const uint16_t* __restrict__ addend,
                 void* __restrict__ out) {
  static_assert(RK == 32 || RK == 64, "the Q slice is held in registers");
  static_assert(!(OF32 && ADD), "a bf16 addend joins bf16 outputs only");
  constexpr int NT = LNW * 64;
  constexpr int KQ = RK / 32;
  constexpr int ZC = TPW * RK / 4;  // float4 chunks of one block's z
  constexpr int ZPT = ZC / NT;
  static_assert(ZC % NT == 0, "z chunks per thread");
  __shared__ __attribute__((aligned(16))) uint16_t zh[2][TPW][RK + 8];
  __shared__ __attribute__((aligned(16))) uint16_t zl[2][TPW][RK + 8];
  __shared__ __attribute__((aligned(16))) float stage[TB][kPart + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int part = blockIdx.y;
  const int dbeg = part * P;
  const int dend = min(D, dbeg + P);
  const int nds = (dend - dbeg) / 64;
  const int ncols = dend - dbeg;
  const int g = lane >> 4;
  const int tl = lane & 15;
  const bool live = wave < nds;
  const int d0 = dbeg + 64 * (live ? wave : nds - 1);
  const int64_t nb = (T + TPW - 1) / TPW;
  const int64_t G = gridDim.x;
  int64_t blk = blockIdx.x;
  if (blk >= nb) return;

  // loads of block b (tokens past T re-read the last token); unconditional
  float4 zn[ZPT];
  uint4 xn[TBW][2], an[TBW][2];
  auto load_block = [&](int64_t b) {
#pragma unroll
    for (int u = 0; u < ZPT; ++u) {
      const int c = tid + u * NT;
      const int64_t trow = min(b * TPW + (4 * c) / RK, T - 1);
      zn[u] = *reinterpret_cast<const float4*>(Z + trow * RK + (4 * c) % RK);
    }
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      const int64_t off = min(b * TPW + 16 * tb + tl, T - 1) * D + d0 + 16 * g;
      const uint4* px = reinterpret_cast<const uint4*>(x + off);
      xn[tb][0] = px[0];
      xn[tb][1] = px[1];
      if constexpr (ADD) {
        const uint4* pa = reinterpret_cast<const uint4*>(addend + off);
        an[tb][0] = pa[0];
        an[tb][1] = pa[1];
      }
    }
  };
  // z of a block, its bf16 split into LDS buffer q
  auto put_z = [&](int q) {
#pragma unroll
    for (int u = 0; u < ZPT; ++u) {
      const int c = tid + u * NT;
      const int tt = (4 * c) / RK;
      const int i = (4 * c) % RK;
      const float zz[4] = {zn[u].x, zn[u].y, zn[u].z, zn[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h = f32_to_bf16(zz[e]);
        zh[q][tt][i + e] = h;
        zl[q][tt][i + e] = f32_to_bf16(zz[e] - bf16_to_f32(h));
      }
    }
  };

  v8bf qh[4][KQ], ql[4][KQ];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int drow = d0 + 16 * (tl >> 2) + 4 * b + (tl & 3);
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const int64_t qo = static_cast<int64_t>(drow) * RK + 32 * kk + 8 * g;
      qh[b][kk] = ld8(QH + qo);
      ql[b][kk] = ld8(QL + qo);
    }
  }
  // this thread's store chunks of a 16-token result block: row and column
  constexpr int CW = OF32 ? 4 : 8;              // values per 16-byte store
  constexpr int SIT = TB * kPart / CW / NT;     // stores per thread
  int sr[SIT], sc[SIT];
#pragma unroll
  for (int it = 0; it < SIT; ++it) {
    const int c = tid + it * NT;
    sr[it] = c / (kPart / CW);
    const int col = (c % (kPart / CW)) * CW;
    sc[it] = col < ncols ? col : col % ncols;
  }
  load_block(blk);
  put_z(0);
  lds_barrier();
  int q = 0;
  for (;;) {
    uint4 xc[TBW][2], ac[TBW][2];
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      xc[tb][0] = xn[tb][0];
      xc[tb][1] = xn[tb][1];
      if constexpr (ADD) {
        ac[tb][0] = an[tb][0];
        ac[tb][1] = an[tb][1];
      }
    }
    const int64_t t0 = blk * TPW;
    const bool more = blk + G < nb;
    // the next block's loads (the last block's again after the final one)
    load_block(more ? blk + G : blk);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      if (live) {
        v4f acc[4];
        acc[0] = v4f{bf16lo(xc[tb][0].x), bf16hi(xc[tb][0].x), bf16lo(xc[tb][0].y), bf16hi(xc[tb][0].y)};
        acc[1] = v4f{bf16lo(xc[tb][0].z), bf16hi(xc[tb][0].z), bf16lo(xc[tb][0].w), bf16hi(xc[tb][0].w)};
        acc[2] = v4f{bf16lo(xc[tb][1].x), bf16hi(xc[tb][1].x), bf16lo(xc[tb][1].y), bf16hi(xc[tb][1].y)};
        acc[3] = v4f{bf16lo(xc[tb][1].z), bf16hi(xc[tb][1].z), bf16lo(xc[tb][1].w), bf16hi(xc[tb][1].w)};
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk) {
          const v8bf bh = *reinterpret_cast<const v8bf*>(&zh[q][16 * tb + tl][32 * kk + 8 * g]);
          const v8bf bl = *reinterpret_cast<const v8bf*>(&zl[q][16 * tb + tl][32 * kk + 8 * g]);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            acc[b] = mfma(qh[b][kk], bh, acc[b]);
            acc[b] = mfma(ql[b][kk], bh, acc[b]);
            acc[b] = mfma(qh[b][kk], bl, acc[b]);
          }
        }
        mfma_drain();
        if constexpr (ADD) {
          const uint32_t aw[8] = {ac[tb][0].x, ac[tb][0].y, ac[tb][0].z, ac[tb][0].w,
                                  ac[tb][1].x, ac[tb][1].y, ac[tb][1].z, ac[tb][1].w};
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            acc[b][0] += bf16lo(aw[2 * b]);
            acc[b][1] += bf16hi(aw[2 * b]);
            acc[b][2] += bf16lo(aw[2 * b + 1]);
            acc[b][3] += bf16hi(aw[2 * b + 1]);
          }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
          *reinterpret_cast<float4*>(&stage[tl][64 * wave + 16 * g + 4 * b]) =
              make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
      }
      lds_barrier();
      // a fixed number of unconditional stores per thread, so that the wait
      // for the next block's loads leaves these stores in flight (with a
      // runtime count the compiler must drain them all first). A row past T
      // holds exactly row T - 1's values (its x, addend and z loads were
      // clamped to that token) and rewrites them there; a column past a short
      // last part rewrites a column of the part.
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int row = sr[it];
        const int col = sc[it];
        const int64_t off = min(t0 + 16 * tb + row, T - 1) * D + dbeg + col;
        if constexpr (OF32) {
          store_stream16(static_cast<float*>(out) + off,
                         *reinterpret_cast<const float4*>(&stage[row][col]));
        } else {
          const float4 s0 = *reinterpret_cast<const float4*>(&stage[row][col]);
          const float4 s1 = *reinterpret_cast<const float4*>(&stage[row][col + 4]);
          const float o[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = f32_to_bf16(o[2 * i]) | (static_cast<uint32_t>(f32_to_bf16(o[2 * i + 1])) << 16);
          store_stream16(static_cast<uint16_t*>(out) + off, make_uint4(w[0], w[1], w[2], w[3]));
        }
      }
      if (tb + 1 < TBW) lds_barrier();
    }
    // the next block's z into the other buffer (its last reader was before
    // the previous iteration's final barrier), then one barrier for both the
    // stage and z
    put_z(q ^ 1);
    lds_barrier();
    if (!more) break;
    q ^= 1;
    blk += G;
  }
}

// Short batches (T <= kSmallT tokens, decode): the two steps on the vector
// ALUs, spread over D instead of over tokens, since a few tokens leave the
// token-blocked kernels a handful of workgroups that each pull the whole basis
// through one CU. Every global load of a thread is issued before its first
// use (compile-time bounded, predicated loops), so a thread waits for memory
// once per phase rather than once per iteration.
//   proj: one workgroup per 256-column chunk c: Zs[c][t][i] = sum over the
//         chunk of Q'[i][d] x[t][d], Q' = Q'h + Q'l (exact in fp32), fp32 FMA
//         in column order; x and 32-row blocks of Q' are staged in LDS.
//   lift: one workgroup per 64 columns: z = sum of the chunks in chunk order
//         (deterministic), then out[t][d] = x[t][d] + sum_i Q[d][i] z[t][i]
//         (+ addend), Q = Qh + Ql.
constexpr int kSmallLift = 64;
constexpr int kSmallMaxD = 16384;

__global__ void __launch_bounds__(256)
asmall_proj_kernel(const uint16_t* __restrict__ x, int T, int D, int RP, int RK,
                   const uint16_t* __restrict__ QtH, const uint16_t* __restrict__ QtL,
                   float* __restrict__ Zs) {
  asmall_proj_body(blockIdx.x, x, T, D, RP, RK, QtH, QtL, Zs);
}

template <bool OF32, bool ADD>
__global__ void __launch_bounds__(256)
asmall_lift_kernel(const uint16_t* __restrict__ x, int T, int D, int RK, int C,
                   const float* __restrict__ Zs, const uint16_t* __restrict__ QH,
                   const uint16_t* __restrict__ QL, const void* __restrict__ addend,
                   void* __restrict__ out) {
  __shared__ float zs[kSmallT][kPrepRmax + 1];
  const int tid = threadIdx.x;
  constexpr int TPT = (kSmallT + 256 / kSmallLift - 1) / (256 / kSmallLift);  // tokens per thread
  const int tt0 = tid / kSmallLift;
  // the thread's column of x (and of the addend) for its tokens, loaded first
  // (unconditional: clamped token and column, unused past T), so that these
  // loads overlap the z loads instead of following the stores one by one
  const int dl = min(blockIdx.x * kSmallLift + (tid & (kSmallLift - 1)), D - 1);
  uint16_t xr[TPT];
  float ar[TPT];
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int64_t off = static_cast<int64_t>(min(tt0 + u * (256 / kSmallLift), T - 1)) * D + dl;
    xr[u] = x[off];
    if constexpr (ADD) {
      if constexpr (OF32) ar[u] = static_cast<const float*>(addend)[off];
      else ar[u] = bf16_to_f32(static_cast<const uint16_t*>(addend)[off]);
    } else {
      ar[u] = 0.0f;
    }
  }
  // the first 32 values of the thread's row of Q (RK is a multiple of 32), also
  // independent of z
  const uint4* qh = reinterpret_cast<const uint4*>(QH + static_cast<int64_t>(dl) * RK);
  const uint4* ql = reinterpret_cast<const uint4*>(QL + static_cast<int64_t>(dl) * RK);
  uint4 hv[4], lv[4];
  auto loadrow = [&](int i0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hv[j] = qh[i0 / 8 + j];
      lv[j] = ql[i0 / 8 + j];
    }
  };
  loadrow(0);
  // z: every partial of a thread's entries loaded at once, summed in chunk order
  for (int o = tid; o < T * RK; o += 256) {
    const int t = o / RK, i = o % RK;
    float z = 0.0f;
    for (int c0 = 0; c0 < C; c0 += 16) {
      float zp[16];
#pragma unroll
      for (int c = 0; c < 16; ++c)
        zp[c] = Zs[(static_cast<int64_t>(min(c0 + c, C - 1)) * T + t) * RK + i];
#pragma unroll
      for (int c = 0; c < 16; ++c) z += c0 + c < C ? zp[c] : 0.0f;
    }
    zs[t][i] = z;
  }
  __syncthreads();
  const int d = blockIdx.x * kSmallLift + (tid & (kSmallLift - 1));
  if (d >= D) return;
  // the thread's row of Q in blocks of 32 values
  float corr[TPT];
#pragma unroll
  for (int u = 0; u < TPT; ++u) corr[u] = 0.0f;
  for (int i0 = 0; i0 < RK; i0 += 32) {
    if (i0 > 0) loadrow(i0);
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
    for (int u = 0; u < TPT; ++u) {
      const int t = min(tt0 + u * (256 / kSmallLift), kSmallT - 1);
#pragma unroll
      for (int i = 0; i < 32; ++i) corr[u] = fmaf(q[i], zs[t][i0 + i], corr[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int t = tt0 + u * (256 / kSmallLift);
    if (t >= T) break;
    const int64_t off = static_cast<int64_t>(t) * D + d;
    float acc = bf16_to_f32(xr[u]) + corr[u];
    if constexpr (ADD) acc += ar[u];
    if constexpr (OF32) static_cast<float*>(out)[off] = acc;
    else static_cast<uint16_t*>(out)[off] = f32_to_bf16(acc);
  }
}

inline int rp_of(int64_t r) { return static_cast<int>((r + 15) / 16 * 16); }
inline int rk_of(int64_t r) { return static_cast<int>((r + 31) / 32 * 32); }
inline size_t a256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

template <int RP>
hipError_t run_yproj(const uint16_t* x, int64_t T, int D, int P, int S, int r, const uint16_t* QtF,
                     float* Zpart, hipStream_t s) {
  // the loop form from 16 D parts on, when every workgroup of a grid of about
  // one per CU gets at least two blocks
  if constexpr (RP <= 64) {
    const int64_t nb = (T + YTPW - 1) / YTPW;
    const int64_t G = std::max<int64_t>(1, device_cus() / S);
    if (S >= 16 && nb >= 2 * G) {
      hipLaunchKernelGGL(yproj_loop_kernel<RP>, dim3(static_cast<unsigned>(G), S), dim3(YNW * 64),
                         0, s, x, T, D, P, QtF, Zpart);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(yproj_kernel<RP>, dim3(static_cast<unsigned>((T + YTPW - 1) / YTPW), S), dim3(YNW * 64),
                     0, s, x, T, D, P, r, QtF, Zpart);
  return hipGetLastError();
}

// z = the sum of the projection's S D-part partials, in part order from zero
// (the order the lift's own sum takes), written over part 0 so that the lift
// reads one partial: its workgroups, one per (64 tokens, D part), would
// otherwise each re-read all S partials of their tokens. Thread c owns float4
// chunk c of every part; it reads them all before it writes part 0's.
__global__ void __launch_bounds__(256)
zsum_kernel(float* __restrict__ Zpart, int64_t n4, int S) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= n4) return;
  float4* zp4 = reinterpret_cast<float4*>(Zpart);
  float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int p0 = 0; p0 < S; p0 += 8) {
    float4 zp[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) zp[q] = zp4[static_cast<int64_t>(min(p0 + q, S - 1)) * n4 + c];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (p0 + q < S) {
        z.x += zp[q].x; z.y += zp[q].y; z.z += zp[q].z; z.w += zp[q].w;
      }
  }
  zp4[c] = z;
}

template <int RP, int RK>
hipError_t run_lift(const uint16_t* x, int64_t T, int D, int P, int S, int SZ, int r,
                    const float* Zpart, const uint16_t* QH, const uint16_t* QL, const void* addend,
                    void* out, bool of32, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T + TPW - 1) / TPW), S);
#define RW4_LIFT(OF, AD)                                                                          \
  if (of32 == OF && (addend != nullptr) == AD) {                                                  \
    hipLaunchKernelGGL((lift_kernel<RP, RK, OF, AD>), grid, dim3(LNW * 64), 0, s, x, T, D, P, SZ, \
                       r, Zpart, QH, QL, addend, out);                                            \
    return hipGetLastError();                                                                     \
  }
  RW4_LIFT(true, false) RW4_LIFT(true, true) RW4_LIFT(false, false) RW4_LIFT(false, true)
#undef RW4_LIFT
  return hipErrorInvalidValue;
}

template <int RK>
hipError_t run_lift_loop(const uint16_t* x, int64_t T, int D, int P, int64_t G, int S,
                         const float* Z, const uint16_t* QH, const uint16_t* QL,
                         const void* addend, void* out, bool of32, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(G), S);
  const uint16_t* ab = static_cast<const uint16_t*>(addend);
  if (of32)
    hipLaunchKernelGGL((lift_loop_kernel<RK, true, false>), grid, dim3(LNW * 64), 0, s, x, T, D, P,
                       Z, QH, QL, ab, out);
  else if (addend != nullptr) {
    if constexpr (RK == 64)
      hipLaunchKernelGGL((lift_loop_kernel<RK, false, true>), grid, dim3(LNW * 64), 0, s, x, T, D,
                         P, Z, QH, QL, ab, out);
    else
      return hipErrorInvalidValue;  // not taken: the one-block kernel serves RK = 32 with addend
  } else
    hipLaunchKernelGGL((lift_loop_kernel<RK, false, false>), grid, dim3(LNW * 64), 0, s, x, T, D,
                       P, Z, QH, QL, ab, out);
  return hipGetLastError();
}

}  // namespace

bool align_mfma_supported(int64_t D, int64_t r) { return r > 0 && r <= 128 && D % 64 == 0; }

int align_parts_count(int64_t D) { return static_cast<int>((D + kPart - 1) / kPart); }

size_t align_zpart_bytes(int64_t T, int64_t D, int64_t r) {
  const int64_t parts = align_small(T, D) ? std::max<int64_t>(align_parts_count(D),
                                                         (D + kSmallChunk - 1) / kSmallChunk)
                                     : align_parts_count(D);
  return a256(static_cast<size_t>(parts) * static_cast<size_t>(T) *
              static_cast<size_t>(rk_of(r)) * 4);
}

size_t align_basis_bytes(int64_t D, int64_t r, bool with_p) {
  const size_t RP = rp_of(r), RK = rk_of(r), Dz = static_cast<size_t>(D);
  size_t n = 2 * a256(RP * Dz * 2) + 2 * a256(Dz * RK * 2) + a256(RP * Dz * 4);
  if (with_p) n += 2 * a256(Dz * RK * 2);
  return n;
}

AlignBasis align_basis(const void* basis, int64_t D, int64_t r, bool with_p) {
  const size_t RP = rp_of(r), RK = rk_of(r), Dz = static_cast<size_t>(D);
  AlignBasis a;
  a.RP = static_cast<int>(RP);
  a.RK = static_cast<int>(RK);
  uint8_t* p = static_cast<uint8_t*>(const_cast<void*>(basis));
  a.QtH = reinterpret_cast<uint16_t*>(p); p += a256(RP * Dz * 2);
  a.QtL = reinterpret_cast<uint16_t*>(p); p += a256(RP * Dz * 2);
  a.QH = reinterpret_cast<uint16_t*>(p);  p += a256(Dz * RK * 2);
  a.QL = reinterpret_cast<uint16_t*>(p);  p += a256(Dz * RK * 2);
  a.QtF = reinterpret_cast<uint16_t*>(p); p += a256(RP * Dz * 4);
  a.PH = with_p ? reinterpret_cast<uint16_t*>(p) : nullptr;
  if (with_p) p += a256(Dz * RK * 2);
  a.PL = with_p ? reinterpret_cast<uint16_t*>(p) : nullptr;
  return a;
}

hipError_t launch_basis_prep(const float* Q, const float* M, int64_t D, int64_t r, bool with_p,
                             void* basis, hipStream_t s) {
  const AlignBasis a = align_basis(basis, D, r, with_p);
  const float norm = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(D)));
  if (with_p && D == kBasisFwhtFast) {
    // one launch (15.1 us in two)
    const int gx = static_cast<int>(D / 64);
    hipLaunchKernelGGL(basis_prep_p4096_kernel,
                       dim3(static_cast<unsigned>(gx * (a.RK / 32) + a.RK)), dim3(256), 0, s, Q, M,
                       static_cast<int>(r), a.RP, a.RK, gx, a.QtH, a.QtL, a.QH, a.QL, a.QtF, norm,
                       a.PH, a.PL);
    return hipGetLastError();
  }
  const dim3 pgrid(static_cast<unsigned>((D + 63) / 64), static_cast<unsigned>(a.RK / 32));
  hipLaunchKernelGGL(basis_prep_kernel, pgrid, dim3(256), 0, s, Q, M, static_cast<int>(D),
                     static_cast<int>(r), a.RP, a.RK, a.QtH, a.QtL, a.QH, a.QL, a.QtF);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !with_p) return e;
  if ((D & (D - 1)) != 0 || D > kBasisFwhtMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(basis_fwht_kernel, dim3(static_cast<unsigned>(a.RK)), dim3(1024), 0, s, Q,
                     static_cast<int>(D), static_cast<int>(r), a.RK, norm, a.PH, a.PL);
  return hipGetLastError();
}

hipError_t launch_yproj(const uint16_t* x, int64_t T, int64_t D, int64_t r, const void* basis,
                        bool with_p, float* Zpart, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const AlignBasis a = align_basis(basis, D, r, with_p);
  const int Di = static_cast<int>(D);
  const int ri = static_cast<int>(r);
  const int S = align_parts_count(D);
  switch (a.RP) {
#define RW4_Y(V) case V: return run_yproj<V>(x, T, Di, kPart, S, ri, a.QtF, Zpart, s);
    RW4_Y(16) RW4_Y(32) RW4_Y(48) RW4_Y(64) RW4_Y(80) RW4_Y(96) RW4_Y(112) RW4_Y(128)
#undef RW4_Y
    default: return hipErrorInvalidValue;
  }
}

bool align_small(int64_t T, int64_t D) { return T >= 1 && T <= kSmallT && D <= kSmallMaxD; }

int align_small_chunks(int64_t D) { return static_cast<int>((D + kSmallChunk - 1) / kSmallChunk); }

hipError_t launch_align_small_project(const uint16_t* x, int64_t T, int64_t D, int64_t r,
                                      const void* basis, bool with_p, float* Zs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!align_small(T, D) || D % 64 != 0 || r < 1 || r > kPrepRmax) return hipErrorInvalidValue;
  const AlignBasis a = align_basis(basis, D, r, with_p);
  hipLaunchKernelGGL(asmall_proj_kernel, dim3(static_cast<unsigned>(align_small_chunks(D))),
                     dim3(256), 0, s, x, static_cast<int>(T), static_cast<int>(D), a.RP, a.RK,
                     a.QtH, a.QtL, Zs);
  return hipGetLastError();
}

hipError_t launch_align_small(const uint16_t* x, void* out, int out_f32, const void* addend,
                              int64_t T, int64_t D, int64_t r, const void* basis, bool with_p,
                              float* Zs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!align_small(T, D) || D % 64 != 0 || D > kSmallMaxD || r < 1 || r > kPrepRmax)
    return hipErrorInvalidValue;
  const AlignBasis a = align_basis(basis, D, r, with_p);
  const int Ti = static_cast<int>(T), Di = static_cast<int>(D);
  const int C = static_cast<int>((D + kSmallChunk - 1) / kSmallChunk);
  hipLaunchKernelGGL(asmall_proj_kernel, dim3(static_cast<unsigned>(C)), dim3(256), 0, s, x, Ti,
                     Di, a.RP, a.RK, a.QtH, a.QtL, Zs);
  const dim3 lg(static_cast<unsigned>((D + kSmallLift - 1) / kSmallLift));
#define RW4_AS(OF, AD)                                                                            \
  if ((out_f32 != 0) == OF && (addend != nullptr) == AD) {                                        \
    hipLaunchKernelGGL((asmall_lift_kernel<OF, AD>), lg, dim3(256), 0, s, x, Ti, Di, a.RK, C, Zs, \
                       a.QH, a.QL, addend, out);                                                  \
    return hipGetLastError();                                                                     \
  }
  RW4_AS(true, false) RW4_AS(true, true) RW4_AS(false, false) RW4_AS(false, true)
#undef RW4_AS
  return hipErrorInvalidValue;
}

size_t align_mfma_workspace(int64_t T, int64_t D, int64_t r) {
  return align_basis_bytes(D, r, false) + align_zpart_bytes(T, D, r);
}

hipError_t launch_align_mfma(const uint16_t* x, void* out, int out_f32, const float* Q,
                             const float* M, const void* addend, int64_t T, int64_t D, int64_t r,
                             void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipError_t e = launch_basis_prep(Q, M, D, r, false, ws, s);
  if (e != hipSuccess) return e;
  float* Zpart = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_basis_bytes(D, r, false));
  if (align_small(T, D))
    return launch_align_small(x, out, out_f32, addend, T, D, r, ws, false, Zpart, s);
  e = launch_yproj(x, T, D, r, ws, false, Zpart, s);
  if (e != hipSuccess) return e;
  return launch_lift(x, out, out_f32, addend, T, D, r, ws, false, Zpart, s);
}

hipError_t launch_lift(const uint16_t* x, void* out, int out_f32, const void* addend, int64_t T,
                       int64_t D, int64_t r, const void* basis, bool with_p, float* Zpart,
                       hipStream_t s) {
  if (T == 0) return hipSuccess;
  const AlignBasis a = align_basis(basis, D, r, with_p);
  const int Di = static_cast<int>(D);
  const int ri = static_cast<int>(r);
  const int S = align_parts_count(D);
  const bool of32 = out_f32 != 0;
  // the loop form from 16 D parts on, when every workgroup of a grid of about
  // one per CU gets at least two blocks. Measured against the one-block
  // kernel: 193.7 -> 152.7 us at T = D = 8192, r = 64 (fp32 out); slower at
  // 8 parts, where two resident one-block workgroups per CU keep more loads
  // in flight than one looping workgroup (which also needs the partials
  // summed first), and with an addend at RK = 32 (its registers for a small
  // basis slice: 76.8 against 72.2 us at T = 4096, D = 8192)
  const int64_t nb = (T + TPW - 1) / TPW;
  const int64_t G = std::max<int64_t>(1, device_cus() / S);
  const bool loop = S >= 16 && a.RK <= 64 && (addend == nullptr || (a.RK == 64 && !of32)) &&
                    nb >= 2 * G;
  // from 16 D parts on, the partials are summed once (in place) for all
  // workgroups: S^2 T RK floats of L2 reads become S T RK
  int SZ = S;
  if (S >= 16) {
    const int64_t n4 = T * rk_of(r) / 4;
    hipLaunchKernelGGL(zsum_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s,
                       Zpart, n4, S);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SZ = 1;
  }
  if (loop) {
    if (a.RK == 32)
      return run_lift_loop<32>(x, T, Di, kPart, G, S, Zpart, a.QH, a.QL, addend, out, of32, s);
    return run_lift_loop<64>(x, T, Di, kPart, G, S, Zpart, a.QH, a.QL, addend, out, of32, s);
  }
  switch (a.RP) {
#define RW4_L(V, K) \
  case V:           \
    return run_lift<V, K>(x, T, Di, kPart, S, SZ, ri, Zpart, a.QH, a.QL, addend, out, of32, s);
    RW4_L(16, 32) RW4_L(32, 32) RW4_L(48, 64) RW4_L(64, 64) RW4_L(80, 96) RW4_L(96, 96)
    RW4_L(112, 128) RW4_L(128, 128)
#undef RW4_L
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rw4
