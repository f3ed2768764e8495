// Offline construction of the alignment's (Q, R_sub) from a residual
// transition T = R_out R_in^T (ReSpinQuant paper notes, key design 2):
//   Delta T = T - I; Q = its top-r left singular vectors; T_sub = Q^T T Q;
//   R_sub = U_sub V_sub^T, the orthogonal polar factor of T_sub.
//
// The top-r singular subspace comes from a randomized range finder with
// subspace iteration (Halko, Martinsson and Tropp, "Finding structure with
// randomness", 2011), in fp64 throughout:
//   Z = Delta T Omega (Omega: D x p Rademacher signs from a counter hash,
//       p = r + 16);
//   q times: Z <- orth(Z); Y = Delta T^T Z; Y <- orth(Y); Z = Delta T Y;
//   Z <- orth(Z); C = (Delta T^T Z)^T (Delta T^T Z) = Z^T Delta T Delta T^T Z;
//   C = W L W^T (eigenvalues descending): Q = Z W[:, :r] (Rayleigh-Ritz).
// orth() is SVQB (Stathopoulos and Wu, 2002): G = Y^T Y = V L V^T,
// Y <- Y V L^-1/2, with columns of eigenvalue below 1e-22 of the largest set
// to zero, so a rank-deficient block (Delta T of rank < p) stays exact.
// The polar factor is T_sub (T_sub^T T_sub)^-1/2 from the same eigensolver:
// a cyclic Jacobi method in one workgroup, the pairs of each step chosen by
// the round-robin ordering so that all n/2 rotations of a step run at once.
// Products with T read it from HBM as fp32 and accumulate in fp64, as sums
// over K parts (register-blocked workgroups of 128 rows, the parts added in
// part order); only Q and R_sub are rounded to fp32 at the end.
#include "common.hpp"
#include "launch.hpp"

namespace rw4 {
namespace {

constexpr int kCPad = 16;      // oversampling of the range finder
constexpr int kCMaxN = 80;     // largest eigenproblem (r <= 64)

// Rademacher sign of entry (d, k) of Omega: bit 0 of a 32-bit mix of the index
__device__ __forceinline__ double omega_sign(uint32_t d, uint32_t k) {
  uint32_t h = d * 0x9E3779B1u ^ (k + 0x7F4A7C15u) * 0x85EBCA77u;
  h ^= h >> 16; h *= 0x7FEB352Du; h ^= h >> 15; h *= 0x846CA68Bu; h ^= h >> 16;
  return (h & 1u) ? -1.0 : 1.0;
}

__global__ void omega_kernel(double* __restrict__ Y, int D, int p) {
  const int64_t n = static_cast<int64_t>(D) * p;
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256)
    Y[e] = omega_sign(static_cast<uint32_t>(e / p), static_cast<uint32_t>(e % p));
}

// Y[i][c] = sum_j op(T)[i][j] X[j][c] - sub X[i][c] for c < nc; X, Y fp64 [D][nc];
// op(T) = T or T^T, T fp32 [D][D] (exact in fp64).
// The same product as partial sums over K parts, register-blocked: a
// workgroup of 256 threads owns 128 output rows x 16 NCPT columns of part q
// (k in [q D / KS, (q + 1) D / KS)); thread (g, c) accumulates rows 8 g .. +7
// and columns c + 16 j (j < NCPT) in fp64, so each k costs 8 + NCPT LDS reads
// for 8 NCPT FMAs. Chunks of 32 k of op(T) (fp32) and X (fp64) are staged in
// LDS (conflict-free: [k][row] with a 129-word pitch), the next chunk fetched
// into registers meanwhile. Part sums go to P[q][i][c]; tsum_kernel adds the
// parts in part order and subtracts sub X.
constexpr int kTRows = 128;
constexpr int kTChunk = 32;

template <bool TR, int NCPT>
__global__ void __launch_bounds__(256)
tpart_kernel(const float* __restrict__ T, int D, const double* __restrict__ X, int nc, int KL,
             double* __restrict__ P) {
  constexpr int NCB = 16 * NCPT;                       // columns of the block
  constexpr int TPT = kTRows * kTChunk / 256;          // T values per thread and chunk
  constexpr int XPT = (kTChunk * NCB + 255) / 256;     // X values per thread and chunk
  __shared__ float Tt[kTChunk][kTRows + 1];
  __shared__ double Xt[kTChunk][NCB];
  const int tid = threadIdx.x;
  const int g = tid >> 4, c = tid & 15;
  const int i0 = blockIdx.x * kTRows;
  const int q = blockIdx.y;
  const int kbeg = q * KL;
  double acc[8][NCPT];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int j = 0; j < NCPT; ++j) acc[a][j] = 0.0;
  float tr[TPT];
  double xr[XPT];
  // loads are unconditional (clamped rows, masked columns), all in flight at once
  auto fetch = [&](int k0) {
#pragma unroll
    for (int m = 0; m < TPT; ++m) {
      const int e = tid + 256 * m;
      if constexpr (TR) {
        const int kk = e / kTRows, row = min(i0 + e % kTRows, D - 1);
        tr[m] = T[static_cast<int64_t>(k0 + kk) * D + row];
      } else {
        const int row = min(i0 + e / kTChunk, D - 1), kk = e % kTChunk;
        tr[m] = T[static_cast<int64_t>(row) * D + k0 + kk];
      }
    }
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int e = min(tid + 256 * m, kTChunk * NCB - 1);
      const int kk = e / NCB, col = e % NCB;
      xr[m] = X[static_cast<int64_t>(k0 + kk) * nc + min(col, nc - 1)];
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int m = 0; m < TPT; ++m) {
      const int e = tid + 256 * m;
      if constexpr (TR) Tt[e / kTRows][e % kTRows] = tr[m];
      else Tt[e % kTChunk][e / kTChunk] = tr[m];
    }
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int e = tid + 256 * m;
      if (e < kTChunk * NCB) Xt[e / NCB][e % NCB] = e % NCB < nc ? xr[m] : 0.0;
    }
  };
  const int nch = KL / kTChunk;
  fetch(kbeg);
  for (int ci = 0; ci < nch; ++ci) {
    stash();
    __syncthreads();
    if (ci + 1 < nch) fetch(kbeg + (ci + 1) * kTChunk);
#pragma unroll 4
    for (int kk = 0; kk < kTChunk; ++kk) {
      double x[NCPT];
#pragma unroll
      for (int j = 0; j < NCPT; ++j) x[j] = Xt[kk][c + 16 * j];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const double t = static_cast<double>(Tt[kk][8 * g + a]);
#pragma unroll
        for (int j = 0; j < NCPT; ++j) acc[a][j] = fma(t, x[j], acc[a][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int i = i0 + 8 * g + a;
    if (i >= D) continue;
#pragma unroll
    for (int j = 0; j < NCPT; ++j) {
      const int col = c + 16 * j;
      if (col < nc) P[(static_cast<int64_t>(q) * D + i) * nc + col] = acc[a][j];
    }
  }
}

// Y[i][c] = sum over the KS parts (in part order) - sub X[i][c]
__global__ void __launch_bounds__(256)
tsum_kernel(const double* __restrict__ P, int KS, int64_t n, const double* __restrict__ X,
            double sub, double* __restrict__ Y) {
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256) {
    double acc = 0.0;
    for (int q0 = 0; q0 < KS; q0 += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = P[static_cast<int64_t>(min(q0 + u, KS - 1)) * n + e];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (q0 + u < KS) acc += v[u];
    }
    Y[e] = acc - sub * X[e];
  }
}

// G[i][j] = sum_d A[d][i] B[d][j] (A [D][na], B [D][nb]); workgroup (i, 16 columns)
__global__ void __launch_bounds__(256)
gram_kernel(const double* __restrict__ A, int na, const double* __restrict__ B, int nb, int D,
            double* __restrict__ G) {
  __shared__ double part[4][16];
  const int i = blockIdx.x;
  const int j0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
  double acc[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) acc[jj] = 0.0;
  for (int d = tid; d < D; d += 256) {
    const double a = A[static_cast<int64_t>(d) * na + i];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      if (j0 + jj < nb) acc[jj] = fma(a, B[static_cast<int64_t>(d) * nb + j0 + jj], acc[jj]);
  }
  // fixed-order reduction: butterflies inside the wave, then the four waves
#pragma unroll
  for (int jj = 0; jj < 16; ++jj)
    for (int o = 32; o > 0; o >>= 1) acc[jj] += __shfl_xor(acc[jj], o);
  if ((tid & 63) == 0)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) part[tid >> 6][jj] = acc[jj];
  __syncthreads();
  if (tid < 16 && j0 + tid < nb)
    G[static_cast<int64_t>(i) * nb + j0 + tid] = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
}

// Y[d][c] = sum_k X[d][k] M[k][c] (X [D][nx], M [nx][nm], Y [D][nm]); Y may not alias X
__global__ void __launch_bounds__(256)
rmul_kernel(const double* __restrict__ X, int nx, const double* __restrict__ Mm, int nm, int D,
            double* __restrict__ Y) {
  __shared__ double Ms[kCMaxN * kCMaxN];
  for (int e = threadIdx.x; e < nx * nm; e += 256) Ms[e] = Mm[e];
  __syncthreads();
  const int64_t n = static_cast<int64_t>(D) * nm;
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t d = e / nm;
    const int c = static_cast<int>(e % nm);
    double acc = 0.0;
    for (int k = 0; k < nx; ++k) acc = fma(X[d * nx + k], Ms[k * nm + c], acc);
    Y[e] = acc;
  }
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return v;
}

// symmetric eigenproblem A = V diag(A') V^T in LDS, n even (<= kCMaxN), 256
// threads. Each round's n/2 disjoint pairs come from the round-robin
// ordering (position 0 fixed, positions 1..n-1 rotated by the round).
__device__ void jacobi_eig(double (*A)[kCMaxN + 1], double (*V)[kCMaxN + 1], int n, double* cs_c,
                          double* cs_s, int* pp, int* qq, double* red) {
  const int tid = threadIdx.x;
  for (int i = tid; i < n * kCMaxN; i += 256) {
    const int row = i / kCMaxN, col = i % kCMaxN;
    if (col < n) V[row][col] = row == col ? 1.0 : 0.0;
  }
  double fro = 0.0;
  for (int e = tid; e < n * n; e += 256) fro += A[e / n][e % n] * A[e / n][e % n];
  fro = block_sum(fro, red);
  const int h = n / 2;
  for (int sweep = 0; sweep < 40; ++sweep) {
    double off = 0.0;
    for (int e = tid; e < n * n; e += 256) {
      const int row = e / n, col = e % n;
      if (col != row) off += A[row][col] * A[row][col];
    }
    off = block_sum(off, red);                      // identical in every thread
    if (!(off > 1e-30 * fro)) break;
    for (int rr = 0; rr < n - 1; ++rr) {
      if (tid < h) {
        const int a = tid == 0 ? 0 : 1 + (tid - 1 + rr) % (n - 1);
        const int b = 1 + (n - 2 - tid + rr) % (n - 1);
        const int p = a < b ? a : b, q = a < b ? b : a;
        const double apq = A[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double tau = (A[q][q] - A[p][p]) / (2.0 * apq);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        pp[tid] = p;
        qq[tid] = q;
        cs_c[tid] = c;
        cs_s[tid] = s;
      }
      __syncthreads();
      // A <- J^T A J: the pairs cover every index once, so each entry lies in
      // exactly one 2 x 2 block (rows of pair k, columns of pair l); a thread
      // applies k's row rotation and then l's column rotation to a block, the
      // same operations in the same order as a row pass followed by a column
      // pass. V <- V J on the pairs' columns.
      for (int e = tid; e < h * h; e += 256) {
        const int k = e / h, l = e % h;
        const int p = pp[k], q = qq[k], u = pp[l], v = qq[l];
        const double ck = cs_c[k], sk = cs_s[k], cl = cs_c[l], sl = cs_s[l];
        const double apu = A[p][u], apv = A[p][v], aqu = A[q][u], aqv = A[q][v];
        const double bpu = ck * apu - sk * aqu, bqu = sk * apu + ck * aqu;
        const double bpv = ck * apv - sk * aqv, bqv = sk * apv + ck * aqv;
        A[p][u] = cl * bpu - sl * bpv;
        A[p][v] = sl * bpu + cl * bpv;
        A[q][u] = cl * bqu - sl * bqv;
        A[q][v] = sl * bqu + cl * bqv;
      }
      for (int e = tid; e < n * h; e += 256) {
        const int row = e / h, l = e % h;
        const int u = pp[l], v = qq[l];
        const double c = cs_c[l], s = cs_s[l];
        const double vu = V[row][u], vv = V[row][v];
        V[row][u] = c * vu - s * vv;
        V[row][v] = s * vu + c * vv;
      }
      __syncthreads();
    }
  }
}

enum SmallMode { SM_SVQB = 0, SM_RR = 1, SM_POLAR = 2 };

// One workgroup. SVQB: G (n x n) -> out = V diag(l^-1/2 or 0) (n x n).
// RR: C (n x n) -> out = the r eigenvectors of the largest eigenvalues, in
// descending order (n x r). POLAR: T_sub (n x n = r x r) -> R fp32 (n x n).
template <int MODE>
__global__ void __launch_bounds__(256)
small_kernel(const double* __restrict__ in, int n, int r, double* __restrict__ out,
             float* __restrict__ out32) {
  // rows padded by one double: column walks spread over the banks
  __shared__ double A[kCMaxN][kCMaxN + 1];
  __shared__ double V[kCMaxN][kCMaxN + 1];
  __shared__ double cs_c[kCMaxN / 2], cs_s[kCMaxN / 2], lam[kCMaxN], red[4];
  __shared__ int pp[kCMaxN / 2], qq[kCMaxN / 2], perm[kCMaxN];
  const int tid = threadIdx.x;
  for (int e = tid; e < n * n; e += 256) {
    const int i = e / n, j = e % n;
    if constexpr (MODE == SM_POLAR) {
      double acc = 0.0;                            // A = T_sub^T T_sub
      for (int k = 0; k < n; ++k) acc = fma(in[k * n + i], in[k * n + j], acc);
      A[i][j] = acc;
    } else {
      A[i][j] = in[e];
    }
  }
  __syncthreads();
  jacobi_eig(A, V, n, cs_c, cs_s, pp, qq, red);
  if (tid < n) lam[tid] = A[tid][tid];
  __syncthreads();
  double lmax = 0.0;
  for (int k = 0; k < n; ++k) lmax = fmax(lmax, lam[k]);
  if constexpr (MODE == SM_SVQB) {
    for (int e = tid; e < n * n; e += 256) {
      const int i = e / n, j = e % n;
      const double l = lam[j];
      out[e] = l > 1e-22 * lmax ? V[i][j] / sqrt(l) : 0.0;
    }
  } else if constexpr (MODE == SM_RR) {
    if (tid < n) {
      int rank = 0;
      for (int k = 0; k < n; ++k)
        rank += (lam[k] > lam[tid]) || (lam[k] == lam[tid] && k < tid);
      perm[rank] = tid;
    }
    __syncthreads();
    for (int e = tid; e < n * r; e += 256) out[e] = V[e / r][perm[e % r]];
  } else {
    // R = (T_sub V) diag(l^-1/2) V^T, eigenvalues below 1e-22 of the largest
    // dropped; T_sub V (scaled) reuses A
    __syncthreads();
    for (int e = tid; e < n * n; e += 256) {
      const int i = e / n, k = e % n;
      double tv = 0.0;
      for (int m = 0; m < n; ++m) tv = fma(in[i * n + m], V[m][k], tv);
      A[i][k] = lam[k] > 1e-22 * lmax ? tv / sqrt(lam[k]) : 0.0;
    }
    __syncthreads();
    for (int e = tid; e < n * n; e += 256) {
      const int i = e / n, j = e % n;
      double acc = 0.0;
      for (int k = 0; k < n; ++k) acc = fma(A[i][k], V[j][k], acc);
      out32[e] = static_cast<float>(acc);
    }
  }
}

__global__ void to_f32_kernel(const double* __restrict__ a, int64_t n, float* __restrict__ o) {
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256)
    o[e] = static_cast<float>(a[e]);
}

inline int64_t a256c(int64_t n) { return (n + 255) & ~static_cast<int64_t>(255); }

}  // namespace

int construct_oversampled(int64_t D, int64_t r) {
  const int64_t p = r + kCPad;
  return static_cast<int>(p < D ? p : D);
}

// K parts of the products: about 256 workgroups of 128 rows, parts of at
// least one 32-value chunk
int construct_kparts(int64_t D) {
  int64_t ks = (256 * kTRows) / D;
  if (ks < 1) ks = 1;
  while (ks > 1 && (D % (ks * kTChunk)) != 0) --ks;
  return static_cast<int>(ks);
}

size_t construct_workspace(int64_t D, int64_t r) {
  const int64_t p = construct_oversampled(D, r);
  return static_cast<size_t>(2 * a256c(D * p * 8) + 2 * a256c(kCMaxN * kCMaxN * 8) +
                             a256c(static_cast<int64_t>(construct_kparts(D)) * D * p * 8));
}

bool construct_supported(int64_t D, int64_t r) {
  return r >= 4 && r <= 64 && r % 4 == 0 && D >= 64 && D % 64 == 0 && D <= 16384 && r <= D;
}

hipError_t launch_construct(const float* T, int64_t D64, int64_t r64, int iters, float* Qout,
                            float* Rout, void* ws, hipStream_t s) {
  if (!construct_supported(D64, r64) || iters < 0 || iters > 32) return hipErrorInvalidValue;
  const int D = static_cast<int>(D64), r = static_cast<int>(r64);
  const int p = construct_oversampled(D64, r64);
  uint8_t* w = static_cast<uint8_t*>(ws);
  double* Y = reinterpret_cast<double*>(w);
  double* Z = reinterpret_cast<double*>(w + a256c(int64_t(D) * p * 8));
  double* G = reinterpret_cast<double*>(w + 2 * a256c(int64_t(D) * p * 8));
  double* Mm = reinterpret_cast<double*>(w + 2 * a256c(int64_t(D) * p * 8) + a256c(kCMaxN * kCMaxN * 8));
  const dim3 b256(256);
  const int64_t ewn = (int64_t(D) * p + 255) / 256;
  const unsigned ew = static_cast<unsigned>(ewn < 4096 ? ewn : 4096);
  double* Pp = reinterpret_cast<double*>(w + 2 * a256c(int64_t(D) * p * 8) +
                                         2 * a256c(kCMaxN * kCMaxN * 8));
  const int KS = construct_kparts(D);
  const dim3 pgrid(static_cast<unsigned>((D + kTRows - 1) / kTRows), static_cast<unsigned>(KS));
  auto tmul = [&](bool tr, const double* X, int nc, double sub, double* Yo) {
    const int KL = D / KS;
#define RW4_TP(NC)                                                                           \
    if ((nc + 15) / 16 == NC) {                                                              \
      if (tr) hipLaunchKernelGGL((tpart_kernel<true, NC>), pgrid, b256, 0, s, T, D, X, nc, KL, Pp); \
      else hipLaunchKernelGGL((tpart_kernel<false, NC>), pgrid, b256, 0, s, T, D, X, nc, KL, Pp); \
    }
    RW4_TP(1) RW4_TP(2) RW4_TP(3) RW4_TP(4) RW4_TP(5)
#undef RW4_TP
    const int64_t n = int64_t(D) * nc;
    const int64_t sb = (n + 255) / 256;
    hipLaunchKernelGGL(tsum_kernel, dim3(static_cast<unsigned>(sb < 4096 ? sb : 4096)), b256, 0, s, Pp,
                       KS, n, X, sub, Yo);
  };
  // X <- orth(X) through tmp
  auto orth = [&](double* X, double* tmp) {
    hipLaunchKernelGGL(gram_kernel, dim3(p, (p + 15) / 16), b256, 0, s, X, p, X, p, D, G);
    hipLaunchKernelGGL((small_kernel<SM_SVQB>), dim3(1), b256, 0, s, G, p, p, Mm, nullptr);
    hipLaunchKernelGGL(rmul_kernel, dim3(ew), b256, 0, s, X, p, Mm, p, D, tmp);
  };
  hipLaunchKernelGGL(omega_kernel, dim3(ew), b256, 0, s, Y, D, p);
  tmul(false, Y, p, 1.0, Z);                        // Z = dT Omega
  for (int it = 0; it < iters; ++it) {
    orth(Z, Y);                                     // Y = orth(Z)
    tmul(true, Y, p, 1.0, Z);                       // Z = dT^T Y
    orth(Z, Y);                                     // Y = orth(Z)
    tmul(false, Y, p, 1.0, Z);                      // Z = dT Y
  }
  orth(Z, Y);                                       // Y: orthonormal range basis
  tmul(true, Y, p, 1.0, Z);                         // Z = dT^T Y
  hipLaunchKernelGGL(gram_kernel, dim3(p, (p + 15) / 16), b256, 0, s, Z, p, Z, p, D, G);
  hipLaunchKernelGGL((small_kernel<SM_RR>), dim3(1), b256, 0, s, G, p, r, Mm, nullptr);
  hipLaunchKernelGGL(rmul_kernel, dim3(ew), b256, 0, s, Y, p, Mm, r, D, Z);  // Z: Q [D][r]
  tmul(false, Z, r, 0.0, Y);                        // Y = T Q [D][r]
  hipLaunchKernelGGL(gram_kernel, dim3(r, (r + 15) / 16), b256, 0, s, Z, r, Y, r, D, G);  // T_sub
  hipLaunchKernelGGL((small_kernel<SM_POLAR>), dim3(1), b256, 0, s, G, r, r, nullptr, Rout);
  hipLaunchKernelGGL(to_f32_kernel, dim3(ew), b256, 0, s, Z, int64_t(D) * r, Qout);
  return hipGetLastError();
}

}  // namespace rw4
