// Host-side launchers of the gfx950 kernels (called by the C ABI after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace rw4 {

// compute units of the current device (256 on MI355X), read once per device
inline int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

enum InMode { IN_BF16 = 0, IN_F32 = 1, IN_SWIGLU = 2 };

// Per-row transform: [SiLU gate] -> [Walsh-Hadamard] -> output.
// Output either fp32 values (yf) or b-bit codes (b = bits, 2..4) + scales
// (+ optional fp32 dump). Codes go to packed INT4 rows, or (tiled, D >= 64)
// to FP6 operand tiles. D must be a power of two in [2, 32768].
hipError_t launch_row(const void* x, int in_mode, int64_t ldx, int64_t T, int64_t D, bool do_fwht,
                      float* yf, uint8_t* codes, bool tiled, float* scales, float* dbg,
                      hipStream_t s, int bits = 4);

// Structured Hadamard transform of rows, y = (H_A (x) K_B) diag(s) x * norm
// with A a power of two, K_B = Paley H_m (m = B in {12, 20, 28}) or the
// identity (m = 0); D = A B <= kKronMaxD, D % 4 == 0. Output fp32 rows (y),
// or b-bit codes + scales (+ fp32 dump) as packed INT4 rows or FP6 tiles
// (then D % 32 == 0, tiles D % 64 == 0). signs nullable ([D] of +-1).
constexpr int kKronMaxD = 16384;
bool kron_order_supported(int64_t m);
hipError_t launch_kron(const void* x, int in_mode, int64_t ldx, int64_t T, int64_t A, int64_t B,
                       int m, const float* signs, float norm, float* y, uint8_t* codes,
                       bool tiled, float* scales, float* dbg, int bits, hipStream_t s);

// Offline (Q, R_sub) of a residual transition T (fp32 [D][D]) on the device,
// fp64 inside; workspace of construct_workspace(D, r) bytes.
bool construct_supported(int64_t D, int64_t r);
size_t construct_workspace(int64_t D, int64_t r);
hipError_t launch_construct(const float* T, int64_t D, int64_t r, int iters, float* Q, float* R,
                            void* ws, hipStream_t s);

// Per-row b-bit quantization for any even D (no transform).
hipError_t launch_quant_generic(const void* x, int in_mode, int64_t ldx, int64_t T, int64_t D,
                                uint8_t* codes, float* scales, hipStream_t s, int bits = 4);

// Low-rank residual alignment out = x + Q (M - I) Q^T x (+ addend).
hipError_t launch_align(const void* x, int x_f32, void* out, int out_f32, const float* Q,
                        const float* M, const void* addend, int64_t T, int64_t D, int64_t r,
                        hipStream_t s);

// Alignment on bf16 MFMA (bf16 x only); workspace from align_mfma_workspace().
bool align_mfma_supported(int64_t D, int64_t r);
size_t align_mfma_workspace(int64_t T, int64_t D, int64_t r);
hipError_t launch_align_mfma(const uint16_t* x, void* out, int out_f32, const float* Q,
                             const float* M, const void* addend, int64_t T, int64_t D, int64_t r,
                             void* ws, hipStream_t s);

// The prepared basis of the matrix-core alignment (depends on Q and M only),
// bf16 hi/lo splits of: the projection operand (Q (M - I)^T)^T [RP][D], the
// lift operand Q [D][RK], and optionally the Hadamard image P = H Q / sqrt(D)
// [D][RK] for the fused prologue (D a power of two <= 4096).
struct AlignBasis {
  uint16_t* QtH; uint16_t* QtL; uint16_t* QH; uint16_t* QL;
  uint16_t* QtF;                // Q'h/Q'l again, in the projection's MFMA fragment order
  uint16_t* PH; uint16_t* PL;   // null without P
  int RP, RK;                   // r padded to 16 and to 32
};
size_t align_basis_bytes(int64_t D, int64_t r, bool with_p);
AlignBasis align_basis(const void* basis, int64_t D, int64_t r, bool with_p);
hipError_t launch_basis_prep(const float* Q, const float* M, int64_t D, int64_t r, bool with_p,
                             void* basis, hipStream_t s);
// per-call projection: Zpart[part][t][i] = ((M - I) Q_part^T x_part)[i] for
// the align_parts_count(D) D parts (z is their sum)
int align_parts_count(int64_t D);
size_t align_zpart_bytes(int64_t T, int64_t D, int64_t r);
hipError_t launch_yproj(const uint16_t* x, int64_t T, int64_t D, int64_t r, const void* basis,
                        bool with_p, float* Zpart, hipStream_t s);
// the whole alignment for short batches (align_small(T, D): 1 <= T <= 16
// tokens, D <= 16384), spread over D: projection into Zs (align_zpart_bytes(T, D, r)
// bytes) and lift, out = x + Q z (+ addend)
bool align_small(int64_t T, int64_t D);
hipError_t launch_align_small(const uint16_t* x, void* out, int out_f32, const void* addend,
                              int64_t T, int64_t D, int64_t r, const void* basis, bool with_p,
                              float* Zs, hipStream_t s);
// the quantizer of rows of a short batch (bf16 [T][4096], optional FWHT,
// packed or tiled codes) and, in the same launch, the short-batch projection
// of the same rows for the prepared basis pb into Zs
bool quant_project_fused(int64_t T, int64_t D);
hipError_t launch_quant_project(const uint16_t* x, int64_t ldx, int64_t T, int64_t D,
                                bool do_fwht, uint8_t* codes, bool tiled, float* scales,
                                float* dbg, int bits, const AlignBasis& pb, float* Zs,
                                hipStream_t s);
// the short-batch projection alone: Zs[c][t][i] for the align_small_chunks(D)
// 256-column chunks c (align_zpart_bytes(T, D, r) bytes)
int align_small_chunks(int64_t D);
hipError_t launch_align_small_project(const uint16_t* x, int64_t T, int64_t D, int64_t r,
                                      const void* basis, bool with_p, float* Zs, hipStream_t s);
// unfused lift out = x + Q z (+ addend), fp32 or bf16 out
hipError_t launch_lift(const uint16_t* x, void* out, int out_f32, const void* addend, int64_t T,
                       int64_t D, int64_t r, const void* basis, bool with_p, float* Zpart,
                       hipStream_t s);

// Fused lift + [Walsh-Hadamard] + INT4 quantization into FP6 tiles (or packed
// INT4 rows [T][D/2] when packed), after launch_yproj: per token,
// u = [H x / sqrt(D)] + P z (P = H Q / sqrt(D) with the transform, Q
// without), codes of u. Needs a basis prepared with P.
bool lfq_supported(int64_t D, int64_t r);
// pre, pre_bytes (optional): the weights of the product that follows; the
// kernel reads one word of each of their 128-byte lines, so that the product
// finds them in the caches (it streams from L2 while HBM is otherwise idle)
hipError_t launch_lift_fwht_quant(const uint16_t* x, int64_t T, int64_t D, int64_t r,
                                  const void* basis, const float* Zpart, bool do_fwht,
                                  uint8_t* tiles, float* s_a, float* dbg, hipStream_t s,
                                  int bits = 4, bool packed = false, const void* pre = nullptr,
                                  size_t pre_bytes = 0);

// W4A4 GEMM, bf16 (dequantized) or raw int32 output.
hipError_t launch_gemm(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                       void* y, bool i32_out, int64_t T, int64_t K, int64_t N, hipStream_t s);

// A residual alignment finished in a short-batch product's epilogue:
// out = bf16((x + Q z) + y) with y the product's bf16 output, bit for bit what
// the short-batch lift gives with y as its addend.
struct GemmResidual {
  const uint16_t* x;   // bf16 [T][N], the skip input
  const uint16_t* QH;  // the prepared basis' bf16 hi/lo rows of Q, [N][RK]
  const uint16_t* QL;
  const float* Zs;     // the short-batch projection of x, [C][T][RK]
  int RK, C;
  uint16_t* out;       // bf16 [T][N]
};
// packed INT4 rows, 1 <= T <= 16, bf16 output y plus the residual
hipError_t launch_gemm_residual(const uint8_t* a, const float* s_a, const uint8_t* w,
                                const float* s_w, uint16_t* y, const GemmResidual& res, int64_t T,
                                int64_t K, int64_t N, hipStream_t s);

// FP6 operand tiles (layout in common.hpp): rows padded to a multiple of 256.
int64_t tiles_rows(int64_t R);
size_t tiles_bytes(int64_t R, int64_t K);
hipError_t launch_tile_codes(const uint8_t* codes, int64_t R, int64_t K, uint8_t* tiles, int* bad,
                             hipStream_t s);
// W4A4 GEMM on FP6 tiles, bf16 (dequantized) or raw int32 output.
hipError_t launch_gemm_tiles(const uint8_t* a, const float* s_a, const uint8_t* w,
                             const float* s_w, void* y, bool i32_out, int64_t T, int64_t K,
                             int64_t N, hipStream_t s);

}  // namespace rw4
