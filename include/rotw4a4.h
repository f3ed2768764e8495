/*
 * rotw4a4.h -- C ABI of the MI355X (gfx950) rotated W4A4 linear data path.
 *
 * The online path of a rotation-quantized transformer linear layer:
 *   low-rank residual alignment  x + Q ((M - I) (Q^T x))
 *   online Walsh-Hadamard transform
 *   per-token symmetric absmax INT4 activation quantization
 *   W4A4 GEMM (int32 accumulation) with per-token x per-channel scale epilogue.
 *
 * Sources (web pages):
 *   [RSQ] "ReSpinQuant: Efficient Layer-Wise LLM Quantization via Subspace
 *         Residual Rotation Approximation" (paper notes), framework flowchart
 *         and key designs 2-3 (T_hat = I + Q(R_sub - I)Q^T; three-step path).
 *   [QS]  "QuaRot 与 SpinQuant", §1.3 (normalized Hadamard) and §2.2 (fast
 *         Walsh-Hadamard transform, power-of-two sizes).
 *   [IQ2] "Infra Quant II", QuaRot "Background" (entries +-1/sqrt(d)) and
 *         "Method" (online Hadamard before the down projection; per-token
 *         absmax/7 activation quantization; INT4 GEMM to INT32, then row scale
 *         x column scale), SpinQuant "MOTIVATION" (symmetric step).
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer (HIP global memory on the current
 *     device) unless stated otherwise. The caller owns every buffer; the
 *     library never allocates or frees device memory. Its one device array
 *     of its own is the scratch of rotated_linear_prepared_noalloc (a static
 *     object of the library's code, one per GPU).
 *   - Matrices are row-major. Activations are [T][D] (token rows).
 *   - bf16 is IEEE-754 binary32's upper 16 bits; conversions to bf16 round to
 *     nearest, ties to even.
 *   - INT4 codes: two's-complement nibbles, two per byte, element 2j in the
 *     low nibble of byte j, rows K-contiguous ([rows][K/2] bytes).
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream). All
 *     work is enqueued on it; calls return after launch. Argument errors are
 *     detected on the host before anything is launched; launch failures
 *     return RW4_ERR_HIP; asynchronous device faults surface at the caller's
 *     next synchronization.
 *   - Pointers to bf16/fp32/int32 arrays, codes and scales must be 16-byte
 *     aligned (RW4_ERR_MISALIGNED otherwise), except M (4-byte).
 *   - T = 0 is a valid empty call: once the sizes, dtypes and flags are
 *     valid it returns RW4_OK without inspecting any pointer or launching.
 *   - The library holds no state between calls and is thread-safe; calls that
 *     write overlapping buffers must be ordered by the caller. (The scratch
 *     of rotated_linear_prepared_noalloc is the one exception: see there.)
 *   - Floating point is IEEE: no fast-math; fp32 division is correctly
 *     rounded; denormals are kept.
 */
#ifndef ROTW4A4_H
#define ROTW4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rw4_status {
  RW4_OK = 0,
  RW4_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad dtype or flag */
  RW4_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement */
  RW4_ERR_MISALIGNED = -3,  /* pointer not 16-byte aligned */
  RW4_ERR_WORKSPACE = -4,   /* workspace missing or too small */
  RW4_ERR_HIP = -5          /* the HIP runtime reported an error at launch */
} rw4_status;

typedef enum rw4_dtype { RW4_BF16 = 0, RW4_F32 = 1, RW4_I32 = 2 } rw4_dtype;

/* flags of rotated_linear; RW4_ABITS(b) selects b-bit activation codes
   (b = 2, 3 or 4; 0 in that field means 4). With RW4_FWHT, RW4_KRON(m)
   (m = 12, 20, 28) makes the transform H_{2^n} (x) H_m over D = 2^n m (see
   hadamard_transform). RW4_HEADS(k) selects the transform across heads,
   H_{n_h} (x) I with n_h = 2^k (see head_hadamard), instead of RW4_FWHT.
   RW4_WPACKED: the weights are packed INT4 rows instead of FP6 tiles. */
enum { RW4_ALIGN = 1, RW4_FWHT = 2, RW4_SWIGLU = 4, RW4_ABITS_SHIFT = 8, RW4_KRON_SHIFT = 16,
       RW4_HEADS_SHIFT = 24, RW4_WPACKED = 1 << 29 };
#define RW4_ABITS(b) ((unsigned)(b) << RW4_ABITS_SHIFT)
#define RW4_KRON(m) ((unsigned)(m) << RW4_KRON_SHIFT)
#define RW4_HEADS(k) ((unsigned)(k) << RW4_HEADS_SHIFT)

/*
 * respin_align -- online low-rank residual alignment [RSQ key design 3].
 *   out[t] = x[t] + Q ((M - I_r) (Q^T x[t]))  (+ addend[t])
 * which equals T_hat x[t] with T_hat = I + Q (M - I) Q^T in SO(D) [RSQ key
 * design 2]. M is the orthogonal r x r sub-rotation (R_sub); the page's small
 * matrix is M - I, which the kernel forms exactly while staging M.
 *   x      [T][D], dtype x_dt (RW4_BF16 or RW4_F32)
 *   out    [T][D], dtype out_dt (RW4_BF16 or RW4_F32); must not alias x
 *   Q      fp32 [D][r], orthonormal columns (not checked)
 *   M      fp32 [r][r]
 *   addend nullable, [T][D] of dtype out_dt, added after the alignment (the
 *          block output of a residual connection); one rounding to out_dt
 *   workspace, ws_bytes: device scratch of respin_align_workspace_size(T, D, r)
 *          bytes (256-byte aligned). With it, bf16 x and D % 64 == 0 run on
 *          bf16 matrix cores (Q and z split into two bf16 terms, fp32
 *          accumulation). NULL / 0 selects the direct fp32-FMA kernel (any
 *          supported shape, slower).
 * Constraints: 0 <= r <= min(D, 128), r % 4 == 0 (r = 0: out = x (+ addend));
 * D >= 1, D % 8 == 0. Arithmetic is fp32.
 */
rw4_status respin_align(const void* x, rw4_dtype x_dt, void* out, rw4_dtype out_dt,
                        const float* Q, const float* M, const void* addend,
                        int64_t T, int64_t D, int64_t r, void* workspace, size_t ws_bytes,
                        void* stream);

/* bytes of workspace respin_align needs for its matrix-core path */
size_t respin_align_workspace_size(int64_t T, int64_t D, int64_t r);

/*
 * fwht -- normalized Walsh-Hadamard transform of every row [QS §2.2; IQ2
 * QuaRot Background]: y[t] = H_D x[t], H_D = Sylvester (natural-order)
 * Hadamard / sqrt(D), entries (-1)^popcount(i&j) / sqrt(D). fp32 butterflies;
 * the scale is one multiply by fl32(1/sqrt(D)) after the last stage.
 *   x  [T][D], dtype x_dt (RW4_BF16 or RW4_F32)
 *   y  fp32 [T][D]; may alias x when x_dt == RW4_F32 (in place)
 * Constraints: D a power of two, 2 <= D <= 32768.
 */
rw4_status fwht(const void* x, rw4_dtype x_dt, float* y, int64_t T, int64_t D, void* stream);

/*
 * quant_act_int4 -- per-row symmetric absmax INT4 quantization [IQ2 QuaRot
 * Method; SpinQuant MOTIVATION]:
 *   scales[t] = fl32(max_i |x[t][i]| / 7)            (IEEE fp32 division)
 *   q         = clamp(rint(fl32(x[t][i] / scales[t])), -8, 7)   (half-even)
 *   all-zero row: scales[t] = 0, codes 0.
 * Rows of a weight matrix [N][K] use the same call (per-output-channel).
 *   x       [T][D], dtype x_dt (RW4_BF16 or RW4_F32)
 *   codes   uint8 [T][D/2] (packed INT4, see conventions)
 *   scales  fp32 [T]
 * Constraints: D even, 2 <= D <= 1048576.
 */
rw4_status quant_act_int4(const void* x, rw4_dtype x_dt, uint8_t* codes, float* scales,
                          int64_t T, int64_t D, void* stream);

/*
 * quant_act_sym -- quant_act_int4 for b-bit codes ["ReSpinQuant" paper notes,
 * 实验 (W3A3 and W4A4 settings); IQ2 FlatQuant Preliminaries (the signed
 * b-bit grid)]:
 *   scales[t] = fl32(max_i |x[t][i]| / (2^(b-1) - 1))
 *   q         = clamp(rint(fl32(x[t][i] / scales[t])), -2^(b-1), 2^(b-1) - 1)
 * Codes are stored as INT4 nibbles like quant_act_int4 (b = 4 is that call).
 *   bits  2, 3 or 4 (otherwise RW4_ERR_INVALID_ARG)
 */
rw4_status quant_act_sym(const void* x, rw4_dtype x_dt, uint8_t* codes, float* scales,
                         int64_t T, int64_t D, int bits, void* stream);

/*
 * w4a4_gemm -- INT4 x INT4 GEMM with int32 accumulation and dequantization
 * [IQ2 QuaRot Method]:
 *   acc[t][n] = sum_k a[t][k] * w[n][k]                  (exact int32)
 *   y[t][n]   = bf16( (fp32(acc) * s_a[t]) * s_w[n] )    (y_dt = RW4_BF16)
 *   y[t][n]   = acc[t][n]                                (y_dt = RW4_I32)
 *   a    uint8 [T][K/2]   packed activation codes;  s_a fp32 [T]
 *   w    uint8 [N][K/2]   packed weight codes;      s_w fp32 [N]
 *   y    [T][N], bf16 or int32 (s_a, s_w unused for RW4_I32 and may be NULL)
 * Constraints: K % 32 == 0, 32 <= K <= 131072; N >= 1.
 */
rw4_status w4a4_gemm(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                     void* y, rw4_dtype y_dt, int64_t T, int64_t K, int64_t N, void* stream);

/*
 * FP6 operand tiles -- the operand format of the matrix-core W4A4 GEMM.
 *
 * gfx950's f8f6f4 matrix instruction multiplies FP6 E2M3 numbers, and E2M3
 * represents every integer in [-7, 7] exactly (the range of a symmetric
 * absmax INT4 quantizer, step absmax / 7 [IQ2 QuaRot Method; SpinQuant
 * MOTIVATION]). A code q is stored as the E2M3 number q: sign bit 5,
 * exponent bits 4..3 (bias 1), mantissa bits 2..0; magnitudes 0..7 encode as
 * 0, 8, 16, 20, 24, 26, 28, 30. With fp32 accumulation every partial sum is an
 * integer below 2^24 (K <= 131072), so the result equals the INT32 sum.
 *
 * Layout of a tiled matrix [R][K] (K % 64 == 0): rows are padded to
 * Rp = ceil(R / 256) * 256 (padding rows hold code 0 when written by
 * w4a4_tile_codes; the GEMM never stores results of padding rows). Tiles of
 * 32 rows x 64 codes, 1536 bytes each; tile (rt, kt) starts at byte
 * (rt * (K / 64) + kt) * 1536. Within a tile, "lane" l (0..63) owns row
 * 32 rt + l % 32 and codes k = 64 kt + 32 (l / 32) + e for e = 0..31, as
 * six-bit fields, field e at bit 6 e of a 192-bit little-endian string whose
 * bytes 0..15 sit at 16 l and bytes 16..23 at 1024 + 8 l within the tile.
 */

/* bytes of the tiled form of an [R][K] code matrix; 0 on bad input.
 * Constraints: R >= 0; K % 64 == 0, 64 <= K <= 131072. */
size_t w4a4_tiles_size(int64_t R, int64_t K);

/*
 * w4a4_tile_codes -- packed INT4 rows (uint8 [R][K/2], conventions above) ->
 * FP6 tiles (w4a4_tiles_size(R, K) bytes, caller-allocated). Offline weight
 * preparation; also usable for activations. A code of -8 has no E2M3 value:
 * it is stored as 0 and, if `bad` (device int, nullable, 4-byte aligned) is
 * given, *bad is set to 1 (the caller clears it before and reads it after).
 * Constraints: as w4a4_tiles_size; R < 2^31 - 256.
 */
rw4_status w4a4_tile_codes(const uint8_t* codes, int64_t R, int64_t K, uint8_t* tiles, int* bad,
                           void* stream);

/*
 * w4a4_gemm_tiles -- the W4A4 GEMM on FP6 tiles [IQ2 QuaRot Method]:
 *   acc[t][n] = sum_k a[t][k] * w[n][k]          (exact)
 *   y[t][n]   = bf16( (fp32(acc) * s_a[t]) * s_w[n] )   or int32 acc
 *   a  tiles of [T][K] (w4a4_tiles_size(T, K) bytes);  s_a fp32 [T]
 *   w  tiles of [N][K] (w4a4_tiles_size(N, K) bytes);  s_w fp32 [N]
 *   y  [T][N] bf16 or int32 (s_a, s_w unused for RW4_I32 and may be NULL)
 * Results equal w4a4_gemm on the same codes bit for bit.
 * Constraints: K % 64 == 0, 64 <= K <= 131072; 1 <= N, T < 2^31 - 256.
 */
rw4_status w4a4_gemm_tiles(const uint8_t* a, const float* s_a, const uint8_t* w,
                           const float* s_w, void* y, rw4_dtype y_dt, int64_t T, int64_t K,
                           int64_t N, void* stream);

/*
 * rotated_linear -- the whole unit: [align] -> [SiLU gate] -> [FWHT] ->
 * per-token INT4 quantization -> W4A4 GEMM -> bf16.
 *   flags  RW4_ALIGN: align the D-wide input with (Q, M, r) first.
 *          RW4_SWIGLU: the input row is a gate|up pair of width 2D; the
 *            quantized vector is SiLU(gate) * up in fp32 (SiLU(g) = g/(1+e^-g)).
 *          RW4_FWHT: Hadamard transform of size D before quantization.
 *          RW4_ABITS(b): b-bit activation codes as quant_act_sym (W3A3 with
 *            3-bit weight codes; the GEMM takes any codes in [-7, 7]).
 *          RW4_KRON(m) with RW4_FWHT: the transform is H_{2^n} (x) H_m of
 *            hadamard_transform (D = 2^n m, m = 12, 20, 28, D <= 16384).
 *          RW4_HEADS(k): the transform across 2^k heads of head_hadamard
 *            instead (no FWHT, ALIGN or SWIGLU; D <= 16384).
 *          RW4_WPACKED: w holds the weight codes as packed INT4 rows
 *            (uint8 [N][D/2], the layout of w4a4_gemm) instead of FP6 tiles;
 *            the activation codes are then packed INT4 rows too and the
 *            product runs as w4a4_gemm (int8 matrix cores; for T <= 16 its
 *            weight-streaming kernel, the decode format). Results are the
 *            same codes, scales and outputs bit for bit as with FP6 tiles of
 *            the same weight codes.
 *          flags = 0: quantize x as is. ALIGN and SWIGLU are exclusive.
 *   x        bf16, T rows of D (or 2D with SWIGLU) values, row stride ldx
 *            elements (ldx >= width, ldx % 8 == 0)
 *   Q, M, r  as respin_align (ignored without RW4_ALIGN)
 *   w, s_w   weight codes as FP6 tiles of [N][D] (w4a4_tile_codes; no code
 *            -8) or, with RW4_WPACKED, as packed INT4 rows [N][D/2], and fp32
 *            scales [N]; the weights must already carry the inverse of every
 *            rotation applied here (e.g. rows Hadamard-transformed along K
 *            when RW4_FWHT is set)
 *   y        bf16 [T][N]
 *   workspace device memory of at least rotated_linear_workspace_size(T, D,
 *            r, flags) bytes, 256-byte aligned. After the call it holds the
 *            activation codes as FP6 tiles of [T][D] at offset 0
 *            (w4a4_tiles_size(T, D) bytes; with RW4_WPACKED packed INT4 rows
 *            [T][D/2] there) and the per-token scales fp32 [T] at offset
 *            rw4_align256(w4a4_tiles_size(T, D)); the rest is internal.
 *   dbg_prequant nullable fp32 [T][D]: if given, receives the fp32 values that
 *            were quantized (for stage-wise checking).
 * Constraints: D a power of two, 64 <= D <= 32768, or with RW4_KRON(m)
 * D = 2^n m, or with RW4_HEADS(k) any D; for both of these D % 64 == 0 and
 * D <= 16384. 1 <= N, T < 2^31 - 256.
 */
rw4_status rotated_linear(const void* x, int64_t ldx, int64_t T, int64_t D,
                          const float* Q, const float* M, int64_t r, unsigned flags,
                          const uint8_t* w, const float* s_w, int64_t N, void* y,
                          void* workspace, size_t ws_bytes, float* dbg_prequant,
                          void* stream);

/* bytes of workspace rotated_linear needs for (T, D, r, flags); 0 on bad input */
size_t rotated_linear_workspace_size(int64_t T, int64_t D, int64_t r, unsigned flags);

/*
 * hadamard_transform -- y = H~ x / sqrt(D) for every row, H~ = (H_{2^n} (x) H_m)
 * diag(s) ["Infra Quant II", QuaRot Background: H_d = H_{2^n} (x) H_m for
 * d = 2^n m, and the randomized H diag(s) with s in {+1, -1}^d]. H_{2^n} is
 * the Sylvester (natural-order) matrix. H_m (m = 12, 20, 28; the pages print
 * none) is Paley's construction: type I (q = m - 1) for 12 and 20, type II
 * (q = m/2 - 1) for 28, rows and columns ordered as the point at infinity,
 * then the integers 0..q-1 mod q. m = 1 is the plain transform. Element f of
 * a row is index (i, j) = (f / m, f % m) of the Kronecker product.
 *   x      [T][ldx] of x_dt (RW4_BF16 or RW4_F32), D values per row
 *   y      fp32 [T][D]; may be x itself (fp32, ldx == D)
 *   signs  nullable, fp32 [D] of +1 / -1 (values not checked)
 * Constraints: m in {1, 12, 20, 28}; D = 2^n m with n >= 0, D % 4 == 0,
 * D <= 16384; ldx >= D, ldx % 4 == 0. Arithmetic is fp32.
 */
rw4_status hadamard_transform(const void* x, rw4_dtype x_dt, int64_t ldx, float* y, int64_t T,
                              int64_t D, int64_t m, const float* signs, void* stream);

/*
 * head_hadamard -- y = (H_{n_h} (x) I_{d_h}) x / sqrt(n_h) for every row: the
 * online transform across attention heads before the output projection
 * ["Infra Quant II", QuaRot Method, value projection: Z <- Z (H_{n_h} (x) I)
 * by reshaping and a Walsh-Hadamard transform; H_{n_h} is symmetric, so this
 * is the same as the row form]. Element h d_h + c belongs to head h.
 *   x [T][ldx] of x_dt; y fp32 [T][n_h d_h] (may be x: fp32, ldx == D)
 * Constraints: n_h a power of two; D = n_h d_h, D % 4 == 0, D <= 16384;
 * ldx >= D, ldx % 4 == 0.
 */
rw4_status head_hadamard(const void* x, rw4_dtype x_dt, int64_t ldx, float* y, int64_t T,
                         int64_t n_h, int64_t d_h, void* stream);

/*
 * respin_construct -- the offline step upstream of the alignment: (Q, R_sub)
 * of a residual transition T = R_out R_in^T ["ReSpinQuant" paper notes, key
 * design 2]: Delta T = T - I; Q = its top-r left singular vectors; T_sub =
 * Q^T T Q; R_sub = U_sub V_sub^T, the orthogonal polar factor of T_sub. Then
 * T_hat = I + Q (R_sub - I) Q^T, and (Q, R_sub) are the (Q, M) of
 * respin_align / respin_prepare_basis.
 * The singular subspace comes from a randomized range finder with `iters`
 * steps of subspace iteration (oversampling 16, fixed pseudo-random start),
 * in fp64; its accuracy depends on the gap between the r-th and the
 * (r + 17)-th singular values of Delta T: each iteration shrinks the error by
 * about their squared ratio (4 steps are ample when the ratio is below 0.3).
 * Q is defined up to a rotation inside degenerate singular subspaces; T_hat
 * depends only on span(Q).
 *   T          fp32 [D][D], row-major (row i is the image coefficients of
 *              output i: y = T x)
 *   Q          fp32 [D][r] out; R_sub fp32 [r][r] out
 *   workspace  device memory of respin_construct_workspace_size(D, r) bytes,
 *              256-byte aligned
 * Constraints: D % 64 == 0, 64 <= D <= 16384; r % 4 == 0, 4 <= r <= min(64, D);
 * 0 <= iters <= 32. Asynchronous on `stream`; argument errors come before any launch.
 */
rw4_status respin_construct(const float* T, int64_t D, int64_t r, int iters, float* Q,
                            float* R_sub, void* workspace, size_t ws_bytes, void* stream);

/* bytes of workspace respin_construct needs; 0 when (D, r) is unsupported */
size_t respin_construct_workspace_size(int64_t D, int64_t r);

/*
 * respin_prepare_basis -- the part of the alignment that depends only on the
 * layer's (Q, M) ["ReSpinQuant" paper notes, key design 3: x + Q (M - I) Q^T x],
 * computed once and kept with the layer's weights, like the weight tiles:
 *   bf16 hi/lo splits of Q in both orientations, (M - I) transposed (fp32),
 *   and, when D is a power of two in [256, 4096] and r <= 64, the Hadamard
 *   image H_D Q / sqrt(D) split the same way ["QuaRot 与 SpinQuant" §2.2: H
 *   is orthogonal and symmetric, so H (x + Q z) = H x + (H Q) z].
 *   Q, M, D, r  as respin_align (1 <= r <= min(D, 128), r % 4 == 0, D % 64 == 0)
 *   basis       device memory of respin_basis_size(D, r) bytes, 256-byte
 *               aligned, owned by the caller; its layout is internal.
 * Asynchronous on `stream`; argument errors are reported before any launch.
 */
rw4_status respin_prepare_basis(const float* Q, const float* M, int64_t D, int64_t r,
                                void* basis, size_t basis_bytes, void* stream);

/* bytes of a prepared basis for (D, r); 0 when (D, r) is unsupported */
size_t respin_basis_size(int64_t D, int64_t r);

/*
 * respin_align_prepared -- respin_align on its matrix-core path with the basis
 * prepared by respin_prepare_basis(Q, M, D, r) instead of (Q, M): the per-call
 * work is the projection z = (M - I) Q^T x and the lift x + Q z ["ReSpinQuant"
 * paper notes, key design 3], with the same results bit for bit as respin_align
 * given a workspace.
 *   x      bf16 [T][D]
 *   out    [T][D] of out_dt (RW4_BF16 or RW4_F32); must not alias x
 *   basis  prepared for (D, r); 256-byte aligned
 *   addend nullable, [T][D] of out_dt, added after the alignment
 *   workspace, ws_bytes: respin_align_prepared_workspace_size(T, D, r) bytes
 *          of device scratch, 256-byte aligned
 * Constraints: those of respin_basis_size (1 <= r <= min(D, 128), r % 4 == 0,
 * D % 64 == 0). Asynchronous on `stream`; argument errors come before any launch.
 */
rw4_status respin_align_prepared(const void* x, void* out, rw4_dtype out_dt, const void* basis,
                                 const void* addend, int64_t T, int64_t D, int64_t r,
                                 void* workspace, size_t ws_bytes, void* stream);

/* bytes of workspace respin_align_prepared needs; 0 on bad input */
size_t respin_align_prepared_workspace_size(int64_t T, int64_t D, int64_t r);

/*
 * respin_align_project_prepared -- the first half of respin_align_prepared for
 * short batches: the projection z = (M - I) Q^T x ["ReSpinQuant" paper notes,
 * key design 3], left in `z` for rotated_linear_prepared_residual, which
 * finishes the alignment inside a product's epilogue.
 *   x      bf16 [T][D], 1 <= T <= 16, D <= 16384
 *   basis  prepared for (D, r) by respin_prepare_basis; 256-byte aligned
 *   z, z_bytes: respin_align_project_size(T, D, r) bytes of device memory,
 *          256-byte aligned; its layout is internal (per-chunk partial sums)
 * Constraints: those of respin_basis_size; larger T is RW4_ERR_UNSUPPORTED.
 * Asynchronous on `stream`; argument errors come before any launch.
 */
rw4_status respin_align_project_prepared(const void* x, int64_t T, int64_t D, const void* basis,
                                         int64_t r, void* z, size_t z_bytes, void* stream);

/* bytes of z respin_align_project_prepared writes; 0 when unsupported */
size_t respin_align_project_size(int64_t T, int64_t D, int64_t r);

/*
 * rotated_linear_prepared -- rotated_linear with the alignment's basis
 * prepared by respin_prepare_basis(Q, M, D, r) instead of (Q, M): same
 * arguments, same results bit for bit, same workspace contents after the
 * call (tiles at 0, scales at rw4_align256(w4a4_tiles_size(T, D))), but no
 * per-call basis preparation. basis may be NULL without RW4_ALIGN or r = 0.
 * Workspace: rotated_linear_prepared_workspace_size(T, D, r, flags) bytes.
 */
rw4_status rotated_linear_prepared(const void* x, int64_t ldx, int64_t T, int64_t D,
                                   const void* basis, int64_t r, unsigned flags,
                                   const uint8_t* w, const float* s_w, int64_t N, void* y,
                                   void* workspace, size_t ws_bytes, float* dbg_prequant,
                                   void* stream);

/*
 * rotated_linear_prepared_project -- rotated_linear_prepared for short
 * batches that also writes the alignment projection of its own input x for
 * another prepared basis (respin_align_project_prepared(x, T, D, proj_basis,
 * proj_r, proj_z, ...), the same bytes): in a decoder layer the skip input
 * of a residual point is also the input of the next quantized linear, so
 * the projection and the quantizer read the same rows, in one launch when
 * D = 4096 ["ReSpinQuant" paper notes, key design 3].
 *   x .. dbg_prequant  as rotated_linear_prepared; flags may not hold
 *          RW4_ALIGN, RW4_SWIGLU or the structured transforms; ldx == D;
 *          1 <= T <= 16
 *   proj_basis, proj_r: prepared for (D, proj_r) by respin_prepare_basis
 *   proj_z, proj_z_bytes: respin_align_project_size(T, D, proj_r) bytes,
 *          256-byte aligned
 * Asynchronous on `stream`; argument errors come before any launch.
 */
rw4_status rotated_linear_prepared_project(const void* x, int64_t ldx, int64_t T, int64_t D,
                                           const void* basis, int64_t r, unsigned flags,
                                           const uint8_t* w, const float* s_w, int64_t N, void* y,
                                           void* workspace, size_t ws_bytes, float* dbg_prequant,
                                           const void* proj_basis, int64_t proj_r, void* proj_z,
                                           size_t proj_z_bytes, void* stream);

/*
 * rotated_linear_prepared_residual -- rotated_linear_prepared for short
 * batches on packed INT4 weights whose product also finishes a residual
 * alignment of the layer: in a decoder layer the alignment sits on the skip
 * connection and the block's output joins after it ["ReSpinQuant" paper
 * notes, key design 2-3], so the product that makes the block output can add
 * it to the aligned skip input directly.
 *   x .. dbg_prequant  as rotated_linear_prepared; flags must hold
 *          RW4_WPACKED and 1 <= T <= 16; y receives the bf16 [T][N] output
 *   res_x  bf16 [T][N], the skip input (N is the alignment's width D)
 *   res_basis, res_r: the alignment's prepared basis (respin_prepare_basis)
 *   res_z, res_z_bytes: respin_align_project_prepared(res_x, T, N, res_basis,
 *          res_r, ...) written before this call on the same stream
 *   res_out bf16 [T][N], must alias none of x, y, res_x:
 *          res_out = bf16(res_x + Q z + y), the same bits as
 *          respin_align_prepared(res_x, res_out, RW4_BF16, res_basis, y, ...)
 * Asynchronous on `stream`; argument errors come before any launch.
 */
rw4_status rotated_linear_prepared_residual(const void* x, int64_t ldx, int64_t T, int64_t D,
                                            const void* basis, int64_t r, unsigned flags,
                                            const uint8_t* w, const float* s_w, int64_t N, void* y,
                                            void* workspace, size_t ws_bytes, float* dbg_prequant,
                                            const void* res_x, const void* res_basis,
                                            int64_t res_r, const void* res_z, size_t res_z_bytes,
                                            void* res_out, void* stream);

/* bytes of workspace rotated_linear_prepared needs; 0 on bad input */
size_t rotated_linear_prepared_workspace_size(int64_t T, int64_t D, int64_t r, unsigned flags);

/*
 * rotated_linear_prepared_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that forbid
 * allocation): rotated_linear_prepared with the same arguments minus the
 * workspace, and the same results bit for bit. Its scratch is a device array
 * of RW4_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * library's first use on that GPU until the process ends; the call allocates
 * and frees nothing.
 *   - Sizes whose workspace (rotated_linear_prepared_workspace_size) exceeds
 *     RW4_NOALLOC_SCRATCH_BYTES return RW4_ERR_UNSUPPORTED before any launch
 *     (e.g. T = 4096 tokens at D = 16384; the 70B-shaped linear does not fit).
 *   - Every call on a GPU uses that GPU's one array: calls that overlap on one
 *     GPU (other streams, other host threads) race and must be ordered by the
 *     caller. The array keeps the last call's contents; none of it needs to
 *     start at zero.
 *   - The activation tiles and scales stay in the library's array (there is
 *     no workspace to read them from).
 * Other arguments, constraints and errors: those of rotated_linear_prepared.
 */
#define RW4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rw4_status rotated_linear_prepared_noalloc(const void* x, int64_t ldx, int64_t T, int64_t D,
                                           const void* basis, int64_t r, unsigned flags,
                                           const uint8_t* w, const float* s_w, int64_t N, void* y,
                                           float* dbg_prequant, void* stream);

/* n rounded up to a multiple of 256 (workspace offsets) */
size_t rw4_align256(size_t n);

/* static, human-readable name of a status code */
const char* rw4_status_string(rw4_status s);

/* ABI version of this header (bumped on any signature change, and when the
 * layout of a prepared basis changes) */
int rw4_abi_version(void);

#define RW4_ABI_VERSION 13

#ifdef __cplusplus
}
#endif

#endif /* ROTW4A4_H */
