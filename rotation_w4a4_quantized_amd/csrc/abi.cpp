// C ABI of the rotated W4A4 path: host-side argument validation, then launch.
// Every check runs before any HIP call, so invalid arguments never touch the
// device (and can be tested without one).
#include <hip/hip_runtime.h>

#include "../../include/rotw4a4.h"
#include "launch.hpp"

namespace {

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline bool fdt(rw4_dtype d) { return d == RW4_BF16 || d == RW4_F32; }
inline rw4_status hip_status(hipError_t e) { return e == hipSuccess ? RW4_OK : RW4_ERR_HIP; }
inline hipStream_t strm(void* s) { return static_cast<hipStream_t>(s); }
inline bool tiles_k_ok(int64_t K) { return K >= 64 && K % 64 == 0 && K <= 131072; }

rw4_status check_align_args(const void* x, rw4_dtype x_dt, const void* out, rw4_dtype out_dt,
                            const float* Q, const float* M, int64_t T, int64_t D, int64_t r) {
  if (!x || !out || T < 0 || D < 1 || r < 0) return RW4_ERR_INVALID_ARG;
  if (!fdt(x_dt) || !fdt(out_dt)) return RW4_ERR_INVALID_ARG;
  if (r > 0 && (!Q || !M)) return RW4_ERR_INVALID_ARG;
  if (r > D || r > 128 || (r % 4) != 0 || (D % 8) != 0) return RW4_ERR_UNSUPPORTED;
  if (D > (int64_t(1) << 30)) return RW4_ERR_UNSUPPORTED;
  if (!al16(x) || !al16(out) || (r > 0 && !al16(Q))) return RW4_ERR_MISALIGNED;
  if (r > 0 && (reinterpret_cast<uintptr_t>(M) & 3u)) return RW4_ERR_MISALIGNED;
  return RW4_OK;
}

// activation code width from the flags (0 means the default 4)
inline int abits(unsigned flags) {
  const int b = static_cast<int>((flags >> RW4_ABITS_SHIFT) & 0xFu);
  return b == 0 ? 4 : b;
}
constexpr unsigned kFlagMask = RW4_ALIGN | RW4_FWHT | RW4_SWIGLU | (0xFu << RW4_ABITS_SHIFT) |
                               (0xFFu << RW4_KRON_SHIFT) | (0x1Fu << RW4_HEADS_SHIFT) |
                               static_cast<unsigned>(RW4_WPACKED);
inline int kron_m(unsigned flags) { return static_cast<int>((flags >> RW4_KRON_SHIFT) & 0xFFu); }
inline int heads_lg(unsigned flags) { return static_cast<int>((flags >> RW4_HEADS_SHIFT) & 0x1Fu); }

// D and the transform flags of the unit: a power-of-two D for the plain
// transform, or D = 2^n m / D = n_h d_h for the structured ones (kernel
// limits: D % 64 == 0 for the tiles, D <= kKronMaxD)
rw4_status check_transform(int64_t D, unsigned flags) {
  const int m = kron_m(flags), lg = heads_lg(flags);
  if (m && lg) return RW4_ERR_INVALID_ARG;
  if (m) {
    if (!(flags & RW4_FWHT)) return RW4_ERR_INVALID_ARG;
    if (!rw4::kron_order_supported(m)) return RW4_ERR_UNSUPPORTED;
    if (D % m != 0 || !pow2(D / m) || D % 64 != 0 || D > rw4::kKronMaxD) return RW4_ERR_UNSUPPORTED;
    return RW4_OK;
  }
  if (lg) {
    if (flags & (RW4_FWHT | RW4_ALIGN | RW4_SWIGLU)) return RW4_ERR_INVALID_ARG;
    if (lg > 14 || D % (int64_t(1) << lg) != 0 || D % 64 != 0 || D > rw4::kKronMaxD)
      return RW4_ERR_UNSUPPORTED;
    return RW4_OK;
  }
  if (!pow2(D) || D < 64 || D > 32768) return RW4_ERR_UNSUPPORTED;
  return RW4_OK;
}

// P (the Hadamard image of the basis) is prepared when the fused prologue can run
inline bool with_p(int64_t D, int64_t r) { return rw4::lfq_supported(D, r); }

// per-call part of the rotated_linear workspace: activation tiles, scales,
// and with alignment the projection's parts (plus fp32 aligned rows when the
// prologue is not fused)
size_t call_ws_bytes(int64_t T, int64_t D, int64_t r) {
  size_t n = rw4_align256(rw4::tiles_bytes(T, D)) + rw4_align256(4u * static_cast<size_t>(T));
  if (r > 0) {
    n += rw4::align_zpart_bytes(T, D, r);
    if (!rw4::lfq_supported(D, r))
      n += rw4_align256(4u * static_cast<size_t>(T) * static_cast<size_t>(D));
  }
  return n;
}

// checks shared by rotated_linear and rotated_linear_prepared (Q, M and the
// basis are checked by the callers)
rw4_status check_linear(const void* x, int64_t ldx, int64_t T, int64_t D, int64_t r,
                        unsigned flags, const uint8_t* w, const float* s_w, int64_t N, void* y,
                        const float* dbg) {
  if (T < 0 || N < 1) return RW4_ERR_INVALID_ARG;
  if (flags & ~kFlagMask) return RW4_ERR_INVALID_ARG;
  if ((flags & RW4_ALIGN) && (flags & RW4_SWIGLU)) return RW4_ERR_INVALID_ARG;
  if (abits(flags) < 2 || abits(flags) > 4) return RW4_ERR_INVALID_ARG;
  const rw4_status ts = check_transform(D, flags);
  if (ts != RW4_OK) return ts;
  if (T == 0) return RW4_OK;
  if (!x || !w || !s_w || !y) return RW4_ERR_INVALID_ARG;
  const int64_t width = (flags & RW4_SWIGLU) ? 2 * D : D;
  if (ldx < width || (ldx % 8) != 0) return RW4_ERR_INVALID_ARG;
  if (flags & RW4_ALIGN) {
    if (r < 0) return RW4_ERR_INVALID_ARG;
    if (r > D || r > 128 || (r % 4) != 0) return RW4_ERR_UNSUPPORTED;
    if (ldx != D) return RW4_ERR_UNSUPPORTED;
    if (r > 0 && !rw4::align_mfma_supported(D, r)) return RW4_ERR_UNSUPPORTED;
  }
  if (T > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return RW4_ERR_UNSUPPORTED;
  if (!al16(x) || !al16(w) || !al16(s_w) || !al16(y)) return RW4_ERR_MISALIGNED;
  if (dbg && !al16(dbg)) return RW4_ERR_MISALIGNED;
  return RW4_OK;
}

// the unit after validation; basis prepared for (D, r) when r > 0
// the short-batch projection of the unit's own input for another basis
struct SideProj {
  const void* basis;
  int64_t r;
  float* z;
};

rw4_status run_linear(const void* x, int64_t ldx, int64_t T, int64_t D, const void* basis,
                      int64_t r, unsigned flags, const uint8_t* w, const float* s_w, int64_t N,
                      void* y, void* workspace, float* dbg, hipStream_t s,
                      const rw4::GemmResidual* res = nullptr, const SideProj* sp = nullptr) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* codes = ws;
  // packed INT4 weights: the activation codes are packed rows [T][D/2] (they
  // fit the tile area) and the product runs on the packed-row GEMM
  const bool pk = (flags & RW4_WPACKED) != 0;
  float* s_a = reinterpret_cast<float*>(ws + rw4_align256(rw4::tiles_bytes(T, D)));
  auto gemm = [&]() {
    if (res)
      return rw4::launch_gemm_residual(codes, s_a, w, s_w, static_cast<uint16_t*>(y), *res, T, D,
                                       N, s);
    return pk ? rw4::launch_gemm(codes, s_a, w, s_w, y, false, T, D, N, s)
              : rw4::launch_gemm_tiles(codes, s_a, w, s_w, y, false, T, D, N, s);
  };
  const void* src = x;
  int in = (flags & RW4_SWIGLU) ? rw4::IN_SWIGLU : rw4::IN_BF16;
  int64_t ld = ldx;
  if (r > 0) {
    float* Zpart = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(s_a) +
                                            rw4_align256(4u * static_cast<size_t>(T)));
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const bool fused = rw4::lfq_supported(D, r);
    float* tmp = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(Zpart) +
                                          rw4::align_zpart_bytes(T, D, r));
    if (!fused && rw4::align_small(T, D)) {
      // a short batch past the fused prologue: the alignment spread over D
      if (rw4::launch_align_small(xb, tmp, 1, nullptr, T, D, r, basis, with_p(D, r), Zpart, s) !=
          hipSuccess)
        return RW4_ERR_HIP;
    } else if (rw4::launch_yproj(xb, T, D, r, basis, with_p(D, r), Zpart, s) != hipSuccess) {
      return RW4_ERR_HIP;
    }
    if (fused) {
      // lift + transform + quantization on chip
      // the product's weights are read ahead into the caches meanwhile
      // (prefill-linear step: GEMM 27.5 -> 25.0 us, prologue 16.5 -> 18.1 us)
      const size_t wbytes = pk ? static_cast<size_t>(N) * static_cast<size_t>(D / 2)
                               : rw4::tiles_bytes(N, D);
      if (rw4::launch_lift_fwht_quant(xb, T, D, r, basis, Zpart, (flags & RW4_FWHT) != 0, codes,
                                      s_a, dbg, s, abits(flags), pk, w, wbytes) != hipSuccess)
        return RW4_ERR_HIP;
      return hip_status(gemm());
    }
    if (!rw4::align_small(T, D) &&
        rw4::launch_lift(xb, tmp, 1, nullptr, T, D, r, basis, with_p(D, r), Zpart, s) != hipSuccess)
      return RW4_ERR_HIP;
    src = tmp;
    in = rw4::IN_F32;
    ld = D;
  }
  hipError_t e;
  if (kron_m(flags) || heads_lg(flags)) {
    const int m = kron_m(flags);
    const int64_t A = m ? D / m : (int64_t(1) << heads_lg(flags));
    const int64_t B = D / A;
    const double c = m ? static_cast<double>(D) : static_cast<double>(A);
    e = rw4::launch_kron(src, in, ld, T, A, B, m, nullptr,
                         static_cast<float>(1.0 / __builtin_sqrt(c)), nullptr, codes, !pk, s_a,
                         dbg, abits(flags), s);
  } else if (sp) {
    // the quantizer and the side projection read the same rows: one launch
    // when the shapes allow, else the projection and then the quantizer
    const rw4::AlignBasis pb = rw4::align_basis(sp->basis, D, sp->r, with_p(D, sp->r));
    const uint16_t* xb = static_cast<const uint16_t*>(src);
    if (in == rw4::IN_BF16 && rw4::quant_project_fused(T, D)) {
      e = rw4::launch_quant_project(xb, ld, T, D, (flags & RW4_FWHT) != 0, codes, !pk, s_a, dbg,
                                    abits(flags), pb, sp->z, s);
    } else {
      e = rw4::launch_align_small_project(xb, T, D, sp->r, sp->basis, with_p(D, sp->r), sp->z, s);
      if (e == hipSuccess)
        e = rw4::launch_row(src, in, ld, T, D, (flags & RW4_FWHT) != 0, nullptr, codes, !pk, s_a,
                            dbg, s, abits(flags));
    }
  } else {
    e = rw4::launch_row(src, in, ld, T, D, (flags & RW4_FWHT) != 0, nullptr, codes, !pk, s_a, dbg,
                        s, abits(flags));
  }
  if (e != hipSuccess) return RW4_ERR_HIP;
  return hip_status(gemm());
}

}  // namespace

extern "C" {

int rw4_abi_version(void) { return RW4_ABI_VERSION; }

size_t rw4_align256(size_t n) { return (n + 255u) & ~static_cast<size_t>(255u); }

const char* rw4_status_string(rw4_status s) {
  switch (s) {
    case RW4_OK: return "ok";
    case RW4_ERR_INVALID_ARG: return "invalid argument";
    case RW4_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case RW4_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case RW4_ERR_WORKSPACE: return "workspace missing or too small";
    case RW4_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

size_t respin_align_workspace_size(int64_t T, int64_t D, int64_t r) {
  if (T < 0 || D < 1 || r < 0 || r > 128) return 0;
  if (!rw4::align_mfma_supported(D, r)) return 0;
  return rw4::align_mfma_workspace(T, D, r);
}

rw4_status respin_align(const void* x, rw4_dtype x_dt, void* out, rw4_dtype out_dt,
                        const float* Q, const float* M, const void* addend, int64_t T, int64_t D,
                        int64_t r, void* workspace, size_t ws_bytes, void* stream) {
  if (T == 0 && D >= 1 && r >= 0 && fdt(x_dt) && fdt(out_dt)) return RW4_OK;
  rw4_status st = check_align_args(x, x_dt, out, out_dt, Q, M, T, D, r);
  if (st != RW4_OK) return st;
  if (addend && !al16(addend)) return RW4_ERR_MISALIGNED;
  if (x == out) return RW4_ERR_INVALID_ARG;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return RW4_ERR_WORKSPACE;
  const bool mfma = workspace && x_dt == RW4_BF16 && rw4::align_mfma_supported(D, r);
  if (mfma && ws_bytes < rw4::align_mfma_workspace(T, D, r)) return RW4_ERR_WORKSPACE;
  if (T == 0) return RW4_OK;
  if (mfma)
    return hip_status(rw4::launch_align_mfma(static_cast<const uint16_t*>(x), out,
                                             out_dt == RW4_F32, Q, M, addend, T, D, r, workspace,
                                             strm(stream)));
  return hip_status(rw4::launch_align(x, x_dt == RW4_F32, out, out_dt == RW4_F32, Q, M, addend, T,
                                      D, r, strm(stream)));
}

rw4_status fwht(const void* x, rw4_dtype x_dt, float* y, int64_t T, int64_t D, void* stream) {
  if (T < 0 || !fdt(x_dt)) return RW4_ERR_INVALID_ARG;
  if (!pow2(D) || D < 2 || D > 32768) return RW4_ERR_UNSUPPORTED;
  if (T == 0) return RW4_OK;
  if (!x || !y) return RW4_ERR_INVALID_ARG;
  if (!al16(x) || !al16(y)) return RW4_ERR_MISALIGNED;
  if (x == static_cast<const void*>(y) && x_dt != RW4_F32) return RW4_ERR_INVALID_ARG;
  return hip_status(rw4::launch_row(x, x_dt == RW4_F32 ? rw4::IN_F32 : rw4::IN_BF16, D, T, D, true,
                                    y, nullptr, false, nullptr, nullptr, strm(stream)));
}

rw4_status hadamard_transform(const void* x, rw4_dtype x_dt, int64_t ldx, float* y, int64_t T,
                              int64_t D, int64_t m, const float* signs, void* stream) {
  if (T < 0 || !fdt(x_dt)) return RW4_ERR_INVALID_ARG;
  if (m != 1 && !rw4::kron_order_supported(m)) return RW4_ERR_UNSUPPORTED;
  if (D < 4 || D % m != 0 || !pow2(D / m) || D % 4 != 0 || D > rw4::kKronMaxD)
    return RW4_ERR_UNSUPPORTED;
  if (T == 0) return RW4_OK;
  if (!x || !y || ldx < D || ldx % 4 != 0) return RW4_ERR_INVALID_ARG;
  if (!al16(x) || !al16(y) || (signs && !al16(signs))) return RW4_ERR_MISALIGNED;
  if (x == static_cast<const void*>(y) && (x_dt != RW4_F32 || ldx != D)) return RW4_ERR_INVALID_ARG;
  const int64_t A = D / m;
  return hip_status(rw4::launch_kron(x, x_dt == RW4_F32 ? rw4::IN_F32 : rw4::IN_BF16, ldx, T, A,
                                     m, m == 1 ? 0 : static_cast<int>(m), signs,
                                     static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(D))),
                                     y, nullptr, false, nullptr, nullptr, 4, strm(stream)));
}

rw4_status head_hadamard(const void* x, rw4_dtype x_dt, int64_t ldx, float* y, int64_t T,
                         int64_t n_h, int64_t d_h, void* stream) {
  if (T < 0 || !fdt(x_dt) || n_h < 1 || d_h < 1) return RW4_ERR_INVALID_ARG;
  if (!pow2(n_h) || n_h * d_h > rw4::kKronMaxD || (n_h * d_h) % 4 != 0) return RW4_ERR_UNSUPPORTED;
  const int64_t D = n_h * d_h;
  if (T == 0) return RW4_OK;
  if (!x || !y || ldx < D || ldx % 4 != 0) return RW4_ERR_INVALID_ARG;
  if (!al16(x) || !al16(y)) return RW4_ERR_MISALIGNED;
  if (x == static_cast<const void*>(y) && (x_dt != RW4_F32 || ldx != D)) return RW4_ERR_INVALID_ARG;
  return hip_status(rw4::launch_kron(x, x_dt == RW4_F32 ? rw4::IN_F32 : rw4::IN_BF16, ldx, T, n_h,
                                     d_h, 0, nullptr,
                                     static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(n_h))),
                                     y, nullptr, false, nullptr, nullptr, 4, strm(stream)));
}

rw4_status quant_act_sym(const void* x, rw4_dtype x_dt, uint8_t* codes, float* scales, int64_t T,
                         int64_t D, int bits, void* stream) {
  if (T < 0 || !fdt(x_dt) || bits < 2 || bits > 4) return RW4_ERR_INVALID_ARG;
  if (D < 2 || (D % 2) != 0 || D > (int64_t(1) << 20)) return RW4_ERR_UNSUPPORTED;
  if (T == 0) return RW4_OK;
  if (!x || !codes || !scales) return RW4_ERR_INVALID_ARG;
  if (!al16(x) || !al16(codes) || !al16(scales)) return RW4_ERR_MISALIGNED;
  const int in = x_dt == RW4_F32 ? rw4::IN_F32 : rw4::IN_BF16;
  if (pow2(D) && D <= 32768)
    return hip_status(rw4::launch_row(x, in, D, T, D, false, nullptr, codes, false, scales,
                                      nullptr, strm(stream), bits));
  return hip_status(rw4::launch_quant_generic(x, in, D, T, D, codes, scales, strm(stream), bits));
}

rw4_status quant_act_int4(const void* x, rw4_dtype x_dt, uint8_t* codes, float* scales, int64_t T,
                          int64_t D, void* stream) {
  return quant_act_sym(x, x_dt, codes, scales, T, D, 4, stream);
}

rw4_status w4a4_gemm(const uint8_t* a, const float* s_a, const uint8_t* w, const float* s_w,
                     void* y, rw4_dtype y_dt, int64_t T, int64_t K, int64_t N, void* stream) {
  if (T < 0 || N < 1) return RW4_ERR_INVALID_ARG;
  if (y_dt != RW4_BF16 && y_dt != RW4_I32) return RW4_ERR_INVALID_ARG;
  if (T == 0 && K >= 32 && K % 32 == 0 && K <= 131072) return RW4_OK;
  if (!a || !w || !y) return RW4_ERR_INVALID_ARG;
  if (y_dt == RW4_BF16 && (!s_a || !s_w)) return RW4_ERR_INVALID_ARG;
  if (K < 32 || (K % 32) != 0 || K > 131072) return RW4_ERR_UNSUPPORTED;
  if (T > (int64_t(1) << 31) - 1 || N > (int64_t(1) << 31) - 1) return RW4_ERR_UNSUPPORTED;
  if (!al16(a) || !al16(w) || !al16(y)) return RW4_ERR_MISALIGNED;
  if (y_dt == RW4_BF16 && (!al16(s_a) || !al16(s_w))) return RW4_ERR_MISALIGNED;
  if (T == 0) return RW4_OK;
  return hip_status(rw4::launch_gemm(a, s_a, w, s_w, y, y_dt == RW4_I32, T, K, N, strm(stream)));
}

size_t w4a4_tiles_size(int64_t R, int64_t K) {
  if (R < 0 || !tiles_k_ok(K)) return 0;
  return rw4::tiles_bytes(R, K);
}

rw4_status w4a4_tile_codes(const uint8_t* codes, int64_t R, int64_t K, uint8_t* tiles, int* bad,
                           void* stream) {
  if (R < 0) return RW4_ERR_INVALID_ARG;
  if (!tiles_k_ok(K)) return RW4_ERR_UNSUPPORTED;
  if (R > (int64_t(1) << 31) - 256) return RW4_ERR_UNSUPPORTED;
  if (R == 0) return RW4_OK;
  if (!codes || !tiles) return RW4_ERR_INVALID_ARG;
  if (!al16(codes) || !al16(tiles)) return RW4_ERR_MISALIGNED;
  if (bad && (reinterpret_cast<uintptr_t>(bad) & 3u)) return RW4_ERR_MISALIGNED;
  return hip_status(rw4::launch_tile_codes(codes, R, K, tiles, bad, strm(stream)));
}

rw4_status w4a4_gemm_tiles(const uint8_t* a, const float* s_a, const uint8_t* w,
                           const float* s_w, void* y, rw4_dtype y_dt, int64_t T, int64_t K,
                           int64_t N, void* stream) {
  if (T < 0 || N < 1) return RW4_ERR_INVALID_ARG;
  if (y_dt != RW4_BF16 && y_dt != RW4_I32) return RW4_ERR_INVALID_ARG;
  if (!tiles_k_ok(K)) return RW4_ERR_UNSUPPORTED;
  if (T > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return RW4_ERR_UNSUPPORTED;
  if (T == 0) return RW4_OK;
  if (!a || !w || !y) return RW4_ERR_INVALID_ARG;
  if (y_dt == RW4_BF16 && (!s_a || !s_w)) return RW4_ERR_INVALID_ARG;
  if (!al16(a) || !al16(w) || !al16(y)) return RW4_ERR_MISALIGNED;
  if (y_dt == RW4_BF16 && (!al16(s_a) || !al16(s_w))) return RW4_ERR_MISALIGNED;
  return hip_status(
      rw4::launch_gemm_tiles(a, s_a, w, s_w, y, y_dt == RW4_I32, T, K, N, strm(stream)));
}

size_t respin_construct_workspace_size(int64_t D, int64_t r) {
  if (!rw4::construct_supported(D, r)) return 0;
  return rw4::construct_workspace(D, r);
}

rw4_status respin_construct(const float* T, int64_t D, int64_t r, int iters, float* Q,
                            float* R_sub, void* workspace, size_t ws_bytes, void* stream) {
  if (!T || !Q || !R_sub || iters < 0 || iters > 32) return RW4_ERR_INVALID_ARG;
  if (!rw4::construct_supported(D, r)) return RW4_ERR_UNSUPPORTED;
  if (!al16(T) || !al16(Q) || !al16(R_sub)) return RW4_ERR_MISALIGNED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      ws_bytes < rw4::construct_workspace(D, r))
    return RW4_ERR_WORKSPACE;
  return hip_status(rw4::launch_construct(T, D, r, iters, Q, R_sub, workspace, strm(stream)));
}

size_t respin_basis_size(int64_t D, int64_t r) {
  if (D < 1 || r < 1 || r > 128 || (r % 4) != 0 || r > D) return 0;
  if (!rw4::align_mfma_supported(D, r)) return 0;
  return rw4::align_basis_bytes(D, r, with_p(D, r));
}

rw4_status respin_prepare_basis(const float* Q, const float* M, int64_t D, int64_t r, void* basis,
                                size_t basis_bytes, void* stream) {
  if (!Q || !M || D < 1 || r < 1) return RW4_ERR_INVALID_ARG;
  const size_t need = respin_basis_size(D, r);
  if (need == 0) return RW4_ERR_UNSUPPORTED;
  if (!al16(Q) || (reinterpret_cast<uintptr_t>(M) & 3u)) return RW4_ERR_MISALIGNED;
  if (!basis || (reinterpret_cast<uintptr_t>(basis) & 255u) || basis_bytes < need)
    return RW4_ERR_WORKSPACE;
  return hip_status(rw4::launch_basis_prep(Q, M, D, r, with_p(D, r), basis, strm(stream)));
}

size_t respin_align_prepared_workspace_size(int64_t T, int64_t D, int64_t r) {
  if (T < 0 || respin_basis_size(D, r) == 0) return 0;
  return rw4::align_zpart_bytes(T, D, r);
}

rw4_status respin_align_prepared(const void* x, void* out, rw4_dtype out_dt, const void* basis,
                                 const void* addend, int64_t T, int64_t D, int64_t r,
                                 void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || D < 1 || r < 1 || !fdt(out_dt)) return RW4_ERR_INVALID_ARG;
  if (respin_basis_size(D, r) == 0) return RW4_ERR_UNSUPPORTED;
  if (T == 0) return RW4_OK;
  if (!x || !out || !basis) return RW4_ERR_INVALID_ARG;
  if (!al16(x) || !al16(out) || (addend && !al16(addend))) return RW4_ERR_MISALIGNED;
  if (reinterpret_cast<uintptr_t>(basis) & 255u) return RW4_ERR_INVALID_ARG;
  if (x == out) return RW4_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      ws_bytes < rw4::align_zpart_bytes(T, D, r))
    return RW4_ERR_WORKSPACE;
  hipStream_t s = strm(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  float* Zpart = static_cast<float*>(workspace);
  if (rw4::align_small(T, D))
    return hip_status(rw4::launch_align_small(xb, out, out_dt == RW4_F32, addend, T, D, r, basis,
                                              with_p(D, r), Zpart, s));
  if (rw4::launch_yproj(xb, T, D, r, basis, with_p(D, r), Zpart, s) != hipSuccess)
    return RW4_ERR_HIP;
  return hip_status(rw4::launch_lift(xb, out, out_dt == RW4_F32, addend, T, D, r, basis,
                                     with_p(D, r), Zpart, s));
}

size_t respin_align_project_size(int64_t T, int64_t D, int64_t r) {
  if (T < 1 || D < 1 || r < 1 || !rw4::align_small(T, D) || respin_basis_size(D, r) == 0) return 0;
  return rw4::align_zpart_bytes(T, D, r);
}

rw4_status respin_align_project_prepared(const void* x, int64_t T, int64_t D, const void* basis,
                                         int64_t r, void* z, size_t z_bytes, void* stream) {
  if (T < 0 || D < 1 || r < 1) return RW4_ERR_INVALID_ARG;
  if (respin_basis_size(D, r) == 0) return RW4_ERR_UNSUPPORTED;
  if (T == 0) return RW4_OK;
  if (!rw4::align_small(T, D)) return RW4_ERR_UNSUPPORTED;
  if (!x || !basis) return RW4_ERR_INVALID_ARG;
  if (!al16(x)) return RW4_ERR_MISALIGNED;
  if (reinterpret_cast<uintptr_t>(basis) & 255u) return RW4_ERR_INVALID_ARG;
  if (!z || (reinterpret_cast<uintptr_t>(z) & 255u) || z_bytes < respin_align_project_size(T, D, r))
    return RW4_ERR_WORKSPACE;
  return hip_status(rw4::launch_align_small_project(static_cast<const uint16_t*>(x), T, D, r,
                                                    basis, with_p(D, r), static_cast<float*>(z),
                                                    strm(stream)));
}

rw4_status rotated_linear_prepared_project(const void* x, int64_t ldx, int64_t T, int64_t D,
                                           const void* basis, int64_t r, unsigned flags,
                                           const uint8_t* w, const float* s_w, int64_t N, void* y,
                                           void* workspace, size_t ws_bytes, float* dbg_prequant,
                                           const void* proj_basis, int64_t proj_r, void* proj_z,
                                           size_t proj_z_bytes, void* stream) {
  rw4_status st = check_linear(x, ldx, T, D, r, flags, w, s_w, N, y, dbg_prequant);
  if (st != RW4_OK || T == 0) return st;
  // the unit's input is the projected x itself: no alignment or gate in the
  // unit, a plain power-of-two transform at most, contiguous rows
  if ((flags & (RW4_ALIGN | RW4_SWIGLU)) || kron_m(flags) || heads_lg(flags) || ldx != D)
    return RW4_ERR_UNSUPPORTED;
  if (proj_r < 1) return RW4_ERR_INVALID_ARG;
  const size_t zb = respin_align_project_size(T, D, proj_r);
  if (zb == 0) return RW4_ERR_UNSUPPORTED;
  if (!proj_basis || (reinterpret_cast<uintptr_t>(proj_basis) & 255u)) return RW4_ERR_INVALID_ARG;
  if (!proj_z || (reinterpret_cast<uintptr_t>(proj_z) & 255u) || proj_z_bytes < zb)
    return RW4_ERR_WORKSPACE;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return RW4_ERR_WORKSPACE;
  if (ws_bytes < call_ws_bytes(T, D, 0)) return RW4_ERR_WORKSPACE;
  const SideProj sp{proj_basis, proj_r, static_cast<float*>(proj_z)};
  return run_linear(x, ldx, T, D, basis, 0, flags, w, s_w, N, y, workspace, dbg_prequant,
                    strm(stream), nullptr, &sp);
}

rw4_status rotated_linear_prepared_residual(const void* x, int64_t ldx, int64_t T, int64_t D,
                                            const void* basis, int64_t r, unsigned flags,
                                            const uint8_t* w, const float* s_w, int64_t N, void* y,
                                            void* workspace, size_t ws_bytes, float* dbg_prequant,
                                            const void* res_x, const void* res_basis,
                                            int64_t res_r, const void* res_z, size_t res_z_bytes,
                                            void* res_out, void* stream) {
  rw4_status st = check_linear(x, ldx, T, D, r, flags, w, s_w, N, y, dbg_prequant);
  if (st != RW4_OK || T == 0) return st;
  if (!(flags & RW4_WPACKED) || T > 16) return RW4_ERR_UNSUPPORTED;
  if (res_r < 1) return RW4_ERR_INVALID_ARG;
  if (respin_align_project_size(T, N, res_r) == 0) return RW4_ERR_UNSUPPORTED;
  if (!res_x || !res_basis || !res_out) return RW4_ERR_INVALID_ARG;
  if (!al16(res_x) || !al16(res_out)) return RW4_ERR_MISALIGNED;
  if (reinterpret_cast<uintptr_t>(res_basis) & 255u) return RW4_ERR_INVALID_ARG;
  if (res_out == res_x || res_out == y || res_out == x) return RW4_ERR_INVALID_ARG;
  if (!res_z || (reinterpret_cast<uintptr_t>(res_z) & 255u) ||
      res_z_bytes < respin_align_project_size(T, N, res_r))
    return RW4_ERR_WORKSPACE;
  const int64_t re = (flags & RW4_ALIGN) ? r : 0;
  if (re > 0 && (!basis || (reinterpret_cast<uintptr_t>(basis) & 255u))) return RW4_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return RW4_ERR_WORKSPACE;
  if (ws_bytes < call_ws_bytes(T, D, re)) return RW4_ERR_WORKSPACE;
  const rw4::AlignBasis a = rw4::align_basis(res_basis, N, res_r, with_p(N, res_r));
  const rw4::GemmResidual res{static_cast<const uint16_t*>(res_x), a.QH, a.QL,
                              static_cast<const float*>(res_z), a.RK, rw4::align_small_chunks(N),
                              static_cast<uint16_t*>(res_out)};
  return run_linear(x, ldx, T, D, basis, re, flags, w, s_w, N, y, workspace, dbg_prequant,
                    strm(stream), &res);
}

size_t rotated_linear_prepared_workspace_size(int64_t T, int64_t D, int64_t r, unsigned flags) {
  if (T < 0 || r < 0 || (flags & ~kFlagMask) || check_transform(D, flags) != RW4_OK) return 0;
  if ((flags & RW4_ALIGN) && r > 0 && respin_basis_size(D, r) == 0) return 0;
  return call_ws_bytes(T, D, (flags & RW4_ALIGN) ? r : 0);
}

rw4_status rotated_linear_prepared(const void* x, int64_t ldx, int64_t T, int64_t D,
                                   const void* basis, int64_t r, unsigned flags, const uint8_t* w,
                                   const float* s_w, int64_t N, void* y, void* workspace,
                                   size_t ws_bytes, float* dbg_prequant, void* stream) {
  rw4_status st = check_linear(x, ldx, T, D, r, flags, w, s_w, N, y, dbg_prequant);
  if (st != RW4_OK || T == 0) return st;
  const int64_t re = (flags & RW4_ALIGN) ? r : 0;
  if (re > 0 && (!basis || (reinterpret_cast<uintptr_t>(basis) & 255u))) return RW4_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return RW4_ERR_WORKSPACE;
  if (ws_bytes < call_ws_bytes(T, D, re)) return RW4_ERR_WORKSPACE;
  return run_linear(x, ldx, T, D, basis, re, flags, w, s_w, N, y, workspace, dbg_prequant,
                    strm(stream));
}

size_t rotated_linear_workspace_size(int64_t T, int64_t D, int64_t r, unsigned flags) {
  const size_t n = rotated_linear_prepared_workspace_size(T, D, r, flags);
  if (n == 0 || !(flags & RW4_ALIGN) || r == 0) return n;
  return n + rw4_align256(respin_basis_size(D, r));
}

rw4_status rotated_linear(const void* x, int64_t ldx, int64_t T, int64_t D, const float* Q,
                          const float* M, int64_t r, unsigned flags, const uint8_t* w,
                          const float* s_w, int64_t N, void* y, void* workspace, size_t ws_bytes,
                          float* dbg_prequant, void* stream) {
  rw4_status st = check_linear(x, ldx, T, D, r, flags, w, s_w, N, y, dbg_prequant);
  if (st != RW4_OK || T == 0) return st;
  const int64_t re = (flags & RW4_ALIGN) ? r : 0;
  if (flags & RW4_ALIGN) {
    st = check_align_args(x, RW4_BF16, x, RW4_F32, Q, M, T, D, r);
    if (st != RW4_OK) return st;
  }
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return RW4_ERR_WORKSPACE;
  if (ws_bytes < rotated_linear_workspace_size(T, D, re, flags)) return RW4_ERR_WORKSPACE;
  hipStream_t s = strm(stream);
  void* basis = nullptr;
  if (re > 0) {
    // the basis goes after the per-call part of the workspace
    basis = static_cast<uint8_t*>(workspace) + call_ws_bytes(T, D, re);
    if (rw4::launch_basis_prep(Q, M, D, re, with_p(D, re), basis, s) != hipSuccess)
      return RW4_ERR_HIP;
  }
  return run_linear(x, ldx, T, D, basis, re, flags, w, s_w, N, y, workspace, dbg_prequant, s);
}

}  // extern "C"
