// rotated_linear_prepared without a caller workspace: the unit's scratch (the
// activation tiles, the per-token scales, the alignment's projection parts
// and, past the fused prologue, the aligned fp32 rows) lives in one
// file-scope device array of RW4_NOALLOC_SCRATCH_BYTES per GPU, so the call
// allocates nothing. For callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops).
//
// The array's name is a host-side stand-in in host code; its device address
// is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address reaches the kernels. Nothing in the scratch
// needs to start at zero: every byte the unit reads back was written earlier
// in the same call (tiles of token rows past T feed only output rows that are
// never stored).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/rotw4a4.h"

namespace {

static __device__ __align__(256) uint8_t scratch[RW4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_ptr[kMaxDevices] = {};
hipError_t g_err[kMaxDevices] = {};
std::once_flag g_once[kMaxDevices];

// device address of this device's copy of the scratch array (nullptr on error)
void* scratch_ptr(int dev) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_err[dev] = e;
    g_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  return g_ptr[dev];
}

}  // namespace

extern "C" rw4_status rotated_linear_prepared_noalloc(const void* x, int64_t ldx, int64_t T,
                                                      int64_t D, const void* basis, int64_t r,
                                                      unsigned flags, const uint8_t* w,
                                                      const float* s_w, int64_t N, void* y,
                                                      float* dbg_prequant, void* stream) {
  const size_t need = rotated_linear_prepared_workspace_size(T, D, r, flags);
  if (need == 0) {
    // invalid sizes or flags: the workspace form reports which, before any launch
    return rotated_linear_prepared(x, ldx, T, D, basis, r, flags, w, s_w, N, y, nullptr, 0,
                                   dbg_prequant, stream);
  }
  if (need > RW4_NOALLOC_SCRATCH_BYTES) return RW4_ERR_UNSUPPORTED;
  if (T == 0)
    return rotated_linear_prepared(x, ldx, T, D, basis, r, flags, w, s_w, N, y, nullptr, 0,
                                   dbg_prequant, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RW4_ERR_HIP;
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return RW4_ERR_HIP;
  return rotated_linear_prepared(x, ldx, T, D, basis, r, flags, w, s_w, N, y, ws,
                                 RW4_NOALLOC_SCRATCH_BYTES, dbg_prequant, stream);
}
