// mxfp8_linear_noalloc: the MXFP8 dense linear layer for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It runs exactly mxfp8_linear's kernels,
// with the workspace taken from a static device array instead of the caller.
//
// The array is `scratch`, MXFP8_NOALLOC_SCRATCH_BYTES (16 MiB), 256-byte
// aligned; every GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory, so the kernels get the address hipGetSymbolAddress returns for the
// current device, fetched on the entry point's first call on that device and
// kept per device.  All calls on one GPU share its array: calls that overlap
// on one GPU (concurrent streams, or several host threads) race.  The
// workspace of mxfp8_linear needs no initialization (every byte a call reads
// was written earlier in the same call), so nothing is cleared between calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "launch.hpp"
#include "mxfp8.h"

namespace {

static_assert(MXFP8_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch is handed out in 256-byte units");
static __device__ __align__(256) uint8_t scratch[MXFP8_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` per device id (null until fetched).
std::atomic<void*> g_scratch[mxfp8::kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, or null if the runtime cannot say.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= mxfp8::kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int mxfp8_linear_noalloc(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                                    const void* s_packed, int64_t N, const void* bias_bf16, void* y_bf16,
                                    int64_t ldy, void* stream) {
  if (int st = mxfp8::linear_check_args(x_bf16, M, K, ldx, w_packed, s_packed, N, bias_bf16, y_bf16, ldy)) return st;
  if (M == 0) return MXFP8_OK;
  // Where the planned path's workspace (the slab kernel's fp32 partials)
  // exceeds the array, a path that fits runs instead.
  const size_t need = mxfp8::linear_workspace_within(M, N, K, MXFP8_NOALLOC_SCRATCH_BYTES);
  if (need > (size_t)MXFP8_NOALLOC_SCRATCH_BYTES) return MXFP8_E_SCRATCH;
  if (int st = mxfp8::check_device_current()) return st;
  void* ws = scratch_ptr();
  if (ws == nullptr) return MXFP8_E_DEVICE;
  return mxfp8::linear_launch(x_bf16, M, K, ldx, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, ws,
                              (hipStream_t)stream, MXFP8_NOALLOC_SCRATCH_BYTES);
}
