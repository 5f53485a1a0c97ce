// C ABI of libmxfp8 (declared in include/mxfp8.h): argument validation on the
// host, device check, path choice by shape, and kernel launches.  Nothing
// here allocates device memory or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "mxfp8.h"

namespace {

constexpr int kMaxDevices = 64;
// Per-device cached answer to "is this a gfx950": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_dev_ok[kMaxDevices];
std::atomic<int> g_force_path{0};

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXFP8_E_DEVICE;
  int s = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXFP8_E_DEVICE;
    s = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? MXFP8_OK : MXFP8_E_DEVICE;
}

int64_t n_pad(int64_t N) { return (N + 127) / 128 * 128; }

int check_packed(const void* wp, const void* sp, int64_t N, int64_t K) {
  if (!wp || !sp) return MXFP8_E_NULLPTR;
  if (N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  if (N > (int64_t)1 << 30 || K > (int64_t)1 << 30) return MXFP8_E_SHAPE;
  if (!aligned(wp, 256) || !aligned(sp, 256)) return MXFP8_E_ALIGN;
  return MXFP8_OK;
}

int check_output(const void* y, int64_t N, int64_t ldy, const void* bias) {
  if (!y) return MXFP8_E_NULLPTR;
  if (ldy < N) return MXFP8_E_LD;
  if (!aligned(y, 2) || (bias && !aligned(bias, 2))) return MXFP8_E_ALIGN;
  return MXFP8_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of the tile path: packed activations (M padded to 128 rows) then
// their packed scales, each 256-byte aligned.
size_t tile_ws_bytes(int64_t M, int64_t K) {
  const size_t mp = (size_t)((M + 127) / 128 * 128);
  return round_up(mp * (size_t)K, 256) + round_up(mp * (size_t)(K / 32), 256);
}

bool use_skinny(int64_t M, int64_t K) {
  if (g_force_path.load(std::memory_order_relaxed) == 1) return false;
  return M <= mxfp8::kSkinnyMaxM && K <= mxfp8::kSkinnyMaxK;
}

}  // namespace

extern "C" {

const char* mxfp8_status_string(int status) {
  switch (status) {
    case MXFP8_OK: return "ok";
    case MXFP8_E_NULLPTR: return "a required pointer is NULL";
    case MXFP8_E_SHAPE: return "invalid shape (sizes must be non-negative, K % 32 == 0 for quantize, K % 256 == 0 and N >= 1 for the GEMM)";
    case MXFP8_E_ALIGN: return "pointer misaligned (see mxfp8.h for each argument's alignment)";
    case MXFP8_E_LD: return "leading dimension too small or not a required multiple";
    case MXFP8_E_WORKSPACE: return "workspace missing or smaller than mxfp8_linear_workspace_bytes";
    case MXFP8_E_DEVICE: return "current HIP device is not a gfx950 (MI355X) or is unavailable";
    case MXFP8_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int mxfp8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* q_e4m3, int64_t ldq,
                       void* s_e8m0, int64_t lds, void* stream) {
  if (M < 0 || K < 0 || K % 32 != 0) return MXFP8_E_SHAPE;
  if (M == 0 || K == 0) return MXFP8_OK;
  if (!x_bf16 || !q_e4m3 || !s_e8m0) return MXFP8_E_NULLPTR;
  if (ldx < K || ldx % 8 != 0 || ldq < K || ldq % 8 != 0 || lds < K / 32) return MXFP8_E_LD;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16)) return MXFP8_E_ALIGN;
  if ((M * (K / 8) + 255) / 256 > INT32_MAX) return MXFP8_E_SHAPE;
  if (int st = check_device()) return st;
  return mxfp8::launch_quantize_act(x_bf16, M, K, ldx, q_e4m3, ldq, s_e8m0, lds, (hipStream_t)stream);
}

int mxfp8_prepared_weight_bytes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes) {
  if (!w_bytes || !s_bytes) return MXFP8_E_NULLPTR;
  if (N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  *w_bytes = (size_t)n_pad(N) * (size_t)K;
  *s_bytes = (size_t)n_pad(N) * (size_t)(K / 32);
  return MXFP8_OK;
}

int mxfp8_prepare_weight(const void* w_e4m3, const void* w_s_e8m0, int64_t N, int64_t K, int64_t ldw,
                         int64_t ldws, void* w_packed, void* s_packed, void* stream) {
  if (int st = check_packed(w_packed, s_packed, N, K)) return st;
  if (!w_e4m3 || !w_s_e8m0) return MXFP8_E_NULLPTR;
  if (ldw < K || ldw % 16 != 0 || ldws < K / 32) return MXFP8_E_LD;
  if (!aligned(w_e4m3, 16)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  return mxfp8::launch_pack_weight(w_e4m3, w_s_e8m0, N, K, ldw, ldws, w_packed, s_packed, (hipStream_t)stream);
}

int mxfp8_unpack_weight(const void* w_packed, const void* s_packed, int64_t N, int64_t K, void* w_e4m3,
                        void* w_s_e8m0, void* stream) {
  if (int st = check_packed(w_packed, s_packed, N, K)) return st;
  if (!w_e4m3 || !w_s_e8m0) return MXFP8_E_NULLPTR;
  if (!aligned(w_e4m3, 16)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  return mxfp8::launch_unpack_weight(w_packed, s_packed, N, K, w_e4m3, w_s_e8m0, (hipStream_t)stream);
}

int mxfp8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return MXFP8_E_NULLPTR;
  if (M < 0 || N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  *bytes = (M == 0 || use_skinny(M, K)) ? 256 : tile_ws_bytes(M, K);
  return MXFP8_OK;
}

int mxfp8_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                 const void* s_packed, int64_t N, const void* bias_bf16, void* y_bf16, int64_t ldy,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0) return MXFP8_E_SHAPE;
  if (int st = check_packed(w_packed, s_packed, N, K)) return st;
  if (M == 0) return MXFP8_OK;
  if (M > (int64_t)1 << 30) return MXFP8_E_SHAPE;
  if (!x_bf16) return MXFP8_E_NULLPTR;
  if (int st = check_output(y_bf16, N, ldy, bias_bf16)) return st;
  if (ldx < K || ldx % 8 != 0) return MXFP8_E_LD;
  if (!aligned(x_bf16, 16)) return MXFP8_E_ALIGN;
  const bool skinny = use_skinny(M, K);
  if (!skinny && (n_pad(M) * (K / 8) + 255) / 256 > INT32_MAX) return MXFP8_E_SHAPE;
  const size_t need = skinny ? 256 : tile_ws_bytes(M, K);
  if (!workspace || workspace_bytes < need) return MXFP8_E_WORKSPACE;
  if (!aligned(workspace, 256)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (skinny)
    return mxfp8::launch_gemm_skinny(x_bf16, ldx, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s);
  uint8_t* q = (uint8_t*)workspace;
  uint8_t* sc = q + round_up((size_t)n_pad(M) * (size_t)K, 256);
  if (int st = mxfp8::launch_quantize_act_packed(x_bf16, M, K, ldx, q, sc, s)) return st;
  return mxfp8::launch_gemm_tile(q, sc, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s);
}

int mxfp8_packed_act_bytes(int64_t M, int64_t K, size_t* q_bytes, size_t* s_bytes) {
  if (!q_bytes || !s_bytes) return MXFP8_E_NULLPTR;
  if (M < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  *q_bytes = (size_t)n_pad(M) * (size_t)K;
  *s_bytes = (size_t)n_pad(M) * (size_t)(K / 32);
  return MXFP8_OK;
}

int mxfp8_quantize_act_packed(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* q_packed,
                              void* s_packed, void* stream) {
  if (M < 0 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  if (M == 0) return MXFP8_OK;
  if (M > (int64_t)1 << 30 || K > (int64_t)1 << 30) return MXFP8_E_SHAPE;
  if (!x_bf16 || !q_packed || !s_packed) return MXFP8_E_NULLPTR;
  if (ldx < K || ldx % 8 != 0) return MXFP8_E_LD;
  if (!aligned(x_bf16, 16) || !aligned(q_packed, 256) || !aligned(s_packed, 256)) return MXFP8_E_ALIGN;
  if ((n_pad(M) * (K / 8) + 255) / 256 > INT32_MAX) return MXFP8_E_SHAPE;
  if (int st = check_device()) return st;
  return mxfp8::launch_quantize_act_packed(x_bf16, M, K, ldx, q_packed, s_packed, (hipStream_t)stream);
}

int mxfp8_gemm_packed(const void* q_packed, const void* s_packed, int64_t M, int64_t K, const void* w_packed,
                      const void* ws_packed, int64_t N, const void* bias_bf16, void* y_bf16, int64_t ldy,
                      void* stream) {
  if (M < 0) return MXFP8_E_SHAPE;
  if (int st = check_packed(w_packed, ws_packed, N, K)) return st;
  if (M == 0) return MXFP8_OK;
  if (M > (int64_t)1 << 30) return MXFP8_E_SHAPE;
  if (!q_packed || !s_packed) return MXFP8_E_NULLPTR;
  if (int st = check_output(y_bf16, N, ldy, bias_bf16)) return st;
  if (!aligned(q_packed, 256) || !aligned(s_packed, 256)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  return mxfp8::launch_gemm_tile(q_packed, s_packed, M, K, w_packed, ws_packed, N, bias_bf16, y_bf16, ldy,
                                 (hipStream_t)stream);
}

int mxfp8_debug_force_path(int path) {
  if (path < 0 || path > 2) return MXFP8_E_SHAPE;
  return g_force_path.exchange(path);
}

}  // extern "C"
