// C ABI of libmxfp8 (declared in include/mxfp8.h): argument validation on the
// host, device check, path choice by shape, and kernel launches.  Nothing
// here allocates device memory or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "shape_table.inc"
#include "mxfp8.h"

namespace {

using mxfp8::kMaxDevices;
// Per-device cached answer to "is this a gfx950": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_dev_ok[kMaxDevices];
// Per-device compute-unit count (0 = not yet queried).
std::atomic<int> g_dev_cus[kMaxDevices];
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
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? MXFP8_OK : MXFP8_E_DEVICE;
}

int64_t n_pad(int64_t N) { return (N + 127) / 128 * 128; }

int check_packed(const void* wp, const void* sp, int64_t N, int64_t K) {
  if (!wp || !sp) return MXFP8_E_NULLPTR;
  if (N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  // A packed 128-row group (128 K bytes) must stay below 2^32 bytes: the GEMM
  // addresses it with 32-bit buffer offsets.
  if (N > (int64_t)1 << 30 || K > (int64_t)1 << 24) return MXFP8_E_SHAPE;
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

// Workspace of the tile path: packed activations (M padded to 128 rows), their
// packed scales, then (split-K shapes) the fp32 partial outputs, each
// 256-byte aligned.
size_t tile_ws_act_bytes(int64_t M, int64_t K) {
  const size_t mp = (size_t)((M + 127) / 128 * 128);
  return round_up(mp * (size_t)K, 256) + round_up(mp * (size_t)(K / 32), 256);
}
size_t tile_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const int splits = mxfp8::gemm_tile_splits(M, N, K);
  const size_t part = splits > 1 ? (size_t)splits * (size_t)M * (size_t)((N + 3) / 4 * 4) * 4 : 0;
  return tile_ws_act_bytes(M, K) + round_up(part, 256);
}

// Test hook state of mxfp8_moe_debug_capture.
std::atomic<void*> g_dbg_act{nullptr}, g_dbg_q{nullptr}, g_dbg_s{nullptr}, g_dbg_ids{nullptr}, g_dbg_wts{nullptr};

int check_moe_shape(int64_t T, int64_t H, int64_t E, int64_t topk, int64_t I) {
  if (T < 0 || H < 256 || H % 256 != 0 || I < 256 || I % 256 != 0) return MXFP8_E_SHAPE;
  if (E < 1 || E > mxfp8::kMoeMaxExperts || topk < 1 || topk > E || topk > mxfp8::kMoeMaxTopk) return MXFP8_E_SHAPE;
  if (H > (1 << 20) || I > (1 << 20) || T > (1 << 24) || T * topk > (1 << 26)) return MXFP8_E_SHAPE;
  if ((T + 1) * H > (int64_t(1) << 32) - 1) return MXFP8_E_SHAPE;   // token rows addressed with 32-bit offsets
  return MXFP8_OK;
}

// Carves the MoE scratch out of a workspace (base may be NULL to size it).
size_t moe_layout(int64_t T, int64_t H, int64_t E, int64_t topk, int64_t I, uint8_t* base, mxfp8::MoeWorkspace* w) {
  const int64_t R = T * topk;
  const int64_t nblk = (T + 15) / 16;
  const int64_t groups_max = (R + (mxfp8::kGroupRowsHost - 1) * E) / mxfp8::kGroupRowsHost;
  const int64_t p_max = (groups_max + 1) * mxfp8::kGroupRowsHost;
  const int64_t mt_max = (groups_max + E) / 2 + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += round_up(bytes > 0 ? bytes : 1, 256);
    return p;
  };
  mxfp8::MoeWorkspace v;
  v.ids = (int*)take(R * 4);
  v.wts = (float*)take(R * 4);
  v.blk_cnt = (int*)take(E * nblk * 4);
  v.blk_off = (int*)take(E * nblk * 4);
  v.seg_off = (int*)take(E * 4);
  v.meta = (int*)take(64);
  v.tile_e = (int*)take(mt_max * 4);
  v.tile_g0 = (int*)take(mt_max * 4);
  v.tile_ng = (int*)take(mt_max * 4);
  v.sorted_row = (int*)take(p_max * 4);
  v.xq = take((T + 1) * H);
  v.xs = take((T + 1) * (H / 32));
  v.a1s = take(p_max * (H / 32));
  v.a2q = take(p_max * I);
  v.a2s = take(p_max * (I / 32));
  v.ys = (float*)take((R + 1) * H * 4);     // row R: spare row for pad rows
  v.p_max = p_max;
  v.mt_max = mt_max;
  if (w) *w = v;
  return off;
}

// GEMM path of a linear call and the K splits of the tile GEMM, from the
// measured shape table (shape_table.inc): the decode kernel (M <= 16,
// K <= 8192), the mid-M kernel (M <= 128, K <= 8192), the split-K slab
// kernel (M <= 128, any K), the medium-tile GEMM (128 x 128 or 128 x 64
// tiles over the whole K) or the large-tile GEMM
// with 1 (persistent), 2, 4 or 8 K splits (a split count s needs (K / 64) %
// (4 s) == 0: each slice a whole number of 128-K step pairs).  A table entry a
// shape cannot take falls back to the tile GEMM / one split.
// mxfp8_debug_force_path can pin the path and the splits.
enum class Path { kTile = 0, kSkinny = 1, kMid = 2, kSlab = 3, kMed = 4, kMed64 = 5 };
struct Plan {
  Path path;
  int splits;   // K splits of the tile GEMM (also when the path is not the tile)
};

int bucket(const int64_t* bounds, int n, int64_t v) {
  for (int i = 0; i < n; ++i)
    if (v <= bounds[i]) return i;
  return n - 1;
}
bool splits_ok(int64_t K, int s) { return s == 1 || ((s == 2 || s == 4 || s == 8) && (K / 64) % (4 * s) == 0); }

Plan linear_plan(int64_t M, int64_t N, int64_t K) {
  const int im = bucket(mxfp8::kShapeTabM, mxfp8::kShapeTabNM, M);
  const int in = bucket(mxfp8::kShapeTabN, mxfp8::kShapeTabNN, N);
  const int ik = bucket(mxfp8::kShapeTabK, mxfp8::kShapeTabNK, K);
  const int code = mxfp8::kShapeTabPlan[im][in][ik];
  int s = mxfp8::kShapeTabTileSplits[im][in][ik];
  if (!splits_ok(K, s)) s = 1;
  Path path = (Path)(code >> 4);
  const int force = g_force_path.load(std::memory_order_relaxed);
  if (force == 1) path = Path::kTile;
  if (force == 3) path = Path::kMid;
  if (force == 4) path = Path::kSkinny;
  if (force == 5) path = Path::kSlab;
  if (force == 6) path = Path::kMed;
  if (force == 7) path = Path::kMed64;
  if (force >= 16) {
    path = Path::kTile;
    if (splits_ok(K, force - 16)) s = force - 16;
  }
  const bool small_k = K <= mxfp8::kSkinnyMaxK;
  if (path == Path::kSkinny && !(small_k && M <= mxfp8::kSkinnyMaxM)) path = Path::kTile;
  if (path == Path::kMid && !(small_k && M <= mxfp8::kMidMaxM)) path = Path::kTile;
  // The slab kernel: M <= 128, and its grid (128-row groups x K slices) and
  // its reduce (one thread per 4 outputs) in 32-bit range.
  // The medium-tile GEMM: one workgroup per (128-row weight group, tile).
  if ((path == Path::kMed || path == Path::kMed64) && n_pad(N) / 128 * ((M + 63) / 64) > INT32_MAX)
    path = Path::kTile;
  if (path == Path::kSlab &&
      (M > mxfp8::kMidMaxM || n_pad(N) / 128 * (K / 256) > INT32_MAX || M * (n_pad(N) / 4) > INT32_MAX))
    path = Path::kTile;
  return {path, s};
}
// The path of a call whose workspace may hold at most `cap` bytes: where the
// slab kernel's fp32 partials would not fit, the decode or mid-M kernel
// (which need at most one packed 128-row group) or the tile GEMM.
Path linear_path(int64_t M, int64_t N, int64_t K, size_t cap = SIZE_MAX) {
  const Path p = linear_plan(M, N, K).path;
  if (p != Path::kSlab || mxfp8::slab_ws_bytes(M, N, K) <= cap) return p;
  if (K <= mxfp8::kSkinnyMaxK) return M <= mxfp8::kSkinnyMaxM ? Path::kSkinny : Path::kMid;
  return Path::kTile;
}
// W4A8 takes the MXFP8 table's paths; the medium-tile GEMM has no 4-bit
// form, so its shapes take the tile path.
Path linear_path_w4a8(int64_t M, int64_t N, int64_t K) {
  const Path p = linear_path(M, N, K);
  return (p == Path::kMed || p == Path::kMed64) ? Path::kTile : p;
}
// The paths whose workspace and launch are the packed quantizer's.
bool packed_path(Path p) { return p == Path::kTile || p == Path::kMed || p == Path::kMed64; }

}  // namespace

int mxfp8::gemm_tile_splits(int64_t M, int64_t N, int64_t K) { return linear_plan(M, N, K).splits; }

// Compute units of the current device (the persistent GEMM's grid); the
// device check caches it on the first call of any entry point.
int mxfp8::device_cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_dev_cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    hipDeviceProp_t prop;
    n = (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0) ? prop.multiProcessorCount
                                                                                         : 256;
    g_dev_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int mxfp8::check_device_current() { return check_device(); }

int mxfp8::slab_steps_per_wave(int64_t N, int64_t K) {
  const int64_t G = (N + 127) / 128, KS = K / 128;
  // The largest of 4, 2 steps per wave that divides K into whole slices and
  // still gives at least 256 workgroups (one per compute unit), else 1.
  for (int spw = 4; spw >= 2; spw /= 2)
    if (KS % (2 * spw) == 0 && G * (KS / (2 * spw)) >= 256) return spw;
  return 1;
}

size_t mxfp8::slab_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t slices = (K / 128) / (2 * slab_steps_per_wave(N, K));
  return round_up((size_t)slices * (size_t)M * (size_t)n_pad(N) * 4, 256);
}

int mxfp8::linear_check_args(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                             const void* s_packed, int64_t N, const void* bias_bf16, const void* y_bf16,
                             int64_t ldy) {
  if (M < 0) return MXFP8_E_SHAPE;
  if (int st = check_packed(w_packed, s_packed, N, K)) return st;
  if (M == 0) return MXFP8_OK;
  if (M > (int64_t)1 << 30) return MXFP8_E_SHAPE;
  if (!x_bf16) return MXFP8_E_NULLPTR;
  if (int st = check_output(y_bf16, N, ldy, bias_bf16)) return st;
  if (ldx < K || ldx % 8 != 0) return MXFP8_E_LD;
  if (!aligned(x_bf16, 16)) return MXFP8_E_ALIGN;
  if (packed_path(linear_path(M, N, K)) && (n_pad(M) * (K / 8) + 255) / 256 > INT32_MAX) return MXFP8_E_SHAPE;
  return MXFP8_OK;
}

size_t mxfp8::linear_workspace_within(int64_t M, int64_t N, int64_t K, size_t cap) {
  if (M == 0) return 256;
  switch (linear_path(M, N, K, cap)) {
    case Path::kSkinny: return mxfp8::skinny_ws_bytes(M, K);
    case Path::kMid: return mxfp8::mid_ws_bytes(M, K);
    case Path::kSlab: return mxfp8::slab_ws_bytes(M, N, K);
    case Path::kMed:
    case Path::kMed64: return tile_ws_act_bytes(M, K);
    default: return tile_ws_bytes(M, N, K);
  }
}

int mxfp8::linear_launch(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                         const void* s_packed, int64_t N, const void* bias_bf16, void* y_bf16, int64_t ldy,
                         void* workspace, hipStream_t s, size_t cap) {
  const Path path = linear_path(M, N, K, cap);
  if (path == Path::kSkinny)
    return mxfp8::launch_gemm_skinny(x_bf16, ldx, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s,
                                     workspace);
  if (path == Path::kMid)
    return mxfp8::launch_gemm_mid(x_bf16, ldx, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s, workspace);
  if (path == Path::kSlab)
    return mxfp8::launch_gemm_slab(x_bf16, ldx, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s, workspace);
  uint8_t* q = (uint8_t*)workspace;
  uint8_t* sc = q + round_up((size_t)n_pad(M) * (size_t)K, 256);
  uint8_t* part = q + tile_ws_act_bytes(M, K);
  if (int st = mxfp8::launch_quantize_act_packed(x_bf16, M, K, ldx, q, sc, s)) return st;
  if (path == Path::kMed || path == Path::kMed64)
    return mxfp8::launch_gemm_med(q, sc, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s,
                                  path == Path::kMed ? 128 : 64);
  return mxfp8::launch_gemm_tile(q, sc, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s,
                                 mxfp8::gemm_tile_splits(M, N, K), part);
}

bool mxfp8::set_lds_limit_once(const void* fn, int bytes, std::atomic<int>* flags) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  int st = flags[dev].load(std::memory_order_acquire);
  if (st == 0) {
    // Two threads may both set it; the call is idempotent.
    st = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess ? 1 : 2;
    flags[dev].store(st, std::memory_order_release);
  }
  return st == 1;
}

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
    case MXFP8_E_SCRATCH:
      return "shape needs more scratch than mxfp8_linear_noalloc's static maximum (MXFP8_NOALLOC_SCRATCH_BYTES); "
             "call mxfp8_linear with a workspace";
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
  *bytes = mxfp8::linear_workspace_within(M, N, K, SIZE_MAX);
  return MXFP8_OK;
}

int mxfp8_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                 const void* s_packed, int64_t N, const void* bias_bf16, void* y_bf16, int64_t ldy,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = mxfp8::linear_check_args(x_bf16, M, K, ldx, w_packed, s_packed, N, bias_bf16, y_bf16, ldy)) return st;
  if (M == 0) return MXFP8_OK;
  size_t need = 0;
  mxfp8_linear_workspace_bytes(M, N, K, &need);
  if (!workspace || workspace_bytes < need) return MXFP8_E_WORKSPACE;
  if (!aligned(workspace, 256)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  return mxfp8::linear_launch(x_bf16, M, K, ldx, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, workspace,
                              (hipStream_t)stream, SIZE_MAX);
}

// ---------------------------------------------------------------- W4A8
int mxfp8_quantize_fp4(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* q_e2m1, int64_t ldq,
                       void* s_e8m0, int64_t lds, void* stream) {
  if (M < 0 || K < 0 || K % 32 != 0) return MXFP8_E_SHAPE;
  if (M == 0 || K == 0) return MXFP8_OK;
  if (!x_bf16 || !q_e2m1 || !s_e8m0) return MXFP8_E_NULLPTR;
  if (ldx < K || ldx % 8 != 0 || ldq < K / 2 || ldq % 4 != 0 || lds < K / 32) return MXFP8_E_LD;
  if (!aligned(x_bf16, 16) || !aligned(q_e2m1, 4)) return MXFP8_E_ALIGN;
  if ((M * (K / 8) + 255) / 256 > INT32_MAX) return MXFP8_E_SHAPE;
  if (int st = check_device()) return st;
  return mxfp8::launch_quantize_fp4(x_bf16, M, K, ldx, q_e2m1, ldq, s_e8m0, lds, (hipStream_t)stream);
}

int mxfp8_prepared_weight_fp4_bytes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes) {
  if (!w_bytes || !s_bytes) return MXFP8_E_NULLPTR;
  if (N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  *w_bytes = (size_t)n_pad(N) * (size_t)(K / 2);
  *s_bytes = (size_t)n_pad(N) * (size_t)(K / 32);
  return MXFP8_OK;
}

int mxfp8_prepare_weight_fp4(const void* w_e2m1, const void* w_s_e8m0, int64_t N, int64_t K, int64_t ldw,
                             int64_t ldws, void* w_packed, void* s_packed, void* stream) {
  if (int st = check_packed(w_packed, s_packed, N, K)) return st;
  if (!w_e2m1 || !w_s_e8m0) return MXFP8_E_NULLPTR;
  if (ldw < K / 2 || ldw % 16 != 0 || ldws < K / 32) return MXFP8_E_LD;
  if (!aligned(w_e2m1, 16)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  return mxfp8::launch_pack_weight_fp4(w_e2m1, w_s_e8m0, N, K, ldw, ldws, w_packed, s_packed, (hipStream_t)stream);
}

int mxfp8_unpack_weight_fp4(const void* w_packed, const void* s_packed, int64_t N, int64_t K, void* w_e2m1,
                            void* w_s_e8m0, void* stream) {
  if (int st = check_packed(w_packed, s_packed, N, K)) return st;
  if (!w_e2m1 || !w_s_e8m0) return MXFP8_E_NULLPTR;
  if (!aligned(w_e2m1, 16)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  return mxfp8::launch_unpack_weight_fp4(w_packed, s_packed, N, K, w_e2m1, w_s_e8m0, (hipStream_t)stream);
}

int mxfp8_linear_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return MXFP8_E_NULLPTR;
  if (M < 0 || N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  if (M == 0) {
    *bytes = 256;
    return MXFP8_OK;
  }
  switch (linear_path_w4a8(M, N, K)) {
    case Path::kSkinny: *bytes = mxfp8::skinny_ws_bytes(M, K); break;
    case Path::kMid: *bytes = mxfp8::mid_ws_bytes(M, K); break;
    case Path::kSlab: *bytes = mxfp8::slab_ws_bytes(M, N, K); break;
    default:
      // K splits: the weight widened to MXFP8 tiles after the split-K
      // workspace; one split: the 4-bit tile GEMM, no widened copy.
      *bytes = tile_ws_bytes(M, N, K) + (mxfp8::gemm_tile_splits(M, N, K) > 1 ? (size_t)n_pad(N) * (size_t)K : 0);
  }
  return MXFP8_OK;
}

int mxfp8_linear_w4a8(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
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
  const Path path = linear_path_w4a8(M, N, K);
  if (path == Path::kTile && (n_pad(M) * (K / 8) + 255) / 256 > INT32_MAX) return MXFP8_E_SHAPE;
  size_t need = 0;
  mxfp8_linear_w4a8_workspace_bytes(M, N, K, &need);
  if (!workspace || workspace_bytes < need) return MXFP8_E_WORKSPACE;
  if (!aligned(workspace, 256)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (path == Path::kSkinny)
    return mxfp8::launch_gemm_skinny_fp4(x_bf16, ldx, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s,
                                         workspace);
  if (path == Path::kMid)
    return mxfp8::launch_gemm_mid_fp4(x_bf16, ldx, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s,
                                      workspace);
  if (path == Path::kSlab)
    return mxfp8::launch_gemm_slab_fp4(x_bf16, ldx, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s,
                                       workspace);
  // Larger M is MFMA-bound: the 4-bit tile GEMM on the packed activations;
  // where the shape table splits K, the weight widened to the MXFP8 tiles
  // (exact) and the split-K MXFP8 tile GEMM.
  uint8_t* q = (uint8_t*)workspace;
  uint8_t* sc = q + round_up((size_t)n_pad(M) * (size_t)K, 256);
  uint8_t* part = q + tile_ws_act_bytes(M, K);
  const int splits = mxfp8::gemm_tile_splits(M, N, K);
  if (int st = mxfp8::launch_quantize_act_packed(x_bf16, M, K, ldx, q, sc, s)) return st;
  if (splits == 1)
    return mxfp8::launch_gemm_tile_w4(q, sc, M, K, w_packed, s_packed, N, bias_bf16, y_bf16, ldy, s);
  uint8_t* w8 = q + tile_ws_bytes(M, N, K);
  if (int st = mxfp8::launch_widen_fp4(w_packed, N, K, w8, s)) return st;
  return mxfp8::launch_gemm_tile(q, sc, M, K, w8, s_packed, N, bias_bf16, y_bf16, ldy, s, splits, part);
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
  if (M > (int64_t)1 << 30 || K > (int64_t)1 << 24) return MXFP8_E_SHAPE;
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

int mxfp8_gemm_prequant_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return MXFP8_E_NULLPTR;
  if (M < 0 || N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  *bytes = M == 0 ? 256 : tile_ws_bytes(M, N, K);
  return MXFP8_OK;
}

int mxfp8_gemm_prequant(const void* q_e4m3, int64_t ldq, const void* s_e8m0, int64_t lds, int64_t M, int64_t K,
                        const void* w_packed, const void* ws_packed, int64_t N, const void* bias_bf16, void* y_bf16,
                        int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0) return MXFP8_E_SHAPE;
  if (int st = check_packed(w_packed, ws_packed, N, K)) return st;
  if (M == 0) return MXFP8_OK;
  if (M > (int64_t)1 << 30) return MXFP8_E_SHAPE;
  if (!q_e4m3 || !s_e8m0) return MXFP8_E_NULLPTR;
  if (int st = check_output(y_bf16, N, ldy, bias_bf16)) return st;
  if (ldq < K || ldq % 16 != 0 || lds < K / 32) return MXFP8_E_LD;
  if (!aligned(q_e4m3, 16)) return MXFP8_E_ALIGN;
  if ((n_pad(M) * (K / 8) + 255) / 256 > INT32_MAX) return MXFP8_E_SHAPE;
  size_t need = 0;
  mxfp8_gemm_prequant_workspace_bytes(M, N, K, &need);
  if (!workspace || workspace_bytes < need) return MXFP8_E_WORKSPACE;
  if (!aligned(workspace, 256)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  // The row-major quantized activations packed like a weight (pad rows zero;
  // their scale byte does not reach the output), then the tile GEMM.
  uint8_t* q = (uint8_t*)workspace;
  uint8_t* sc = q + round_up((size_t)n_pad(M) * (size_t)K, 256);
  uint8_t* part = q + tile_ws_act_bytes(M, K);
  if (int st = mxfp8::launch_pack_weight(q_e4m3, s_e8m0, M, K, ldq, lds, q, sc, s)) return st;
  return mxfp8::launch_gemm_tile(q, sc, M, K, w_packed, ws_packed, N, bias_bf16, y_bf16, ldy, s,
                                 mxfp8::gemm_tile_splits(M, N, K), part);
}

int mxfp8_moe_prepared_bytes(int64_t E, int64_t H, int64_t I, size_t* w13_bytes, size_t* s13_bytes,
                             size_t* w2_bytes, size_t* s2_bytes) {
  if (!w13_bytes || !s13_bytes || !w2_bytes || !s2_bytes) return MXFP8_E_NULLPTR;
  if (int st = check_moe_shape(0, H, E, 1, I)) return st;
  *w13_bytes = (size_t)E * 2 * I * H;
  *s13_bytes = (size_t)E * 2 * I * (H / 32);
  *w2_bytes = (size_t)E * H * I;
  *s2_bytes = (size_t)E * H * (I / 32);
  return MXFP8_OK;
}

int mxfp8_moe_prepare_weights(const void* w13_e4m3, const void* w13_s_e8m0, const void* w2_e4m3,
                              const void* w2_s_e8m0, int64_t E, int64_t H, int64_t I, void* w13_packed,
                              void* s13_packed, void* w2_packed, void* s2_packed, void* stream) {
  if (int st = check_moe_shape(0, H, E, 1, I)) return st;
  if (!w13_e4m3 || !w13_s_e8m0 || !w2_e4m3 || !w2_s_e8m0 || !w13_packed || !s13_packed || !w2_packed || !s2_packed)
    return MXFP8_E_NULLPTR;
  if (!aligned(w13_e4m3, 16) || !aligned(w2_e4m3, 16)) return MXFP8_E_ALIGN;
  if (!aligned(w13_packed, 256) || !aligned(s13_packed, 256) || !aligned(w2_packed, 256) || !aligned(s2_packed, 256))
    return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (int st = mxfp8::launch_pack_weight_gate_up(w13_e4m3, w13_s_e8m0, E, I, H, w13_packed, s13_packed, s))
    return st;
  return mxfp8::launch_pack_weight(w2_e4m3, w2_s_e8m0, E * H, I, I, I / 32, w2_packed, s2_packed, s);
}

int mxfp8_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, size_t* bytes) {
  if (!bytes) return MXFP8_E_NULLPTR;
  if (int st = check_moe_shape(T, H, E, topk, I)) return st;
  *bytes = moe_layout(T, H, E, topk, I, nullptr, nullptr);
  return MXFP8_OK;
}

int mxfp8_moe_grouped(const void* x_bf16, const float* logits_f32, int64_t T, int64_t H, int64_t E, int64_t topk,
                      int64_t I, const void* w13_packed, const void* s13_packed, const void* w2_packed,
                      const void* s2_packed, void* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = check_moe_shape(T, H, E, topk, I)) return st;
  if (T == 0) return MXFP8_OK;
  if (!x_bf16 || !logits_f32 || !w13_packed || !s13_packed || !w2_packed || !s2_packed || !y_bf16)
    return MXFP8_E_NULLPTR;
  if (!aligned(x_bf16, 16) || !aligned(y_bf16, 16) || !aligned(logits_f32, 4)) return MXFP8_E_ALIGN;
  if (!aligned(w13_packed, 256) || !aligned(s13_packed, 256) || !aligned(w2_packed, 256) || !aligned(s2_packed, 256))
    return MXFP8_E_ALIGN;
  const size_t need = moe_layout(T, H, E, topk, I, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return MXFP8_E_WORKSPACE;
  if (!aligned(workspace, 256)) return MXFP8_E_ALIGN;
  if (int st = check_device()) return st;
  mxfp8::MoeArgs a;
  a.x = x_bf16;
  a.logits = logits_f32;
  a.T = T;
  a.H = H;
  a.E = E;
  a.topk = topk;
  a.I = I;
  a.w13p = w13_packed;
  a.s13p = s13_packed;
  a.w2p = w2_packed;
  a.s2p = s2_packed;
  a.y = y_bf16;
  a.dbg_act = g_dbg_act.load();
  a.dbg_q = g_dbg_q.load();
  a.dbg_s = g_dbg_s.load();
  a.dbg_ids = g_dbg_ids.load();
  a.dbg_wts = g_dbg_wts.load();
  moe_layout(T, H, E, topk, I, (uint8_t*)workspace, &a.ws);
  return mxfp8::launch_moe(a, (hipStream_t)stream);
}

int mxfp8_moe_debug_capture(void* act_bf16, void* act_e4m3, void* act_e8m0, void* ids_i32, void* wts_f32) {
  const int n = (act_bf16 != nullptr) + (act_e4m3 != nullptr) + (act_e8m0 != nullptr) + (ids_i32 != nullptr) +
                (wts_f32 != nullptr);
  if (n != 0 && n != 5) return MXFP8_E_NULLPTR;
  if (n == 5 && (!aligned(act_bf16, 8) || !aligned(act_e4m3, 4) || !aligned(ids_i32, 4) || !aligned(wts_f32, 4)))
    return MXFP8_E_ALIGN;
  // Published one at a time: set them between calls, not concurrently with one.
  g_dbg_act.store(act_bf16);
  g_dbg_q.store(act_e4m3);
  g_dbg_s.store(act_e8m0);
  g_dbg_ids.store(ids_i32);
  g_dbg_wts.store(wts_f32);
  return MXFP8_OK;
}

int mxfp8_debug_force_path(int path) {
  const bool tile_splits = path == 17 || path == 18 || path == 20 || path == 24;
  if (!(path >= 0 && path <= 7) && !tile_splits) return MXFP8_E_SHAPE;
  return g_force_path.exchange(path);
}

int mxfp8_debug_plan(int64_t M, int64_t N, int64_t K, int* path, int* splits) {
  if (!path || !splits) return MXFP8_E_NULLPTR;
  if (M < 1 || N < 1 || K < 256 || K % 256 != 0) return MXFP8_E_SHAPE;
  const Plan pl = linear_plan(M, N, K);
  *path = (int)pl.path;
  *splits = pl.path == Path::kTile ? pl.splits : 1;
  return MXFP8_OK;
}

}  // extern "C"
