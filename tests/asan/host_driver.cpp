// Host-side check of libmxfp8's C ABI under AddressSanitizer and UBSan: the
// library's host code (api.cpp) built for the CPU, the HIP runtime calls it
// makes and the kernel launchers replaced by stubs.  Each stub launcher
// writes every byte its kernel would write -- workspace regions and outputs,
// with the extents the kernels use -- so a workspace carved too small, a
// pointer outside the caller's buffer or an extent computed wrong becomes an
// ASan report.  Buffers are malloc'ed at exactly the sizes the library asks
// for.  Prints "host driver ok" and exits 0 when every check passed.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "launch.hpp"
#include "mxfp8.h"

// ---------------------------------------------------------------- HIP stubs
// One gfx950 device with 256 compute units.
extern "C" hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* p, int) {
  std::memset(p, 0, sizeof(*p));
  std::strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
  p->multiProcessorCount = 256;
  return hipSuccess;
}
extern "C" hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) { return hipSuccess; }

// ---------------------------------------------------------------- launch stubs
namespace {
int g_launches = 0;
void touch(void* p, size_t bytes) {
  if (bytes) std::memset(p, 0xA5, bytes);   // ASan checks every byte
  ++g_launches;
}
size_t mpad(int64_t m) { return (size_t)((m + 127) / 128 * 128); }
void touch_rows(void* y, int64_t rows, int64_t cols, int64_t ld, size_t elem) {
  for (int64_t r = 0; r < rows; ++r) std::memset((uint8_t*)y + (size_t)r * ld * elem, 0x5A, (size_t)cols * elem);
}
}  // namespace

namespace mxfp8 {
int launch_quantize_act(const void*, int64_t M, int64_t K, int64_t, void* q, int64_t ldq, void* s, int64_t lds,
                        hipStream_t) {
  touch_rows(q, M, K, ldq, 1);
  touch_rows(s, M, K / 32, lds, 1);
  touch(nullptr, 0);
  return 0;
}
int launch_quantize_act_packed(const void*, int64_t M, int64_t K, int64_t, void* qp, void* sp, hipStream_t) {
  touch(qp, mpad(M) * K);
  touch(sp, mpad(M) * (K / 32));
  return 0;
}
int launch_pack_weight(const void*, const void*, int64_t N, int64_t K, int64_t, int64_t, void* wp, void* sp,
                       hipStream_t) {
  touch(wp, mpad(N) * K);
  touch(sp, mpad(N) * (K / 32));
  return 0;
}
int launch_pack_weight_gate_up(const void*, const void*, int64_t E, int64_t I, int64_t K, void* wp, void* sp,
                               hipStream_t) {
  touch(wp, (size_t)E * 2 * I * K);
  touch(sp, (size_t)E * 2 * I * (K / 32));
  return 0;
}
int launch_unpack_weight(const void*, const void*, int64_t N, int64_t K, void* w, void* ws, hipStream_t) {
  touch(w, mpad(N) * K);
  touch(ws, mpad(N) * (K / 32));
  return 0;
}
int launch_gemm_tile(const void*, const void*, int64_t M, int64_t, const void*, const void*, int64_t N, const void*,
                     void* y, int64_t ldy, hipStream_t, int splits, void* part) {
  if (splits > 1) touch(part, (size_t)splits * M * ((N + 3) / 4 * 4) * 4);
  touch_rows(y, M, N, ldy, 2);
  touch(nullptr, 0);
  return 0;
}
int launch_gemm_tile_w4(const void*, const void*, int64_t M, int64_t, const void*, const void*, int64_t N,
                        const void*, void* y, int64_t ldy, hipStream_t) {
  touch_rows(y, M, N, ldy, 2);
  return 0;
}
int launch_gemm_skinny(const void*, int64_t, int64_t M, int64_t, const void*, const void*, int64_t N, const void*,
                       void* y, int64_t ldy, hipStream_t, void*) {
  touch_rows(y, M, N, ldy, 2);
  touch(nullptr, 0);
  return 0;
}
int launch_gemm_skinny_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                           int64_t N, const void* b, void* y, int64_t ldy, hipStream_t s, void* ws) {
  return launch_gemm_skinny(x, ldx, M, K, wp, sp, N, b, y, ldy, s, ws);
}
int launch_gemm_mid(const void*, int64_t, int64_t M, int64_t K, const void*, const void*, int64_t N, const void*,
                    void* y, int64_t ldy, hipStream_t, void* ws) {
  touch(ws, (size_t)kGroupRowsHost * K + (size_t)kGroupRowsHost * (K / 32));   // one packed 128-row group
  touch_rows(y, M, N, ldy, 2);
  return 0;
}
int launch_gemm_med(const void*, const void*, int64_t M, int64_t, const void*, const void*, int64_t N, const void*,
                    void* y, int64_t ldy, hipStream_t, int) {
  touch_rows(y, M, N, ldy, 2);
  return 0;
}
int launch_gemm_slab(const void*, int64_t, int64_t M, int64_t K, const void*, const void*, int64_t N, const void*,
                     void* y, int64_t ldy, hipStream_t, void* ws) {
  // one fp32 partial [M, N_pad] per K slice, then the reduce's bf16 rows
  const int64_t slices = (K / 128) / (2 * slab_steps_per_wave(N, K));
  touch(ws, (size_t)slices * M * mpad(N) * 4);
  touch_rows(y, M, N, ldy, 2);
  return 0;
}
int launch_gemm_slab_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                         int64_t N, const void* b, void* y, int64_t ldy, hipStream_t s, void* ws) {
  return launch_gemm_slab(x, ldx, M, K, wp, sp, N, b, y, ldy, s, ws);
}
int launch_gemm_mid_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                        const void* b, void* y, int64_t ldy, hipStream_t s, void* ws) {
  return launch_gemm_mid(x, ldx, M, K, wp, sp, N, b, y, ldy, s, ws);
}
int launch_pack_weight_fp4(const void*, const void*, int64_t N, int64_t K, int64_t, int64_t, void* wp, void* sp,
                           hipStream_t) {
  touch(wp, mpad(N) * (K / 2));
  touch(sp, mpad(N) * (K / 32));
  return 0;
}
int launch_unpack_weight_fp4(const void*, const void*, int64_t N, int64_t K, void* w, void* ws, hipStream_t) {
  touch(w, mpad(N) * (K / 2));
  touch(ws, mpad(N) * (K / 32));
  return 0;
}
int launch_widen_fp4(const void*, int64_t N, int64_t K, void* w8, hipStream_t) {
  touch(w8, mpad(N) * K);
  return 0;
}
int launch_quantize_fp4(const void*, int64_t M, int64_t K, int64_t, void* q, int64_t ldq, void* s, int64_t lds,
                        hipStream_t) {
  touch_rows(q, M, K / 2, ldq, 1);
  touch_rows(s, M, K / 32, lds, 1);
  touch(nullptr, 0);
  return 0;
}
int launch_moe(const MoeArgs& a, hipStream_t) {
  const MoeWorkspace& w = a.ws;
  const int64_t R = a.T * a.topk, nblk = (a.T + 15) / 16;
  touch(w.ids, R * 4);
  touch(w.wts, R * 4);
  touch(w.blk_cnt, nblk * a.E * 4);
  touch(w.blk_off, nblk * a.E * 4);
  touch(w.seg_off, a.E * 4);
  touch(w.meta, 2 * 4);
  touch(w.tile_e, w.mt_max * 4);
  touch(w.tile_g0, w.mt_max * 4);
  touch(w.tile_ng, w.mt_max * 4);
  touch(w.sorted_row, w.p_max * 4);
  touch(w.xq, (a.T + 1) * a.H);
  touch(w.xs, (a.T + 1) * (a.H / 32));
  touch(w.a1s, w.p_max * (a.H / 32));
  touch(w.a2q, w.p_max * a.I);
  touch(w.a2s, w.p_max * (a.I / 32));
  touch(w.ys, (R + 1) * a.H * 4);
  touch(a.y, a.T * a.H * 2);
  return 0;
}
}  // namespace mxfp8

// ---------------------------------------------------------------- driver
namespace {
int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

// Exact-size aligned allocation (the end of the buffer is the end of the heap block).
uint8_t* alloc_exact(size_t bytes) {
  void* p = nullptr;
  if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0) std::abort();
  return (uint8_t*)p;
}

void linear_case(int64_t M, int64_t N, int64_t K, int64_t ldy_extra, bool fp4) {
  size_t ws = 0;
  CHECK((fp4 ? mxfp8_linear_w4a8_workspace_bytes(M, N, K, &ws) : mxfp8_linear_workspace_bytes(M, N, K, &ws)) == 0);
  size_t wb = 0, sb = 0;
  CHECK((fp4 ? mxfp8_prepared_weight_fp4_bytes(N, K, &wb, &sb) : mxfp8_prepared_weight_bytes(N, K, &wb, &sb)) == 0);
  uint8_t* x = alloc_exact((size_t)M * K * 2);
  uint8_t* wp = alloc_exact(wb);
  uint8_t* sp = alloc_exact(sb);
  uint8_t* bias = alloc_exact((size_t)N * 2);
  const int64_t ldy = N + ldy_extra;
  uint8_t* y = alloc_exact((size_t)M * ldy * 2);
  uint8_t* w = alloc_exact(ws);
  const int st = fp4 ? mxfp8_linear_w4a8(x, M, K, K, wp, sp, N, bias, y, ldy, w, ws, nullptr)
                     : mxfp8_linear(x, M, K, K, wp, sp, N, bias, y, ldy, w, ws, nullptr);
  CHECK(st == 0);
  // one byte short is refused
  if (M > 0) CHECK((fp4 ? mxfp8_linear_w4a8(x, M, K, K, wp, sp, N, bias, y, ldy, w, ws - 1, nullptr)
                        : mxfp8_linear(x, M, K, K, wp, sp, N, bias, y, ldy, w, ws - 1, nullptr)) == MXFP8_E_WORKSPACE);
  for (uint8_t* p : {x, wp, sp, bias, y, w}) std::free(p);
}

void moe_case(int64_t T, int64_t H, int64_t E, int64_t k, int64_t I) {
  size_t ws = 0, w13 = 0, s13 = 0, w2 = 0, s2 = 0;
  CHECK(mxfp8_moe_workspace_bytes(T, H, I, E, k, &ws) == 0);
  CHECK(mxfp8_moe_prepared_bytes(E, H, I, &w13, &s13, &w2, &s2) == 0);
  uint8_t* x = alloc_exact((size_t)T * H * 2);
  float* logits = (float*)alloc_exact((size_t)T * E * 4);
  uint8_t* p13 = alloc_exact(w13);
  uint8_t* q13 = alloc_exact(s13);
  uint8_t* p2 = alloc_exact(w2);
  uint8_t* q2 = alloc_exact(s2);
  uint8_t* y = alloc_exact((size_t)T * H * 2);
  uint8_t* w = alloc_exact(ws);
  CHECK(mxfp8_moe_grouped(x, logits, T, H, E, k, I, p13, q13, p2, q2, y, w, ws, nullptr) == 0);
  // prepare: reads checkpoint-layout weights, writes the packed ones
  uint8_t* c13 = alloc_exact((size_t)E * 2 * I * H);
  uint8_t* c13s = alloc_exact((size_t)E * 2 * I * (H / 32));
  uint8_t* c2 = alloc_exact((size_t)E * H * I);
  uint8_t* c2s = alloc_exact((size_t)E * H * (I / 32));
  CHECK(mxfp8_moe_prepare_weights(c13, c13s, c2, c2s, E, H, I, p13, q13, p2, q2, nullptr) == 0);
  for (uint8_t* p : {x, (uint8_t*)logits, p13, q13, p2, q2, y, w, c13, c13s, c2, c2s}) std::free(p);
}
}  // namespace

int main() {
  // Every GEMM path of both layers, ragged shapes, ldy > N, split-K tiles.
  const int64_t shapes[][3] = {{1, 130, 256},   {7, 4096, 4096}, {16, 255, 8192}, {17, 1, 256},    {100, 384, 768},
                               {128, 4096, 4096}, {129, 200, 1024}, {300, 640, 512}, {256, 2048, 4096}, {5, 130, 8448},
                               {1031, 1000, 512}};
  for (const auto& s : shapes)
    for (int fp4 = 0; fp4 < 2; ++fp4)
      for (int64_t extra : {0, 24}) linear_case(s[0], s[1], s[2], extra, fp4 != 0);
  for (int path : {1, 3, 5, 6, 7})   // forced paths
  {
    const int prev = mxfp8_debug_force_path(path);
    linear_case(9, 384, 1024, 8, false);
    linear_case(100, 130, 512, 0, true);
    mxfp8_debug_force_path(prev);
  }
  // Quantizers, pack / unpack, the packed entries, the test GEMM.
  {
    const int64_t M = 37, K = 1024, N = 300;
    uint8_t* x = alloc_exact((size_t)M * K * 2);
    uint8_t* q = alloc_exact((size_t)M * K);
    uint8_t* s = alloc_exact((size_t)M * (K / 32));
    CHECK(mxfp8_quantize_act(x, M, K, K, q, K, s, K / 32, nullptr) == 0);
    uint8_t* q4 = alloc_exact((size_t)M * (K / 2));
    CHECK(mxfp8_quantize_fp4(x, M, K, K, q4, K / 2, s, K / 32, nullptr) == 0);
    size_t qb = 0, sb = 0;
    CHECK(mxfp8_packed_act_bytes(M, K, &qb, &sb) == 0);
    uint8_t* qp = alloc_exact(qb);
    uint8_t* sp = alloc_exact(sb);
    CHECK(mxfp8_quantize_act_packed(x, M, K, K, qp, sp, nullptr) == 0);
    size_t wb = 0, wsb = 0;
    CHECK(mxfp8_prepared_weight_bytes(N, K, &wb, &wsb) == 0);
    uint8_t* w = alloc_exact((size_t)N * K);
    uint8_t* wsc = alloc_exact((size_t)N * (K / 32));
    uint8_t* wp = alloc_exact(wb);
    uint8_t* wps = alloc_exact(wsb);
    CHECK(mxfp8_prepare_weight(w, wsc, N, K, K, K / 32, wp, wps, nullptr) == 0);
    uint8_t* uw = alloc_exact(wb);
    uint8_t* us = alloc_exact(wsb);
    CHECK(mxfp8_unpack_weight(wp, wps, N, K, uw, us, nullptr) == 0);
    uint8_t* y = alloc_exact((size_t)M * N * 2);
    CHECK(mxfp8_gemm_packed(qp, sp, M, K, wp, wps, N, nullptr, y, N, nullptr) == 0);
    size_t pw = 0;
    CHECK(mxfp8_gemm_prequant_workspace_bytes(M, N, K, &pw) == 0);
    uint8_t* pws = alloc_exact(pw);
    CHECK(mxfp8_gemm_prequant(q, K, s, K / 32, M, K, wp, wps, N, nullptr, y, N, pws, pw, nullptr) == 0);
    size_t w4b = 0, s4b = 0;
    CHECK(mxfp8_prepared_weight_fp4_bytes(N, K, &w4b, &s4b) == 0);
    uint8_t* w4 = alloc_exact((size_t)N * (K / 2));
    uint8_t* w4p = alloc_exact(w4b);
    uint8_t* s4p = alloc_exact(s4b);
    CHECK(mxfp8_prepare_weight_fp4(w4, wsc, N, K, K / 2, K / 32, w4p, s4p, nullptr) == 0);
    uint8_t* uw4 = alloc_exact(w4b);
    uint8_t* us4 = alloc_exact(s4b);
    CHECK(mxfp8_unpack_weight_fp4(w4p, s4p, N, K, uw4, us4, nullptr) == 0);
    for (uint8_t* p : {x, q, s, q4, qp, sp, w, wsc, wp, wps, uw, us, y, pws, w4, w4p, s4p, uw4, us4}) std::free(p);
  }
  // The routed MoE layer: ragged token counts, the largest E and top-k.
  moe_case(200, 256, 8, 2, 256);
  moe_case(37, 256, 256, 16, 256);
  moe_case(1, 512, 4, 1, 512);
  moe_case(4096, 2048, 128, 8, 768);
  // Invalid arguments return before any launch.
  const int before = g_launches;
  CHECK(mxfp8_linear(nullptr, 4, 256, 256, nullptr, nullptr, 4, nullptr, nullptr, 4, nullptr, 0, nullptr) != 0);
  CHECK(mxfp8_moe_grouped(nullptr, nullptr, 4, 256, 8, 9, 256, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                          nullptr) == MXFP8_E_SHAPE);
  CHECK(g_launches == before);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host driver ok: %d launches checked\n", g_launches);
  return 0;
}
