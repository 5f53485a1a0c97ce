// One-time weight preparation: the checkpoint's MXFP8 weight (E4M3 [N, K],
// UE8M0 [N, K/32] linear layout) -> the packed tiles both GEMM paths read
// (layout described in common.hpp).  The preparation step of vLLM PR #52204
// (process_weights_after_loading, "implementation breakdown" of its digest):
// keep the logical [:N, :K/32] scale region, pad N to a multiple of 128,
// reorder for the GEMM.  Pad rows get zero elements and scale byte 127 (1.0).
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

// One thread per 16-byte chunk of W_p.
__global__ __launch_bounds__(256) void pack_w_kernel(const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
                                                     int64_t KS, int64_t total, uint8_t* __restrict__ wp) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t tile = t >> 10;  // 1024 chunks per 16 KiB tile
  const int slot = (int)(t & 1023);
  const int64_t g = tile / KS, ks = tile - g * KS;
  const int r = slot >> 3;
  const int c = (slot & 7) ^ (r & 7);
  const int64_t n = g * kGroupRows + r;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (n < N) v = *reinterpret_cast<const uint4*>(w + n * ldw + ks * kStepK + c * 16);
  reinterpret_cast<uint4*>(wp)[t] = v;
}

// One thread per 4-byte (one row, one K step) scale word of S_p.
__global__ __launch_bounds__(256) void pack_s_kernel(const uint8_t* __restrict__ ws, int64_t ldws, int64_t N,
                                                     int64_t KS, int64_t total, uint32_t* __restrict__ sp) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t tile = t >> 7;  // 128 rows per tile
  const int r = (int)(t & 127);
  const int64_t g = tile / KS, ks = tile - g * KS;
  const int64_t n = g * kGroupRows + r;
  uint32_t d = 0x7F7F7F7Fu;
  if (n < N) {
    const uint8_t* p = ws + n * ldws + ks * 4;
    d = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
  }
  sp[t] = d;
}

__global__ __launch_bounds__(256) void unpack_w_kernel(const uint8_t* __restrict__ wp, int64_t K, int64_t KS,
                                                       int64_t total, uint8_t* __restrict__ w) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t tile = t >> 10;
  const int slot = (int)(t & 1023);
  const int64_t g = tile / KS, ks = tile - g * KS;
  const int r = slot >> 3;
  const int c = (slot & 7) ^ (r & 7);
  const int64_t n = g * kGroupRows + r;
  *reinterpret_cast<uint4*>(w + n * K + ks * kStepK + c * 16) = reinterpret_cast<const uint4*>(wp)[t];
}

__global__ __launch_bounds__(256) void unpack_s_kernel(const uint32_t* __restrict__ sp, int64_t K, int64_t KS,
                                                       int64_t total, uint8_t* __restrict__ ws) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t tile = t >> 7;
  const int r = (int)(t & 127);
  const int64_t g = tile / KS, ks = tile - g * KS;
  const int64_t n = g * kGroupRows + r;
  const uint32_t d = sp[t];
  uint8_t* p = ws + n * (K / 32) + ks * 4;
  p[0] = (uint8_t)d;
  p[1] = (uint8_t)(d >> 8);
  p[2] = (uint8_t)(d >> 16);
  p[3] = (uint8_t)(d >> 24);
}

int launch_pack_weight(const void* w, const void* ws, int64_t N, int64_t K, int64_t ldw, int64_t ldws,
                       void* wp, void* sp, hipStream_t stream) {
  const int64_t KS = K / kStepK;
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int64_t tw = G * KS * (kTileBytes / 16);
  const int64_t ts = G * KS * kGroupRows;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)((tw + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)w, ldw, N, KS, tw, (uint8_t*)wp);
  hipLaunchKernelGGL(pack_s_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)ws, ldws, N, KS, ts, (uint32_t*)sp);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_unpack_weight(const void* wp, const void* sp, int64_t N, int64_t K, void* w, void* ws,
                         hipStream_t stream) {
  const int64_t KS = K / kStepK;
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int64_t tw = G * KS * (kTileBytes / 16);
  const int64_t ts = G * KS * kGroupRows;
  hipLaunchKernelGGL(unpack_w_kernel, dim3((unsigned)((tw + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)wp, K, KS, tw, (uint8_t*)w);
  hipLaunchKernelGGL(unpack_s_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, stream,
                     (const uint32_t*)sp, K, KS, ts, (uint8_t*)ws);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
