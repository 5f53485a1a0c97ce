// One-time weight preparation: the checkpoint's MXFP8 weight (E4M3 [N, K],
// UE8M0 [N, K/32] linear layout) -> the packed tiles both GEMM paths read
// (layout described in common.hpp).  The preparation step of vLLM PR #52204
// (process_weights_after_loading, "implementation breakdown" of its digest):
// keep the logical [:N, :K/32] scale region, pad N to a multiple of 128,
// reorder for the GEMM.  Pad rows get zero elements and scale byte 127 (1.0).
//
// The inverse (unpack) serves tests and tooling; the packed activations of
// the large-M path use the same layout, so it unpacks those as well.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

constexpr int kChunksPerTile = kTileBytes / 16;  // 512

// Source row of packed row n: n itself, or (gate_up_I > 0) the gate/up
// interleave of stacked [E * 2I] expert weights described in launch.hpp.
__device__ inline int64_t src_row(int64_t n, int64_t gate_up_I) {
  if (gate_up_I == 0) return n;
  const int64_t per = 2 * gate_up_I;
  const int64_t e = n / per, p = n - e * per;
  const int64_t t = p / 256, h = (p / 128) & 1, q = p & 127;
  const int64_t row = q < 64 ? t * 128 + h * 64 + q : gate_up_I + t * 128 + h * 64 + (q - 64);
  return e * per + row;
}

// Packed chunk t (16 bytes, in storage order) -> its 128-row group g, step
// ks, row r inside the group and logical chunk c: group-major, then 16-row
// band, then step, then (row in band, chunk position).
struct ChunkPos {
  int64_t g, ks;
  int r, c;
};
__device__ inline ChunkPos chunk_pos(int64_t t, int64_t KS) {
  const int64_t per_group = KS * kChunksPerTile;
  ChunkPos p;
  p.g = t / per_group;
  const int64_t rem = t - p.g * per_group;
  const int64_t band = rem / (KS * 64);
  const int64_t rem2 = rem - band * (KS * 64);
  p.ks = rem2 >> 6;
  const int slot = (int)(rem2 & 63);
  p.r = (int)band * 16 + (slot >> 2);
  p.c = (slot & 3) ^ swz(p.r);
  return p;
}

// One thread per 16-byte chunk of the packed data.
__global__ __launch_bounds__(256) void pack_w_kernel(const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
                                                     int64_t KS, int64_t total, uint8_t* __restrict__ wp,
                                                     int64_t gate_up_I) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const ChunkPos cp = chunk_pos(t, KS);
  const int64_t g = cp.g, ks = cp.ks;
  const int r = cp.r, c = cp.c;
  const int64_t n = g * kGroupRows + r;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (n < N) v = *reinterpret_cast<const uint4*>(w + src_row(n, gate_up_I) * ldw + ks * kStepK + c * 16);
  reinterpret_cast<uint4*>(wp)[t] = v;
}

// One thread per (row, 64-element K step): its two scale bytes.
__global__ __launch_bounds__(256) void pack_s_kernel(const uint8_t* __restrict__ ws, int64_t ldws, int64_t N,
                                                     int64_t KS, int64_t total, uint8_t* __restrict__ sp,
                                                     int64_t gate_up_I) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t tile = t / kGroupRows;
  const int r = (int)(t % kGroupRows);
  const int64_t g = tile / KS, ks = tile - g * KS;
  const int64_t n = g * kGroupRows + r;
  uint8_t b0 = 0x7F, b1 = 0x7F;
  if (n < N) {
    const uint8_t* p = ws + src_row(n, gate_up_I) * ldws + ks * 2;
    b0 = p[0];
    b1 = p[1];
  }
  uint8_t* d = sp + tile * kTileScaleBytes;
  d[scale_off(r, 0)] = b0;
  d[scale_off(r, 1)] = b1;
}

__global__ __launch_bounds__(256) void unpack_w_kernel(const uint8_t* __restrict__ wp, int64_t K, int64_t KS,
                                                       int64_t total, uint8_t* __restrict__ w) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const ChunkPos cp = chunk_pos(t, KS);
  const int64_t n = cp.g * kGroupRows + cp.r;
  *reinterpret_cast<uint4*>(w + n * K + cp.ks * kStepK + cp.c * 16) = reinterpret_cast<const uint4*>(wp)[t];
}

__global__ __launch_bounds__(256) void unpack_s_kernel(const uint8_t* __restrict__ sp, int64_t K, int64_t KS,
                                                       int64_t total, uint8_t* __restrict__ ws) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t tile = t / kGroupRows;
  const int r = (int)(t % kGroupRows);
  const int64_t g = tile / KS, ks = tile - g * KS;
  const int64_t n = g * kGroupRows + r;
  const uint8_t* d = sp + tile * kTileScaleBytes;
  uint8_t* p = ws + n * (K / 32) + ks * 2;
  p[0] = d[scale_off(r, 0)];
  p[1] = d[scale_off(r, 1)];
}

static int pack(const void* w, const void* ws, int64_t N, int64_t K, int64_t ldw, int64_t ldws, void* wp,
                void* sp, int64_t gate_up_I, hipStream_t stream) {
  const int64_t KS = K / kStepK;
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int64_t tw = G * KS * kChunksPerTile;
  const int64_t ts = G * KS * kGroupRows;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)((tw + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)w, ldw, N, KS, tw, (uint8_t*)wp, gate_up_I);
  hipLaunchKernelGGL(pack_s_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)ws, ldws, N, KS, ts, (uint8_t*)sp, gate_up_I);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_pack_weight(const void* w, const void* ws, int64_t N, int64_t K, int64_t ldw, int64_t ldws,
                       void* wp, void* sp, hipStream_t stream) {
  return pack(w, ws, N, K, ldw, ldws, wp, sp, 0, stream);
}

int launch_pack_weight_gate_up(const void* w, const void* ws, int64_t E, int64_t I, int64_t K, void* wp, void* sp,
                               hipStream_t stream) {
  return pack(w, ws, E * 2 * I, K, K, K / 32, wp, sp, I, stream);
}

// MXFP4 weights (two E2M1 elements per byte along K, element 2j in the low
// nibble): a 128-element K step of a 16-row band is the same 1 KiB piece as an
// E4M3 piece of a 64-element step (64 bytes per row, four 16-byte chunks, the
// same chunk swizzle, bands KS4 = K / 128 pieces long) -- a lane of the scaled
// MFMA with an E2M1 operand takes 16 bytes = 32 consecutive K of one row,
// like the E4M3 lane takes 16 bytes = 16 K -- so the byte packing is pack_w
// over K / 2 bytes per row.  The UE8M0 scales are per 32 elements either way:
// pack_s unchanged.
int launch_pack_weight_fp4(const void* w, const void* ws, int64_t N, int64_t K, int64_t ldw, int64_t ldws,
                           void* wp, void* sp, hipStream_t stream) {
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int64_t KS4 = K / 128, KS = K / kStepK;
  const int64_t tw = G * KS4 * kChunksPerTile;
  const int64_t ts = G * KS * kGroupRows;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)((tw + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)w, ldw, N, KS4, tw, (uint8_t*)wp, (int64_t)0);
  hipLaunchKernelGGL(pack_s_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)ws, ldws, N, KS, ts, (uint8_t*)sp, (int64_t)0);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Packed MXFP4 tiles -> packed MXFP8 tiles of the same values (every E2M1
// value is an E4M3 value; the scales are unchanged), for the tile GEMM.  One
// thread per 16-byte E4M3 chunk: chunk c8 (16 elements) of row r in 64-K step
// s is half (c8 & 1) of E2M1 chunk 2 (s & 1) + c8 / 2 of row r in 128-K step
// s / 2.  E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 are the E4M3 bytes
// 0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C; the sign bit moves from
// bit 3 to bit 7.
__device__ inline uint32_t e2m1_to_e4m3(uint32_t c) {
  constexpr uint32_t lo = 0x3C383000u, hi = 0x4C484440u;   // bytes of the 8 magnitudes
  const uint32_t m = c & 7u;
  const uint32_t b = ((m < 4 ? lo : hi) >> (8 * (m & 3))) & 0xFFu;
  return b | ((c & 8u) << 4);
}
__global__ __launch_bounds__(256) void widen_fp4_kernel(const uint8_t* __restrict__ w4, int64_t KS, int64_t total,
                                                        uint8_t* __restrict__ w8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const ChunkPos cp = chunk_pos(t, KS);                    // E4M3 chunk: 64-K step s
  const int64_t g = cp.g, s = cp.ks;
  const int r = cp.r, c8 = cp.c;
  const int c4 = 2 * (int)(s & 1) + (c8 >> 1);
  const int64_t KS4 = KS / 2;                              // E2M1 steps of 128 K
  const uint8_t* src = w4 + g * KS4 * kTileBytes + packed_off(r, s >> 1, c4, KS4) + (c8 & 1) * 8;
  const uint2 v = *reinterpret_cast<const uint2*>(src);
  const uint32_t in[2] = {v.x, v.y};
  uint32_t out[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = in[d >> 1] >> (16 * (d & 1));      // four nibbles = four elements
    out[d] = e2m1_to_e4m3(w & 0xF) | (e2m1_to_e4m3((w >> 4) & 0xF) << 8) |
             (e2m1_to_e4m3((w >> 8) & 0xF) << 16) | (e2m1_to_e4m3((w >> 12) & 0xF) << 24);
  }
  reinterpret_cast<uint4*>(w8)[t] = make_uint4(out[0], out[1], out[2], out[3]);
}

int launch_widen_fp4(const void* w4, int64_t N, int64_t K, void* w8, hipStream_t stream) {
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int64_t KS = K / kStepK;
  const int64_t total = G * KS * kChunksPerTile;
  hipLaunchKernelGGL(widen_fp4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)w4, KS, total, (uint8_t*)w8);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_unpack_weight(const void* wp, const void* sp, int64_t N, int64_t K, void* w, void* ws,
                         hipStream_t stream) {
  const int64_t KS = K / kStepK;
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int64_t tw = G * KS * kChunksPerTile;
  const int64_t ts = G * KS * kGroupRows;
  hipLaunchKernelGGL(unpack_w_kernel, dim3((unsigned)((tw + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)wp, K, KS, tw, (uint8_t*)w);
  hipLaunchKernelGGL(unpack_s_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)sp, K, KS, ts, (uint8_t*)ws);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Inverse of launch_pack_weight_fp4: the byte packing is that of an E4M3
// operand of K / 2 bytes per row (K / 128 pieces of 64 bytes), the scales
// those of a K-element row.
int launch_unpack_weight_fp4(const void* wp, const void* sp, int64_t N, int64_t K, void* w, void* ws,
                             hipStream_t stream) {
  const int64_t KS4 = K / 128, KS = K / kStepK;
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int64_t tw = G * KS4 * kChunksPerTile;
  const int64_t ts = G * KS * kGroupRows;
  hipLaunchKernelGGL(unpack_w_kernel, dim3((unsigned)((tw + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)wp, K / 2, KS4, tw, (uint8_t*)w);
  hipLaunchKernelGGL(unpack_s_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)sp, K, KS, ts, (uint8_t*)ws);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
