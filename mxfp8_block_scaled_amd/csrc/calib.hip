// Calibration kernels of the benchmark (libmxfp8_calib.so): what this GPU
// sustains, measured, for the two resources the layer is bound by.  They
// compute nothing of the layer; bench.py reports the layer's rates against
// them next to the published peaks.
//
//  * read stream: every workgroup reads its contiguous chunk of a buffer in
//    16-byte loads (eight in flight per thread) and folds them into one
//    word, so no load can be dropped; one word per workgroup is stored.
//    Timed over copies larger than the last-level cache it gives the HBM
//    read bandwidth a kernel can reach; over one 16 MiB copy per launch it
//    gives the floor of a decode-sized weight read.
//  * scaled MFMA: every wave issues back-to-back
//    v_mfma_scale_f32_16x16x128_f8f6f4 on register operands (eight
//    independent accumulators, so no MFMA waits for the previous result),
//    then stores the sum of its accumulators.  Each MFMA is 2 * 16 * 16 * 128
//    flops; the rate over a grid that fills the chip is the MFMA throughput
//    the chip sustains at its clock under that load.
//  * L2 -> CU stream: every workgroup (one per CU) reads the same small
//    buffer over and over, so after the first pass it is served by the die's
//    L2; the bytes a CU receives per second is the rate at which one CU pulls
//    operands from L2, the quantity the tile GEMMs' operand copies spend.
//    Two forms: 16-byte loads into registers (folded into one word), and
//    direct L2 -> LDS copies (buffer_load ... lds, the tile loops' path).
//  * empty kernel: launched back to back on one stream, the time per launch
//    is the floor under any call that is one kernel launch (dispatch, the
//    caches' acquire and release around a kernel, the drain).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void calib_read_kernel(const uint4* __restrict__ src, uint64_t per_block16,
                                                         uint32_t* __restrict__ sink) {
  // Workgroup b reads its own contiguous chunk, eight 16-byte loads in flight
  // per thread (measured on MI355X: 6.2 TB/s over 1 GiB, where a grid-stride
  // walk over the whole buffer reached 5.5).
  uint32_t acc = 0;
  const uint4* p = src + (uint64_t)blockIdx.x * per_block16;
  for (uint64_t i = threadIdx.x; i < per_block16; i += 256 * 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (i + u * 256 < per_block16) ? p[i + u * 256] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // Fold the wave, then one word per workgroup (wave 0 lane 0 of each).
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void calib_mfma_kernel(int iters, uint32_t seed, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;
  v8i a, b;
  for (int e = 0; e < 8; ++e) {
    // E4M3 bytes in a normal range (exponent field 4..11): finite products.
    uint32_t h = (t * 0x9E3779B1u) ^ (seed + 0x85EBCA6Bu * (uint32_t)e);
    h ^= h >> 15;
    a[e] = (int)((h & 0x3F3F3F3Fu) | 0x20202020u);
    b[e] = (int)(((h >> 1) & 0x3F3F3F3Fu) | 0x20202020u);
  }
  v4f acc[8];
  for (int k = 0; k < 8; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
  const int sa = 127, sb = 127;   // scale 2^0
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[k], 0, 0, 0, sa, 0, sb);
  }
  float s = 0.f;
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[t] = s;
}

// Workgroup of 256 threads re-reading [src, src + bytes) reps times; 16-byte
// loads, eight in flight per thread.
__global__ __launch_bounds__(256) void calib_l2_read_kernel(const uint4* __restrict__ src, uint32_t n16, int reps,
                                                            uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (int r = 0; r < reps; ++r) {
    for (uint32_t i = threadIdx.x; i < n16; i += 256 * 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (i + u * 256 < n16) ? src[i + u * 256] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

// The same traffic as direct L2 -> LDS copies: each wave moves 1 KiB per
// buffer_load_dwordx4 ... lds into one of 16 LDS slots of its own, with up
// to 15 copies in flight, walking [0, bytes) reps times (bytes a multiple of
// 4 KiB: each wave takes every fourth KiB).  The LDS contents are never read.
__global__ __launch_bounds__(256) void calib_l2_lds_kernel(const uint8_t* __restrict__ src, uint32_t bytes, int reps) {
  __shared__ __attribute__((aligned(16))) uint8_t slots[4][16][1024];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint64_t b = (uint64_t)(uintptr_t)src;
  typedef int i4v __attribute__((ext_vector_type(4)));
  i4v rsrc;
  rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  rsrc[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  rsrc[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  rsrc[3] = 0x00020000;
  const uint32_t voff = (threadIdx.x & 63) * 16u;
  int k = 0;
  for (int r = 0; r < reps; ++r) {
    for (uint32_t off = (uint32_t)wave * 1024u; off < bytes; off += 4096u) {
      const uint32_t lds = (uint32_t)(uintptr_t)&slots[wave][k & 15][0];
      asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds\n\ts_waitcnt vmcnt(15)"
                   ::"v"(voff), "s"(rsrc), "s"(off), "s"(lds)
                   : "memory", "m0");
      ++k;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ void calib_empty_kernel() {}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16 * blocks, 16-byte aligned) at src with
// `blocks` workgroups of 256 threads, each a contiguous bytes / blocks
// chunk; sink receives one word per workgroup.  Returns 0, -2 for invalid
// arguments, or -7 if the launch failed.
int mxfp8_calib_read(const void* src, uint64_t bytes, int blocks, void* sink, void* stream) {
  if (!src || !sink || blocks < 1 || bytes % (16 * (uint64_t)blocks) != 0 || ((uintptr_t)src & 15) != 0) return -2;
  hipLaunchKernelGGL(calib_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16 / (uint64_t)blocks, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// blocks x 256 threads, each wave iters x 8 scaled MFMAs (16x16x128 E4M3):
// 2 * 16 * 16 * 128 * 8 * iters flops per wave.  out: blocks * 256 floats.
int mxfp8_calib_mfma(int blocks, int iters, void* out, void* stream) {
  if (!out || blocks < 1 || iters < 1) return -2;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters, 12345u,
                     (float*)out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// blocks x 256 threads, each workgroup re-reading the bytes at src (16-byte
// aligned, a multiple of 4096) reps times, into registers (lds == 0) or by
// direct L2 -> LDS copies (lds != 0); sink: one word per workgroup.
int mxfp8_calib_l2(const void* src, uint32_t bytes, int blocks, int reps, int lds, void* sink, void* stream) {
  if (!src || !sink || blocks < 1 || reps < 1 || bytes == 0 || bytes % 4096 != 0 || ((uintptr_t)src & 15) != 0)
    return -2;
  if (lds)
    hipLaunchKernelGGL(calib_l2_lds_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)src, bytes, reps);
  else
    hipLaunchKernelGGL(calib_l2_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, bytes / 16u, reps, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// One launch of an empty kernel of blocks x threads (threads <= 1024).
int mxfp8_calib_empty(int blocks, int threads, void* stream) {
  if (blocks < 1 || threads < 1 || threads > 1024) return -2;
  hipLaunchKernelGGL(calib_empty_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
