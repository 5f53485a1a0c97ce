// Split-K "slab" MXFP8 linear layer for M <= 128 at any K, with the
// activation quantization fused in (and its W4A8 form: MXFP4 weights as the
// MFMA's E2M1 A operand, the same activations).
//
// Up to M = 128 the weight is still the dominant HBM stream, but every
// workgroup of a kernel that owns a few weight rows over the whole K has to
// read the whole activation; at M = 128 those re-reads from L2 are 8 times the
// weight bytes, and L2 -> CU bandwidth, not HBM, sets the time.  Here a
// workgroup owns a whole 128-row group of the packed weight (eight 16-row
// bands) but only a slice of K (kSK = 2 kSpw steps of 128), so it needs only
// the activation slab [M, 128 kSK]:
//  1. the workgroup loads its bf16 slab, coalesced, then issues the weight
//     loads of its slice (loads return in issue order: the slab arrives
//     first and is converted while the weights stream);
//  2. it quantizes the slab by the MX rule into LDS (four lanes per 32-block,
//     amax by two quad exchanges, gfx950's scaled converter), each element
//     once per workgroup;
//  3. wave (band b, half h) runs one v_mfma_scale_f32_16x16x128_f8f6f4 per
//     (step of its half, 16-row group of the slab), the weight band as the A
//     operand and the slab rows from LDS as B;
//  4. the two halves are added in K order through LDS and the fp32 partial
//     [M, 128] of the slice is stored; a second kernel adds the K slices in
//     order with the bias and rounds once to bf16.
// Workgroups of one K slice run on one die (the slab is read from that die's
// L2 by all of them).  Per workgroup at M = 128, K = 4096 (kSpw = 2, 8
// slices): 128 KiB of bf16 slab, 64 KiB of weights, 64 KiB of partials,
// against 528 KiB of activations + 64 KiB of weights per workgroup when each
// owns 16 rows over the whole K.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;

}  // namespace

template <int kSpw, int kMG>
struct SlabLds {
  static constexpr int kSK = 2 * kSpw;                // 128-K steps per workgroup
  static constexpr int kRows = 16 * kMG;              // slab rows (M rounded up to 16)
  static constexpr int kChunksRow = kSK * 16;         // 16-byte bf16 chunks per slab row
  static constexpr int kPitch = kSK * 128 + 16;       // E4M3 bytes per staged row (+16: rows on distinct banks)
  static constexpr int kScaleRow = kSK * 4;           // UE8M0 bytes per staged row
  static constexpr int kSlab = kRows * kPitch + kRows * kScaleRow;
  static constexpr int kRed = 8 * kMG * 64 * 16;      // one half's partial sums [8 bands][kMG][64 lanes] x 16 B
  static constexpr int kBytes = kSlab > kRed ? kSlab : kRed;
  static constexpr int kLoads = (kRows * kChunksRow + kThreads - 1) / kThreads;   // 16-byte loads per thread
};

// x: bf16 [M, K] (row stride ldx elements); wp, sp: the packed weight (G
// groups of 128 rows; kFp4: packed MXFP4, one 1 KiB piece per band and
// 128-K step); part: fp32 [K / (128 kSK)][M][ldp], ldp = 128 G.
template <bool kFp4, int kSpw, int kMG>
__global__ __launch_bounds__(kThreads) void gemm_slab_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                             int K, const uint8_t* __restrict__ wp,
                                                             const uint8_t* __restrict__ sp, int G,
                                                             float* __restrict__ part, int64_t ldp) {
  using L = SlabLds<kSpw, kMG>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* xq = smem;                          // slab rows, E4M3
  uint8_t* xs = smem + L::kRows * L::kPitch;   // their scales
  v4f* red = reinterpret_cast<v4f*>(smem);     // reused for the partial sums after the MFMAs

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  // Work item = slice * G + group; a die takes a contiguous run of items,
  // i.e. whole slices when G is a multiple of the workgroups per die.
  const int item = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int slice = item / G, grp = item - slice * G;
  const int s0 = slice * L::kSK;               // first 128-K step of the slice
  const int KTs = K / kStepK;                          // packed scale tiles along K
  const int KTw = kFp4 ? K / 128 : K / kStepK;         // packed weight tiles along K

  // 1. The slab: rows [0, M), K [128 s0, 128 (s0 + kSK)), chunk c = tid +
  // 1024 j is 16 bytes of row c / kChunksRow.  Rows are a multiple of four
  // chunks, so the four lanes of a quad hold one 32-block (or are all past
  // the last row).
  const int total = M * L::kChunksRow;
  const uint16_t* xsl = x + (size_t)s0 * 128;
  uint4 xa[L::kLoads];
#pragma unroll
  for (int j = 0; j < L::kLoads; ++j) {
    xa[j] = make_uint4(0u, 0u, 0u, 0u);
    const int c = tid + kThreads * j;
    if (c < total) {
      const int row = c / L::kChunksRow, col = c % L::kChunksRow;
      xa[j] = *reinterpret_cast<const uint4*>(xsl + (size_t)row * ldx + col * 8);
    }
  }

  // 2. Weight loads: wave (band b, half h) takes steps s0 + h kSpw + u of
  // rows 16 b .. 16 b + 15 of the group: E4M3 pieces 2 ks and 2 ks + 1 of the
  // band, chunk g of row r (the band is one contiguous run along K); E2M1
  // (kFp4) piece ks, chunk g = K [32g, 32g + 32) of the step.  Block 4 ks + g
  // of this lane is block g & 1 of scale tile 2 ks + g / 2.
  const int b = wave & 7, h = wave >> 3;
  const int r = 16 * b + i;
  const uint8_t* wrow = wp + (size_t)grp * KTw * kTileBytes + packed_off(r, 0, g, KTw);
  const uint8_t* srow = sp + (size_t)grp * KTs * kTileScaleBytes + scale_off(r, g & 1);
  uint4 w0[kSpw], w1[kSpw];
  uint32_t wsd[kSpw];
#pragma unroll
  for (int u = 0; u < kSpw; ++u) {
    const int ks = s0 + h * kSpw + u;
    if constexpr (kFp4) {
      w0[u] = *reinterpret_cast<const uint4*>(wrow + (size_t)ks * kPieceBytes);
      w1[u] = make_uint4(0u, 0u, 0u, 0u);   // an E2M1 operand uses four registers
    } else {
      const uint8_t* wt = wrow + (size_t)(2 * ks) * kPieceBytes;
      w0[u] = *reinterpret_cast<const uint4*>(wt);
      w1[u] = *reinterpret_cast<const uint4*>(wt + kPieceBytes);
    }
    wsd[u] = srow[(size_t)(2 * ks + (g >> 1)) * kTileScaleBytes];
  }
  // Every load above this point: the scheduler would otherwise start the
  // first conversion (and its wait) before the last weight loads issue.
  __builtin_amdgcn_sched_barrier(0);

  // 3. Quantize the slab into LDS: amax of a 32-block over its quad by two
  // DPP exchanges, scale byte by the MX rule, elements through the scaled
  // converter (saturating at +-448).
#pragma unroll
  for (int j = 0; j < L::kLoads; ++j) {
    const int c = tid + kThreads * j;
    if (c < total) {
      const int row = c / L::kChunksRow, col = c % L::kChunksRow;
      const uint32_t wv[4] = {xa[j].x, xa[j].y, xa[j].z, xa[j].w};
      u16x2 m = {0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) m = absmax_pk(m, wv[e]);
      uint32_t mm = max((uint32_t)m[0], (uint32_t)m[1]);
      mm = max(mm, (uint32_t)__builtin_amdgcn_mov_dpp((int)mm, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
      mm = max(mm, (uint32_t)__builtin_amdgcn_mov_dpp((int)mm, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
      const uint32_t sb = (uint32_t)max((int)(mm >> 7) - 8, 0);
      uint32_t qv[2];
      cvt8s(wv, mx_scale_value(sb), qv);
      *reinterpret_cast<uint2*>(xq + row * L::kPitch + col * 8) = make_uint2(qv[0], qv[1]);
      if ((lane & 3) == 0) xs[row * L::kScaleRow + col / 4] = (uint8_t)sb;
    }
  }
  __syncthreads();

  // 4. MFMAs: lane (i, g) of row group mg takes slab row 16 mg + i (rows
  // past M repeat row M - 1; their outputs are dropped), K [16g, 16g+16) and
  // [64+16g, 64+16g+16) of the step, and the scale of block g.
  v4f acc[kMG];
#pragma unroll
  for (int mg = 0; mg < kMG; ++mg) acc[mg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < kSpw; ++u) {
    const v8i wa{(int)w0[u].x, (int)w0[u].y, (int)w0[u].z, (int)w0[u].w,
                 (int)w1[u].x, (int)w1[u].y, (int)w1[u].z, (int)w1[u].w};
    const int sl = h * kSpw + u;   // step inside the slab
#pragma unroll
    for (int mg = 0; mg < kMG; ++mg) {
      const int row = min(16 * mg + i, M - 1);
      const uint8_t* p = xq + row * L::kPitch + sl * 128 + 16 * g;
      const uint4 b0 = *reinterpret_cast<const uint4*>(p);
      const uint4 b1 = *reinterpret_cast<const uint4*>(p + 64);
      const int xsc = xs[row * L::kScaleRow + sl * 4 + g];
      const v8i xb{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      // A format: 0 = E4M3, 4 = E2M1; B (the activations) E4M3.
      acc[mg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb, acc[mg], kFp4 ? 4 : 0, 0, 0, (int)wsd[u],
                                                                 0, xsc);
    }
  }

  // 5. Add the two halves in K order (the slab is dead: its LDS holds the
  // second half's sums), then store the slice's partial: lane (i, g) of band
  // b, row group mg holds D[n = 16 b + 4 g + e][m = 16 mg + i], e = 0..3.
  __syncthreads();
  if (h == 1) {
#pragma unroll
    for (int mg = 0; mg < kMG; ++mg) red[(b * kMG + mg) * 64 + lane] = acc[mg];
  }
  __syncthreads();
  if (h == 1) return;
  float* pbase = part + (size_t)slice * M * ldp + (size_t)grp * 128 + 16 * b + 4 * g;
#pragma unroll
  for (int mg = 0; mg < kMG; ++mg) {
    const v4f s = acc[mg] + red[(b * kMG + mg) * 64 + lane];
    const int m = 16 * mg + i;
    if (m < M) *reinterpret_cast<float4*>(pbase + (size_t)m * ldp) = make_float4(s[0], s[1], s[2], s[3]);
  }
}

namespace {

template <bool kFp4, int kSpw, int kMG>
int launch_slab_k(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int G,
                  int slices, float* part, int64_t ldp, hipStream_t stream) {
  constexpr int lds = SlabLds<kSpw, kMG>::kBytes;
  static std::atomic<int> lds_set[kMaxDevices];
  if (!set_lds_limit_once((const void*)gemm_slab_kernel<kFp4, kSpw, kMG>, lds, lds_set)) return -7;
  hipLaunchKernelGGL((gemm_slab_kernel<kFp4, kSpw, kMG>), dim3((unsigned)(G * slices)), dim3(kThreads), lds, stream,
                     (const uint16_t*)x, ldx, (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)sp, G, part, ldp);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

template <bool kFp4, int kSpw>
int launch_slab_s(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int G,
                  int slices, float* part, int64_t ldp, hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return launch_slab_k<kFp4, kSpw, 1>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    case 2: return launch_slab_k<kFp4, kSpw, 2>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    case 3: return launch_slab_k<kFp4, kSpw, 3>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    case 4: return launch_slab_k<kFp4, kSpw, 4>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    case 5: return launch_slab_k<kFp4, kSpw, 5>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    case 6: return launch_slab_k<kFp4, kSpw, 6>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    case 7: return launch_slab_k<kFp4, kSpw, 7>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    case 8: return launch_slab_k<kFp4, kSpw, 8>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
    default: return -2;
  }
}

}  // namespace

namespace {
template <bool kFp4>
int launch_slab(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  const int spw = slab_steps_per_wave(N, K);
  const int G = (int)((N + 127) / 128);
  const int slices = (int)((K / 128) / (2 * spw));
  const int64_t ldp = (int64_t)G * 128;
  float* part = (float*)ws;
  int st = -2;
  if (spw == 4) st = launch_slab_s<kFp4, 4>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
  if (spw == 2) st = launch_slab_s<kFp4, 2>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
  if (spw == 1) st = launch_slab_s<kFp4, 1>(x, ldx, M, K, wp, sp, G, slices, part, ldp, stream);
  if (st) return st;
  return launch_splitk_reduce(part, slices, M, N, ldp, bias, y, ldy, stream);
}
}  // namespace

int launch_gemm_slab(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                     const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  return launch_slab<false>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream, ws);
}

int launch_gemm_slab_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                         int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  return launch_slab<true>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream, ws);
}

}  // namespace mxfp8
