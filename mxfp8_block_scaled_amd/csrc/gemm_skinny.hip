// Skinny (decode-shaped, M <= 16) MXFP8 linear layer in one kernel, with the
// activation quantization fused in.
//
// At M <= 16 the layer streams the whole packed weight once (N*K bytes plus
// 1/32 of that in scales): it is bound by HBM bandwidth and by how many
// requests are in flight.  One workgroup owns 16 weight rows over the whole K;
// each of its 16 waves owns a run of 128-deep K steps (a K slice) and works
// on its own, with no workgroup barrier before the final reduction:
//  1. it loads the bf16 activations of its slice, M rows, coalesced, then
//     issues the weight loads of the same steps.  Loads return in issue
//     order, so the activations (L2 hits after the first workgroup) arrive
//     first and are converted while the weight stream is still in flight;
//  2. it quantizes the slice by the MX rule (four lanes per 32-block, amax by
//     two quad exchanges, gfx950's scaled converter) into its own LDS rows;
//  3. it reads its MFMA operands back from those rows and runs one
//     v_mfma_scale_f32_16x16x128_f8f6f4 per step (weight rows as the A
//     operand, activation rows as B);
//  4. the 16 per-wave partial sums are reduced through LDS in K order; wave 0
//     adds the bias and writes bf16.
// Each activation element is loaded and converted once per workgroup, by the
// one wave whose slice holds it; no quantized copy is written to memory and
// no second launch is needed at any M.
// Operand bytes of lane (i, g) of the MFMA (common.hpp): K [16g, 16g+16) and
// [64+16g, 64+16g+16) of the step; the scale of MX block b comes from lane
// group b.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;

}  // namespace

// kSteps: the most K steps one wave owns (K <= 16 * kSteps * 128).
template <int kSteps>
struct SkinnyLds {
  static constexpr int kChunksRow = kSteps * 16;    // 16-byte bf16 chunks per row of a wave's K slice
  static constexpr int kPitch = kSteps * 128 + 16;  // E4M3 bytes per staged row (+16: rows on distinct banks)
  static constexpr int kScaleRow = kSteps * 4;      // UE8M0 bytes per staged row
  static constexpr int kWave = 16 * kPitch + 16 * kScaleRow;
  static constexpr int kRed = kWaves * 64 * 16;     // partial sums [16 waves][64 lanes] x 16 bytes
  static constexpr int kBytes = kRed + kWaves * kWave;
};

template <bool kFp4, int kSteps>
__global__ __launch_bounds__(kThreads) void gemm_skinny_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K, const uint8_t* __restrict__ wp,
    const uint8_t* __restrict__ sp, int N, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t ldy, int vec_store) {
  using L = SkinnyLds<kSteps>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  v4f* red = reinterpret_cast<v4f*>(smem);
  uint8_t* xq = smem + L::kRed + wave * L::kWave;   // this wave's staged E4M3 rows
  uint8_t* xs = xq + 16 * L::kPitch;                // and their scales
  // Dies take contiguous runs of 16-row blocks (whole 128-row groups of the
  // packed weight per die: measured 6 % faster than the dispatch order).
  const int n0 = xcd_remap((int)blockIdx.x, (int)gridDim.x) * 16;
  const int grp = n0 / kGroupRows;
  const int r = (n0 % kGroupRows) + i;
  const int KTs = K / kStepK;                      // packed scale tiles along K
  const int KTw = kFp4 ? K / 128 : K / kStepK;     // packed weight tiles along K
  const int KS = K / 128;                          // MFMA steps along K
  const int kb = (KS * wave) / kWaves, nsteps = (KS * (wave + 1)) / kWaves - kb;
  // Steps past the wave's run reload its last valid step (never used), so
  // the loads need no branch on the step count.
  int ks_of[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) ks_of[u] = min(kb + u, KS - 1);

  // 1. Wave 0's bias values (columns n0 + 4g .. + 3, index clamped to N - 1;
  // those past N are never stored), issued first so their latency hides
  // under the weight stream.  The loads are unconditional buffer loads, so
  // they sit above the scheduling barrier below and cannot be sunk into the
  // epilogue, where each would cost a full memory latency; for the other
  // waves (and a null bias) the buffer is empty and they return 0 without a
  // memory access.  They are ordinary compiler-tracked loads: the
  // compiler's own wait covers their first use.
  const bool has_bias = bias != nullptr;
  const __amdgpu_buffer_rsrc_t brsrc = raw_rsrc(bias, (has_bias && wave == 0) ? (uint32_t)N * 2u : 0u);
  uint32_t braw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    braw[e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(brsrc, (uint32_t)min(n0 + 4 * g + e, N - 1) * 2u, 0, 0);

  // 2. The wave's activation slice, coalesced: M rows x kSteps steps of bf16,
  // chunk c = lane + 64 q is 16 bytes of row c / kChunksRow.  Loads return in
  // issue order, so these (L2 hits after the first workgroup) are converted
  // while the weight stream issued next is still in flight.
  const int total = M * L::kChunksRow;
  uint4 xa[kSteps * 4];
#pragma unroll
  for (int q = 0; q < kSteps * 4; ++q) {
    xa[q] = make_uint4(0u, 0u, 0u, 0u);
    const int c = lane + 64 * q;
    if (c < total) {
      const int row = c / L::kChunksRow, col = c % L::kChunksRow;
      xa[q] = *reinterpret_cast<const uint4*>(x + (size_t)row * ldx + (size_t)ks_of[col / 16] * 128 + (col % 16) * 8);
    }
  }

  // 3. Weight loads of the wave's steps: E4M3, pieces 2ks and 2ks+1 of the
  // workgroup's 16-row band, chunk g of row r; E2M1 (kFp4), piece ks, chunk
  // g = K [32g, 32g + 32) of the step (16 bytes either way).  The band is one
  // contiguous run over K, so the workgroup streams one 64 KiB run (at
  // K = 4096).  This lane's block 4ks + g is block g & 1 of scale tile
  // 2ks + g/2.
  const uint8_t* wrow = wp + (size_t)grp * KTw * kTileBytes + packed_off(r, 0, g, KTw);
  const uint8_t* srow = sp + (size_t)grp * KTs * kTileScaleBytes + scale_off(r, g & 1);
  uint4 w0[kSteps], w1[kSteps];
  uint32_t wsd[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const int ks = ks_of[u];
    if constexpr (kFp4) {
      w0[u] = *reinterpret_cast<const uint4*>(wrow + (size_t)ks * kPieceBytes);
    } else {
      const uint8_t* wt = wrow + (size_t)(2 * ks) * kPieceBytes;
      w0[u] = *reinterpret_cast<const uint4*>(wt);
      w1[u] = *reinterpret_cast<const uint4*>(wt + kPieceBytes);
    }
    wsd[u] = srow[(size_t)(2 * ks + (g >> 1)) * kTileScaleBytes];
  }
  // Keep every load above this point: the scheduler would otherwise start
  // the first conversion (and its wait) before the last weight loads issue.
  __builtin_amdgcn_sched_barrier(0);

  // 4. Quantize the slice into the wave's LDS rows: four lanes per 32-block
  // (chunks 4j..4j+3 of a row), amax over their 32 elements by two lane
  // exchanges, scale byte by the MX rule, elements through gfx950's scaled
  // converter.  total is a multiple of 16, so a four-lane group is either
  // all in range or all zeros (those write rows >= M, which are never read).
#pragma unroll
  for (int q = 0; q < kSteps * 4; ++q) {
    if (64 * q < total) {
      const int c = lane + 64 * q;
      const int row = c / L::kChunksRow, col = c % L::kChunksRow;
      const uint32_t wv[4] = {xa[q].x, xa[q].y, xa[q].z, xa[q].w};
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
  // The wave reads back what it wrote: LDS executes one wave's accesses in
  // order; this keeps the compiler from moving the reads above the writes.
  asm volatile("" ::: "memory");

  // 5. Operands: lane (i, g) takes row i (lanes i >= M repeat row M - 1; their
  // outputs are dropped), K [16g, 16g+16) and [64+16g, 64+16g+16) of each
  // step and the scale of block g.  A step past the wave's run gets zero
  // activation bytes (E4M3 +0): it adds exactly nothing.
  const int rr = min(i, M - 1);
  v8i xb[kSteps];
  int xscale[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const uint8_t* p = xq + rr * L::kPitch + u * 128 + 16 * g;
    const uint4 b0 = *reinterpret_cast<const uint4*>(p);
    const uint4 b1 = *reinterpret_cast<const uint4*>(p + 64);
    xscale[u] = xs[rr * L::kScaleRow + u * 4 + g];
    xb[u] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    if (u >= nsteps) xb[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // 6. One MFMA per step (weight rows as the A operand, activations as B).
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    v8i wa;
    wa[0] = (int)w0[u].x; wa[1] = (int)w0[u].y; wa[2] = (int)w0[u].z; wa[3] = (int)w0[u].w;
    if constexpr (kFp4) {
      wa[4] = 0; wa[5] = 0; wa[6] = 0; wa[7] = 0;   // an E2M1 operand uses four registers
    } else {
      wa[4] = (int)w1[u].x; wa[5] = (int)w1[u].y; wa[6] = (int)w1[u].z; wa[7] = (int)w1[u].w;
    }
    // A format: 0 = E4M3, 4 = E2M1; B (activations) E4M3.
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb[u], acc, kFp4 ? 4 : 0, 0, 0, (int)wsd[u], 0,
                                                           xscale[u]);
  }

  // 7. Reduce the partial sums in K order; lane (i, g) of wave 0 holds
  // D[n = 4g + j][m = i], j = 0..3.
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  v4f part[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) part[w] = red[w * 64 + lane];
  __builtin_amdgcn_sched_barrier(0);   // all 16 reads in flight before the first add
  acc = part[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) acc += part[w];
  if (i >= M) return;
  const int n = n0 + 4 * g;
  if (n >= N) return;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = acc[e] + __uint_as_float(braw[e] << 16);
  uint16_t* yrow = y + (size_t)i * ldy;
  const uint32_t lo = pack_bf16x2(v[0], v[1]);
  const uint32_t hi = pack_bf16x2(v[2], v[3]);
  if (vec_store && n + 3 < N) {
    *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
  } else {
    yrow[n] = (uint16_t)lo;
    if (n + 1 < N) yrow[n + 1] = (uint16_t)(lo >> 16);
    if (n + 2 < N) yrow[n + 2] = (uint16_t)hi;
    if (n + 3 < N) yrow[n + 3] = (uint16_t)(hi >> 16);
  }
}

namespace {
template <bool kFp4, int kSteps>
int launch_skinny_k(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                    const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  constexpr int lds = SkinnyLds<kSteps>::kBytes;
  static std::atomic<int> lds_set[kMaxDevices];
  if (!set_lds_limit_once((const void*)gemm_skinny_kernel<kFp4, kSteps>, lds, lds_set)) return -7;
  const int blocks = (int)((N + 15) / 16);
  const int vec = (ldy % 4 == 0) && (((uintptr_t)y & 7) == 0);
  hipLaunchKernelGGL((gemm_skinny_kernel<kFp4, kSteps>), dim3(blocks), dim3(kThreads), lds, stream,
                     (const uint16_t*)x, ldx, (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)sp, (int)N,
                     (const uint16_t*)bias, (uint16_t*)y, ldy, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

template <bool kFp4>
int launch_skinny(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                  const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  static_assert(kSkinnyMaxK <= kWaves * 4 * 128, "a wave owns at most four K steps");
  if (K <= kWaves * 2 * 128) return launch_skinny_k<kFp4, 2>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream);
  return launch_skinny_k<kFp4, 4>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream);
}
}  // namespace

int launch_gemm_skinny(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                       int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  (void)ws;
  return launch_skinny<false>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream);
}

int launch_gemm_skinny_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                           int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  (void)ws;
  return launch_skinny<true>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream);
}

}  // namespace mxfp8
