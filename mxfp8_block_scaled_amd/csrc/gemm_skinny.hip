// Skinny (decode-shaped, M <= 16) MXFP8 linear layer in one kernel, with the
// activation quantization fused in.
//
// At M <= 16 the layer streams the whole packed weight once (N*K bytes plus
// 1/32 of that in scales): it is bound by HBM bandwidth and by how many
// requests are in flight.  One workgroup owns 16 weight rows over the whole K:
//  1. each of its 16 waves first issues the loads of its share of those rows
//     (one 128-deep K step = 2 x 16 bytes per lane), so the HBM latency runs
//     while the rest of the prologue works;
//  2. the workgroup quantizes the M real activation rows (M x K bf16, read
//     from L2) once, cooperatively, into LDS -- E4M3 bytes and UE8M0 scales
//     by the MX rule, with gfx950's scaled converter.  From kSkinnyPreqM rows
//     on, every workgroup converting the same M x K activations costs more
//     than one extra launch: the row-major quantizer (quant.hip) runs first
//     and the workgroups copy its bytes instead (kPreq);
//  3. each wave runs one v_mfma_scale_f32_16x16x128_f8f6f4 per K step
//     (weight rows as the A operand, activation rows as B, from LDS);
//  4. the 16 per-wave partial sums are reduced through LDS; wave 0 adds the
//     bias and writes bf16.
// Operand bytes of lane (i, g) of the MFMA (common.hpp): K [16g, 16g+16) and
// [64+16g, 64+16g+16) of the step; the scale of MX block b comes from lane
// group b.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSteps = 4;   // K steps per wave: K <= 16 * 4 * 128 = 8192
constexpr int kBatch = 8;      // activation chunks in flight per thread

}  // namespace

// LDS: activations [16][K + 16] E4M3 bytes (row pitch K + 16 puts the 16
// rows' fragment reads on distinct banks), scales [16][K/32], partial sums
// [16 waves][64 lanes] x 16 bytes.
template <bool kPreq, bool kFp4>
__global__ __launch_bounds__(kThreads) void gemm_skinny_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K, const uint8_t* __restrict__ wp,
    const uint8_t* __restrict__ sp, int N, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t ldy, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int pitch = K + 16;
  uint8_t* xq = smem;
  uint8_t* xs = smem + 16 * pitch;
  v4f* red = reinterpret_cast<v4f*>(xs + 16 * (K / 32));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  // Dies take contiguous runs of 16-row blocks (whole 128-row groups of the
  // packed weight per die: measured 6 % faster than the dispatch order).
  const int n0 = xcd_remap((int)blockIdx.x, (int)gridDim.x) * 16;
  const int grp = n0 / kGroupRows;
  const int r = (n0 % kGroupRows) + i;
  const int KTs = K / kStepK;                      // packed scale tiles along K
  const int KTw = kFp4 ? K / 128 : K / kStepK;     // packed weight tiles along K
  const int KS = K / 128;                          // MFMA steps along K
  const int kb = (KS * wave) / kWaves, ke = (KS * (wave + 1)) / kWaves;

  // 1. Weight loads for this wave's steps: E4M3, pieces 2ks and 2ks+1 of the
  // workgroup's 16-row band, chunk g of row r; E2M1 (kFp4), piece ks, chunk
  // g = K [32g, 32g + 32) of the step (16 bytes either way).  The band is one
  // contiguous run over K, so the workgroup streams one 64 KiB run (at
  // K = 4096).  This lane's block 4ks + g is block g & 1 of scale tile
  // 2ks + g/2.
  const uint8_t* wrow = wp + (size_t)grp * KTw * kTileBytes + packed_off(r, 0, g, KTw);
  const uint8_t* srow = sp + (size_t)grp * KTs * kTileScaleBytes + scale_off(r, g & 1);
  uint4 w0[kMaxSteps], w1[kMaxSteps];
  uint32_t wsd[kMaxSteps];
#pragma unroll
  for (int u = 0; u < kMaxSteps; ++u) {
    if (kb + u < ke) {
      if constexpr (kFp4) {
        w0[u] = *reinterpret_cast<const uint4*>(wrow + (size_t)(kb + u) * kPieceBytes);
      } else {
        const uint8_t* wt = wrow + (size_t)(2 * (kb + u)) * kPieceBytes;
        w0[u] = *reinterpret_cast<const uint4*>(wt);
        w1[u] = *reinterpret_cast<const uint4*>(wt + kPieceBytes);
      }
      wsd[u] = srow[(size_t)(2 * (kb + u) + (g >> 1)) * kTileScaleBytes];
    }
  }

  if constexpr (kPreq) {
    // 2'. Copy the quantized activations (E4M3 [M][K], then UE8M0 [M][K/32],
    // both row-major at x) into LDS.
    const uint8_t* xqg = reinterpret_cast<const uint8_t*>(x);
    const uint8_t* xsg = xqg + (size_t)M * K;
    const int per_row16 = K / 16;
    for (int c = tid; c < M * per_row16; c += kThreads) {
      const int row = c / per_row16, col = (c - row * per_row16) * 16;
      *reinterpret_cast<uint4*>(xq + row * pitch + col) = *reinterpret_cast<const uint4*>(xqg + (size_t)row * K + col);
    }
    for (int c = tid; c < M * (K / 128); c += kThreads)
      *reinterpret_cast<uint32_t*>(xs + c * 4) = *reinterpret_cast<const uint32_t*>(xsg + (size_t)c * 4);
  } else {
  // 2. Quantize x[0:M, 0:K] into LDS: four threads per 32-element block,
  // eight elements (16 bytes) each; a thread issues the loads of up to
  // kBatch chunks before converting any, so their L2 latencies overlap.
  const int per_row = K / 8;
  const int chunks = M * per_row;
  for (int c0 = tid; c0 < chunks; c0 += kBatch * kThreads) {
    uint4 v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * kThreads;
      if (c < chunks) {
        const int row = c / per_row, c8 = c - row * per_row;
        v[b] = *reinterpret_cast<const uint4*>(x + (size_t)row * ldx + c8 * 8);
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * kThreads;
      if (c < chunks) {
        const int row = c / per_row, c8 = c - row * per_row;
        const uint32_t wv[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
        u16x2 m = {0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) m = absmax_pk(m, wv[e]);
        uint32_t mm = max((uint32_t)m[0], (uint32_t)m[1]);
        mm = max(mm, (uint32_t)__shfl_xor((int)mm, 1));
        mm = max(mm, (uint32_t)__shfl_xor((int)mm, 2));
        const uint32_t sb = (uint32_t)max((int)(mm >> 7) - 8, 0);
        uint32_t q[2];
        cvt8s(wv, mx_scale_value(sb), q);
        *reinterpret_cast<uint2*>(xq + row * pitch + c8 * 8) = make_uint2(q[0], q[1]);
        if ((c8 & 3) == 0) xs[row * (K / 32) + (c8 >> 2)] = (uint8_t)sb;
      }
    }
  }
  }
  __syncthreads();

  // 3. MFMA steps.  Lanes i >= M use row M-1 (their outputs are dropped).
  const int m = min(i, M - 1);
  const uint8_t* xr = xq + m * pitch + 16 * g;
  const uint8_t* sr = xs + m * (K / 32) + g;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < kMaxSteps; ++u) {
    if (kb + u < ke) {
      const int ks = kb + u;
      const uint4 b0 = *reinterpret_cast<const uint4*>(xr + ks * 128);
      const uint4 b1 = *reinterpret_cast<const uint4*>(xr + ks * 128 + 64);
      const int xscale = sr[ks * 4];
      v8i wa, xb;
      wa[0] = (int)w0[u].x; wa[1] = (int)w0[u].y; wa[2] = (int)w0[u].z; wa[3] = (int)w0[u].w;
      if constexpr (kFp4) {
        wa[4] = 0; wa[5] = 0; wa[6] = 0; wa[7] = 0;   // an E2M1 operand uses four registers
      } else {
        wa[4] = (int)w1[u].x; wa[5] = (int)w1[u].y; wa[6] = (int)w1[u].z; wa[7] = (int)w1[u].w;
      }
      xb[0] = (int)b0.x; xb[1] = (int)b0.y; xb[2] = (int)b0.z; xb[3] = (int)b0.w;
      xb[4] = (int)b1.x; xb[5] = (int)b1.y; xb[6] = (int)b1.z; xb[7] = (int)b1.w;
      const int wscale = (int)wsd[u];
      // A format: 0 = E4M3, 4 = E2M1; B (activations) E4M3.
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb, acc, kFp4 ? 4 : 0, 0, 0, wscale, 0, xscale);
    }
  }

  // 4. Reduce the waves' partial sums; lane (i, g) of wave 0 holds
  // D[n = 4g + j][m = i], j = 0..3.
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) acc += red[w * 64 + lane];
  if (i >= M) return;
  const int n = n0 + 4 * g;
  if (n >= N) return;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = acc[e];
    if (bias != nullptr && n + e < N) v[e] += __uint_as_float((uint32_t)bias[n + e] << 16);
  }
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
template <bool kFp4>
int launch_skinny(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                  const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  const int blocks = (int)((N + 15) / 16);
  const int vec = (ldy % 4 == 0) && (((uintptr_t)y & 7) == 0);
  const size_t lds = (size_t)16 * (K + 16) + (size_t)16 * (K / 32) + (size_t)kWaves * 64 * 16;
  constexpr int kMaxLds = 16 * (kSkinnyMaxK + 16) + 16 * (kSkinnyMaxK / 32) + kWaves * 64 * 16;
  static const bool lds_ok =
      hipFuncSetAttribute((const void*)gemm_skinny_kernel<false, kFp4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kMaxLds) == hipSuccess &&
      hipFuncSetAttribute((const void*)gemm_skinny_kernel<true, kFp4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kMaxLds) == hipSuccess;
  if (!lds_ok) return -7;
  if (M >= kSkinnyPreqM) {
    // ws: E4M3 [M][K] then UE8M0 [M][K/32], row-major (skinny_ws_bytes).
    uint8_t* q = (uint8_t*)ws;
    if (int st = launch_quantize_act(x, M, K, ldx, q, K, q + M * K, K / 32, stream)) return st;
    hipLaunchKernelGGL((gemm_skinny_kernel<true, kFp4>), dim3(blocks), dim3(kThreads), lds, stream,
                       (const uint16_t*)q, K, (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)sp, (int)N,
                       (const uint16_t*)bias, (uint16_t*)y, ldy, vec);
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<false, kFp4>), dim3(blocks), dim3(kThreads), lds, stream,
                       (const uint16_t*)x, ldx, (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)sp, (int)N,
                       (const uint16_t*)bias, (uint16_t*)y, ldy, vec);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
}  // namespace

int launch_gemm_skinny(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                       int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  return launch_skinny<false>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream, ws);
}

int launch_gemm_skinny_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                           int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  return launch_skinny<true>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream, ws);
}

}  // namespace mxfp8
