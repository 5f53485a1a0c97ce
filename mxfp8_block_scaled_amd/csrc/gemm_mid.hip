// Mid-M (16 < M <= 128) MXFP8 linear layer: the decode kernel's structure
// carried to a few hundred activation rows.
//
// The weight still streams once (N*K bytes plus scales) and dominates the
// HBM traffic up to M = 128; what grows with M is the activation traffic.
// One workgroup owns 16 weight rows over the whole K, each of its 16 waves a
// run of 128-deep K steps (as in the decode kernel), and keeps its weight
// fragments in registers while it walks the activation rows in groups of 16:
//  1. the activations are quantized once, beforehand, into the packed
//     operand layout (one 128-row group, pad rows zero), so each workgroup
//     reads 1.03 bytes per activation element from L2 instead of 2 and
//     converts nothing;
//  2. every wave issues its weight loads, then a ring of activation operand
//     loads (row 16 mg + i, K [16g, 16g+16) and [64+16g, 64+16g+16) of a step,
//     and the scale of block g), refilled behind each MFMA.  In the packed
//     layout each of those loads is one whole 1 KiB piece (the same
//     addressing as the weight's), where row-major rows would spread a load
//     over 16 cache lines and use half of each (measured 2.7 us per 16 rows);
//  3. one v_mfma_scale_f32_16x16x128_f8f6f4 per (row group, step), the
//     weight as the A operand, into one accumulator per row group;
//  4. the 16 waves' partial sums are reduced through LDS in K order, wave mg
//     reducing row group mg; bias in fp32, one rounding to bf16.
// Every workgroup reads the whole quantized activation (L2 hits after the
// first ones): at M = 128 that is 8 times the workgroup's weight bytes and
// what bounds the kernel; the large-tile GEMM takes over above M = 128.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;

}  // namespace

// kFp4: packed MXFP4 weight (E2M1 A operand); kSteps: the most K steps one
// wave owns (K <= 16 * kSteps * 128); kMG: 16-row activation groups
// (M <= 16 * kMG <= 128).  xp, xsp: the packed activations (group 0).
// LDS: partial sums [kMG][16 waves][64 lanes] x 16 bytes.
template <bool kFp4, int kSteps, int kMG>
__global__ __launch_bounds__(kThreads) void gemm_mid_kernel(
    const uint8_t* __restrict__ xp, const uint8_t* __restrict__ xsp, int M, int K, const uint8_t* __restrict__ wp,
    const uint8_t* __restrict__ sp, int N, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t ldy, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  v4f* red = reinterpret_cast<v4f*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int n0 = xcd_remap((int)blockIdx.x, (int)gridDim.x) * 16;
  const int grp = n0 / kGroupRows;
  const int r = (n0 % kGroupRows) + i;
  const int KTs = K / kStepK;                      // packed scale tiles along K
  const int KTw = kFp4 ? K / 128 : K / kStepK;     // packed weight tiles along K
  const int KS = K / 128;                          // MFMA steps along K
  const int kb = (KS * wave) / kWaves, nsteps = (KS * (wave + 1)) / kWaves - kb;
  // Steps past the wave's run reload its last valid step (never used), so
  // no load needs a branch.
  int ks_of[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) ks_of[u] = min(kb + u, KS - 1);

  // 1. The reducing waves' bias values (columns n0 + 4g .. + 3, index clamped
  // to N - 1; those past N are never stored), issued first as unconditional
  // buffer loads (above the scheduling barrier below, so the compiler cannot
  // sink them into the epilogue); the other waves' buffer is empty and reads
  // zeros without a memory access.  Compiler-tracked: its own wait covers
  // the first use.
  const bool has_bias = bias != nullptr;
  const __amdgpu_buffer_rsrc_t brsrc = raw_rsrc(bias, (has_bias && wave < kMG) ? (uint32_t)N * 2u : 0u);
  uint32_t braw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    braw[e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(brsrc, (uint32_t)min(n0 + 4 * g + e, N - 1) * 2u, 0, 0);

  // 2. Weight loads of the wave's steps (the decode kernel's addressing):
  // E4M3 pieces 2ks and 2ks+1 of the workgroup's 16-row band, chunk g of row
  // r; E2M1 (kFp4) piece ks, chunk g.  Block 4ks + g of this lane is block
  // g & 1 of scale tile 2ks + g/2.
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

  // 3. Activation operands: unit j = (row group j / kSteps, step j % kSteps),
  // kRing of them in flight.  Rows past M are the layout's zero pad rows
  // (their outputs are dropped).
  constexpr int kUnits = kMG * kSteps;
  constexpr int kRingMax = kSteps == 2 ? 5 : 3;   // what fits the registers
  constexpr int kRing = kUnits < kRingMax ? kUnits : kRingMax;
  uint4 a0[kRing], a1[kRing];
  uint32_t asc[kRing];
  auto load_unit = [&](int j, int slot) {
    const int row = 16 * (j / kSteps) + i;
    const int ks = ks_of[j % kSteps];
    const uint8_t* p = xp + packed_off(row, 2 * ks, g, KTs);
    a0[slot] = *reinterpret_cast<const uint4*>(p);
    a1[slot] = *reinterpret_cast<const uint4*>(p + kPieceBytes);
    asc[slot] = xsp[(size_t)(2 * ks + (g >> 1)) * kTileScaleBytes + scale_off(row, g & 1)];
  };
#pragma unroll
  for (int j = 0; j < kRing; ++j) load_unit(j, j);
  __builtin_amdgcn_sched_barrier(0);

  v8i wa[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    wa[u][0] = (int)w0[u].x; wa[u][1] = (int)w0[u].y; wa[u][2] = (int)w0[u].z; wa[u][3] = (int)w0[u].w;
    if constexpr (kFp4) {
      wa[u][4] = 0; wa[u][5] = 0; wa[u][6] = 0; wa[u][7] = 0;   // an E2M1 operand uses four registers
    } else {
      wa[u][4] = (int)w1[u].x; wa[u][5] = (int)w1[u].y; wa[u][6] = (int)w1[u].z; wa[u][7] = (int)w1[u].w;
    }
  }
  v4f acc[kMG];
#pragma unroll
  for (int mg = 0; mg < kMG; ++mg) acc[mg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const int slot = j % kRing, mg = j / kSteps, u = j % kSteps;
    v8i xb{(int)a0[slot].x, (int)a0[slot].y, (int)a0[slot].z, (int)a0[slot].w,
           (int)a1[slot].x, (int)a1[slot].y, (int)a1[slot].z, (int)a1[slot].w};
    // A step past the wave's run adds nothing: zero activation bytes (+0).
    if (u >= nsteps) xb = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    // A format: 0 = E4M3, 4 = E2M1; B (activations) E4M3.
    acc[mg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[u], xb, acc[mg], kFp4 ? 4 : 0, 0, 0,
                                                               (int)wsd[u], 0, (int)asc[slot]);
    if (j + kRing < kUnits) load_unit(j + kRing, slot);
    // Keep the ring's order: the scheduler would otherwise hoist later MFMAs
    // (independent accumulators) above this refill and wait on it at once.
    __builtin_amdgcn_sched_barrier(0);
  }

  // 4. Reduce: wave mg sums row group mg's 16 partials in K order; lane
  // (i, g) then holds D[n = 4g + e][m = 16 mg + i], e = 0..3.
#pragma unroll
  for (int mg = 0; mg < kMG; ++mg) red[(mg * kWaves + wave) * 64 + lane] = acc[mg];
  __syncthreads();
  if (wave >= kMG) return;
  const int mg = wave;
  v4f part[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) part[w] = red[(mg * kWaves + w) * 64 + lane];
  __builtin_amdgcn_sched_barrier(0);   // all 16 reads in flight before the first add
  v4f s = part[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) s += part[w];
  const int m = 16 * mg + i;
  const int n = n0 + 4 * g;
  if (m >= M || n >= N) return;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = s[e] + __uint_as_float(braw[e] << 16);
  uint16_t* yrow = y + (size_t)m * ldy;
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
template <bool kFp4, int kSteps, int kMG>
int launch_mid_k(const uint8_t* xp, const uint8_t* xsp, int64_t M, int64_t K, const void* wp, const void* sp,
                 int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  constexpr int lds = kMG * kWaves * 64 * 16;
  static std::atomic<int> lds_set[kMaxDevices];
  if (!set_lds_limit_once((const void*)gemm_mid_kernel<kFp4, kSteps, kMG>, lds, lds_set)) return -7;
  const int blocks = (int)((N + 15) / 16);
  const int vec = (ldy % 4 == 0) && (((uintptr_t)y & 7) == 0);
  hipLaunchKernelGGL((gemm_mid_kernel<kFp4, kSteps, kMG>), dim3(blocks), dim3(kThreads), lds, stream, xp, xsp,
                     (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)sp, (int)N, (const uint16_t*)bias,
                     (uint16_t*)y, ldy, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

template <bool kFp4, int kSteps>
int launch_mid_s(const uint8_t* xp, const uint8_t* xsp, int64_t M, int64_t K, const void* wp, const void* sp,
                 int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return launch_mid_k<kFp4, kSteps, 1>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    case 2: return launch_mid_k<kFp4, kSteps, 2>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    case 3: return launch_mid_k<kFp4, kSteps, 3>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    case 4: return launch_mid_k<kFp4, kSteps, 4>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    case 5: return launch_mid_k<kFp4, kSteps, 5>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    case 6: return launch_mid_k<kFp4, kSteps, 6>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    case 7: return launch_mid_k<kFp4, kSteps, 7>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    case 8: return launch_mid_k<kFp4, kSteps, 8>(xp, xsp, M, K, wp, sp, N, bias, y, ldy, stream);
    default: return -2;
  }
}

template <bool kFp4>
int launch_mid(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
               const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  static_assert(kMidMaxM <= 16 * 8 && kSkinnyMaxK <= kWaves * 4 * 128, "row groups and steps per wave");
  // ws: the packed activations of one 128-row group, E4M3 tiles then scale
  // tiles (mid_ws_bytes).
  uint8_t* q = (uint8_t*)ws;
  uint8_t* s = q + (size_t)kGroupRows * K;
  if (int st = launch_quantize_act_packed(x, M, K, ldx, q, s, stream)) return st;
  if (K <= kWaves * 2 * 128) return launch_mid_s<kFp4, 2>(q, s, M, K, wp, sp, N, bias, y, ldy, stream);
  return launch_mid_s<kFp4, 4>(q, s, M, K, wp, sp, N, bias, y, ldy, stream);
}
}  // namespace

int launch_gemm_mid(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                    const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  return launch_mid<false>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream, ws);
}

int launch_gemm_mid_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                        int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws) {
  return launch_mid<true>(x, ldx, M, K, wp, sp, N, bias, y, ldy, stream, ws);
}

}  // namespace mxfp8
