// Skinny (decode-shaped, M <= 16) MXFP8 linear layer in one kernel: the
// activation quantization is fused into the GEMM's operand load.
//
// At M <= 16 the layer streams the whole packed weight once (N*K bytes + 1/32
// of that in scales) and is bound by HBM bandwidth; the activations are a few
// KiB and stay in L2.  Each workgroup owns 16 weight rows over the whole K;
// its waves split K and each streams its share with independent 16-byte
// loads, quantizing the matching activation blocks in registers, and one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 128-element K step (weight as the A
// operand: 16 n x 16 m).  The per-wave partial sums are reduced through LDS;
// wave 0 adds bias and writes bf16.
//
// Operand bytes of lane (i, g) (common.hpp): K [16g, 16g+16) and
// [64+16g, 64+16g+16) of the step, i.e. halves of MX blocks g/2 and 2+g/2.
// Lanes g and g^1 (lane ^ 16) hold the two halves of the same two blocks and
// combine their block maxima with one exchange.  The MFMA takes the scale of
// block b from lane group b, so groups 1 and 2 swap one scale (lane ^ 48).
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace {

constexpr int kWaves = 8;
constexpr int kUnroll = 4;

struct StepLoads {
  uint4 w0, w1;          // weight operand, two 16-byte halves
  uint32_t wsd;          // the weight row's scale word holding this lane's block
  uint4 x0, x1, x2, x3;  // 32 bf16 activations: 16 at 16g, 16 at 64 + 16g
};

// One 128-deep K step = packed tiles 2ks and 2ks+1.  Lane (i, g) takes chunk g
// of row r from each; its scale (MX block g of the step) is byte g&1 of the
// row's word in tile 2ks + g/2.
__device__ inline void step_load(StepLoads& L, const uint8_t* wrow, int woff, const uint8_t* srow, int g,
                                 const uint16_t* xrow, int ks) {
  const uint8_t* wt = wrow + (size_t)(2 * ks) * kTileBytes + woff;
  L.w0 = *reinterpret_cast<const uint4*>(wt);
  L.w1 = *reinterpret_cast<const uint4*>(wt + kTileBytes);
  L.wsd = (uint32_t)*reinterpret_cast<const uint16_t*>(srow + (size_t)(2 * ks + (g >> 1)) * kTileScaleBytes);
  const uint16_t* xk = xrow + (size_t)ks * 128;
  L.x0 = *reinterpret_cast<const uint4*>(xk);
  L.x1 = *reinterpret_cast<const uint4*>(xk + 8);
  L.x2 = *reinterpret_cast<const uint4*>(xk + 64);
  L.x3 = *reinterpret_cast<const uint4*>(xk + 72);
}

__device__ inline v4f step_compute(const StepLoads& L, int g, v4f acc) {
  const uint32_t h0[8] = {L.x0.x, L.x0.y, L.x0.z, L.x0.w, L.x1.x, L.x1.y, L.x1.z, L.x1.w};
  const uint32_t h1[8] = {L.x2.x, L.x2.y, L.x2.z, L.x2.w, L.x3.x, L.x3.y, L.x3.z, L.x3.w};
  uint32_t m0 = 0, m1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m0 = absmax_bits(m0, h0[i]);
    m1 = absmax_bits(m1, h1[i]);
  }
  m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 16));
  m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 16));
  const uint32_t s0 = mx_scale_byte(m0);  // block g/2
  const uint32_t s1 = mx_scale_byte(m1);  // block 2 + g/2
  // Lane group b must present the scale of block b: group 0 has block 0 (s0),
  // group 3 has block 3 (s1); groups 1 and 2 trade (block 1 lives in groups
  // 2/3 as s0, block 2 in groups 0/1 as s1).
  const uint32_t give = (g >= 2) ? s0 : s1;
  const uint32_t got = (uint32_t)__shfl_xor((int)give, 48);
  const uint32_t xscale = (g == 0) ? s0 : (g == 3) ? s1 : got;
  uint32_t q[8];
  cvt8(h0, mx_inv_scale(s0), q);
  cvt8(h0 + 4, mx_inv_scale(s0), q + 2);
  cvt8(h1, mx_inv_scale(s1), q + 4);
  cvt8(h1 + 4, mx_inv_scale(s1), q + 6);
  v8i xb, wa;
#pragma unroll
  for (int i = 0; i < 8; ++i) xb[i] = (int)q[i];
  wa[0] = (int)L.w0.x; wa[1] = (int)L.w0.y; wa[2] = (int)L.w0.z; wa[3] = (int)L.w0.w;
  wa[4] = (int)L.w1.x; wa[5] = (int)L.w1.y; wa[6] = (int)L.w1.z; wa[7] = (int)L.w1.w;
  const int wscale = (int)(L.wsd >> (8 * (g & 1)));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb, acc, 0, 0, 0, wscale, 0, (int)xscale);
}

}  // namespace

__global__ __launch_bounds__(64 * kWaves) void gemm_skinny_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K, const uint8_t* __restrict__ wp,
    const uint8_t* __restrict__ sp, int N, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t ldy, int vec_store) {
  __shared__ v4f red[kWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int grp = n0 / kGroupRows;
  const int r = (n0 % kGroupRows) + i;
  const int KT = K / kStepK;   // packed tiles along K
  const int KS = K / 128;      // MFMA steps along K

  const uint8_t* wrow = wp + (size_t)grp * KT * kTileBytes;
  const int woff = tile_off(r, g);
  const uint8_t* srow = sp + (size_t)grp * KT * kTileScaleBytes + r * 2;
  const int m = min(i, M - 1);
  const uint16_t* xrow = x + (size_t)m * ldx + 16 * g;

  const int kb = (KS * wave) / kWaves, ke = (KS * (wave + 1)) / kWaves;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int ks = kb;
  for (; ks + kUnroll <= ke; ks += kUnroll) {
    StepLoads L[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) step_load(L[u], wrow, woff, srow, g, xrow, ks + u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc = step_compute(L[u], g, acc);
  }
  for (; ks < ke; ++ks) {
    StepLoads L;
    step_load(L, wrow, woff, srow, g, xrow, ks);
    acc = step_compute(L, g, acc);
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) acc += red[w][lane];
  // Lane (i, g) holds D[n = 4g + j][m = i], j = 0..3.
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

int launch_gemm_skinny(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                       int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  const int blocks = (int)((N + 15) / 16);
  const int vec = (ldy % 4 == 0) && (((uintptr_t)y & 7) == 0);
  hipLaunchKernelGGL(gemm_skinny_kernel, dim3(blocks), dim3(64 * kWaves), 0, stream, (const uint16_t*)x, ldx,
                     (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)sp, (int)N, (const uint16_t*)bias,
                     (uint16_t*)y, ldy, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
