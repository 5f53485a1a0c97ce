// Large-M block-scaled MXFP8 GEMM with the layer's epilogue.
//
//   y[m, n] = bf16( sum_b 2^(sa[m,b]-127) 2^(sw[n,b]-127) sum_{k in b} qa[m,k] qw[n,k] + bias[n] )
//
// (the mm_mxfp8 GEMM of vLLM PR #52204's apply_weights, A[M, K] x B[K, N_pad]
// with both operands K-major, followed by the slice to the logical N and the
// bias add of its §Purpose, folded into one epilogue).
//
// The K loop is tile_core.hpp's 256 x 256 tile on 16x16x128 MFMAs
// (mainloop16).  Here:
//  * Workgroups are dispatched round-robin over the 8 XCDs; the tile index is
//    remapped so that each XCD works on a contiguous, M-grouped range of tiles
//    and its private L2 sees the reuse of weight and activation K-slices.
//  * Epilogue (tile::store16): fp32 staged through LDS, bias added in fp32,
//    one rounding to bf16, 16-byte non-temporal stores covering whole
//    256-byte row segments.
#include "common.hpp"
#include "launch.hpp"
#include "tile_core.hpp"

namespace mxfp8 {

namespace {

using tile::kStage;
using tile::kThreads;
// Tiles along M per group of the tile order: the 32 workgroups of a die then
// share 4 activation and 8 weight tiles at a time (measured against 2, 8 and
// 16: 2 % faster at M = N = K = 4096, 0.7 % on M = 16384 N = 5120 K = 2048,
// the same at M = 8192 N = 28672 K = 8192).
constexpr int kGroupM = 4;

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void gemm_tile_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ qsp, int M, int K,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ wsp, int N, int GN, int GM,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n,
    int vec_store, int splits, float* __restrict__ part, int64_t ldp) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st3[kStage];

  // Split-K: workgroup b takes K slice b % splits of tile b / splits.
  const int split = (int)blockIdx.x % splits;
  // Tile order: XCD-contiguous, then groups of kGroupM tiles along M.
  const int total = tiles_m * tiles_n;
  const int logical = tile::xcd_remap((int)blockIdx.x / splits, total);
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;

  const int KS = K / kStepK;
  const size_t op_stride = (size_t)KS * kTileBytes;     // bytes per 128-row group
  const size_t sc_stride = (size_t)KS * kTileScaleBytes;
  const int wa = min(2 * tn, GN - 1), wb = min(2 * tn + 1, GN - 1);
  const int xa = min(2 * tm, GM - 1), xb = min(2 * tm + 1, GM - 1);

  const int ksl = KS / splits;                           // steps of this slice (multiple of 4)
  // The slice starts at step split * ksl of every band (data) and of the
  // scale tiles; bands stay KS pieces apart.
  const size_t k0 = (size_t)split * ksl * kPieceBytes, s0 = (size_t)split * ksl * kTileScaleBytes;

  v4f acc[8][8];
  tile::mainloop16(st0, st1, st2, st3, wp + wa * op_stride + k0, wp + wb * op_stride + k0, qp + xa * op_stride + k0,
                 qp + xb * op_stride + k0, wsp + wa * sc_stride + s0, wsp + wb * sc_stride + s0,
                 qsp + xa * sc_stride + s0, qsp + xb * sc_stride + s0, ksl, acc, KS);

  if (splits == 1) {
    tile::store16(st0, st1, st2, st3, acc, y, ldy, tm * 256, M, tn * 256, N, bias, vec_store);
  } else {
    // fp32 partial of this slice: part[split][m][n], row stride ldp (% 4 == 0).
    tile::store16(st0, st1, st2, st3, acc, part + (size_t)split * M * ldp, ldp, tm * 256, M, tn * 256, N,
                  (const uint16_t*)nullptr, 1);
  }
}

// The same GEMM as a persistent kernel (no split-K): workgroup w runs tiles
// w, w + G, w + 2G, ... of the same XCD-contiguous, M-grouped order, with the
// copies of each next tile overlapping the end of the current one
// (tile::persistent16).  G is a multiple of 8, so dispatch index i G + w
// lands on the XCD that xcd_remap assigns to it.
__global__ __launch_bounds__(kThreads, 1) void gemm_persistent_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ qsp, int M, int K,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ wsp, int N, int GN, int GM,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n,
    int vec_store) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st3[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t epi[tile::kEpiBytes];
  __shared__ __attribute__((aligned(16))) uint8_t blds[tile::kBiasBytes];

  const int total = tiles_m * tiles_n;
  const int KS = K / kStepK;
  const size_t op_stride = (size_t)KS * kTileBytes;
  const size_t sc_stride = (size_t)KS * kTileScaleBytes;
  auto decode = [&](int bidx) {
    const int logical = tile::xcd_remap(bidx, total);
    const int per_group = kGroupM * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_group = logical - group * per_group;
    const int tm = first_m + in_group % gm;
    const int tn = in_group / gm;
    const int wa = min(2 * tn, GN - 1), wb = min(2 * tn + 1, GN - 1);
    const int xa = min(2 * tm, GM - 1), xb = min(2 * tm + 1, GM - 1);
    tile::Job16 j;
    j.wga = wp + wa * op_stride;
    j.wgb = wp + wb * op_stride;
    j.xga = qp + xa * op_stride;
    j.xgb = qp + xb * op_stride;
    j.swa = wsp + wa * sc_stride;
    j.swb = wsp + wb * sc_stride;
    j.sxa = qsp + xa * sc_stride;
    j.sxb = qsp + xb * sc_stride;
    j.row0 = tm * 256;
    j.col0 = tn * 256;
    return j;
  };
  tile::persistent16(st0, st1, st2, st3, epi, blds, total, KS, decode, y, ldy, M, N, bias, vec_store);
}

// W4A8: the persistent GEMM with the weight operand as packed MXFP4 (the
// 4-bit loop of persistent16_run: two 50 KiB step buffers, each one 128-K
// step of 4-bit weights, E4M3 activations and both scale tiles).  The weight
// group of 128 rows holds KS/2 pieces per band; the scales are laid out as
// for MXFP8.
__global__ __launch_bounds__(kThreads, 1) void gemm_persistent_w4_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ qsp, int M, int K,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ wsp, int N, int GN, int GM,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n,
    int vec_store) {
  __shared__ __attribute__((aligned(16))) uint8_t buf0[tile::kW4Buf];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[tile::kW4Buf];
  __shared__ __attribute__((aligned(16))) uint8_t epi[tile::kEpiBytes];
  __shared__ __attribute__((aligned(16))) uint8_t blds[tile::kBiasBytes];

  const int total = tiles_m * tiles_n;
  const int KS = K / kStepK;
  const size_t op_stride = (size_t)KS * kTileBytes;          // activations: bytes per 128-row group
  const size_t w_stride = (size_t)(KS / 2) * kTileBytes;     // 4-bit weights: half of that
  const size_t sc_stride = (size_t)KS * kTileScaleBytes;
  auto decode = [&](int bidx, bool) {
    const int logical = tile::xcd_remap(bidx, total);
    const int per_group = kGroupM * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_group = logical - group * per_group;
    const int tm = first_m + in_group % gm;
    const int tn = in_group / gm;
    const int wa = min(2 * tn, GN - 1), wb = min(2 * tn + 1, GN - 1);
    const int xa = min(2 * tm, GM - 1), xb = min(2 * tm + 1, GM - 1);
    tile::Job16 j;
    j.wga = wp + wa * w_stride;
    j.wgb = wp + wb * w_stride;
    j.xga = qp + xa * op_stride;
    j.xgb = qp + xb * op_stride;
    j.swa = wsp + wa * sc_stride;
    j.swb = wsp + wb * sc_stride;
    j.sxa = qsp + xa * sc_stride;
    j.sxb = qsp + xb * sc_stride;
    j.row0 = tm * 256;
    j.col0 = tn * 256;
    return j;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1;
  tile::persistent16_run<1, tile::kBiasSlot, true, true, true>(
      buf0, buf0 + tile::kOpBytes, buf1, buf1 + tile::kOpBytes, blds, total, KS, decode,
      [&](const tile::Job16& j) { return tile::W4Src(j.wga, j.wgb, j.xga, j.xgb, j.swa, j.swb, j.sxa, j.sxb, KS); },
      [&](const tile::Job16& j) { return tile::bias_rsrc(bias, j.col0, N); },
      [&](tile::i4v r, uint8_t* slot) { tile::b2l_4((uint32_t)(wn * 256 + lane * 4), r, 0u, slot + wave * 256); },
      [&](int) {}, [&](v4f (&acc)[8][8], const uint8_t* slot) { tile::bias_init16(acc, slot + wave * 256); },
      [&](const v4f (&acc)[8][8], const tile::Job16& j, const uint8_t*) {
        return tile::epi16(epi, acc, y, ldy, j.row0, M, j.col0, N, vec_store) ? 32 : 0;
      });
}

// y[m][n] = bf16( sum_s part[s][m][n] + bias[n] ), slices added in order.
// vec: y rows 8-byte aligned (ldy % 4 == 0), so four columns go out as one
// 8-byte store.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                            int64_t ldp, const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y, int64_t ldy, int vec) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one thread per 4 columns
  const int64_t per_row = (N + 3) / 4;
  if (t >= (int64_t)M * per_row) return;
  const int64_t m = t / per_row;
  const int n = (int)(t - m * per_row) * 4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < splits; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(part + ((size_t)sp * M + m) * ldp + n);
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  float b[4] = {0.f, 0.f, 0.f, 0.f};
  if (bias != nullptr)
    for (int e = 0; e < 4; ++e) b[e] = (n + e < N) ? __uint_as_float((uint32_t)bias[n + e] << 16) : 0.f;
  const uint32_t lo = pack_bf16x2(a.x + b[0], a.y + b[1]), hi = pack_bf16x2(a.z + b[2], a.w + b[3]);
  uint16_t* d = y + m * ldy + n;
  if (vec && n + 3 < N) {
    *reinterpret_cast<uint2*>(d) = make_uint2(lo, hi);
    return;
  }
  d[0] = (uint16_t)lo;
  if (n + 1 < N) d[1] = (uint16_t)(lo >> 16);
  if (n + 2 < N) d[2] = (uint16_t)hi;
  if (n + 3 < N) d[3] = (uint16_t)(hi >> 16);
}

int launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t N, int64_t ldp, const void* bias,
                         void* y, int64_t ldy, hipStream_t stream) {
  const int64_t threads = M * ((N + 3) / 4);
  const int vec = (ldy % 4 == 0) && (((uintptr_t)y & 7) == 0);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, part,
                     splits, (int)M, (int)N, ldp, (const uint16_t*)bias, (uint16_t*)y, ldy, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_gemm_tile(const void* qp, const void* sp, int64_t M, int64_t K, const void* wp, const void* wsp,
                     int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, int splits,
                     void* part) {
  const int64_t GN = (N + kGroupRows - 1) / kGroupRows;
  const int64_t GM = (M + kGroupRows - 1) / kGroupRows;
  const int tiles_n = (int)((GN + 1) / 2);
  const int tiles_m = (int)((GM + 1) / 2);
  const int vec = (ldy % 8 == 0 && ((uintptr_t)y & 15) == 0) ? 2 : (ldy % 4 == 0 && ((uintptr_t)y & 7) == 0) ? 1 : 0;
  const int64_t ldp = (N + 3) / 4 * 4;
  if (splits == 1) {
    const int total = tiles_m * tiles_n;
    const int cus = device_cu_count();
    const int grid = total <= cus ? total : (cus >= 8 ? cus - cus % 8 : cus);
    hipLaunchKernelGGL(gemm_persistent_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, (const uint8_t*)qp,
                       (const uint8_t*)sp, (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)wsp, (int)N, (int)GN,
                       (int)GM, (const uint16_t*)bias, (uint16_t*)y, ldy, tiles_m, tiles_n, vec);
    return hipGetLastError() == hipSuccess ? 0 : -7;
  }
  hipLaunchKernelGGL(gemm_tile_kernel, dim3((unsigned)(tiles_m * tiles_n * splits)), dim3(kThreads), 0, stream,
                     (const uint8_t*)qp, (const uint8_t*)sp, (int)M, (int)K, (const uint8_t*)wp,
                     (const uint8_t*)wsp, (int)N, (int)GN, (int)GM, (const uint16_t*)bias, (uint16_t*)y, ldy,
                     tiles_m, tiles_n, vec, splits, (float*)part, ldp);
  if (hipGetLastError() != hipSuccess) return -7;
  if (splits > 1) return launch_splitk_reduce((const float*)part, splits, M, N, ldp, bias, y, ldy, stream);
  return 0;
}

int launch_gemm_tile_w4(const void* qp, const void* sp, int64_t M, int64_t K, const void* w4p, const void* wsp,
                        int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  const int64_t GN = (N + kGroupRows - 1) / kGroupRows;
  const int64_t GM = (M + kGroupRows - 1) / kGroupRows;
  const int tiles_n = (int)((GN + 1) / 2);
  const int tiles_m = (int)((GM + 1) / 2);
  const int vec = (ldy % 8 == 0 && ((uintptr_t)y & 15) == 0) ? 2 : (ldy % 4 == 0 && ((uintptr_t)y & 7) == 0) ? 1 : 0;
  const int total = tiles_m * tiles_n;
  const int cus = device_cu_count();
  const int grid = total <= cus ? total : (cus >= 8 ? cus - cus % 8 : cus);
  hipLaunchKernelGGL(gemm_persistent_w4_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, (const uint8_t*)qp,
                     (const uint8_t*)sp, (int)M, (int)K, (const uint8_t*)w4p, (const uint8_t*)wsp, (int)N, (int)GN,
                     (int)GM, (const uint16_t*)bias, (uint16_t*)y, ldy, tiles_m, tiles_n, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
