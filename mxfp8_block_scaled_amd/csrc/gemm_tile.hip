// Large-M block-scaled MXFP8 GEMM with the layer's epilogue.
//
//   y[m, n] = bf16( sum_b 2^(sa[m,b]-127) 2^(sw[n,b]-127) sum_{k in b} qa[m,k] qw[n,k] + bias[n] )
//
// (the mm_mxfp8 GEMM of vLLM PR #52204's apply_weights, A[M, K] x B[K, N_pad]
// with both operands K-major, followed by the slice to the logical N and the
// bias add of its §Purpose, folded into one epilogue).
//
// The K loop is tile_core.hpp's 256 x 256 tile.  Here:
//  * Workgroups are dispatched round-robin over the 8 XCDs; the tile index is
//    remapped so that each XCD works on a contiguous, M-grouped range of tiles
//    and its private L2 sees the reuse of weight and activation K-slices.
//  * Epilogue (tile::store_bf16): fp32 staged through LDS, bias added in fp32,
//    one rounding to bf16, 8-byte stores covering whole 256-byte row segments.
#include "common.hpp"
#include "launch.hpp"
#include "tile_core.hpp"

namespace mxfp8 {

namespace {

using tile::kStage;
using tile::kThreads;
constexpr int kGroupM = 8;                            // tiles along M per group of the tile order

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void gemm_tile_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ qsp, int M, int K,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ wsp, int N, int GN, int GM,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n,
    int vec_store) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st3[kStage];

  // Tile order: XCD-contiguous, then groups of kGroupM tiles along M.
  const int total = tiles_m * tiles_n;
  const int logical = tile::xcd_remap((int)blockIdx.x, total);
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

  v16f acc[4][4];
  tile::mainloop(st0, st1, st2, st3, wp + wa * op_stride, wp + wb * op_stride, qp + xa * op_stride,
                 qp + xb * op_stride, wsp + wa * sc_stride, wsp + wb * sc_stride, qsp + xa * sc_stride,
                 qsp + xb * sc_stride, KS, acc);

  tile::store_bf16(st0, st1, st2, st3, acc, y, ldy, tm * 256, M, tn * 256, N, bias, vec_store);
}

int launch_gemm_tile(const void* qp, const void* sp, int64_t M, int64_t K, const void* wp, const void* wsp,
                     int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  const int64_t GN = (N + kGroupRows - 1) / kGroupRows;
  const int64_t GM = (M + kGroupRows - 1) / kGroupRows;
  const int tiles_n = (int)((GN + 1) / 2);
  const int tiles_m = (int)((GM + 1) / 2);
  const int vec = (ldy % 4 == 0) && (((uintptr_t)y & 7) == 0);
  hipLaunchKernelGGL(gemm_tile_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0, stream,
                     (const uint8_t*)qp, (const uint8_t*)sp, (int)M, (int)K, (const uint8_t*)wp,
                     (const uint8_t*)wsp, (int)N, (int)GN, (int)GM, (const uint16_t*)bias, (uint16_t*)y, ldy,
                     tiles_m, tiles_n, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
