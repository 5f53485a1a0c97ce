// Medium-tile MXFP8 GEMM: one 128-row weight group x kMT (128 or 64)
// activation rows per workgroup over the whole K, for the shapes whose
// 256 x 256 tiles would leave most of the chip idle (M of a few hundred to a
// few thousand at moderate N) and whose split-K partials cost more than they
// save.
//
// The tile GEMMs here copy their operands from L2 into LDS at 40-50 GB/s per
// CU (the persistent 256 x 256 GEMM: 47 GB/s), so a tile's time follows its
// operand bytes, (rows_n + rows_m) * K.  At M = 1024, N = K = 4096 the
// 256 x 256 tiling has 64 tiles of 2 MiB each (64 CUs busy for 45 us); the
// 128 x 128 tiling has 256 tiles of 1 MiB.  The fp32 accumulators of a
// 128 x 128 tile are 64 registers per lane and its four 64-K stages 68 KiB,
// so two workgroups share a CU and cover each other's waits.
//
//  * Waves 2 x 2: wave (wn, wm) owns weight rows 32 a + 16 wn + i (a = 0..3)
//    and activation rows 32 b + 16 wm + i (b < kMT / 32) of the tile, one
//    v_mfma_scale_f32_16x16x128_f8f6f4 per (a, b) per 128-K step, the weight
//    as the A operand.  With rows interleaved that way the byte of a row's
//    scale inside its packed scale word (rows r + 32 k, byte k) is a (resp.
//    b), an immediate op_sel.
//  * A 64-K stage holds the weight group's eight 1 KiB pieces, the tile's
//    kMT / 16 activation pieces and the two 256-byte scale tiles, copied
//    straight into LDS (buffer_load ... lds); a 128-K step reads a pair of
//    stages; two pairs in flight.
//  * Epilogue: bias added to the fp32 sums, one rounding to bf16, staged in
//    LDS and stored as whole 256-byte row segments.
#include "common.hpp"
#include "launch.hpp"
#include "tile_core.hpp"

namespace mxfp8 {

namespace {

constexpr int kMedThreads = 256;

template <int kMT>
struct MedLds {
  static constexpr int kW = kGroupRows * kStepK;   // 8192: the weight group's rows of one 64-K stage
  static constexpr int kX = kMT * kStepK;          // the tile's activation rows
  // + scale tiles: weight at kW + kX, activations + 256; two more 256-byte
  // slots take the copies of waves 2 and 3, so every wave issues the same
  // number of copies (the waits count them per wave).
  static constexpr int kStage = kW + kX + 1024;
  static constexpr int kBytes = 4 * kStage;
  static constexpr int kCopies = 2 * (2 + kMT / 64 + 1);   // per wave per 128-K step
  static constexpr int kPitchY = 128 * 2 + 16;              // staged bf16 output row
  static_assert(kMT * kPitchY <= kBytes, "the output staging fits in the stages");
};

}  // namespace

// qp, sp: packed activations (rows padded to 128), wp, wsp: the packed weight
// (G = ceil(N / 128) groups); y [M, N] bf16, row stride ldy.  vec: y rows
// 16-byte aligned (ldy % 8 == 0), so a row segment of 8 columns is one
// 16-byte store.
template <int kMT>
__global__ __launch_bounds__(kMedThreads, 2) void gemm_med_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ sp, int M, int K, const uint8_t* __restrict__ wp,
    const uint8_t* __restrict__ wsp, int N, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy,
    int tiles_m, int vec) {
  using L = MedLds<kMT>;
  constexpr int kNB = kMT / 32;                    // activation row blocks per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int i = lane & 15, g = lane >> 4;
  // Work item = weight group * tiles_m + activation tile; a die takes a
  // contiguous run of items, i.e. a few weight groups (from its own L2).
  const int item = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tn = item / tiles_m, tm = item - tn * tiles_m;
  const int KS = K / kStepK;                       // 64-K stages
  const int P = KS / 2;                            // 128-K steps (K % 256 == 0: even, >= 2)

  // Bias of the lane's 16 output columns 32 a + 16 wn + 4 g + j of the group
  // (columns past N read 0 and are never stored); compiler-tracked loads,
  // issued first.
  const int n0 = tn * kGroupRows;
  const __amdgpu_buffer_rsrc_t brsrc = raw_rsrc(bias, bias != nullptr ? (uint32_t)N * 2u : 0u);
  uint32_t braw[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      braw[a][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
          brsrc, (uint32_t)(n0 + 32 * a + 16 * wn + 4 * g + j) * 2u, 0, 0);

  // Copy sources.  Weight group tn: band b, 64-K step ks at (b KS + ks) KiB
  // of the group; wave w copies bands w and w + 4.  Activations: group
  // tm (kMT = 128) or rows 64 h .. 64 h + 63 of group tm / 2, h = tm % 2
  // (kMT = 64): bands w, w + 4 resp. 4 h + w.  Scale tiles: 256 bytes per
  // 64-K step, wave 0 (and 2) the weight's, wave 1 (and 3) the activations'.
  const int h = kMT == 64 ? (tm & 1) : 0;
  const int xg = kMT == 64 ? (tm >> 1) : tm;
  const uint32_t gbytes = (uint32_t)KS * kTileBytes, sbytes = (uint32_t)KS * kTileScaleBytes;
  const tile::i4v wr = tile::buffer_rsrc(wp + (size_t)tn * gbytes, gbytes);
  const tile::i4v xr = tile::buffer_rsrc(qp + (size_t)xg * gbytes, gbytes);
  const tile::i4v sr = tile::buffer_rsrc((wave & 1) ? sp + (size_t)xg * sbytes : wsp + (size_t)tn * sbytes, sbytes);
  const uint32_t lo16 = (uint32_t)lane * 16u;
  const uint32_t vw0 = (uint32_t)wave * KS * kPieceBytes + lo16, vw1 = vw0 + 4u * KS * kPieceBytes;
  const uint32_t vx0 = (uint32_t)(kMT == 64 ? 4 * h + wave : wave) * KS * kPieceBytes + lo16;
  const uint32_t vx1 = vx0 + 4u * KS * kPieceBytes;
  const uint32_t vs = (uint32_t)lane * 4u;
  auto issue_stage = [&](int ks, uint8_t* st) {
    const uint32_t off = (uint32_t)ks * kPieceBytes;
    tile::b2l_16(vw0, wr, off, st + wave * 1024);
    tile::b2l_16(vw1, wr, off, st + 4096 + wave * 1024);
    tile::b2l_16(vx0, xr, off, st + L::kW + wave * 1024);
    if constexpr (kMT == 128) tile::b2l_16(vx1, xr, off, st + L::kW + 4096 + wave * 1024);
    tile::b2l_4(vs, sr, (uint32_t)ks * kTileScaleBytes, st + L::kW + L::kX + wave * 256);
  };
  auto stage_ptr = [&](int s) { return smem + s * L::kStage; };

  // Fragment offsets inside a stage: rows 32 a + 16 wn + i share the swizzle
  // of row i (it reads bits 2-3 of the row only).
  const int offW = 16 * wn * kStepK + tile_off(i, g);
  const int offX = L::kW + 16 * wm * kStepK + tile_off(i, g);
  // Scale words: lane (i, g) supplies MX block g of the 128-K step, block
  // g % 2 of stage g / 2; the word of row 16 w + i holds rows 16 w + i + 32 k
  // in byte k.  For kMT = 64 the tile's rows are 64 h + ... of the group, so
  // its bytes are 2 h + b: the word is shifted by 16 h bits.
  const int offSW = L::kW + L::kX + (16 * wn + i) * 8 + (g & 1) * 4;
  const int offSX = L::kW + L::kX + 256 + (16 * wm + i) * 8 + (g & 1) * 4;
  auto rd16 = [](const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); };
  auto frag = [&](const uint8_t* ev, const uint8_t* od, int off) {
    const uint4 lo = rd16(ev + off), hi = rd16(od + off);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  v4f acc[4][kNB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b) acc[a][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  issue_stage(0, stage_ptr(0));
  issue_stage(1, stage_ptr(1));
  issue_stage(2, stage_ptr(2));
  issue_stage(3, stage_ptr(3));
  for (int p = 0; p < P; ++p) {
    // Step p has landed in every wave's share once at most the copies of
    // step p + 1 are outstanding; the barrier makes that true for all waves.
    if (p + 1 < P)
      tile::wait_vmcnt<L::kCopies>();
    else
      tile::wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const uint8_t* ev = stage_ptr(2 * (p & 1));
    const uint8_t* od = ev + L::kStage;
    v8i wf[4], xf[kNB];
#pragma unroll
    for (int a = 0; a < 4; ++a) wf[a] = frag(ev, od, offW + 32 * kStepK * a);
#pragma unroll
    for (int b = 0; b < kNB; ++b) xf[b] = frag(ev, od, offX + 32 * kStepK * b);
    const int sw = *reinterpret_cast<const int*>(((g >> 1) ? od : ev) + offSW);
    int sx = *reinterpret_cast<const int*>(((g >> 1) ? od : ev) + offSX);
    if constexpr (kMT == 64) sx = (int)((uint32_t)sx >> (16 * h));
    // Every wave has its operands of this pair: its stages may be refilled.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (p + 2 < P) {
      issue_stage(2 * p + 4, stage_ptr(2 * (p & 1)));
      issue_stage(2 * p + 5, stage_ptr(2 * (p & 1) + 1));
    }
    tile::static_for<0, 4>([&](auto A) {
      constexpr int a = decltype(A)::value;
      tile::static_for<0, kNB>([&](auto B) {
        constexpr int b = decltype(B)::value;
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[a], xf[b], acc[a][b], 0, 0, a, sw, b, sx);
      });
    });
  }

  // Epilogue: every wave is past the last barrier (no stage is read again
  // and no copy is in flight).  Lane (i, g) holds D[n = 32 a + 16 wn + 4 g + j]
  // [m = 32 b + 16 wm + i]: bias, one rounding, staged row-major in LDS.
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = acc[a][b][j] + __uint_as_float(braw[a][j] << 16);
      const int m = 32 * b + 16 * wm + i, n = 32 * a + 16 * wn + 4 * g;
      *reinterpret_cast<uint2*>(smem + m * L::kPitchY + n * 2) = make_uint2(pack_bf16x2(v[0], v[1]),
                                                                            pack_bf16x2(v[2], v[3]));
    }
  __syncthreads();
  // Thread t stores columns 8 (t % 16) .. + 7 of row t / 16 + 16 q.
  const int c8 = (tid & 15) * 8;
  const int mt0 = tm * kMT;
#pragma unroll
  for (int q = 0; q < kMT / 16; ++q) {
    const int r = (tid >> 4) + 16 * q;
    const int m = mt0 + r;
    if (m >= M) break;
    const int n = n0 + c8;
    if (n >= N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(smem + r * L::kPitchY + c8 * 2);
    uint16_t* dst = y + (size_t)m * ldy + n;
    if (vec && n + 7 < N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
  }
}

namespace {
template <int kMT>
int launch_med_k(const void* qp, const void* sp, int64_t M, int64_t K, const void* wp, const void* wsp, int64_t N,
                 const void* bias, void* y, int64_t ldy, hipStream_t stream) {
  constexpr int lds = MedLds<kMT>::kBytes;
  static std::atomic<int> lds_set[kMaxDevices];
  if (!set_lds_limit_once((const void*)gemm_med_kernel<kMT>, lds, lds_set)) return -7;
  const int G = (int)((N + kGroupRows - 1) / kGroupRows);
  const int tiles_m = (int)((M + kMT - 1) / kMT);
  const int vec = (ldy % 8 == 0) && (((uintptr_t)y & 15) == 0);
  hipLaunchKernelGGL((gemm_med_kernel<kMT>), dim3((unsigned)(G * tiles_m)), dim3(kMedThreads), lds, stream,
                     (const uint8_t*)qp, (const uint8_t*)sp, (int)M, (int)K, (const uint8_t*)wp, (const uint8_t*)wsp,
                     (int)N, (const uint16_t*)bias, (uint16_t*)y, ldy, tiles_m, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
}  // namespace

int launch_gemm_med(const void* qp, const void* sp, int64_t M, int64_t K, const void* wp, const void* wsp, int64_t N,
                    const void* bias, void* y, int64_t ldy, hipStream_t stream, int mt) {
  if (mt == 64) return launch_med_k<64>(qp, sp, M, K, wp, wsp, N, bias, y, ldy, stream);
  return launch_med_k<128>(qp, sp, M, K, wp, wsp, N, bias, y, ldy, stream);
}

}  // namespace mxfp8
