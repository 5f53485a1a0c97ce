// Large-M block-scaled MXFP8 GEMM with the layer's epilogue.
//
//   y[m, n] = bf16( sum_b 2^(sa[m,b]-127) 2^(sw[n,b]-127) sum_{k in b} qa[m,k] qw[n,k] + bias[n] )
//
// (the mm_mxfp8 GEMM of vLLM PR #52204's apply_weights, A[M, K] x B[K, N_pad]
// with both operands K-major, followed by the slice to the logical N and the
// bias add of its §Purpose, folded into one epilogue).
//
// Design (gfx950):
//  * Workgroup tile 256 (n, weight rows) x 256 (m, activation rows), 4 waves
//    as 2 x 2, each wave 128 x 128 = 4 x 4 v_mfma_scale_f32_32x32x64_f8f6f4
//    tiles.  The weight is the MFMA A operand, so each lane's results are 4
//    consecutive n of one output row m: one 8-byte bf16 store per 4 values.
//  * K advances 128 bytes (4 MX blocks) per stage.  A stage is 32 KiB of
//    weight + 32 KiB of activations + 2 x 1 KiB of scales, copied straight
//    from global memory into LDS with global_load_lds_dwordx4 / _dword (no
//    VGPR staging).  Two stages double-buffer the K loop: the copy of step
//    k+1 is in flight while step k computes.
//  * The packed weight tile is already in LDS order; activation rows are
//    placed with the same XOR swizzle (common.hpp) by choosing which global
//    chunk each lane fetches, so LDS fragment reads are bank-conflict free.
//  * Workgroups are dispatched round-robin over the 8 XCDs; the tile index is
//    remapped so that each XCD works on a contiguous, M-grouped range of tiles
//    and its private L2 sees the reuse of weight and activation K-slices.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kThreads = 256;
constexpr int kWBytes = kBN * kStepK;  // 32768
constexpr int kXBytes = kBM * kStepK;  // 32768
constexpr int kWSBytes = kBN * 4;      // 1024
constexpr int kXSBytes = kBM * 4;      // 1024
constexpr int kStage = kWBytes + kXBytes + kWSBytes + kXSBytes;
constexpr int kStages = 2;
constexpr int kGroupM = 8;  // tiles along M per group of the tile order
constexpr int kXCD = 8;

typedef __attribute__((address_space(3))) void lds_void;

__device__ inline void g2l_16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}
__device__ inline void g2l_4(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 4, 0, 0);
}

__device__ inline v8i lds_frag(const uint8_t* base, int row, int c0, int c1) {
  const uint4 a = *reinterpret_cast<const uint4*>(base + swz_slot(row, c0) * 16);
  const uint4 b = *reinterpret_cast<const uint4*>(base + swz_slot(row, c1) * 16);
  v8i v;
  v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
  v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  return v;
}

// Bijection from dispatch order to a tile order in which XCD x (which gets
// workgroups x, x+8, x+16, ...) owns one contiguous range of tiles.
__device__ inline int xcd_remap(int bid, int total) {
  const int xcd = bid % kXCD, k = bid / kXCD;
  const int per = total / kXCD, rem = total % kXCD;
  return (xcd < rem) ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void gemm_tile_kernel(
    const uint8_t* __restrict__ xq, int64_t ldq, const uint8_t* __restrict__ xs, int64_t lds, int M, int K,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ sp, int N, int G,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n,
    int vec_store) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Tile order: XCD-contiguous, then groups of kGroupM tiles along M.
  const int total = tiles_m * tiles_n;
  const int logical = xcd_remap((int)blockIdx.x, total);
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;

  const int m0 = tm * kBM;
  const int KS = K / kStepK;
  const int ga = min(2 * tn, G - 1), gb = min(2 * tn + 1, G - 1);
  const uint8_t* wt0 = wp + (size_t)ga * KS * kTileBytes + tid * 16;
  const uint8_t* wt1 = wp + (size_t)gb * KS * kTileBytes + tid * 16;
  const uint8_t* st = sp + (size_t)(tid < 128 ? ga : gb) * KS * kTileScaleBytes + (tid & 127) * 4;

  // Activation chunk fetched by this lane in copy round q: LDS slot
  // q*256 + tid holds row r = q*32 + tid/8, chunk (tid%8) ^ (r%8).
  const int xc = (tid & 7) ^ ((tid >> 3) & 7);
  const uint8_t* xrow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = min(m0 + q * 32 + (tid >> 3), M - 1);
    xrow[q] = xq + (size_t)r * ldq + xc * 16;
  }
  const uint8_t* xsrow = xs + (size_t)min(m0 + tid, M - 1) * lds;

  auto issue = [&](int ks, int stage) {
    uint8_t* base = smem + stage * kStage + wave * 1024;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      g2l_16(((q < 4) ? wt0 : wt1) + (size_t)ks * kTileBytes + (q & 3) * 4096, base + q * 4096);
#pragma unroll
    for (int q = 0; q < 8; ++q) g2l_16(xrow[q] + (size_t)ks * kStepK, base + kWBytes + q * 4096);
    uint8_t* sbase = smem + stage * kStage + kWBytes + kXBytes + wave * 256;
    g2l_4(st + (size_t)ks * kTileScaleBytes, sbase);
    g2l_4(xsrow + ks * 4, sbase + kWSBytes);
  };

  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 31, lg = lane >> 5;

  v16f acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int ks = 0; ks < KS; ++ks) {
    const int stage = ks & 1;
    if (ks + 1 < KS) issue(ks + 1, stage ^ 1);
    const uint8_t* wb = smem + stage * kStage;
    const uint8_t* xb = wb + kWBytes;
    const uint32_t* wsc = reinterpret_cast<const uint32_t*>(wb + kWBytes + kXBytes);
    const uint32_t* xsc = reinterpret_cast<const uint32_t*>(wb + kWBytes + kXBytes + kWSBytes);
    // Lane group lg supplies the scale of MX block (2j + lg) of this K step.
    int sw[4], sx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sw[i] = (int)(wsc[wn * 128 + 32 * i + li] >> (8 * lg));
      sx[i] = (int)(xsc[wm * 128 + 32 * i + li] >> (8 * lg));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v8i fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = lds_frag(wb, wn * 128 + 32 * i + li, 4 * j + lg, 4 * j + 2 + lg);
        fb[i] = lds_frag(xb, wm * 128 + 32 * i + li, 4 * j + lg, 4 * j + 2 + lg);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (j == 0)
            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a], fb[b], acc[a][b], 0, 0, 0, sw[a],
                                                                        0, sx[b]);
          else
            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a], fb[b], acc[a][b], 0, 0, 2, sw[a],
                                                                        2, sx[b]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // Epilogue: lane holds n = nb + 8*(r/4) + 4*lg + r%4 for m = mb + li.
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int nb = tn * kBN + wn * 128 + 32 * a + 4 * lg;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int m = m0 + wm * 128 + 32 * b + li;
      if (m >= M) continue;
      uint16_t* yrow = y + (size_t)m * ldy;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int n = nb + 8 * rr;
        if (n >= N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[a][b][4 * rr + e];
          if (bias != nullptr && n + e < N) v[e] += __uint_as_float((uint32_t)bias[n + e] << 16);
        }
        if (vec_store && n + 3 < N) {
          const uint32_t lo = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
          *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yrow[n + e] = (uint16_t)f32_to_bf16_rne(v[e]);
        }
      }
    }
  }
}

int launch_gemm_tile(const void* q, int64_t ldq, const void* s, int64_t lds, int64_t M, int64_t K,
                     const void* wp, const void* sp, int64_t N, const void* bias, void* y, int64_t ldy,
                     hipStream_t stream) {
  const int64_t G = (N + kGroupRows - 1) / kGroupRows;
  const int tiles_n = (int)((G + 1) / 2);
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int vec = (ldy % 4 == 0) && (((uintptr_t)y & 7) == 0);
  hipLaunchKernelGGL(gemm_tile_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0, stream,
                     (const uint8_t*)q, ldq, (const uint8_t*)s, lds, (int)M, (int)K, (const uint8_t*)wp,
                     (const uint8_t*)sp, (int)N, (int)G, (const uint16_t*)bias, (uint16_t*)y, ldy, tiles_m,
                     tiles_n, vec);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
