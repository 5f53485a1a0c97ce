// Top-k routed MXFP8 mixture-of-experts layer (the grouped variant of the
// linear layer): BF16 activations and fp32 router logits in, BF16 out.
//
// What is computed ("feat(moe): add unified block-scale FP8 support",
// flashinfer PR #4026, walkthrough and sequence diagram: BF16 activations are
// quantized to MXFP8 inside the MoE; "Feature/sm100 low latency nvfp4
// kernels", flashinfer PR #1214, Highlights: the "Renormalize" routing, top-k
// then softmax over the k; "Add support for FlashInfer mxfp8", sglang PR
// #18945: fused w13 (gate + up) and w2 expert weights, MXFP8 with 32-K UE8M0
// scales):
//   ids, w   = top-k of the token's logits (ties: lower expert id), softmax
//              over those k;
//   h        = deq(q(x_t)) . deq(W13[e])^T            for each selected e,
//   act      = bf16( silu(h[:I]) * h[I:] ),  q(act) = MX quantization along I,
//   o_j      = deq(q(act_j)) . deq(W2[e_j])^T  (fp32 accumulation),
//   y_t      = bf16( sum_j w_j . o_j ), the products and the sum in fp32.
//
// Pipeline (one stream, every step deterministic):
//  1. route    one wave per token: k rounds of a wave arg-max, softmax over
//              the k; per-block (16-token) expert histograms; the token's
//              row of x MX-quantized once, row-major, into xq / xs; the
//              sorted-row list filled with -1.
//  2. plan     one workgroup: per-expert counts, expert segments of the
//              sorted row space padded to 128-row groups, per-block offsets,
//              the M-tile list (256 rows = two groups of one expert).
//  3. scatter  row (t, j) -> its position in its expert's segment, in
//              increasing t*k + j order (wave ballots + per-wave counts).
//  4. gather   the expert-sorted scale tiles of the GEMM operand gathered
//              from the token rows' scales (pad rows: scale 0); row T of xq
//              (all zero) for pad rows.
//  5. gemm1    per (M-tile, 256-row slice of W13[e]) the shared tile loop,
//              its activation rows copied from the quantized x by row index;
//              W13 is packed with gate and up rows interleaved so that each
//              lane holds gate and up of the same intermediate index; the
//              epilogue applies SiLU-gating, rounds to bf16, MX-quantizes
//              along I and writes the packed operand of gemm2.
//  6. gemm2    per (M-tile, 256-row slice of W2[e]): the tile loop; each
//              real row's fp32 accumulators written to its slot row t*k + j
//              (pad rows: a spare row).
//  7. combine  y_t = bf16( sum_j w_j * ys[t*k + j] ), each product rounded to
//              fp32, the sum in fp32 in slot order, one rounding; a token's
//              k slot rows are contiguous.
#include <algorithm>
#include <cfloat>
#include <climits>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tile_core.hpp"

namespace mxfp8 {

namespace {

constexpr int kRouteTokens = 16;   // tokens (one wave each) per route / scatter block

__device__ inline bool route_better(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }

}  // namespace

// ---------------------------------------------------------------- 1. route
// One wave per token also MX-quantizes the token's row of x into xq / xs
// (row-major), by quant_act_kernel's rule and lane layout: four lanes per
// 32-element block, 8 elements each, the block maximum over the four lanes
// by two lane exchanges.  Its loads go out before the routing, so they are in
// flight while the wave selects the experts.  Every block also fills its
// share of the sorted-row list with -1 (the scatter writes the real rows
// after the plan).
__global__ __launch_bounds__(1024) void moe_route_kernel(const float* __restrict__ logits, int T, int E, int topk,
                                                         int* __restrict__ ids, float* __restrict__ wts,
                                                         int* __restrict__ blk_cnt, int nblk,
                                                         const uint16_t* __restrict__ x, int H,
                                                         uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                                         int* __restrict__ sorted_row, int p_max) {
  __shared__ int hist[kMoeMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) hist[e] = 0;
  {
    // p_max is a multiple of 128: 16-byte stores, a contiguous share per block.
    const int n4 = p_max / 4, per = (n4 + nblk - 1) / nblk;
    const int b0 = blockIdx.x * per, b1 = min(b0 + per, n4);
    for (int i = b0 + tid; i < b1; i += 1024) reinterpret_cast<int4*>(sorted_row)[i] = make_int4(-1, -1, -1, -1);
  }
  __syncthreads();
  const int t = blockIdx.x * kRouteTokens + wave;
  if (t < T) {
    // The first (up to) four 8-element chunks of this lane in the row.
    const int nc8 = H / 8;
    const uint16_t* xr = x + (int64_t)t * H;
    uint4 xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c8 = u * 64 + lane;
      xv[u] = c8 < nc8 ? *reinterpret_cast<const uint4*>(xr + c8 * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
    float v[4];
    bool ok[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      ok[c] = e < E;
      v[c] = ok[c] ? logits[(int64_t)t * E + e] : 0.0f;
      // NaN compares false both ways: read it as -inf, so every round still
      // finds a candidate (topk <= E) and every selected id is an expert.
      // The routing of such a token is meaningless, but stays in bounds.
      if (v[c] != v[c]) v[c] = -INFINITY;
    }
    float selv = 0.0f;
    int seli = 0;
    for (int j = 0; j < topk; ++j) {
      float bv = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (ok[c] && route_better(v[c], lane + 64 * c, bv, bi)) {
          bv = v[c];
          bi = lane + 64 * c;
        }
      // The best (value, index) of the wave: quads (DPP lane exchanges),
      // then 8- and 16-lane rows (mirrors), then rows and halves (gfx950 row
      // swaps); all VALU.  The order is a strict total order, so the result
      // is the same for any reduction tree.
      auto take = [&](float ov, int oi) {
        if (route_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      };
      auto dpp = [&](auto ctrl) {
        constexpr int c = decltype(ctrl)::value;
        const int ovb = __builtin_amdgcn_update_dpp(0, __float_as_int(bv), c, 0xF, 0xF, true);
        const int oi = __builtin_amdgcn_update_dpp(0, bi, c, 0xF, 0xF, true);
        take(__int_as_float(ovb), oi);
      };
      dpp(std::integral_constant<int, 0xB1>{});    // quad_perm [1, 0, 3, 2]
      dpp(std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
      dpp(std::integral_constant<int, 0x141>{});   // row_half_mirror
      dpp(std::integral_constant<int, 0x140>{});   // row_mirror
      {
        const auto sv = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
        const auto si = __builtin_amdgcn_permlane16_swap((uint32_t)bi, (uint32_t)bi, false, false);
        take(__uint_as_float(sv[0]), (int)si[0]);
        take(__uint_as_float(sv[1]), (int)si[1]);
      }
      {
        const auto sv = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
        const auto si = __builtin_amdgcn_permlane32_swap((uint32_t)bi, (uint32_t)bi, false, false);
        take(__uint_as_float(sv[0]), (int)si[0]);
        take(__uint_as_float(sv[1]), (int)si[1]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (lane + 64 * c == bi) ok[c] = false;
      if (lane == j) {
        selv = bv;
        seli = min(max(bi, 0), E - 1);   // always an expert id (see the NaN note above)
      }
    }
    // Selection 0 is the largest logit.
    const float mx = __shfl(selv, 0);
    const float z = lane < topk ? expf(selv - mx) : 0.0f;
    float s = z;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane < topk) {
      ids[(int64_t)t * topk + lane] = seli;
      wts[(int64_t)t * topk + lane] = z / s;
      atomicAdd(&hist[seli], 1);
    }
    // MX quantization of the row (H % 256 == 0, so a block's four lanes are
    // always all in range or all out).
    uint8_t* qr = xq + (int64_t)t * H;
    uint8_t* sr = xs + (int64_t)t * (H / 32);
    for (int base = 0; base < nc8; base += 256) {
      if (base > 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c8 = base + u * 64 + lane;
          xv[u] = c8 < nc8 ? *reinterpret_cast<const uint4*>(xr + c8 * 8) : make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c8 = base + u * 64 + lane;
        const uint32_t w[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
        u16x2 mp = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) mp = absmax_pk(mp, w[i]);
        uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
        m = quad_max(m);
        const uint32_t sb = (uint32_t)max((int)(m >> 7) - 8, 0);
        uint32_t qd[2];
        cvt8s(w, mx_scale_value(sb), qd);
        if (c8 < nc8) {
          *reinterpret_cast<uint2*>(qr + c8 * 8) = make_uint2(qd[0], qd[1]);
          if ((c8 & 3) == 0) sr[c8 >> 2] = (uint8_t)sb;
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) blk_cnt[(int64_t)blockIdx.x * E + e] = hist[e];
}

// ---------------------------------------------------------------- 2. plan
// meta[0] = number of M-tiles, meta[1] = number of 128-row groups in use.
// One workgroup; every phase is parallel over experts and blocks.  Stores
// count in the same vmcnt as loads, so each phase issues its loads, waits
// once, and only then stores.  (The route kernel fills the sorted-row list
// with -1.)
constexpr int kPlanChunk = 32;

__global__ __launch_bounds__(1024) void moe_plan_kernel(const int* __restrict__ blk_cnt, int nblk, int E,
                                                        int* __restrict__ blk_off, int* __restrict__ seg_off,
                                                        int* __restrict__ tile_e, int* __restrict__ tile_g0,
                                                        int* __restrict__ tile_ng, int* __restrict__ meta) {
  __shared__ int part[1024];
  __shared__ int cnt[kMoeMaxExperts], gstart[kMoeMaxExperts], tstart[kMoeMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Thread (c, e) = (tid / E, tid % E) owns blocks [b0, b1) of expert e; the
  // counts are stored block-major ([nblk][E]), so a wave's load reads
  // consecutive experts of one block (contiguous bytes).
  const int tpe = 1024 / E;                       // threads per expert (E <= 256: >= 4)
  const int e = tid % E, c = tid / E;
  const bool mine = c < tpe;
  const int per = (nblk + tpe - 1) / tpe;
  const int b0 = min(c * per, nblk), b1 = min(b0 + per, nblk);
  // (Indices are clamped rather than the loads predicated, so a chunk's loads
  // are straight-line code and overlap.)
  auto load_chunk = [&](int b, int (&v)[kPlanChunk]) {
#pragma unroll
    for (int u = 0; u < kPlanChunk; ++u) v[u] = blk_cnt[(int64_t)min(b + u, b1 - 1) * E + e];
  };
  int sum = 0;
  // With at most one chunk per thread (T <= 32 * 16 * 1024 / E tokens) the
  // counts stay in registers for the offsets below.
  const bool one_chunk = b1 - b0 <= kPlanChunk;
  int v0[kPlanChunk];
  if (mine)
    for (int b = b0; b < b1; b += kPlanChunk) {
      int v[kPlanChunk];
      load_chunk(b, v);
#pragma unroll
      for (int u = 0; u < kPlanChunk; ++u) {
        sum += (b + u < b1) ? v[u] : 0;
        v0[u] = v[u];
      }
    }
  part[tid] = sum;
  __syncthreads();
  if (tid < E) {
    int t = 0;
    for (int k = 0; k < tpe; ++k) t += part[k * E + tid];
    cnt[tid] = t;
  }
  __syncthreads();
  // Exclusive scan of groups and M-tiles over experts: wave 0, lane l holds
  // experts 4l .. 4l+3.
  if (wave == 0) {
    int g4[4], t4[4], gs = 0, ts = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = 4 * lane + u;
      const int groups = x < E ? (cnt[x] + kGroupRows - 1) / kGroupRows : 0;
      g4[u] = gs;
      t4[u] = ts;
      gs += groups;
      ts += (groups + 1) / 2;
    }
    int gi = gs, ti = ts;                          // inclusive scan across lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int go = __shfl_up(gi, off), to = __shfl_up(ti, off);
      if (lane >= off) {
        gi += go;
        ti += to;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = 4 * lane + u;
      if (x < E) {
        gstart[x] = gi - gs + g4[u];
        tstart[x] = ti - ts + t4[u];
      }
    }
    if (lane == 63) {
      meta[0] = ti;
      meta[1] = gi;
    }
  }
  __syncthreads();
  if (mine) {
    int run = 0;
    for (int k = 0; k < c; ++k) run += part[k * E + e];
    for (int b = b0; b < b1; b += kPlanChunk) {
      int v[kPlanChunk];
      if (one_chunk) {
#pragma unroll
        for (int u = 0; u < kPlanChunk; ++u) v[u] = v0[u];
      } else {
        load_chunk(b, v);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
#pragma unroll
      for (int u = 0; u < kPlanChunk; ++u) {
        if (b + u < b1) blk_off[(int64_t)(b + u) * E + e] = run;
        run += (b + u < b1) ? v[u] : 0;
      }
    }
  }
  if (tid < E) {
    const int groups = (cnt[tid] + kGroupRows - 1) / kGroupRows;
    seg_off[tid] = gstart[tid] * kGroupRows;
    for (int u = 0; 2 * u < groups; ++u) {
      tile_e[tstart[tid] + u] = tid;
      tile_g0[tstart[tid] + u] = gstart[tid] + 2 * u;
      tile_ng[tstart[tid] + u] = min(2, groups - 2 * u);
    }
  }
}

// ---------------------------------------------------------------- 3. scatter
__global__ __launch_bounds__(256) void moe_scatter_kernel(const int* __restrict__ ids, int R, int topk, int E,
                                                          const int* __restrict__ blk_off,
                                                          const int* __restrict__ seg_off,
                                                          int* __restrict__ sorted_row) {
  __shared__ int wcnt[4][kMoeMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * kMoeMaxExperts; i += 256) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const int rows = kRouteTokens * topk;
  const int r = blockIdx.x * rows + tid;
  const bool valid = tid < rows && r < R;
  const int e = valid ? ids[r] : -1;
  // Rank among the lower lanes of this wave routed to the same expert.
  uint64_t todo = __ballot(valid);
  int local = 0;
  while (todo != 0) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int e0 = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(e == e0);
    if (e == e0) local = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == leader) wcnt[wave][e0] = __popcll(m);
    todo &= ~m;
  }
  __syncthreads();
  if (valid) {
    int pos = seg_off[e] + blk_off[(int64_t)blockIdx.x * E + e] + local;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
    sorted_row[pos] = r;
  }
}

// ---------------------------------------------------------------- 4. gather
// The token rows are MX-quantized once, row-major (quant.hip's row-major
// kernel, into xq / xs with one extra all-zero row T for pad positions); the
// gate/up GEMM then copies its activation rows straight from xq by row index.
// What remains is the scale tile of the expert-sorted operand, in the packed
// lane-major layout: one thread per 4-byte word w of the 256-byte block of
// (group g, step ks), which holds MX block w & 1 of the step for the rows
// (w >> 1) + 32 i, i = 0..3 (byte i).  Pad rows get scale byte 0.  Block 0
// also clears row T of xq.
__global__ __launch_bounds__(256) void moe_gather_scales_kernel(const uint8_t* __restrict__ xs, int H, int topk,
                                                                const int* __restrict__ sorted_row,
                                                                const int* __restrict__ meta, int KS,
                                                                uint8_t* __restrict__ a1s,
                                                                uint8_t* __restrict__ zero_row) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x * 16; i < H; i += 256 * 16) *reinterpret_cast<uint4*>(zero_row + i) = make_uint4(0, 0, 0, 0);
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over (p_max / 128) * KS * 64
  const int64_t blk = t >> 6;                                    // g * KS + ks
  const int64_t g = blk / KS;
  if (g >= meta[1]) return;
  const int ks = (int)(blk - g * KS);
  const int w = (int)(t & 63);
  const int b = w & 1, r0 = w >> 1;
  const int nb = H / 32;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int src = sorted_row[g * kGroupRows + r0 + 32 * i];
    const uint32_t sb = src >= 0 ? xs[(int64_t)(src / topk) * nb + 2 * ks + b] : 0u;
    word |= sb << (8 * i);
  }
  *reinterpret_cast<uint32_t*>(a1s + blk * kTileScaleBytes + 4 * w) = word;
}

// ---------------------------------------------------------------- 5. gemm1
// Persistent over the (M-tile, 256-row slice nt of W13[e]) list, on the
// 16x16x128 tile loop (tile::persistent16_run).  Packed W13 row p of an
// expert's slice nt holds, for wave half wn = (p / 128) % 2 and q = p % 128:
// gate row nt*128 + wn*64 + q (q < 64) or up row I + nt*128 + wn*64 + q - 64
// (q >= 64).  In the loop's lane layout acc[a][b][j] (a < 4) is then the gate
// and acc[a + 4][b][j] the up value of intermediate index
// i = nt*128 + wn*64 + 16a + 4g + j, for tile row m = wm*128 + 16b + li
// (lane = li + 16 g): gate and up of one index meet in one lane.
// The activation rows are copied from the token rows of xq by row index
// (GBufSrc).  The row indices of the workgroup's next tile are copied into
// LDS at the start of the current one, so building its copy source needs no
// global load while copies are in flight.
struct Moe1Job {
  const uint8_t *wga, *wgb, *swa, *swb, *sxa, *sxb;
  uint32_t rowoff[4];   // byte offsets in xq of tile rows tid / 4 + 64 i
  int g0, ng, nt;
};

__global__ __launch_bounds__(tile::kThreads, 1) void moe_gemm1_kernel(
    const uint8_t* __restrict__ xq, int T, int topk, const uint8_t* __restrict__ a1s,
    const uint8_t* __restrict__ w13p, const uint8_t* __restrict__ s13p, const int* __restrict__ meta,
    const int* __restrict__ tile_e, const int* __restrict__ tile_g0, const int* __restrict__ tile_ng,
    const int* __restrict__ sorted_row, int H, int I, uint8_t* __restrict__ a2q, uint8_t* __restrict__ a2s,
    uint16_t* __restrict__ dbg_act, uint8_t* __restrict__ dbg_q, uint8_t* __restrict__ dbg_s) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[tile::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[tile::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[tile::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st3[tile::kStage];
  __shared__ __attribute__((aligned(16))) int rowbuf[256];   // sorted_row of the next tile's rows
  const int NT = (2 * I) / 256;
  const int total = meta[0] * NT;
  const int KS = H / kStepK, KS2 = I / kStepK;
  const size_t op_stride = (size_t)KS * kTileBytes, sc_stride = (size_t)KS * kTileScaleBytes;
  const uint32_t xq_bytes = (uint32_t)(((int64_t)T + 1) * H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  auto decode = [&](int bidx, bool later) {
    const int logical = tile::xcd_remap(bidx, total);
    const int mt = logical / NT, nt = logical % NT;
    const int e = tile_e[mt], g0 = tile_g0[mt], ng = tile_ng[mt];
    const uint8_t* we = w13p + (size_t)e * (size_t)(2 * I) * (size_t)H;
    const uint8_t* se = s13p + (size_t)e * (size_t)(2 * I) * (size_t)(H / 32);
    Moe1Job j;
    j.wga = we + (2 * nt) * op_stride;
    j.wgb = we + (2 * nt + 1) * op_stride;
    j.swa = se + (2 * nt) * sc_stride;
    j.swb = se + (2 * nt + 1) * sc_stride;
    j.sxa = a1s + (size_t)g0 * sc_stride;
    j.sxb = a1s + (size_t)(g0 + 1) * sc_stride;
    j.g0 = g0;
    j.ng = ng;
    j.nt = nt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Row T of xq is all zero: pad rows and rows past the tile's groups.
      const int m = (tid >> 2) + 64 * i;
      int tok = T;
      if (m < ng * kGroupRows) {
        const int src = later ? rowbuf[m] : sorted_row[g0 * kGroupRows + m];
        if (src >= 0) tok = src / topk;
      }
      j.rowoff[i] = (uint32_t)tok * (uint32_t)H;
    }
    return j;
  };
  auto make_src = [&](const Moe1Job& j) {
    return tile::GBufSrc(j.wga, j.wgb, j.swa, j.swb, j.sxa, j.sxb, xq, xq_bytes, j.rowoff, KS);
  };
  auto tile_start = [&](int bnext) {
    if (bnext >= total) return;
    const int mt = tile::xcd_remap(bnext, total) / NT;
    const int g0 = tile_g0[mt], ng = tile_ng[mt];
    // Wave w copies rows 64 w .. 64 w + 63 (past the tile's groups: zeros, unused).
    const tile::i4v r = tile::buffer_rsrc(sorted_row + (size_t)g0 * kGroupRows, (uint32_t)(ng * kGroupRows * 4));
    tile::b2l_4((uint32_t)((wave * 64 + lane) * 4), r, 0u, reinterpret_cast<const uint8_t*>(rowbuf) + wave * 256);
  };
  // The tile's two groups of the gated operand and of its scales, as buffers
  // (rows outside the tile's groups are given an offset past the end, so
  // every wave issues the same 48 stores per tile).
  const int64_t qgroup = (int64_t)KS2 * kTileBytes, sgroup = (int64_t)KS2 * kTileScaleBytes;
  auto epilogue = [&](const v4f (&acc)[8][8], const Moe1Job& j, const uint8_t*) {
    const int ks = 2 * j.nt + wn;                 // the 64-K step of this wave's intermediate indices
    const int valid = j.ng * kGroupRows;
    const __amdgpu_buffer_rsrc_t qb = raw_rsrc(a2q + (size_t)j.g0 * qgroup, (uint32_t)(2 * qgroup));
    const __amdgpu_buffer_rsrc_t sbuf = raw_rsrc(a2s + (size_t)j.g0 * sgroup, (uint32_t)(2 * sgroup));
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const int ml = wm * 128 + 16 * bb + li;     // row inside the tile
      const bool row_ok = ml < valid;
      const int pos = j.g0 * kGroupRows + ml;
      const int g = pos / kGroupRows, rr = pos % kGroupRows;
      const int src = (dbg_act != nullptr && row_ok) ? sorted_row[pos] : -1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // MX block h of the step: a = 2h, 2h + 1 of this lane and of the
        // lanes li + 16 g' (32 values).  Gated activation rounded to bf16,
        // value e = 4t + jj being a = 2h + t, j = jj.
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float o[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int e = 2 * p + hh, a = 2 * h + (e >> 2), jj = e & 3;
            // silu(g) = g / (1 + e^-g), with e^-g = 2^(-g log2 e) from the
            // hardware exp2 and the hardware reciprocal (each within about an
            // ulp of fp32; far below the bf16 rounding that follows).  For
            // g < -88 the exponential overflows to +inf and silu(g) -> 0.
            const float gt = acc[a][bb][jj], up = acc[a + 4][bb][jj];
            const float ex = __builtin_amdgcn_exp2f(-gt * 1.44269504088896341f);
            o[hh] = gt * __builtin_amdgcn_rcpf(1.0f + ex) * up;
          }
          w[p] = pack_bf16x2(o[0], o[1]);
        }
        u16x2 mp = {0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p) mp = absmax_pk(mp, w[p]);
        uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
        // Maximum over the four lanes li + 16 g' (rows of 16 lanes): the
        // gfx950 row swaps with both operands m give the exchanges with the
        // lanes 16 and 32 apart as VALU operations (no LDS permute, whose
        // queue the next tile's copies fill at this point).
        {
          const auto s16 = __builtin_amdgcn_permlane16_swap(m, m, false, false);
          m = max((uint32_t)s16[0], (uint32_t)s16[1]);
          const auto s32 = __builtin_amdgcn_permlane32_swap(m, m, false, false);
          m = max((uint32_t)s32[0], (uint32_t)s32[1]);
        }
        const uint32_t sb = (uint32_t)max((int)(m >> 7) - 8, 0);
        uint32_t q[2];
        cvt8s(w, mx_scale_value(sb), q);
        {
          // bytes j = 0..3 of a = 2h + t sit at k = 16a + 4g + j of step ks
          const uint32_t gq = (uint32_t)((g - j.g0) * qgroup), gs = (uint32_t)((g - j.g0) * sgroup);
          const uint32_t o0 = gq + (uint32_t)packed_off(rr, ks, 2 * h, KS2) + 4 * lg;
          const uint32_t o1 = gq + (uint32_t)packed_off(rr, ks, 2 * h + 1, KS2) + 4 * lg;
          const uint32_t os = gs + (uint32_t)(ks * kTileScaleBytes + scale_off(rr, h));
          const uint32_t off_end = 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b32(q[0], qb, (int)(row_ok ? o0 : off_end), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(q[1], qb, (int)(row_ok ? o1 : off_end), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, sbuf, (int)(row_ok && lg == 0 ? os : off_end), 0, 0);
        }
        if (src >= 0) {
          const int iblk = j.nt * 128 + wn * 64 + 32 * h;     // first intermediate index of the block
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int i0 = iblk + 16 * t + 4 * lg;
            uint16_t* da = dbg_act + (int64_t)src * I + i0;
            da[0] = (uint16_t)w[2 * t];
            da[1] = (uint16_t)(w[2 * t] >> 16);
            da[2] = (uint16_t)w[2 * t + 1];
            da[3] = (uint16_t)(w[2 * t + 1] >> 16);
            *reinterpret_cast<uint32_t*>(dbg_q + (int64_t)src * I + i0) = q[t];
          }
          if (lg == 0) dbg_s[(int64_t)src * (I / 32) + iblk / 32] = (uint8_t)sb;
        }
      }
    }
    return dbg_act != nullptr ? 0 : 48;   // (the debug copies' stores depend on the rows)
  };
  tile::persistent16_run<0, 0, true, false, false>(st0, st1, st2, st3, nullptr, total, KS, decode, make_src,
                                                   [](const Moe1Job&) { return tile::buffer_rsrc(nullptr, 0); },
                                                   [](tile::i4v, uint8_t*) {}, tile_start,
                                                   [](v4f (&)[8][8], const uint8_t*) {}, epilogue);
}

// ---------------------------------------------------------------- 6. gemm2
// Persistent over the (M-tile, 256-row slice of W2[e]) list on the same
// loop.  Side data of a tile: the sorted_row entries of its 256 rows (wave
// w copies rows 64 w ..), so the epilogue finds each row's slot row t*k + j
// in LDS.  Epilogue: each row's fp32 accumulators, as they are, staged 16
// rows x 64 columns at a time through the wave's LDS region and stored as
// whole 256-byte row segments, four rows per store (storing each lane's 4
// columns straight from the accumulators, 64-byte pieces of 16 rows per
// store, was 4 % slower on the layer).  The routing weight is applied by the
// combine: multiplying here took every accumulator through VGPRs, and the
// kernel then spilled inside its MFMA loop.  Pad rows and rows past the
// tile's groups go to the spare row R, so every wave issues exactly 64
// stores per tile.
struct Moe2Job {
  const uint8_t *wga, *wgb, *xga, *xgb, *swa, *swb, *sxa, *sxb;
  const int* rows;      // sorted_row of the tile's first row
  int ng, col0;
};

__global__ __launch_bounds__(tile::kThreads, 1) void moe_gemm2_kernel(
    const uint8_t* __restrict__ a2q, const uint8_t* __restrict__ a2s, const uint8_t* __restrict__ w2p,
    const uint8_t* __restrict__ s2p, const int* __restrict__ meta, const int* __restrict__ tile_e,
    const int* __restrict__ tile_g0, const int* __restrict__ tile_ng, const int* __restrict__ sorted_row,
    int p_max, int H, int I, int R, float* __restrict__ ys) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[tile::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[tile::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[tile::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st3[tile::kStage];
  constexpr int kRowSlot = 256 * 4;               // the tile's 256 slot rows
  __shared__ __attribute__((aligned(16))) uint8_t side[2 * kRowSlot];
  constexpr int kPitchF = 68;                     // fp32 per staged row (64 + 4 pad)
  __shared__ __attribute__((aligned(16))) float stage_epi[4][16 * kPitchF];
  const int NT = H / 256;
  const int total = meta[0] * NT;
  const int KS = I / kStepK;
  const size_t op_stride = (size_t)KS * kTileBytes, sc_stride = (size_t)KS * kTileScaleBytes;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  auto decode = [&](int bidx, bool) {
    const int logical = tile::xcd_remap(bidx, total);
    const int mt = logical / NT, nt = logical % NT;
    const int e = tile_e[mt], g0 = tile_g0[mt], ng = tile_ng[mt];
    const uint8_t* we = w2p + (size_t)e * (size_t)H * (size_t)I;
    const uint8_t* se = s2p + (size_t)e * (size_t)H * (size_t)(I / 32);
    Moe2Job j;
    j.wga = we + (2 * nt) * op_stride;
    j.wgb = we + (2 * nt + 1) * op_stride;
    j.xga = a2q + (size_t)g0 * op_stride;
    j.xgb = a2q + (size_t)(g0 + 1) * op_stride;
    j.swa = se + (2 * nt) * sc_stride;
    j.swb = se + (2 * nt + 1) * sc_stride;
    j.sxa = a2s + (size_t)g0 * sc_stride;
    j.sxb = a2s + (size_t)(g0 + 1) * sc_stride;
    j.rows = sorted_row + (size_t)g0 * kGroupRows;
    j.ng = ng;
    j.col0 = nt * 256;
    return j;
  };
  auto make_src = [&](const Moe2Job& j) {
    return tile::BufSrc(j.wga, j.wgb, j.xga, j.xgb, j.swa, j.swb, j.sxa, j.sxb, KS, KS);
  };
  // One resource from the tile's first sorted row to the end of sorted_row
  // (p_max entries): rows g0 * 128 .. + 255 are in range (p_max holds a
  // spare group).
  auto side_of = [&](const Moe2Job& j) {
    return tile::buffer_rsrc(j.rows, (uint32_t)(((int64_t)p_max - (j.rows - sorted_row)) * 4));
  };
  auto side_copy = [&](tile::i4v r, uint8_t* slot) {
    tile::b2l_4((uint32_t)((wave * 64 + lane) * 4), r, 0u, slot + wave * 256);
  };
  auto epilogue = [&](const v4f (&acc)[8][8], const Moe2Job& j, const uint8_t* slot) {
    const int* rmap = reinterpret_cast<const int*>(slot);
    const int valid = j.ng * kGroupRows;
    float* reg = stage_epi[wave];
    const int rr = lane >> 4, cc = (lane & 15) * 4;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // Rows 16 k .. + 15 of the wave's block, columns 64 hf .. + 63: staged
        // (a wave's LDS operations run in order: no waits), read back as 16
        // lanes per row, stored as 4 whole 256-byte row segments.
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<v4f*>(reg + li * kPitchF + 16 * a + 4 * lg) = acc[4 * hf + a][k];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4f v = *reinterpret_cast<const v4f*>(reg + (rr + 4 * q) * kPitchF + cc);
          const int ml = wm * 128 + 16 * k + rr + 4 * q;
          const int sr = rmap[ml];
          const bool real = ml < valid && sr >= 0;
          *reinterpret_cast<v4f*>(ys + (size_t)(real ? sr : R) * H + j.col0 + wn * 128 + 64 * hf + cc) = v;
        }
      }
    }
    return 64;
  };
  tile::persistent16_run<1, kRowSlot, false, false, false>(st0, st1, st2, st3, side, total, KS, decode, make_src,
                                                           side_of, side_copy, [](int) {},
                                                           [](v4f (&)[8][8], const uint8_t*) {}, epilogue);
}

// ---------------------------------------------------------------- 7. combine
// Each product is rounded to fp32 before it is added (contraction into
// fused multiply-adds is off in the loop), as the sum's definition has it.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ ys,
                                                          const float* __restrict__ wts, int T, int H, int topk,
                                                          uint16_t* __restrict__ y) {
  const int64_t t4 = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one thread per 8 columns of a token
  const int per_row = H / 8;
  if (t4 >= (int64_t)T * per_row) return;
  const int64_t t = t4 / per_row;
  const int c = (int)(t4 - t * per_row);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
#pragma clang fp contract(off)
    const float* r = ys + (t * topk + j) * H + c * 8;
    const float w = wts[t * topk + j];
    const float4 a = *reinterpret_cast<const float4*>(r), b = *reinterpret_cast<const float4*>(r + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] += w * v[i];
  }
  *reinterpret_cast<uint4*>(y + t * H + c * 8) = make_uint4(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]),
                                                            pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7]));
}

// ---------------------------------------------------------------- launcher
int launch_moe(const MoeArgs& a, hipStream_t stream) {
  const int nblk = (int)((a.T + kRouteTokens - 1) / kRouteTokens);
  const int R = (int)(a.T * a.topk);
  hipLaunchKernelGGL(moe_route_kernel, dim3(nblk), dim3(1024), 0, stream, a.logits, (int)a.T, (int)a.E,
                     (int)a.topk, a.ws.ids, a.ws.wts, a.ws.blk_cnt, nblk, (const uint16_t*)a.x, (int)a.H, a.ws.xq,
                     a.ws.xs, a.ws.sorted_row, (int)a.ws.p_max);
  if (a.dbg_ids != nullptr) {
    hipMemcpyAsync(a.dbg_ids, a.ws.ids, (size_t)R * 4, hipMemcpyDeviceToDevice, stream);
    hipMemcpyAsync(a.dbg_wts, a.ws.wts, (size_t)R * 4, hipMemcpyDeviceToDevice, stream);
  }
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(1024), 0, stream, a.ws.blk_cnt, nblk, (int)a.E, a.ws.blk_off,
                     a.ws.seg_off, a.ws.tile_e, a.ws.tile_g0, a.ws.tile_ng, a.ws.meta);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(nblk), dim3(256), 0, stream, a.ws.ids, R, (int)a.topk, (int)a.E,
                     a.ws.blk_off, a.ws.seg_off, a.ws.sorted_row);
  const int KS1 = (int)(a.H / kStepK);
  hipLaunchKernelGGL(moe_gather_scales_kernel, dim3((unsigned)(a.ws.p_max / kGroupRows * KS1 / 4)), dim3(256), 0,
                     stream, a.ws.xs, (int)a.H, (int)a.topk, a.ws.sorted_row, a.ws.meta, KS1, a.ws.a1s,
                     a.ws.xq + a.T * a.H);
  // Both GEMMs are persistent: at most one workgroup per CU (a multiple of 8,
  // one per XCD each), each running tiles b, b + grid, ... of the device-side
  // tile list; workgroups past its length return at once.
  const int64_t nt1 = 2 * a.I / 256, nt2 = a.H / 256;
  const int cus = device_cu_count();
  const int64_t pgrid = cus >= 8 ? cus - cus % 8 : cus;
  const unsigned g1 = (unsigned)std::min<int64_t>(a.ws.mt_max * nt1, pgrid);
  const unsigned g2 = (unsigned)std::min<int64_t>(a.ws.mt_max * nt2, pgrid);
  hipLaunchKernelGGL(moe_gemm1_kernel, dim3(g1), dim3(tile::kThreads), 0, stream,
                     a.ws.xq, (int)a.T, (int)a.topk, a.ws.a1s, (const uint8_t*)a.w13p, (const uint8_t*)a.s13p, a.ws.meta, a.ws.tile_e,
                     a.ws.tile_g0, a.ws.tile_ng, a.ws.sorted_row, (int)a.H, (int)a.I, a.ws.a2q, a.ws.a2s,
                     (uint16_t*)a.dbg_act, (uint8_t*)a.dbg_q, (uint8_t*)a.dbg_s);
  hipLaunchKernelGGL(moe_gemm2_kernel, dim3(g2), dim3(tile::kThreads), 0, stream, a.ws.a2q, a.ws.a2s,
                     (const uint8_t*)a.w2p, (const uint8_t*)a.s2p, a.ws.meta, a.ws.tile_e, a.ws.tile_g0,
                     a.ws.tile_ng, a.ws.sorted_row, (int)a.ws.p_max, (int)a.H, (int)a.I, R, a.ws.ys);
  const int64_t cb_total = a.T * (a.H / 8);
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((cb_total + 255) / 256)), dim3(256), 0, stream, a.ws.ys,
                     a.ws.wts, (int)a.T, (int)a.H, (int)a.topk, (uint16_t*)a.y);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
