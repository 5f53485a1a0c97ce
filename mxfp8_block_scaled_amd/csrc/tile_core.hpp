// The K loop of the 256 x 256 block-scaled MXFP8 tile shared by the dense
// layer's GEMM and the two grouped GEMMs of the MoE layer: both operands in
// the packed tile layout of common.hpp, fp32 accumulators in AGPRs.
//
// Design (gfx950):
//  * Workgroup tile 256 (n, weight rows) x 256 (m, activation rows), 4 waves
//    as 2 x 2, each wave 128 x 128 = 4 x 4 v_mfma_scale_f32_32x32x64_f8f6f4
//    tiles.  The weight is the MFMA A operand, so lane (li, lg) of wave
//    (wn, wm) ends with acc[a][b][r] = D[n = wn*128 + 32a + 8(r/4) + 4lg + r%4]
//    [m = wm*128 + 32b + li].
//  * A stage is four contiguous 4 KiB runs (two 128-row groups per operand)
//    and four 256-byte scale runs, copied straight into LDS by
//    global_load_lds_dwordx4 / _dword (no VGPR staging).
//  * K advances 64 per stage; four LDS stages (4 x 33 KiB).  Each stage lives
//    in its own __shared__ array and the loop is unrolled by four, so every
//    LDS access names a distinct array: the compiler then needs no blanket
//    vmcnt(0) before the fragment reads, and the loop waits only for the
//    stage it is about to use (partial vmcnt).
//  * Software pipeline per 64-K step s: the MFMA operands of s are already in
//    registers; each of the step's 16 MFMAs is followed by one of the 9 copies
//    of step s+4 (into the buffer that held s) and by a slice of the LDS
//    fragment reads of step s+1.  The copies then trickle into the memory
//    pipeline at the MFMA rate instead of stalling the wave in a burst, and
//    the fragment reads are hidden under the MFMAs.  One barrier per step.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mxfp8 {
namespace tile {

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 (indices usable
// as compile-time constants, e.g. MFMA op_sel values).
template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

constexpr int kThreads = 256;
constexpr int kOpBytes = 256 * kStepK;                // one operand's 256 rows x 64 K-bytes
constexpr int kScaleRegion = 1024;                    // 256 x 2 B weight + 256 x 2 B activation scales
constexpr int kStage = 2 * kOpBytes + kScaleRegion;   // 33792
constexpr int kLoadsPerStage = 9;                     // per thread: 4 + 4 data, 1 scale

// Direct global -> LDS copies (each lane moves 16 or 4 bytes to
// lds_wave_base + lane * size).  Issued from inline assembly so that the
// compiler does not track them: the loop orders them itself with explicit
// vmcnt waits, and the compiler's own waits for its own global loads can only
// be more conservative, never less.  The ISA needs one wait state between the
// m0 write and the LDS-DMA load that reads it.
__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }
__device__ inline void g2l_16(const void* g, const uint8_t* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr(lds_wave_base))
               : "memory", "m0");
}
__device__ inline void g2l_4(const void* g, const uint8_t* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr(lds_wave_base))
               : "memory", "m0");
}

using mxfp8::xcd_remap;

template <int N>
__device__ inline void wait_vmcnt() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == kLoadsPerStage) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else if constexpr (N == 2 * kLoadsPerStage) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(27)" ::: "memory");
}

// Row-gathered activation operand: instead of a packed group, the 16 bytes
// thread tid copies for tile row m and step ks come from p[i] + ks * 64,
// where i = 0..3 stands for m = tid / 4 + 64 i and p[i] points at that row's
// source (a row-major E4M3 matrix with K bytes per row) plus the logical
// 16-byte chunk that lands in LDS slot tid % 4 of the packed layout, i.e.
// chunk (tid % 4) ^ ((tid / 16) % 4).
struct GatherX {
  const uint8_t* p[4];
};

// acc = the tile's product over all KS 64-K steps.  wga / wgb: the packed
// weight groups of tile rows 0-127 / 128-255 at step 0; xga / xgb: the packed
// activation groups (kGatherX: unused, gx gives the rows instead); swa, swb,
// sxa, sxb: the scale tiles of all four at step 0 (always packed).
// KS must be a multiple of 4 and at least 4.  Every thread of the 256-thread
// workgroup calls this; st0..st3 are the workgroup's four stage arrays.
template <bool kGatherX = false>
__device__ __forceinline__ void mainloop(uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3,
                                         const uint8_t* wga, const uint8_t* wgb, const uint8_t* xga,
                                         const uint8_t* xgb, const uint8_t* swa, const uint8_t* swb,
                                         const uint8_t* sxa, const uint8_t* sxb, int KS, v16f (&acc)[4][4],
                                         GatherX gx = {}) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
  const uint8_t* w0 = wga + tid * 16;
  const uint8_t* w1 = wgb + tid * 16;
  const uint8_t* x0 = xga + tid * 16;
  const uint8_t* x1 = xgb + tid * 16;
  // Scale words: wave 0 weight rows 0-127, 1 weight rows 128-255, 2
  // activation rows 0-127, 3 activation rows 128-255.
  const uint8_t* ssrc = (wave == 0 ? swa : wave == 1 ? swb : wave == 2 ? sxa : sxb) + lane * 4;


#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // Fragments of one 64-deep K step (both operands, with the scale bytes of
  // the lane's rows: lane group lg supplies MX block lg of the step).
  struct Frags {
    v8i a[4], b[4];
    int sa, sb;     // scale bytes of the lane's 4 rows (byte i: row li + 32 i)
  };
  // Lane offsets inside a stage: rows R0 + 32 i share the swizzle of R0
  // (swz depends on bits 2-3 of the row only), so fragment i is 2048 i bytes
  // further; the scales of the lane's four rows are one 4-byte word.
  const int offWa = tile_off(wn * 128 + li, lg), offWb = tile_off(wn * 128 + li, 2 + lg);
  const int offXa = kOpBytes + tile_off(wm * 128 + li, lg), offXb = kOpBytes + tile_off(wm * 128 + li, 2 + lg);
  const int offSw = 2 * kOpBytes + wn * kTileScaleBytes + scale_off(li, lg);
  const int offSx = 2 * kOpBytes + 2 * kTileScaleBytes + wm * kTileScaleBytes + scale_off(li, lg);
  auto rd16 = [](const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); };
  // Copy j (0..8) of this thread's share of step ks into stage st.
  auto dma_one = [&](int j, int ks, uint8_t* st) {
    uint8_t* base = st + wave * 1024;
    const size_t off = (size_t)ks * kTileBytes;
    switch (j) {
      case 0: g2l_16(w0 + off, base); break;
      case 1: g2l_16(w0 + off + 4096, base + 4096); break;
      case 2: g2l_16(w1 + off, base + 8192); break;
      case 3: g2l_16(w1 + off + 4096, base + 12288); break;
      case 4:
        if constexpr (kGatherX) g2l_16(gx.p[0] + (size_t)ks * kStepK, base + kOpBytes);
        else g2l_16(x0 + off, base + kOpBytes);
        break;
      case 5:
        if constexpr (kGatherX) g2l_16(gx.p[1] + (size_t)ks * kStepK, base + kOpBytes + 4096);
        else g2l_16(x0 + off + 4096, base + kOpBytes + 4096);
        break;
      case 6:
        if constexpr (kGatherX) g2l_16(gx.p[2] + (size_t)ks * kStepK, base + kOpBytes + 8192);
        else g2l_16(x1 + off, base + kOpBytes + 8192);
        break;
      case 7:
        if constexpr (kGatherX) g2l_16(gx.p[3] + (size_t)ks * kStepK, base + kOpBytes + 12288);
        else g2l_16(x1 + off + 4096, base + kOpBytes + 12288);
        break;
      default: g2l_4(ssrc + (size_t)ks * kTileScaleBytes, st + 2 * kOpBytes + wave * 256); break;
    }
  };
  // Part j (0..15) of the fragment reads of a stage (parts 8..15 are empty).
  // The scale words go first: read after the fragments (parts 8, 9) they
  // cost the loop about 12 % (measured).
  auto read_part = [&](int j, const uint8_t* st, Frags& f) {
    if (j == 0) f.sa = *reinterpret_cast<const int*>(st + offSw);
    if (j == 1) f.sb = *reinterpret_cast<const int*>(st + offSx);
    if (j < 8) {
      const int i = j >> 1;
      if ((j & 1) == 0) {
        const uint4 a0 = rd16(st + offWa + 2048 * i), a1 = rd16(st + offWb + 2048 * i);
        f.a[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      } else {
        const uint4 b0 = rd16(st + offXa + 2048 * i), b1 = rd16(st + offXb + 2048 * i);
        f.b[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
    }
  };

  // One K step s.  On entry the fragments of s are in registers (cur) and
  // the copies of s+1 .. s+3 are in flight.  Wait until s+1 has landed in
  // every wave (own vmcnt, then the barrier); then each of the 16 MFMAs of s
  // is followed by one copy of s+4 (into the buffer that held s) and one
  // part of the fragment reads of s+1, so the copy and read traffic is spread
  // over the MFMA stream.  Before the next barrier every wave drains its LDS
  // reads, so the buffer of s+1 may be refilled after it.
  auto step = [&](auto do_issue, auto later, auto do_next, int s, uint8_t* st_free, const uint8_t* st_next,
                  const Frags& cur, Frags& nxt) {
    wait_vmcnt<decltype(later)::value * kLoadsPerStage>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 16>([&](auto J) {
      constexpr int j = decltype(J)::value;
      // op_sel picks byte (row block) j >> 2 of the weight scales and j & 3
      // of the activation scales.
      acc[j >> 2][j & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          cur.a[j >> 2], cur.b[j & 3], acc[j >> 2][j & 3], 0, 0, j >> 2, cur.sa, j & 3, cur.sb);
      if constexpr (decltype(do_issue)::value) {
        if (j < kLoadsPerStage) dma_one(j, s + 4, st_free);
      }
      if constexpr (decltype(do_next)::value) read_part(j, st_next, nxt);
      __builtin_amdgcn_sched_barrier(0);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  using T = std::true_type;
  using F = std::false_type;
  using L0 = std::integral_constant<int, 0>;
  using L1 = std::integral_constant<int, 1>;
  using L2 = std::integral_constant<int, 2>;

  // KS is a multiple of 4 (K % 256 == 0) and at least 4.
  Frags f0, f1;
  // Stage-major issue order: vmcnt retires loads in order, so "at most 27
  // outstanding" means all of stage 0 has landed.
#pragma unroll
  for (int j = 0; j < kLoadsPerStage; ++j) dma_one(j, 0, st0);
#pragma unroll
  for (int j = 0; j < kLoadsPerStage; ++j) dma_one(j, 1, st1);
#pragma unroll
  for (int j = 0; j < kLoadsPerStage; ++j) dma_one(j, 2, st2);
#pragma unroll
  for (int j = 0; j < kLoadsPerStage; ++j) dma_one(j, 3, st3);
  wait_vmcnt<3 * kLoadsPerStage>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int j = 0; j < 16; ++j) read_part(j, st0, f0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  int ks = 0;
  for (; ks + 8 <= KS; ks += 4) {
    step(T{}, L2{}, T{}, ks, st0, st1, f0, f1);
    step(T{}, L2{}, T{}, ks + 1, st1, st2, f1, f0);
    step(T{}, L2{}, T{}, ks + 2, st2, st3, f0, f1);
    step(T{}, L2{}, T{}, ks + 3, st3, st0, f1, f0);
  }
  // Last four steps: nothing left to copy.
  step(F{}, L2{}, T{}, ks, st0, st1, f0, f1);
  step(F{}, L1{}, T{}, ks + 1, st1, st2, f1, f0);
  step(F{}, L0{}, T{}, ks + 2, st2, st3, f0, f1);
  step(F{}, L0{}, F{}, ks + 3, st3, st0, f1, f0);

}


constexpr int kEpiPitch = 132;                        // floats per staged row (128 + 4 pad)

// The layer's epilogue for one tile: y[m][n] = bf16(acc + bias[n]) for tile
// rows m with row0 + m < row_end and columns col0 + n < N (bias may be null).
// Lane (li, lg) holds n = 32a + 8(r/4) + 4lg + r%4, m = 32b + li of its
// wave's 128 x 128 block.  Each wave stages 64 rows (b = 2h, 2h+1) at a time
// in its own LDS stage buffer, then reads them back as 4 consecutive n per
// lane (a wave instruction covers two whole 256-byte output row segments),
// adds the bias in fp32 and rounds once to bf16.  vec_store: y is 8-byte
// aligned and ldy % 4 == 0.  The stage buffers must be free (the K loop is
// over in every wave).  kRowScale: tile row m is first multiplied by
// row_scale[m] (an LDS array of 256 floats), i.e. bf16(acc * s[m] + bias[n]).
// OutT = float writes the fp32 values instead (no rounding; 16-byte stores,
// requires y 16-byte aligned and ldy % 4 == 0 when vec_store).  kRowMap:
// tile row m goes to output row row_map[m] (an LDS array of 256 ints; a
// negative entry is not stored) instead of row0 + m, row_end is not used,
// and every column of the tile must be < N with vec_store set.
template <bool kRowScale = false, typename OutT = uint16_t, bool kRowMap = false>
__device__ __forceinline__ void store_bf16(uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3,
                                           const v16f (&acc)[4][4], OutT* __restrict__ y, int64_t ldy,
                                           int row0, int row_end, int col0, int N,
                                           const uint16_t* __restrict__ bias, int vec_store,
                                           const float* row_scale = nullptr, const int* row_map = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
  // Lane (li, lg) holds n = 32a + 8(r/4) + 4lg + r%4, m = 32b + li of the
  // wave's 128 x 128 block.  Stage 64 rows (b = 2h, 2h+1) at a time in this
  // wave's own LDS buffer, then read them back as 4 consecutive n per lane
  // (a wave instruction covers two whole 256-byte output row segments).
  float* stage = reinterpret_cast<float*>(wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3);
  const int n4 = lane & 31;
  const int rsub = lane >> 5;
  const int nl = col0 + wn * 128 + 4 * n4;
  float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (bias != nullptr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float b = __uint_as_float((uint32_t)bias[min(nl + e, N - 1)] << 16);
      bv[e] = (nl + e < N) ? b : 0.0f;
    }
  }
  const bool full_n = nl + 3 < N;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const v16f& v = acc[a][2 * h + b2];
          float4 f = make_float4(v[4 * rr], v[4 * rr + 1], v[4 * rr + 2], v[4 * rr + 3]);
          *reinterpret_cast<float4*>(stage + (32 * b2 + li) * kEpiPitch + 32 * a + 8 * rr + 4 * lg) = f;
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int m_first = row0 + wm * 128 + 64 * h + rsub;
    const int rows_left = row_end - m_first;          // this lane's rows are m_first + 2 it
    const float* src = stage + rsub * kEpiPitch + 4 * n4;
    OutT* dst = y + (size_t)max(m_first, 0) * ldy + nl;
    if constexpr (kRowMap) {
#pragma unroll
      for (int it = 0; it < 32; ++it) {
        float4 f = *reinterpret_cast<const float4*>(src + 2 * it * kEpiPitch);
        const int tm = m_first - row0 + 2 * it;
        if constexpr (kRowScale) {
          const float sc = row_scale[tm];
          f.x *= sc; f.y *= sc; f.z *= sc; f.w *= sc;
        }
        const int dr = row_map[tm];
        if (dr >= 0) {
          OutT* d = y + (size_t)dr * ldy + nl;
          if constexpr (sizeof(OutT) == 4) {
            *reinterpret_cast<float4*>(d) = make_float4(f.x + bv[0], f.y + bv[1], f.z + bv[2], f.w + bv[3]);
          } else {
            *reinterpret_cast<uint2*>(d) =
                make_uint2(pack_bf16x2(f.x + bv[0], f.y + bv[1]), pack_bf16x2(f.z + bv[2], f.w + bv[3]));
          }
        }
      }
    } else if (vec_store && full_n && rows_left >= 63) {
#pragma unroll
      for (int it = 0; it < 32; ++it) {
        float4 f = *reinterpret_cast<const float4*>(src + 2 * it * kEpiPitch);
        if constexpr (kRowScale) {
          const float sc = row_scale[m_first - row0 + 2 * it];
          f.x *= sc; f.y *= sc; f.z *= sc; f.w *= sc;
        }
        if constexpr (sizeof(OutT) == 4) {
          *reinterpret_cast<float4*>(dst + (size_t)(2 * it) * ldy) =
              make_float4(f.x + bv[0], f.y + bv[1], f.z + bv[2], f.w + bv[3]);
        } else {
          *reinterpret_cast<uint2*>(dst + (size_t)(2 * it) * ldy) =
              make_uint2(pack_bf16x2(f.x + bv[0], f.y + bv[1]), pack_bf16x2(f.z + bv[2], f.w + bv[3]));
        }
      }
    } else if (nl < N) {
      for (int it = 0; 2 * it < rows_left && it < 32; ++it) {
        float4 f = *reinterpret_cast<const float4*>(src + 2 * it * kEpiPitch);
        if constexpr (kRowScale) {
          const float sc = row_scale[m_first - row0 + 2 * it];
          f.x *= sc; f.y *= sc; f.z *= sc; f.w *= sc;
        }
        OutT* d = dst + (size_t)(2 * it) * ldy;
        if constexpr (sizeof(OutT) == 4) {
          d[0] = f.x + bv[0];
          if (nl + 1 < N) d[1] = f.y + bv[1];
          if (nl + 2 < N) d[2] = f.z + bv[2];
          if (nl + 3 < N) d[3] = f.w + bv[3];
        } else {
          const uint32_t lo = pack_bf16x2(f.x + bv[0], f.y + bv[1]);
          const uint32_t hi = pack_bf16x2(f.z + bv[2], f.w + bv[3]);
          d[0] = (uint16_t)lo;
          if (nl + 1 < N) d[1] = (uint16_t)(lo >> 16);
          if (nl + 2 < N) d[2] = (uint16_t)hi;
          if (nl + 3 < N) d[3] = (uint16_t)(hi >> 16);
        }
      }
    }
    // The next half overwrites the same rows: finish the reads first.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

}  // namespace tile
}  // namespace mxfp8
