// The K loops of the 256 x 256 block-scaled MXFP8 tile: mainloop16 (the
// dense layer's GEMM, on 16x16x128 MFMAs, described at its definition) and
// mainloop (the two grouped GEMMs of the MoE layer, on 32x32x64 MFMAs).  Both
// read operands in the packed tile layout of common.hpp and keep fp32
// accumulators in AGPRs.
//
// Design of mainloop (gfx950):
//  * Workgroup tile 256 (n, weight rows) x 256 (m, activation rows), 4 waves
//    as 2 x 2, each wave 128 x 128 = 4 x 4 v_mfma_scale_f32_32x32x64_f8f6f4
//    tiles.  The weight is the MFMA A operand, so lane (li, lg) of wave
//    (wn, wm) ends with acc[a][b][r] = D[n = wn*128 + 32a + 8(r/4) + 4lg + r%4]
//    [m = wm*128 + 32b + li].
//  * A stage is sixteen 1 KiB pieces (two 128-row groups per operand, eight
//    16-row bands each) and four 256-byte scale runs, copied straight into
//    LDS by global_load_lds_dwordx4 / _dword (no VGPR staging).
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

typedef int i4v __attribute__((ext_vector_type(4)));

// Buffer resource (raw, untyped) over [base, base + bytes): loads past the
// end return zeros instead of touching memory.
__device__ inline i4v buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  // The descriptor lives in scalar registers: every lane holds the same
  // value, and readfirstlane says so to the compiler.
  i4v r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));     // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;                   // 32-bit data format, no swizzle
  return r;
}
// Buffer -> LDS copies: lane l moves 16 (or 4) bytes from base + voff + soff
// to lds_wave_base + 16 l (or 4 l).  The per-lane offset is fixed for the
// whole loop and the step advances in the scalar offset, so a copy costs no
// vector address arithmetic.
__device__ inline void b2l_16(uint32_t voff, i4v rsrc, uint32_t soff, const uint8_t* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(soff), "s"(lds_addr(lds_wave_base))
               : "memory", "m0");
}
__device__ inline void b2l_4(uint32_t voff, i4v rsrc, uint32_t soff, const uint8_t* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(soff), "s"(lds_addr(lds_wave_base))
               : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are
// outstanding (they retire in issue order).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt takes 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

// This thread's share of one 64-K stage: nine copies, j = 0..3 the weight
// rows (bands 0-3 and 4-7 of each 128-row group: wave w copies the 1 KiB
// piece of band w, resp. w + 4), 4..7 the activation rows, 8 the wave's
// 256-byte scale run (wave 0 weight rows 0-127, 1 weight rows 128-255, 2
// activation rows 0-127, 3 activation rows 128-255).  KSband: the steps of
// the operand's full K (the distance between bands is KSband pieces).
template <bool kGatherX>
struct StageSrc {
  const uint8_t *w0, *w1, *x0, *x1, *ssrc;
  size_t hi;                 // from band w to band w + 4
  GatherX gx;
  int wave;

  __device__ __forceinline__ StageSrc(const uint8_t* wga, const uint8_t* wgb, const uint8_t* xga,
                                      const uint8_t* xgb, const uint8_t* swa, const uint8_t* swb,
                                      const uint8_t* sxa, const uint8_t* sxb, GatherX g, int KSband) {
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t lo = (size_t)wave * KSband * kPieceBytes + (tid & 63) * 16;
    hi = (size_t)4 * KSband * kPieceBytes;
    w0 = wga + lo;
    w1 = wgb + lo;
    x0 = xga + lo;
    x1 = xgb + lo;
    ssrc = (wave == 0 ? swa : wave == 1 ? swb : wave == 2 ? sxa : sxb) + (tid & 63) * 4;
    gx = g;
  }

  // Copy j of step ks into stage st.
  __device__ __forceinline__ void issue(int j, int ks, uint8_t* st) const {
    uint8_t* base = st + wave * 1024;
    const size_t off = (size_t)ks * kPieceBytes;
    switch (j) {
      case 0: g2l_16(w0 + off, base); break;
      case 1: g2l_16(w0 + hi + off, base + 4096); break;
      case 2: g2l_16(w1 + off, base + 8192); break;
      case 3: g2l_16(w1 + hi + off, base + 12288); break;
      case 4:
        if constexpr (kGatherX) g2l_16(gx.p[0] + (size_t)ks * kStepK, base + kOpBytes);
        else g2l_16(x0 + off, base + kOpBytes);
        break;
      case 5:
        if constexpr (kGatherX) g2l_16(gx.p[1] + (size_t)ks * kStepK, base + kOpBytes + 4096);
        else g2l_16(x0 + hi + off, base + kOpBytes + 4096);
        break;
      case 6:
        if constexpr (kGatherX) g2l_16(gx.p[2] + (size_t)ks * kStepK, base + kOpBytes + 8192);
        else g2l_16(x1 + off, base + kOpBytes + 8192);
        break;
      case 7:
        if constexpr (kGatherX) g2l_16(gx.p[3] + (size_t)ks * kStepK, base + kOpBytes + 12288);
        else g2l_16(x1 + hi + off, base + kOpBytes + 12288);
        break;
      default: g2l_4(ssrc + (size_t)ks * kTileScaleBytes, st + 2 * kOpBytes + wave * 256); break;
    }
  }
};

// The same nine copies per 64-K stage as StageSrc, as buffer loads (packed
// operands only).  The group pointers may start inside the group's K (a
// split-K slice: step ks0 of every band); KSband is the full K's step count,
// the distance between bands.  A group holds at most 2^32 bytes (K < 2^25).
struct BufSrc {
  i4v w0, w1, x0, x1, sc;
  uint32_t vlo, vhi, soff_lane;
  int wave;

  BufSrc() = default;

  __device__ __forceinline__ BufSrc(const uint8_t* wga, const uint8_t* wgb, const uint8_t* xga,
                                    const uint8_t* xgb, const uint8_t* swa, const uint8_t* swb,
                                    const uint8_t* sxa, const uint8_t* sxb, int KS, int KSband) {
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t data = (uint32_t)KSband * kTileBytes, scales = (uint32_t)KS * kTileScaleBytes;
    w0 = buffer_rsrc(wga, data);
    w1 = buffer_rsrc(wgb, data);
    x0 = buffer_rsrc(xga, data);
    x1 = buffer_rsrc(xgb, data);
    sc = buffer_rsrc(wave == 0 ? swa : wave == 1 ? swb : wave == 2 ? sxa : sxb, scales);
    vlo = (uint32_t)wave * KSband * kPieceBytes + (uint32_t)(tid & 63) * 16;
    vhi = vlo + 4u * KSband * kPieceBytes;
    soff_lane = (uint32_t)(tid & 63) * 4;
  }

  __device__ __forceinline__ void issue(int j, int ks, uint8_t* st) const {
    uint8_t* base = st + wave * 1024;
    const uint32_t off = (uint32_t)ks * kPieceBytes;
    switch (j) {
      case 0: b2l_16(vlo, w0, off, base); break;
      case 1: b2l_16(vhi, w0, off, base + 4096); break;
      case 2: b2l_16(vlo, w1, off, base + 8192); break;
      case 3: b2l_16(vhi, w1, off, base + 12288); break;
      case 4: b2l_16(vlo, x0, off, base + kOpBytes); break;
      case 5: b2l_16(vhi, x0, off, base + kOpBytes + 4096); break;
      case 6: b2l_16(vlo, x1, off, base + kOpBytes + 8192); break;
      case 7: b2l_16(vhi, x1, off, base + kOpBytes + 12288); break;
      default: b2l_4(soff_lane, sc, (uint32_t)ks * kTileScaleBytes, st + 2 * kOpBytes + wave * 256); break;
    }
  }
};

// BufSrc with a row-gathered activation operand: the 16 bytes thread tid
// copies for tile row m = tid / 4 + 64 i (i = 0..3) in 64-K step ks come from
// byte vx[i] + 64 ks of a row-major E4M3 matrix (resource xr, one row of K
// bytes per token), vx[i] being the row's offset plus the logical chunk that
// lands in LDS slot tid % 4 of the packed layout, chunk (tid % 4) ^ swz(m).
// Weights and all four scale tiles are packed, as in BufSrc.
struct GBufSrc {
  i4v w0, w1, xr, sc;
  uint32_t vlo, vhi, soff_lane;
  uint32_t vx[4];
  int wave;

  GBufSrc() = default;

  __device__ __forceinline__ GBufSrc(const uint8_t* wga, const uint8_t* wgb, const uint8_t* swa,
                                     const uint8_t* swb, const uint8_t* sxa, const uint8_t* sxb,
                                     const uint8_t* xrows, uint32_t xrows_bytes, const uint32_t (&rowoff)[4],
                                     int KS) {
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t data = (uint32_t)KS * kTileBytes, scales = (uint32_t)KS * kTileScaleBytes;
    w0 = buffer_rsrc(wga, data);
    w1 = buffer_rsrc(wgb, data);
    xr = buffer_rsrc(xrows, xrows_bytes);
    sc = buffer_rsrc(wave == 0 ? swa : wave == 1 ? swb : wave == 2 ? sxa : sxb, scales);
    vlo = (uint32_t)wave * KS * kPieceBytes + (uint32_t)(tid & 63) * 16;
    vhi = vlo + 4u * KS * kPieceBytes;
    soff_lane = (uint32_t)(tid & 63) * 4;
    const uint32_t chunk = (uint32_t)(((tid & 3) ^ swz(tid >> 2)) * 16);   // rows tid / 4 + 64 i share it
#pragma unroll
    for (int i = 0; i < 4; ++i) vx[i] = rowoff[i] + chunk;
  }

  __device__ __forceinline__ void issue(int j, int ks, uint8_t* st) const {
    uint8_t* base = st + wave * 1024;
    const uint32_t off = (uint32_t)ks * kPieceBytes, xoff = (uint32_t)ks * kStepK;
    switch (j) {
      case 0: b2l_16(vlo, w0, off, base); break;
      case 1: b2l_16(vhi, w0, off, base + 4096); break;
      case 2: b2l_16(vlo, w1, off, base + 8192); break;
      case 3: b2l_16(vhi, w1, off, base + 12288); break;
      case 4: b2l_16(vx[0], xr, xoff, base + kOpBytes); break;
      case 5: b2l_16(vx[1], xr, xoff, base + kOpBytes + 4096); break;
      case 6: b2l_16(vx[2], xr, xoff, base + kOpBytes + 8192); break;
      case 7: b2l_16(vx[3], xr, xoff, base + kOpBytes + 12288); break;
      default: b2l_4(soff_lane, sc, (uint32_t)ks * kTileScaleBytes, st + 2 * kOpBytes + wave * 256); break;
    }
  }
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
  const StageSrc<kGatherX> src(wga, wgb, xga, xgb, swa, swb, sxa, sxb, gx, KS);

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
  auto dma_one = [&](int j, int ks, uint8_t* st) { src.issue(j, ks, st); };
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


// c += A x B on v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 operands, the
// accumulator updated in place in AGPRs.  Written as inline assembly because
// the compiler, given the builtin in this loop, gives most of the 64
// accumulators a new destination on every MFMA and then shuffles them with
// hundreds of AGPR/VGPR copies per step.  op_sel / op_sel_hi carry bit 0 /
// bit 1 of the byte each scale operand is taken from.  The assembly is
// opaque to the compiler's hazard checks, so it carries its own: two wait
// states in front (a VALU write of a source register needs them before an
// MFMA reads it; the operands normally come straight from LDS reads, which
// the compiler's lgkmcnt waits cover); an accumulator is read again only 64
// MFMAs later inside the loop, and the loop ends with enough wait states
// before the epilogue reads the accumulators.
template <int kSelA, int kSelB>
__device__ __forceinline__ void mfma16(v4f& c, const v8i& a, const v8i& b, int sa, int sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0]"
               : "+a"(c)
               : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(kSelA & 1), "n"(kSelB & 1), "n"(kSelA >> 1), "n"(kSelB >> 1));
}

// c += A x B with A (the weight) in E2M1: one 16-byte register quad per lane
// holds K [32g, 32g + 32) of the lane's row (cbsz:4 selects the format); the
// scales and everything else as in mfma16.
template <int kSelA, int kSelB>
__device__ __forceinline__ void mfma16w4(v4f& c, const i4v& a, const v8i& b, int sa, int sb) {
  asm volatile(
      "s_nop 1\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0] cbsz:4"
      : "+a"(c)
      : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(kSelA & 1), "n"(kSelB & 1), "n"(kSelA >> 1), "n"(kSelB >> 1));
}

// Copy source of the 4-bit weight tile (persistent16_run<..., kW4 = true>).
// A step buffer of 50 KiB holds one 128-K step: the weights as packed MXFP4
// (a 128-K step of a 16-row band is one 1 KiB piece, bands KS/2 pieces
// apart: 16 KiB for the 256 rows at offset 0), the activations' even and odd
// 64-K stages at kOpBytes and 2 kOpBytes (as in a stage pair), and the scale
// tiles of the two 64-K steps (weights and activations, 1 KiB each) at
// 3 kOpBytes and 3 kOpBytes + 1024.  issue(j, s, st): j = 0..3 weight pieces
// of 128-K step s (bands w, w + 4 of the two groups), 4..7 activation pieces
// of 64-K step s as BufSrc, 8 and 9 the wave's 256-byte scale run of 64-K
// step s into the even or odd scale slot.
struct W4Src {
  i4v w0, w1, x0, x1, sc;
  uint32_t wlo, whi, xlo, xhi, soff_lane;
  int wave;

  W4Src() = default;

  __device__ __forceinline__ W4Src(const uint8_t* wga, const uint8_t* wgb, const uint8_t* xga, const uint8_t* xgb,
                                   const uint8_t* swa, const uint8_t* swb, const uint8_t* sxa, const uint8_t* sxb,
                                   int KS) {
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KS4 = KS / 2;
    w0 = buffer_rsrc(wga, (uint32_t)KS4 * kTileBytes);
    w1 = buffer_rsrc(wgb, (uint32_t)KS4 * kTileBytes);
    x0 = buffer_rsrc(xga, (uint32_t)KS * kTileBytes);
    x1 = buffer_rsrc(xgb, (uint32_t)KS * kTileBytes);
    sc = buffer_rsrc(wave == 0 ? swa : wave == 1 ? swb : wave == 2 ? sxa : sxb, (uint32_t)KS * kTileScaleBytes);
    wlo = (uint32_t)wave * KS4 * kPieceBytes + (uint32_t)(tid & 63) * 16;
    whi = wlo + 4u * KS4 * kPieceBytes;
    xlo = (uint32_t)wave * KS * kPieceBytes + (uint32_t)(tid & 63) * 16;
    xhi = xlo + 4u * KS * kPieceBytes;
    soff_lane = (uint32_t)(tid & 63) * 4;
  }

  __device__ __forceinline__ void issue(int j, int s, uint8_t* st) const {
    uint8_t* base = st + wave * 1024;
    const uint32_t off = (uint32_t)s * kPieceBytes;
    switch (j) {
      case 0: b2l_16(wlo, w0, off, base); break;
      case 1: b2l_16(whi, w0, off, base + 4096); break;
      case 2: b2l_16(wlo, w1, off, base + 8192); break;
      case 3: b2l_16(whi, w1, off, base + 12288); break;
      case 4: b2l_16(xlo, x0, off, base + kOpBytes); break;
      case 5: b2l_16(xhi, x0, off, base + kOpBytes + 4096); break;
      case 6: b2l_16(xlo, x1, off, base + kOpBytes + 8192); break;
      case 7: b2l_16(xhi, x1, off, base + kOpBytes + 12288); break;
      case 8: b2l_4(soff_lane, sc, (uint32_t)s * kTileScaleBytes, st + 3 * kOpBytes + wave * 256); break;
      default: b2l_4(soff_lane, sc, (uint32_t)s * kTileScaleBytes, st + 3 * kOpBytes + 1024 + wave * 256); break;
    }
  }
};
constexpr int kW4Buf = 3 * kOpBytes + 2048;          // 51200: one 128-K step of the 4-bit tile

// The same 256 x 256 tile on v_mfma_scale_f32_16x16x128_f8f6f4.  A 16x16x128
// MFMA does the work of half a 32x32x64 one with the same operand bytes per
// flop and a quarter of the accumulator traffic, and on gfx950 the chip
// sustains a higher clock on it under a full MFMA load (measured: 8 % more
// MFMA throughput than 32x32x64 at the power limit).
//
//  * Each wave's 128 x 128 block is 8 x 8 MFMA tiles of 16 x 16; lane (i, g)
//    (i = lane % 16, g = lane / 16) ends with acc[a][b][j] =
//    D[n = wn*128 + 16a + 4g + j][m = wm*128 + 16b + i].
//  * One MFMA consumes 128 K: bytes K [16g, 16g+16) come from chunk g of the
//    even 64-K tile and K [64+16g, ...) from chunk g of the odd one, so a
//    128-K step reads a pair of the 64-K stages (st0, st1 or st2, st3); the
//    global layout and the copies are those of the 64-K loop.
//  * Per step: all eight weight fragments (64 registers) and the scale words
//    stay in registers for the whole step; the activation fragment of tile
//    column b + 2 is read from LDS during the eight MFMAs of column b.  So the
//    weight half and the scales of a stage pair are consumed at the end of
//    the previous step, the activation half only during the step: the
//    weight-and-scale copies of step p + 2 go out after a barrier early in
//    step p (after its first column), the activation copies after a second
//    barrier before column 6, once every wave holds its last activation
//    fragment of the pair.
//  * Scale words: lane (i, g) supplies MX block g of the step, i.e. block
//    g % 2 of tile g / 2; word e holds rows 16e + i + 32k (byte k), so tile a
//    uses word a % 2, op_sel a / 2.
__device__ __forceinline__ void mainloop16(uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3,
                                           const uint8_t* wga, const uint8_t* wgb, const uint8_t* xga,
                                           const uint8_t* xgb, const uint8_t* swa, const uint8_t* swb,
                                           const uint8_t* sxa, const uint8_t* sxb, int KS, v4f (&acc)[8][8],
                                           int KSband = 0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 15, lg = lane >> 4;
  const BufSrc src(wga, wgb, xga, xgb, swa, swb, sxa, sxb, KS, KSband > 0 ? KSband : KS);

#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // Registers carried from step to step: the eight weight fragments and the
  // scale words of the current step, and four activation fragment buffers
  // (column b in buffer b % 4; columns 0 and 1 are in place at the start of
  // a step).  A weight fragment is overwritten with the next step's right
  // after its last MFMA.
  struct State {
    v8i a[8];
    v8i bf[4];
    int sa[2], sb[2];
  };
  // Rows R0 + 16 a share the swizzle of R0, so tile a is 1024 a bytes further.
  const int offA = tile_off(wn * 128 + li, lg);
  const int offB = kOpBytes + tile_off(wm * 128 + li, lg);
  // Scale word e of the lane: tile lg / 2 of the pair, block lg % 2.
  const int offS = 2 * kOpBytes + scale_off(li, lg & 1);
  const int swA = wn * kTileScaleBytes, swB = 2 * kTileScaleBytes + wm * kTileScaleBytes;
  auto rd16 = [](const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); };
  auto frag = [&](const uint8_t* ev, const uint8_t* od, int off) {
    const uint4 lo = rd16(ev + off), hi = rd16(od + off);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto rd_scale = [&](const uint8_t* ev, const uint8_t* od, int base, int e) {
    const uint8_t* st = (lg >> 1) ? od : ev;
    return *reinterpret_cast<const int*>(st + offS + base + 128 * e);
  };
  // Weight-and-scale copies of step q into pair (ev, od): ten per thread;
  // activation copies: eight.
  auto issue_w = [&](int k, int q, uint8_t* ev, uint8_t* od) {
    const int t = k / 5, c = k % 5;
    src.issue(c < 4 ? c : 8, 2 * q + t, t ? od : ev);
  };
  auto issue_x = [&](int k, int q, uint8_t* ev, uint8_t* od) {
    const int t = k >> 2;
    src.issue(4 + (k & 3), 2 * q + t, t ? od : ev);
  };

  // One 128-K step p on pair (ev, od); (nev, nod) holds step p + 1.  No
  // LDS wait sits at a step boundary: the reads of step p + 1 issued in the
  // last columns have at least eight MFMAs to land before their first use,
  // and activation column b + 2 is read during column b.
  auto step = [&](auto do_issue, auto do_next, int p, uint8_t* ev, uint8_t* od, const uint8_t* nev,
                  const uint8_t* nod, State& S) {
    int nsa[2], nsb[2];
    static_for<0, 64>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int b = j >> 3, a = j & 7;
      if constexpr (j == 8) {
        // Every wave has read this pair's weight half and scales (end of the
        // previous step): the copies of step p + 2 may overwrite them.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (j == 48) {
        // Columns 6 and 7: every wave holds its last activation fragment of
        // this pair, and step p + 1 has landed (the only copies issued since
        // are the ten weight-and-scale copies of step p + 2).
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<decltype(do_issue)::value ? 10 : 0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma16<(a >> 1), (b >> 1)>(acc[a][b], S.a[a], S.bf[b & 3], S.sa[a & 1], S.sb[b & 1]);
      if constexpr (decltype(do_issue)::value) {
        if constexpr (j >= 8 && j < 18) issue_w(j - 8, p + 2, ev, od);
        if constexpr (j >= 48 && j < 56) issue_x(j - 48, p + 2, ev, od);
      }
      if constexpr (a == 0 && b < 6) S.bf[(b + 2) & 3] = frag(ev, od, offB + 1024 * (b + 2));
      if constexpr (decltype(do_next)::value) {
        if constexpr (j == 48) {
          nsa[0] = rd_scale(nev, nod, swA, 0);
          nsa[1] = rd_scale(nev, nod, swA, 1);
          S.bf[0] = frag(nev, nod, offB);              // column 4 was the last user
        }
        if constexpr (j == 49) { nsb[0] = rd_scale(nev, nod, swB, 0); nsb[1] = rd_scale(nev, nod, swB, 1); }
        if constexpr (j == 56) S.bf[1] = frag(nev, nod, offB + 1024);   // column 5 was the last user
        if constexpr (j >= 56) S.a[a] = frag(nev, nod, offA + 1024 * a);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (decltype(do_next)::value) {
      S.sa[0] = nsa[0]; S.sa[1] = nsa[1];
      S.sb[0] = nsb[0]; S.sb[1] = nsb[1];
    }
  };
  using T = std::true_type;
  using F = std::false_type;

  const int P = KS / 2;      // 128-K steps: even, at least 2
  State S;
  // Issue order: weights+scales of step 0, activations of step 0, then step 1.
#pragma unroll
  for (int k = 0; k < 10; ++k) issue_w(k, 0, st0, st1);
#pragma unroll
  for (int k = 0; k < 8; ++k) issue_x(k, 0, st0, st1);
#pragma unroll
  for (int k = 0; k < 10; ++k) issue_w(k, 1, st2, st3);
#pragma unroll
  for (int k = 0; k < 8; ++k) issue_x(k, 1, st2, st3);
  asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  S.sa[0] = rd_scale(st0, st1, swA, 0);
  S.sa[1] = rd_scale(st0, st1, swA, 1);
  S.sb[0] = rd_scale(st0, st1, swB, 0);
  S.sb[1] = rd_scale(st0, st1, swB, 1);
#pragma unroll
  for (int a = 0; a < 8; ++a) S.a[a] = frag(st0, st1, offA + 1024 * a);
  S.bf[0] = frag(st0, st1, offB);
  S.bf[1] = frag(st0, st1, offB + 1024);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  int p = 0;
  for (; p + 4 <= P; p += 2) {
    step(T{}, T{}, p, st0, st1, st2, st3, S);
    step(T{}, T{}, p + 1, st2, st3, st0, st1, S);
  }
  step(F{}, T{}, p, st0, st1, st2, st3, S);
  step(F{}, F{}, p + 1, st2, st3, st0, st1, S);
  // The last MFMAs must retire before anything reads the accumulators.
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
}

// Staging of one 64-row half (m = 64 h .. 64 h + 63 of the wave's block) into
// the wave's LDS buffer as rows of 128 fp32 n values, pitch kEpiPitch.
template <int kPitch>
__device__ __forceinline__ void stage_half(float* stage, const v16f (&acc)[4][4], int h, int lane) {
  const int li = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const v16f& v = acc[a][2 * h + b2];
        float4 f = make_float4(v[4 * rr], v[4 * rr + 1], v[4 * rr + 2], v[4 * rr + 3]);
        *reinterpret_cast<float4*>(stage + (32 * b2 + li) * kPitch + 32 * a + 8 * rr + 4 * lg) = f;
      }
}
template <int kPitch>
__device__ __forceinline__ void stage_half(float* stage, const v4f (&acc)[8][8], int h, int lane) {
  const int li = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b2 = 0; b2 < 4; ++b2) {
      const v4f& v = acc[a][4 * h + b2];
      *reinterpret_cast<float4*>(stage + (16 * b2 + li) * kPitch + 16 * a + 4 * lg) =
          make_float4(v[0], v[1], v[2], v[3]);
    }
}

constexpr int kEpiPitch = 132;                        // floats per staged row (128 + 4 pad)

// The layer's epilogue for one tile: y[m][n] = bf16(acc + bias[n]) for tile
// rows m with row0 + m < row_end and columns col0 + n < N (bias may be null).
// acc is either loop's accumulator set (v16f[4][4] of the 32x32x64 loop or
// v4f[8][8] of the 16x16x128 one).  Each wave stages 64 rows at a time
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
template <bool kRowScale = false, typename OutT = uint16_t, bool kRowMap = false, typename Acc>
__device__ __forceinline__ void store_bf16(uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3,
                                           const Acc& acc, OutT* __restrict__ y, int64_t ldy,
                                           int row0, int row_end, int col0, int N,
                                           const uint16_t* __restrict__ bias, int vec_store,
                                           const float* row_scale = nullptr, const int* row_map = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  // Stage 64 rows of the wave's 128 x 128 block at a time in this wave's own
  // LDS buffer (stage_half, for either accumulator layout), then read them
  // back as 4 consecutive n per lane (a wave instruction covers two whole
  // 256-byte output row segments).
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
    stage_half<kEpiPitch>(stage, acc, h, lane);
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

// Epilogue of the 16x16x128 loop (the dense layer): y[m][n] = OutT(acc +
// bias[n]) for tile rows m with row0 + m < row_end and columns col0 + n < N.
// OutT = uint16_t: bf16 (one rounding after the fp32 bias add), written with
// non-temporal stores (the output is not read again, so it need not displace
// operand tiles in L2); OutT = float: the fp32 values (split-K partials; bias
// must be null).  Each wave stages 64 rows of its 128 x 128 block at a time in
// its own LDS stage buffer and reads them back so that a lane holds 8
// consecutive columns of one row: lanes 16G + 8r + q (G = 0..3, r = 0..1,
// q = 0..7) take row 2 (G / 2) + r of a 4-row pass and columns
// 64 (G % 2) + 8 q ..+7; a store instruction then covers 4 whole 256-byte
// row segments (bf16), and the 16 lanes of a read group hit 16 distinct LDS
// bank quads (the pitch of 132 floats shifts the second row by one quad).
// Reads are batched eight passes at a time before one wait.  vec_store: 2 =
// y 16-byte aligned and ldy % 8 == 0, 1 = 8-byte aligned and ldy % 4 == 0,
// 0 = neither.  The stage buffers must be free (the K loop is over in every
// wave).
template <typename OutT>
__device__ __forceinline__ void store16(uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3,
                                        const v4f (&acc)[8][8], OutT* __restrict__ y, int64_t ldy, int row0,
                                        int row_end, int col0, int N, const uint16_t* __restrict__ bias,
                                        int vec_store) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  float* stage = reinterpret_cast<float*>(wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3);
  const int G = lane >> 4, r = (lane >> 3) & 1, q = lane & 7;
  const int prow = 2 * (G >> 1) + r;
  const int nloc = 64 * (G & 1) + 8 * q;
  const int nl = col0 + wn * 128 + nloc;
  const bool full8 = nl + 7 < N;
  float bv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float b = 0.0f;
    if (bias != nullptr) b = __uint_as_float((uint32_t)bias[min(nl + e, N - 1)] << 16);
    bv[e] = (nl + e < N) ? b : 0.0f;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    stage_half<kEpiPitch>(stage, acc, h, lane);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int mbase = row0 + wm * 128 + 64 * h + prow;     // this lane's rows: mbase + 4 it
#pragma unroll
    for (int batch = 0; batch < 2; ++batch) {
      float4 lo[8], hi[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float* src = stage + (prow + 4 * (8 * batch + k)) * kEpiPitch + nloc;
        lo[k] = *reinterpret_cast<const float4*>(src);
        hi[k] = *reinterpret_cast<const float4*>(src + 4);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int m = mbase + 4 * (8 * batch + k);
        if (m >= row_end || nl >= N) continue;
        const float v[8] = {lo[k].x + bv[0], lo[k].y + bv[1], lo[k].z + bv[2], lo[k].w + bv[3],
                            hi[k].x + bv[4], hi[k].y + bv[5], hi[k].z + bv[6], hi[k].w + bv[7]};
        OutT* d = y + (size_t)m * ldy + nl;
        if constexpr (sizeof(OutT) == 4) {
          if (vec_store && full8) {
            *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
          } else {
            for (int e = 0; e < 8; ++e)
              if (nl + e < N) d[e] = v[e];
          }
        } else {
          const u4v w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7])};
          if (vec_store == 2 && full8) {
            __builtin_nontemporal_store(w, reinterpret_cast<u4v*>(d));
          } else if (vec_store == 1 && full8) {
            *reinterpret_cast<uint2*>(d) = make_uint2(w[0], w[1]);
            *reinterpret_cast<uint2*>(d + 4) = make_uint2(w[2], w[3]);
          } else {
            for (int e = 0; e < 8; ++e)
              if (nl + e < N) d[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent form of the 16x16x128 loop for the dense layer.  A workgroup
// runs tiles blockIdx.x, blockIdx.x + gridDim.x, ... and the copy stream
// never stops at a tile boundary: the last two steps of a tile copy the next
// tile's first two steps (the same slots and stage pairs as inside a tile),
// and the last step reads the next tile's first fragments.  The epilogue then
// runs with the next tile's data already in LDS and in registers, so no tile
// after the first waits for its prologue copies.  The epilogue stages through
// its own small LDS region (bf16, 16 rows per pass) instead of the stage
// buffers, which hold the next tile by then.  The bias of a tile (its 256
// columns, zeros past N) is copied into one of two LDS slots together with
// the tile's second step.
// ---------------------------------------------------------------------------
constexpr int kEpiRows = 16;                          // rows per staging pass
constexpr int kEpiPitchH = 136;                       // bf16 per staged row (128 + 8 pad)
constexpr int kEpiWaveBytes = kEpiRows * kEpiPitchH * 2;   // 4352
constexpr int kEpiBytes = 4 * kEpiWaveBytes;          // 17408
constexpr int kBiasSlot = 4 * 256;                    // one tile's bias: 256 B per wave
constexpr int kBiasBytes = 2 * kBiasSlot;

struct Job16 {
  const uint8_t *wga, *wgb, *xga, *xgb, *swa, *swb, *sxa, *sxb;
  int row0, col0;
};

// Resource over the bias of columns [col0, col0 + 256) that exist (none if
// bias is null): loads past the end read zeros.
__device__ inline i4v bias_rsrc(const uint16_t* bias, int col0, int N) {
  if (bias == nullptr) return buffer_rsrc(nullptr, 0);
  const int valid = max(0, min(256, N - col0));
  return buffer_rsrc(reinterpret_cast<const uint8_t*>(bias) + 2 * (size_t)col0, (uint32_t)valid * 2);
}

// The accumulators of a tile start at its bias (fp32, exact from bf16), so
// that the MFMAs add the products to it and the epilogue only rounds: this
// wave's 128 bias values are at bias_slot (zeros past N or without a bias);
// acc[a][k][e] is column 16 a + 4 lg + e of the wave's 128.
__device__ __forceinline__ void bias_init16(v4f (&acc)[8][8], const uint8_t* bias_slot) {
  const int lg = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const uint2 w = *reinterpret_cast<const uint2*>(bias_slot + (16 * a + 4 * lg) * 2);
    const v4f v = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[a][k] = v;
  }
}

// Epilogue of one tile of the persistent loop: y = bf16(acc) for rows
// < row_end and columns < N, the accumulators having started at the bias
// (bias_init16).  Wave (wn, wm) stages its 128 x 128 block 16 rows at a time
// as bf16 in its own kEpiWaveBytes region (lane (i, g) writes columns
// 16a + 4g .. +3 of row i for a = 0..7), reads each pass back as 8
// consecutive columns per lane (4 rows per read) and writes 16-byte
// non-temporal stores covering whole 256-byte row segments.  Returns true
// when the wave issued exactly 32 stores (block fully in range,
// vec_store == 2).
__device__ __forceinline__ bool epi16(uint8_t* epi, const v4f (&acc)[8][8], uint16_t* __restrict__ y, int64_t ldy,
                                      int row0, int row_end, int col0, int N, int vec_store) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 15, lg = lane >> 4;
  uint8_t* reg = epi + wave * kEpiWaveBytes;
  const int nw = col0 + wn * 128, mw = row0 + wm * 128;
  const bool full = vec_store == 2 && mw + 128 <= row_end && nw + 128 <= N;
  const int rr = lane >> 4, cc = (lane & 15) * 8;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const v4f v = acc[a][k];
      const uint2 w = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      *reinterpret_cast<uint2*>(reg + (li * kEpiPitchH + 16 * a + 4 * lg) * 2) = w;
    }
    // No waits around the read-back: a wave's LDS operations execute in
    // issue order, so the reads see this pass's writes and the next pass's
    // writes follow these reads; the stores wait for the read data.  (Same
    // output bit for bit; 1-1.5 % faster on prefill and the headline shape.)
    u4v t[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = *reinterpret_cast<const u4v*>(reg + ((rr + 4 * r) * kEpiPitchH + cc) * 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mw + 16 * k + rr + 4 * r, n = nw + cc;
      uint16_t* d = y + (size_t)m * ldy + n;
      if (full) {
        __builtin_nontemporal_store(t[r], reinterpret_cast<u4v*>(d));
      } else if (m < row_end && n < N) {
        if (vec_store == 2 && n + 7 < N) {
          *reinterpret_cast<u4v*>(d) = t[r];
        } else {
          for (int e = 0; e < 8; ++e)
            if (n + e < N) d[e] = (uint16_t)(t[r][e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
  return full;
}

// The persistent loop over any tile list.
//  * decode(b, later) gives tile b's job (any struct); later is false only
//    for the workgroup's first tile (decoded before any copy is in flight).
//  * make_src(job): its copy source (BufSrc or GBufSrc).
//  * Side data: kSide LDS-DMA copies per wave, issued by side_copy(side_of(job),
//    slot) together with the tile's second step into one of two slots of
//    kSideSlot bytes at side_lds (e.g. the tile's bias).  The epilogue of the
//    tile finds it there: epilogue(acc, job, slot) stores the tile and returns
//    the number of vector memory operations the wave issued in it when that
//    is exactly 32, 48 or 64 (the next tile's first wait then lets them stay
//    in flight), else 0.
//  * tile_start(b_next) runs at the start of each tile with the index of the
//    workgroup's next tile (may be >= total); vector memory operations it
//    issues are complete by the tile's first barrier after its first wait.
//  * kAccInit: acc_init(acc, slot) sets the tile's accumulators from its side
//    data (this wave's own copies, complete when it runs); otherwise they
//    start at zero.
//  * kCarry: the last step of a tile reads the next tile's first fragments
//    (held in registers through the epilogue); otherwise they are read from
//    LDS after the epilogue (their stage pair is not refilled before the
//    next tile's first barrier), which frees those registers for an
//    epilogue that needs them.
//  * kW4: the weight operand is packed MXFP4 (W4Src, mfma16w4): a 128-K step
//    is one step buffer of kW4Buf bytes, passed as (st0, st1) = (buffer 0,
//    buffer 0 + kOpBytes) and (st2, st3) likewise for buffer 1, so that the
//    activation stages sit where a stage pair puts them; six weight and scale
//    copies per step instead of ten.
// total: tiles of the list; gridDim.x % 8 == 0 keeps every workgroup's tiles
// on one XCD under xcd_remap.
template <int kSide, int kSideSlot, bool kCarry, bool kW4, bool kAccInit, typename Decode, typename MakeSrc,
          typename SideOf, typename SideCopy, typename TileStart, typename AccInit, typename Epilogue>
__device__ __forceinline__ void persistent16_run(uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3,
                                                 uint8_t* side_lds, int total, int KS, Decode decode,
                                                 MakeSrc make_src, SideOf side_of, SideCopy side_copy,
                                                 TileStart tile_start, AccInit acc_init, Epilogue epilogue) {
  static_assert(kSide >= 0 && kSide <= 4, "side copies per wave");
  int b = blockIdx.x;
  if (b >= total) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  using AFrag = typename std::conditional<kW4, i4v, v8i>::type;
  constexpr int kWCopies = kW4 ? 6 : 10;         // weight + scale copies per 128-K step
  struct State {
    AFrag a[8];
    v8i bf[4];
    int sa[2], sb[2];
  };
  const int offA = tile_off(wn * 128 + li, lg);
  const int offB = kOpBytes + tile_off(wm * 128 + li, lg);
  const int offS = 2 * kOpBytes + scale_off(li, lg & 1);
  const int swA = wn * kTileScaleBytes, swB = 2 * kTileScaleBytes + wm * kTileScaleBytes;
  auto rd16 = [](const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); };
  auto frag = [&](const uint8_t* ev, const uint8_t* od, int off) {
    const uint4 lo = rd16(ev + off), hi = rd16(od + off);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // The weight fragment of tile row block a: 32 bytes from the stage pair, or
  // (kW4) 16 bytes of the step buffer's 4-bit weights.
  auto frag_a = [&](const uint8_t* ev, const uint8_t* od, int a) -> AFrag {
    if constexpr (kW4) {
      const uint4 v = rd16(ev + offA + 1024 * a);
      return i4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    } else {
      return frag(ev, od, offA + 1024 * a);
    }
  };
  auto rd_scale = [&](const uint8_t* ev, const uint8_t* od, int base, int e) {
    if constexpr (kW4) {
      return *reinterpret_cast<const int*>(ev + 3 * kOpBytes + (lg >> 1) * 1024 + scale_off(li, lg & 1) + base +
                                           128 * e);
    } else {
      const uint8_t* st = (lg >> 1) ? od : ev;
      return *reinterpret_cast<const int*>(st + offS + base + 128 * e);
    }
  };
  using Job = decltype(decode(0, false));
  using Src = decltype(make_src(decode(0, false)));
  auto issue_w = [&](const Src& sr, int k, int q, uint8_t* ev, uint8_t* od) {
    if constexpr (kW4) {
      if (k < 4) sr.issue(k, q, ev);
      else sr.issue(4 + k, 2 * q + (k - 4), ev);      // scale slots 8, 9
    } else {
      const int t = k / 5, c = k % 5;
      sr.issue(c < 4 ? c : 8, 2 * q + t, t ? od : ev);
    }
  };
  auto issue_x = [&](const Src& sr, int k, int q, uint8_t* ev, uint8_t* od) {
    const int t = k >> 2;
    sr.issue(4 + (k & 3), 2 * q + t, t ? od : ev);
  };
  auto issue_side = [&](i4v r, int buf) { side_copy(r, side_lds + buf * kSideSlot); };

  v4f acc[8][8];
  State S;
  // One 128-K step on pair (ev, od); (nev, nod) holds the next step (of this
  // tile or the next).  Copies step q of sr into this pair when kIssue, or
  // (kRtIssue) when the runtime flag rt_issue is set: weights and scales
  // after column 1, activations after column 6, and with with_side also the
  // side data of sr's tile into slot bbuf.  The wait before column 6 needs the
  // next step's copies: besides the weight copies issued in this step (if
  // any), vm_extra stores of the previous epilogue may still be in flight
  // after them (32, 48 or 64, or 0 when unknown; with 64 the wait allows 63, the
  // counter's limit: the step's copies are older than all of them).  The next step's fragments are always
  // read (after the last tile they are stale and unused).
  auto step = [&](auto kIssue, auto kRtIssue, auto with_side, auto kVm, auto kNext, bool rt_issue, uint8_t* ev, uint8_t* od,
                  const uint8_t* nev, const uint8_t* nod, const Src& sr, int q, int vm_extra, i4v brs, int bbuf) {
    constexpr bool kI = decltype(kIssue)::value, kR = decltype(kRtIssue)::value;
    const bool issue = kI || (kR && rt_issue);
    int nsa[2], nsb[2];
    static_for<0, 64>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int bb = j >> 3, a = j & 7;
      if constexpr (j == 8) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (j == 48) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const bool extra = decltype(kVm)::value && vm_extra == 32;
        const bool extra48 = decltype(kVm)::value && vm_extra == 48;
        const bool extra64 = decltype(kVm)::value && vm_extra == 64;
        if constexpr (kI) {
          if (extra64) wait_vmcnt<63>();
          else if (extra48) wait_vmcnt<kWCopies + 48>();
          else if (extra) wait_vmcnt<kWCopies + 32>();
          else wait_vmcnt<kWCopies>();
        } else {
          if (extra64) {
            wait_vmcnt<63>();
          } else if (issue) {
            if (extra48) wait_vmcnt<kWCopies + 48>();
            else if (extra) wait_vmcnt<kWCopies + 32>();
            else wait_vmcnt<kWCopies>();
          } else {
            if (extra48) wait_vmcnt<48>();
            else if (extra) wait_vmcnt<32>();
            else wait_vmcnt<0>();
          }
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kW4) mfma16w4<(a >> 1), (bb >> 1)>(acc[a][bb], S.a[a], S.bf[bb & 3], S.sa[a & 1], S.sb[bb & 1]);
      else mfma16<(a >> 1), (bb >> 1)>(acc[a][bb], S.a[a], S.bf[bb & 3], S.sa[a & 1], S.sb[bb & 1]);
      if constexpr (kI || kR) {
        if (issue) {
          if constexpr (j >= 8 && j < 8 + kWCopies) issue_w(sr, j - 8, q, ev, od);
          if constexpr (j >= 48 && j < 56) issue_x(sr, j - 48, q, ev, od);
          if constexpr (decltype(with_side)::value && j == 56) issue_side(brs, bbuf);
        }
      }
      if constexpr (a == 0 && bb < 6) S.bf[(bb + 2) & 3] = frag(ev, od, offB + 1024 * (bb + 2));
      if constexpr (decltype(kNext)::value) {
        if constexpr (j == 48) {
          nsa[0] = rd_scale(nev, nod, swA, 0);
          nsa[1] = rd_scale(nev, nod, swA, 1);
          S.bf[0] = frag(nev, nod, offB);
        }
        if constexpr (j == 49) { nsb[0] = rd_scale(nev, nod, swB, 0); nsb[1] = rd_scale(nev, nod, swB, 1); }
        if constexpr (j == 56) S.bf[1] = frag(nev, nod, offB + 1024);
        if constexpr (j >= 56) S.a[a] = frag_a(nev, nod, a);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (decltype(kNext)::value) {
      S.sa[0] = nsa[0]; S.sa[1] = nsa[1];
      S.sb[0] = nsb[0]; S.sb[1] = nsb[1];
    }
  };
  // The first fragments of the step in (ev, od).
  auto read_first = [&](const uint8_t* ev, const uint8_t* od) {
    S.sa[0] = rd_scale(ev, od, swA, 0);
    S.sa[1] = rd_scale(ev, od, swA, 1);
    S.sb[0] = rd_scale(ev, od, swB, 0);
    S.sb[1] = rd_scale(ev, od, swB, 1);
#pragma unroll
    for (int a = 0; a < 8; ++a) S.a[a] = frag_a(ev, od, a);
    S.bf[0] = frag(ev, od, offB);
    S.bf[1] = frag(ev, od, offB + 1024);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  using T = std::true_type;
  using F = std::false_type;

  Job cur = decode(b, false);
  Src src = make_src(cur);
  // First tile: its two first steps and its bias, then its first fragments.
#pragma unroll
  for (int k = 0; k < kWCopies; ++k) issue_w(src, k, 0, st0, st1);
#pragma unroll
  for (int k = 0; k < 8; ++k) issue_x(src, k, 0, st0, st1);
#pragma unroll
  for (int k = 0; k < kWCopies; ++k) issue_w(src, k, 1, st2, st3);
#pragma unroll
  for (int k = 0; k < 8; ++k) issue_x(src, k, 1, st2, st3);
  if constexpr (kSide > 0) issue_side(side_of(cur), 0);
  wait_vmcnt<kWCopies + 8 + kSide>();
  __builtin_amdgcn_s_barrier();
  read_first(st0, st1);

  const int P = KS / 2;       // 128-K steps per tile: even, at least 2
  const i4v nob = buffer_rsrc(nullptr, 0);
  int vm_extra = 0, buf = 0;
  for (;;) {
    tile_start(b + (int)gridDim.x);
    if constexpr (kAccInit) {
      // The tile's side data is older than the previous epilogue's stores
      // (none before the first tile).
      if (vm_extra == 64) wait_vmcnt<63>();
      else if (vm_extra == 32) wait_vmcnt<32>();
      else wait_vmcnt<0>();
      acc_init(acc, side_lds + buf * kSideSlot);
    } else {
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      // (an AGPR-only definition of the zeros: the MoE GEMMs' register
      // allocation otherwise gives some accumulators VGPR homes and spills)
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) asm volatile("" : "+a"(acc[a][c]));
    }
    int p = 0;
    if (P >= 4) {
      // The first step alone may find the previous epilogue's stores in
      // flight (see step).
      step(T{}, F{}, F{}, T{}, T{}, true, st0, st1, st2, st3, src, 2, vm_extra, nob, 0);
      step(T{}, F{}, F{}, F{}, T{}, true, st2, st3, st0, st1, src, 3, 0, nob, 0);
      for (p = 2; p + 4 <= P; p += 2) {
        step(T{}, F{}, F{}, F{}, T{}, true, st0, st1, st2, st3, src, p + 2, 0, nob, 0);
        step(T{}, F{}, F{}, F{}, T{}, true, st2, st3, st0, st1, src, p + 3, 0, nob, 0);
      }
      vm_extra = 0;
    }
    // The next tile is decoded only now, so its sources do not occupy
    // registers during the loop above.  With no step above, what tile_start
    // issued has not been waited for yet: wait for it (and every wave's).
    if (P < 4) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
    }
    const int nb = b + (int)gridDim.x;
    const bool has_next = nb < total;
    const Job nxt = decode(has_next ? nb : b, true);
    const Src nsrc = make_src(nxt);
    step(F{}, T{}, F{}, T{}, T{}, has_next, st0, st1, st2, st3, nsrc, 0, vm_extra, nob, 0);
    step(F{}, T{}, std::integral_constant<bool, (kSide > 0)>{}, F{}, std::integral_constant<bool, kCarry>{}, has_next,
         st2, st3, st0, st1, nsrc, 1, 0, side_of(nxt), buf ^ 1);
    // The last MFMAs must retire before the epilogue reads the accumulators.
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    const int nvm = (int)epilogue(acc, cur, side_lds + buf * kSideSlot);
    if (!has_next) break;
    if constexpr (!kCarry) read_first(st0, st1);
    vm_extra = (nvm == 32 || nvm == 48 || nvm == 64) ? nvm : 0;
    src = nsrc;
    cur = nxt;
    b = nb;
    buf ^= 1;
  }
}

// The dense layer's persistent GEMM: tiles of packed operands, bf16 output
// with bias (epi16).
template <typename Decode>
__device__ __forceinline__ void persistent16(uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3, uint8_t* epi,
                                             uint8_t* bias_lds, int total, int KS, Decode decode,
                                             uint16_t* __restrict__ y, int64_t ldy, int M, int N,
                                             const uint16_t* __restrict__ bias, int vec_store) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1;
  // Side data: the tile's 256 bias values; wave w copies the 128 of its
  // columns (wn * 128 ..) into its own 256 bytes of the slot.
  persistent16_run<1, kBiasSlot, true, false, true>(
      st0, st1, st2, st3, bias_lds, total, KS, [&](int bidx, bool) { return decode(bidx); },
      [&](const Job16& j) { return BufSrc(j.wga, j.wgb, j.xga, j.xgb, j.swa, j.swb, j.sxa, j.sxb, KS, KS); },
      [&](const Job16& j) { return bias_rsrc(bias, j.col0, N); },
      [&](i4v r, uint8_t* slot) { b2l_4((uint32_t)(wn * 256 + lane * 4), r, 0u, slot + wave * 256); },
      [&](int) {}, [&](v4f (&acc)[8][8], const uint8_t* slot) { bias_init16(acc, slot + wave * 256); },
      [&](const v4f (&acc)[8][8], const Job16& j, const uint8_t*) {
        return epi16(epi, acc, y, ldy, j.row0, M, j.col0, N, vec_store) ? 32 : 0;
      });
}

}  // namespace tile
}  // namespace mxfp8
