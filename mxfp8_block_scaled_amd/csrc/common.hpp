// Shared device/host helpers of libmxfp8: MX block quantization, the packed
// weight layout, and the gfx950 scaled-MFMA operand conventions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Packed operand layout.  The one-time weight preparation writes it, and so
// does the activation quantizer of the large-M path (the same layout with M
// in place of N), so both GEMM operands are read the same way.  Rows are
// padded to a multiple of 128 ("pad N to 128" in the weight preparation step
// of vLLM PR #52204); K is a multiple of 256.  Rows are cut into 128-row
// groups, each group into eight 16-row bands, and K into 64-byte steps:
//
//   data[g]      = KS * 8 KiB, band-major: the 1 KiB piece of band b (rows
//                  16b .. 16b+15 of the group) and step ks sits at
//                  (b * KS + ks) * 1024, so one band is a contiguous run over
//                  the whole K (a decode workgroup that owns 16 rows streams
//                  one run: measured 4.1 us for a 16 MiB weight against
//                  4.7 us when each band is 1 KiB pieces at an 8 KiB stride).
//                  Inside a piece, row r at (r % 16) * 64 has 4 chunks of 16
//                  bytes; logical chunk c (K bytes [16c, 16c+16) of the step)
//                  sits at chunk position c ^ swz(r), swz(r) = q ^ 2 (q & 1) with
//                  q = (r >> 2) & 3 (bits 2-3 of the row only).  Measured on
//                  gfx950 with a 16-wave LDS probe over every swizzle of
//                  this form: a ds_read_b128 in which lane i + 16 g reads
//                  row R0 + i, chunk g (16x16x128 operand) or lane i + 32 g
//                  reads row R0 + i, chunk g (32x32x64 operand) takes 2.1
//                  cycles with this swizzle for both; the plain (r >> 2) & 3
//                  is conflict-free only for the second (3.5 cycles for the
//                  first), no swizzle for neither;
//   scale[g][ks] = 256 B: 128 rows x 2 UE8M0 bytes (MX blocks 2ks, 2ks+1),
//                  lane-major: the byte of row r, block b sits at
//                  (r % 32) * 8 + b * 4 + r / 32, so one 4-byte read gives a
//                  32x32 MFMA lane (row r % 32, block b) the scales of its
//                  rows r % 32 + 32 i, i = 0..3 (the MFMA picks byte i with
//                  the scale operand's op_sel).
//
// A GEMM stage (128 rows x one step) is eight 1 KiB pieces; a workgroup
// copies each to LDS unchanged with one direct global->LDS load per wave, so
// in LDS the stage is the 8 KiB tile of rows 0..127 at r * 64 (tile_off).
// ---------------------------------------------------------------------------
constexpr int kGroupRows = 128;
constexpr int kStepK = 64;
constexpr int kXCD = 8;                          // accelerator dies; workgroup b runs on die b % 8

// Bijection from dispatch order to a work order in which XCD x (which gets
// workgroups x, x+8, x+16, ...) owns one contiguous range of work items, so
// the items that share operands in one die's L2 run there together.
__device__ inline int xcd_remap(int bid, int total) {
  const int xcd = bid % kXCD, k = bid / kXCD;
  const int per = total / kXCD, rem = total % kXCD;
  return (xcd < rem) ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}
// Raw buffer resource over [base, base + bytes) for compiler-tracked buffer
// loads (__builtin_amdgcn_raw_buffer_load_*): a load at or past `bytes`
// returns zero without touching memory, so a null base with bytes = 0 reads
// zeros.  Word 3 selects the 32-bit data format, no swizzle.
__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr int kTileBytes = kGroupRows * kStepK;   // 8192
constexpr int kTileScaleBytes = kGroupRows * 2;   // 256

__host__ __device__ inline int swz(int r) {
  const int q = (r >> 2) & 3;
  return q ^ ((q & 1) << 1);
}
// Byte offset of logical chunk c of row r inside a tile (128 rows x 64 bytes,
// rows consecutive: one stage in LDS).
__host__ __device__ inline int tile_off(int r, int c) { return r * kStepK + ((c ^ swz(r)) << 4); }
constexpr int kPieceBytes = 16 * kStepK;         // 1024: one 16-row band x one step
// Byte offset, inside the data of a 128-row group with KS steps, of logical
// chunk c of row r (0..127) in step ks.
__host__ __device__ inline int64_t packed_off(int r, int64_t ks, int c, int64_t KS) {
  return ((int64_t)(r >> 4) * KS + ks) * kPieceBytes + (r & 15) * kStepK + ((c ^ swz(r)) << 4);
}
// Byte offset of the scale of row r (0..127), block b (0..1) inside a scale tile.
__host__ __device__ inline int scale_off(int r, int b) { return (r & 31) * 8 + b * 4 + (r >> 5); }

// ---------------------------------------------------------------------------
// Scaled MFMA operand conventions on gfx950 (pinned by probes on the device):
//
// v_mfma_scale_f32_16x16x128_f8f6f4: lane l = i + 16 g (i = row/col index,
//   g = 0..3).  Its 32 operand bytes are K [16g, 16g+16) followed by
//   K [64+16g, 64+16g+16).  The UE8M0 scale of MX block b (K [32b, 32b+32))
//   is taken from the scale register of lane i + 16 b (byte chosen by
//   op_sel).  Result: lane l holds D[4g + j][i], j = 0..3.
//
// v_mfma_scale_f32_32x32x64_f8f6f4: lane l = i + 32 g (g = 0..1).  Operand
//   bytes K [16g, 16g+16) then K [32+16g, 32+16g+16); the scale of block b
//   comes from lane i + 32 b.  Result: lane l holds
//   D[8 (r/4) + 4 g + (r%4)][i], r = 0..15.
//
// Format code 0 selects E4M3 for both operands.
// ---------------------------------------------------------------------------

// bf16 helpers (raw 16-bit words).
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two bf16 (round to nearest even) packed in one word, low
// half = a: one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Magnitude bits (fp32 layout) of the two bf16 elements of a word.  Integer
// order of these bit patterns equals the order of the magnitudes for every
// finite value, so the block maximum can be taken on integers.
__device__ inline uint32_t absmax_bits(uint32_t acc, uint32_t w) {
  uint32_t lo = (w << 16) & 0x7FFF0000u;
  uint32_t hi = w & 0x7FFF0000u;
  return max(acc, max(lo, hi));
}

// UE8M0 scale byte of a block from the fp32 bits of its largest magnitude:
// shared exponent floor(log2 amax) - 8, clamped at -127 (byte 0).  For a
// normal fp32 amax the exponent field F gives floor(log2 amax) = F - 127, so
// the byte is F - 127 - 8 + 127 = F - 8.  A zero or subnormal amax (F = 0)
// lands on byte 0.  bf16 magnitudes have F <= 254, so the byte is <= 246.
__device__ inline uint32_t mx_scale_byte(uint32_t amax_bits) {
  int f = (int)(amax_bits >> 23);
  return (uint32_t)max(f - 8, 0);
}

// 2^(-e_s) as fp32 for a scale byte s (e_s = s - 127): exponent field 254 - s,
// always a normal number for s in [0, 246].
__device__ inline float mx_inv_scale(uint32_t sbyte) { return __uint_as_float((254u - sbyte) << 23); }

// Two bf16 elements (one word) -> two E4M3 bytes, scaled by 2^(-e_s) and
// saturated to +-448; the hardware convert rounds to nearest even.  The
// product is exact (power-of-two scaling; f32 denormals are kept).
template <bool kHiWord>
__device__ inline uint32_t cvt2(uint32_t w, float inv, uint32_t old) {
  float a = __builtin_amdgcn_fmed3f(bf16_lo(w) * inv, -448.0f, 448.0f);
  float b = __builtin_amdgcn_fmed3f(bf16_hi(w) * inv, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHiWord);
}

// Four bf16 words (8 elements) -> two dwords of E4M3 bytes, in element order.
__device__ inline void cvt8(const uint32_t* w, float inv, uint32_t* q) {
  uint32_t d0 = cvt2<false>(w[0], inv, 0u);
  d0 = cvt2<true>(w[1], inv, d0);
  uint32_t d1 = cvt2<false>(w[2], inv, 0u);
  d1 = cvt2<true>(w[3], inv, d1);
  q[0] = d0;
  q[1] = d1;
}

// ---------------------------------------------------------------------------
// The same element conversion with gfx950's scaled converter
// v_cvt_scalef32_pk_fp8_bf16: two bf16 -> two E4M3 bytes of RNE(x / scale),
// one instruction per pair, bf16 subnormals and signed zero handled (probed
// on the device against the rule for every bf16 value under scales 2^-127,
// 2^-20..2^20, 2^119, 2^127: identical wherever |x / scale| < 512).  It does
// not saturate: a value that rounds past 448 becomes the NaN code 0x7F/0xFF,
// which fix_sat turns into 0x7E/0xFE, i.e. the saturation to +-448.
// ---------------------------------------------------------------------------
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// 2^(s - 127) as fp32 for a scale byte s in [0, 246] (s = 0 is the fp32
// subnormal 2^-127).
__device__ inline float mx_scale_value(uint32_t sbyte) {
  return __uint_as_float(sbyte ? (sbyte << 23) : 0x00400000u);
}

template <bool kHiWord>
__device__ inline uint32_t cvt2s(uint32_t w, float scale, uint32_t old) {
  const s16x2 o = __builtin_bit_cast(s16x2, old);
  const bf16x2 v = __builtin_bit_cast(bf16x2, w);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, v, scale, kHiWord));
}

// Bytes whose low 7 bits are all ones (E4M3 NaN) step down to 0x7E / 0xFE.
__device__ inline uint32_t fix_sat(uint32_t q) {
  const uint32_t m = ((q & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
  return q - (m >> 7);
}

// Four bf16 words (8 elements) -> two dwords of E4M3 bytes with the scale
// 2^(e_s) passed as a value.
__device__ inline void cvt8s(const uint32_t* w, float scale, uint32_t* q) {
  uint32_t d0 = cvt2s<false>(w[0], scale, 0u);
  d0 = cvt2s<true>(w[1], scale, d0);
  uint32_t d1 = cvt2s<false>(w[2], scale, 0u);
  d1 = cvt2s<true>(w[3], scale, d1);
  q[0] = fix_sat(d0);
  q[1] = fix_sat(d1);
}

// Running maximum of bf16 magnitudes, two lanes of 16 bits (v_pk_max_u16 on
// the sign-cleared words; integer order = magnitude order for finite bf16).
// Maximum of m over the four lanes of a quad (lanes 4q .. 4q + 3): two DPP
// quad_perm exchanges ([1, 0, 3, 2], then [2, 3, 0, 1]), VALU only.
__device__ inline uint32_t quad_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, true));
  return max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, true));
}

__device__ inline u16x2 absmax_pk(u16x2 acc, uint32_t w) {
  return __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
}
// Scale byte from a packed maximum: bf16 exponent field F = bits >> 7 equals
// the fp32 one, so the byte is max(F - 8, 0) as in mx_scale_byte.
__device__ inline uint32_t mx_scale_byte_bf16(u16x2 m) {
  const uint32_t b = max((uint32_t)m[0], (uint32_t)m[1]);
  return (uint32_t)max((int)(b >> 7) - 8, 0);
}

}  // namespace mxfp8
