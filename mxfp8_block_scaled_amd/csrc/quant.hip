// Activation quantization: bf16 [M, K] -> E4M3 [M, K] + UE8M0 [M, K/32].
//
// The on-the-fly activation quantize of "[Kernel] Add FlashInfer TRTLLM MXFP8
// linear backend" (vLLM PR #52204, §Purpose), with the OCP MX conversion rule
// (shared exponent floor(log2 amax) - 8, RNE, saturate to +-448) and the
// linear row-major scale layout.
//
// HBM-bound: 2 bytes read + 1 + 1/32 bytes written per element.  Four
// consecutive lanes own one 32-element block, each loading 16 contiguous
// bytes (8 elements), so a wave's loads cover 1 KiB of one or more rows
// without gaps; the block maximum (packed 16-bit integer max of the
// magnitudes) is combined across the four lanes with two lane exchanges, the
// elements go through the hardware scaled converter (common.hpp), and each
// lane writes its 8 E4M3 bytes as one 8-byte store.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp8 {

// Each thread converts CPT chunks 256 apart (every pass of the workgroup
// covers 256 consecutive chunks, 4 KiB of bf16) and issues all their loads
// before converting any, so several loads per lane are in flight.  CPT = 4
// for large inputs (measured 3-5 % faster from 16384 x 2048 up); CPT = 1
// keeps enough workgroups for small ones.
template <typename Idx, int CPT>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                        Idx chunks_per_row, Idx total,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        uint8_t* __restrict__ s, int64_t lds) {
  const Idx t0 = (Idx)blockIdx.x * (256 * CPT) + threadIdx.x;
  uint4 v[CPT];
  Idx rows[CPT], c8s[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    Idx t = t0 + (Idx)k * 256;
    // Threads past the end come in whole groups of four (total and the
    // pass size are multiples of 4), so they only exchange among themselves.
    if (t >= total) t = total - 1;
    rows[k] = t / chunks_per_row;
    c8s[k] = t - rows[k] * chunks_per_row;
    v[k] = *reinterpret_cast<const uint4*>(x + (int64_t)rows[k] * ldx + (int64_t)c8s[k] * 8);
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const bool valid = t0 + (Idx)k * 256 < total;
    const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
    u16x2 mp = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) mp = absmax_pk(mp, w[i]);
    uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
    m = quad_max(m);
    const uint32_t sb = (uint32_t)max((int)(m >> 7) - 8, 0);
    uint32_t qd[2];
    cvt8s(w, mx_scale_value(sb), qd);
    if (valid) {
      const Idx row = rows[k], c8 = c8s[k];
      *reinterpret_cast<uint2*>(q + (int64_t)row * ldq + (int64_t)c8 * 8) = make_uint2(qd[0], qd[1]);
      if ((c8 & 3) == 0) s[(int64_t)row * lds + (int64_t)(c8 >> 2)] = (uint8_t)sb;
    }
  }
}

// Same quantization, written in the packed operand layout of common.hpp for
// the large-M GEMM (rows padded to a multiple of 128; pad rows are written as
// zero elements with scale byte 0, so every byte the GEMM reads is defined).
// A workgroup owns one 16-row band and SPW consecutive 64-K steps, i.e. SPW
// consecutive 1 KiB pieces, one contiguous run of the packed data.  Its
// waves read whole row segments (SPW * 128 contiguous bytes per row, four
// lanes per 32-block as in quant_act_kernel), write the E4M3 bytes into the
// pieces' layout in LDS, and the workgroup then copies the SPW KiB out with
// 16-byte stores; the scale bytes go straight to the scale tiles.
template <int SPW>
__global__ __launch_bounds__(256) void quant_act_packed_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                               int64_t KS, int64_t nsg, uint8_t* __restrict__ qp,
                                                               uint8_t* __restrict__ sp) {
  constexpr int kLanesPerRow = SPW * 8;            // 8 elements per lane
  constexpr int kRowsPerWave = 64 / kLanesPerRow;
  __shared__ __attribute__((aligned(16))) uint8_t buf[SPW * kPieceBytes];
  const int64_t band = (int64_t)blockIdx.x / nsg;  // global 16-row band
  const int64_t s0 = ((int64_t)blockIdx.x - band * nsg) * SPW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l = lane % kLanesPerRow;
  const int s = l >> 3, c16 = (l & 7) >> 1, half = l & 1;   // step, chunk, half of the lane's 8 bytes
  const int64_t g = band >> 3;
#pragma unroll
  for (int pass = 0; pass < 16 / (4 * kRowsPerWave); ++pass) {
    const int rb = (pass * 4 + wave) * kRowsPerWave + lane / kLanesPerRow;   // row in the band
    const int64_t row = band * 16 + rb;
    const int r = (int)(row & (kGroupRows - 1));                           // row in the group
    uint32_t v4[4] = {0u, 0u, 0u, 0u};
    if (row < M) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + row * ldx + s0 * kStepK + l * 8);
      v4[0] = v.x; v4[1] = v.y; v4[2] = v.z; v4[3] = v.w;
    }
    u16x2 mp = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) mp = absmax_pk(mp, v4[i]);
    uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
    m = quad_max(m);
    const uint32_t sb = (uint32_t)max((int)(m >> 7) - 8, 0);
    uint32_t qd[2];
    cvt8s(v4, mx_scale_value(sb), qd);
    *reinterpret_cast<uint2*>(buf + s * kPieceBytes + rb * kStepK + ((c16 ^ swz(r)) << 4) + half * 8) =
        make_uint2(qd[0], qd[1]);
    if ((l & 3) == 0) sp[(g * KS + s0 + s) * kTileScaleBytes + scale_off(r, (l >> 2) & 1)] = (uint8_t)sb;
  }
  __syncthreads();
  uint8_t* dst = qp + g * KS * kTileBytes + ((band & 7) * KS + s0) * kPieceBytes;
#pragma unroll
  for (int o = tid * 16; o < SPW * kPieceBytes; o += 256 * 16)
    *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(buf + o);
}

// MXFP4 quantization (bf16 [M, K] -> E2M1 [M, K/2] packed two per byte,
// element 2j in the low nibble, + UE8M0 [M, K/32]): the MX rule with the
// E2M1 element type (shared exponent floor(log2 amax) - 2, RNE, saturate to
// +-6), for preparing W4A8 weights.  Same thread layout as quant_act_kernel;
// gfx950's v_cvt_scalef32_pk_fp4_bf16 converts two bf16 into the two nibbles
// of one byte as RNE(x / scale), saturating (E2M1 has no NaN or infinity).
template <typename Idx>
__global__ __launch_bounds__(256) void quant_fp4_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                        Idx chunks_per_row, Idx total, uint8_t* __restrict__ q,
                                                        int64_t ldq, uint8_t* __restrict__ s, int64_t lds) {
  Idx t = (Idx)blockIdx.x * 256 + threadIdx.x;
  const bool valid = t < total;
  if (!valid) t = total - 1;
  const Idx row = t / chunks_per_row;
  const Idx c8 = t - row * chunks_per_row;
  const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)row * ldx + (int64_t)c8 * 8);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  u16x2 mp = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) mp = absmax_pk(mp, w[i]);
  uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
  m = quad_max(m);
  const uint32_t sb = (uint32_t)max((int)(m >> 7) - 2, 0);    // E2M1 emax = 2
  const float scale = mx_scale_value(sb);
  uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, w[0]), scale, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[1]), scale, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[2]), scale, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[3]), scale, 3);
  if (valid) {
    *reinterpret_cast<uint32_t*>(q + (int64_t)row * ldq + (int64_t)c8 * 4) = d;
    if ((c8 & 3) == 0) s[(int64_t)row * lds + (int64_t)(c8 >> 2)] = (uint8_t)sb;
  }
}

int launch_quantize_fp4(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq, void* s,
                        int64_t lds, hipStream_t stream) {
  const int64_t per_row = K / 8;
  const int64_t total = M * per_row;
  const int64_t blocks = (total + 255) / 256;
  if (total < ((int64_t)1 << 32)) {
    hipLaunchKernelGGL(quant_fp4_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (uint32_t)per_row, (uint32_t)total, (uint8_t*)q, ldq,
                       (uint8_t*)s, lds);
  } else {
    hipLaunchKernelGGL(quant_fp4_kernel<uint64_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (uint64_t)per_row, (uint64_t)total, (uint8_t*)q, ldq,
                       (uint8_t*)s, lds);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_quantize_act_packed(const void* x, int64_t M, int64_t K, int64_t ldx, void* qp, void* sp,
                               hipStream_t stream) {
  const int64_t m_pad = (M + kGroupRows - 1) / kGroupRows * kGroupRows;
  const int64_t KS = K / kStepK;            // a multiple of 4 (K % 256 == 0)
  const int64_t bands = m_pad / 16;
  // Eight steps per workgroup (one 8 KiB run) where that still gives the
  // chip over a thousand workgroups; fewer for small inputs (a 128-row group
  // at K = 4096 gets 256 workgroups of two steps instead of 64 of eight).
  if (KS % 8 == 0 && bands * (KS / 8) >= 1024) {
    hipLaunchKernelGGL(quant_act_packed_kernel<8>, dim3((unsigned)(bands * (KS / 8))), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (int)M, KS, KS / 8, (uint8_t*)qp, (uint8_t*)sp);
  } else if (bands * (KS / 4) >= 1024) {
    hipLaunchKernelGGL(quant_act_packed_kernel<4>, dim3((unsigned)(bands * (KS / 4))), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (int)M, KS, KS / 4, (uint8_t*)qp, (uint8_t*)sp);
  } else {
    hipLaunchKernelGGL(quant_act_packed_kernel<2>, dim3((unsigned)(bands * (KS / 2))), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (int)M, KS, KS / 2, (uint8_t*)qp, (uint8_t*)sp);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq, void* s,
                        int64_t lds, hipStream_t stream) {
  const int64_t per_row = K / 8;
  const int64_t total = M * per_row;
  const bool wide = total >= (int64_t)256 * 4 * 2048;       // still >= 2048 workgroups at 4 chunks
  const int cpt = wide ? 4 : 1;
  const int64_t blocks = (total + 256 * cpt - 1) / (256 * cpt);
  auto go = [&](auto kern, auto idx) {
    using Idx = decltype(idx);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)x, ldx, (Idx)per_row,
                       (Idx)total, (uint8_t*)q, ldq, (uint8_t*)s, lds);
  };
  if (total < ((int64_t)1 << 32)) {
    if (wide) go(quant_act_kernel<uint32_t, 4>, uint32_t{});
    else go(quant_act_kernel<uint32_t, 1>, uint32_t{});
  } else {
    go(quant_act_kernel<uint64_t, 4>, uint64_t{});
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
