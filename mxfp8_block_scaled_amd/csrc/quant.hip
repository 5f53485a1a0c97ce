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

template <typename Idx>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                        Idx chunks_per_row, Idx total,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        uint8_t* __restrict__ s, int64_t lds) {
  Idx t = (Idx)blockIdx.x * 256 + threadIdx.x;
  const bool valid = t < total;
  // Threads past the end come in whole groups of four (total and the block
  // size are multiples of 4), so they only exchange among themselves.
  if (!valid) t = total - 1;
  const Idx row = t / chunks_per_row;
  const Idx c8 = t - row * chunks_per_row;
  const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)row * ldx + (int64_t)c8 * 8);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  u16x2 mp = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) mp = absmax_pk(mp, w[i]);
  uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  const uint32_t sb = (uint32_t)max((int)(m >> 7) - 8, 0);
  uint32_t qd[2];
  cvt8s(w, mx_scale_value(sb), qd);
  if (valid) {
    *reinterpret_cast<uint2*>(q + (int64_t)row * ldq + (int64_t)c8 * 8) = make_uint2(qd[0], qd[1]);
    if ((c8 & 3) == 0) s[(int64_t)row * lds + (int64_t)(c8 >> 2)] = (uint8_t)sb;
  }
}

// Same quantization, written in the packed operand layout of common.hpp for
// the large-M GEMM (rows padded to a multiple of 128; pad rows are written as
// zero elements with scale byte 0, so every byte the GEMM reads is defined).
// A wave owns two adjacent rows of a 128-row group and four consecutive
// 64-K steps: it reads 512 contiguous bytes of each row (consecutive waves
// continue along the same rows) and writes, in each of its four 1 KiB pieces
// (the rows' band, consecutive steps), the two rows' 128 contiguous bytes
// (one whole cache line).
template <typename Idx>
__global__ __launch_bounds__(256) void quant_act_packed_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                               Idx total, int64_t KS,
                                                               uint8_t* __restrict__ qp, uint8_t* __restrict__ sp) {
  const Idx t = (Idx)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;  // total is a multiple of 64: whole waves leave
  const Idx w = t >> 6;                     // wave: (g * 64 + row pair) * (KS / 4) + step quad
  const int lane = (int)(t & 63);
  const Idx nq = (Idx)(KS >> 2);
  const Idx gp = w / nq;
  const int64_t quad = (int64_t)(w - gp * nq);
  const int64_t g = (int64_t)(gp >> 6);
  const int r = (int)((gp & 63) * 2) + (lane >> 5);   // row inside the 128-row group
  const int c = lane & 31;                            // 8-element chunk inside the 4 steps
  const int64_t ks = quad * 4 + (c >> 3);
  const int c8 = c & 7;                               // chunk inside the 64-K step
  const int64_t row = g * kGroupRows + r;
  uint32_t v4[4] = {0u, 0u, 0u, 0u};
  if (row < M) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + row * ldx + ks * kStepK + c8 * 8);
    v4[0] = v.x; v4[1] = v.y; v4[2] = v.z; v4[3] = v.w;
  }
  u16x2 mp = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) mp = absmax_pk(mp, v4[i]);
  uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  const uint32_t sb = (uint32_t)max((int)(m >> 7) - 8, 0);
  uint32_t qd[2];
  cvt8s(v4, mx_scale_value(sb), qd);
  const int64_t tile = g * KS + ks;
  uint8_t* dst = qp + g * KS * kTileBytes + packed_off(r, ks, c8 >> 1, KS) + (c8 & 1) * 8;
  *reinterpret_cast<uint2*>(dst) = make_uint2(qd[0], qd[1]);
  if ((c8 & 3) == 0) sp[tile * kTileScaleBytes + scale_off(r, c8 >> 2)] = (uint8_t)sb;
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
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
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
  const int64_t KS = K / kStepK;
  const int64_t total = m_pad * (K / 8);    // (m_pad / 2) row pairs x (KS / 4) step quads x 64 lanes
  const int64_t blocks = total / 256;
  if (total < ((int64_t)1 << 32)) {
    hipLaunchKernelGGL(quant_act_packed_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (int)M, (uint32_t)total, KS, (uint8_t*)qp, (uint8_t*)sp);
  } else {
    hipLaunchKernelGGL(quant_act_packed_kernel<uint64_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (int)M, (uint64_t)total, KS, (uint8_t*)qp, (uint8_t*)sp);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq, void* s,
                        int64_t lds, hipStream_t stream) {
  const int64_t per_row = K / 8;
  const int64_t total = M * per_row;
  const int64_t blocks = (total + 255) / 256;
  if (total < ((int64_t)1 << 32)) {
    hipLaunchKernelGGL(quant_act_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (uint32_t)per_row, (uint32_t)total, (uint8_t*)q, ldq,
                       (uint8_t*)s, lds);
  } else {
    hipLaunchKernelGGL(quant_act_kernel<uint64_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, ldx, (uint64_t)per_row, (uint64_t)total, (uint8_t*)q, ldq,
                       (uint8_t*)s, lds);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace mxfp8
