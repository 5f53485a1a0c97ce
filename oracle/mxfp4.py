"""MXFP4 weights x MXFP8 activations (W4A8) linear layer, in plain numpy float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Nothing here is shared
with the HIP path.

What is computed, and where it is defined
-----------------------------------------
* The weight format "MxE2m1" with 32-element UE8M0 scales, against "MxE4m3"
  activations (the W4A8 mode exposed through the unified MoE API of
  flashinfer, "Expose TRTLLM-gen MxFP4xMxFP8 (W4A8)...", its "Changes"
  list: MXFP4 weights with 32-element UE8M0 scales, MXFP8 activation
  preparation).
* E2M1 as defined by the OCP Microscaling v1.0 element formats: 1 sign bit,
  2 exponent bits with bias 1, 1 mantissa bit, no infinities or NaN;
  magnitudes 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6.
* The conversion rule, by the same OCP MX scalar-to-MX procedure as the
  MXFP8 oracle with the E2M1 element type:
      shared exponent  e_s = floor(log2(max_i |v_i|)) - 2      (2 = E2M1 emax)
      element          P_i = E2M1_RNE(clamp(v_i / 2^e_s, -6, 6)).
  The same readings as for E4M3 (each listed in the design doc): an all-zero block
  gets e_s = -127, e_s is clamped to [-127, 127], ties go to the even code
  (mantissa bit 0), out-of-range values saturate, and a value that rounds to
  zero keeps its sign.
* Byte packing of the weight at the boundary (a reading: the pages do not
  print it): two elements per byte along K, element 2j in the low nibble and
  element 2j + 1 in the high nibble.
* The layer: ``y[m, n] = sum_k deq8(A)[m, k] * deq4(W)[n, k] + bias[n]``, with
  A the activations MX-quantized to E4M3 exactly as in the MXFP8 layer.
"""

import numpy as np

from .mx import E8M0_BIAS, MX_BLOCK, _ldexp, dequantize_mx, e8m0_decode, floor_log2, quantize_mx

E2M1_EXP_BIAS = 1
E2M1_MANT_BITS = 1
E2M1_EMAX = 2          # exponent of the top binade: 6 = 1.5 * 2^2
E2M1_EMIN = 0          # smallest normal exponent: 2^0
E2M1_MAX = 6.0
SCALE_EXP_MIN = -127
SCALE_EXP_MAX = 127


def e2m1_decode(c):
    """E2M1 code(s) (0..15, one per element) -> float64 value, from the bit
    layout: sign bit 3, exponent field bits 2..1, mantissa bit 0."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x8) != 0, -1.0, 1.0)
    efield = (c >> E2M1_MANT_BITS) & 0x3
    mant = c & 0x1
    sub = mant * 2.0 ** (1 - E2M1_EXP_BIAS - E2M1_MANT_BITS)            # m * 2^-1
    nrm = (1.0 + mant / 2.0) * _ldexp(1.0, efield - E2M1_EXP_BIAS)      # 1.m * 2^(E-1)
    return sign * np.where(efield == 0, sub, nrm)


def e2m1_encode(t):
    """Real value(s) t -> E2M1 code(s): saturate to +-6, then round to nearest
    even on E2M1's grid.  The grid spacing for |t| in binade [2^k, 2^(k+1)) is
    2^(k-1) for k >= 0; magnitudes below 1 (the subnormal range) use the
    spacing of the lowest binade, 2^-1."""
    t = np.asarray(t, dtype=np.float64)
    neg = np.signbit(t)
    a = np.minimum(np.abs(t), E2M1_MAX)
    k = np.where(a > 0, floor_log2(a), E2M1_EMIN)
    k = np.maximum(k, E2M1_EMIN)
    qexp = k - E2M1_MANT_BITS
    r = _ldexp(np.rint(_ldexp(a, -qexp)), qexp)         # ties to even
    kr = floor_log2(r)
    normal = (r > 0) & (kr >= E2M1_EMIN)
    efield = np.where(normal, kr + E2M1_EXP_BIAS, 0)
    mant = np.where(normal, _ldexp(r, -kr) * 2.0 - 2.0, r * 2.0).astype(np.int64)
    code = (efield.astype(np.int64) << E2M1_MANT_BITS) | mant
    return np.where(neg, code | 0x8, code).astype(np.uint8)


def scale_exponent_fp4(block_amax):
    """floor(log2(amax)) - 2, clamped to [-127, 127]; an all-zero block gives
    -127."""
    amax = np.asarray(block_amax, dtype=np.float64)
    e = np.where(amax > 0, floor_log2(amax) - E2M1_EMAX, SCALE_EXP_MIN)
    return np.clip(e, SCALE_EXP_MIN, SCALE_EXP_MAX).astype(np.int64)


def quantize_mxfp4(x):
    """MXFP4-quantize a real matrix ``x[R, C]`` (C % 32 == 0) along its rows.
    Returns ``(codes, s)``: ``codes`` uint8 E2M1 codes ``[R, C]`` (one element
    per entry, values 0..15) and ``s`` uint8 UE8M0 bytes ``[R, C // 32]``."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK != 0:
        raise ValueError(f"quantize_mxfp4 needs [R, C] with C % 32 == 0, got {x.shape}")
    R, C = x.shape
    xb = x.reshape(R, C // MX_BLOCK, MX_BLOCK)
    e_s = scale_exponent_fp4(np.max(np.abs(xb), axis=2))
    codes = e2m1_encode(_ldexp(xb, -e_s[:, :, None])).reshape(R, C)
    return codes, (e_s + E8M0_BIAS).astype(np.uint8)


def pack_fp4(codes):
    """E2M1 codes ``[R, C]`` (C even) -> bytes ``[R, C // 2]``: element 2j in
    the low nibble, element 2j + 1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed):
    """Inverse of ``pack_fp4``."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize_mxfp4(packed, s):
    """Packed E2M1 bytes ``[R, C // 2]`` and UE8M0 ``s[R, >= C // 32]`` ->
    float64 ``[R, C]``."""
    codes = unpack_fp4(packed)
    R, C = codes.shape
    scale = np.repeat(e8m0_decode(np.asarray(s, dtype=np.uint8)[:R, : C // MX_BLOCK]), MX_BLOCK, axis=1)
    return e2m1_decode(codes) * scale


def linear_w4a8_ref(x, w_packed, w_s, bias=None, N=None):
    """The W4A8 linear layer, unrounded (float64).

    ``x[M, K]`` real activations (bf16 values), MX-quantized to E4M3 here;
    ``w_packed[>= N, K // 2]`` packed E2M1 weight bytes and ``w_s[>= N,
    >= K // 32]`` their UE8M0 scales (only ``[:N]`` is read); ``bias[N]``
    optional.  Returns ``y[M, N]`` float64 before the final bf16 cast."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % 256 != 0:
        raise ValueError("the layer requires K % 256 == 0")
    if N is None:
        N = np.asarray(w_packed).shape[0]
    qa, sa = quantize_mx(x)
    A = dequantize_mx(qa, sa)
    W = dequantize_mxfp4(np.asarray(w_packed)[:N, : K // 2], np.asarray(w_s)[:N, : K // MX_BLOCK])
    y = A @ W.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :N]
    return y
