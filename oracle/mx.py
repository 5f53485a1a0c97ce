"""MXFP8 quantization and the dequantized linear layer, in plain numpy float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Nothing here is fast
and nothing here is shared with the HIP path.

What is computed, and where it is defined
-----------------------------------------
* Element format E4M3 ("float8_e4m3fn"): the activations and weights of the
  layer are ``torch.float8_e4m3fn`` (prhub digest of vLLM PR #52204, "key code
  excerpts": the fake quantize op returns an ``float8_e4m3fn`` tensor of the
  input's shape).  Bit layout per the OCP 8-bit floating point specification
  (OFP8): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, S.1111.111 is NaN, largest finite magnitude 1.75 * 2^8 = 448,
  smallest subnormal 2^-9.
* Scale format UE8M0: one unsigned power-of-two exponent byte per 32 elements
  along K ("mxfp4/mxfp8 use UE8M0 scale factors with sfVecSize 32" in the
  review of flashinfer PR #1214, fp4Quantize.cpp; the linear ``[N, K // 32]``
  scale view in the test helper ``_make_layer`` of the vLLM PR #52204 digest).
  Value 2^(byte - 127); byte 0xFF is NaN.
* The conversion rule (none of the pages print it): the OCP Microscaling (MX)
  v1.0 scalar-to-MX conversion for an E4M3 element type,
      shared exponent  e_s = floor(log2(max_i |v_i|)) - 8      (8 = E4M3 emax)
      element          P_i = E4M3_RNE(clamp(v_i / 2^e_s, -448, 448)).
  Readings taken where the rule leaves a step open (each listed in the design doc):
  an all-zero block gets e_s = -127 (scale byte 0x00); e_s is clamped to
  [-127, 127]; rounding is round-to-nearest, ties to even, also among
  subnormals; out-of-range values saturate to +-448 (never NaN); the sign of a
  value that rounds to zero is kept (-0 -> 0x80).
* The layer: ``y[m, n] = sum_k deq(A)[m, k] * deq(W)[n, k] + bias[n]`` for the
  logical ``n < N`` (vLLM PR #52204, §Purpose: quantize activations, run the
  MXFP8 GEMM, slice the padded output back to its logical width, add bias).
"""

import numpy as np

# Element format constants, straight from the OFP8 E4M3 definition.
E4M3_EXP_BIAS = 7
E4M3_MANT_BITS = 3
E4M3_EMAX = 8          # exponent of the top binade: 448 = 1.75 * 2^8
E4M3_EMIN = -6         # smallest normal exponent: 2^-6
E4M3_MAX = 448.0
MX_BLOCK = 32          # elements sharing one UE8M0 scale
E8M0_BIAS = 127
SCALE_EXP_MIN = -127   # smallest encodable scale exponent (byte 0x00)
SCALE_EXP_MAX = 127    # largest finite scale exponent (byte 0xFE)


def floor_log2(a):
    """floor(log2(a)) for float64 a > 0, exactly: the unbiased exponent field
    of a normal float64 (the rare subnormals go through np.frexp).  Entries
    with a <= 0 are returned as 0 (callers mask them)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    e = ((a.view(np.int64) >> 52) & 0x7FF) - 1023
    sub = (e == -1023) & (a > 0)
    if np.any(sub):
        _, p = np.frexp(a[sub])
        e[sub] = p - 1
    return np.where(a > 0, e, 0)


def _ldexp(x, e):
    """x * 2^e, exact (numpy's fast loop wants an int32 exponent)."""
    return np.ldexp(x, np.asarray(e).astype(np.int32))


def bf16_round(x):
    """Round real values to the nearest bfloat16 (ties to even), returned as
    float64.  bfloat16 keeps 8 significant bits, exponents down to -126 for
    normals and a fixed quantum of 2^-133 below that; magnitudes that round
    to 2^128 or beyond overflow to infinity."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    k = np.where(a > 0, floor_log2(a), -126)
    k = np.maximum(k, -126)
    qexp = k - 7
    r = _ldexp(np.rint(_ldexp(a, -qexp)), qexp)
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isnan(x), np.nan, r)
    return np.copysign(r, x)


def e4m3_decode(q):
    """E4M3 byte(s) -> float64 value, from the bit layout."""
    b = np.asarray(q, dtype=np.uint8).astype(np.int64)
    sign = np.where((b & 0x80) != 0, -1.0, 1.0)
    efield = (b >> E4M3_MANT_BITS) & 0xF
    mant = b & 0x7
    sub = mant * 2.0 ** (1 - E4M3_EXP_BIAS - E4M3_MANT_BITS)           # m * 2^-9
    nrm = (1.0 + mant / 8.0) * _ldexp(1.0, efield - E4M3_EXP_BIAS)    # 1.m * 2^(E-7)
    val = sign * np.where(efield == 0, sub, nrm)
    return np.where((b & 0x7F) == 0x7F, np.nan, val)


def e8m0_decode(s):
    """UE8M0 byte(s) -> float64 power of two 2^(s - 127); 0xFF is NaN."""
    s = np.asarray(s, dtype=np.uint8).astype(np.int64)
    return np.where(s == 0xFF, np.nan, _ldexp(1.0, s - E8M0_BIAS))


def e4m3_encode(t):
    """Real value(s) t -> E4M3 byte(s): saturate to +-448, then round to
    nearest even on E4M3's grid.

    The grid spacing (quantum) for |t| in binade [2^k, 2^(k+1)) is 2^(k-3) for
    k >= -6; every smaller magnitude (the subnormals) uses the spacing of the
    lowest binade, 2^-9.  Rounding to a multiple of the quantum may carry into
    the next binade, which simply yields the next representable number.
    """
    t = np.asarray(t, dtype=np.float64)
    neg = np.signbit(t)
    a = np.minimum(np.abs(t), E4M3_MAX)                  # saturate
    k = np.where(a > 0, floor_log2(a), E4M3_EMIN)        # floor(log2 a)
    k = np.maximum(k, E4M3_EMIN)
    qexp = k - E4M3_MANT_BITS
    n = np.rint(_ldexp(a, -qexp))                        # numpy rint: ties to even
    r = _ldexp(n, qexp)                                  # rounded magnitude, exact
    # Encode the (exactly representable) magnitude r.
    kr = floor_log2(r)
    normal = (r > 0) & (kr >= E4M3_EMIN)
    efield = np.where(normal, kr + E4M3_EXP_BIAS, 0)
    mant = np.where(normal,
                    _ldexp(r, -kr) * 8.0 - 8.0,          # (r / 2^k - 1) * 8
                    np.ldexp(r, 9))                      # r / 2^-9
    mant = mant.astype(np.int64)
    code = (efield.astype(np.int64) << E4M3_MANT_BITS) | mant
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def scale_exponent(block_amax):
    """Shared exponent of a block from its max magnitude:
    floor(log2(amax)) - 8, clamped to [-127, 127]; an all-zero block gives
    -127.  floor(log2) is taken exactly from the exponent bits, never from a
    floating log2."""
    amax = np.asarray(block_amax, dtype=np.float64)
    e = np.where(amax > 0, floor_log2(amax) - E4M3_EMAX, SCALE_EXP_MIN)
    return np.clip(e, SCALE_EXP_MIN, SCALE_EXP_MAX).astype(np.int64)


def quantize_mx(x):
    """MX-quantize a real matrix ``x[R, C]`` (C % 32 == 0) along its rows.

    Returns ``(q, s)``: ``q`` uint8 E4M3 bytes ``[R, C]`` and ``s`` uint8
    UE8M0 bytes ``[R, C // 32]`` (row-major, the "linear" scale layout).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK != 0:
        raise ValueError(f"quantize_mx needs [R, C] with C % 32 == 0, got {x.shape}")
    R, C = x.shape
    xb = x.reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    e_s = scale_exponent(amax)
    t = _ldexp(xb, -e_s[:, :, None])                     # exact power-of-two scaling
    q = e4m3_encode(t).reshape(R, C)
    s = (e_s + E8M0_BIAS).astype(np.uint8)
    return q, s


def dequantize_mx(q, s):
    """``q[R, C]`` E4M3 bytes and ``s[R, >= C // 32]`` UE8M0 bytes -> float64."""
    q = np.asarray(q, dtype=np.uint8)
    R, C = q.shape
    s = np.asarray(s, dtype=np.uint8)[:R, : C // MX_BLOCK]
    scale = np.repeat(e8m0_decode(s), MX_BLOCK, axis=1)
    return e4m3_decode(q) * scale


def gemm_dequant(qa, sa, qw, sw, N=None):
    """``acc[m, n] = sum_k deq(A)[m, k] * deq(W)[n, k]`` for ``n < N`` in
    float64.  Products of dequantized values are exact in float64; only the
    summation rounds (relative error below K * 2^-53)."""
    qw = np.asarray(qw, dtype=np.uint8)
    if N is None:
        N = qw.shape[0]
    A = dequantize_mx(qa, sa)
    W = dequantize_mx(qw[:N], np.asarray(sw)[:N])
    return A @ W.T


def linear_ref(x, w_q, w_s, bias=None, N=None):
    """The MXFP8 dense linear layer, unrounded (float64).

    ``x[M, K]`` real activations (bf16 values), quantized here by the MX rule;
    ``w_q[>= N, K]`` / ``w_s[>= N, >= K // 32]`` the MXFP8 weight (linear scale
    layout, only the logical ``[:N, :K // 32]`` region is read, as the prepare
    step of vLLM PR #52204 slices it); ``bias[N]`` optional.
    Returns ``y[M, N]`` float64 before the final bf16 cast.
    """
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % 256 != 0:
        raise ValueError("the layer requires K % 256 == 0")
    if N is None:
        N = np.asarray(w_q).shape[0]
    qa, sa = quantize_mx(x)
    y = gemm_dequant(qa, sa, np.asarray(w_q)[:N, :K], np.asarray(w_s)[:N, : K // MX_BLOCK], N)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :N]
    return y
