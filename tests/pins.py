"""Checks that pin the oracle to things other than itself.

Each ``check_*`` takes the oracle function under test as an argument and raises
AssertionError on a mismatch, so ``test_oracle_*.py`` run them against the real
oracle and ``test_oracle_mutations.py`` runs them against planted mistakes to
show that they would catch them.

Independent references used here (none re-types the oracle's formula):
* torch's CPU ``float32 -> float8_e4m3fn`` cast (round to nearest even, keeps
  -0, exact subnormals) and its ``float8_e4m3fn -> float32`` widening;
* the IEEE-754 exponent field of the fp32 block maximum, read from the bits,
  for floor(log2(amax));
* exact rational arithmetic (``fractions.Fraction``) for the GEMM;
* closed forms (constant and one-hot operands, power-of-two equivariance).
"""

from fractions import Fraction

import numpy as np
import torch

E4M3 = torch.float8_e4m3fn


def all_finite_bf16():
    """Every finite bf16 bit pattern, as float32 values (65280 of them)."""
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).to(torch.float32)
    return vals[torch.isfinite(vals)]


def torch_e4m3_bytes(t_f32):
    """E4M3 bytes of fp32 values already inside [-448, 448], via torch."""
    return t_f32.to(E4M3).view(torch.uint8).numpy()


def torch_e4m3_values(b):
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(E4M3).to(torch.float64).numpy()


def library_quantize(x_bf16):
    """MX quantization composed from library pieces only: the block maximum's
    fp32 exponent field gives floor(log2 amax) (subnormal / zero maxima have
    field 0 and land on the clamped exponent -127), torch's cast rounds."""
    xf = x_bf16.to(torch.float32)
    R, C = xf.shape
    xb = xf.reshape(R, C // 32, 32)
    amax = xb.abs().amax(dim=2)
    field = (amax.view(torch.int32) >> 23) & 0xFF
    e_s = torch.clamp(field.to(torch.int64) - 127 - 8, -127, 127)
    scale = torch.pow(2.0, (-e_s).to(torch.float64)).to(torch.float64)
    t = (xb.to(torch.float64) * scale[:, :, None]).clamp(-448.0, 448.0).to(torch.float32)
    q = torch_e4m3_bytes(t).reshape(R, C)
    s = (e_s + 127).to(torch.uint8).numpy()
    return q, s


def check_decode(decode):
    b = np.arange(256, dtype=np.uint8)
    ours = decode(b)
    ref = torch_e4m3_values(b)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def check_encode_exhaustive(encode, exps=range(-127, 120)):
    """Every finite bf16 value times every scale 2^-e, clamped to +-448, must
    encode like torch's cast."""
    v = all_finite_bf16().to(torch.float64)
    for e in exps:
        t = torch.clamp(v * (2.0 ** -e), -448.0, 448.0)
        ref = torch_e4m3_bytes(t.to(torch.float32))
        ours = encode(t.numpy())
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, (e, t[bad[:5]].tolist(), ours[bad[:5]], ref[bad[:5]])


def check_quantize_vs_library(quantize, x_bf16):
    q, s = quantize(x_bf16.to(torch.float64).numpy())
    q2, s2 = library_quantize(x_bf16)
    assert np.array_equal(s, s2), np.argwhere(s != s2)[:5]
    assert np.array_equal(q, q2), np.argwhere(q != q2)[:5]


def check_worked_examples(quantize, rows):
    """rows: (block values list of 32, index, scale byte, element byte)."""
    for vals, idx, sb, qb, note in rows:
        q, s = quantize(np.array([vals], dtype=np.float64))
        assert int(s[0, 0]) == sb, (note, int(s[0, 0]), sb)
        assert int(q[0, idx]) == qb, (note, hex(int(q[0, idx])), hex(qb))


def fraction_gemm(qa, sa, qw, sw, bias=None):
    """Exact rational sum_k deq(A)[m,k] deq(W)[n,k] (+ bias)."""
    va = torch_e4m3_values(qa)
    vw = torch_e4m3_values(qw)
    M, K = qa.shape
    N = qw.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for b in range(K // 32):
                part = Fraction(0)
                for i in range(32 * b, 32 * b + 32):
                    part += Fraction(float(va[m, i])) * Fraction(float(vw[n, i]))
                acc += part * Fraction(2) ** (int(sa[m, b]) - 127) * Fraction(2) ** (int(sw[n, b]) - 127)
            if bias is not None:
                acc += Fraction(float(bias[n]))
            out[m][n] = acc
    return out


def check_gemm_bruteforce(linear, quantize, x_bf16, w_bf16, bias_bf16=None):
    qw, sw = quantize(w_bf16.to(torch.float64).numpy())
    qa, sa = library_quantize(x_bf16)
    b = None if bias_bf16 is None else bias_bf16.to(torch.float64).numpy()
    exact = fraction_gemm(qa, sa, qw, sw, b)
    y = linear(x_bf16.to(torch.float64).numpy(), qw, sw, b)
    va = np.abs(torch_e4m3_values(qa)) * np.repeat(2.0 ** (sa.astype(np.int64) - 127), 32, 1)
    vw = np.abs(torch_e4m3_values(qw)) * np.repeat(2.0 ** (sw.astype(np.int64) - 127), 32, 1)
    mag = va @ vw.T + (0 if b is None else np.abs(b)[None, :])
    K = x_bf16.shape[1]
    for m in range(y.shape[0]):
        for n in range(y.shape[1]):
            err = abs(Fraction(float(y[m, n])) - exact[m][n])
            assert err <= Fraction(K + 2) * Fraction(2) ** -53 * Fraction(float(mag[m, n])), (m, n)


def check_one_hot_w(linear, quantize, x_bf16, perm):
    """W[n, perm[n]] = 1 -> y[m, n] = deq(A)[m, perm[n]] exactly."""
    N, K = len(perm), x_bf16.shape[1]
    w = np.zeros((N, K))
    w[np.arange(N), perm] = 1.0
    qw, sw = quantize(w)
    y = linear(x_bf16.to(torch.float64).numpy(), qw, sw, None)
    qa, sa = library_quantize(x_bf16)
    deqa = torch_e4m3_values(qa) * np.repeat(2.0 ** (sa.astype(np.int64) - 127), 32, 1)
    assert np.array_equal(y, deqa[:, perm])


def check_one_hot_a(linear, quantize, w_bf16, perm, bias_bf16=None):
    """x[m, perm[m]] = 1 -> y[m, n] = deq(W)[n, perm[m]] (+ bias[n]) exactly."""
    M, K = len(perm), w_bf16.shape[1]
    x = np.zeros((M, K))
    x[np.arange(M), perm] = 1.0
    qw, sw = library_quantize(w_bf16)
    b = None if bias_bf16 is None else bias_bf16.to(torch.float64).numpy()
    y = linear(x, qw, sw, b)
    deqw = torch_e4m3_values(qw) * np.repeat(2.0 ** (sw.astype(np.int64) - 127), 32, 1)
    exp = deqw[:, perm].T + (0 if b is None else b[None, :])
    assert np.array_equal(y, exp)


def check_constant(linear, quantize, M, N, K, c, bias=None):
    """x = 1, W = c (a power of two): y = K * c (+ bias) exactly."""
    qw, sw = quantize(np.full((N, K), c))
    y = linear(np.ones((M, K)), qw, sw, bias)
    exp = np.full((M, N), K * c) + (0 if bias is None else np.asarray(bias)[None, :])
    assert np.array_equal(y, exp)


def check_equivariance(linear, quantize, x_bf16, w_bf16, j):
    qw, sw = quantize(w_bf16.to(torch.float64).numpy())
    x = x_bf16.to(torch.float64).numpy()
    assert np.array_equal(linear(x * 2.0 ** j, qw, sw, None), 2.0 ** j * linear(x, qw, sw, None))


# ---------------------------------------------------------------------------
# MXFP4 (E2M1) pins.  References independent of the oracle's formulas: the
# format's value table (tests/golden/e2m1_format.txt), a brute-force
# nearest-value search over that table with ties to the even code, and the
# MXFP8 oracle (pinned above) for the layer: every E2M1 value is an E4M3
# value, so the W4A8 layer equals the MXFP8 layer on the widened weight.
# ---------------------------------------------------------------------------

def e2m1_table(path):
    codes, vals = [], []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v, _ = [f.strip() for f in line.split("|")]
        codes.append(int(c))
        vals.append(float(v))
    return np.array(codes), np.array(vals)


def check_e2m1_decode(decode, table_path):
    codes, vals = e2m1_table(table_path)
    assert np.array_equal(decode(codes.astype(np.uint8)), vals)
    neg = decode((codes | 8).astype(np.uint8))
    assert np.array_equal(neg, -vals) and np.all(np.signbit(neg))


def bruteforce_e2m1(t, table_path):
    """Nearest E2M1 magnitude by exhaustive search over the format's table,
    after saturation to the largest value; exact ties go to the code whose
    mantissa bit is 0; the sign is kept (also for zero)."""
    codes, vals = e2m1_table(table_path)
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(t), vals.max())
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer an even code (mantissa bit 0)
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    out = codes[pick].astype(np.int64)
    return np.where(np.signbit(t), out | 8, out).astype(np.uint8)


def check_e2m1_encode(encode, table_path):
    """Every finite bf16 value times 2^j for j in [-12, 12], against the
    brute-force search (about 1.6 M cases)."""
    base = all_finite_bf16().numpy().astype(np.float64)
    for j in range(-12, 13):
        t = np.ldexp(base, j)
        t = t[np.isfinite(t)]
        assert np.array_equal(encode(t), bruteforce_e2m1(t, table_path)), j


def check_fp4_worked_examples(quantize, rows):
    for vals, idx, sb, qc, note in rows:
        q, s = quantize(np.array([vals], dtype=np.float64))
        assert int(s[0, 0]) == sb, (note, int(s[0, 0]), sb)
        assert int(q[0, idx]) == qc, (note, int(q[0, idx]), qc)


def check_w4a8_vs_mxfp8(linear_w4a8, pack, x_bf16, codes, w_s, decode4, bias=None):
    """The W4A8 layer on (codes, w_s) equals the pinned MXFP8 layer on the
    same weight written as E4M3 bytes (torch's cast of the decoded values,
    exact because every E2M1 value is an E4M3 value), with the same scales."""
    import oracle
    vals = decode4(codes)
    w8 = torch_e4m3_bytes(torch.from_numpy(vals.astype(np.float32)))
    assert np.array_equal(torch_e4m3_values(w8), vals)
    x = x_bf16.to(torch.float64).numpy()
    b = None if bias is None else bias.to(torch.float64).numpy()
    y4 = linear_w4a8(x, pack(codes), w_s, b)
    y8 = oracle.linear_ref(x, w8, w_s, b)
    assert np.array_equal(y4, y8)


def check_silu(silu):
    """SiLU, z * sigmoid(z) (the gate activation of the routed MoE layer),
    against three things that do not share its formula:
      * torch.nn.functional.silu in float64 over z in [-100, 100] and at
        magnitudes where exp overflows (|z| up to 1e4);
      * the identity silu(z) - silu(-z) = z (z sigmoid(z) + z sigmoid(-z) = z),
        which fixes the sign convention of the exponent;
      * the closed form silu(ln 3) = (3/4) ln 3 and silu(0) = 0."""
    z = np.concatenate([np.linspace(-100.0, 100.0, 20001), [-1e4, -745.0, -700.0, 700.0, 745.0, 1e4]])
    with np.errstate(over="ignore"):
        got = np.asarray(silu(z), dtype=np.float64)
        mirror = np.asarray(silu(-z), dtype=np.float64)
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.all(np.isfinite(got)), "silu must stay finite where exp overflows"
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-300), float(np.max(np.abs(got - ref)))
    core = np.abs(z) <= 100
    assert np.allclose((got - mirror)[core], z[core], rtol=1e-13, atol=1e-13)
    ln3 = np.log(3.0)
    assert abs(float(silu(np.array([ln3]))[0]) - 0.75 * ln3) <= 1e-15
    assert float(silu(np.array([0.0]))[0]) == 0.0
