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
