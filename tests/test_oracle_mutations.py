"""Plant plausible mistakes in (copies of) the oracle and check that the pins
catch every one of them.  The mistakes live here, on the CPU, never in the
product path."""

import numpy as np
import pytest
import torch

import oracle
from oracle import mx
from mxfp8_block_scaled_amd import synth
from tests import pins
from tests.test_oracle_codec import load_worked_examples


def _encode_variant(round_fn=np.rint, sat=448.0, sub_exp=-6, keep_neg_zero=True):
    def enc(t):
        t = np.asarray(t, dtype=np.float64)
        neg = np.signbit(t) if keep_neg_zero else (t < 0)
        a = np.minimum(np.abs(t), sat)
        _, p = np.frexp(a)
        k = np.maximum(np.where(a > 0, p - 1, sub_exp), sub_exp)
        r = np.ldexp(round_fn(np.ldexp(a, -(k - 3))), k - 3)
        _, pr = np.frexp(r)
        kr = pr - 1
        normal = (r > 0) & (kr >= -6)
        ef = np.where(normal, kr + 7, 0)
        mant = np.where(normal, np.ldexp(r, -kr) * 8 - 8, np.ldexp(r, 9))
        mant = np.clip(mant, 0, 7).astype(np.int64)  # keep codes in range
        ef = np.clip(ef, 0, 15).astype(np.int64)
        code = (ef << 3) | mant
        return np.where(neg, code | 0x80, code).astype(np.uint8)
    return enc


def _quantize_with(encode=mx.e4m3_encode, emax=8, floor_fn=None):
    def q(x):
        x = np.asarray(x, dtype=np.float64)
        R, C = x.shape
        xb = x.reshape(R, C // 32, 32)
        amax = np.max(np.abs(xb), axis=2)
        if floor_fn is None:
            _, p = np.frexp(amax)
            e = p - 1
        else:
            e = floor_fn(amax)
        e_s = np.clip(np.where(amax > 0, e - emax, -127), -127, 127).astype(np.int64)
        t = np.ldexp(xb, -e_s[:, :, None])
        return encode(t).reshape(R, C), (e_s + 127).astype(np.uint8)
    return q


def _data():
    g = torch.Generator().manual_seed(21)
    return synth.scale_stress(synth.randn_bf16((16, 256), 1.0, g), seed=22)


def _caught(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


ENCODE_MUTANTS = {
    "round half away from zero": _encode_variant(round_fn=lambda v: np.floor(v + 0.5)),
    "truncate instead of round": _encode_variant(round_fn=np.floor),
    "no saturation (clamp at 480)": _encode_variant(sat=480.0),
    "subnormal quantum 2^-10": _encode_variant(sub_exp=-7),
    "negative zero loses its sign": _encode_variant(keep_neg_zero=False),
}


@pytest.mark.parametrize("name", list(ENCODE_MUTANTS))
def test_encode_mutants_caught(name):
    enc = ENCODE_MUTANTS[name]
    q = _quantize_with(encode=enc)
    checks = [
        lambda: pins.check_encode_exhaustive(enc, exps=range(-10, 3)),
        lambda: pins.check_worked_examples(q, load_worked_examples()),
        lambda: pins.check_quantize_vs_library(q, _data()),
    ]
    assert any(_caught(c) for c in checks)


QUANT_MUTANTS = {
    "scale exponent off by one (emax 7)": _quantize_with(emax=7),
    "scale from ceil(log2 amax)": _quantize_with(floor_fn=lambda a: np.ceil(np.log2(np.where(a > 0, a, 1)))),
    "scale from rounded log2": _quantize_with(floor_fn=lambda a: np.round(np.log2(np.where(a > 0, a, 1)))),
}


@pytest.mark.parametrize("name", list(QUANT_MUTANTS))
def test_quantize_mutants_caught(name):
    q = QUANT_MUTANTS[name]
    checks = [
        lambda: pins.check_quantize_vs_library(q, _data()),
        lambda: pins.check_worked_examples(q, load_worked_examples()),
    ]
    assert any(_caught(c) for c in checks)


def _linear_variant(kind):
    def lin(x, qw, sw, b):
        x = np.asarray(x, dtype=np.float64)
        qa, sa = oracle.quantize_mx(x)
        if kind == "scale of neighbouring block":
            sa = np.roll(sa, 1, axis=1)
        if kind == "weight scale row shifted":
            sw = np.roll(sw, 1, axis=0)
        A = oracle.dequantize_mx(qa, sa)
        W = oracle.dequantize_mx(qw, sw)
        if kind == "weight K reversed":
            W = W[:, ::-1]
        if kind == "last K block dropped":
            A = A.copy()
            A[:, -32:] = 0
        y = A @ W.T
        if b is not None and kind != "bias dropped":
            y = y + (b[None, :] if kind != "bias sign flipped" else -b[None, :])
        return y
    return lin


LINEAR_MUTANTS = ["scale of neighbouring block", "weight scale row shifted", "weight K reversed",
                  "last K block dropped", "bias dropped", "bias sign flipped"]


@pytest.mark.parametrize("kind", LINEAR_MUTANTS)
def test_linear_mutants_caught(kind):
    lin = _linear_variant(kind)
    g = torch.Generator().manual_seed(5)
    x = synth.scale_stress(synth.randn_bf16((2, 256), 1.0, g), seed=6)
    w = synth.scale_stress(synth.randn_bf16((3, 256), 0.02, g), seed=7)
    b = synth.randn_bf16((3,), 0.1, g)
    perm = torch.randperm(256, generator=g)[:4].numpy()
    checks = [
        lambda: pins.check_gemm_bruteforce(lin, oracle.quantize_mx, x, w, b),
        lambda: pins.check_one_hot_w(lin, oracle.quantize_mx, x, perm),
        lambda: pins.check_one_hot_a(lin, oracle.quantize_mx, w, perm, b),
    ]
    assert any(_caught(c) for c in checks)


def test_real_oracle_passes_the_same_checks():
    lin = _linear_variant("none")
    g = torch.Generator().manual_seed(5)
    x = synth.scale_stress(synth.randn_bf16((2, 256), 1.0, g), seed=6)
    w = synth.scale_stress(synth.randn_bf16((3, 256), 0.02, g), seed=7)
    b = synth.randn_bf16((3,), 0.1, g)
    pins.check_gemm_bruteforce(lin, oracle.quantize_mx, x, w, b)


SILU_MUTANTS = {
    "exponent sign flipped, z / (1 + e^z)": lambda z: z / (1.0 + np.exp(z)),
    "sigmoid without the factor z": lambda z: 1.0 / (1.0 + np.exp(-z)),
    "z * sigmoid(-z)": lambda z: z * np.exp(-z) / (1.0 + np.exp(-z)),
    "sigmoid of z/2": lambda z: z / (1.0 + np.exp(-z / 2)),
}


@pytest.mark.parametrize("name", list(SILU_MUTANTS))
def test_silu_mutants_caught(name):
    assert _caught(lambda: pins.check_silu(SILU_MUTANTS[name]))


def test_real_silu_passes():
    pins.check_silu(oracle.moe.silu)
