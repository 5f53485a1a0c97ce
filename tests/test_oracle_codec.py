"""Pins of the oracle's E4M3 / UE8M0 codec and MX quantizer (CPU only)."""

import os

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_amd import synth
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_examples.txt")


def load_worked_examples():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        el, other, sb, qb, note = [c.strip() for c in line.split("|")]
        vals = [float.fromhex(el), float.fromhex(other)] + [0.0] * 30
        rows.append((vals, 0, int(sb, 16), int(qb, 16), note))
    return rows


def test_decode_matches_torch_all_bytes():
    pins.check_decode(oracle.e4m3_decode)


def test_e8m0_decode():
    s = np.arange(256, dtype=np.uint8)
    v = oracle.e8m0_decode(s)
    assert np.isnan(v[255])
    assert np.array_equal(v[:255], np.array([2.0 ** (i - 127) for i in range(255)]))


def test_encode_exhaustive_vs_torch():
    """All finite bf16 values x every scale exponent in [-127, 119]."""
    pins.check_encode_exhaustive(oracle.e4m3_encode)


def test_encode_decode_roundtrip_all_codes():
    b = np.arange(256, dtype=np.uint8)
    finite = (b & 0x7F) != 0x7F
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(b[finite])), b[finite])


def test_worked_examples():
    rows = load_worked_examples()
    assert len(rows) >= 20
    pins.check_worked_examples(oracle.quantize_mx, rows)


@pytest.mark.parametrize("kind", ["normal", "outliers", "stress", "tiny", "huge", "zeros"])
def test_quantize_vs_library(kind):
    g = torch.Generator().manual_seed(11)
    if kind == "normal":
        x = synth.randn_bf16((64, 512), 1.0, g)
    elif kind == "outliers":
        x = synth.activations(64, 512, 1.0, g, 0.01, 50.0)
    elif kind == "stress":
        x = synth.scale_stress(synth.randn_bf16((64, 512), 1.0, g), seed=5)
    elif kind == "tiny":
        x = (torch.randn(64, 512, generator=g) * 2.0 ** -128).to(torch.bfloat16)
    elif kind == "huge":
        x = (torch.randn(64, 512, generator=g) * 2.0 ** 125).to(torch.bfloat16)
    else:
        x = synth.randn_bf16((64, 512), 1.0, g)
        x[:, 64:128] = 0
        x[1, 200:232] = -0.0
    pins.check_quantize_vs_library(oracle.quantize_mx, x)


def _blocks_data():
    g = torch.Generator().manual_seed(3)
    parts = [synth.randn_bf16((32, 1024), 1.0, g),
             synth.scale_stress(synth.randn_bf16((32, 1024), 1.0, g), seed=4),
             synth.activations(32, 1024, 1.0, g, 0.01, 50.0)]
    return torch.cat(parts).to(torch.float64).numpy()


def test_invariants():
    x = _blocks_data()
    q, s = oracle.quantize_mx(x)
    # (i) finite input never yields a NaN scale or a NaN element.
    assert not np.any(s == 0xFF)
    assert not np.any((q & 0x7F) == 0x7F)
    # (ii) the largest element of a block with an unclamped scale sits in the
    # top binade: field 1111, mantissa <= 110 (t_max in [256, 448]).
    mag = (q & 0x7F).reshape(q.shape[0], -1, 32).max(axis=2)
    sel = s > 0
    assert np.all((mag[sel] >= 0x78) & (mag[sel] <= 0x7E))
    # (iii) error bound: half an E4M3 ulp of t times the scale, or the clamp.
    e_s = s.astype(np.int64) - 127
    scale = np.repeat(2.0 ** e_s, 32, axis=1)
    t = x / scale
    deq = oracle.dequantize_mx(q, s)
    err = np.abs(deq - x)
    a = np.abs(t)
    k = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    half_ulp = 2.0 ** (k - 3) / 2 * scale
    clamped = a > 448
    assert np.all(err[~clamped] <= half_ulp[~clamped])
    assert np.all(err[clamped] == np.abs(x[clamped]) - 448 * scale[clamped])
    # (iv) idempotence.
    q2, s2 = oracle.quantize_mx(deq)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # (vi) sign symmetry: negation flips bit 7 only.
    q3, s3 = oracle.quantize_mx(-x)
    assert np.array_equal(q3, q ^ 0x80) and np.array_equal(s3, s)


@pytest.mark.parametrize("j", [-5, -1, 1, 3])
def test_scale_equivariance(j):
    x = _blocks_data()
    q, s = oracle.quantize_mx(x)
    q2, s2 = oracle.quantize_mx(x * 2.0 ** j)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2.astype(int), s.astype(int) + j)


def test_bf16_round_vs_torch():
    g = torch.Generator().manual_seed(2)
    f = torch.cat([torch.randn(100000, generator=g) * 10.0 ** torch.randint(-40, 38, (100000,), generator=g),
                   pins.all_finite_bf16(),
                   torch.tensor([3.4e38, -3.4e38, 1e-45, -1e-45, 0.0, -0.0])])
    ref = f.to(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.bf16_round(f.to(torch.float64).numpy())
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
