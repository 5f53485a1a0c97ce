"""Pins of the oracle's MXFP4 (E2M1) codec, quantizer and W4A8 layer (CPU
only), and planted mistakes that the pins must catch."""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mxfp4
from mxfp8_block_scaled_amd import synth
from tests import pins

GOLD = os.path.join(os.path.dirname(__file__), "golden")
TABLE = os.path.join(GOLD, "e2m1_format.txt")
EXAMPLES = os.path.join(GOLD, "mxfp4_worked_examples.txt")


def load_fp4_examples():
    rows = []
    for line in open(EXAMPLES):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        el, other, sb, qc, note = [c.strip() for c in line.split("|")]
        rows.append(([float.fromhex(el), float.fromhex(other)] + [0.0] * 30, 0, int(sb, 16), int(qc, 16), note))
    return rows


def test_e2m1_decode_table():
    pins.check_e2m1_decode(oracle.e2m1_decode, TABLE)


def test_e2m1_encode_bruteforce():
    pins.check_e2m1_encode(oracle.e2m1_encode, TABLE)


def test_e2m1_roundtrip_all_codes():
    c = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.e2m1_encode(oracle.e2m1_decode(c)), c)


def test_fp4_worked_examples():
    rows = load_fp4_examples()
    assert len(rows) >= 15
    pins.check_fp4_worked_examples(oracle.quantize_mxfp4, rows)


def test_pack_nibble_order():
    # element 2j in the low nibble, element 2j + 1 in the high nibble
    codes = np.array([[0x1, 0x2, 0xF, 0x8]], dtype=np.uint8)
    assert oracle.pack_fp4(codes).tolist() == [[0x21, 0x8F]]
    assert np.array_equal(oracle.unpack_fp4(oracle.pack_fp4(codes)), codes)


@pytest.mark.parametrize("kind", ["normal", "stress", "tiny"])
def test_quantize_invariants(kind):
    g = torch.Generator().manual_seed(21)
    x = synth.randn_bf16((32, 512), 1.0, g).to(torch.float64).numpy()
    if kind == "stress":
        r = torch.randint(-16, 17, (32, 16), generator=g).numpy()
        x = x * np.repeat(np.ldexp(1.0, r), 32, axis=1)
    elif kind == "tiny":
        x = x * 2.0 ** -120
    q, s = oracle.quantize_mxfp4(x)
    qb = q.reshape(32, 16, 32)
    mags = oracle.e2m1_decode(qb & 7)
    live = s > 0
    # (i) the largest code of every block whose exponent was not clamped
    # lies in the top binade (4 or 6): amax / 2^e_s is in [4, 8)
    assert np.all(np.isin(mags.max(axis=2)[live], [4.0, 6.0]))
    # (ii) idempotence
    q2, s2 = oracle.quantize_mxfp4(oracle.dequantize_mxfp4(oracle.pack_fp4(q), s))
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    # (iii) sign symmetry: quantize(-x) flips bit 3 only
    qn, sn = oracle.quantize_mxfp4(-x)
    assert np.array_equal(qn, q ^ 8) and np.array_equal(sn, s)
    # (iv) power-of-two equivariance away from the clamps
    ok = (s > 8) & (s < 240)
    qe, se = oracle.quantize_mxfp4(x * 8.0)
    assert np.array_equal(se[ok], s[ok] + 3)
    assert np.array_equal(qe.reshape(32, 16, 32)[ok], qb[ok])


def _fp4_case(M, N, K, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    x = synth.randn_bf16((M, K), 1.0, g)
    w = synth.randn_bf16((N, K), 0.02, g).to(torch.float64).numpy()
    codes, ws = oracle.quantize_mxfp4(w)
    b = synth.randn_bf16((N,), 0.1, g) if bias else None
    return x, codes, ws, b


@pytest.mark.parametrize("M,N,K,seed", [(7, 130, 256, 1), (33, 96, 512, 2), (1, 256, 768, 3)])
def test_w4a8_equals_mxfp8_on_widened_weight(M, N, K, seed):
    x, codes, ws, b = _fp4_case(M, N, K, seed)
    pins.check_w4a8_vs_mxfp8(oracle.linear_w4a8_ref, oracle.pack_fp4, x, codes, ws, oracle.e2m1_decode, b)


def test_w4a8_logical_n_slice():
    x, codes, ws, b = _fp4_case(5, 64, 256, 4)
    y_full = oracle.linear_w4a8_ref(x.to(torch.float64).numpy(), oracle.pack_fp4(codes), ws,
                                    b.to(torch.float64).numpy())
    y_sl = oracle.linear_w4a8_ref(x.to(torch.float64).numpy(), oracle.pack_fp4(codes), ws,
                                  b.to(torch.float64).numpy(), N=40)
    assert np.array_equal(y_sl, y_full[:, :40])


# ---------------------------------------------------------------------------
# Planted mistakes (in copies of the oracle, on the CPU): each must be caught.
# ---------------------------------------------------------------------------

def _enc_variant(tie="even", sat=6.0, sub_q=0.5, keep_neg_zero=True):
    def enc(t):
        t = np.asarray(t, dtype=np.float64)
        neg = np.signbit(t) if keep_neg_zero else (t < 0)
        a = np.minimum(np.abs(t), sat)
        _, p = np.frexp(a)
        k = np.maximum(np.where(a > 0, p - 1, 0), 0)
        q = np.where(k == 0, sub_q, np.ldexp(1.0, k - 1))
        n = a / q
        r = (np.floor(n + 0.5) if tie == "away" else np.floor(n) if tie == "trunc" else np.rint(n)) * q
        r = np.minimum(r, 6.0)
        vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        code = np.abs(r[:, None] - vals[None, :]).argmin(axis=1)
        return np.where(neg, code | 8, code).astype(np.uint8)
    return enc


@pytest.mark.parametrize("mutant", [
    _enc_variant(tie="away"),
    _enc_variant(tie="trunc"),
    _enc_variant(sat=4.0),
    _enc_variant(sub_q=1.0),
    _enc_variant(keep_neg_zero=False),
])
def test_mutant_encoders_are_caught(mutant):
    with pytest.raises(AssertionError):
        pins.check_e2m1_encode(mutant, TABLE)


def _quantize_emax(emax):
    def q(x):
        x = np.asarray(x, dtype=np.float64)
        R, C = x.shape
        xb = x.reshape(R, C // 32, 32)
        amax = np.max(np.abs(xb), axis=2)
        _, p = np.frexp(amax)
        e_s = np.clip(np.where(amax > 0, p - 1 - emax, -127), -127, 127).astype(np.int64)
        return mxfp4.e2m1_encode(np.ldexp(xb, -e_s[:, :, None])).reshape(R, C), (e_s + 127).astype(np.uint8)
    return q


@pytest.mark.parametrize("emax", [1, 3])
def test_mutant_scale_rule_is_caught(emax):
    with pytest.raises(AssertionError):
        pins.check_fp4_worked_examples(_quantize_emax(emax), load_fp4_examples())


def test_mutant_nibble_order_is_caught():
    def swapped(codes):
        c = np.asarray(codes, dtype=np.uint8)
        return (c[:, 1::2] | (c[:, 0::2] << 4)).astype(np.uint8)
    x, codes, ws, b = _fp4_case(3, 32, 256, 5)
    with pytest.raises(AssertionError):
        pins.check_w4a8_vs_mxfp8(oracle.linear_w4a8_ref, swapped, x, codes, ws, oracle.e2m1_decode, b)


def test_mutant_layer_scale_misread_is_caught():
    """A layer that reads the weight scale of the neighbouring block."""
    def bad(x, wp, w_s, bias=None, N=None):
        return oracle.linear_w4a8_ref(x, wp, np.roll(np.asarray(w_s), 1, axis=1), bias, N)
    x, codes, ws, b = _fp4_case(4, 32, 512, 6)
    ws = ws.copy()
    ws[:, 1] += 1      # make neighbouring blocks' scales differ
    with pytest.raises(AssertionError):
        pins.check_w4a8_vs_mxfp8(bad, oracle.pack_fp4, x, codes, ws, oracle.e2m1_decode, b)
