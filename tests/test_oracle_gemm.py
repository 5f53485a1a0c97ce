"""Pins of the oracle's dequantized GEMM / linear layer (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_amd import synth
from tests import pins


def lin(x, qw, sw, b):
    return oracle.linear_ref(x, qw, sw, b)


@pytest.mark.parametrize("M,N,K,bias", [(3, 5, 256, False), (2, 4, 512, True), (1, 7, 256, True)])
def test_fraction_bruteforce(M, N, K, bias):
    g = torch.Generator().manual_seed(M * 100 + N)
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N)
    b = synth.randn_bf16((N,), 0.1, g) if bias else None
    pins.check_gemm_bruteforce(lin, oracle.quantize_mx, x, w, b)


def test_one_hot_w_pins_k_and_n_mapping():
    g = torch.Generator().manual_seed(7)
    x = synth.scale_stress(synth.randn_bf16((9, 512), 1.0, g), seed=9)
    perm = torch.randperm(512, generator=g)[:37].numpy()
    pins.check_one_hot_w(lin, oracle.quantize_mx, x, perm)


def test_one_hot_a_pins_weight_mapping_and_bias():
    g = torch.Generator().manual_seed(8)
    w = synth.scale_stress(synth.randn_bf16((130, 256), 0.02, g), seed=10)
    b = synth.randn_bf16((130,), 0.1, g)
    perm = torch.randperm(256, generator=g)[:11].numpy()
    pins.check_one_hot_a(lin, oracle.quantize_mx, w, perm, b)


@pytest.mark.parametrize("c", [0.25, 2.0 ** -9, 448.0])
def test_constant_operands(c):
    pins.check_constant(lin, oracle.quantize_mx, 3, 5, 512, c, bias=np.arange(5) * 0.5)


@pytest.mark.parametrize("j", [-3, 2])
def test_power_of_two_equivariance(j):
    g = torch.Generator().manual_seed(12)
    x = synth.randn_bf16((6, 512), 1.0, g)
    w = synth.randn_bf16((10, 512), 0.02, g)
    pins.check_equivariance(lin, oracle.quantize_mx, x, w, j)


def test_logical_n_slice_ignores_padding_rows():
    """Rows >= N of the weight (physical padding) never reach the output."""
    g = torch.Generator().manual_seed(13)
    x = synth.randn_bf16((4, 256), 1.0, g)
    w = synth.randn_bf16((256, 256), 0.02, g)
    qw, sw = oracle.quantize_mx(w.double().numpy())
    y = oracle.linear_ref(x.double().numpy(), qw, sw, None, N=130)
    qw2 = qw.copy()
    qw2[130:] = 0x7E
    sw2 = sw.copy()
    sw2[130:] = 0xF0
    y2 = oracle.linear_ref(x.double().numpy(), qw2, sw2, None, N=130)
    assert y.shape == (4, 130) and np.array_equal(y, y2)


def test_k_not_multiple_of_256_rejected():
    with pytest.raises(ValueError):
        oracle.linear_ref(np.zeros((1, 224)), np.zeros((4, 224), np.uint8), np.zeros((4, 7), np.uint8))


@pytest.mark.parametrize("shape", [(1, 130, 256), (7, 256, 512), (128, 130, 768)])
def test_pages_cosine_check(shape):
    """The vLLM PR #52204 test's acceptance rule, on the oracle: cosine
    similarity with the unquantized bf16 product above 0.98, seed 0, x and W
    both ~ N(0, 1) bf16, shapes (M, N, K) as in that test."""
    torch.manual_seed(0)
    m, n, k = shape
    x = torch.randn((m, k), dtype=torch.bfloat16)
    w = torch.randn((n, k), dtype=torch.bfloat16)
    qw, sw = oracle.quantize_mx(w.double().numpy())
    y = oracle.bf16_round(oracle.linear_ref(x.double().numpy(), qw, sw))
    ref = x.double().numpy() @ w.double().numpy().T
    cos = (y * ref).sum() / np.sqrt((y * y).sum() * (ref * ref).sum())
    assert y.shape == (m, n)
    assert cos > 0.98
