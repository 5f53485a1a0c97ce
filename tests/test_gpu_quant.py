"""Activation quantization on the GPU vs the oracle: bit-exact bytes."""

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_amd import api, synth
from tests import gpu_util

pytestmark = pytest.mark.gpu


def _check_exact(x, label):
    print("CASE", label, tuple(x.shape), flush=True)
    q, s = gpu_util.gpu_quantize(x)
    q2, s2 = oracle.quantize_mx(x.to(torch.float64).numpy())
    bad_s = np.argwhere(s != s2)
    bad_q = np.argwhere(q != q2)
    assert bad_s.size == 0, (label, bad_s[:5], s[tuple(bad_s[0])], s2[tuple(bad_s[0])])
    assert bad_q.size == 0, (label, bad_q[:5], q[tuple(bad_q[0])], q2[tuple(bad_q[0])])


def test_exhaustive_bf16_times_scale_exponent():
    x = gpu_util.exhaustive_quant_input()
    assert x.numel() > 8_000_000
    _check_exact(x, "exhaustive")


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_config_activations(cfg):
    x, _, _ = synth.config_inputs(cfg)
    if x.shape[0] > 2048:   # full size on the GPU, oracle on sampled rows (rows are independent)
        q, s = api.quantize_act(x.to(gpu_util.dev()))
        torch.cuda.synchronize()
        rows = torch.randperm(x.shape[0], generator=torch.Generator().manual_seed(cfg))[:256]
        rows = torch.cat([rows, torch.tensor([0, x.shape[0] - 1])])
        q2, s2 = oracle.quantize_mx(x[rows].to(torch.float64).numpy())
        assert np.array_equal(q[rows.to(q.device)].cpu().numpy(), q2)
        assert np.array_equal(s[rows.to(s.device)].cpu().numpy(), s2)
    else:
        _check_exact(x, f"config{cfg}")


@pytest.mark.parametrize("M", [1, 7, 16, 128])
def test_decode_activations_with_outliers(M):
    x, _, _ = synth.config_inputs(2, M)
    _check_exact(x, f"decode M={M}")


@pytest.mark.parametrize("kind", ["stress", "zeros_signed", "tiny", "huge", "ragged"])
def test_edge_inputs(kind):
    g = torch.Generator().manual_seed(17)
    if kind == "stress":
        x = synth.scale_stress(synth.randn_bf16((129, 1024), 1.0, g), seed=3)
    elif kind == "zeros_signed":
        x = synth.randn_bf16((33, 256), 1.0, g)
        x[:, :64] = 0.0
        x[::2, 64:96] = -0.0
    elif kind == "tiny":
        x = (torch.randn(40, 512, generator=g) * 2.0 ** -127).to(torch.bfloat16)
    elif kind == "huge":
        x = (torch.randn(40, 512, generator=g) * 2.0 ** 125).to(torch.bfloat16)
    else:  # K not a multiple of 256 and odd M: quantize alone only needs K % 32
        x = synth.randn_bf16((37, 96), 1.0, g)
    _check_exact(x, kind)


def test_strided_rows_and_empty():
    g = torch.Generator().manual_seed(5)
    big = synth.randn_bf16((20, 512), 1.0, g).to(gpu_util.dev())
    x = big[:, :256]                      # row stride 512 elements
    M, K = x.shape
    q = torch.full((M, 272), 0xAB, dtype=torch.uint8, device=x.device)   # ldq 272 > K
    s = torch.full((M, 12), 0xCD, dtype=torch.uint8, device=x.device)    # lds 12 > K/32
    st = api.mxfp8_quantize_act(x.data_ptr(), M, K, 512, q.data_ptr(), 272, s.data_ptr(), 12,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    q2, s2 = oracle.quantize_mx(x.cpu().to(torch.float64).numpy())
    assert np.array_equal(q[:, :K].cpu().numpy(), q2)
    assert np.array_equal(s[:, :8].cpu().numpy(), s2)
    assert bool((q[:, K:] == 0xAB).all()) and bool((s[:, 8:] == 0xCD).all())   # padding untouched
    assert api.mxfp8_quantize_act(x.data_ptr(), 0, K, 512, q.data_ptr(), 272, s.data_ptr(), 12, None) == 0
