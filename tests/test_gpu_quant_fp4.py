"""MXFP4 quantization on the GPU (mxfp8_quantize_fp4) vs the oracle's
quantize_mxfp4 + pack_fp4: bit-exact bytes and scales."""

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_amd import api, synth
from tests import gpu_util

pytestmark = pytest.mark.gpu


def _check_exact(x, label):
    print("CASE fp4", label, tuple(x.shape), flush=True)
    q, s = api.quantize_fp4(x.to(gpu_util.dev()))
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    codes, s2 = oracle.quantize_mxfp4(x.to(torch.float64).numpy())
    q2 = oracle.pack_fp4(codes)
    bad_s = np.argwhere(s != s2)
    assert bad_s.size == 0, (label, bad_s[:5], s[tuple(bad_s[0])], s2[tuple(bad_s[0])])
    bad_q = np.argwhere(q != q2)
    assert bad_q.size == 0, (label, bad_q[:5], hex(q[tuple(bad_q[0])]), hex(q2[tuple(bad_q[0])]))


def test_exhaustive_bf16_times_scale_exponent():
    """Every finite bf16 value under every scale exponent the rule can give
    (blocks anchored at the top of each binade, both signs)."""
    x = gpu_util.exhaustive_quant_input()
    _check_exact(x, "exhaustive")


@pytest.mark.parametrize("kind", ["normal", "stress", "zeros_signed", "tiny", "huge", "ragged_k"])
def test_inputs(kind):
    g = torch.Generator().manual_seed(29)
    if kind == "normal":
        x = synth.randn_bf16((300, 2048), 0.02, g)
    elif kind == "stress":
        x = synth.scale_stress(synth.randn_bf16((129, 1024), 1.0, g), seed=5)
    elif kind == "zeros_signed":
        x = synth.randn_bf16((33, 256), 1.0, g)
        x[:, :64] = 0.0
        x[::2, 64:96] = -0.0
    elif kind == "tiny":
        x = (synth.randn_bf16((16, 512), 1.0, g).float() * 2.0 ** -128).to(torch.bfloat16)
    elif kind == "huge":
        x = (synth.randn_bf16((16, 512), 1.0, g).float() * 2.0 ** 120).to(torch.bfloat16)
    else:
        x = synth.randn_bf16((7, 96), 1.0, g)       # K % 32 == 0 but not % 256
    _check_exact(x, kind)


def test_strided_rows():
    g = torch.Generator().manual_seed(31)
    big = synth.randn_bf16((20, 1024 + 64), 1.0, g).to(gpu_util.dev())
    x = big[:, :1024]
    q = torch.empty((20, 512 + 32), dtype=torch.uint8, device=gpu_util.dev())
    s = torch.empty((20, 32 + 4), dtype=torch.uint8, device=gpu_util.dev())
    st = api.mxfp8_quantize_fp4(x.data_ptr(), 20, 1024, x.stride(0), q.data_ptr(), q.stride(0), s.data_ptr(),
                                s.stride(0), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    codes, s2 = oracle.quantize_mxfp4(x.cpu().to(torch.float64).numpy())
    assert np.array_equal(q[:, :512].cpu().numpy(), oracle.pack_fp4(codes))
    assert np.array_equal(s[:, :32].cpu().numpy(), s2)


def test_quantize_then_w4a8_layer():
    """bf16 weight -> GPU MXFP4 quantizer -> prepare -> W4A8 layer, against
    the oracle's layer on the oracle's quantization of the same weight."""
    g = torch.Generator().manual_seed(37)
    M, N, K = 5, 384, 1024
    x = synth.randn_bf16((M, K), 1.0, g)
    w = synth.randn_bf16((N, K), 0.02, g)
    q, s = api.quantize_fp4(w.to(gpu_util.dev()))
    pw = api.prepare_weight_fp4(q, s)
    y = api.linear(x.to(gpu_util.dev()), pw).float().cpu().numpy()
    codes, ws = oracle.quantize_mxfp4(w.to(torch.float64).numpy())
    xn = x.to(torch.float64).numpy()
    r = oracle.linear_w4a8_ref(xn, oracle.pack_fp4(codes), ws)
    from tests.test_gpu_w4a8 import tolerance4
    gpu_util.compare(y, r, tolerance4(xn, codes, ws, K), "quantize_fp4 -> w4a8")
