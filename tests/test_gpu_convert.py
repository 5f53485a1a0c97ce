"""The offline checkpoint converter on the GPU: safetensors in, MX bytes out,
bit-exact with the oracle's quantizers; other tensors copied unchanged."""

import os
import tempfile

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_amd import convert, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_convert_roundtrip(fmt):
    from safetensors.torch import load_file, save_file
    g = torch.Generator().manual_seed(41)
    tensors = {
        "layer.0.proj.weight": synth.randn_bf16((96, 256), 0.02, g),
        "layer.0.proj.bias": synth.randn_bf16((96,), 0.1, g),
        "layer.0.norm.weight": synth.randn_bf16((256,), 1.0, g),          # 1-D: copied
        "layer.1.up.weight": synth.scale_stress(synth.randn_bf16((64, 512), 0.02, g), seed=3),
        "layer.1.odd.weight": synth.randn_bf16((8, 48), 1.0, g),           # K % 32 == 16: copied
    }
    with tempfile.TemporaryDirectory() as d:
        src, dst = os.path.join(d, "in.safetensors"), os.path.join(d, "out.safetensors")
        save_file(tensors, src)
        names = convert.convert(src, dst, fmt=fmt, device="cuda:0")
        assert sorted(names) == ["layer.0.proj.weight", "layer.1.up.weight"]
        out = load_file(dst)
    for name in names:
        x = tensors[name].to(torch.float64).numpy()
        if fmt == "mxfp8":
            q, s = oracle.quantize_mx(x)
        else:
            codes, s = oracle.quantize_mxfp4(x)
            q = oracle.pack_fp4(codes)
        assert np.array_equal(out[name + ".qdata"].numpy(), q), name
        assert np.array_equal(out[name + ".scale"].numpy(), s), name
    for name in ["layer.0.proj.bias", "layer.0.norm.weight", "layer.1.odd.weight"]:
        assert torch.equal(out[name], tensors[name])
