"""mxfp8_linear_noalloc (the entry point for callers that cannot allocate
device memory) against mxfp8_linear, through the C ABI: the same kernels, so
the outputs must be bit-identical.  Per GEMM path, two calls in a row on the
static scratch, the second with a smaller input; then a shape too large for
the scratch is refused before anything is launched."""

import pytest
import torch

from mxfp8_block_scaled_amd import api, synth
from tests import gpu_util

pytestmark = pytest.mark.gpu


def _call_both(x, pw, bias, N):
    d = gpu_util.dev()
    M, K = x.shape
    s = torch.cuda.current_stream(d).cuda_stream
    bp = None if bias is None else bias.data_ptr()
    y_ref = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device=d)   # ldy > N: columns >= N untouched
    y_new = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device=d)
    ws = torch.zeros(api.mxfp8_linear_workspace_bytes(M, N, K), dtype=torch.uint8, device=d)
    assert api.mxfp8_linear(x.data_ptr(), M, K, K, pw.w_packed.data_ptr(), pw.s_packed.data_ptr(), N, bp,
                            y_ref.data_ptr(), N + 8, ws.data_ptr(), ws.numel(), s) == 0
    assert api.mxfp8_linear_noalloc(x.data_ptr(), M, K, K, pw.w_packed.data_ptr(), pw.s_packed.data_ptr(), N, bp,
                                    y_new.data_ptr(), N + 8, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(y_new.view(torch.int16), y_ref.view(torch.int16))
    assert bool((y_new[:, N:].float() == 7.0).all())


@pytest.mark.parametrize("label,Ms,N,K", [
    ("decode", (16, 3), 4096, 4096),
    ("mid-M", (128, 40), 4096, 4096),
    ("tile", (300, 200), 640, 1024),
    ("tile split-K", (256, 129), 512, 2048),
])
def test_noalloc_matches_linear(label, Ms, N, K):
    g = torch.Generator().manual_seed(sum(Ms) + N + K)
    d = gpu_util.dev()
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N)
    pw = gpu_util.gpu_prepare(w)
    bias = synth.randn_bf16((N,), 0.1, g).to(d)
    for M in Ms:
        need = api.mxfp8_linear_workspace_bytes(M, N, K)
        print(f"CASE noalloc {label} M={M} N={N} K={K} scratch={need}", flush=True)
        assert need <= api.NOALLOC_SCRATCH_BYTES
        x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M).to(d)
        _call_both(x, pw, bias if M % 2 == 0 else None, N)


def test_noalloc_refuses_too_large():
    M, N, K = 16384, 5120, 2048
    assert api.mxfp8_linear_workspace_bytes(M, N, K) > api.NOALLOC_SCRATCH_BYTES
    P = 0x10000   # never dereferenced: the size check returns before any launch
    assert api.mxfp8_linear_noalloc(P, M, K, K, P, P, N, None, P, N, None) == -8
