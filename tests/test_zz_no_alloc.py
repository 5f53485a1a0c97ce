"""mxfp8_linear_noalloc (the entry point for callers that cannot allocate
device memory) against mxfp8_linear, through the C ABI: the same kernels, so
the outputs must be bit-identical.  Per GEMM path, two calls in a row on the
static scratch, the second with a smaller input; a slab-kernel shape whose
fp32 partials exceed the scratch runs the mid-M kernel instead; then a shape
too large for the scratch is refused before anything is launched."""

import pytest
import torch

from mxfp8_block_scaled_amd import api, synth
from tests import gpu_util

pytestmark = pytest.mark.gpu


def _call_both(x, pw, bias, N, force_ref=0, force_new=0):
    """mxfp8_linear under path forcing force_ref, mxfp8_linear_noalloc under
    force_new (0: the shape table's choice for both)."""
    d = gpu_util.dev()
    M, K = x.shape
    s = torch.cuda.current_stream(d).cuda_stream
    bp = None if bias is None else bias.data_ptr()
    y_ref = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device=d)   # ldy > N: columns >= N untouched
    y_new = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device=d)
    prev = api.mxfp8_debug_force_path(force_ref)
    try:
        ws = torch.zeros(api.mxfp8_linear_workspace_bytes(M, N, K), dtype=torch.uint8, device=d)
        assert api.mxfp8_linear(x.data_ptr(), M, K, K, pw.w_packed.data_ptr(), pw.s_packed.data_ptr(), N, bp,
                                y_ref.data_ptr(), N + 8, ws.data_ptr(), ws.numel(), s) == 0
        api.mxfp8_debug_force_path(force_new)
        assert api.mxfp8_linear_noalloc(x.data_ptr(), M, K, K, pw.w_packed.data_ptr(), pw.s_packed.data_ptr(), N,
                                        bp, y_new.data_ptr(), N + 8, s) == 0
    finally:
        api.mxfp8_debug_force_path(prev)
    torch.cuda.synchronize()
    assert torch.equal(y_new.view(torch.int16), y_ref.view(torch.int16))
    assert bool((y_new[:, N:].float() == 7.0).all())


@pytest.mark.parametrize("label,Ms,N,K,force", [
    ("decode", (16, 3), 4096, 4096, 0),
    ("mid-M", (128, 40), 4096, 4096, 0),
    ("slab", (64, 17), 4096, 8192, 5),
    ("medium tile", (1024, 300), 640, 1024, 6),
    ("medium tile, 64 rows", (513, 200), 384, 2048, 7),
    ("tile", (300, 200), 640, 1024, 0),
    ("tile split-K", (256, 129), 512, 2048, 0),
])
def test_noalloc_matches_linear(label, Ms, N, K, force):
    g = torch.Generator().manual_seed(sum(Ms) + N + K)
    d = gpu_util.dev()
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N)
    pw = gpu_util.gpu_prepare(w)
    bias = synth.randn_bf16((N,), 0.1, g).to(d)
    for M in Ms:
        prev = api.mxfp8_debug_force_path(force)
        try:
            need = api.mxfp8_linear_workspace_bytes(M, N, K)
            plan = api.mxfp8_debug_plan(M, N, K)
        finally:
            api.mxfp8_debug_force_path(prev)
        print(f"CASE noalloc {label} M={M} N={N} K={K} plan={plan} scratch={need}", flush=True)
        assert need <= api.NOALLOC_SCRATCH_BYTES
        x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M).to(d)
        _call_both(x, pw, bias if M % 2 == 0 else None, N, force, force)


def test_noalloc_slab_partials_over_scratch_run_mid():
    """M = 32, N = 16500, K = 8192 on the slab kernel needs 8 slices of fp32
    partials [32, 16512] (16.9 MB, above the 16 MiB scratch): the
    allocation-free entry runs the mid-M kernel, bit-identical to
    mxfp8_linear forced onto that kernel."""
    M, N, K = 32, 16500, 8192
    d = gpu_util.dev()
    prev = api.mxfp8_debug_force_path(5)
    try:
        assert api.mxfp8_debug_plan(M, N, K)[0] == 3
        assert api.mxfp8_linear_workspace_bytes(M, N, K) == 8 * M * 16512 * 4 > api.NOALLOC_SCRATCH_BYTES
    finally:
        api.mxfp8_debug_force_path(prev)
    g = torch.Generator(device=d).manual_seed(11)
    w = (torch.randn((N, K), generator=g, device=d) * 0.02).to(torch.bfloat16)
    wq, ws = api.quantize_act(w)
    pw = api.prepare_weight(wq, ws)
    del w, wq, ws
    x = torch.randn((M, K), generator=g, device=d).to(torch.bfloat16)
    bias = (torch.randn((N,), generator=g, device=d) * 0.1).to(torch.bfloat16)
    print(f"CASE noalloc slab over scratch M={M} N={N} K={K}", flush=True)
    _call_both(x, pw, bias, N, force_ref=3, force_new=5)


def test_noalloc_refuses_too_large():
    M, N, K = 16384, 5120, 2048
    assert api.mxfp8_linear_workspace_bytes(M, N, K) > api.NOALLOC_SCRATCH_BYTES
    P = 0x10000   # never dereferenced: the size check returns before any launch
    assert api.mxfp8_linear_noalloc(P, M, K, K, P, P, N, None, P, N, None) == -8
