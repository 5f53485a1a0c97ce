"""The MXFP8 linear layer on the GPU vs the oracle (tolerance derived in
tests/gpu_util.py), plus exact pins, layout round trip, path agreement and
HIP-graph replay."""

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_amd import api, synth
from tests import gpu_util

pytestmark = pytest.mark.gpu


def test_prepare_unpack_roundtrip():
    g = torch.Generator().manual_seed(2)
    for N, K in [(130, 256), (256, 512), (1, 768), (300, 1024)]:
        print("CASE roundtrip", N, K, flush=True)
        wq = torch.randint(0, 256, (N, K), generator=g, dtype=torch.uint8)
        ws = torch.randint(0, 256, (N + 3, K // 32 + 5), generator=g, dtype=torch.uint8)  # larger, strided
        pw = api.prepare_weight(wq.to(gpu_util.dev()), ws.to(gpu_util.dev()))
        w2, s2 = pw.unpack()
        torch.cuda.synchronize()
        n_pad = (N + 127) // 128 * 128
        assert w2.shape == (n_pad, K) and s2.shape == (n_pad, K // 32)
        assert torch.equal(w2[:N].cpu(), wq)
        assert torch.equal(s2[:N].cpu(), ws[:N, : K // 32])
        assert bool((w2[N:] == 0).all()) and bool((s2[N:] == 127).all())


@pytest.mark.parametrize("path", [1, 2, 6, 7])
def test_one_hot_weight_exact(path):
    """W[n, perm[n]] = 1: y[m, n] = bf16(deq(A)[m, perm[n]]) exactly (a single
    nonzero term per output).  Pins the MFMA operand/scale lane mapping, the K
    and N indexing, padding and zero-scale blocks, on the tile GEMM, the
    automatic path at M = 9 and the medium-tile GEMM's two tile heights."""
    M = 9 if path == 2 else 300
    g = torch.Generator().manual_seed(4)
    K, N = 512, 200
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=8)
    perm = torch.randint(0, K, (N,), generator=g)
    w = torch.zeros(N, K, dtype=torch.bfloat16)
    w[torch.arange(N), perm] = 1.0
    pw = gpu_util.gpu_prepare(w)
    prev = api.mxfp8_debug_force_path(path)
    try:
        y = api.linear(x.to(gpu_util.dev()), pw).float().cpu().numpy()
    finally:
        api.mxfp8_debug_force_path(prev)
    qa, sa = oracle.quantize_mx(x.double().numpy())
    deqa = oracle.dequantize_mx(qa, sa)
    exp = oracle.bf16_round(deqa[:, perm.numpy()])
    assert np.array_equal(y, exp)


@pytest.mark.parametrize("path", [1, 2, 6, 7])
def test_one_hot_activation_exact(path):
    """x[m, perm[m]] = 1 (scale-stressed weight): y[m, n] = bf16(deq(W)[n, perm[m]] + bias[n])."""
    M = 11 if path == 2 else 260
    g = torch.Generator().manual_seed(6)
    K, N = 768, 384
    perm = torch.randint(0, K, (M,), generator=g)
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    x[torch.arange(M), perm] = 1.0
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=9)
    bias = synth.randn_bf16((N,), 0.1, g)
    pw = gpu_util.gpu_prepare(w)
    prev = api.mxfp8_debug_force_path(path)
    try:
        y = api.linear(x.to(gpu_util.dev()), pw, bias.to(gpu_util.dev())).float().cpu().numpy()
    finally:
        api.mxfp8_debug_force_path(prev)
    wq, ws = gpu_util.oracle_weight(w)
    deqw = oracle.dequantize_mx(wq, ws)
    # one fp32 add of the bias: exact here? compare after the same fp32 add + bf16 rounding
    v = (deqw[:, perm.numpy()].T.astype(np.float32) + bias.float().numpy()[None, :]).astype(np.float64)
    assert np.array_equal(y, oracle.bf16_round(v))


def test_config1_single():
    x, w, b = synth.config_inputs(1)
    gpu_util.run_linear_and_check(x, w, b, "config1", force_path=0)
    gpu_util.run_linear_and_check(x, w, b, "config1-tile", force_path=1)


@pytest.mark.parametrize("M", [1, 7, 16, 128])
def test_config2_decode(M):
    x, w, b = synth.config_inputs(2, M)
    gpu_util.run_linear_and_check(x, w, b, f"config2 M={M}")


@pytest.mark.parametrize("M,N,K", [(m, n, k) for m in (1, 2, 3, 5, 15, 16, 17, 33, 127, 128, 129, 257)
                                   for n, k in ((1, 256), (130, 512), (255, 768), (384, 256))])
def test_edge_grid(M, N, K):
    g = torch.Generator().manual_seed(M * 1000 + N + K)
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M + 1)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N + 2)
    b = synth.randn_bf16((N,), 0.1, g) if (M + N) % 2 else None
    gpu_util.run_linear_and_check(x, w, b, f"edge {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(5, 130, 512), (17, 1, 256), (48, 255, 768), (64, 130, 1024),
                                   (80, 384, 2048), (90, 255, 512), (100, 384, 8192), (128, 4096, 4096),
                                   (113, 200, 6144)])
def test_mid_path(M, N, K):
    """The mid-M kernel (automatic for 16 < M <= 128; path 3 forces it at
    M = 5): 1..4 K steps per wave (K = 6144 leaves one of four empty), 1..8
    row groups with a ragged last one, ragged N, bias on and off."""
    g = torch.Generator().manual_seed(M * 31 + N + K)
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M + 5)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N + 6)
    b = synth.randn_bf16((N,), 0.1, g) if M % 2 == 0 else None
    st = gpu_util.run_linear_and_check(x, w, b, f"mid {M}x{N}x{K}", force_path=3)
    assert st["over_bound"] == 0


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (5, 130, 512), (17, 1, 256), (48, 255, 768), (64, 130, 1024),
                                   (80, 384, 2048), (90, 255, 512), (100, 384, 8192), (128, 4096, 4096),
                                   (113, 200, 6144), (33, 4096, 8192), (127, 1000, 2048), (9, 1024, 16384),
                                   (128, 512, 10240)])
def test_slab_path(M, N, K):
    """The split-K slab kernel (path 5 forces it): 1, 2 and 4 K steps per
    wave (4 at N = 4096, K = 8192; 2 at N = K = 4096 and at N = 1024,
    K = 16384; 1 where fewer than 256 workgroups would result), 1..8 row
    groups with a ragged last one, one K slice (K = 256) up to 40, K above
    the other small-M kernels' limit, ragged N, bias on and off."""
    g = torch.Generator().manual_seed(M * 37 + N + K)
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M + 7)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N + 8)
    b = synth.randn_bf16((N,), 0.1, g) if M % 2 == 0 else None
    st = gpu_util.run_linear_and_check(x, w, b, f"slab {M}x{N}x{K}", force_path=5)
    assert st["over_bound"] == 0


@pytest.mark.parametrize("force", [6, 7])
@pytest.mark.parametrize("M,N,K", [(1, 130, 256), (17, 1, 512), (64, 384, 768), (100, 255, 1024), (129, 130, 2048),
                                   (200, 1000, 256), (300, 640, 4096), (513, 384, 1024), (1024, 520, 8448)])
def test_med_path(M, N, K, force):
    """The medium-tile GEMM (path 6: 128 x 128 tiles, 7: 128 x 64): one and
    many tiles along M and N, ragged last tiles in both, K from one 128-K
    step pair to 66 steps, bias on and off."""
    g = torch.Generator().manual_seed(M * 13 + N + K + force)
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M + 3)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N + 4)
    b = synth.randn_bf16((N,), 0.1, g) if (M + N) % 2 else None
    st = gpu_util.run_linear_and_check(x, w, b, f"med{force} {M}x{N}x{K}", force_path=force)
    assert st["over_bound"] == 0


@pytest.mark.parametrize("M,N,K", [(1, 130, 8192), (7, 384, 6144), (16, 255, 8192), (4, 256, 8448)])
def test_decode_large_k(M, N, K):
    """The decode kernel with four K steps per wave (K = 6144: one of them
    empty; K = 8192: the largest K it takes) and, at K = 8448, the shape
    falling back to the tile GEMM."""
    g = torch.Generator().manual_seed(M * 7 + N + K)
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M + 11)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N + 12)
    b = synth.randn_bf16((N,), 0.1, g) if M % 2 == 0 else None
    st = gpu_util.run_linear_and_check(x, w, b, f"decode {M}x{N}x{K}")
    assert st["over_bound"] == 0


def test_skinny_and_tile_paths_agree():
    """Same inputs through both GEMM paths: each within the bound of the
    oracle; their difference stays within the sum of the two bounds."""
    for M in (1, 5, 16):
        x, w, b = synth.config_inputs(2, M)
        s1 = gpu_util.run_linear_and_check(x, w, b, f"skinny M={M}", force_path=2)
        s2 = gpu_util.run_linear_and_check(x, w, b, f"tile M={M}", force_path=1)
        assert s1["over_bound"] == 0 and s2["over_bound"] == 0


def test_packed_entries_match_linear():
    """mxfp8_quantize_act_packed + mxfp8_gemm_packed are the two kernels of
    mxfp8_linear's large-M path: same bytes out."""
    g = torch.Generator().manual_seed(3)
    x = synth.randn_bf16((300, 512), 1.0, g).to(gpu_util.dev())
    w = synth.randn_bf16((260, 512), 0.02, g)
    b = synth.randn_bf16((260,), 0.1, g).to(gpu_util.dev())
    pw = gpu_util.gpu_prepare(w)
    pa = api.quantize_act_packed(x)
    y1 = api.gemm_packed(pa, pw, b)
    y2 = api.linear(x, pw, b)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("M,K", [(1, 256), (130, 512), (300, 768), (256, 1024),
                                 (4096, 2048), (2048, 2048), (5504, 768)])
def test_packed_activation_quantizer_bit_exact(M, K):
    """The packed-layout quantizer writes exactly the oracle's bytes (checked
    after unpacking), with zero pad rows and zero scales.  The launch takes
    two, four or eight 64-K steps per workgroup by grid size: the small
    shapes take two, (2048, 2048) and (5504, 768) four (the latter because
    its step count is not a multiple of eight), (4096, 2048) eight."""
    g = torch.Generator().manual_seed(M + K)
    x = synth.scale_stress(synth.activations(M, K, 1.0, g, 0.01, 50.0), seed=M)
    pa = api.quantize_act_packed(x.to(gpu_util.dev()))
    q, s = pa.unpack()
    torch.cuda.synchronize()
    q2, s2 = oracle.quantize_mx(x.to(torch.float64).numpy())
    assert np.array_equal(q[:M].cpu().numpy(), q2)
    assert np.array_equal(s[:M].cpu().numpy(), s2)
    assert bool((q[M:] == 0).all()) and bool((s[M:] == 0).all())


def test_deterministic_repeat():
    x, w, b = synth.config_inputs(2, 16)
    pw = gpu_util.gpu_prepare(w)
    xs, bs = x.to(gpu_util.dev()), b.to(gpu_util.dev())
    ys = [api.linear(xs, pw, bs) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:])


def test_leading_dims_and_output_contiguity():
    g = torch.Generator().manual_seed(9)
    x = synth.randn_bf16((2, 3, 256), 1.0, g).to(gpu_util.dev())
    w = synth.randn_bf16((130, 256), 0.02, g)
    pw = gpu_util.gpu_prepare(w)
    y = api.linear(x, pw)
    assert y.shape == (2, 3, 130) and y.is_contiguous()
    y2 = api.linear(x.reshape(6, 256), pw)
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(6, 130), y2)


def test_hip_graph_replay_matches_eager():
    """The layer captured into a HIP graph and replayed several times, with
    eager work in between, matches the eager result every time (vLLM PR
    #52204 tested CUDA-graph capture and replay the same way)."""
    for M in (7, 300):
        x, w, b = synth.config_inputs(1) if M == 7 else synth.linear_inputs(M, 640, 512, seed=4)
        pw = gpu_util.gpu_prepare(w)
        xs = x.to(gpu_util.dev())
        bs = None if b is None else b.to(gpu_util.dev())
        eager = api.linear(xs, pw, bs).clone()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            api.linear(xs, pw, bs)        # warm the workspace outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            out = api.linear(xs, pw, bs)
        for it in range(4):
            out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), (M, it)
            _ = api.linear(xs, pw, bs)    # eager work between replays
            torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(1, 130, 256), (7, 256, 512), (128, 130, 768)])
def test_pages_cosine_check(shape):
    """vLLM PR #52204's own acceptance rule on its own shapes: seed 0, x and W
    ~ N(0,1) bf16; cosine similarity with the unquantized product > 0.98;
    output shape (m, n) and contiguous."""
    torch.manual_seed(0)
    m, n, k = shape
    x = torch.randn((m, k), dtype=torch.bfloat16)
    w = torch.randn((n, k), dtype=torch.bfloat16)
    pw = gpu_util.gpu_prepare(w)
    y = api.linear(x.to(gpu_util.dev()), pw)
    ref = x.float() @ w.float().t()
    cos = torch.nn.functional.cosine_similarity(y.float().cpu().flatten(), ref.flatten(), dim=0)
    assert y.shape == (m, n) and y.is_contiguous()
    assert cos.item() > 0.98


@pytest.mark.parametrize("cfg", [3, 4])
def test_full_size_sampled(cfg):
    """Full-size configs in the launch configuration the bench times; the
    oracle checks sampled rows x columns (quantization is row-local, so the
    samples are exact sub-problems), including the last row and column."""
    x, w, b = synth.config_inputs(cfg)
    M, K = x.shape
    N = w.shape[0]
    print("CASE full", cfg, M, N, K, flush=True)
    pw = gpu_util.gpu_prepare(w)
    y = api.linear(x.to(gpu_util.dev()), pw, None if b is None else b.to(gpu_util.dev()))
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(100 + cfg)
    rows = torch.cat([torch.randperm(M, generator=gen)[:96], torch.tensor([0, M - 1])])
    cols = torch.cat([torch.randperm(N, generator=gen)[:96], torch.tensor([0, N - 1])])
    ys = y[rows.to(y.device)][:, cols.to(y.device)].float().cpu().numpy()
    wq, ws = gpu_util.oracle_weight(w[cols])
    xn = x[rows].to(torch.float64).numpy()
    bn = None if b is None else b[cols].to(torch.float64).numpy()
    r = oracle.linear_ref(xn, wq, ws, bn)
    gpu_util.compare(ys, r, gpu_util.tolerance(xn, wq, ws, len(cols), K), f"config{cfg} sampled")


@pytest.mark.parametrize("M,N,K", [(4100, 16500, 256), (2000, 9000, 768), (1031, 32768, 512)])
def test_persistent_ragged_sampled(M, N, K):
    """More tiles than workgroups with ragged M and N: every workgroup of the
    persistent GEMM runs several tiles, edge tiles sit between full ones (the
    next tile's first wait then covers an unknown number of stores), the bias
    copy is cut at N, and K = 256 has a single pair of steps per tile.
    Sampled rows x columns, including the first and last row and column,
    against the oracle."""
    g = torch.Generator().manual_seed(M + N + K)
    x = synth.randn_bf16((M, K), 1.0, g)
    w = synth.randn_bf16((N, K), 0.02, g)
    b = synth.randn_bf16((N,), 0.1, g)
    print("CASE persistent", M, N, K, flush=True)
    pw = gpu_util.gpu_prepare(w)
    y = api.linear(x.to(gpu_util.dev()), pw, b.to(gpu_util.dev()))
    torch.cuda.synchronize()
    rows = torch.cat([torch.randperm(M, generator=g)[:96], torch.tensor([0, M - 1])])
    cols = torch.cat([torch.randperm(N, generator=g)[:96], torch.tensor([0, N - 1])])
    ys = y[rows.to(y.device)][:, cols.to(y.device)].float().cpu().numpy()
    wq, ws = gpu_util.oracle_weight(w[cols])
    xn = x[rows].to(torch.float64).numpy()
    r = oracle.linear_ref(xn, wq, ws, b[cols].to(torch.float64).numpy())
    gpu_util.compare(ys, r, gpu_util.tolerance(xn, wq, ws, len(cols), K), f"persistent {M}x{N}x{K} sampled")


def _strided_case(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=seed + 1)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=seed + 2)
    b = synth.randn_bf16((N,), 0.1, g)
    return x, w, b


@pytest.mark.parametrize("path,M", [(0, 7), (1, 7), (0, 100), (1, 100), (0, 300)])
def test_strided_io_and_canary(path, M):
    """ldx > K and ldy > N through the C ABI on every GEMM path (decode and
    mid-M kernels automatic at M = 7 and 100, the tile GEMM forced there and
    automatic at M = 300): x is a view into a wider buffer whose extra
    columns hold huge values, y is written into a wider buffer whose columns
    >= N hold a canary.  The canary must survive, the extra x columns must
    not leak into the result, and y[:, :N] matches the oracle."""
    N, K = 200, 768
    x, w, b = _strided_case(M, N, K, seed=M + path)
    d = gpu_util.dev()
    ldx, ldy = K + 72, N + 24
    xbuf = torch.full((M, ldx), 3.0e38, dtype=torch.bfloat16)
    xbuf[:, :K] = x
    xbuf = xbuf.to(d)
    ybuf = torch.full((M, ldy), -7.0, dtype=torch.bfloat16, device=d)
    pw = gpu_util.gpu_prepare(w)
    bd = b.to(d)
    prev = api.mxfp8_debug_force_path(path)
    try:
        ws = torch.zeros(api.mxfp8_linear_workspace_bytes(M, N, K), dtype=torch.uint8, device=d)
        st = api.mxfp8_linear(xbuf.data_ptr(), M, K, ldx, pw.w_packed.data_ptr(), pw.s_packed.data_ptr(), N,
                              bd.data_ptr(), ybuf.data_ptr(), ldy, ws.data_ptr(), ws.numel(),
                              torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        api.mxfp8_debug_force_path(prev)
    assert st == 0
    yb = ybuf.float().cpu().numpy()
    assert np.all(yb[:, N:] == -7.0), "columns >= N were written"
    wq, wsc = gpu_util.oracle_weight(w)
    xn = x.to(torch.float64).numpy()
    r = oracle.linear_ref(xn, wq, wsc, b.to(torch.float64).numpy())
    gpu_util.compare(yb[:, :N], r, gpu_util.tolerance(xn, wq, wsc, N, K), f"strided path{path} M{M}")



@pytest.mark.parametrize("M,N,K", [(2000, 9000, 768), (4352, 4352, 1024), (2304, 8192, 2048)])
def test_persistent_store_paths_bit_exact(M, N, K):
    """The persistent GEMM's two epilogue store paths on multi-tile
    workgroups: with ldy % 8 == 0 full wave blocks leave as 16-byte
    non-temporal stores (and their count lets the next tile's first copies
    wait past them), with ldy odd every element is stored on its own.  More
    tiles than workgroups, so each workgroup runs several tiles; ragged M and
    N put partial tiles between full ones.  Both layouts must hold the same
    bits in every element, and neither may write the canary columns >= N."""
    g = torch.Generator().manual_seed(M + 7 * N + K)
    x = synth.randn_bf16((M, K), 1.0, g)
    w = synth.randn_bf16((N, K), 0.02, g)
    b = synth.randn_bf16((N,), 0.1, g)
    d = gpu_util.dev()
    xd, bd = x.to(d), b.to(d)
    pw = gpu_util.gpu_prepare(w)
    print("CASE store paths", M, N, K, flush=True)
    outs = []
    prev = api.mxfp8_debug_force_path(17)        # tile GEMM, one K split: the persistent kernel
    try:
        assert api.mxfp8_debug_plan(M, N, K) == (0, 1)
        for ldy in (N + 8, N + 3):
            ybuf = torch.full((M, ldy), -7.0, dtype=torch.bfloat16, device=d)
            ws = torch.zeros(api.mxfp8_linear_workspace_bytes(M, N, K), dtype=torch.uint8, device=d)
            st = api.mxfp8_linear(xd.data_ptr(), M, K, K, pw.w_packed.data_ptr(), pw.s_packed.data_ptr(), N,
                                  bd.data_ptr(), ybuf.data_ptr(), ldy, ws.data_ptr(), ws.numel(),
                                  torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            assert st == 0
            assert bool((ybuf[:, N:] == -7.0).all()), f"ldy {ldy}: columns >= N were written"
            outs.append(ybuf[:, :N].contiguous())
    finally:
        api.mxfp8_debug_force_path(prev)
    same = outs[0].view(torch.int16) == outs[1].view(torch.int16)
    assert bool(same.all()), f"{int((~same).sum())} elements differ, first at {(~same).nonzero()[0].tolist()}"
    # And sampled rows x columns against the oracle.
    rows = torch.cat([torch.randperm(M, generator=g)[:64], torch.tensor([0, M - 1])])
    cols = torch.cat([torch.randperm(N, generator=g)[:64], torch.tensor([0, N - 1])])
    ys = outs[0][rows.to(d)][:, cols.to(d)].float().cpu().numpy()
    wq, wsc = gpu_util.oracle_weight(w[cols])
    xn = x[rows].to(torch.float64).numpy()
    r = oracle.linear_ref(xn, wq, wsc, b[cols].to(torch.float64).numpy())
    gpu_util.compare(ys, r, gpu_util.tolerance(xn, wq, wsc, len(cols), K), f"store paths {M}x{N}x{K} sampled")


def _prequant_bound(A, W, r, K):
    acc = (K / 64.0) * 2.0 ** -10 * np.outer(np.abs(A).max(axis=1), np.abs(W).max(axis=1)) \
        + K * 2.0 ** -23 * (np.abs(A) @ np.abs(W).T)
    return (1 + 2.0 ** -8) * acc + 2.0 ** -133


@pytest.mark.parametrize("M,N,K", [(300, 130, 512), (256, 2048, 4096), (7, 384, 768), (129, 200, 1024)])
def test_gemm_prequant_oracle_codes(M, N, K):
    """The GEMM alone, driven by activations the oracle's side chose: random
    E4M3 codes (every finite code, both signs) and random scale bytes, in
    the boundary's row-major layout through mxfp8_gemm_prequant.  The result
    is checked against the oracle's exact dequantized product with the GEMM
    bound, so a GEMM error cannot hide behind a matching quantizer error.
    (256, 2048, 4096) has 8 tiles: K split 8 ways."""
    rng = np.random.default_rng(M * 7 + N + K)
    codes = rng.integers(0, 254, size=(M, K), dtype=np.int64)
    qa = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)     # skip the NaN code 0x7F (and 0xFF)
    sa = rng.integers(110, 140, size=(M, K // 32 + 3), dtype=np.int64).astype(np.uint8)   # wider than K/32
    g = torch.Generator().manual_seed(M + N)
    w = synth.scale_stress(synth.randn_bf16((N, K), 0.02, g), seed=N)
    bias = synth.randn_bf16((N,), 0.1, g)
    pw = gpu_util.gpu_prepare(w)
    d = gpu_util.dev()
    y = api.gemm_prequant(torch.from_numpy(qa).to(d), torch.from_numpy(sa).to(d), pw, bias.to(d))
    torch.cuda.synchronize()
    wq, ws = gpu_util.oracle_weight(w)
    A = oracle.dequantize_mx(qa, sa[:, : K // 32])
    W = oracle.dequantize_mx(wq, ws)
    r = oracle.gemm_dequant(qa, sa[:, : K // 32], wq, ws) + bias.to(torch.float64).numpy()[None, :]
    gpu_util.compare(y.float().cpu().numpy(), r, _prequant_bound(A, W, r, K), f"prequant {M}x{N}x{K}")


def test_gemm_prequant_matches_linear_tile_path():
    """Quantizing on the GPU and feeding the bytes to mxfp8_gemm_prequant
    gives mxfp8_linear's tile-path output bit for bit (the same GEMM on the
    same packed bytes; pad rows differ only in a scale byte that multiplies
    zeros)."""
    g = torch.Generator().manual_seed(12)
    d = gpu_util.dev()
    for M, N, K in [(300, 640, 1024), (64, 256, 512)]:
        x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=M).to(d)
        w = synth.randn_bf16((N, K), 0.02, g)
        b = synth.randn_bf16((N,), 0.1, g).to(d)
        pw = gpu_util.gpu_prepare(w)
        q, s = api.quantize_act(x)
        y1 = api.gemm_prequant(q, s, pw, b)
        prev = api.mxfp8_debug_force_path(1)
        try:
            y2 = api.linear(x, pw, b)
        finally:
            api.mxfp8_debug_force_path(prev)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), (M, N, K)


@pytest.mark.parametrize("splits", [1, 2, 4, 8])
def test_forced_tile_splits(splits):
    """Every K split count the shape table may choose, on a ragged shape
    (M = 300, N = 650: 2 x 3 tiles with a ragged last row and column tile)
    whose K = 2048 (32 64-K steps) takes all of them: each within the derived
    bound of the oracle's exact product."""
    g = torch.Generator().manual_seed(500 + splits)
    x = synth.randn_bf16((300, 2048), 1.0, g)
    w = synth.randn_bf16((650, 2048), 0.02, g)
    b = synth.randn_bf16((650,), 0.1, g)
    prev = api.mxfp8_debug_force_path(16 + splits)
    try:
        assert api.mxfp8_debug_plan(300, 650, 2048) == (0, splits)
    finally:
        api.mxfp8_debug_force_path(prev)
    gpu_util.run_linear_and_check(x, w, b, f"tile splits {splits}", force_path=16 + splits)
