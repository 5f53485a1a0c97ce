"""The W4A8 layer (MXFP4 weights x MXFP8 activations) on the GPU vs the
oracle (oracle/mxfp4.py), with the GEMM tolerance of tests/gpu_util.py
applied to the dequantized MXFP4 weight, plus exact one-hot pins on both
paths (the 4-bit decode kernel for M <= 16, the 4-bit tile GEMM above; the
widened-weight split-K GEMM where the shape table splits K)."""

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_amd import api, synth
from tests import gpu_util

pytestmark = pytest.mark.gpu


def prepare(codes, ws):
    d = gpu_util.dev()
    return api.prepare_weight_fp4(torch.from_numpy(oracle.pack_fp4(codes)).to(d), torch.from_numpy(ws).to(d))


def test_prepare_unpack_roundtrip_fp4():
    """prepare_weight_fp4 then unpack gives back the E2M1 bytes and the
    [:N, :K/32] scales exactly, with zero pad rows and scale byte 127."""
    g = torch.Generator().manual_seed(3)
    d = gpu_util.dev()
    for N, K in [(130, 256), (256, 512), (1, 768), (300, 1024), (128, 4096)]:
        print("CASE roundtrip fp4", N, K, flush=True)
        w4 = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)
        ws = torch.randint(0, 256, (N + 3, K // 32 + 5), generator=g, dtype=torch.uint8)  # larger, strided
        pw = api.prepare_weight_fp4(w4.to(d), ws.to(d))
        w2, s2 = pw.unpack()
        torch.cuda.synchronize()
        n_pad = (N + 127) // 128 * 128
        assert w2.shape == (n_pad, K // 2) and s2.shape == (n_pad, K // 32)
        assert torch.equal(w2[:N].cpu(), w4)
        assert torch.equal(s2[:N].cpu(), ws[:N, : K // 32])
        assert bool((w2[N:] == 0).all()) and bool((s2[N:] == 127).all())


def tolerance4(x_np, codes, ws, K):
    qa, sa = oracle.quantize_mx(x_np)
    A = oracle.dequantize_mx(qa, sa)
    W = oracle.dequantize_mxfp4(oracle.pack_fp4(codes), ws)
    acc = (K / 64.0) * 2.0 ** -10 * np.outer(np.abs(A).max(axis=1), np.abs(W).max(axis=1)) \
        + K * 2.0 ** -23 * (np.abs(A) @ np.abs(W).T)
    return (1 + 2.0 ** -8) * acc + 2.0 ** -133


def run_and_check(M, N, K, seed, bias=True, force_path=0, x_std=1.0, stress=False):
    g = torch.Generator().manual_seed(seed)
    x = synth.randn_bf16((M, K), x_std, g)
    if stress:
        x = synth.scale_stress(x, seed=seed + 100)
    w = synth.randn_bf16((N, K), 0.02, g).to(torch.float64).numpy()
    codes, ws = oracle.quantize_mxfp4(w)
    b = synth.randn_bf16((N,), 0.1, g) if bias else None
    label = f"w4a8 M{M} N{N} K{K} path{force_path}"
    print("CASE", label, flush=True)
    pw = prepare(codes, ws)
    prev = api.mxfp8_debug_force_path(force_path)
    try:
        y = api.linear(x.to(gpu_util.dev()), pw, None if b is None else b.to(gpu_util.dev()))
        torch.cuda.synchronize()
    finally:
        api.mxfp8_debug_force_path(prev)
    assert y.shape == (M, N) and y.is_contiguous()
    xn = x.to(torch.float64).numpy()
    r = oracle.linear_w4a8_ref(xn, oracle.pack_fp4(codes), ws, None if b is None else b.to(torch.float64).numpy())
    return gpu_util.compare(y.float().cpu().numpy(), r, tolerance4(xn, codes, ws, K), label)


@pytest.mark.parametrize("M,N,K", [
    (1, 4096, 4096), (7, 4096, 4096), (9, 4096, 4096), (16, 4096, 4096),   # decode (4-bit kernel)
    (3, 130, 256), (15, 384, 768), (2, 1, 512),                            # ragged N, small K
    (5, 200, 8192), (12, 256, 6144),                                       # four K steps per wave
])
def test_decode_parity(M, N, K):
    run_and_check(M, N, K, seed=M * 7 + N)


@pytest.mark.parametrize("M,N,K", [(300, 640, 512), (129, 200, 1024), (128, 4096, 4096), (17, 130, 256)])
def test_tile_path_parity(M, N, K):
    """The tile path (automatic above M = 128, forced below): the 4-bit tile
    GEMM where the shape table takes one K split, else the weight widened to
    MXFP8 tiles (exact) for the split-K GEMM."""
    run_and_check(M, N, K, seed=M + N, force_path=1 if M <= 128 else 0)


@pytest.mark.parametrize("M,N,K,force", [
    (300, 650, 2048, 17),     # 4-bit tile GEMM: 2 x 3 tiles, ragged last row and column tile
    (300, 650, 2048, 18),     # the widened split-K route on the same shape
    (520, 130, 256, 17),      # K = 256: one 128-K step pair per tile
    (257, 300, 8448, 17),     # K > 8192, 66 steps
])
def test_w4_tile_forced_parity(M, N, K, force):
    run_and_check(M, N, K, seed=M + 5 * N + K, force_path=force)


@pytest.mark.parametrize("M,N,K", [(300, 650, 2048), (520, 130, 256), (257, 300, 8448), (2048, 1536, 4096)])
def test_w4_tile_vs_mxfp8_tile(M, N, K):
    """The 4-bit tile GEMM (E2M1 weight operand) and the MXFP8 tile GEMM fed
    the same weight values as E4M3 bytes, both with one K split.  The scaled
    MFMA does not return the same bits for the two operand formats, so each
    element may differ by the two kernels' error bounds together (each is
    within its bound of the exact product, tests/gpu_util.py)."""
    g = torch.Generator().manual_seed(M + N + K)
    xc = synth.randn_bf16((M, K), 1.0, g)
    x = xc.to(gpu_util.dev())
    w = synth.randn_bf16((N, K), 0.02, g).to(torch.float64).numpy()
    codes, ws = oracle.quantize_mxfp4(w)
    w8 = torch.from_numpy(oracle.e2m1_decode(codes).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    pw8 = api.prepare_weight(w8.to(gpu_util.dev()), torch.from_numpy(ws).to(gpu_util.dev()))
    pw4 = prepare(codes, ws)
    prev = api.mxfp8_debug_force_path(17)
    try:
        assert api.mxfp8_debug_plan(M, N, K) == (0, 1)
        y8 = api.linear(x, pw8).double().cpu().numpy()
        y4 = api.linear(x, pw4).double().cpu().numpy()
    finally:
        api.mxfp8_debug_force_path(prev)
    bound = 2 * (2.0 ** -8 * np.maximum(np.abs(y8), np.abs(y4)) + tolerance4(xc.double().numpy(), codes, ws, K))
    diff = np.abs(y8 - y4)
    print("W4 vs MXFP8 tile", (M, N, K), {"identical": float(np.mean(diff == 0)),
                                         "max_diff_over_bound": float((diff / bound).max())}, flush=True)
    assert np.all(diff <= bound)


def test_one_hot_weight_exact_w4_tile():
    """W[n, perm[n]] = 1 on the 4-bit tile GEMM (M = 300: two M-tiles, the
    second ragged): y[m, n] = bf16(deq(A)[m, perm[n]]) exactly; pins the
    E2M1 weight fragment (nibble order, chunk of each lane group) and the
    weight scale slots of the 4-bit step buffer."""
    g = torch.Generator().manual_seed(71)
    M, K, N = 300, 1024, 300
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=12)
    perm = torch.randint(0, K, (N,), generator=g).numpy()
    w = np.zeros((N, K))
    w[np.arange(N), perm] = 1.0
    codes, ws = oracle.quantize_mxfp4(w)
    pw = prepare(codes, ws)
    prev = api.mxfp8_debug_force_path(17)
    try:
        y = api.linear(x.to(gpu_util.dev()), pw).float().cpu().numpy()
    finally:
        api.mxfp8_debug_force_path(prev)
    qa, sa = oracle.quantize_mx(x.double().numpy())
    exp = oracle.bf16_round(oracle.dequantize_mx(qa, sa)[:, perm])
    assert np.array_equal(y, exp)


@pytest.mark.parametrize("M,N,K", [(17, 130, 256), (40, 384, 768), (128, 4096, 4096), (100, 200, 8192), (5, 256, 512)])
def test_mid_path_parity(M, N, K):
    """16 < M <= 128 streams the 4-bit weight once through the mid-M kernel
    (path 3 forces it at M = 5; K = 8192 gives four steps per wave)."""
    run_and_check(M, N, K, seed=M + 3 * N, force_path=3)


@pytest.mark.parametrize("M,N,K", [(5, 256, 512), (40, 384, 768), (128, 4096, 4096), (9, 1024, 16384),
                                   (100, 200, 10240), (33, 4096, 8192)])
def test_slab_path_parity(M, N, K):
    """The split-K slab kernel with the 4-bit weight (path 5 forces it): 1, 2
    and 4 K steps per wave, 1..8 row groups, K above the decode and mid-M
    kernels' limit."""
    run_and_check(M, N, K, seed=M + 7 * N + K, force_path=5)


@pytest.mark.parametrize("path", [0, 1, 5])
def test_scale_stress_both_paths(path):
    run_and_check(13, 256, 512, seed=31, force_path=path, stress=True)


@pytest.mark.parametrize("M", [5, 40])
def test_one_hot_weight_exact(M):
    """W[n, perm[n]] = 1 (E2M1 code 6 = 4 under scale 2^-2): y[m, n] =
    bf16(deq(A)[m, perm[n]]) exactly.  Pins the 4-bit operand's nibble order,
    lane mapping and the weight scale lookup (M = 5: decode kernel), and the
    4-bit operand of the mid-M kernel (M = 40)."""
    g = torch.Generator().manual_seed(17)
    K, N = 512, 200
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=9)
    perm = torch.randint(0, K, (N,), generator=g).numpy()
    w = np.zeros((N, K))
    w[np.arange(N), perm] = 1.0
    codes, ws = oracle.quantize_mxfp4(w)
    pw = prepare(codes, ws)
    y = api.linear(x.to(gpu_util.dev()), pw).float().cpu().numpy()
    qa, sa = oracle.quantize_mx(x.double().numpy())
    exp = oracle.bf16_round(oracle.dequantize_mx(qa, sa)[:, perm])
    assert np.array_equal(y, exp)


def test_w4a8_matches_mxfp8_on_widened_weight():
    """The GPU W4A8 layer and the GPU MXFP8 layer fed the same weight (E2M1
    values written as E4M3 bytes by torch's cast, same scales) agree bit for
    bit on the split-K tile route (the same MXFP8 GEMM after the exact
    widening of the 4-bit weight)."""
    g = torch.Generator().manual_seed(23)
    M, N, K = 64, 256, 1024
    x = synth.randn_bf16((M, K), 1.0, g).to(gpu_util.dev())
    w = synth.randn_bf16((N, K), 0.02, g).to(torch.float64).numpy()
    codes, ws = oracle.quantize_mxfp4(w)
    w8 = torch.from_numpy(oracle.e2m1_decode(codes).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    pw8 = api.prepare_weight(w8.to(gpu_util.dev()), torch.from_numpy(ws).to(gpu_util.dev()))
    pw4 = prepare(codes, ws)
    prev = api.mxfp8_debug_force_path(18)
    try:
        assert api.mxfp8_debug_plan(M, N, K) == (0, 2)
        y8 = api.linear(x, pw8)
        y4 = api.linear(x, pw4)
        torch.cuda.synchronize()
    finally:
        api.mxfp8_debug_force_path(prev)
    assert torch.equal(y8, y4)


@pytest.mark.parametrize("path", [1, 3, 5])
def test_one_hot_weight_exact_forced(path):
    """The one-hot pin at M = 40 on the widened tile GEMM (path 1), on the
    mid-M kernel's 4-bit operand (path 3) and on the slab kernel's (path 5)."""
    g = torch.Generator().manual_seed(18)
    M, K, N = 40, 1024, 200
    x = synth.scale_stress(synth.randn_bf16((M, K), 1.0, g), seed=10)
    perm = torch.randint(0, K, (N,), generator=g).numpy()
    w = np.zeros((N, K))
    w[np.arange(N), perm] = 1.0
    codes, ws = oracle.quantize_mxfp4(w)
    pw = prepare(codes, ws)
    prev = api.mxfp8_debug_force_path(path)
    try:
        y = api.linear(x.to(gpu_util.dev()), pw).float().cpu().numpy()
    finally:
        api.mxfp8_debug_force_path(prev)
    qa, sa = oracle.quantize_mx(x.double().numpy())
    exp = oracle.bf16_round(oracle.dequantize_mx(qa, sa)[:, perm])
    assert np.array_equal(y, exp)
