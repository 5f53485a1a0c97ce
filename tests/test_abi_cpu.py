"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before touching a device."""

import ctypes
import os
import re

import numpy as np
import pytest

from mxfp8_block_scaled_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")

pytestmark = pytest.mark.skipif(not os.path.exists(api.lib_path()), reason="libmxfp8.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp8_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "mxfp8_linear" in names and "mxfp8_quantize_act" in names
    handle = ctypes.CDLL(api.lib_path())
    for n in names:
        assert hasattr(handle, n), n


def test_status_strings():
    for s in range(0, -9, -1):
        assert api.mxfp8_status_string(s) != "unknown status"
    assert api.mxfp8_status_string(-99) == "unknown status"


def test_prepared_weight_bytes():
    assert api.mxfp8_prepared_weight_bytes(130, 256) == (256 * 256, 256 * 8)
    assert api.mxfp8_prepared_weight_bytes(4096, 4096) == (4096 * 4096, 4096 * 128)
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_prepared_weight_bytes(130, 224)
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_prepared_weight_bytes(0, 256)


P = 0x10000  # a fake, 256-byte aligned "device" address; never dereferenced


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


GPU_VISIBLE = _gpu_visible()


def expect_no_device(fn, *args):
    """A call whose arguments are all valid: without a gfx950 the library
    answers MXFP8_E_DEVICE before launching anything.  Where a GPU is visible
    the call would launch kernels on the fake address P, so it is not made;
    the rejection cases around it return before any device call either way."""
    if GPU_VISIBLE:
        return
    assert fn(*args) == -6


def test_quantize_validation():
    f = api.mxfp8_quantize_act
    assert f(P, 4, 48, 48, P, 48, P, 2, None) == -2         # K % 32
    assert f(P, -1, 64, 64, P, 64, P, 2, None) == -2        # M < 0
    assert f(P, 0, 64, 64, P, 64, P, 2, None) == 0          # empty: no-op
    assert f(None, 4, 64, 64, P, 64, P, 2, None) == -1
    assert f(P, 4, 64, 32, P, 64, P, 2, None) == -4         # ldx < K
    assert f(P, 4, 64, 68, P, 64, P, 2, None) == -4         # ldx % 8
    assert f(P, 4, 64, 64, P, 64, P, 1, None) == -4         # lds < K/32
    assert f(P + 8, 4, 64, 64, P, 64, P, 2, None) == -3     # x alignment
    expect_no_device(f, P, 4, 64, 64, P, 64, P, 2, None)         # valid, but no gfx950 device here


def test_prepare_validation():
    f = api.mxfp8_prepare_weight
    assert f(P, P, 130, 224, 224, 7, P, P, None) == -2      # K % 256
    assert f(P, P, 0, 256, 256, 8, P, P, None) == -2
    assert f(None, P, 130, 256, 256, 8, P, P, None) == -1
    assert f(P, P, 130, 256, 256, 8, None, P, None) == -1
    assert f(P, P, 130, 256, 255, 8, P, P, None) == -4
    assert f(P, P, 130, 256, 256, 7, P, P, None) == -4
    assert f(P, P, 130, 256, 256, 8, P + 16, P, None) == -3
    expect_no_device(f, P, P, 130, 256, 256, 8, P, P, None)


def test_linear_validation():
    f = api.mxfp8_linear
    ws = api.mxfp8_linear_workspace_bytes(512, 130, 256)
    assert ws >= 512 * 256 + 512 * 8
    ok = (P, 512, 256, 256, P, P, 130, None, P, 130, P, ws, None)
    expect_no_device(f, *ok)
    bad = list(ok); bad[2] = 320; assert f(*bad) == -2          # K % 256
    bad = list(ok); bad[6] = 0; assert f(*bad) == -2            # N < 1
    bad = list(ok); bad[1] = -3; assert f(*bad) == -2
    bad = list(ok); bad[1] = 0; assert f(*bad) == 0             # M == 0 no-op
    bad = list(ok); bad[0] = None; assert f(*bad) == -1
    bad = list(ok); bad[8] = None; assert f(*bad) == -1
    bad = list(ok); bad[9] = 129; assert f(*bad) == -4          # ldy < N
    bad = list(ok); bad[3] = 200; assert f(*bad) == -4          # ldx < K
    bad = list(ok); bad[10] = None; assert f(*bad) == -5
    bad = list(ok); bad[11] = ws - 1; assert f(*bad) == -5
    bad = list(ok); bad[4] = P + 64; assert f(*bad) == -3       # packed weight alignment
    bad = list(ok); bad[0] = P + 2; assert f(*bad) == -3


def _round_up(v, a):
    return (v + a - 1) // a * a


def _expected_ws(M, N, K):
    """Workspace of the plan the library reports: nothing stored on the decode
    path; one 128-row group of packed activations (E4M3 tiles, then scale
    tiles) on the mid-M path; the tile path's padded packed activations, then
    the fp32 partials of its K splits."""
    path, s = api.mxfp8_debug_plan(M, N, K)
    if path == 1:
        return 256
    if path == 2:
        return 128 * K + 128 * (K // 32)
    if path == 3:
        # the slab kernel's fp32 partials: one [M, N_pad] per K slice; a slice
        # is 2 spw 128-K steps, spw the largest of 4, 2 that still leaves
        # >= 256 workgroups (N_pad / 128 per slice), else 1
        G, KS = (N + 127) // 128, K // 128
        spw = next((v for v in (4, 2) if KS % (2 * v) == 0 and G * (KS // (2 * v)) >= 256), 1)
        return _round_up((KS // (2 * spw)) * M * G * 128 * 4, 256)
    mp = (M + 127) // 128 * 128
    act = _round_up(mp * K, 256) + _round_up(mp * (K // 32), 256)
    if path in (4, 5):   # the medium-tile GEMM: the packed activations only
        return act
    part = s * M * ((N + 3) // 4 * 4) * 4 if s > 1 else 0
    return act + _round_up(part, 256)


def test_linear_paths_workspace():
    """Workspace per planned path; K > 8192 always takes the tile path; the
    forced paths move shapes between paths and split counts."""
    ws = api.mxfp8_linear_workspace_bytes
    for M, N, K in [(1, 4096, 4096), (16, 4096, 4096), (17, 4096, 4096), (128, 4096, 4096), (129, 4096, 4096),
                    (8, 4096, 8448), (300, 700, 2048), (4096, 4096, 1024), (64, 256, 512)]:
        assert ws(M, N, K) == _expected_ws(M, N, K), (M, N, K)
    assert api.mxfp8_debug_plan(8, 4096, 8448)[0] in (0, 3)         # K > 8192: tile or slab
    prev = api.mxfp8_debug_force_path(1)
    try:
        assert api.mxfp8_debug_plan(64, 4096, 4096)[0] == 0
        assert ws(64, 4096, 4096) == _expected_ws(64, 4096, 4096) >= 128 * 4096 + 128 * 128
        api.mxfp8_debug_force_path(3)
        assert api.mxfp8_debug_plan(8, 4096, 4096) == (2, 1)
        assert ws(8, 4096, 4096) == 128 * 4096 + 128 * 128           # mid path forced at M = 8
        assert api.mxfp8_debug_plan(200, 4096, 4096)[0] == 0        # above 128: the tile path
        api.mxfp8_debug_force_path(4)
        assert api.mxfp8_debug_plan(16, 4096, 4096) == (1, 1)
        assert ws(16, 4096, 4096) == 256
        assert api.mxfp8_debug_plan(17, 4096, 4096)[0] != 1         # decode kernel only to M = 16
        api.mxfp8_debug_force_path(5)
        for M, N, K in [(1, 256, 256), (128, 4096, 4096), (33, 4096, 8192), (100, 384, 8192), (113, 200, 6144)]:
            assert api.mxfp8_debug_plan(M, N, K) == (3, 1), (M, N, K)
            assert ws(M, N, K) == _expected_ws(M, N, K), (M, N, K)
        assert ws(128, 4096, 4096) == 8 * 128 * 4096 * 4              # 8 slices of 512 K
        assert ws(33, 4096, 8192) == 8 * 33 * 4096 * 4                # 8 slices of 1024 K
        assert api.mxfp8_debug_plan(129, 4096, 4096)[0] == 0        # above 128: the tile path
        assert api.mxfp8_debug_plan(64, 4096, 8448) == (3, 1)        # any K
        assert ws(64, 4096, 8448) == _expected_ws(64, 4096, 8448)
        for sp in (1, 2, 4, 8):
            api.mxfp8_debug_force_path(16 + sp)
            assert api.mxfp8_debug_plan(300, 700, 2048) == (0, sp)   # K / 64 = 32 takes every split count
            assert ws(300, 700, 2048) == _expected_ws(300, 700, 2048)
        api.mxfp8_debug_force_path(24)
        assert api.mxfp8_debug_plan(300, 700, 1280) == (0, 1)       # 20 steps: 8 slices do not divide
        api.mxfp8_debug_force_path(6)
        assert api.mxfp8_debug_plan(1024, 4096, 4096) == (4, 1)
        assert ws(1024, 4096, 4096) == _expected_ws(1024, 4096, 4096) == 1024 * 4096 + 1024 * 128
        api.mxfp8_debug_force_path(7)
        assert api.mxfp8_debug_plan(300, 700, 2048) == (5, 1)
        assert ws(300, 700, 2048) == _expected_ws(300, 700, 2048)
        for bad in (-1, 8, 16, 19, 25, 40):
            assert api.mxfp8_debug_force_path(bad) == -2
    finally:
        api.mxfp8_debug_force_path(prev)
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_debug_plan(0, 256, 512)
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_debug_plan(4, 256, 500)
    f = api.mxfp8_linear
    need = ws(64, 256, 512)
    ok = (P, 64, 512, 512, P, P, 256, None, P, 256, P, need, None)
    expect_no_device(f, *ok)                                           # valid, but no gfx950 device here
    bad = list(ok); bad[11] = need - 1; assert f(*bad) == -5
    bad = list(ok); bad[10] = P + 128; assert f(*bad) == -3       # workspace 256-byte alignment
    g = api.mxfp8_linear_w4a8
    if api.mxfp8_debug_plan(64, 256, 512)[0] != 0:
        # decode, mid-M and slab kernels have 4-bit forms with the same workspace
        assert api.mxfp8_linear_w4a8_workspace_bytes(64, 256, 512) == need
    expect_no_device(g, *ok)


def _shape_table():
    """The compiled-in shape table, parsed from its source."""
    import re
    text = open(os.path.join(ROOT, "mxfp8_block_scaled_amd", "csrc", "shape_table.inc")).read()
    bounds = {}
    for ax in "MNK":
        m = re.search(r"kShapeTab%s\[kShapeTabN%s\] = \{([^}]*)\}" % (ax, ax), text)
        bounds[ax] = [int(v) for v in m.group(1).split(",")]
    def arr(name):
        m = re.search(name + r"\[kShapeTabNM\]\[kShapeTabNN\]\[kShapeTabNK\] = (\{.*?\n\});", text, re.S)
        vals = [int(v) for v in re.findall(r"\d+", m.group(1))]
        nm, nn, nk = (len(bounds[a]) for a in "MNK")
        assert len(vals) == nm * nn * nk
        return [[[vals[(i * nn + j) * nk + k] for k in range(nk)] for j in range(nn)] for i in range(nm)]
    return bounds, arr("kShapeTabPlan"), arr("kShapeTabTileSplits")


def test_shape_table_well_formed_and_dispatched():
    """Every table entry names a path and a split count; the library's plan
    is the table's entry for the shape's bucket, limited by what each kernel
    takes (decode M <= 16 and mid-M M <= 128, both K <= 8192; the slab
    kernel M <= 128; s splits need (K/64) % (4s) == 0), checked over random
    shapes."""
    bounds, plan, tsplit = _shape_table()
    for ax in "MNK":
        assert bounds[ax] == sorted(bounds[ax]) and len(set(bounds[ax])) == len(bounds[ax])
    for i, row in enumerate(plan):
        for j, col in enumerate(row):
            for k, code in enumerate(col):
                assert code >> 4 in (0, 1, 2, 3, 4, 5) and (code & 15) in (1, 2, 4, 8)
                assert tsplit[i][j][k] in (1, 2, 4, 8)

    def bucket(ax, v):
        for i, b in enumerate(bounds[ax]):
            if v <= b:
                return i
        return len(bounds[ax]) - 1

    rng = np.random.default_rng(7)
    for _ in range(3000):
        M = int(rng.choice([rng.integers(1, 300), rng.integers(1, 20000)]))
        N = int(rng.integers(1, 40000))
        K = int(rng.integers(1, 80)) * 256
        i, j, k = bucket("M", M), bucket("N", N), bucket("K", K)
        path, s = plan[i][j][k] >> 4, tsplit[i][j][k]
        if path == 1 and not (M <= 16 and K <= 8192):
            path = 0
        if path == 2 and not (M <= 128 and K <= 8192):
            path = 0
        if path == 3 and M > 128:
            path = 0
        if s != 1 and (K // 64) % (4 * s) != 0:
            s = 1
        assert api.mxfp8_debug_plan(M, N, K) == (path, s if path == 0 else 1), (M, N, K)


def test_packed_entries_validation():
    assert api.mxfp8_packed_act_bytes(300, 512) == (384 * 512, 384 * 16)
    f = api.mxfp8_quantize_act_packed
    expect_no_device(f, P, 4, 512, 512, P, P, None)
    assert f(P, 4, 288, 288, P, P, None) == -2               # K % 256
    assert f(P, 4, 512, 500, P, P, None) == -4
    assert f(P, 4, 512, 512, P + 16, P, None) == -3          # packed output alignment
    assert f(P, 0, 512, 512, P, P, None) == 0
    g = api.mxfp8_gemm_packed
    ok = (P, P, 64, 256, P, P, 130, None, P, 130, None)
    expect_no_device(g, *ok)
    bad = list(ok); bad[0] = None; assert g(*bad) == -1
    bad = list(ok); bad[1] = P + 4; assert g(*bad) == -3
    bad = list(ok); bad[9] = 100; assert g(*bad) == -4
    bad = list(ok); bad[3] = 320; assert g(*bad) == -2


def test_force_path_hook():
    prev = api.mxfp8_debug_force_path(1)
    assert api.mxfp8_debug_force_path(prev) == 1
    assert api.mxfp8_debug_force_path(9) == -2                        # unknown: refused, nothing changed
    assert api.mxfp8_debug_force_path(prev) == prev


def test_moe_sizes():
    E, H, I = 128, 2048, 768
    assert api.mxfp8_moe_prepared_bytes(E, H, I) == (E * 2 * I * H, E * 2 * I * H // 32, E * H * I, E * H * I // 32)
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_moe_prepared_bytes(E, H, 640)        # I % 256
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_moe_prepared_bytes(257, H, I)        # too many experts
    T, k = 4096, 8
    ws = api.mxfp8_moe_workspace_bytes(T, H, I, E, k)
    # at least the tokens quantized once, the expert-sorted scales and operand of
    # the down projection, and the fp32 routing-weighted expert output rows
    rows = T * k
    assert ws >= T * (H + H // 32) + rows * (H // 32 + I + I // 32 + 4 * H)
    assert api.mxfp8_moe_workspace_bytes(0, H, I, E, k) > 0
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_moe_workspace_bytes(T, H, I, E, 17)  # top-k above 16
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_moe_workspace_bytes(T, H, I, 4, 8)   # top-k above E


def test_moe_validation():
    T, H, E, k, I = 64, 256, 8, 2, 256
    ws = api.mxfp8_moe_workspace_bytes(T, H, I, E, k)
    f = api.mxfp8_moe_grouped
    ok = [P, P, T, H, E, k, I, P, P, P, P, P, P, ws, None]
    expect_no_device(f, *ok)                                # valid, but no gfx950 device here
    bad = list(ok); bad[2] = 0; assert f(*bad) == 0    # T == 0 no-op
    bad = list(ok); bad[3] = 320; assert f(*bad) == -2
    bad = list(ok); bad[6] = 128; assert f(*bad) == -2
    bad = list(ok); bad[5] = 0; assert f(*bad) == -2
    bad = list(ok); bad[0] = None; assert f(*bad) == -1
    bad = list(ok); bad[1] = None; assert f(*bad) == -1
    bad = list(ok); bad[11] = None; assert f(*bad) == -1
    bad = list(ok); bad[0] = P + 8; assert f(*bad) == -3
    bad = list(ok); bad[7] = P + 16; assert f(*bad) == -3
    bad = list(ok); bad[12] = None; assert f(*bad) == -5
    bad = list(ok); bad[13] = ws - 1; assert f(*bad) == -5
    bad = list(ok); bad[12] = P + 128; assert f(*bad) == -3
    g = api.mxfp8_moe_prepare_weights
    okp = [P, P, P, P, E, H, I, P, P, P, P, None]
    expect_no_device(g, *okp)
    bad = list(okp); bad[6] = 300; assert g(*bad) == -2
    bad = list(okp); bad[2] = None; assert g(*bad) == -1
    bad = list(okp); bad[8] = P + 4; assert g(*bad) == -3


def test_moe_debug_hook():
    assert api.mxfp8_moe_debug_capture(P, None, None, None, None) == -1
    assert api.mxfp8_moe_debug_capture(P, P, P, P, None) == -1
    assert api.mxfp8_moe_debug_capture(P + 2, P, P, P, P) == -3
    assert api.mxfp8_moe_debug_capture(P, P, P, P, P) == 0
    assert api.mxfp8_moe_debug_capture(None, None, None, None, None) == 0


def test_w4a8_sizes_and_validation():
    assert api.mxfp8_prepared_weight_fp4_bytes(130, 256) == (256 * 128, 256 * 8)
    assert api.mxfp8_prepared_weight_fp4_bytes(4096, 4096) == (4096 * 2048, 4096 * 128)
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_prepared_weight_fp4_bytes(130, 384)
    # workspace: decode and mid-M shapes as the MXFP8 layer; on the tile path
    # the 4-bit GEMM (one K split) needs nothing more, the split-K route adds
    # the weight widened to MXFP8 tiles (N padded to 128 rows x K bytes)
    assert api.mxfp8_linear_w4a8_workspace_bytes(7, 4096, 4096) == api.mxfp8_linear_workspace_bytes(7, 4096, 4096)
    assert api.mxfp8_linear_w4a8_workspace_bytes(16, 4096, 4096) == api.mxfp8_linear_workspace_bytes(16, 4096, 4096)
    assert api.mxfp8_linear_workspace_bytes(16, 4096, 8192) == _expected_ws(16, 4096, 8192)
    bounds, _, tsplit = _shape_table()

    def bucket(ax, v):
        return next((i for i, b in enumerate(bounds[ax]) if v <= b), len(bounds[ax]) - 1)

    for M, N, K in [(512, 130, 256), (300, 700, 2048), (4096, 4096, 4096), (256, 4096, 4096)]:
        path, sp = api.mxfp8_debug_plan(M, N, K)
        if path in (4, 5):
            # no 4-bit medium-tile GEMM: the tile path with the table's K splits
            sp = tsplit[bucket("M", M)][bucket("N", N)][bucket("K", K)]
            sp = sp if (K // 64) % (4 * sp) == 0 else 1
            mp = (M + 127) // 128 * 128
            act = _round_up(mp * K, 256) + _round_up(mp * (K // 32), 256)
            tile = act + (_round_up(sp * M * ((N + 3) // 4 * 4) * 4, 256) if sp > 1 else 0)
            extra = (N + 127) // 128 * 128 * K if sp > 1 else 0
            assert api.mxfp8_linear_w4a8_workspace_bytes(M, N, K) == tile + extra, (M, N, K)
            continue
        extra = (N + 127) // 128 * 128 * K if path == 0 and sp > 1 else 0
        assert api.mxfp8_linear_w4a8_workspace_bytes(M, N, K) == api.mxfp8_linear_workspace_bytes(M, N, K) + extra
    prev = api.mxfp8_debug_force_path(18)          # tile GEMM, 2 K splits: the widened route
    try:
        assert (api.mxfp8_linear_w4a8_workspace_bytes(300, 700, 2048)
                == api.mxfp8_linear_workspace_bytes(300, 700, 2048) + 768 * 2048)
        api.mxfp8_debug_force_path(17)             # one split: the 4-bit tile GEMM
        assert api.mxfp8_linear_w4a8_workspace_bytes(300, 700, 2048) == api.mxfp8_linear_workspace_bytes(300, 700, 2048)
    finally:
        api.mxfp8_debug_force_path(prev)
    p = api.mxfp8_prepare_weight_fp4
    expect_no_device(p, P, P, 130, 256, 128, 8, P, P, None)       # valid (ldw = K/2), no device
    assert p(P, P, 130, 224, 112, 7, P, P, None) == -2       # K % 256
    assert p(P, P, 130, 256, 112, 8, P, P, None) == -4       # ldw < K/2
    assert p(P, P, 130, 256, 136, 8, P, P, None) == -4       # ldw % 16
    assert p(P + 8, P, 130, 256, 128, 8, P, P, None) == -3
    assert p(None, P, 130, 256, 128, 8, P, P, None) == -1
    f = api.mxfp8_linear_w4a8
    ws = api.mxfp8_linear_w4a8_workspace_bytes(512, 130, 256)
    ok = (P, 512, 256, 256, P, P, 130, None, P, 130, P, ws, None)
    expect_no_device(f, *ok)
    bad = list(ok); bad[11] = ws - 1; assert f(*bad) == -5   # workspace too small
    bad = list(ok); bad[2] = 320; assert f(*bad) == -2
    bad = list(ok); bad[1] = 0; assert f(*bad) == 0
    bad = list(ok); bad[4] = P + 64; assert f(*bad) == -3
    bad = list(ok); bad[9] = 100; assert f(*bad) == -4


def test_quantize_fp4_validation():
    f = api.mxfp8_quantize_fp4
    expect_no_device(f, P, 4, 64, 64, P, 32, P, 2, None)          # valid, no device
    assert f(P, 4, 48, 48, P, 24, P, 2, None) == -2          # K % 32
    assert f(P, 0, 64, 64, P, 32, P, 2, None) == 0
    assert f(P, 4, 64, 64, P, 30, P, 2, None) == -4          # ldq < K/2
    assert f(P, 4, 64, 64, P, 34, P, 2, None) == -4          # ldq % 4
    assert f(P, 4, 64, 64, P + 2, 32, P, 2, None) == -3      # q alignment
    assert f(None, 4, 64, 64, P, 32, P, 2, None) == -1


def test_noalloc_validation():
    """mxfp8_linear_noalloc: mxfp8_linear's checks, then the static scratch
    limit (MXFP8_E_SCRATCH), all before any device call."""
    f = api.mxfp8_linear_noalloc
    ok = (P, 64, 512, 512, P, P, 256, None, P, 256, None)
    expect_no_device(f, *ok)
    bad = list(ok); bad[2] = 320; assert f(*bad) == -2          # K % 256
    bad = list(ok); bad[1] = 0; assert f(*bad) == 0             # M == 0 no-op
    bad = list(ok); bad[0] = None; assert f(*bad) == -1
    bad = list(ok); bad[9] = 100; assert f(*bad) == -4          # ldy < N
    bad = list(ok); bad[4] = P + 64; assert f(*bad) == -3
    assert api.mxfp8_linear_workspace_bytes(16384, 5120, 2048) > api.NOALLOC_SCRATCH_BYTES
    assert f(P, 16384, 2048, 2048, P, P, 5120, None, P, 5120, None) == -8
    assert api.mxfp8_linear_workspace_bytes(128, 4096, 8192) <= api.NOALLOC_SCRATCH_BYTES


def test_calibration_library_exports_and_rejects():
    """The benchmark's calibration library (read stream, scaled-MFMA loop)
    loads, exports its two entry points and rejects invalid arguments before
    any launch."""
    path = os.path.join(os.path.dirname(api.lib_path()), "libmxfp8_calib.so")
    if not os.path.exists(path):
        pytest.skip("libmxfp8_calib.so not built")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.mxfp8_calib_read.argtypes = [vp, ctypes.c_uint64, ctypes.c_int, vp, vp]
    lib.mxfp8_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    assert lib.mxfp8_calib_read(None, 1 << 20, 64, P, None) == -2
    assert lib.mxfp8_calib_read(P, (1 << 20) + 16, 64, P, None) == -2       # not 16 * blocks divisible
    assert lib.mxfp8_calib_read(P + 8, 1 << 20, 64, P, None) == -2          # alignment
    assert lib.mxfp8_calib_mfma(0, 10, P, None) == -2
    assert lib.mxfp8_calib_mfma(4, 10, None, None) == -2


def test_gemm_prequant_validation():
    """mxfp8_gemm_prequant (the GEMM given row-major quantized activations):
    sizes and argument checks, all before any device call."""
    ws = api.mxfp8_gemm_prequant_workspace_bytes(300, 130, 512)
    assert ws >= 384 * 512 + 384 * 16
    assert api.mxfp8_gemm_prequant_workspace_bytes(0, 130, 512) == 256
    with pytest.raises(api.MXFP8Error):
        api.mxfp8_gemm_prequant_workspace_bytes(300, 130, 500)
    f = api.mxfp8_gemm_prequant
    ok = (P, 512, P, 16, 300, 512, P, P, 130, None, P, 130, P, ws, None)
    expect_no_device(f, *ok)
    bad = list(ok); bad[4] = 0; assert f(*bad) == 0              # M == 0 no-op
    bad = list(ok); bad[5] = 320; assert f(*bad) == -2           # K % 256
    bad = list(ok); bad[0] = None; assert f(*bad) == -1
    bad = list(ok); bad[1] = 500; assert f(*bad) == -4           # ldq < K
    bad = list(ok); bad[1] = 520; assert f(*bad) == -4           # ldq % 16
    bad = list(ok); bad[3] = 15; assert f(*bad) == -4            # lds < K/32
    bad = list(ok); bad[0] = P + 8; assert f(*bad) == -3         # q alignment
    bad = list(ok); bad[13] = ws - 1; assert f(*bad) == -5
    bad = list(ok); bad[11] = 100; assert f(*bad) == -4          # ldy < N
