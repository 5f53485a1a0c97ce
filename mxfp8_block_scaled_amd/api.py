"""Thin Python binding over libmxfp8.so (ctypes).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the layer runs in the library's HIP kernels.  If the
library has not been built, the first call raises ``MXFP8Error``; there is no
fallback.

Names mirror the C ABI (include/mxfp8.h): ``mxfp8_quantize_act``,
``mxfp8_prepare_weight``, ``mxfp8_linear``, ... take raw pointers and sizes;
``quantize_act``, ``prepare_weight`` and ``linear`` are the tensor-level
wrappers (the apply path of vLLM PR #52204: assert bf16, view the input as
``[-1, K]``, run the layer, restore the leading dims).
"""

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp8.so")
_lib = None
_lock = threading.Lock()

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

_SIGNATURES = {
    "mxfp8_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "mxfp8_quantize_act": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp], ctypes.c_int),
    "mxfp8_prepared_weight_bytes": ([_i64, _i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_prepare_weight": ([_vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mxfp8_unpack_weight": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mxfp8_linear_workspace_bytes": ([_i64, _i64, _i64, ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_linear": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _sz, _vp], ctypes.c_int),
    "mxfp8_packed_act_bytes": ([_i64, _i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_quantize_act_packed": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mxfp8_gemm_packed": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp], ctypes.c_int),
    "mxfp8_debug_force_path": ([ctypes.c_int], ctypes.c_int),
    "mxfp8_debug_plan": ([_i64, _i64, _i64, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "mxfp8_moe_prepared_bytes": ([_i64, _i64, _i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                  ctypes.POINTER(_sz), ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_moe_prepare_weights": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mxfp8_moe_workspace_bytes": ([_i64, _i64, _i64, _i64, _i64, ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_moe_grouped": ([_vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                          ctypes.c_int),
    "mxfp8_moe_debug_capture": ([_vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mxfp8_quantize_fp4": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp], ctypes.c_int),
    "mxfp8_prepared_weight_fp4_bytes": ([_i64, _i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_prepare_weight_fp4": ([_vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mxfp8_unpack_weight_fp4": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mxfp8_linear_w4a8_workspace_bytes": ([_i64, _i64, _i64, ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_linear_w4a8": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _sz, _vp], ctypes.c_int),
    "mxfp8_linear_noalloc": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp], ctypes.c_int),
    "mxfp8_gemm_prequant_workspace_bytes": ([_i64, _i64, _i64, ctypes.POINTER(_sz)], ctypes.c_int),
    "mxfp8_gemm_prequant": ([_vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _sz, _vp],
                            ctypes.c_int),
}

# Static scratch of mxfp8_linear_noalloc (bytes; MXFP8_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024


class MXFP8Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().mxfp8_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


def lib_path():
    return _LIB_PATH


def lib():
    """Load libmxfp8.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise RuntimeError(
                        f"libmxfp8.so not built at {_LIB_PATH}; run "
                        "`python -m mxfp8_block_scaled_amd.build` (hipcc, gfx950)")
                handle = ctypes.CDLL(_LIB_PATH)
                for name, (args, res) in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.argtypes = args
                    fn.restype = res
                _lib = handle
    return _lib


def _check(status, where):
    if status != 0:
        raise MXFP8Error(status, where)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# Raw C-ABI mirrors (pointers are ints or None; stream is an int handle)
# ---------------------------------------------------------------------------

def mxfp8_status_string(status):
    return lib().mxfp8_status_string(status).decode()


def mxfp8_quantize_act(x, M, K, ldx, q, ldq, s, lds, stream):
    return lib().mxfp8_quantize_act(x, M, K, ldx, q, ldq, s, lds, stream)


def mxfp8_prepared_weight_bytes(N, K):
    w, s = _sz(), _sz()
    _check(lib().mxfp8_prepared_weight_bytes(N, K, ctypes.byref(w), ctypes.byref(s)),
           "mxfp8_prepared_weight_bytes")
    return w.value, s.value


def mxfp8_prepare_weight(w, ws, N, K, ldw, ldws, wp, sp, stream):
    return lib().mxfp8_prepare_weight(w, ws, N, K, ldw, ldws, wp, sp, stream)


def mxfp8_unpack_weight(wp, sp, N, K, w, ws, stream):
    return lib().mxfp8_unpack_weight(wp, sp, N, K, w, ws, stream)


def mxfp8_linear_workspace_bytes(M, N, K):
    b = _sz()
    _check(lib().mxfp8_linear_workspace_bytes(M, N, K, ctypes.byref(b)), "mxfp8_linear_workspace_bytes")
    return b.value


def mxfp8_linear(x, M, K, ldx, wp, sp, N, bias, y, ldy, ws, ws_bytes, stream):
    return lib().mxfp8_linear(x, M, K, ldx, wp, sp, N, bias, y, ldy, ws, ws_bytes, stream)


def mxfp8_linear_noalloc(x, M, K, ldx, wp, sp, N, bias, y, ldy, stream):
    return lib().mxfp8_linear_noalloc(x, M, K, ldx, wp, sp, N, bias, y, ldy, stream)


def mxfp8_quantize_fp4(x, M, K, ldx, q, ldq, s, lds, stream):
    return lib().mxfp8_quantize_fp4(x, M, K, ldx, q, ldq, s, lds, stream)


def quantize_fp4(x):
    """bf16 ``[M, K]`` (GPU) -> (uint8 ``[M, K/2]`` packed E2M1, uint8 ``[M, K/32]``
    UE8M0), the MX rule with E2M1 elements."""
    assert x.dtype == torch.bfloat16
    _require_cuda(x, "x")
    if x.stride(-1) != 1 or x.stride(0) % 8 != 0 or x.data_ptr() % 16 != 0:
        x = x.contiguous()
    M, K = x.shape
    q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(mxfp8_quantize_fp4(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(s), s.stride(0),
                              _stream(x.device)), "mxfp8_quantize_fp4")
    return q, s


def mxfp8_prepared_weight_fp4_bytes(N, K):
    w, s = _sz(), _sz()
    _check(lib().mxfp8_prepared_weight_fp4_bytes(N, K, ctypes.byref(w), ctypes.byref(s)),
           "mxfp8_prepared_weight_fp4_bytes")
    return w.value, s.value


def mxfp8_prepare_weight_fp4(w, ws, N, K, ldw, ldws, wp, sp, stream):
    return lib().mxfp8_prepare_weight_fp4(w, ws, N, K, ldw, ldws, wp, sp, stream)


def mxfp8_unpack_weight_fp4(wp, sp, N, K, w, ws, stream):
    return lib().mxfp8_unpack_weight_fp4(wp, sp, N, K, w, ws, stream)


def mxfp8_linear_w4a8_workspace_bytes(M, N, K):
    b = _sz()
    _check(lib().mxfp8_linear_w4a8_workspace_bytes(M, N, K, ctypes.byref(b)), "mxfp8_linear_w4a8_workspace_bytes")
    return b.value


def mxfp8_linear_w4a8(x, M, K, ldx, wp, sp, N, bias, y, ldy, ws, ws_bytes, stream):
    return lib().mxfp8_linear_w4a8(x, M, K, ldx, wp, sp, N, bias, y, ldy, ws, ws_bytes, stream)


def mxfp8_packed_act_bytes(M, K):
    q, s = _sz(), _sz()
    _check(lib().mxfp8_packed_act_bytes(M, K, ctypes.byref(q), ctypes.byref(s)), "mxfp8_packed_act_bytes")
    return q.value, s.value


def mxfp8_quantize_act_packed(x, M, K, ldx, qp, sp, stream):
    return lib().mxfp8_quantize_act_packed(x, M, K, ldx, qp, sp, stream)


def mxfp8_gemm_packed(qp, sp, M, K, wp, wsp, N, bias, y, ldy, stream):
    return lib().mxfp8_gemm_packed(qp, sp, M, K, wp, wsp, N, bias, y, ldy, stream)


def mxfp8_gemm_prequant_workspace_bytes(M, N, K):
    b = _sz()
    _check(lib().mxfp8_gemm_prequant_workspace_bytes(M, N, K, ctypes.byref(b)), "mxfp8_gemm_prequant_workspace_bytes")
    return b.value


def mxfp8_gemm_prequant(q, ldq, s, lds, M, K, wp, wsp, N, bias, y, ldy, ws, ws_bytes, stream):
    return lib().mxfp8_gemm_prequant(q, ldq, s, lds, M, K, wp, wsp, N, bias, y, ldy, ws, ws_bytes, stream)


def gemm_prequant(q, s, pw, bias=None):
    """The block-scaled GEMM + epilogue on row-major quantized activations
    (uint8 E4M3 ``q[M, K]``, UE8M0 ``s[M, >= K/32]``, GPU): bf16 ``[M, N]``."""
    q = _as_bytes(q)
    s = _as_bytes(s)
    _require_cuda(q, "q")
    if q.stride(-1) != 1 or q.stride(0) % 16 != 0 or q.data_ptr() % 16 != 0:
        q = q.contiguous()
    if s.stride(-1) != 1:
        s = s.contiguous()
    M, K = q.shape
    assert K == pw.K
    y = torch.empty((M, pw.N), dtype=torch.bfloat16, device=q.device)
    ws = torch.empty(mxfp8_gemm_prequant_workspace_bytes(M, pw.N, K), dtype=torch.uint8, device=q.device)
    _check(mxfp8_gemm_prequant(_ptr(q), q.stride(0), _ptr(s), s.stride(0), M, K, _ptr(pw.w_packed), _ptr(pw.s_packed),
                               pw.N, _ptr(bias), _ptr(y), y.stride(0), _ptr(ws), ws.numel(), _stream(q.device)),
           "mxfp8_gemm_prequant")
    return y


def mxfp8_debug_force_path(path):
    return lib().mxfp8_debug_force_path(path)


def mxfp8_debug_plan(M, N, K):
    """(path, splits) mxfp8_linear takes for M x N x K: path 0 = large-tile
    GEMM, 1 = decode kernel, 2 = mid-M kernel."""
    p, sp = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().mxfp8_debug_plan(M, N, K, ctypes.byref(p), ctypes.byref(sp)), "mxfp8_debug_plan")
    return p.value, sp.value


# ---------------------------------------------------------------------------
# Tensor-level API
# ---------------------------------------------------------------------------

def _require_cuda(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def quantize_act(x):
    """bf16 ``x[M, K]`` (GPU) -> (E4M3 bytes uint8 ``[M, K]``, UE8M0 bytes uint8 ``[M, K/32]``)."""
    assert x.dtype == torch.bfloat16, f"MXFP8 quantization takes bfloat16, got {x.dtype}"
    _require_cuda(x, "x")
    x2 = x.reshape(-1, x.shape[-1])
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()
    M, K = x2.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(mxfp8_quantize_act(_ptr(x2), M, K, x2.stride(0), _ptr(q), K, _ptr(s), K // 32,
                              _stream(x.device)), "mxfp8_quantize_act")
    return q, s


class PreparedWeight:
    """An MXFP8 weight after the one-time preparation: packed payload and
    scales (opaque layout, N padded to 128) plus the logical output size."""

    def __init__(self, w_packed, s_packed, N, K):
        self.w_packed = w_packed
        self.s_packed = s_packed
        self.N = N
        self.K = K

    @property
    def device(self):
        return self.w_packed.device

    def unpack(self):
        """(E4M3 ``[N_pad, K]``, UE8M0 ``[N_pad, K/32]``) as uint8 tensors."""
        n_pad = (self.N + 127) // 128 * 128
        w = torch.empty((n_pad, self.K), dtype=torch.uint8, device=self.device)
        s = torch.empty((n_pad, self.K // 32), dtype=torch.uint8, device=self.device)
        _check(mxfp8_unpack_weight(_ptr(self.w_packed), _ptr(self.s_packed), self.N, self.K, _ptr(w), _ptr(s),
                                   _stream(self.device)), "mxfp8_unpack_weight")
        return w, s


def _as_bytes(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def prepare_weight(w_q, w_s):
    """MXFP8 weight ``w_q`` E4M3 ``[N, K]`` (uint8 or float8_e4m3fn) with UE8M0
    scales ``w_s`` ``[>= N, >= K/32]`` (uint8) -> PreparedWeight."""
    w_q = _as_bytes(w_q)
    w_s = _as_bytes(w_s)
    _require_cuda(w_q, "w_q")
    N, K = w_q.shape
    if w_q.stride(-1) != 1:
        w_q = w_q.contiguous()
    if w_s.stride(-1) != 1:
        w_s = w_s.contiguous()
    wb, sb = mxfp8_prepared_weight_bytes(N, K)
    wp = torch.empty(wb, dtype=torch.uint8, device=w_q.device)
    sp = torch.empty(sb, dtype=torch.uint8, device=w_q.device)
    _check(mxfp8_prepare_weight(_ptr(w_q), _ptr(w_s), N, K, w_q.stride(0), w_s.stride(0), _ptr(wp), _ptr(sp),
                                _stream(w_q.device)), "mxfp8_prepare_weight")
    return PreparedWeight(wp, sp, N, K)


_workspaces = {}
# Buffers a larger shape replaced.  They are never freed: a HIP graph captured
# earlier, or work still queued on the stream, may hold their addresses.
_retired = []


def _cache_key(device, stream):
    d = torch.device(device)
    idx = d.index if d.index is not None else torch.cuda.current_device()
    return idx, int(stream.cuda_stream)


def workspace(M, N, K, device):
    """A zero-initialised workspace big enough for mxfp8_linear at (M, N, K),
    cached per (device, current stream) and grown on demand (allocation
    happens here, never in the library).  Calls sharing a workspace must be
    ordered on one stream, hence one buffer per stream; a buffer that a
    larger shape replaces stays allocated for the life of the process, so a
    captured graph or queued work that still uses it never sees freed memory."""
    return _workspace_sized(mxfp8_linear_workspace_bytes(M, N, K), device)


def _workspace_sized(need, device, cache=None, zero=True):
    cache = _workspaces if cache is None else cache
    key = _cache_key(device, torch.cuda.current_stream(device))
    ws = cache.get(key)
    if ws is None or ws.numel() < need:
        if ws is not None:
            _retired.append(ws)
        size = max(need, 256)
        ws = torch.zeros(size, dtype=torch.uint8, device=device) if zero else \
            torch.empty(size, dtype=torch.uint8, device=device)
        cache[key] = ws
    return ws


class PreparedWeightFP4(PreparedWeight):
    """An MXFP4 weight after the one-time preparation (packed E2M1 payload,
    N_pad * K / 2 bytes, and its UE8M0 scales)."""

    def unpack(self):
        """(E2M1 ``[N_pad, K/2]``, two codes per byte, UE8M0 ``[N_pad, K/32]``)
        as uint8 tensors."""
        n_pad = (self.N + 127) // 128 * 128
        w = torch.empty((n_pad, self.K // 2), dtype=torch.uint8, device=self.device)
        s = torch.empty((n_pad, self.K // 32), dtype=torch.uint8, device=self.device)
        _check(mxfp8_unpack_weight_fp4(_ptr(self.w_packed), _ptr(self.s_packed), self.N, self.K, _ptr(w), _ptr(s),
                                       _stream(self.device)), "mxfp8_unpack_weight_fp4")
        return w, s


def prepare_weight_fp4(w_e2m1, w_s):
    """MXFP4 weight: ``w_e2m1`` uint8 ``[N, K/2]`` (two E2M1 codes per byte,
    element 2j in the low nibble) with UE8M0 scales ``w_s`` ``[>= N, >= K/32]``
    -> PreparedWeightFP4."""
    w_e2m1 = _as_bytes(w_e2m1)
    w_s = _as_bytes(w_s)
    _require_cuda(w_e2m1, "w_e2m1")
    N, K2 = w_e2m1.shape
    K = 2 * K2
    if w_e2m1.stride(-1) != 1 or w_e2m1.stride(0) % 16 != 0:
        w_e2m1 = w_e2m1.contiguous()
    if w_s.stride(-1) != 1:
        w_s = w_s.contiguous()
    wb, sb = mxfp8_prepared_weight_fp4_bytes(N, K)
    wp = torch.empty(wb, dtype=torch.uint8, device=w_e2m1.device)
    sp = torch.empty(sb, dtype=torch.uint8, device=w_e2m1.device)
    _check(mxfp8_prepare_weight_fp4(_ptr(w_e2m1), _ptr(w_s), N, K, w_e2m1.stride(0), w_s.stride(0), _ptr(wp),
                                    _ptr(sp), _stream(w_e2m1.device)), "mxfp8_prepare_weight_fp4")
    return PreparedWeightFP4(wp, sp, N, K)


def linear(x, pw, bias=None, out=None, workspace=None):
    """The MXFP8 dense linear layer: ``y = bf16(deq(q(x)) @ deq(W).T + bias)``.

    ``x`` bf16 ``[..., K]`` (GPU), ``pw`` a PreparedWeight (MXFP8) or a
    PreparedWeightFP4 (MXFP4, the W4A8 layer), ``bias`` bf16 ``[N]``
    or None.  Returns bf16 ``[..., N]`` (contiguous).  ``workspace``: an
    optional uint8 GPU tensor of at least ``mxfp8_linear_workspace_bytes``
    (``mxfp8_linear_w4a8_workspace_bytes`` for MXFP4) bytes, 256-byte
    aligned, owned by the caller; by default a cached buffer per (device,
    stream) is used."""
    assert x.dtype == torch.bfloat16, f"MXFP8 linear requires bfloat16 activations, got {x.dtype}"
    _require_cuda(x, "x")
    K = pw.K
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K)
    if x2.stride(-1) != 1 or x2.stride(0) % 8 != 0 or x2.data_ptr() % 16 != 0:
        x2 = x2.contiguous()
    M = x2.shape[0]
    N = pw.N
    if bias is not None:
        assert bias.dtype == torch.bfloat16 and bias.numel() == N
        bias = bias.contiguous()
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if isinstance(pw, PreparedWeightFP4):
        ws = workspace if workspace is not None else \
            _workspace_sized(mxfp8_linear_w4a8_workspace_bytes(M, N, K), x.device)
        _check(mxfp8_linear_w4a8(_ptr(x2), M, K, x2.stride(0), _ptr(pw.w_packed), _ptr(pw.s_packed), N,
                                 _ptr(bias), _ptr(y), y.stride(0), _ptr(ws), ws.numel(), _stream(x.device)),
               "mxfp8_linear_w4a8")
        return y.view(*lead, N)
    ws = workspace if workspace is not None else _workspace_sized(mxfp8_linear_workspace_bytes(M, N, K), x.device)
    _check(mxfp8_linear(_ptr(x2), M, K, x2.stride(0), _ptr(pw.w_packed), _ptr(pw.s_packed), N, _ptr(bias),
                        _ptr(y), y.stride(0), _ptr(ws), ws.numel(), _stream(x.device)), "mxfp8_linear")
    return y.view(*lead, N)


class PackedActivation:
    """Activations quantized into the GEMM's packed operand layout (rows padded
    to 128): the first kernel of the large-M path."""

    def __init__(self, q_packed, s_packed, M, K):
        self.q_packed = q_packed
        self.s_packed = s_packed
        self.M = M
        self.K = K

    def unpack(self):
        """(E4M3 ``[M_pad, K]``, UE8M0 ``[M_pad, K/32]``) as uint8 tensors."""
        return PreparedWeight(self.q_packed, self.s_packed, self.M, self.K).unpack()


def quantize_act_packed(x):
    """bf16 ``x[M, K]`` (GPU, K % 256 == 0) -> PackedActivation."""
    assert x.dtype == torch.bfloat16
    _require_cuda(x, "x")
    x2 = x.reshape(-1, x.shape[-1])
    if x2.stride(-1) != 1 or x2.stride(0) % 8 != 0 or x2.data_ptr() % 16 != 0:
        x2 = x2.contiguous()
    M, K = x2.shape
    qb, sb = mxfp8_packed_act_bytes(M, K)
    qp = torch.empty(qb, dtype=torch.uint8, device=x.device)
    sp = torch.empty(sb, dtype=torch.uint8, device=x.device)
    _check(mxfp8_quantize_act_packed(_ptr(x2), M, K, x2.stride(0), _ptr(qp), _ptr(sp), _stream(x.device)),
           "mxfp8_quantize_act_packed")
    return PackedActivation(qp, sp, M, K)


def gemm_packed(pa, pw, bias=None):
    """The GEMM + epilogue on packed activations (the second kernel of the
    large-M path)."""
    assert pa.K == pw.K
    y = torch.empty((pa.M, pw.N), dtype=torch.bfloat16, device=pa.q_packed.device)
    _check(mxfp8_gemm_packed(_ptr(pa.q_packed), _ptr(pa.s_packed), pa.M, pa.K, _ptr(pw.w_packed),
                             _ptr(pw.s_packed), pw.N, _ptr(bias), _ptr(y), y.stride(0),
                             _stream(pa.q_packed.device)), "mxfp8_gemm_packed")
    return y


# ---------------------------------------------------------------------------
# Routed MoE
# ---------------------------------------------------------------------------

def mxfp8_moe_prepared_bytes(E, H, I):
    out = [_sz() for _ in range(4)]
    _check(lib().mxfp8_moe_prepared_bytes(E, H, I, *[ctypes.byref(o) for o in out]), "mxfp8_moe_prepared_bytes")
    return tuple(o.value for o in out)


def mxfp8_moe_prepare_weights(w13, s13, w2, s2, E, H, I, w13p, s13p, w2p, s2p, stream):
    return lib().mxfp8_moe_prepare_weights(w13, s13, w2, s2, E, H, I, w13p, s13p, w2p, s2p, stream)


def mxfp8_moe_workspace_bytes(T, H, I, E, topk):
    b = _sz()
    _check(lib().mxfp8_moe_workspace_bytes(T, H, I, E, topk, ctypes.byref(b)), "mxfp8_moe_workspace_bytes")
    return b.value


def mxfp8_moe_grouped(x, logits, T, H, E, topk, I, w13p, s13p, w2p, s2p, y, ws, ws_bytes, stream):
    return lib().mxfp8_moe_grouped(x, logits, T, H, E, topk, I, w13p, s13p, w2p, s2p, y, ws, ws_bytes, stream)


def mxfp8_moe_debug_capture(act, q, s, ids, wts):
    return lib().mxfp8_moe_debug_capture(act, q, s, ids, wts)


class MoEWeights:
    """Expert weights after the one-time preparation (opaque packed layouts)."""

    def __init__(self, w13p, s13p, w2p, s2p, E, H, I):
        self.w13p, self.s13p, self.w2p, self.s2p = w13p, s13p, w2p, s2p
        self.E, self.H, self.I = E, H, I

    @property
    def device(self):
        return self.w13p.device


def moe_prepare_weights(w13_q, w13_s, w2_q, w2_s):
    """MXFP8 expert weights -> MoEWeights.

    ``w13_q`` E4M3 ``[E, 2I, H]`` (gate rows then up rows) with UE8M0 ``w13_s``
    ``[E, 2I, H/32]``; ``w2_q`` ``[E, H, I]`` with ``w2_s`` ``[E, H, I/32]``
    (uint8 or float8_e4m3fn, GPU)."""
    w13_q, w13_s, w2_q, w2_s = (_as_bytes(t).contiguous() for t in (w13_q, w13_s, w2_q, w2_s))
    _require_cuda(w13_q, "w13_q")
    E, two_i, H = w13_q.shape
    I = two_i // 2
    assert w2_q.shape == (E, H, I) and w13_s.shape == (E, 2 * I, H // 32) and w2_s.shape == (E, H, I // 32)
    b = mxfp8_moe_prepared_bytes(E, H, I)
    outs = [torch.empty(n, dtype=torch.uint8, device=w13_q.device) for n in b]
    _check(mxfp8_moe_prepare_weights(_ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s), E, H, I,
                                     *[_ptr(o) for o in outs], _stream(w13_q.device)), "mxfp8_moe_prepare_weights")
    return MoEWeights(*outs, E, H, I)


_moe_workspaces = {}


def moe_workspace(T, H, I, E, topk, device):
    """The MoE layer's workspace, cached per (device, current stream) like
    ``workspace`` (superseded buffers are kept, never freed)."""
    return _workspace_sized(mxfp8_moe_workspace_bytes(T, H, I, E, topk), device, cache=_moe_workspaces, zero=False)


def moe_grouped(x, logits, mw, topk, out=None):
    """The MXFP8 routed MoE layer: ``x`` bf16 ``[T, H]``, ``logits`` fp32
    ``[T, E]``, ``mw`` MoEWeights -> bf16 ``[T, H]``."""
    assert x.dtype == torch.bfloat16, f"MXFP8 MoE takes bfloat16 activations, got {x.dtype}"
    assert logits.dtype == torch.float32
    _require_cuda(x, "x")
    x = x.contiguous()
    logits = logits.contiguous()
    T, H = x.shape
    assert H == mw.H and logits.shape == (T, mw.E)
    y = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    ws = moe_workspace(T, H, mw.I, mw.E, topk, x.device)
    _check(mxfp8_moe_grouped(_ptr(x), _ptr(logits), T, H, mw.E, topk, mw.I, _ptr(mw.w13p), _ptr(mw.s13p),
                             _ptr(mw.w2p), _ptr(mw.s2p), _ptr(y), _ptr(ws), ws.numel(), _stream(x.device)),
           "mxfp8_moe_grouped")
    return y


def moe_debug_capture(act=None, q=None, s=None, ids=None, wts=None):
    """Test hook: capture, per row t*k + j, the gated activation (bf16
    ``[T*k, I]``), its MX quantization (``[T*k, I]`` / ``[T*k, I/32]`` uint8),
    the routed expert (int32 ``[T*k]``) and routing weight (fp32 ``[T*k]``) of
    later MoE calls; no arguments turns it off."""
    _check(mxfp8_moe_debug_capture(_ptr(act), _ptr(q), _ptr(s), _ptr(ids), _ptr(wts)), "mxfp8_moe_debug_capture")
