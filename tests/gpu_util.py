"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the oracle on the same seeded inputs, compare.

The GEMM tolerance is derived from the arithmetic of the HIP path (no number
is fitted to observed errors):
  * each scaled MFMA instruction (K = 64 or 128 elements) returns its partial
    sum with an error below 2^-12 of its largest product term (measured on
    gfx950 against exact sums; the bound used is 2^-10, four times that);
  * the partials are added in fp32 (error <= 2^-24 per add of the running
    sum, bounded by K * 2^-24 * sum |terms|);
  * bias is added in fp32 and the result rounded once to bf16 (half an ulp:
    <= 2^-8 relative).
So for every output  |y - r| <= 2^-8 |r| + (1 + 2^-8) [ (K/64) 2^-10 Amax(m) Wmax(n)
                                                    + K 2^-23 S(m, n) ] + 2^-133,
with r the oracle's exact value, Amax / Wmax the largest dequantized magnitude
in row m of A / row n of W, S = sum_k |A[m,k]| |W[n,k]|.  On top of this the
aggregate criteria: normwise ||y - r|| / ||r|| <= 2^-7 and the layer's "max
relative error 2e-2" read as max |y - r| / max(|r|, 2^-4 rms(r)) <= 2e-2.
"""

import numpy as np
import torch

import oracle
from mxfp8_block_scaled_amd import api


def dev():
    return torch.device("cuda", 0)


def gpu_quantize(x_bf16_cpu):
    """Quantize on the GPU; returns CPU numpy (q, s)."""
    q, s = api.quantize_act(x_bf16_cpu.to(dev()))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def gpu_prepare(w_bf16_cpu):
    """Quantize the bf16 weight with the HIP quantizer and prepare it."""
    wq, ws = api.quantize_act(w_bf16_cpu.to(dev()))
    return api.prepare_weight(wq, ws)


def oracle_weight(w_bf16_cpu):
    return oracle.quantize_mx(w_bf16_cpu.to(torch.float64).numpy())


def tolerance(x_np, wq, ws, N, K):
    """Per-element bound terms (everything but the 2^-8 |r| part)."""
    qa, sa = oracle.quantize_mx(x_np)
    A = oracle.dequantize_mx(qa, sa)
    W = oracle.dequantize_mx(wq[:N], ws[:N])
    amax = np.abs(A).max(axis=1)
    wmax = np.abs(W).max(axis=1)
    S = np.abs(A) @ np.abs(W).T
    acc = (K / 64.0) * 2.0 ** -10 * np.outer(amax, wmax) + K * 2.0 ** -23 * S
    return (1 + 2.0 ** -8) * acc + 2.0 ** -133


def compare(y, r, acc_bound, label=""):
    """y: GPU output (float64 numpy of bf16 values); r: exact oracle values."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{label}: non-finite outputs"
    err = np.abs(y - r)
    bound = 2.0 ** -8 * np.abs(r) + acc_bound
    over = err > bound
    stats = {
        "label": label,
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "normwise": float(np.linalg.norm(y - r) / max(np.linalg.norm(r), 1e-300)) if err.size else 0.0,
        "over_bound": int(over.sum()),
        "elements": int(err.size),
    }
    if err.size:
        rms = np.sqrt(np.mean(r * r))
        stats["max_rel_2e-2_metric"] = float((err / np.maximum(np.abs(r), 2.0 ** -4 * rms + 1e-300)).max())
        # the same with the floor max(|r|, 1e-3 max|r|) of the survey's reading
        stats["max_rel_survey_floor"] = float((err / np.maximum(np.abs(r), 1e-3 * np.abs(r).max() + 1e-300)).max())
        stats["max_err_over_bound"] = float((err / bound).max())
    print("PARITY", stats, flush=True)
    assert stats["over_bound"] == 0, (label, stats, np.argwhere(over)[:5])
    if err.size:
        assert stats["normwise"] <= 2.0 ** -7, stats
        assert stats["max_rel_2e-2_metric"] <= 2e-2, stats
    return stats


def run_linear_and_check(x, w, bias, label, force_path=0, N_logical=None):
    """x [M,K], w [N,K], bias [N] or None: bf16 CPU tensors."""
    N, K = w.shape
    pw = gpu_prepare(w)
    prev = api.mxfp8_debug_force_path(force_path)
    try:
        y = api.linear(x.to(dev()), pw, None if bias is None else bias.to(dev()))
        torch.cuda.synchronize()
    finally:
        api.mxfp8_debug_force_path(prev)
    assert y.shape == (x.shape[0], N) and y.is_contiguous()
    wq, ws = oracle_weight(w)
    xn = x.to(torch.float64).numpy()
    bn = None if bias is None else bias.to(torch.float64).numpy()
    r = oracle.linear_ref(xn, wq, ws, bn)
    return compare(y.float().cpu().numpy(), r, tolerance(xn, wq, ws, N, K), label)


def exhaustive_quant_input():
    """Blocks that together hold every finite bf16 value under every scale
    exponent the rule can produce.  For each bf16 binade E (including the
    subnormal ones) the block maximum is pinned to the largest value of that
    binade, and the other 31 slots walk every bf16 magnitude not above it,
    both signs.  Returns a bf16 CPU tensor [R, 2048]."""
    pos = np.arange(0, 0x7F80, dtype=np.uint16)  # all finite non-negative patterns, magnitude order
    blocks = []
    for E in range(-133, 128):
        if E >= -126:
            anchor = np.uint16(((E + 127) << 7) | 0x7F)
        else:
            anchor = np.uint16((1 << (E + 134)) - 1)  # subnormal binade: mantissa < 2^(E+134)
        vals = pos[pos <= anchor]
        vals = np.concatenate([vals, vals | np.uint16(0x8000)])
        nblk = (len(vals) + 30) // 31
        pad = np.zeros(nblk * 31, dtype=np.uint16)
        pad[: len(vals)] = vals
        b = np.empty((nblk, 32), dtype=np.uint16)
        b[:, 0] = anchor | np.uint16(0x8000 * (E & 1))
        b[:, 1:] = pad.reshape(nblk, 31)
        blocks.append(b)
    allb = np.concatenate(blocks)
    per_row = 64
    rows = (len(allb) + per_row - 1) // per_row
    full = np.zeros((rows * per_row, 32), dtype=np.uint16)
    full[: len(allb)] = allb
    return torch.from_numpy(full.reshape(rows, per_row * 32).view(np.int16)).view(torch.bfloat16)
