"""Benchmark of the MXFP8 dense linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-cpu]

Prints ONE JSON line.  The headline workload is the large compute-bound layer
M=8192, N=28672, K=8192 (x ~ N(0,1), W ~ N(0,0.01) MXFP8, bf16 bias): a step is
one pass of the whole hot path over that batch -- activation quantization
into the GEMM's packed layout (mxfp8_quantize_act_packed) then the
block-scaled GEMM with its bias/bf16 epilogue (mxfp8_gemm_packed), the same
two kernels mxfp8_linear launches for M > 128 (and for any M when K > 8192).
The one-time weight preparation runs before the timed region.  ``value`` is
2*M*N*K / step time in TFLOP/s, inputs resident in HBM.

Also reported: ``roofline`` for the dominant kernel (the GEMM) from HIP events
on the launch stream inside the timed region; ``sweep`` with the other
workload shapes (M=7 single layer, the decode sweep M in {1,7,16,128} at
N=K=4096 with the weights rotated through 48 copies so they do not sit in the
256 MB last-level cache, the M=16384 prefill shape, and the standalone
quantizer, and one forward of the routed MoE layer at its full size);
``ceilings``, what this GPU sustains as measured by the calibration kernels
of libmxfp8_calib.so (scaled-MFMA rate, 1 GiB HBM read rate, one 16 MiB read
per launch and one read of the W4A8 decode weight's 8.5 MiB per launch, the
time per launch of an empty kernel), with the headline GEMM's fraction of the measured MFMA rate
(``roofline.frac_of_measured``) and each sweep row's fraction of the
measured read rate; ``cpu_baseline``, the CPU oracle timed on a bounded
sample of the headline workload.  The untimed warm-up runs at least
``--warmup`` steps and at least ``--warmup-ms`` (300) of wall time, since
the clock ramps up over the first ~50 ms of load.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_FP8_TFLOPS = 5000.0   # MI355X dense FP8 / MXFP8 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_tile_large.json")
GEMM_SOURCES = ["mxfp8_block_scaled_amd/csrc/gemm_tile.hip", "mxfp8_block_scaled_amd/csrc/tile_core.hpp",
                "mxfp8_block_scaled_amd/csrc/common.hpp"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50,
                   help="untimed steps first; the warm-up also runs for at least --warmup-ms of wall time "
                        "(the GPU clock ramps up over the first ~50 ms of load)")
    p.add_argument("--warmup-ms", type=float, default=300.0)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    return p.parse_args()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(bytes_per_launch_expected):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs, or
    None if they were taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash(GEMM_SOURCES):
        return None
    return t.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus N > 1 is not supported "
                                   "(the layer shards by N or K across GPUs as described in DESIGN.md, "
                                   "but no multi-GPU path is built)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from mxfp8_block_scaled_amd import api, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    # ---------------- headline workload: M=8192, N=28672, K=8192 ----------------
    x, w_g, bias = synth.config_inputs(4, device=dev)
    M, K = x.shape
    N = w_g.shape[0]
    wq, ws = api.quantize_act(w_g)
    pw = api.prepare_weight(wq, ws)
    del wq, ws, w_g
    qb, sb = api.mxfp8_packed_act_bytes(M, K)
    q = torch.empty(qb, dtype=torch.uint8, device=dev)
    s = torch.empty(sb, dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = api.mxfp8_quantize_act_packed(x.data_ptr(), M, K, K, q.data_ptr(), s.data_ptr(), sptr)
        if ev is not None:
            ev[1].record(stream)
        st |= api.mxfp8_gemm_packed(q.data_ptr(), s.data_ptr(), M, K, pw.w_packed.data_ptr(),
                                    pw.s_packed.data_ptr(), N, bias.data_ptr(), y.data_ptr(), N, sptr)
        if ev is not None:
            ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"launch failed: {st}")

    # Untimed warm-up: at least --warmup steps and at least --warmup-ms of
    # wall time, whichever is longer.
    tw0 = time.perf_counter()
    nwarm = 0
    while nwarm < args.warmup or (time.perf_counter() - tw0) * 1e3 < args.warmup_ms:
        for _ in range(10):
            step()
        nwarm += 10
        torch.cuda.synchronize()
    warmup_ms = (time.perf_counter() - tw0) * 1e3
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    quant_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gemm_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    quant_bytes = M * K * (2 + 1 + 1 / 32)

    # Same shape through the single product entry point, for reference.
    ws_t = api.workspace(M, N, K, dev)
    for _ in range(10):
        api.linear(x, pw, bias, out=y)
    torch.cuda.synchronize()
    for _ in range(3):   # the last of three repeats (first-use transient of the new workspace)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            api.linear(x, pw, bias, out=y)
        e1.record(stream)
        torch.cuda.synchronize()
        linear_ms = e0.elapsed_time(e1) / args.steps
    del ws_t

    out = {
        "metric": "mxfp8_linear TFLOP/s & % MFMA peak (M=1..16384); act-quant GB/s % HBM",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": nwarm,
        "warmup_ms": round(warmup_ms, 1),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 (MXFP8, fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded; x ~ N(0,1) bf16, W ~ N(0,0.01) quantized to MXFP8, bias ~ N(0,0.1))",
        "config": {"workload": "large compute-bound MXFP8 linear M=8192 N=28672 K=8192 with bias",
                   "M": M, "N": N, "K": K, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100 * value / PEAK_MFMA_FP8_TFLOPS, 2),
        "kernels_ms": {"act_quant": round(quant_ms, 4), "gemm": round(gemm_ms, 4),
                       "mxfp8_linear_entry": round(linear_ms, 4)},
        "act_quant": {"GB/s": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                      "pct_hbm": round(100 * quant_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_MFMA_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_MFMA_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(None), "kernel": "gemm_persistent_kernel"},
    }
    del q, s, y, x

    # Measured ceilings of this GPU (calibration kernels), and the headline
    # GEMM against the measured MFMA rate.
    ceil = ceilings(torch, dev, stream)
    out["ceilings"] = ceil
    if ceil.get("mfma_tflops"):
        out["roofline"]["frac_of_measured"] = round(gemm_tflops / ceil["mfma_tflops"], 4)
    if ceil.get("l2_to_lds_gbs_per_cu"):
        # The GEMM's operand copies: every 256 x 256 tile copies its 512 rows
        # of K bytes (plus 1/32 in scales) from L2 into LDS; per CU per second
        # against what one CU pulls from L2 in the calibration kernel.
        tiles = ((M + 255) // 256) * ((N + 255) // 256)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        copy_gbs = tiles * 512 * K * (1 + 1 / 32) / cus / (gemm_ms * 1e-3) / 1e9
        out["roofline"]["copy_gbs_per_cu"] = round(copy_gbs, 1)
        out["roofline"]["frac_of_copy_ceiling"] = round(copy_gbs / ceil["l2_to_lds_gbs_per_cu"], 4)

    if not args.no_sweep:
        out["sweep"] = sweep(api, synth, torch, np, dev, stream)
        floor = ceil.get("read_16mib_us")
        for row in out["sweep"]:
            if floor and row.get("workload", "").startswith("decode M="):
                # the weight read alone (16 MiB + scales) at the measured floor
                row["pct_of_read_floor"] = round(100 * floor * (4096 * 4096 * (1 + 1 / 32)) / (16 << 20) / row["us"], 1)
            if ceil.get("read_w4_4096x4096_us") and row.get("workload", "").startswith("decode W4A8 M="):
                # the MXFP4 weight read alone, measured at its own size
                row["pct_of_read_floor"] = round(100 * ceil["read_w4_4096x4096_us"] / row["us"], 1)
            if ceil.get("hbm_read_gbs") and "GB/s" in row:
                row["pct_of_measured_hbm"] = round(100 * row["GB/s"] / ceil["hbm_read_gbs"], 1)
            if row.get("workload", "").startswith("single ") and ceil.get("launch_floor_us"):
                # a one-kernel call against an empty kernel of the same grid
                row["launch_floor_us"] = ceil["launch_floor_us"]
                row["x_launch_floor"] = round(row["us"] / ceil["launch_floor_us"], 2)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bcp = torch.empty_like(a)
        for _ in range(3):
            bcp.copy_(a)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = 1 << 30

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(synth, np, torch)

    print(json.dumps(out))


def ceilings(torch, dev, stream):
    """What this GPU sustains, measured with libmxfp8_calib.so: the scaled
    16x16x128 MFMA rate over a grid that fills the chip, the HBM read rate
    of a 1 GiB stream, and the time of one 16 MiB read per launch rotating
    over 48 copies (the floor of a decode-sized weight read)."""
    import ctypes
    path = os.path.join(ROOT, "mxfp8_block_scaled_amd", "libmxfp8_calib.so")
    if not os.path.exists(path):
        return {"error": "libmxfp8_calib.so not built"}
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.mxfp8_calib_read.argtypes = [vp, ctypes.c_uint64, ctypes.c_int, vp, vp]
    lib.mxfp8_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    lib.mxfp8_calib_empty.argtypes = [ctypes.c_int, ctypes.c_int, vp]
    lib.mxfp8_calib_l2.argtypes = [vp, ctypes.c_uint32, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    sptr = stream.cuda_stream
    out = {}
    # one launch of an empty kernel, back to back on the stream: the floor
    # under a one-kernel call (9 x 1024 threads: the M=7, N=130 layer's grid;
    # 256 x 1024: the decode kernel's at N = 4096)
    for blocks, key in ((9, "launch_floor_us"), (256, "launch_floor_256wg_us")):
        for _ in range(50):
            lib.mxfp8_calib_empty(blocks, 1024, sptr)
        torch.cuda.synchronize()
        ms = min(time_calls(lambda r: lib.mxfp8_calib_empty(blocks, 1024, sptr), 500, stream, torch)
                 for _ in range(3))
        out[key] = round(ms * 1e3, 3)
    # scaled MFMA: 4096 waves x iters x 8 MFMAs of 2*16*16*128 flops
    blocks, iters = 1024, 1500
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    for _ in range(3):
        lib.mxfp8_calib_mfma(blocks, iters, sink.data_ptr(), sptr)
    torch.cuda.synchronize()
    ms = min(time_calls(lambda r: lib.mxfp8_calib_mfma(blocks, iters, sink.data_ptr(), sptr), 5, stream, torch)
             for _ in range(3))
    flops = blocks * 4 * iters * 8 * 2.0 * 16 * 16 * 128
    out["mfma_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    # 1 GiB read stream (best of two grid sizes)
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    words = torch.empty(8192, dtype=torch.int32, device=dev)
    best = None
    for blocks in (4096, 8192):
        for _ in range(3):
            lib.mxfp8_calib_read(big.data_ptr(), big.numel(), blocks, words.data_ptr(), sptr)
        torch.cuda.synchronize()
        ms = min(time_calls(lambda r: lib.mxfp8_calib_read(big.data_ptr(), big.numel(), blocks, words.data_ptr(),
                                                           sptr), 10, stream, torch) for _ in range(3))
        best = ms if best is None else min(best, ms)
    out["hbm_read_gbs"] = round(big.numel() / (best * 1e-3) / 1e9, 1)
    del big
    # one read of n16 bytes per launch over 48 rotated copies (> 3x the
    # last-level cache at 16 MiB), best of three grid sizes
    def read_floor_us(n16):
        pool = torch.empty(48 * n16, dtype=torch.uint8, device=dev)
        best = None
        for blocks in (512, 1024, 2048):
            for r in range(96):
                lib.mxfp8_calib_read(pool.data_ptr() + (r % 48) * n16, n16, blocks, words.data_ptr(), sptr)
            torch.cuda.synchronize()
            ms = min(time_calls(lambda r: lib.mxfp8_calib_read(pool.data_ptr() + (r % 48) * n16, n16, blocks,
                                                               words.data_ptr(), sptr), 480, stream, torch)
                     for _ in range(3))
            best = ms if best is None else min(best, ms)
        del pool
        return round(best * 1e3, 3)

    out["read_16mib_us"] = read_floor_us(16 << 20)
    # the MXFP4 weight of the W4A8 decode rows: 4096 x 4096 E2M1 + scales
    out["read_w4_4096x4096_us"] = read_floor_us(4096 * 4096 // 2 + 4096 * 4096 // 32)
    # L2 -> CU: one workgroup per CU re-reading one 1 MiB buffer (served by
    # each die's L2 after the first pass), into registers and by direct
    # L2 -> LDS copies; GB/s per CU
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    l2buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    reps = 100
    for lds, key in ((0, "l2_to_vgpr_gbs_per_cu"), (1, "l2_to_lds_gbs_per_cu")):
        for _ in range(2):
            lib.mxfp8_calib_l2(l2buf.data_ptr(), l2buf.numel(), cus, reps, lds, words.data_ptr(), sptr)
        torch.cuda.synchronize()
        ms = min(time_calls(lambda r: lib.mxfp8_calib_l2(l2buf.data_ptr(), l2buf.numel(), cus, reps, lds,
                                                         words.data_ptr(), sptr), 3, stream, torch)
                 for _ in range(3))
        out[key] = round(l2buf.numel() * reps / (ms * 1e-3) / 1e9, 1)
    del l2buf
    print(f"ceilings: {out}", file=sys.stderr, flush=True)
    return out


def time_calls(fn, reps, stream, torch):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        fn(r)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def sweep(api, synth, torch, np, dev, stream):
    rows = []
    sptr = stream.cuda_stream

    def linear_entry(x_list, pw_list, b, M, N, K, y, reps, label, extra=None, w4=False):
        if w4:
            ws_t = torch.zeros(api.mxfp8_linear_w4a8_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
            entry = api.mxfp8_linear_w4a8
        else:
            ws_t = api.workspace(M, N, K, dev)
            entry = api.mxfp8_linear

        def fn(r):
            xx = x_list[r % len(x_list)]
            pp = pw_list[r % len(pw_list)]
            st = entry(xx.data_ptr(), M, K, K, pp.w_packed.data_ptr(), pp.s_packed.data_ptr(), N,
                       None if b is None else b.data_ptr(), y.data_ptr(), N, ws_t.data_ptr(), ws_t.numel(), sptr)
            if st != 0:
                raise RuntimeError(st)
        # Untimed warm-up, then three timed repeats; the last is reported.  A
        # shape's first calls on freshly allocated buffers run slower for a
        # few milliseconds (prefill: 163 us in the first repeat, 153-155 us
        # after), longer than a warm-up of a few calls covers.
        for r in range(max(5, reps // 2)):
            fn(r)
        torch.cuda.synchronize()
        tries = [time_calls(fn, reps, stream, torch) for _ in range(3)]
        print(f"{label}: " + " ".join(f"{t * 1e3:.2f}" for t in tries) + " us", file=sys.stderr, flush=True)
        ms = tries[-1]
        flops = 2.0 * M * N * K
        alg_bytes = M * K * 2 + N * K * (0.5 if w4 else 1.0) + N * K / 32 + (0 if b is None else 2 * N) + M * N * 2
        row = {"workload": label, "M": M, "N": N, "K": K, "us": round(ms * 1e3, 3),
               "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 3),
               "GB/s": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
               "pct_mfma_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_FP8_TFLOPS, 2),
               "pct_hbm": round(100 * alg_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
        if extra:
            row.update(extra)
        rows.append(row)

    # single layer, M=7 N=130 K=256 (launch-latency bound)
    x, w, b = synth.config_inputs(1, device=dev)
    wq, ws = api.quantize_act(w)
    pw = api.prepare_weight(wq, ws)
    y = torch.empty((7, 130), dtype=torch.bfloat16, device=dev)
    linear_entry([x], [pw], b, 7, 130, 256, y, 200, "single M=7 N=130 K=256")

    # decode sweep, weights rotated over 48 copies (> 3x the 256 MB MALL)
    w, bd = synth.decode_weight(device=dev)
    wq, ws = api.quantize_act(w)
    pw0 = api.prepare_weight(wq, ws)
    copies = [pw0] + [api.PreparedWeight(pw0.w_packed.clone(), pw0.s_packed.clone(), pw0.N, pw0.K)
                      for _ in range(47)]
    for M in (1, 7, 16, 128):
        xm, _, _ = synth.config_inputs(2, M, device=dev)
        xs = [xm.clone() for _ in range(8)]
        y = torch.empty((M, 4096), dtype=torch.bfloat16, device=dev)
        linear_entry(xs, copies, bd, M, 4096, 4096, y, 480, f"decode M={M} N=4096 K=4096",
                     {"weight_copies_rotated": 48})
        # The same 48 calls captured once in a HIP graph and replayed: the
        # per-call time without the host's per-launch cost.
        rows[-1]["graph_replay_us"] = graph_replay_us(api, torch, dev, xs, copies, bd, M, y)
    del copies, pw0

    # W4A8 decode: the same bf16 decode weight quantized to MXFP4 by the
    # library, the same rotation over 48 copies
    w4, s4 = api.quantize_fp4(w)
    pw4 = api.prepare_weight_fp4(w4, s4)
    copies4 = [pw4] + [api.PreparedWeightFP4(pw4.w_packed.clone(), pw4.s_packed.clone(), pw4.N, pw4.K)
                       for _ in range(47)]
    for M in (1, 7, 16):
        xm, _, _ = synth.config_inputs(2, M, device=dev)
        xs = [xm.clone() for _ in range(8)]
        y = torch.empty((M, 4096), dtype=torch.bfloat16, device=dev)
        linear_entry(xs, copies4, bd, M, 4096, 4096, y, 480, f"decode W4A8 M={M} N=4096 K=4096",
                     {"weight_copies_rotated": 48}, w4=True)
    del copies4, pw4

    # prefill QKV shape, M=16384 N=5120 K=2048, no bias
    xd, w, _ = synth.config_inputs(3, device=dev)
    wq, ws = api.quantize_act(w)
    pw = api.prepare_weight(wq, ws)
    y = torch.empty((16384, 5120), dtype=torch.bfloat16, device=dev)
    linear_entry([xd], [pw], None, 16384, 5120, 2048, y, 50, "prefill_qkv M=16384 N=5120 K=2048")

    # routed MoE layer: 4096 tokens, H=2048, 128 experts, top-8, I=768
    rows.append(moe_row(api, synth, torch, dev, stream))

    # standalone quantizer on the prefill activations
    q = torch.empty((16384, 2048), dtype=torch.uint8, device=dev)
    s = torch.empty((16384, 64), dtype=torch.uint8, device=dev)

    def qf(r):
        api.mxfp8_quantize_act(xd.data_ptr(), 16384, 2048, 2048, q.data_ptr(), 2048, s.data_ptr(), 64,
                               stream.cuda_stream)
    for r in range(50):
        qf(r)
    ms = [time_calls(qf, 100, stream, torch) for _ in range(3)][-1]
    nb = 16384 * 2048 * (2 + 1 + 1 / 32)
    rows.append({"workload": "act-quant M=16384 K=2048", "us": round(ms * 1e3, 3),
                 "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                 "pct_hbm": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)})
    return rows


def graph_replay_us(api, torch, dev, xs, copies, bias, M, y, replays=10):
    """Per-call time of mxfp8_linear over the 48 weight copies, captured in a
    HIP graph on a side stream and replayed (checked against eager first)."""
    N, K = copies[0].N, copies[0].K
    ws_t = api.workspace(M, N, K, dev)
    side = torch.cuda.Stream(device=dev)

    def calls(sp):
        for r, pp in enumerate(copies):
            st = api.mxfp8_linear(xs[r % len(xs)].data_ptr(), M, K, K, pp.w_packed.data_ptr(),
                                  pp.s_packed.data_ptr(), N, bias.data_ptr(), y.data_ptr(), N, ws_t.data_ptr(),
                                  ws_t.numel(), sp)
            if st != 0:
                raise RuntimeError(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls(side.cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream(dev)
    e0.record(cur)
    for _ in range(replays):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / (replays * len(copies)), 3)


def moe_row(api, synth, torch, dev, stream):
    """One forward of the MoE layer (every kernel of mxfp8_moe_grouped).
    FLOPs count the routed rows only (2 T k (2I H + H I)); bytes are the
    minimum a forward must move: both expert weights with their scales, x,
    logits and y."""
    c = synth.MOE_CONFIG
    T, H, E, k, inter = c["T"], c["H"], c["E"], c["topk"], c["I"]
    x, logits, w13, w2 = synth.moe_inputs(device=dev)
    q13, s13 = api.quantize_act(w13.reshape(E * 2 * inter, H))
    q2, s2 = api.quantize_act(w2.reshape(E * H, inter))
    del w13, w2
    mw = api.moe_prepare_weights(q13.view(E, 2 * inter, H), s13.view(E, 2 * inter, H // 32),
                                 q2.view(E, H, inter), s2.view(E, H, inter // 32))
    del q13, s13, q2, s2
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    for _ in range(10):
        api.moe_grouped(x, logits, mw, k, out=y)
    torch.cuda.synchronize()
    # the last of three repeats, as for the linear shapes
    tries = [time_calls(lambda r: api.moe_grouped(x, logits, mw, k, out=y), 20, stream, torch) for _ in range(3)]
    print("moe: " + " ".join(f"{t * 1e3:.2f}" for t in tries) + " us", file=sys.stderr, flush=True)
    ms = tries[-1]
    flops = 2.0 * T * k * (2 * inter * H + H * inter)
    nbytes = E * (2 * inter * H + H * inter) * (1 + 1 / 32) + T * H * 2 * 2 + T * E * 4
    return {"workload": f"moe T={T} H={H} E={E} top{k} I={inter}", "us": round(ms * 1e3, 3),
            "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 3), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "pct_mfma_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_FP8_TFLOPS, 2),
            "pct_hbm": round(100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}


def cpu_baseline(synth, np, torch):
    """The oracle as it stands, on a bounded sample of the headline workload:
    4096 activation rows x 16384 weight rows x the full K = 8192, drawn with
    the workload's distributions (quantize both, exact dequantized fp64
    product, bias; about 10-20 s on a 16-core host).  Reported in the
    metric's unit.  cores: the threads it used (the BLAS pool; the
    quantization runs on one); host_cpus: os.cpu_count()."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    c = synth.LINEAR_CONFIGS[4]
    Ms, Ns, K = 4096, 16384, c["K"]
    x, w, b = synth.linear_inputs(Ms, Ns, K, c["seed"], c["x_std"], c["w_std"], c["bias_std"])
    xs = x.to(torch.float64).numpy()
    wsub = w.to(torch.float64).numpy()
    bs = b.to(torch.float64).numpy()
    t0 = time.perf_counter()
    wq, wsc = oracle.quantize_mx(wsub)
    oracle.linear_ref(xs, wq, wsc, bs)
    dt = time.perf_counter() - t0
    flops = 2.0 * Ms * Ns * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "host_cpus": os.cpu_count(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"M={Ms} x N={Ns} x K={K} slice of the M=8192 N=28672 K=8192 "
                      "workload: MX-quantize x and W (numpy, 1 thread), fp64 dequantized product "
                      "(BLAS threads) + bias"}


if __name__ == "__main__":
    main()
