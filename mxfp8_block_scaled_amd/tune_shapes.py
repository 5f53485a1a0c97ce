"""Measure the GEMM paths of ``mxfp8_linear`` over a grid of shapes on the
current GPU and write the shape table the library dispatches from
(``csrc/shape_table.inc``; rebuild the library afterwards).

    python -m mxfp8_block_scaled_amd.tune_shapes --csv profiles/shape_table_mi355x.csv --inc
    python -m mxfp8_block_scaled_amd.tune_shapes --from-rules --inc    # no GPU: the fixed cut-offs

The table has buckets along M, N and K (BOUNDS below); a shape falls in the
first bucket whose bound is >= its size on each axis, and the last bucket
takes everything larger.  For each bucket the upper corner (M, N, K) is timed
under every GEMM path that applies to it:

* the decode kernel (M <= 16, K <= 8192),
* the mid-M kernel (M <= 128, K <= 8192),
* the split-K slab kernel (M <= 128, any K),
* the medium-tile GEMM, 128 x 128 and 128 x 64 tiles over the whole K
  (shapes with at most 4096 such tiles),
* the large-tile GEMM with s = 1 (persistent), 2, 4 or 8 K splits
  ((K / 64) % (4 s) == 0; split counts whose grid exceeds four workgroups
  per CU are not tried).

A timing is the whole ``mxfp8_linear`` call (activation quantization
included, bias on) averaged over back-to-back calls in HIP events, the best
of three rounds; weight copies are rotated so that a small weight does not
stay in cache from one call to the next.  The fastest candidate becomes the
bucket's plan and the fastest large-tile candidate its split count (used
where the tile GEMM runs whatever M is: ``mxfp8_gemm_prequant`` and the
large-M W4A8 path).  The CSV keeps every timing.
"""

import argparse
import datetime
import os
import sys

BOUNDS = {
    "M": [1, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192],
    "N": [1024, 2048, 4096, 8192, 16384, 32768],
    "K": [1024, 2048, 4096, 8192, 16384],
}
PATH_CODE = {"tile": 0, "decode": 1, "mid": 2, "slab": 3, "med128": 4, "med64": 5}
SKINNY_MAX_M, MID_MAX_M, SMALL_K = 16, 128, 8192
INC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "shape_table.inc")


def splits_ok(K, s):
    """A K slice must be a whole number of 128-K step pairs: (K/64) % (4s) == 0."""
    return s == 1 or (s in (2, 4, 8) and (K // 64) % (4 * s) == 0)


def candidates(M, N, K, cus=256):
    """(name, force value) of every path that applies to M x N x K."""
    out = []
    if M <= SKINNY_MAX_M and K <= SMALL_K:
        out.append(("decode", 4))
    if M <= MID_MAX_M and K <= SMALL_K:
        out.append(("mid", 3))
    if M <= MID_MAX_M:
        out.append(("slab", 5))
    groups = (N + 127) // 128
    if groups * ((M + 127) // 128) <= 4096:
        out.append(("med128", 6))
    if groups * ((M + 63) // 64) <= 4096:
        out.append(("med64", 7))
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    for s in (1, 2, 4, 8):
        if splits_ok(K, s) and (s == 1 or tiles * s <= 4 * cus):
            out.append((f"tile{s}", 16 + s))
    return out


def rules_plan(M, N, K):
    """The fixed cut-offs the table replaces: (path, tile splits)."""
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    s = 1
    while s < 8 and tiles * s * 2 <= 256 and (K // 64) % (8 * s) == 0:
        s *= 2
    s = s if tiles < 128 else 1
    if K <= SMALL_K and M <= SKINNY_MAX_M:
        return "decode", s
    if K <= SMALL_K and M <= MID_MAX_M:
        return "mid", s
    return "tile", s


def write_inc(plan, tile_splits, source, path=INC):
    nm, nn, nk = (len(BOUNDS[a]) for a in "MNK")

    def arr(t):
        rows = []
        for im in range(nm):
            inner = ", ".join("{" + ", ".join(str(t[im][i_n][ik]) for ik in range(nk)) + "}" for i_n in range(nn))
            rows.append("    {" + inner + "}")
        return "{\n" + ",\n".join(rows) + "\n}"

    text = f"""// Shape table of mxfp8_linear, written by mxfp8_block_scaled_amd/tune_shapes.py
// ({source}).  A shape (M, N, K) falls in the first bucket whose bound is
// >= its size on each axis (the last bucket takes everything larger).
// kShapeTabPlan: path << 4 | K splits of the fastest candidate measured at the
// bucket's upper corner (path 0 large-tile GEMM, 1 decode kernel, 2 mid-M
// kernel, 3 split-K slab kernel, 4 / 5 medium-tile GEMM with 128 / 64
// activation rows per tile); kShapeTabTileSplits: K splits of the fastest large-tile candidate.
#pragma once
#include <cstdint>

namespace mxfp8 {{
constexpr int kShapeTabNM = {nm}, kShapeTabNN = {nn}, kShapeTabNK = {nk};
constexpr int64_t kShapeTabM[kShapeTabNM] = {{{", ".join(map(str, BOUNDS["M"]))}}};
constexpr int64_t kShapeTabN[kShapeTabNN] = {{{", ".join(map(str, BOUNDS["N"]))}}};
constexpr int64_t kShapeTabK[kShapeTabNK] = {{{", ".join(map(str, BOUNDS["K"]))}}};
constexpr uint8_t kShapeTabPlan[kShapeTabNM][kShapeTabNN][kShapeTabNK] = {arr(plan)};
constexpr uint8_t kShapeTabTileSplits[kShapeTabNM][kShapeTabNN][kShapeTabNK] = {arr(tile_splits)};
}}  // namespace mxfp8
"""
    with open(path, "w") as f:
        f.write(text)


def grid():
    for im, M in enumerate(BOUNDS["M"]):
        for i_n, N in enumerate(BOUNDS["N"]):
            for ik, K in enumerate(BOUNDS["K"]):
                yield im, i_n, ik, M, N, K


def empty_tables():
    nm, nn, nk = (len(BOUNDS[a]) for a in "MNK")
    return ([[[0] * nk for _ in range(nn)] for _ in range(nm)], [[[1] * nk for _ in range(nn)] for _ in range(nm)])


def from_rules():
    plan, tsplit = empty_tables()
    for im, i_n, ik, M, N, K in grid():
        path, s = rules_plan(M, N, K)
        plan[im][i_n][ik] = (PATH_CODE[path] << 4) | (s if path == "tile" else 1)
        tsplit[im][i_n][ik] = s
    return plan, tsplit


def measure(out_csv):
    import torch
    from mxfp8_block_scaled_amd import api

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev).manual_seed(1234)
    plan, tsplit = empty_tables()
    records = []
    weights = {}

    def get_weights(N, K):
        if (N, K) not in weights:
            weights.clear()
            torch.cuda.empty_cache()
            w = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            q, s = api.quantize_act(w)
            pw = api.prepare_weight(q, s)
            del w, q, s
            copies = max(1, min(64, -(-(256 << 20) // (N * K))))
            weights[(N, K)] = [pw] + [api.PreparedWeight(pw.w_packed.clone(), pw.s_packed.clone(), N, K)
                                      for _ in range(copies - 1)]
        return weights[(N, K)]

    # (N, K) outermost, so each weight is prepared once.
    order = sorted(grid(), key=lambda c: (c[1], c[2], c[0]))
    for im, i_n, ik, M, N, K in order:
        pws = get_weights(N, K)
        x = (torch.randn((M, K), generator=gen, device=dev)).to(torch.bfloat16)
        bias = (torch.randn((N,), generator=gen, device=dev) * 0.1).to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        times = {}
        for name, force in candidates(M, N, K, cus):
            prev = api.mxfp8_debug_force_path(force)
            try:
                ws = torch.empty(max(256, api.mxfp8_linear_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
                it = [0]

                def call():
                    pw = pws[it[0] % len(pws)]
                    it[0] += 1
                    st = api.mxfp8_linear(x.data_ptr(), M, K, K, pw.w_packed.data_ptr(), pw.s_packed.data_ptr(), N,
                                          bias.data_ptr(), y.data_ptr(), N, ws.data_ptr(), ws.numel(), stream)
                    if st != 0:
                        raise api.MXFP8Error(st, "mxfp8_linear")

                for _ in range(3):
                    call()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(3):
                    call()
                e1.record()
                torch.cuda.synchronize()
                est = e0.elapsed_time(e1) / 3 * 1e3
                n = max(3, min(200, int(3000.0 / max(est, 1e-3))))
                best = est
                for _ in range(3):
                    e0.record()
                    for _ in range(n):
                        call()
                    e1.record()
                    torch.cuda.synchronize()
                    best = min(best, e0.elapsed_time(e1) / n * 1e3)
                times[name] = round(best, 3)
                del ws
            finally:
                api.mxfp8_debug_force_path(prev)
        best = min(times, key=times.get)
        tiles = {k: v for k, v in times.items() if k.startswith("tile")}
        best_tile = min(tiles, key=tiles.get)
        s_best = int(best[4:]) if best.startswith("tile") else 1
        plan[im][i_n][ik] = (PATH_CODE["tile" if best.startswith("tile") else best] << 4) | s_best
        tsplit[im][i_n][ik] = int(best_tile[4:])
        rules = rules_plan(M, N, K)
        rules_name = rules[0] if rules[0] != "tile" else f"tile{rules[1]}"
        records.append({"M": M, "N": N, "K": K, "us": times, "best": best, "best_tile": best_tile,
                        "fixed_rules": rules_name, "fixed_rules_us": times.get(rules_name)})
        print(f"M={M} N={N} K={K}: best {best} {times[best]:.2f} us  (fixed rules {rules_name} "
              f"{times.get(rules_name, float('nan')):.2f} us)", flush=True)
        del x, bias, y
    props = torch.cuda.get_device_properties(dev)
    device = f"{torch.cuda.get_device_name(dev)}, {getattr(props, 'gcnArchName', '?').split(':')[0]}"
    date = datetime.date.today().isoformat()
    if out_csv:
        names = ["decode", "mid", "slab", "med128", "med64", "tile1", "tile2", "tile4", "tile8"]
        os.makedirs(os.path.dirname(os.path.abspath(out_csv)), exist_ok=True)
        with open(out_csv, "w") as f:
            f.write(f"# mxfp8_linear per GEMM path, microseconds per call ({device}, {cus} CUs, {date})\n")
            root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
            args = [os.path.relpath(a, root) if os.path.isabs(a) else a for a in sys.argv[1:]]
            f.write("# python -m mxfp8_block_scaled_amd.tune_shapes " + " ".join(args) + "\n")
            f.write("# whole call (quantization included, bias on), mean of back-to-back calls in HIP events, best "
                    "of 3 rounds, rotated weight copies; empty = path does not apply\n")
            f.write("M,N,K," + ",".join(names) + ",best,best_tile,fixed_rules\n")
            for r in records:
                f.write(f"{r['M']},{r['N']},{r['K']}," + ",".join(str(r['us'].get(n, '')) for n in names)
                        + f",{r['best']},{r['best_tile']},{r['fixed_rules']}\n")
    return plan, tsplit, f"measured on {device}, {date}"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--from-rules", action="store_true", help="no measurement: the fixed cut-offs")
    ap.add_argument("--csv", default=None, help="write every timing here")
    ap.add_argument("--inc", action="store_true", help="write the table (csrc/shape_table.inc)")
    ap.add_argument("--inc-out", default=INC, help="where --inc writes the table")
    a = ap.parse_args()
    if a.from_rules:
        plan, tsplit = from_rules()
        source = "the fixed cut-offs, no measurement"
    else:
        plan, tsplit, source = measure(a.csv)
    if a.inc:
        write_inc(plan, tsplit, source, a.inc_out)
        print("wrote", a.inc_out)


if __name__ == "__main__":
    main()
