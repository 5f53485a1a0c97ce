"""Offline conversion of a bf16 checkpoint's linear weights to MXFP8 or MXFP4.

The pages serve an MXFP8 model that was converted from its bf16 release
offline, before the server starts ([SGL#18945] "Add support for FlashInfer
mxfp8", §Benchmarking and Profiling: the set-up that converts the checkpoint);
the conversion is the same MX quantization as the activations', applied once
to the stored weights.

    python -m mxfp8_block_scaled_amd.convert IN.safetensors OUT.safetensors \
        [--format mxfp8|mxfp4] [--include REGEX] [--device cuda:0]

Every 2-D bf16 tensor whose name matches ``--include`` (default: names ending
in ``weight``) and whose last dimension is a multiple of 32 is quantized on
the GPU by the library's MX quantizer (mxfp8_quantize_act for E4M3 elements,
mxfp8_quantize_fp4 for E2M1 elements packed two per byte) and written as two
uint8 tensors, ``<name>.qdata`` ([N, K] E4M3 bytes, or [N, K/2] E2M1 pairs)
and ``<name>.scale`` ([N, K/32] UE8M0); the file's metadata records the
format.  Everything else is copied unchanged.  The checkpoint is read with
safetensors (no pickle).  The outputs are what ``prepare_weight`` and
``prepare_weight_fp4`` take.
"""

import argparse
import re

import torch


def convert(src, dst, fmt="mxfp8", include=r"weight$", device="cuda:0"):
    from safetensors import safe_open
    from safetensors.torch import save_file

    from . import api

    pat = re.compile(include)
    out = {}
    converted = []
    with safe_open(src, framework="pt", device="cpu") as f:
        meta = dict(f.metadata() or {})
        for name in f.keys():
            t = f.get_tensor(name)
            if t.dtype == torch.bfloat16 and t.dim() == 2 and t.shape[1] % 32 == 0 and pat.search(name):
                x = t.to(device)
                q, s = api.quantize_act(x) if fmt == "mxfp8" else api.quantize_fp4(x)
                out[name + ".qdata"] = q.cpu()
                out[name + ".scale"] = s.cpu()
                converted.append(name)
            else:
                out[name] = t
    meta["mx_format"] = fmt
    meta["mx_converted"] = ",".join(converted)
    save_file(out, dst, metadata=meta)
    return converted


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("src")
    p.add_argument("dst")
    p.add_argument("--format", choices=["mxfp8", "mxfp4"], default="mxfp8")
    p.add_argument("--include", default=r"weight$")
    p.add_argument("--device", default="cuda:0")
    a = p.parse_args(argv)
    names = convert(a.src, a.dst, a.format, a.include, a.device)
    print(f"converted {len(names)} tensors to {a.format}")


if __name__ == "__main__":
    main()
