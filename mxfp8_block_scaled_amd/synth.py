"""Seeded synthetic inputs for the MXFP8 linear layer and the MoE layer.

This module only draws random numbers (torch CPU generators, so every machine
gets the same bytes) and casts them to bf16 by round-to-nearest-even.  It holds
none of the layer's arithmetic; the HIP path and the CPU oracle both consume
what it returns.

Workloads (sizes and distributions of the layer's benchmark shapes):

  1 "single"      M=7, N=130 (physically padded to 256), K=256; x ~ N(0,1),
                  W ~ N(0,0.02), bias ~ N(0,0.1); seed 0.
  2 "decode"      M in {1,7,16,128}, N=K=4096; x ~ N(0,1) with a Bernoulli(0.01)
                  element mask scaled x50 (applied in fp32 before the bf16
                  cast); W ~ N(0,0.02); bias ~ N(0,0.1); seed 1.  W and bias
                  are drawn first and shared by all M; x for each M comes from
                  its own generator seeded 1 * 100003 + M.
  3 "prefill_qkv" M=16384, N=5120, K=2048; x ~ N(0,1); W ~ N(0,0.02); no bias;
                  seed 2.
  4 "large"       M=8192, N=28672, K=8192; x ~ N(0,1); W ~ N(0,0.01);
                  bias ~ N(0,0.1); seed 3.
  5 "moe"         T=4096 tokens, H=2048, E=128 experts, top-8, I=768;
                  x ~ N(0,1); router logits fp32 ~ N(0,1); w13 [E, 2I, H] and
                  w2 [E, H, I] ~ N(0,0.02); seed 4.

Draw order inside one generator: x, (outlier mask), W, bias; MoE: x, logits,
w13, w2.

Every function takes ``device``: "cpu" (default) draws with torch's CPU
generator, so tests and the oracle see the same bytes on every machine; a GPU
device draws the same distributions with that device's generator (a
different random stream), which the benchmark uses to create its
multi-gigabyte inputs in place.
"""

import torch

LINEAR_CONFIGS = {
    1: dict(name="single", M=7, N=130, K=256, x_std=1.0, w_std=0.02, bias_std=0.1, seed=0),
    2: dict(name="decode", Ms=(1, 7, 16, 128), N=4096, K=4096, x_std=1.0, w_std=0.02,
            bias_std=0.1, outlier_frac=0.01, outlier_scale=50.0, seed=1),
    3: dict(name="prefill_qkv", M=16384, N=5120, K=2048, x_std=1.0, w_std=0.02,
            bias_std=None, seed=2),
    4: dict(name="large", M=8192, N=28672, K=8192, x_std=1.0, w_std=0.01, bias_std=0.1,
            seed=3),
}

MOE_CONFIG = dict(name="moe", T=4096, H=2048, E=128, topk=8, I=768, x_std=1.0,
                  logit_std=1.0, w_std=0.02, seed=4)


def _gen(seed, device="cpu"):
    return torch.Generator(device=device).manual_seed(int(seed))


def randn_bf16(shape, std, gen):
    """N(0, std^2) drawn in fp32, cast to bf16 (RNE)."""
    return (torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device) * std).to(torch.bfloat16)


def activations(M, K, std, gen, outlier_frac=0.0, outlier_scale=1.0):
    x = torch.randn(M, K, generator=gen, dtype=torch.float32, device=gen.device) * std
    if outlier_frac > 0:
        mask = torch.rand(M, K, generator=gen, device=gen.device) < outlier_frac
        x = torch.where(mask, x * outlier_scale, x)
    return x.to(torch.bfloat16)


def linear_inputs(M, N, K, seed, x_std=1.0, w_std=0.02, bias_std=0.1,
                  outlier_frac=0.0, outlier_scale=1.0, device="cpu"):
    """(x bf16 [M,K], W bf16 [N,K], bias bf16 [N] or None) on ``device``."""
    g = _gen(seed, device)
    x = activations(M, K, x_std, g, outlier_frac, outlier_scale)
    w = randn_bf16((N, K), w_std, g)
    bias = randn_bf16((N,), bias_std, g) if bias_std else None
    return x, w, bias


def config_inputs(cfg, M=None, device="cpu"):
    """Inputs of one linear workload; for "decode" pass the M of the sweep."""
    c = LINEAR_CONFIGS[cfg]
    if cfg == 2:
        if M is None:
            raise ValueError("the decode workload needs M")
        w, bias = decode_weight(cfg, device)
        x = activations(M, c["K"], c["x_std"], _gen(c["seed"] * 100003 + M, device),
                        c["outlier_frac"], c["outlier_scale"])
        return x, w, bias
    return linear_inputs(c["M"], c["N"], c["K"], c["seed"], c["x_std"], c["w_std"],
                         c["bias_std"], device=device)


def decode_weight(cfg=2, device="cpu"):
    """Just the shared (W, bias) of the decode workload, drawn as config_inputs
    draws them."""
    c = LINEAR_CONFIGS[cfg]
    g = _gen(c["seed"], device)
    w = randn_bf16((c["N"], c["K"]), c["w_std"], g)
    bias = randn_bf16((c["N"],), c["bias_std"], g)
    return w, bias


def scale_stress(t, seed, block=32, lo=-16, hi=16):
    """Multiply every run of ``block`` consecutive elements along the last dim
    by 2^r, r ~ U{lo..hi} (exact in bf16 for these magnitudes).  Spreads the
    blocks over many scale exponents so that a permuted or misindexed scale
    cannot hide behind two dominant exponents."""
    g = _gen(seed)
    rows, cols = t.shape
    r = torch.randint(lo, hi + 1, (rows, cols // block), generator=g)
    f = torch.pow(2.0, r.to(torch.float32)).repeat_interleave(block, dim=1)
    return (t.to(torch.float32) * f).to(t.dtype)


def moe_inputs(T=None, H=None, E=None, topk=None, inter=None, seed=None, w_std=None, device="cpu"):
    """(x bf16 [T,H], logits fp32 [T,E], w13 bf16 [E,2I,H], w2 bf16 [E,H,I]) on ``device``."""
    c = dict(MOE_CONFIG)
    T = T or c["T"]
    H = H or c["H"]
    E = E or c["E"]
    inter = inter or c["I"]
    seed = c["seed"] if seed is None else seed
    w_std = w_std or c["w_std"]
    g = _gen(seed, device)
    x = randn_bf16((T, H), c["x_std"], g)
    logits = torch.randn(T, E, generator=g, dtype=torch.float32, device=g.device) * c["logit_std"]
    w13 = randn_bf16((E, 2 * inter, H), w_std, g)
    w2 = randn_bf16((E, H, inter), w_std, g)
    return x, logits, w13, w2
