"""Pins of the oracle's routed MoE layer (CPU only)."""

import numpy as np
import torch

import oracle
from mxfp8_block_scaled_amd import synth
from tests import pins


def test_routing_topk_then_softmax():
    logits = np.array([[0.5, 2.0, -1.0, 2.0, 1.0],
                       [0.0, 0.0, 0.0, 0.0, 0.0]])
    ids, w = oracle.route_topk_softmax(logits, 3)
    # ties go to the lower expert id
    assert ids.tolist() == [[1, 3, 4], [0, 1, 2]]
    e = np.exp([2.0, 2.0, 1.0])
    assert np.allclose(w[0], e / e.sum(), rtol=0, atol=1e-15)
    assert np.allclose(w[1], [1 / 3] * 3, rtol=0, atol=1e-15)


def test_routing_matches_torch_topk_on_distinct_logits():
    g = torch.Generator().manual_seed(1)
    logits = torch.randn(64, 128, generator=g)
    ids, w = oracle.route_topk_softmax(logits.double().numpy(), 8)
    tv, ti = torch.topk(logits.double(), 8, dim=1)
    assert np.array_equal(ids, ti.numpy())
    assert np.allclose(w, torch.softmax(tv, dim=1).numpy(), rtol=0, atol=1e-15)


def _dense_moe_via_linear(x, logits, w13q, w13s, w2q, w2s, topk):
    """The same layer composed from the already pinned dense linear oracle,
    one (token, slot) at a time: an independent route through the arithmetic."""
    T, H = x.shape
    inter = w13q.shape[1] // 2
    ids, wts = oracle.route_topk_softmax(logits, topk)
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            h = oracle.linear_ref(x[t:t + 1], w13q[e], w13s[e])[0]
            gate, up = h[:inter], h[inter:]
            a = oracle.bf16_round(torch.nn.functional.silu(torch.from_numpy(gate)).numpy() * up)
            y[t] += wts[t, j] * oracle.linear_ref(a[None, :], w2q[e], w2s[e])[0]
    return y


def test_moe_matches_per_token_composition():
    T, H, E, k, inter = 6, 256, 5, 2, 256
    x, logits, w13, w2 = synth.moe_inputs(T, H, E, k, inter, seed=3)
    w13q = np.stack([oracle.quantize_mx(w13[e].double().numpy())[0] for e in range(E)])
    w13s = np.stack([oracle.quantize_mx(w13[e].double().numpy())[1] for e in range(E)])
    w2q = np.stack([oracle.quantize_mx(w2[e].double().numpy())[0] for e in range(E)])
    w2s = np.stack([oracle.quantize_mx(w2[e].double().numpy())[1] for e in range(E)])
    xd, ld = x.double().numpy(), logits.double().numpy()
    y = oracle.moe_ref(xd, ld, w13q, w13s, w2q, w2s, k)
    y2 = _dense_moe_via_linear(xd, ld, w13q, w13s, w2q, w2s, k)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_moe_single_expert_one_hot_closed_form():
    """E=1, top-1 (weight 1): with W13 = [I_gate; c * I_up] and W2 = identity
    block, y = bf16(silu(a) * c*a) requantized: check against a hand-built
    chain of pinned pieces."""
    H = inter = 256
    x = torch.linspace(-2, 2, H).to(torch.bfloat16)[None, :]
    w13 = np.zeros((1, 2 * inter, H))
    w13[0, :inter] = np.eye(H)
    w13[0, inter:] = 0.5 * np.eye(H)
    w2 = np.eye(H)[None]
    q13, s13 = oracle.quantize_mx(w13[0])
    q2, s2 = oracle.quantize_mx(w2[0])
    y = oracle.moe_ref(x.double().numpy(), np.zeros((1, 1)), q13[None], s13[None], q2[None], s2[None], 1)
    qa, sa = pins.library_quantize(x)
    a = pins.torch_e4m3_values(qa) * np.repeat(2.0 ** (sa.astype(np.int64) - 127), 32, 1)
    act = oracle.bf16_round(torch.nn.functional.silu(torch.from_numpy(a)).numpy() * (0.5 * a))
    qb, sb = pins.library_quantize(torch.from_numpy(act).to(torch.bfloat16))
    exp = pins.torch_e4m3_values(qb) * np.repeat(2.0 ** (sb.astype(np.int64) - 127), 32, 1)
    assert np.allclose(y, exp, rtol=0, atol=0)


def test_silu_pinned():
    """The oracle's SiLU against torch's float64 SiLU, the odd-part identity
    and a closed form (tests/pins.py check_silu)."""
    pins.check_silu(oracle.moe.silu)
