"""Top-k routed MXFP8 mixture-of-experts layer, in plain numpy float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed, and where it is defined
-----------------------------------------
* Routing "Renormalize (TopK -> Softmax)": take the k largest router logits of
  a token, then a softmax over just those k (flashinfer PR #1214, "Highlights",
  flexible routing methods).  Ties between equal logits go to the lower
  expert id (a reading: the page does not order ties).
* Per selected expert: a fused gate/up projection ``[2I, H]`` on the
  MX-quantized token, SiLU-gating, a down projection ``[H, I]`` on the
  MX-quantized gated activation, then the routing-weighted sum over the k
  experts (the BF16-activations-in, routed-expert pipeline of flashinfer PR
  #4026's walkthrough; the fused w13 / w2 expert weights of sglang PR #18945's
  FlashInfer CUTLASS MXFP8 MoE changes).
* Readings (each listed in the design doc): rows ``[0, I)`` of w13 are the gate and
  rows ``[I, 2I)`` the up projection; ``act = silu(gate) * up`` with
  ``silu(z) = z / (1 + exp(-z))``; the gated activation is rounded to bf16
  before it is MX-quantized along I; the combined output is what the caller
  rounds to bf16.
"""

import numpy as np

from .mx import bf16_round, dequantize_mx, quantize_mx


def route_topk_softmax(logits, topk):
    """``logits[T, E]`` -> ``(ids[T, topk] int64, weights[T, topk] float64)``.

    ids are ordered by descending logit, ties by ascending expert id."""
    logits = np.asarray(logits, dtype=np.float64)
    order = np.lexsort((np.broadcast_to(np.arange(logits.shape[1]), logits.shape),
                        -logits), axis=1)
    ids = order[:, :topk]
    sel = np.take_along_axis(logits, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids.astype(np.int64), z / z.sum(axis=1, keepdims=True)


def silu(z):
    return z / (1.0 + np.exp(-z))


def moe_ref(x, logits, w13_q, w13_s, w2_q, w2_s, topk, act_override=None,
            return_act=False):
    """MXFP8 MoE forward, unrounded (float64).

    x        [T, H]        real activations (bf16 values)
    logits   [T, E]        router logits (fp32 values)
    w13_q/s  [E, 2I, H] / [E, 2I, H/32]   gate rows then up rows, MXFP8
    w2_q/s   [E, H, I]  / [E, H, I/32]    MXFP8
    act_override  optional [T*topk, I] bf16-valued gated activations, indexed
             by (token, slot) = t * topk + j, used instead of the oracle's own
             (the "staged" comparison: makes the requantization bit-exact
             against an external intermediate).
    Returns ``y[T, H]`` float64 (and, when ``return_act``, the bf16-rounded
    gated activations ``[T*topk, I]`` and the routing ids / weights).
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E, two_i, _ = w13_q.shape
    inter = two_i // 2
    ids, wts = route_topk_softmax(logits, topk)
    qx, sx = quantize_mx(x)
    xd = dequantize_mx(qx, sx)
    act = np.zeros((T * topk, inter), dtype=np.float64)
    y = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        tok, slot = np.nonzero(ids == e)
        if tok.size == 0:
            continue
        w13 = dequantize_mx(w13_q[e], w13_s[e])
        h = xd[tok] @ w13.T
        a = bf16_round(silu(h[:, :inter]) * h[:, inter:])
        rows = tok * topk + slot
        if act_override is not None:
            a = np.asarray(act_override, dtype=np.float64)[rows]
        act[rows] = a
        qa, sa = quantize_mx(a)
        w2 = dequantize_mx(w2_q[e], w2_s[e])
        ye = dequantize_mx(qa, sa) @ w2.T
        y[tok] += wts[tok, slot][:, None] * ye
    if return_act:
        return y, act, ids, wts
    return y
