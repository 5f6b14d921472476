"""Rounding budget of the matrix-core prefill, modelled on the CPU (no GPU, no HIP code).

The fused forward kernel takes three roundings that the fp64 definition does not:

* fold: without bias and QK-norm, scale * log2(e) is multiplied into q once and the product is
  rounded to bf16, so the q.k products emit log2-unit logits directly;
* P: the probabilities are rounded to bf16, the operand type of the P.V products (the row sum
  uses the same rounded values);
* output: a bf16 output is rounded once more at the end.

Each step is applied alone, and then together, to the definition (page "Neural Network
primitives from NNlib.jl", section "Attention": softmax of the scaled logits over the allowed
keys, times v) on three (batch, head) slices of the causal bf16 prefill workload, B4 H16 D128
L4096. The modelled errors are what the GPU parity tests measure on the whole output at that
size (relative L2 about 2.0e-3 with an fp32 output and 2.55e-3 with a bf16 output), so the
kernel's error is these three roundings and nothing else. The test holds the budget: the fold
and the bf16 probabilities together stay at or below 2.5e-3 relative L2 (fp32 output), and all
three within the bf16 bar of 5e-3.
"""
import numpy as np

import workloads as W


def _bf16(x):
    """Round to bf16 (nearest, ties to even) through fp32, back to float64."""
    return W.bf16_to_f32(W.f32_to_bf16(np.asarray(x, dtype=np.float32))).astype(np.float64)


def _causal_attention(s2, v, round_p):
    """Softmax over the causal keys of log2-unit logits s2, times v (the row sum over the same,
    possibly rounded, probabilities)."""
    L = s2.shape[0]
    s2 = np.where(np.tril(np.ones((L, L), dtype=bool)), s2, -np.inf)
    p = np.exp2(s2 - s2.max(axis=1, keepdims=True))
    if round_p:
        p = _bf16(p)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def test_prefill_rounding_budget():
    w = W.causal_prefill()
    q, k, v = (W.widen(getattr(w, n), "bf16") for n in ("q", "k", "v"))
    c = w.scale * np.log2(np.e)
    names = ("fold", "p", "fold+p", "out", "all")
    sq = dict.fromkeys(names, 0.0)
    ref2 = 0.0
    for b, h in ((0, 0), (1, 5), (3, 15)):
        qq, kk, vv = (x[b, :, h].astype(np.float64) for x in (q, k, v))
        s_exact = (qq @ kk.T) * c
        s_fold = _bf16(qq.astype(np.float32) * np.float32(c)) @ kk.T
        o = _causal_attention(s_exact, vv, False)
        got = {"fold": _causal_attention(s_fold, vv, False), "p": _causal_attention(s_exact, vv, True)}
        got["fold+p"] = _causal_attention(s_fold, vv, True)
        got["out"] = _bf16(o)
        got["all"] = _bf16(got["fold+p"])
        ref2 += float(np.sum(o * o))
        for n in names:
            sq[n] += float(np.sum((got[n] - o) ** 2))
    rel = {n: float(np.sqrt(sq[n] / ref2)) for n in names}
    print("modelled relative L2:", {n: f"{r:.3e}" for n, r in rel.items()})
    # each rounding alone is of the size of half a bf16 ulp spread over the sums
    for n in ("fold", "p", "out"):
        assert 5e-4 < rel[n] < 2.5e-3, (n, rel[n])
    assert rel["fold+p"] <= 2.5e-3
    assert rel["all"] <= 5e-3
