"""Scalar pure-Python attention for tiny shapes (oracle; test infrastructure only).

A second implementation of the definition in ``oracle/sdpa.py`` (page "Neural Network
primitives from NNlib.jl", sections "Attention" and "Arguments"), written with Python
floats, ``math.exp`` and explicit loops over every index and no numpy arithmetic, so
that it shares no vectorised step with the fp64 oracle it checks. The K/V head of a
query head is found by repeating every K/V head Hq/Hkv times in a list, which is the
explicit form of grouped-query sharing.

Use it for shapes up to a few thousand logits; it is slow on purpose.
"""
import math


def _lst(x):
    return None if x is None else (x.tolist() if hasattr(x, "tolist") else x)


def _entry(a4, b, h, i, j):
    """a4[b][h][i][j] with size-1 dims broadcast."""
    pb = a4[b if len(a4) > 1 else 0]
    ph = pb[h if len(pb) > 1 else 0]
    pi = ph[i if len(ph) > 1 else 0]
    return pi[j if len(pi) > 1 else 0]


def _normalise(vec, eps=1e-6):
    ms = sum(x * x for x in vec) / len(vec)
    d = math.sqrt(ms + eps)
    return [x / d for x in vec]


def sdpa_brute(q, k, v, bias=None, mask=None, scale=None, is_causal=False, q_offset=0,
               kv_lengths=None, q_lengths=None, qk_norm=False):
    """Same arguments and result layout as ``oracle.sdpa`` (returns nested lists)."""
    q, k, v = _lst(q), _lst(k), _lst(v)
    bias, mask = _lst(bias), _lst(mask)
    B, Lq, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Lkv, Hkv, Dv = len(k[0]), len(k[0][0]), len(v[0][0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)

    def per_b(x, default):
        if x is None:
            return [default] * B
        if isinstance(x, int):
            return [x] * B
        x = list(_lst(x))
        return [int(x[0])] * B if len(x) == 1 else [int(t) for t in x]

    kvl = per_b(kv_lengths, Lkv)
    kvl = [min(max(t, 0), Lkv) for t in kvl]
    ql = [min(max(t, 0), Lq) for t in per_b(q_lengths, Lq)]
    head_list = []                       # explicit repetition of every K/V head
    for g in range(Hkv):
        head_list += [g] * (Hq // Hkv)

    out = [[[[0.0] * Dv for _ in range(Hq)] for _ in range(Lq)] for _ in range(B)]
    for b in range(B):
        if is_causal == "bottom_right":
            off = kvl[b] - ql[b]
        elif is_causal:
            off = per_b(q_offset, 0)[b]
        else:
            off = None
        for i in range(Lq):
            for h in range(Hq):
                g = head_list[h]
                qi = q[b][i][h]
                if qk_norm:
                    qi = _normalise(qi)
                logits = []
                for j in range(Lkv):
                    ok = j < kvl[b]
                    if off is not None and j > off + i:
                        ok = False
                    if mask is not None and not _entry(mask, b, h, i, j):
                        ok = False
                    if not ok:
                        logits.append(None)
                        continue
                    kj = k[b][j][g]
                    if qk_norm:
                        kj = _normalise(kj)
                    dot = 0.0
                    for d in range(D):
                        dot += qi[d] * kj[d]
                    s = scale * dot
                    if bias is not None:
                        s += float(_entry(bias, b, h, i, j))
                    logits.append(s)
                if i >= ql[b]:
                    continue                                 # zero output past q_lengths
                finite = [s for s in logits if s is not None and s != -math.inf]
                if not finite:
                    out[b][i][h] = [math.nan] * Dv
                    continue
                m = max(finite)
                num = [0.0] * Dv
                den = 0.0
                for j, s in enumerate(logits):
                    if s is None or s == -math.inf:
                        continue
                    w = math.exp(s - m)
                    den += w
                    for d in range(Dv):
                        num[d] += w * v[b][j][g][d]
                out[b][i][h] = [x / den for x in num]
    return out
