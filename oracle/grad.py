"""The gradient of attention with respect to query, key, value and scale, in fp64, and the
log-sum-exp of the logits that the fused gradient starts from.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the page "Neural Network primitives from NNlib.jl", section "Fused implementation"
(the fused call has a gradient with respect to query, key, value and scale, which forms the
weights again; a query with no allowed key, whose output is NaN, takes no part in it; a call
with a bias takes the materialized path, which also gives the gradient with respect to the
bias) and "Arguments" (q_lengths: the output past q_lengths is zero, so it depends on no
input).

With the logits s_ij = scale * <q_i, k_j> (+ bias_ij) over the allowed keys of query i, the
weights P_i = softmax(s_i) and the output o_i = sum_j P_ij v_j, a cotangent dO of the output
propagates by the chain rule, one step at a time:

  dv_j     += sum_i P_ij dO_i                                  (o is linear in v)
  dP_ij     = <dO_i, v_j>                                      (o is linear in P)
  dS_ij     = P_ij (dP_ij - sum_j' P_ij' dP_ij')               (Jacobian of the softmax)
  dq_i      = scale * sum_j dS_ij k_j
  dk_j     += scale * sum_i dS_ij q_i
  dscale    = sum_ij dS_ij <q_i, k_j>
  dbias_ij  = dS_ij   (summed over the dims the bias broadcasts)

Under grouped-query attention a key/value head collects the sums of every query head that
reads it. Rows with no allowed key and rows at or past q_lengths contribute nothing.
"""
import numpy as np

from .sdpa import _bcast, _per_batch, allowed_matrix, causal_offsets, kv_head_of


def _prepare(q, k, v, scale, is_causal, q_offset, kv_lengths, q_lengths):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Lq, Hq, D = q.shape
    Lkv, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or v.shape[:3] != k.shape[:3] or k.shape[3] != D or Hq % Hkv:
        raise ValueError("q/k/v shapes do not agree")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    kvl = [min(max(t, 0), Lkv) for t in _per_batch(kv_lengths, B, Lkv)]
    ql = [min(max(t, 0), Lq) for t in _per_batch(q_lengths, B, Lq)]
    offs = causal_offsets(is_causal, q_offset, None if kv_lengths is None else kvl,
                          None if q_lengths is None else ql, B, Lq, Lkv)
    return q, k, v, float(scale), kvl, ql, offs


def _logits(q, k, b, h, g, scale, bias, mask, offs, kvl, B, Hq):
    """Logits [Lq][Lkv] of (b, h) with -inf at the keys the query may not attend."""
    Lq, Lkv = q.shape[1], k.shape[1]
    s = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
    if bias is not None:
        plane = _bcast(bias, b, h, B, Hq)
        s = s + np.broadcast_to(plane, (Lq, Lkv))
    allowed = allowed_matrix(np.arange(Lq), Lkv, b, h, B, Hq, mask,
                             None if offs is None else offs[b], kvl[b])
    return np.where(allowed, s, -np.inf), allowed


def sdpa_lse(q, k, v, bias=None, mask=None, scale=None, is_causal=False, q_offset=0,
             kv_lengths=None, q_lengths=None):
    """Natural-log log-sum-exp of the allowed logits, [B][Hq][Lq] fp64.

    -inf for a query with no allowed key and for the queries at or past q_lengths (they attend
    nothing: their output is NaN or zero). exp(s_ij - lse_i) are then the weights.
    """
    q, k, v, scale, kvl, ql, offs = _prepare(q, k, v, scale, is_causal, q_offset, kv_lengths, q_lengths)
    B, Lq, Hq, _ = q.shape
    Hkv = k.shape[2]
    mask = None if mask is None else np.asarray(mask)
    bias = None if bias is None else np.asarray(bias, dtype=np.float64)
    lse = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            s, allowed = _logits(q, k, b, h, kv_head_of(h, Hq, Hkv), scale, bias, mask, offs, kvl, B, Hq)
            allowed &= s > -np.inf
            for i in range(ql[b]):
                if allowed[i].any():
                    m = s[i][allowed[i]].max()
                    lse[b, h, i] = m + np.log(np.sum(np.exp(s[i][allowed[i]] - m)))
    return lse


def sdpa_grad(q, k, v, dout, bias=None, mask=None, scale=None, is_causal=False, q_offset=0,
              kv_lengths=None, q_lengths=None):
    """Cotangents of q, k, v, scale (and bias) for the output cotangent ``dout``.

    dout [B][Lq][Hq][Dv]. Returns a dict with dq [B][Lq][Hq][D], dk [B][Lkv][Hkv][D],
    dv [B][Lkv][Hkv][Dv], dscale (float) and, with a bias, dbias of the bias's own shape.
    dscale_abs is the sum of the magnitudes of dscale's terms: the terms of each row cancel (its
    dS sums to zero), so a rounding error in dscale is measured against this sum.
    """
    q, k, v, scale, kvl, ql, offs = _prepare(q, k, v, scale, is_causal, q_offset, kv_lengths, q_lengths)
    dout = np.asarray(dout, dtype=np.float64)
    B, Lq, Hq, D = q.shape
    Hkv = k.shape[2]
    mask = None if mask is None else np.asarray(mask)
    bias = None if bias is None else np.asarray(bias, dtype=np.float64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dbias = None if bias is None else np.zeros_like(bias)
    dscale = dscale_abs = 0.0
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s, allowed = _logits(q, k, b, h, g, scale, bias, mask, offs, kvl, B, Hq)
            allowed &= s > -np.inf               # a bias of -inf masks too
            # rows that take part: inside q_lengths, with at least one allowed key
            part = allowed.any(axis=1) & (np.arange(Lq) < ql[b])
            P = np.zeros_like(s)
            for i in np.nonzero(part)[0]:
                e = np.where(allowed[i], np.exp(s[i] - s[i][allowed[i]].max()), 0.0)
                P[i] = e / e.sum()
            dO = np.where(part[:, None], dout[b, :, h, :], 0.0)
            keep = (np.arange(k.shape[1]) < kvl[b])[:, None]   # rows past kv_lengths: padding
            V, K, Q = np.where(keep, v[b, :, g, :], 0.0), np.where(keep, k[b, :, g, :], 0.0), q[b, :, h, :]
            dv[b, :, g, :] += P.T @ dO
            dP = np.where(allowed, dO @ V.T, 0.0)     # keys that are not attended take no part
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[b, :, h, :] = scale * (dS @ K)
            dk[b, :, g, :] += scale * (dS.T @ Q)
            terms = np.where(allowed, dS * (Q @ K.T), 0.0)
            dscale += float(np.sum(terms))
            dscale_abs += float(np.sum(np.abs(terms)))
            if dbias is not None:
                d = dS.sum(axis=0, keepdims=True) if bias.shape[2] == 1 else dS
                d = d.sum(axis=1, keepdims=True) if bias.shape[3] == 1 else d
                dbias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0] += d
    out = {"dq": dq, "dk": dk, "dv": dv, "dscale": dscale, "dscale_abs": dscale_abs}
    if dbias is not None:
        out["dbias"] = dbias
    return out
