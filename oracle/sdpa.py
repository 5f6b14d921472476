"""Scaled dot-product attention as its plain, materialized definition, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the page "Neural Network primitives from NNlib.jl", section "Attention", its
"Arguments" list and the section "Fused implementation". For batch b, query head h
and query i:

  1. (optional) per-head RMS norm of every query and key vector (TensorTonic page
     "Static Arguments in jit"), eps 1e-6; values are not normalised;
  2. logits s_ij = scale * <q_i, k_j>; scale defaults to 1/sqrt(qk_head_dim) and
     multiplies the dot products only ("Arguments": scale);
  3. s_ij += bias[b, h, i, j] when a bias is given, broadcasting dims of size 1
     ("Arguments": bias); the bias is not scaled;
  4. key j is allowed when every given condition allows it ("Arguments", the rule that
     mask, is_causal and kv_lengths combine by AND):
       mask[b, h, i, j] is true;
       is_causal: j <= off_b + i, with off_b = q_offset (true) or
                  kv_len_b - q_len_b (:bottom_right, sizes of the arrays where the
                  lengths are not given);
       kv_lengths: j < kv_lengths[b];
  5. softmax over the allowed keys, then the weighted sum of the value rows. A query
     with no allowed key has output NaN ("Fused implementation"); queries at or past
     q_lengths[b] have output 0 ("Arguments": q_lengths).

Grouped-query attention ("Attention"): k and v have Hkv heads, Hq is a multiple of
Hkv, and query head h reads K/V head floor(h / (Hq/Hkv)), i.e. each K/V head serves a
contiguous run of query heads (the pages only say the heads are shared; this reading
equals repeating every K/V head Hq/Hkv times in a row).

Layout: q [B][Lq][Hq][D], k [B][Lkv][Hkv][D], v [B][Lkv][Hkv][Dv] (the NNlib
column-major (head_dim, heads, seq, batch) order, stored C-order); bias and mask are
[B][H][Lq][Lkv] or broadcastable to it. Output [B][Lq][Hq][Dv].

The weights of one query row are formed whole (the materialized implementation of the
"Fused implementation" section); rows are processed in chunks only to bound memory.
"""
import numpy as np

from .rms_norm import rms_rows

_CHUNK_ELEMS = 1 << 23        # logits per chunk: 64 MiB of fp64


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """K/V head read by query head h under grouped-query attention."""
    return h // (Hq // Hkv)


def _per_batch(x, B, default):
    """An int, None or [B] array -> list of B python ints (None -> default)."""
    if x is None:
        return [default] * B
    a = np.asarray(x).reshape(-1)
    if a.size == 1:
        return [int(a[0])] * B
    if a.size != B:
        raise ValueError("per-batch argument needs one entry per batch element")
    return [int(t) for t in a]


def causal_offsets(is_causal, q_offset, kv_lengths, q_lengths, B, Lq, Lkv):
    """off_b of the causal rule j <= off_b + i, or None when not causal."""
    if is_causal is False or is_causal is None:
        return None
    if is_causal is True:
        return _per_batch(q_offset, B, 0)
    if is_causal == "bottom_right":
        kvl = _per_batch(kv_lengths, B, Lkv)
        ql = _per_batch(q_lengths, B, Lq)
        return [kvl[b] - ql[b] for b in range(B)]
    raise ValueError("is_causal must be False, True or 'bottom_right'")


def _bcast(a, b, h, B, H):
    """The [Lq][Lkv] plane of a [Bb][Hb][Lq][Lkv] array for (b, h), honouring size-1 dims."""
    if a.ndim != 4:
        raise ValueError("bias/mask must be 4-D [B][H][Lq][Lkv] (size-1 dims broadcast)")
    if a.shape[0] not in (1, B) or a.shape[1] not in (1, H):
        raise ValueError("bias/mask batch/head dims must be 1 or full")
    return a[b if a.shape[0] > 1 else 0, h if a.shape[1] > 1 else 0]


def allowed_matrix(rows, Lkv, b, h, B, H, mask, off, kv_len):
    """Boolean [len(rows)][Lkv]: which keys each query row may attend (AND of the conditions)."""
    rows = np.asarray(rows)
    j = np.arange(Lkv)[None, :]
    allowed = np.ones((rows.size, Lkv), dtype=bool)
    if mask is not None:
        plane = _bcast(mask, b, h, B, H)
        if plane.shape[0] == 1:
            allowed &= plane[0][None, :] != 0
        else:
            allowed &= plane[rows] != 0
    if off is not None:
        allowed &= j <= off + rows[:, None]
    if kv_len is not None:
        allowed &= j < kv_len
    return allowed


def sdpa(q, k, v, bias=None, mask=None, scale=None, is_causal=False, q_offset=0,
         kv_lengths=None, q_lengths=None, qk_norm=False, rows=None, return_weights=False):
    """fp64 attention output [B][n][Hq][Dv] for query rows ``rows`` (default: all).

    q, k, v: float arrays (bf16 inputs are passed as their exact float values).
    bias: float [Bb][Hb][Lq][Lkv] or None. mask: bool/uint8 of the same kind or None.
    scale: None means 1/sqrt(qk_head_dim). is_causal: False, True or "bottom_right".
    q_offset: int or [B]. kv_lengths, q_lengths: None, int or [B]; they are clamped to
    [0, Lkv] and [0, Lq] (the pages do not say what lengths beyond the arrays mean). ``return_weights`` also returns the weights [B][Hq][n][Lkv] (small shapes).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Lq, Hq, D = q.shape
    Bk, Lkv, Hkv, Dk = k.shape
    Bv, Lv, Hv, Dv = v.shape
    if Dk != D or (Bk, Bv) != (B, B) or Lv != Lkv or Hv != Hkv:
        raise ValueError("q/k/v shapes do not agree")
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    kvl = None if kv_lengths is None else [min(max(t, 0), Lkv) for t in _per_batch(kv_lengths, B, Lkv)]
    ql = None if q_lengths is None else [min(max(t, 0), Lq) for t in _per_batch(q_lengths, B, Lq)]
    offs = causal_offsets(is_causal, q_offset, kvl, ql, B, Lq, Lkv)
    if qk_norm:
        q = rms_rows(q)
        k = rms_rows(k)
    bias64 = None if bias is None else np.asarray(bias)
    mask_a = None if mask is None else np.asarray(mask)

    out = np.zeros((B, rows.size, Hq, Dv), dtype=np.float64)
    weights = np.zeros((B, Hq, rows.size, Lkv)) if return_weights else None
    chunk = max(1, _CHUNK_ELEMS // max(Lkv, 1))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            # keys past kv_lengths are padding: they are not part of the key set at all
            n = Lkv if kvl is None else kvl[b]
            K = k[b, :n, g, :]
            V = v[b, :n, g, :]
            for c0 in range(0, rows.size, chunk):
                r = rows[c0:c0 + chunk]
                s = scale * (q[b, r, h, :] @ K.T)                       # step 2
                if bias64 is not None:                                  # step 3
                    plane = _bcast(bias64, b, h, B, Hq)
                    plane = plane[0][None, :] if plane.shape[0] == 1 else plane[r]
                    s = s + plane[:, :n].astype(np.float64)
                allowed = allowed_matrix(r, Lkv, b, h, B, Hq, mask_a,   # step 4
                                         None if offs is None else offs[b],
                                         None if kvl is None else kvl[b])[:, :n]
                s = np.where(allowed, s, -np.inf)
                m = np.max(s, axis=1, keepdims=True) if n else np.full((r.size, 1), -np.inf)
                none = ~np.isfinite(m[:, 0]) & (m[:, 0] < 0)           # no allowed key (or all -inf)
                p = np.exp(s - np.where(none[:, None], 0.0, m))         # step 5
                p[~allowed] = 0.0
                l = p.sum(axis=1, keepdims=True)
                o = (p @ V) / np.where(l > 0, l, 1.0)
                o[none] = np.nan
                if ql is not None:
                    o[r >= ql[b]] = 0.0
                out[b, c0:c0 + r.size, h, :] = o
                if return_weights:
                    w = p / np.where(l > 0, l, 1.0)
                    w[none] = np.nan
                    weights[b, h, c0:c0 + r.size, :n] = w
    return (out, weights) if return_weights else out
