"""Attention over packed sequences, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the page "Neural Network primitives from NNlib.jl", section "Packed sequences", and
its "Arguments" entries q_segments, kv_segments and maxlen. The inputs hold sequences one
after the other along the sequence dimension, with no batch dimension. Segment s of the
queries attends segment s of the keys and values only, as batch element s of a padded batch
would: the causal rule, q_offset, q_lengths and kv_lengths apply within the segment, with one
entry per segment. kv_segments defaults to q_segments; the lengths have to add up to the
arrays' sequence lengths; a bias or a mask is not supported; maxlen only bounds the segment
lengths and changes nothing in the result.

Each segment is computed here as its own call of the plain definition (``oracle.sdpa`` with
batch 1), and its output rows are placed at the segment's rows.
"""
import numpy as np

from .sdpa import sdpa


def _entry(x, s):
    """Entry s of a per-segment argument (an int applies to every segment)."""
    if x is None or np.isscalar(x):
        return x
    return int(np.asarray(x).reshape(-1)[s])


def sdpa_packed(q, k, v, q_segments, kv_segments=None, maxlen=None, scale=None, is_causal=False,
                q_offset=0, kv_lengths=None, q_lengths=None, qk_norm=False):
    """fp64 output [Lq_total][Hq][Dv] of packed attention.

    q [Lq_total][Hq][D], k [Lkv_total][Hkv][D], v [Lkv_total][Hkv][Dv] (float arrays);
    q_segments, kv_segments: segment lengths. q_offset, kv_lengths, q_lengths: None, an int,
    or one entry per segment. Raises ValueError when the lengths do not add up to the arrays
    or a segment is longer than maxlen (both outside what the pages allow).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qs = [int(t) for t in np.asarray(q_segments).reshape(-1)]
    ks = qs if kv_segments is None else [int(t) for t in np.asarray(kv_segments).reshape(-1)]
    if len(ks) != len(qs):
        raise ValueError("q_segments and kv_segments differ in count")
    if min(qs + ks, default=0) < 0 or sum(qs) != q.shape[0] or sum(ks) != k.shape[0]:
        raise ValueError("segment lengths must be >= 0 and add up to the sequence lengths")
    if maxlen is not None and max(qs + ks, default=0) > maxlen:
        raise ValueError("a segment is longer than maxlen")
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    out = np.zeros(q.shape[:2] + (v.shape[-1],), dtype=np.float64)
    a = c = 0
    for s, (n, m) in enumerate(zip(qs, ks)):
        if n > 0:
            out[a:a + n] = sdpa(q[None, a:a + n], k[None, c:c + m], v[None, c:c + m], scale=scale,
                                is_causal=is_causal, q_offset=_entry(q_offset, s) or 0,
                                kv_lengths=_entry(kv_lengths, s), q_lengths=_entry(q_lengths, s),
                                qk_norm=qk_norm)[0]
        a += n
        c += m
    return out
