"""Pins of the packed-sequence oracle against other statements of the same operation (CPU).

Page "Neural Network primitives from NNlib.jl", section "Packed sequences": segment s of the
queries attends segment s of the keys and values only, as a batch element does in a padded
batch, with is_causal, q_offset, q_lengths and kv_lengths taken per segment.
"""
import numpy as np
import pytest

import oracle


def _padded(x, segs):
    """[total][H][D] -> [S][max(segs)][H][D], zero-padded."""
    S, n = len(segs), max(max(segs), 1)
    out = np.zeros((S, n) + x.shape[1:])
    a = 0
    for s, m in enumerate(segs):
        out[s, :m] = x[a:a + m]
        a += m
    return out


@pytest.mark.parametrize("is_causal,q_offset", [(False, 0), (True, 0), (True, [0, 1, -2, 3, 5]),
                                                  ("bottom_right", 0)])
@pytest.mark.parametrize("with_lengths", [False, True])
def test_packed_equals_padded_batch(is_causal, q_offset, with_lengths):
    rng = np.random.default_rng(40)
    qs, ks = [5, 0, 12, 3, 7], [6, 2, 12, 1, 9]
    Hq, Hkv, D, Dv = 4, 2, 8, 6
    q = rng.standard_normal((sum(qs), Hq, D))
    k = rng.standard_normal((sum(ks), Hkv, D))
    v = rng.standard_normal((sum(ks), Hkv, Dv))
    kvl = [4, 1, 12, 0, 9] if with_lengths else None
    ql = [3, 0, 12, 2, 7] if with_lengths else None
    got = oracle.sdpa_packed(q, k, v, qs, ks, is_causal=is_causal, q_offset=q_offset, kv_lengths=kvl,
                             q_lengths=ql)
    # the padded batch: every segment a batch element, the segment sizes as lengths (the given
    # lengths cut to them)
    pkv = [min(a, b) for a, b in zip(kvl, ks)] if with_lengths else ks
    pq = [min(a, b) for a, b in zip(ql, qs)] if with_lengths else qs
    ref = oracle.sdpa(_padded(q, qs), _padded(k, ks), _padded(v, ks), is_causal=is_causal,
                      q_offset=np.array(q_offset) if isinstance(q_offset, list) else q_offset,
                      kv_lengths=np.array(pkv), q_lengths=np.array(pq))
    a = 0
    for s, n in enumerate(qs):
        np.testing.assert_allclose(got[a:a + n], ref[s, :n], rtol=0, atol=1e-12, equal_nan=True)
        a += n


def test_packed_nnlib_example_is_block_diagonal_causal():
    # "Examples": three documents of 5, 12 and 3 positions packed in one sequence of 20 (8 heads
    # of 16, uniform inputs), each attending causally to itself only -- the whole sequence under
    # a block-diagonal causal mask, computed by the brute-force oracle
    rng = np.random.default_rng(41)
    segs = [5, 12, 3]
    x = rng.random((20, 8, 16))
    got = oracle.sdpa_packed(x, x, x, segs, is_causal=True)
    seg_of = np.repeat(np.arange(3), segs)
    i, j = np.meshgrid(np.arange(20), np.arange(20), indexing="ij")
    mask = (seg_of[i] == seg_of[j]) & (j <= i)
    ref = np.array(oracle.sdpa_brute(x[None], x[None], x[None], mask=mask[None, None]))[0]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_packed_single_segment_is_the_plain_call():
    rng = np.random.default_rng(42)
    q, k, v = rng.standard_normal((9, 2, 4)), rng.standard_normal((11, 2, 4)), rng.standard_normal((11, 2, 4))
    got = oracle.sdpa_packed(q, k, v, [9], [11], is_causal="bottom_right")
    ref = oracle.sdpa(q[None], k[None], v[None], is_causal="bottom_right")[0]
    np.testing.assert_array_equal(got, ref)


def test_packed_rejects_lengths_that_do_not_add_up():
    q = np.zeros((6, 1, 4))
    with pytest.raises(ValueError):
        oracle.sdpa_packed(q, q, q, [2, 3])
    with pytest.raises(ValueError):
        oracle.sdpa_packed(q, q, q, [2, 4], maxlen=3)
