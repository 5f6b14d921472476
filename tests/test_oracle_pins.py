"""Pins of the fp64 oracle to facts the pages and the mathematics fix (CPU only).

Each test cites the passage it checks. Together they are chosen so that a plausible
mistake in the oracle (a dropped term, a wrong sign or index, a transposed operand,
a scaled bias, a wrong K/V head, an off-by-one in a causal rule) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import sdpa, sdpa_brute, per_head_rms_norm, rms_rows

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------------------------------
# Per-head RMS norm: the three printed worked examples (TensorTonic "Static Arguments in
# jit", "Examples"), the eps pin and the constraints domain ("Constraints").
# ------------------------------------------------------------------------------------------
def _golden():
    with open(os.path.join(HERE, "golden", "rms_norm_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_rms_norm_printed_examples(idx):
    g = _golden()
    ex = g["examples"][idx]
    res = per_head_rms_norm(np.array(ex["x"], dtype=np.float32), ex["num_heads"])
    tol = g["print_resolution"] * 0.5 + 1e-9       # printed to 6 decimals
    np.testing.assert_allclose(res["heads"], np.array(ex["heads"]), rtol=0, atol=tol)
    np.testing.assert_allclose(res["merged"], np.array(ex["merged"]), rtol=0, atol=tol)


def test_rms_norm_eps_value_is_pinned_by_the_examples():
    # The printed 0.365146 needs eps = 1e-6 inside the root; eps = 0 or 1e-5 misses it.
    x = np.array([[[0.1, 0.2, 0.3, 0.4]]])
    assert abs(per_head_rms_norm(x, 1)["heads"][0, 0, 0, 0] - 0.365146) <= 5e-7
    assert abs(per_head_rms_norm(x, 1, eps=0.0)["heads"][0, 0, 0, 0] - 0.365146) > 1e-6
    assert abs(per_head_rms_norm(x, 1, eps=1e-5)["heads"][0, 0, 0, 0] - 0.365146) > 1e-6


def test_rms_norm_constraints_domain():
    rng = np.random.default_rng(5)
    for _ in range(200):
        B, T = rng.integers(1, 4), rng.integers(1, 5)
        H = int(rng.choice([1, 2, 3, 4, 6]))
        Dh = int(rng.integers(1, 13 // H + 1))
        D = H * Dh
        if D < 2 or D > 12:
            continue
        x = rng.standard_normal((B, T, D)) * rng.choice([1e-3, 1.0, 50.0])
        zero_h = rng.integers(0, H)
        x.reshape(B, T, H, Dh)[:, :, zero_h, :] = 0.0           # a head may be all zero
        r = per_head_rms_norm(x, H)
        heads = r["heads"]
        assert heads.shape == (B, H, T, Dh)
        np.testing.assert_array_equal(heads[:, zero_h], 0.0)
        # every head: mean square of the output = ms / (ms + eps)
        ms_in = np.mean(x.reshape(B, T, H, Dh) ** 2, axis=-1)
        ms_out = np.mean(heads ** 2, axis=-1).transpose(0, 2, 1)
        np.testing.assert_allclose(ms_out, ms_in / (ms_in + 1e-6), rtol=1e-12, atol=1e-15)
        # merged keeps the original feature order: head h is features h*Dh..(h+1)*Dh-1
        for h in range(H):
            np.testing.assert_array_equal(r["merged"][:, :, h * Dh:(h + 1) * Dh], heads[:, h])


# ------------------------------------------------------------------------------------------
# The oracle against the independent scalar brute force, tiny shapes, every option.
# ------------------------------------------------------------------------------------------
CASES = [
    dict(),
    dict(is_causal=True),
    dict(is_causal=True, q_offset=[1, -1]),
    dict(is_causal="bottom_right"),
    dict(is_causal="bottom_right", kv_lengths=[5, 3]),
    dict(kv_lengths=[4, 7]),
    dict(bias=(2, 4, 5, 7)),
    dict(bias=(1, 4, 1, 7)),
    dict(bias=(2, 1, 5, 1)),
    dict(mask=(2, 4, 5, 7)),
    dict(mask=(1, 1, 5, 7), is_causal=True, kv_lengths=[6, 2]),
    dict(bias=(1, 4, 5, 7), mask=(2, 1, 5, 7), is_causal="bottom_right", kv_lengths=[7, 5]),
    dict(qk_norm=True),
    dict(qk_norm=True, bias=(2, 4, 5, 7), is_causal=True, q_offset=2),
    dict(scale=0.0),
    dict(scale=-1.7),
    dict(q_lengths=[3, 5], is_causal="bottom_right", kv_lengths=[7, 4]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("hkv", [4, 2, 1])
def test_oracle_matches_brute_force(case, hkv):
    opts = dict(CASES[case])
    B, Lq, Lkv, Hq, D, Dv = 2, 5, 7, 4, 3, 2
    seed = 100 * case + hkv
    q, k, v = rnd(seed, B, Lq, Hq, D), rnd(seed + 1, B, Lkv, hkv, D), rnd(seed + 2, B, Lkv, hkv, Dv)
    if "bias" in opts:
        opts["bias"] = rnd(seed + 3, *opts["bias"]) * 2.0
    if "mask" in opts:
        opts["mask"] = (np.random.default_rng(seed + 4).random(opts["mask"]) < 0.6).astype(np.uint8)
    a = sdpa(q, k, v, **opts)
    b = np.array(sdpa_brute(q, k, v, **opts))
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12, equal_nan=True)


# ------------------------------------------------------------------------------------------
# Closed forms and stated semantics
# ------------------------------------------------------------------------------------------
def test_weights_rows_sum_to_one_and_vanish_off_the_allowed_set():
    q, k, v = rnd(1, 2, 6, 2, 4), rnd(2, 2, 9, 2, 4), rnd(3, 2, 9, 2, 4)
    mask = (np.random.default_rng(4).random((2, 2, 6, 9)) < 0.5).astype(np.uint8)
    mask[..., 0] = 1
    _, w = sdpa(q, k, v, mask=mask, is_causal=True, q_offset=3, return_weights=True)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-13)
    allowed = (mask != 0) & (np.arange(9)[None, None, None, :] <= 3 + np.arange(6)[None, None, :, None])
    assert np.all(w[~allowed] == 0.0)
    assert np.all(w[allowed] > 0.0)


def test_v_of_ones_gives_ones():
    q, k = rnd(5, 1, 4, 2, 8), rnd(6, 1, 10, 2, 8)
    v = np.ones((1, 10, 2, 3))
    out = sdpa(q, k, v, bias=rnd(7, 1, 2, 4, 10), is_causal=True, q_offset=2, kv_lengths=7)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("how", ["scale0", "q0"])
def test_constant_logits_give_mean_of_allowed_values(how):
    B, Lq, Lkv, H, D = 2, 5, 9, 2, 4
    q = np.zeros((B, Lq, H, D)) if how == "q0" else rnd(8, B, Lq, H, D)
    k, v = rnd(9, B, Lkv, H, D), rnd(10, B, Lkv, H, D)
    kvl = [6, 9]
    out = sdpa(q, k, v, scale=0.0 if how == "scale0" else 1.3, is_causal=True, q_offset=1, kv_lengths=kvl)
    for b in range(B):
        for i in range(Lq):
            n = min(1 + i + 1, kvl[b])                   # keys j <= 1 + i and j < kvl
            np.testing.assert_allclose(out[b, i], v[b, :n].mean(axis=0), rtol=0, atol=1e-14)


def test_bias_enters_unscaled():
    # q = 0: the logits are the bias alone, whatever the scale; weights are exp(bias)
    B, Lq, Lkv, H, D = 1, 3, 6, 2, 4
    q = np.zeros((B, Lq, H, D))
    k, v = rnd(11, B, Lkv, H, D), rnd(12, B, Lkv, H, 3)
    bias = rnd(13, 1, H, Lq, Lkv)
    out = sdpa(q, k, v, bias=bias, scale=3.0)
    w = np.exp(bias[0])                                  # [H][Lq][Lkv]
    ref = np.einsum("hij,jhd->ihd", w, v[0]) / w.sum(-1).T[:, :, None]
    np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=1e-14)


def test_scale_multiplies_the_dot_product():
    # two keys: the weight of key 0 is sigmoid(scale*(q.k0 - q.k1))
    q = np.array([[[[1.0, 2.0]]]])
    k = np.array([[[[0.5, -1.0]], [[2.0, 1.0]]]])
    v = np.array([[[[1.0]], [[0.0]]]])
    for scale in (None, 0.3, -2.0):
        s = 1 / math.sqrt(2) if scale is None else scale
        w0 = 1.0 / (1.0 + math.exp(-s * ((0.5 - 2.0) - (2.0 + 2.0))))
        assert abs(sdpa(q, k, v, scale=scale)[0, 0, 0, 0] - w0) < 1e-15


def test_single_key_returns_its_value_row():
    q, k, v = rnd(14, 2, 3, 4, 8), rnd(15, 2, 1, 2, 8), rnd(16, 2, 1, 2, 5)
    out = sdpa(q, k, v, bias=rnd(17, 2, 4, 3, 1))
    for h in range(4):
        np.testing.assert_array_equal(out[:, :, h, :], np.broadcast_to(v[:, :, h // 2, :], (2, 3, 5)))
    # causal row 0 with offset 0 sees key 0 only
    k2, v2 = rnd(18, 1, 6, 1, 8), rnd(19, 1, 6, 1, 5)
    out2 = sdpa(rnd(20, 1, 6, 1, 8), k2, v2, is_causal=True)
    np.testing.assert_array_equal(out2[0, 0, 0], v2[0, 0, 0])


def test_is_causal_equals_explicit_lower_triangular_mask():
    L = 11
    q, k, v = rnd(21, 2, L, 3, 6), rnd(22, 2, L, 3, 6), rnd(23, 2, L, 3, 6)
    tril = np.tril(np.ones((L, L), dtype=np.uint8))[None, None]   # query i sees keys 0..i
    np.testing.assert_allclose(sdpa(q, k, v, is_causal=True), sdpa(q, k, v, mask=tril), rtol=0, atol=1e-15)


def test_bottom_right_equals_offset_kv_minus_q():
    q, k, v = rnd(24, 2, 4, 2, 6), rnd(25, 2, 10, 2, 6), rnd(26, 2, 10, 2, 6)
    np.testing.assert_array_equal(sdpa(q, k, v, is_causal="bottom_right"),
                                  sdpa(q, k, v, is_causal=True, q_offset=6))


def test_nnlib_decode_example_equivalence():
    # NNlib page, "Examples": a 64-slot cache, 3 new queries per batch element after
    # 10/20/30/40 cached keys; :bottom_right with kv_lengths 13/23/33/43 equals
    # is_causal=true with q_offset 10/20/30/40 and the same kv_lengths.
    rng = np.random.default_rng(27)
    q = rng.random((4, 3, 8, 16))            # (16, 8, 3, 4) in NNlib order
    k = rng.random((4, 64, 8, 16))
    v = k.copy()                             # the example passes k = v
    kvl = np.array([13, 23, 33, 43])
    a = sdpa(q, k, v, is_causal="bottom_right", kv_lengths=kvl)
    b = sdpa(q, k, v, is_causal=True, q_offset=[10, 20, 30, 40], kv_lengths=kvl)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (4, 3, 8, 16)
    # the last new query of each batch element sees exactly its kv_lengths keys
    for bb in range(4):
        for h in range(8):
            s = q[bb, 2, h] @ k[bb, :kvl[bb], h].T / 4.0
            p = np.exp(s - s.max())
            np.testing.assert_allclose(a[bb, 2, h], p @ v[bb, :kvl[bb], h] / p.sum(), rtol=1e-13)


def test_nnlib_example_shapes():
    rng = np.random.default_rng(28)
    q = rng.random((4, 20, 8, 16))            # NNlib (16, 8, 20, 4)
    k = rng.random((4, 30, 8, 16))            # NNlib (16, 8, 30, 4)
    assert sdpa(q, k, k).shape == (4, 20, 8, 16)
    k2 = rng.random((4, 30, 2, 16))           # 8 query heads over 2 K/V heads
    y = sdpa(q, k2, k2, kv_lengths=[12, 30, 30, 30])
    assert y.shape == (4, 20, 8, 16)
    # padding: batch 0 equals slicing its first 12 keys
    np.testing.assert_allclose(y[:1], sdpa(q[:1], k2[:1, :12], k2[:1, :12]), rtol=0, atol=1e-15)


def test_gqa_equals_repeated_kv_heads():
    Hq, Hkv = 6, 2
    q, k, v = rnd(29, 2, 5, Hq, 4), rnd(30, 2, 7, Hkv, 4), rnd(31, 2, 7, Hkv, 3)
    rep_k, rep_v = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    np.testing.assert_array_equal(sdpa(q, k, v, is_causal=True), sdpa(q, rep_k, rep_v, is_causal=True))
    # MQA: a single K/V head
    np.testing.assert_array_equal(sdpa(q, k[:, :, :1], v[:, :, :1]),
                                  sdpa(q, np.repeat(k[:, :, :1], Hq, 2), np.repeat(v[:, :, :1], Hq, 2)))


def test_kv_lengths_equals_slicing_and_ignores_a_nan_tail():
    q, k, v = rnd(32, 2, 4, 2, 5), rnd(33, 2, 9, 2, 5), rnd(34, 2, 9, 2, 5)
    kvl = [3, 9]
    k_nan, v_nan = k.copy(), v.copy()
    k_nan[0, 3:] = np.nan
    v_nan[0, 3:] = np.nan
    out = sdpa(q, k_nan, v_nan, kv_lengths=kvl)
    np.testing.assert_allclose(out[0:1], sdpa(q[:1], k[:1, :3], v[:1, :3]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[1:2], sdpa(q[1:], k[1:], v[1:]), rtol=0, atol=1e-15)
    # out-of-range lengths clamp
    np.testing.assert_array_equal(sdpa(q, k, v, kv_lengths=[99, 9]), sdpa(q, k, v))


def test_fully_masked_queries_are_nan():
    q, k, v = rnd(35, 1, 3, 1, 4), rnd(36, 1, 5, 1, 4), rnd(37, 1, 5, 1, 4)
    assert np.isnan(sdpa(q, k, v, kv_lengths=0)).all()
    out = sdpa(q, k, v, is_causal=True, q_offset=-1)     # row 0 sees no key; rows 1, 2 do
    assert np.isnan(out[0, 0]).all() and np.isfinite(out[0, 1:]).all()
    mask = np.ones((1, 1, 3, 5), dtype=np.uint8)
    mask[0, 0, 1] = 0
    out = sdpa(q, k, v, mask=mask)
    assert np.isnan(out[0, 1]).all() and np.isfinite(out[0, [0, 2]]).all()
    k0 = np.zeros((1, 0, 1, 4))
    assert np.isnan(sdpa(q, k0, k0)).all()


def test_bias_shift_invariance_and_minus_inf_bias_is_a_mask():
    q, k, v = rnd(38, 2, 4, 2, 4), rnd(39, 2, 6, 2, 4), rnd(40, 2, 6, 2, 4)
    bias = rnd(41, 2, 2, 4, 6)
    row_const = rnd(42, 2, 2, 4, 1) * 10
    np.testing.assert_allclose(sdpa(q, k, v, bias=bias), sdpa(q, k, v, bias=bias + row_const), rtol=0, atol=1e-12)
    mask = (np.random.default_rng(43).random((2, 2, 4, 6)) < 0.6).astype(np.uint8)
    mask[..., 0] = 1
    ninf = np.where(mask != 0, bias, -np.inf)
    np.testing.assert_allclose(sdpa(q, k, v, bias=ninf), sdpa(q, k, v, bias=bias, mask=mask), rtol=0, atol=1e-15)


def test_joint_key_permutation_invariance():
    q, k, v = rnd(44, 2, 5, 2, 4), rnd(45, 2, 8, 2, 4), rnd(46, 2, 8, 2, 3)
    bias = rnd(47, 2, 2, 5, 8)
    mask = (np.random.default_rng(48).random((2, 2, 5, 8)) < 0.7).astype(np.uint8)
    perm = np.random.default_rng(49).permutation(8)
    a = sdpa(q, k, v, bias=bias, mask=mask)
    b = sdpa(q, k[:, perm], v[:, perm], bias=bias[..., perm], mask=mask[..., perm])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13, equal_nan=True)


def test_q_offset_chunk_invariance():
    L, c, n = 12, 5, 4
    q, k, v = rnd(50, 1, L, 2, 4), rnd(51, 1, L, 2, 4), rnd(52, 1, L, 2, 4)
    full = sdpa(q, k, v, is_causal=True)
    chunk = sdpa(q[:, c:c + n], k, v, is_causal=True, q_offset=c)
    np.testing.assert_allclose(full[:, c:c + n], chunk, rtol=0, atol=1e-15)
    rows = sdpa(q, k, v, is_causal=True, rows=[c, c + 3])
    np.testing.assert_array_equal(rows, full[:, [c, c + 3]])


def test_q_offset_without_causal_has_no_effect():
    q, k, v = rnd(53, 1, 4, 1, 4), rnd(54, 1, 6, 1, 4), rnd(55, 1, 6, 1, 4)
    np.testing.assert_array_equal(sdpa(q, k, v, q_offset=3), sdpa(q, k, v))


def test_q_lengths_zero_rows():
    q, k, v = rnd(56, 2, 5, 1, 4), rnd(57, 2, 6, 1, 4), rnd(58, 2, 6, 1, 4)
    out = sdpa(q, k, v, q_lengths=[2, 5])
    assert np.all(out[0, 2:] == 0.0)
    np.testing.assert_array_equal(out[0, :2], sdpa(q, k, v)[0, :2])


def test_qk_norm_is_per_row_rms_of_q_and_k_only():
    q, k, v = rnd(59, 1, 3, 2, 8) * 5, rnd(60, 1, 4, 2, 8) * 3, rnd(61, 1, 4, 2, 8) * 7
    a = sdpa(q, k, v, qk_norm=True)
    b = sdpa(rms_rows(q), rms_rows(k), v)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)
    # nearly invariant to a positive rescaling of a q or k row (exactly so but for eps,
    # which is 1e-7 of these rows' mean squares)
    q2, k2 = q.copy(), k.copy()
    q2[0, 1, 0] *= 13.0
    k2[0, 2, 1] *= 0.5
    np.testing.assert_allclose(sdpa(q2, k2, v, qk_norm=True), a, rtol=0, atol=1e-5)
    # ... and a row of zeros stays zero: its logits are 0 (the NaN-free eps case)
    k3 = k.copy()
    k3[0, :, 0] = 0.0
    out = sdpa(q, k3, v, qk_norm=True)
    np.testing.assert_allclose(out[0, :, 0:1], np.broadcast_to(v[0, :, 0].mean(0), (3, 1, 8)), atol=1e-14)


def test_two_key_closed_form_with_gqa_and_causal():
    # hand-checkable: query head h uses K/V head h // 2; causal with offset 0
    q = np.zeros((1, 2, 4, 1)); k = np.zeros((1, 2, 2, 1)); v = np.zeros((1, 2, 2, 1))
    q[0, :, :, 0] = [[1.0, 2.0, 3.0, 4.0], [0.5, -1.0, 1.5, -2.0]]
    k[0, :, :, 0] = [[1.0, -1.0], [2.0, 0.5]]
    v[0, :, :, 0] = [[10.0, 20.0], [30.0, 40.0]]
    out = sdpa(q, k, v, scale=1.0, is_causal=True)
    # row 0 sees key 0 only
    np.testing.assert_array_equal(out[0, 0, :, 0], [10.0, 10.0, 20.0, 20.0])
    # row 1, head 2 (K/V head 1): logits 1.5*(-1), 1.5*0.5
    s0, s1 = -1.5, 0.75
    w1 = math.exp(s1) / (math.exp(s0) + math.exp(s1))
    assert abs(out[0, 1, 2, 0] - (20.0 * (1 - w1) + 40.0 * w1)) < 1e-13
    # row 1, head 1 (K/V head 0): logits -1*1, -1*2
    w1 = math.exp(-2.0) / (math.exp(-1.0) + math.exp(-2.0))
    assert abs(out[0, 1, 1, 0] - (10.0 * (1 - w1) + 30.0 * w1)) < 1e-13
