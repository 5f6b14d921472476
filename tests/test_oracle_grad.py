"""Pins of the gradient oracle (CPU): central finite differences of the forward oracle, which
is pinned on its own, and identities that hold for any input.

Page "Neural Network primitives from NNlib.jl", section "Fused implementation": the gradient
with respect to query, key, value and scale (and, on the materialized path, the bias); a query
whose output is NaN takes no part.

The loss is L = sum over the finite output rows of <dO, out>, so that its gradient is the
cotangent the oracle propagates from dO. A dropped term, a wrong sign, a transposed operand or
a head mapped to the wrong K/V head changes some entry by far more than the tolerance.
"""
import numpy as np
import pytest

import oracle

H_STEP = 1e-6


def _loss(args, kw, dout):
    o = oracle.sdpa(*args, **kw)
    return float(np.sum(np.where(np.isnan(o), 0.0, o * dout)))


def _fd(args, kw, dout, which):
    """Central differences of the loss in every element of args[which] (0 q, 1 k, 2 v)."""
    x = args[which]
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        a = [t.copy() for t in args]
        a[which][idx] += H_STEP
        up = _loss(a, kw, dout)
        a[which][idx] -= 2 * H_STEP
        g[idx] = (up - _loss(a, kw, dout)) / (2 * H_STEP)
    return g


CASES = {
    "plain": dict(B=1, Lq=3, Lkv=4, Hq=2, Hkv=2, D=3, Dv=2, kw={}),
    "gqa_causal_offset": dict(B=2, Lq=3, Lkv=5, Hq=4, Hkv=2, D=3, Dv=3,
                              kw=dict(is_causal=True, q_offset=np.array([1, 2]))),
    "bottom_right_lengths": dict(B=2, Lq=4, Lkv=5, Hq=2, Hkv=1, D=2, Dv=3,
                                 kw=dict(is_causal="bottom_right", kv_lengths=np.array([3, 5]),
                                         q_lengths=np.array([4, 2]))),
    "mask_with_empty_row": dict(B=1, Lq=4, Lkv=4, Hq=2, Hkv=1, D=3, Dv=2, kw="mask"),
    "scale": dict(B=1, Lq=3, Lkv=3, Hq=1, Hkv=1, D=4, Dv=2, kw=dict(scale=-0.7)),
}


def _make(case, seed):
    c = CASES[case]
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((c["B"], c["Lq"], c["Hq"], c["D"]))
    k = rng.standard_normal((c["B"], c["Lkv"], c["Hkv"], c["D"]))
    v = rng.standard_normal((c["B"], c["Lkv"], c["Hkv"], c["Dv"]))
    dout = rng.standard_normal((c["B"], c["Lq"], c["Hq"], c["Dv"]))
    kw = c["kw"]
    if kw == "mask":
        m = rng.random((1, c["Hq"], c["Lq"], c["Lkv"])) < 0.6
        m[0, 1, 2, :] = False                    # a query that attends nothing: NaN row
        m[0, :, :, 0] |= np.eye(c["Lq"], c["Lkv"], dtype=bool)[:, 0]
        kw = dict(mask=m)
    return q, k, v, dout, kw


@pytest.mark.parametrize("case", sorted(CASES))
def test_grad_qkv_equal_finite_differences(case):
    q, k, v, dout, kw = _make(case, 50 + sorted(CASES).index(case))
    g = oracle.sdpa_grad(q, k, v, dout, **kw)
    for which, name in enumerate(("dq", "dk", "dv")):
        fd = _fd([q, k, v], kw, dout, which)
        np.testing.assert_allclose(g[name], fd, rtol=0, atol=1e-7, err_msg=f"{case} {name}")


@pytest.mark.parametrize("case", sorted(CASES))
def test_grad_scale_equals_finite_difference(case):
    q, k, v, dout, kw = _make(case, 60 + sorted(CASES).index(case))
    scale = kw.get("scale", 1.0 / np.sqrt(q.shape[-1]))
    kw2 = {a: b for a, b in kw.items() if a != "scale"}
    up = _loss([q, k, v], dict(kw2, scale=scale + H_STEP), dout)
    dn = _loss([q, k, v], dict(kw2, scale=scale - H_STEP), dout)
    g = oracle.sdpa_grad(q, k, v, dout, **kw)
    assert abs(g["dscale"] - (up - dn) / (2 * H_STEP)) < 1e-7


@pytest.mark.parametrize("bshape", [(1, 2, 3, 4), (1, 1, 1, 4), (1, 2, 3, 1)])
def test_grad_bias_equals_finite_differences(bshape):
    rng = np.random.default_rng(70)
    q, k, v = rng.standard_normal((1, 3, 2, 2)), rng.standard_normal((1, 4, 1, 2)), rng.standard_normal((1, 4, 1, 2))
    dout = rng.standard_normal((1, 3, 2, 2))
    bias = rng.standard_normal(bshape)
    g = oracle.sdpa_grad(q, k, v, dout, bias=bias, is_causal="bottom_right")
    fd = np.zeros_like(bias)
    for idx in np.ndindex(bias.shape):
        b = bias.copy()
        b[idx] += H_STEP
        up = _loss([q, k, v], dict(bias=b, is_causal="bottom_right"), dout)
        b[idx] -= 2 * H_STEP
        fd[idx] = (up - _loss([q, k, v], dict(bias=b, is_causal="bottom_right"), dout)) / (2 * H_STEP)
    np.testing.assert_allclose(g["dbias"], fd, rtol=0, atol=1e-7)


def test_grad_of_rows_without_part_is_zero():
    # an empty row (NaN output) and rows past q_lengths give no gradient, whatever dO holds there
    q, k, v, dout, kw = _make("mask_with_empty_row", 80)
    g = oracle.sdpa_grad(q, k, v, dout, **kw)
    assert np.all(g["dq"][0, 2, 1] == 0)
    g2 = oracle.sdpa_grad(q, k, v, dout, q_lengths=np.array([2]))
    assert np.all(g2["dq"][0, 2:] == 0)
    d2 = dout.copy()
    d2[0, 2:] = 1e6
    g3 = oracle.sdpa_grad(q, k, v, d2, q_lengths=np.array([2]))
    for n in ("dk", "dv"):
        np.testing.assert_array_equal(g2[n], g3[n])


def test_grad_identities():
    # the weights sum to one, so dS sums to zero over each row: a shift of all logits of a row
    # changes nothing, and the bias gradient rows sum to zero. q . dq summed equals
    # scale * dscale (dq is scale * dS K), and the dv of a constant dO row is that row times
    # the weight the key gets
    rng = np.random.default_rng(90)
    q, k, v = rng.standard_normal((2, 5, 4, 8)), rng.standard_normal((2, 7, 2, 8)), rng.standard_normal((2, 7, 2, 6))
    dout = rng.standard_normal((2, 5, 4, 6))
    g = oracle.sdpa_grad(q, k, v, dout, bias=np.zeros((2, 4, 5, 7)), scale=0.3, is_causal=True,
                         q_offset=np.array([2, 3]))
    np.testing.assert_allclose(g["dbias"].sum(axis=3), 0, atol=1e-12)
    np.testing.assert_allclose(np.sum(q * g["dq"]), 0.3 * g["dscale"], rtol=1e-10)
    # the GQA sum: dk of a shared head equals the sum of dk from the query heads taken as
    # separate heads over repeated K/V
    kr, vr = np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2)
    gr = oracle.sdpa_grad(q, kr, vr, dout, scale=0.3, is_causal=True, q_offset=np.array([2, 3]))
    g0 = oracle.sdpa_grad(q, k, v, dout, scale=0.3, is_causal=True, q_offset=np.array([2, 3]))
    np.testing.assert_allclose(g0["dk"], gr["dk"][:, :, 0::2] + gr["dk"][:, :, 1::2], atol=1e-12)
    np.testing.assert_allclose(g0["dv"], gr["dv"][:, :, 0::2] + gr["dv"][:, :, 1::2], atol=1e-12)
    np.testing.assert_allclose(g0["dq"], gr["dq"], atol=1e-12)


@pytest.mark.parametrize("kw", [{}, dict(is_causal=True, q_offset=1), dict(kv_lengths=np.array([3, 0]))])
def test_lse_gives_the_weights(kw):
    # exp(s - lse) reproduces the weights of the forward oracle, row by row; -inf where a row
    # attends nothing
    rng = np.random.default_rng(95)
    q, k, v = rng.standard_normal((2, 4, 2, 3)), rng.standard_normal((2, 6, 1, 3)), rng.standard_normal((2, 6, 1, 3))
    lse = oracle.sdpa_lse(q, k, v, **kw)
    _, w = oracle.sdpa(q, k, v, return_weights=True, **kw)
    s = np.einsum("bihd,bjd->bhij", q, k[:, :, 0, :]) / np.sqrt(3)
    for b in range(2):
        for h in range(2):
            for i in range(4):
                if np.isnan(w[b, h, i]).all():
                    assert lse[b, h, i] == -np.inf
                    continue
                nz = w[b, h, i] > 0
                np.testing.assert_allclose(np.exp(s[b, h, i][nz] - lse[b, h, i]), w[b, h, i][nz], rtol=1e-12)
