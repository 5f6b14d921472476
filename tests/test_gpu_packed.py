"""GPU parity of sdpa_fwd_packed (packed sequences) against the fp64 oracle (MI355X only).

Page "Neural Network primitives from NNlib.jl", section "Packed sequences": segment s of the
queries attends segment s of the keys and values only, with is_causal, q_offset, q_lengths and
kv_lengths applied per segment. Segment lengths sit on and around the 128-row query tiles and
64-key tiles, include empty segments, and differ between q and k/v.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev, assert_close
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu


def packed_case(seed, qs, ks, Hq, Hkv, D, dtype, dist="normal"):
    rng = np.random.default_rng([seed, 3])
    draw = (lambda s: rng.random(s, dtype=np.float32)) if dist == "uniform" else \
        (lambda s: rng.standard_normal(s, dtype=np.float32))
    q = workloads.to_storage(draw((sum(qs), Hq, D)), dtype)
    k = workloads.to_storage(draw((sum(ks), Hkv, D)), dtype)
    v = workloads.to_storage(draw((sum(ks), Hkv, D)), dtype)
    return q, k, v


def run_packed(q, k, v, qs, ks, dtype, out_dtype=torch.float32, **kw):
    kvs = None if ks is None else torch.as_tensor(ks, dtype=torch.int32, device="cuda")
    out = sa.sdpa_packed(dev(q, dtype), dev(k, dtype), dev(v, dtype), torch.as_tensor(qs, dtype=torch.int32, device="cuda"),
                         kvs, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out


def test_packed_nnlib_example(lib):
    # "Examples": three documents of 5, 12 and 3 positions in one sequence of 20, 8 heads of 16,
    # uniform inputs, each attending causally to itself only
    say("packed nnlib example [5, 12, 3]")
    segs = [5, 12, 3]
    x, _, _ = packed_case(51, segs, segs, 8, 8, 16, "f32", dist="uniform")
    out = run_packed(x, x, x, segs, None, "f32", is_causal=True)
    assert tuple(out.shape) == (20, 8, 16)
    assert_close(out.cpu().numpy(), oracle.sdpa_packed(x, x, x, segs, is_causal=True), "f32", "nnlib packed")


QS = [300, 0, 1, 127, 128, 129, 513, 64]
KS = [310, 5, 1, 200, 128, 129, 513, 70]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("hkv", [4, 1])
@pytest.mark.parametrize("mode", ["plain", "causal", "causal_offsets", "bottom_right", "lengths"])
def test_packed_features(lib, mode, hkv, D, dtype):
    ks = KS if mode in ("bottom_right", "lengths", "plain") else QS
    kw = {}
    if mode == "causal":
        kw = dict(is_causal=True)
    elif mode == "causal_offsets":
        kw = dict(is_causal=True, q_offset=[0, 3, 0, -5, 10, 0, 2, 7])
    elif mode == "bottom_right":
        kw = dict(is_causal="bottom_right")
    elif mode == "lengths":
        kw = dict(is_causal="bottom_right", kv_lengths=[250, 5, 0, 200, 64, 100, 513, 1],
                  q_lengths=[300, 0, 1, 100, 128, 1, 500, 64])
    say(f"packed {mode} hkv={hkv} D={D} {dtype}")
    q, k, v = packed_case(52 + D + hkv, QS, ks, 4, hkv, D, dtype)
    okw = {key: (np.array(val, dtype=np.int32) if isinstance(val, list) else val) for key, val in kw.items()}
    gkw = {key: (torch.tensor(val, dtype=torch.int32, device="cuda") if isinstance(val, list) else val)
           for key, val in kw.items()}
    out = run_packed(q, k, v, QS, ks, dtype, **gkw)
    f = lambda a: workloads.widen(a, dtype)
    ref = oracle.sdpa_packed(f(q), f(k), f(v), QS, ks, **okw)
    assert_close(out.cpu().numpy(), ref, dtype, f"packed {mode}")


def test_packed_many_segments(lib):
    # more than 64 segments: the segment scan runs over several chunks of lanes
    rng = np.random.default_rng(53)
    qs = [int(t) for t in rng.integers(0, 40, size=150)]
    ks = [int(t) + 3 for t in qs]
    say(f"packed {len(qs)} segments, {sum(qs)} query rows")
    q, k, v = packed_case(54, qs, ks, 4, 2, 128, "bf16")
    out = run_packed(q, k, v, qs, ks, "bf16", is_causal="bottom_right", maxlen=max(qs + ks))
    f = workloads.bf16_to_f32
    assert_close(out.cpu().numpy(), oracle.sdpa_packed(f(q), f(k), f(v), qs, ks, is_causal="bottom_right"),
                 "bf16", "packed 150 segments")
    out2 = run_packed(q, k, v, qs, ks, "bf16", is_causal="bottom_right")        # no maxlen: same launch result
    np.testing.assert_array_equal(out.cpu().numpy(), out2.cpu().numpy())


def test_packed_qk_norm_and_f16_out(lib):
    say("packed qk_norm, f16 out")
    q, k, v = packed_case(55, QS, QS, 4, 2, 128, "f16")
    out = run_packed(q, k, v, QS, None, "f16", out_dtype=torch.float16, is_causal=True, qk_norm=True)
    assert out.dtype == torch.float16
    f = lambda a: workloads.widen(a, "f16")
    assert_close(out.float().cpu().numpy(), oracle.sdpa_packed(f(q), f(k), f(v), QS, is_causal=True, qk_norm=True),
                 "f16", "packed qk_norm")


def test_packed_equals_padded_batch_on_gpu(lib):
    # the same numbers as the padded batch through sdpa_fwd with the segments' sizes as lengths:
    # the kernel sees the same tiles of each segment in both layouts
    say("packed vs padded batch, bitwise")
    qs, ks = [200, 130, 7], [260, 64, 7]
    q, k, v = packed_case(56, qs, ks, 4, 2, 128, "bf16")
    out = run_packed(q, k, v, qs, ks, "bf16", is_causal="bottom_right").cpu().numpy()
    S, mq, mk = len(qs), max(qs), max(ks)
    Q = np.zeros((S, mq) + q.shape[1:], np.uint16)
    K = np.zeros((S, mk) + k.shape[1:], np.uint16)
    V = np.zeros((S, mk) + v.shape[1:], np.uint16)
    a = c = 0
    for s in range(S):
        Q[s, :qs[s]] = q[a:a + qs[s]]; K[s, :ks[s]] = k[c:c + ks[s]]; V[s, :ks[s]] = v[c:c + ks[s]]
        a += qs[s]; c += ks[s]
    pad = sa.sdpa(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), is_causal="bottom_right",
                  kv_lengths=torch.tensor(ks, dtype=torch.int32, device="cuda"),
                  q_lengths=torch.tensor(qs, dtype=torch.int32, device="cuda"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    pad = pad.cpu().numpy()
    a = 0
    for s in range(S):
        np.testing.assert_array_equal(out[a:a + qs[s]], pad[s, :qs[s]])
        a += qs[s]
