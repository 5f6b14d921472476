"""GPU parity of kv_cache_update (bit-exact), sdpa_decode (oracle tolerance) and the
per-head RMS norm (printed examples) on MI355X."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev, assert_close
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_kv_cache_update_bit_exact(lib, dtype):
    say(f"kv_cache_update {dtype}")
    rng = np.random.default_rng(3)
    B, cap, H, D, T = 5, 40, 3, 24, 3
    mk = lambda s: workloads.to_storage(rng.standard_normal(s, dtype=np.float32), dtype)
    kc, vc, kn, vn = mk((B, cap, H, D)), mk((B, cap, H, D)), mk((B, T, H, D)), mk((B, T, H, D))
    widx = np.array([0, 37, 39, -2, 12], dtype=np.int32)        # tail rows past the cache are skipped
    ek, ev = oracle.kv_cache_update(kc, vc, kn, vn, widx)
    tkc, tvc = dev(kc, dtype), dev(vc, dtype)
    sa.kv_cache_update(tkc, tvc, dev(kn, dtype), dev(vn, dtype), torch.as_tensor(widx, device="cuda"))
    torch.cuda.synchronize()
    view = np.uint32 if dtype == "f32" else np.uint16
    gk = tkc.cpu().view(torch.int32 if dtype == "f32" else torch.int16).numpy().view(view)
    gv = tvc.cpu().view(torch.int32 if dtype == "f32" else torch.int16).numpy().view(view)
    np.testing.assert_array_equal(gk, ek.view(view))
    np.testing.assert_array_equal(gv, ev.view(view))


def decode_case(B, Hq, Hkv, D, cap, kv_min, kv_max, base):
    return workloads.gqa_decode(B=B, Hq=Hq, Hkv=Hkv, D=D, capacity=cap, kv_min=kv_min, kv_max=kv_max, base=base)


def run_decode(d: workloads.Decode, num_splits=0, out_dtype=torch.float32):
    q = dev(d.q, d.dtype)
    kc, vc = dev(d.k_cache, d.dtype), dev(d.v_cache, d.dtype)
    sa.kv_cache_update(kc, vc, dev(d.k_new, d.dtype), dev(d.v_new, d.dtype),
                       torch.as_tensor(d.write_index, device="cuda"))
    kvl = torch.as_tensor(d.kv_lengths, device="cuda")
    out = sa.sdpa_decode(q, kc, vc, kvl, scale=d.scale, num_splits=num_splits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, kc, vc


def oracle_decode(d: workloads.Decode, batches=None):
    kc, vc = oracle.kv_cache_update(d.k_cache, d.v_cache, d.k_new, d.v_new, d.write_index)
    bs = range(d.q.shape[0]) if batches is None else batches
    outs = []
    for b in bs:
        n = int(d.kv_lengths[b])
        f = lambda a: workloads.widen(a, d.dtype)
        outs.append(oracle.sdpa(f(d.q[b:b + 1]), f(kc[b:b + 1, :n]), f(vc[b:b + 1, :n]), scale=d.scale,
                                is_causal="bottom_right")[0])
    return np.stack(outs)


@pytest.mark.parametrize("shape", [(4, 32, 8, 128, 700, 1, 700), (3, 8, 8, 128, 300, 60, 300),
                                   (2, 16, 2, 128, 1000, 500, 1000), (3, 8, 2, 64, 200, 1, 200),
                                   (2, 12, 4, 96, 150, 20, 150)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_decode_small(lib, shape, num_splits):
    B, Hq, Hkv, D, cap, lo, hi = shape
    say(f"decode {shape} splits={num_splits}")
    d = decode_case(B, Hq, Hkv, D, cap, lo, hi, base=500 + B + Hq)
    out, _, _ = run_decode(d, num_splits)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()                                # the NaN-poisoned tail is never read
    assert_close(got, oracle_decode(d), "bf16", f"decode {shape}")


def test_decode_equals_fwd_bottom_right(lib):
    say("decode vs fwd")
    d = decode_case(3, 16, 4, 128, 520, 100, 520, base=601)
    out, kc, vc = run_decode(d)
    q = dev(d.q, "bf16")
    kvl = torch.as_tensor(d.kv_lengths, device="cuda")
    ref = sa.sdpa(q, kc, vc, is_causal="bottom_right", kv_lengths=kvl, scale=d.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # same operation, but the two kernels round differently (the forward kernel folds the scale
    # into bf16 Q and sums over 64-key tiles, decode sums bf16 P over 1024-key splits and merges
    # them), so they agree to the bf16 bar rather than bit for bit
    assert_close(out.cpu().numpy(), ref.cpu().numpy(), "bf16", "decode vs fwd")
    assert_close(out.cpu().numpy(), oracle_decode(d), "bf16", "decode vs oracle")


def test_decode_zero_length_is_nan(lib):
    say("decode zero length")
    d = decode_case(2, 8, 2, 128, 128, 1, 128, base=602)
    q = dev(d.q, "bf16")
    kc, vc = dev(d.k_cache, "bf16"), dev(d.v_cache, "bf16")
    kvl = torch.tensor([0, 5], dtype=torch.int32, device="cuda")
    out = sa.sdpa_decode(q, kc, vc, kvl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[0]).all() and np.isfinite(got[1]).all()


def test_incremental_decode_matches_causal_prefill(lib):
    # Flax discussion: nnx.MultiHeadAttention(8, 512) decodes with a cache of 100 positions
    # (8 heads x 64 features), the cache growing one position per step.
    say("incremental decode 8x64, cache 100")
    B, H, D, cap, steps = 1, 8, 64, 100, 99
    rng = np.random.default_rng(17)
    ks = workloads.f32_to_bf16(rng.random((B, steps, H, D), dtype=np.float32))
    vs = workloads.f32_to_bf16(rng.random((B, steps, H, D), dtype=np.float32))
    qs = workloads.f32_to_bf16(rng.random((B, steps, H, D), dtype=np.float32))
    kc = torch.zeros(B, cap, H, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kd, vd, qd = dev(ks, "bf16"), dev(vs, "bf16"), dev(qs, "bf16")
    outs = []
    for t in range(steps):
        sa.kv_cache_update(kc, vc, kd[:, t:t + 1], vd[:, t:t + 1], torch.tensor([t], dtype=torch.int32, device="cuda"))
        outs.append(sa.sdpa_decode(qd[:, t:t + 1], kc, vc, torch.tensor([t + 1], dtype=torch.int32, device="cuda"),
                                   out_dtype=torch.float32))
    got = torch.cat(outs, dim=1).cpu().numpy()
    f = workloads.bf16_to_f32
    ref = oracle.sdpa(f(qs), f(ks), f(vs), is_causal=True)
    assert_close(got, ref, "bf16", "incremental decode")


def test_head_rms_norm_printed_examples(lib):
    with open(os.path.join(HERE, "golden", "rms_norm_examples.json")) as fh:
        g = json.load(fh)
    for ex in g["examples"]:
        say(f"rms norm example heads={ex['num_heads']}")
        x = torch.tensor(ex["x"], dtype=torch.float32, device="cuda")
        r = sa.per_head_rms_norm(x, ex["num_heads"])
        torch.cuda.synchronize()
        tol = g["print_resolution"] * 0.5 + 1e-6      # printed to 6 decimals, fp32 arithmetic
        np.testing.assert_allclose(r["heads"].cpu().numpy(), np.array(ex["heads"]), rtol=0, atol=tol)
        np.testing.assert_allclose(r["merged"].cpu().numpy(), np.array(ex["merged"]), rtol=0, atol=tol)


def test_head_rms_norm_random_vs_oracle(lib):
    say("rms norm random")
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 5, 6, 128), dtype=np.float32) * 3
    x[1, 2, 4] = 0.0
    y = sa.head_rms_norm(torch.as_tensor(x, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.rms_rows(x)
    np.testing.assert_allclose(y.cpu().numpy(), ref, rtol=0, atol=2e-6)
    assert np.all(y.cpu().numpy()[1, 2, 4] == 0.0)


@pytest.mark.parametrize("hq,hkv", [(16, 16), (16, 8), (32, 8), (32, 4), (32, 2), (16, 1)])
def test_decode_tile_and_split_edges(lib, hq, hkv):
    # the matrix-core decode works in 32-key tiles and 1024-key splits: lengths on and around
    # both edges, every query-heads-per-K/V-head ratio it takes (1..16), default splits
    lens = np.array([1, 2, 31, 32, 33, 63, 511, 512, 513, 1023, 1024, 1025, 1040, 2047, 2048, 2080],
                    dtype=np.int32)
    say(f"decode edges hq={hq} hkv={hkv}")
    d = decode_case(len(lens), hq, hkv, 128, 2080, 2080, 2080, base=700 + hq + hkv)
    d.kv_lengths = lens                                   # rows past each length are never read
    out, _, _ = run_decode(d)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, oracle_decode(d), "bf16", f"decode edges {hq}/{hkv}")


@pytest.mark.parametrize("B", [130, 260])
def test_decode_large_batches(lib, B):
    # 130 sequences: the linear work order locates items across three 64-sequence chunks;
    # 260: more sequences than that order takes, so the (split, sequence) grid
    say(f"decode batch {B}")
    d = decode_case(B, 8, 2, 128, 1100, 1, 1100, base=730 + B)
    out, _, _ = run_decode(d)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, oracle_decode(d), "bf16", f"decode batch {B}")


def test_decode_batch_above_64(lib):
    # more sequences than one wave's lanes: the one-workgroup-per-split form
    say("decode batch 70")
    d = decode_case(70, 8, 2, 128, 600, 1, 600, base=720)
    out, _, _ = run_decode(d)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, oracle_decode(d), "bf16", "decode batch 70")


def decode_case_t(B, Hq, Hkv, D, T, cap, kv_min, kv_max, base):
    return workloads.gqa_decode(B=B, Hq=Hq, Hkv=Hkv, D=D, capacity=cap, kv_min=kv_min, kv_max=kv_max, base=base,
                                q_len=T)


@pytest.mark.parametrize("shape,num_splits", [
    ((3, 32, 8, 128, 3, 700, 1, 700), 0),      # 4 heads x 3 tokens in one column group
    ((2, 16, 2, 128, 4, 1100, 2, 1100), 0),    # 8 x 4: two column groups
    ((2, 8, 8, 128, 16, 600, 20, 600), 0),     # 1 x 16 tokens
    ((2, 32, 2, 128, 2, 1040, 1000, 1040), 0),  # 16 x 2: two groups, lengths around the split edges
    ((70, 8, 2, 128, 3, 600, 1, 600), 0),      # more sequences than one wave's lanes
    ((3, 32, 8, 128, 3, 700, 1, 700), 3),      # explicit splits: the general kernel
    ((3, 8, 2, 64, 3, 300, 1, 300), 0),        # head dim 64: the general kernel
    ((2, 8, 8, 128, 20, 300, 30, 300), 0),     # 20 tokens: the general kernel
])
def test_decode_multi_token(lib, shape, num_splits):
    # query t of sequence b attends keys [0, kv_lengths[b] - T + t]; a sequence shorter than T
    # leaves its first queries with no key at all (NaN rows, in the same places as the oracle)
    B, Hq, Hkv, D, T, cap, lo, hi = shape
    say(f"decode T={T} {shape} splits={num_splits}")
    d = decode_case_t(B, Hq, Hkv, D, T, cap, lo, hi, base=740 + B + Hq + T)
    out, _, _ = run_decode(d, num_splits)
    assert out.shape == (B, T, Hq, D)
    assert_close(out.cpu().numpy(), oracle_decode(d), "bf16", f"decode T={T} {shape}")


def test_decode_three_queries_nnlib_cache_example(lib):
    # NNlib "Examples": three new queries against caches of kv_lengths [13, 23, 33, 43] behave
    # as q_offset [10, 20, 30, 40]; the same lengths here, 8 heads of 128
    say("decode T=3 at kv_lengths 13, 23, 33, 43")
    d = decode_case_t(4, 8, 8, 128, 3, 48, 48, 48, base=760)
    d.kv_lengths = np.array([13, 23, 33, 43], dtype=np.int32)
    out, kc, vc = run_decode(d)
    assert np.isfinite(out.cpu().numpy()).all()
    assert_close(out.cpu().numpy(), oracle_decode(d), "bf16", "decode T=3 vs oracle")
    # the cache slots past kv_lengths hold NaN sentinels: sdpa_fwd is told the lengths too, as
    # decode is (a causally masked NaN value row would still poison the product, 0 * NaN)
    q = dev(d.q, "bf16")
    kvl = torch.as_tensor(d.kv_lengths, device="cuda")
    ref = sa.sdpa(q, kc, vc, is_causal=True, q_offset=torch.tensor([10, 20, 30, 40], dtype=torch.int32, device="cuda"),
                  kv_lengths=kvl, scale=d.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref.cpu().numpy(), "bf16", "decode T=3 vs fwd with q_offset")


@pytest.mark.parametrize("T", [1, 3])
def test_decode_f16(lib, T):
    # f16 caches: the matrix-core pass on its f16 MFMA, one and several query tokens
    say(f"decode f16 T={T}")
    d = workloads.gqa_decode(B=3, Hq=32, Hkv=8, D=128, capacity=1100, kv_min=1, kv_max=1100, base=780 + T,
                             q_len=T, dtype="f16")
    for od in (torch.float32, torch.float16):
        out, _, _ = run_decode(d, out_dtype=od)
        assert out.dtype == od
        assert_close(out.float().cpu().numpy(), oracle_decode(d), "f16", f"decode f16 T={T} out {od}")


def test_head_rms_norm_f16(lib):
    say("rms norm f16")
    rng = np.random.default_rng(9)
    x = workloads.to_storage(rng.standard_normal((2, 5, 6, 64), dtype=np.float32) * 3, "f16")
    y = sa.head_rms_norm(torch.as_tensor(x, device="cuda"))
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    ref = oracle.rms_rows(x.astype(np.float32))
    # one f16 rounding of results below ~4: half an ulp is at most 2^-9
    np.testing.assert_allclose(y.float().cpu().numpy(), ref, rtol=2 ** -10, atol=2 ** -12)


@pytest.mark.parametrize("B", [64, 260])
def test_decode_repeatable(lib, B):
    # the direct loads that refill a stage of the LDS ring wait for the reads of what they
    # replace: repeated calls give the same bits (a refill overtaking those reads once made one
    # workgroup in a thousand read the next tile)
    say(f"decode repeatable B={B}")
    d = decode_case(B, 8, 2, 128, 1100, 1, 1100, base=730 + B)
    outs = [run_decode(d)[0].cpu().numpy() for _ in range(8)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
