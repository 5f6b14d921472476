"""GPU parity of sdpa_fwd against the fp64 oracle (MI355X only).

Sizes are chosen so the oracle finishes in seconds while the kernels still see several tiles
and a ragged tail. Every option of the NNlib "Arguments" list that the ABI exposes is covered,
alone and combined, in fp32 and bf16, with GQA, MQA and plain multi-head layouts.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev, gpu_inputs, run_gpu, run_oracle, assert_close, per_batch
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu


def test_tiny_f32_workload(lib):
    w = workloads.tiny_f32()
    say("tiny_f32 B1 H2 D16 L64")
    got = run_gpu(w).cpu().numpy()
    assert_close(got, run_oracle(w), "f32", "tiny_f32")


def test_nnlib_examples(lib):
    # page "Neural Network primitives from NNlib.jl", "Examples": shapes in (head_dim, heads, seq,
    # batch) order, inputs uniform in [0, 1) as there
    say("nnlib examples")
    basic = workloads.random_attention(11, 4, 20, 30, 8, 8, 16, dist="uniform")
    assert_close(run_gpu(basic).cpu().numpy(), run_oracle(basic), "f32", "basic (16,8,20,4)")
    gqa = workloads.random_attention(12, 4, 20, 30, 8, 2, 16, dist="uniform")
    out = run_gpu(gqa)
    assert tuple(out.shape) == (4, 20, 8, 16)
    assert_close(out.cpu().numpy(), run_oracle(gqa), "f32", "gqa 8 over 2")
    gqa.kv_lengths = np.array([12, 30, 30, 30], dtype=np.int32)
    assert_close(run_gpu(gqa).cpu().numpy(), run_oracle(gqa), "f32", "padded kv_lengths")
    dec = workloads.random_attention(13, 4, 3, 64, 8, 8, 16, dist="uniform")
    dec.is_causal, dec.kv_lengths = "bottom_right", np.array([13, 23, 33, 43], dtype=np.int32)
    a = run_gpu(dec).cpu().numpy()
    assert_close(a, run_oracle(dec), "f32", "decode bottom_right")
    dec.is_causal, dec.q_offset = True, np.array([10, 20, 30, 40], dtype=np.int32)
    b = run_gpu(dec).cpu().numpy()
    np.testing.assert_array_equal(a, b)          # the two spellings are the same call


FEATURES = [
    dict(),
    dict(is_causal=True),
    dict(is_causal=True, q_offset=[37, -5]),
    dict(is_causal="bottom_right", kv_lengths=[150, 61]),
    dict(kv_lengths=[129, 3]),
    dict(bias_shape=(2, 4, 130, 150)),
    dict(bias_shape=(1, 4, 1, 150), is_causal=True),
    dict(bias_shape=(2, 1, 130, 1), kv_lengths=[100, 150]),
    dict(mask_shape=(2, 4, 130, 150)),
    dict(mask_shape=(1, 1, 130, 150), is_causal="bottom_right"),
    dict(mask_shape=(2, 1, 130, 150), bias_shape=(1, 4, 130, 150), is_causal=True, q_offset=20,
         kv_lengths=[140, 90]),
    dict(qk_norm=True),
    dict(qk_norm=True, is_causal=True, bias_shape=(2, 4, 130, 150)),
    dict(scale=0.0),
    dict(scale=-0.3, is_causal=True),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("hkv", [4, 1])
@pytest.mark.parametrize("case", range(len(FEATURES)))
def test_features(lib, case, hkv, D, dtype):
    f = dict(FEATURES[case])
    kvl = f.pop("kv_lengths", None)
    qo = f.pop("q_offset", 0)
    w = workloads.random_attention(1000 + case * 7 + hkv + D, 2, 130, 150, 4, hkv, D, dtype=dtype,
                                   bias_dtype="bf16" if dtype == "bf16" else "f32",   # f16: fp32 bias
                                   q_offset=np.array(qo, dtype=np.int32) if isinstance(qo, list) else qo,
                                   kv_lengths=None if kvl is None else np.array(kvl, dtype=np.int32), **f)
    say(f"features case={case} {FEATURES[case]} hkv={hkv} D={D} {dtype}")
    assert_close(run_gpu(w).cpu().numpy(), run_oracle(w), dtype, f"case {case}")
    if w.mask is not None and dtype != "f32":
        # the block-info path gives the same numbers as the dense mask
        info = run_gpu(w, use_mask_info=True, bq=128, bkv=64).cpu().numpy()
        np.testing.assert_array_equal(info, run_gpu(w).cpu().numpy())


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_value_head_dim_differs(lib, dtype):
    w = workloads.random_attention(77, 2, 70, 90, 4, 2, 64, Dv=32, dtype=dtype, is_causal=True)
    say(f"Dv != D {dtype}")
    assert_close(run_gpu(w).cpu().numpy(), run_oracle(w), dtype, "dv=32")


def test_q_lengths_zero_rows(lib):
    w = workloads.random_attention(78, 2, 50, 60, 2, 2, 64, dtype="bf16", is_causal="bottom_right")
    ql = np.array([20, 50], dtype=np.int32)
    say("q_lengths")
    got = run_gpu(w, q_lengths=ql).cpu().numpy()
    ref = run_oracle(w, q_lengths=ql)
    assert np.all(got[0, 20:] == 0.0)
    assert_close(got, ref, "bf16", "q_lengths")


def test_bf16_output(lib):
    w = workloads.random_attention(79, 2, 200, 200, 4, 2, 128, dtype="bf16", is_causal=True)
    say("bf16 output")
    got = run_gpu(w, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert_close(got, run_oracle(w), "bf16", "bf16 out")


def test_fully_masked_rows_are_nan(lib):
    say("fully masked rows")
    w = workloads.random_attention(80, 2, 40, 70, 2, 1, 64, dtype="bf16", is_causal=True,
                                   q_offset=np.array([-3, 0], dtype=np.int32))
    got = run_gpu(w).cpu().numpy()
    assert np.isnan(got[0, :3]).all() and np.isfinite(got[0, 3:]).all()
    assert_close(got, run_oracle(w), "bf16", "negative offset")
    w.kv_lengths = np.array([0, 70], dtype=np.int32)
    got = run_gpu(w).cpu().numpy()
    assert np.isnan(got[0]).all()
    assert_close(got, run_oracle(w), "bf16", "kv_lengths 0")
    w2 = workloads.random_attention(81, 1, 40, 70, 2, 2, 64, dtype="bf16", mask_shape=(1, 2, 40, 70))
    w2.mask[0, 1, 7] = 0
    got = run_gpu(w2).cpu().numpy()
    assert np.isnan(got[0, 7, 1]).all()
    assert_close(got, run_oracle(w2), "bf16", "all-false mask row")


def test_empty_keys_and_queries(lib):
    say("empty")
    w = workloads.random_attention(82, 2, 5, 0, 2, 2, 64, dtype="bf16")
    assert np.isnan(run_gpu(w).cpu().numpy()).all()
    w = workloads.random_attention(83, 2, 0, 9, 2, 2, 64, dtype="bf16")
    assert run_gpu(w).shape == (2, 0, 2, 64)


@pytest.mark.parametrize("causal", [False, "bottom_right"])
def test_kv_tail_poison_is_never_read(lib, causal):
    # keys past kv_lengths hold NaN: the output must not see them (0 * NaN would be NaN)
    w = workloads.random_attention(84, 2, 100, 200, 4, 2, 128, dtype="bf16", is_causal=causal,
                                   kv_lengths=np.array([77, 130], dtype=np.int32))
    for b, n in enumerate(w.kv_lengths):
        w.k[b, n:] = workloads.BF16_NAN_BITS
        w.v[b, n:] = workloads.BF16_NAN_BITS
    say(f"nan tail causal={causal}")
    got = run_gpu(w).cpu().numpy()
    if not causal:
        assert np.isfinite(got).all()
    else:
        # kv_len 77 < q_len 100: the first 23 queries of batch 0 see no key (NaN by the pages)
        assert np.isnan(got[0, :23]).all() and np.isfinite(got[0, 23:]).all() and np.isfinite(got[1]).all()
    assert_close(got, run_oracle(w), "bf16", "nan tail")


def test_strided_views(lib):
    # q/k/v as views with padded strides (heads-major storage transposed into [B][L][H][D])
    say("strided views")
    g = torch.Generator().manual_seed(5)
    qb = torch.randn(2, 4, 90, 64 + 8, generator=g)[..., :64]
    kb = torch.randn(2, 2, 110, 64, generator=g)
    vb = torch.randn(2, 2, 110, 64, generator=g)
    q = qb.to(torch.bfloat16).cuda().transpose(1, 2)
    k = kb.to(torch.bfloat16).cuda().transpose(1, 2)
    v = vb.to(torch.bfloat16).cuda().transpose(1, 2)
    out_store = torch.empty(2, 4, 90, 64, dtype=torch.float32, device="cuda")
    out = out_store.transpose(1, 2)
    sa.sdpa(q, k, v, is_causal=True, out=out)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q.float().cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy(), is_causal=True)
    assert_close(out.cpu().numpy(), ref, "bf16", "strided")


def test_bias_minus_inf_acts_as_mask(lib):
    say("bias -inf")
    w = workloads.random_attention(85, 1, 64, 96, 2, 2, 64, dtype="f32", bias_shape=(1, 2, 64, 96))
    w.bias[0, :, :, 50:] = -np.inf
    got = run_gpu(w).cpu().numpy()
    m = np.ones((1, 1, 64, 96), dtype=np.uint8)
    m[..., 50:] = 0
    w2 = workloads.random_attention(85, 1, 64, 96, 2, 2, 64, dtype="f32", bias_shape=(1, 2, 64, 96))
    w2.mask = m
    assert_close(got, run_oracle(w2), "f32", "bias -inf vs mask")


@pytest.mark.parametrize("variant", ["dense", "info"])
def test_debug_allowed_mask_bit_exact(lib, variant):
    say(f"allowed mask {variant}")
    B, Lq, Lkv, H = 2, 77, 200, 3
    rng = np.random.default_rng(9)
    mask = workloads.block_sparse_mask(Lq, Lkv, 32, k=9, shape_prefix=(2, 1))
    q = torch.zeros(B, Lq, H, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, Lkv, H, 64, dtype=torch.bfloat16, device="cuda")
    md = dev(mask, "u8")
    info = sa.build_block_mask_info(md, 32, 64) if variant == "info" else None
    for causal, qo, kvl, ql in [(False, 0, None, None), (True, [5, -2], [150, 200], None),
                                ("bottom_right", 0, [180, 64], [77, 50]), (True, 120, None, None)]:
        got = sa.debug_allowed_mask(q, k, None if info else md, mask_info=info, is_causal=causal,
                                    q_offset=per_batch(np.array(qo, dtype=np.int32)) if isinstance(qo, list) else qo,
                                    kv_lengths=per_batch(np.array(kvl, dtype=np.int32)) if kvl else None,
                                    q_lengths=per_batch(np.array(ql, dtype=np.int32)) if ql else None).cpu().numpy()
        kvl_c = [min(max(x, 0), Lkv) for x in kvl] if kvl else None
        ql_c = ql if ql else None
        offs = oracle.causal_offsets(causal, qo, kvl_c, ql_c, B, Lq, Lkv)
        for b in range(B):
            for h in range(H):
                ref = oracle.allowed_matrix(np.arange(Lq), Lkv, b, h, B, H, mask,
                                            None if offs is None else offs[b], None if kvl_c is None else kvl_c[b])
                np.testing.assert_array_equal(got[b, h], ref.astype(np.uint8))


@pytest.mark.parametrize("D", [64, 128])
def test_f16_bias_and_f16_output(lib, D):
    # an f16 bias (the general kernel) and f16 outputs (both kernels) against the oracle
    say(f"f16 bias, f16 out, D={D}")
    w = workloads.random_attention(91 + D, 2, 130, 150, 4, 2, D, dtype="f16", bias_shape=(2, 4, 130, 150),
                                   bias_dtype="f16", is_causal=True)
    assert_close(run_gpu(w).cpu().numpy(), run_oracle(w), "f16", "f16 bias")
    w2 = workloads.random_attention(95 + D, 2, 130, 150, 4, 2, D, dtype="f16", is_causal=True)
    out = run_gpu(w2, out_dtype=torch.float16)
    assert out.dtype == torch.float16
    assert_close(out.float().cpu().numpy(), run_oracle(w2), "f16", "f16 out")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bias_shape", [(2, 4, 130, 150), (1, 4, 130, 150), (2, 1, 1, 150)])
def test_bf16_bias_fused_path_d64(lib, dtype, bias_shape):
    # a bf16 bias at head dim 64 enters the q.k MFMAs as their start value; 150 keys leave a
    # ragged 6-key tail whose bias is loaded element by element; with block info as well
    w = workloads.random_attention(4100 + bias_shape[0] + bias_shape[2], 2, 130, 150, 4, 2, 64, dtype=dtype,
                                   bias_shape=bias_shape, bias_dtype="bf16", mask_shape=(1, 1, 130, 150))
    say(f"bf16 bias fused D=64 {dtype} {bias_shape}")
    assert_close(run_gpu(w).cpu().numpy(), run_oracle(w), dtype, "bias dense mask")
    assert_close(run_gpu(w, use_mask_info=True, bq=128, bkv=64).cpu().numpy(), run_oracle(w), dtype, "bias info")


@pytest.mark.parametrize("D,dtype,bias_dtype", [(64, "bf16", "bf16"), (128, "bf16", "bf16"), (64, "bf16", "f32"),
                                                (128, "f16", "f32"), (32, "bf16", "bf16")])
def test_bias_at_dtype_minimum_is_finite(lib, D, dtype, bias_dtype):
    # an additive mask filled with the bias dtype's most negative finite value: the logits stay
    # finite ("Arguments": the bias is added to the logits), so a row whose every key carries it
    # is the mean of the values, and such keys get no weight in a row that also has ordinary
    # keys. Covers the fused bias (D 64, bf16), the per-element bias (D 128, f32 bias) and the
    # general kernel (D 32); a -inf bias stays a masked key
    say(f"bias at the dtype minimum D={D} {dtype} bias {bias_dtype}")
    w = workloads.random_attention(4200 + D, 2, 130, 150, 4, 2, D, dtype=dtype, bias_shape=(2, 4, 130, 150),
                                   bias_dtype=bias_dtype, is_causal=True, q_offset=20)
    lo = np.finfo(np.float32).min if bias_dtype == "f32" else None
    if bias_dtype == "bf16":
        w.bias[0, :, 3, :] = 0xFF7F                           # bf16 -3.39e38: the whole row
        w.bias[1, :, 70, :75] = 0xFF7F                        # half of a row
        w.bias[1, 2, 100, :] = 0xFF80                         # -inf: the whole row is masked
    else:
        w.bias[0, :, 3, :] = lo
        w.bias[1, :, 70, :75] = lo
        w.bias[1, 2, 100, :] = -np.inf
    ref = run_oracle(w)
    assert np.isfinite(ref[0, 3]).all() and np.isnan(ref[1, 100, 2]).all()
    assert_close(run_gpu(w).cpu().numpy(), ref, dtype, "bias at the dtype minimum")


@pytest.mark.parametrize("shape", [(2, 16, 16), (4, 8, 2)])
def test_causal_grouped_head_order_whole_output(lib, shape):
    # a causal launch with B * Hq a multiple of 32 takes the grouped order (every XCD runs its
    # heads four at a time, longest query tile first), as the full-size causal prefill does;
    # every element against the oracle, with 640 queries (five 128-row tiles)
    B, Hq, Hkv = shape
    say(f"causal grouped order B{B} Hq{Hq} Hkv{Hkv} D128 L640")
    w = workloads.random_attention(4300 + Hq, B, 640, 640, Hq, Hkv, 128, dtype="bf16", is_causal=True)
    t = gpu_inputs(w)
    out = torch.full((B, 640, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    sa.sdpa(t["q"], t["k"], t["v"], is_causal=True, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), run_oracle(w), "bf16", "grouped causal order")


def test_side_stream(lib):
    # a call on a side stream: the binding's temporaries (per-batch lengths from a host list,
    # the workspace, the default output) are made on that stream, so the result equals the same
    # call on the current stream
    say("side stream")
    w = workloads.random_attention(4400, 3, 130, 150, 4, 2, 128, dtype="bf16", is_causal="bottom_right",
                                   kv_lengths=np.array([150, 77, 9], dtype=np.int32))
    t = gpu_inputs(w)
    ref = sa.sdpa(t["q"], t["k"], t["v"], is_causal="bottom_right", kv_lengths=[150, 77, 9], out_dtype=torch.float32)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    got = sa.sdpa(t["q"], t["k"], t["v"], is_causal="bottom_right", kv_lengths=[150, 77, 9], out_dtype=torch.float32,
                  stream=s)
    d = workloads.gqa_decode(B=3, Hq=8, Hkv=2, D=128, capacity=300, kv_min=50, kv_max=300, base=4401)
    kc, vc = dev(d.k_cache, "bf16"), dev(d.v_cache, "bf16")
    qd = dev(d.q, "bf16")
    torch.cuda.synchronize()
    sa.kv_cache_update(kc, vc, dev(d.k_new, "bf16"), dev(d.v_new, "bf16"), d.write_index.tolist(), stream=s)
    od = sa.sdpa_decode(qd, kc, vc, d.kv_lengths.tolist(), scale=d.scale, out_dtype=torch.float32, stream=s)
    s.synchronize()
    # rows of the third sequence before its 9 keys attend nothing: NaN in both
    assert torch.equal(torch.isnan(got), torch.isnan(ref)) and torch.isnan(got).any()
    assert torch.equal(torch.nan_to_num(got, nan=5.0), torch.nan_to_num(ref, nan=5.0))
    assert_close(got.cpu().numpy(), run_oracle(w), "bf16", "side stream prefill")
    ekc, evc = oracle.kv_cache_update(d.k_cache, d.v_cache, d.k_new, d.v_new, d.write_index)
    f = workloads.bf16_to_f32
    refd = np.stack([oracle.sdpa(f(d.q[b:b + 1]), f(ekc[b:b + 1, :d.kv_lengths[b]]), f(evc[b:b + 1, :d.kv_lengths[b]]),
                                 scale=d.scale, is_causal="bottom_right")[0] for b in range(3)])
    assert_close(od.cpu().numpy(), refd, "bf16", "side stream decode")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_logit_jumps_move_the_running_max(lib, dtype, D, causal):
    # keys 0..63 give logits near 1 (log2 units), keys 64..191 near 130 and keys 192.. near 260:
    # the running max set by the first tile is far below the later logits, whose exponentials
    # would overflow against it; the kernels must move the max before those reach P.V
    say(f"logit jumps D={D} {dtype} causal={causal}")
    B, L, H = 1, 300, 2
    rng = np.random.default_rng(77 + D)
    q = np.ones((B, L, H, D), dtype=np.float32)
    k = np.empty((B, L, H, D), dtype=np.float32)
    lvl = np.where(np.arange(L) < 64, 0.1, np.where(np.arange(L) < 192, 8.0, 16.0)) * math.sqrt(128 / D)
    k[:] = (lvl[None, :, None, None] * (1.0 + 0.002 * (np.arange(L) % 7))[None, :, None, None])
    v = rng.standard_normal((B, L, H, D), dtype=np.float32)
    w = workloads.Attention("jumps", dtype, workloads.to_storage(q, dtype), workloads.to_storage(k, dtype),
                            workloads.to_storage(v, dtype), scale=1.0 / math.sqrt(D), is_causal=causal)
    ref = run_oracle(w)
    assert np.isfinite(ref).all()
    assert_close(run_gpu(w).cpu().numpy(), ref, dtype, "logit jumps")


@pytest.mark.parametrize("slope", [0.3, 2.0])
@pytest.mark.parametrize("D,bias_dtype,info", [(64, "bf16", False), (64, "bf16", True), (128, "bf16", False),
                                               (64, "f32", False), (128, "f32", True)])
def test_rising_bias_moves_the_running_max(lib, slope, D, bias_dtype, info):
    # a bias rising along the keys, slope * (j - i) (the ALiBi form of the fourth workload, with
    # a steep slope): a row's max grows by slope * 64 per 64-key tile, so the kernels move it on
    # many tiles, each time past the new maximum. slope 2 moves it on every tile, slope 0.3 on
    # about every third; causal with a random mask, also through block info
    say(f"rising bias slope {slope} D={D} bias {bias_dtype} info={info}")
    B, Lq, Lkv, H = 2, 200, 400, 4
    w = workloads.random_attention(4300 + D + int(10 * slope), B, Lq, Lkv, H, 2, D, dtype="bf16",
                                   bias_shape=(1, H, Lq, Lkv), bias_dtype=bias_dtype,
                                   mask_shape=(1, 1, Lq, Lkv), mask_p=0.6, is_causal=True, q_offset=150)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lkv)[None, :]
    ramp = slope * (j - i).astype(np.float64) * (1.0 + 0.25 * np.arange(H))[:, None, None]
    w.bias = (workloads.f64_to_bf16(ramp) if bias_dtype == "bf16" else ramp.astype(np.float32))[None]
    ref = run_oracle(w)
    assert_close(run_gpu(w, use_mask_info=info, bq=128, bkv=64).cpu().numpy(), ref, "bf16",
                 f"rising bias slope {slope}")


def test_path_queries_name_the_kernels_that_run(lib):
    # the benchmark's shapes on the matrix cores (the stored-dS gradient with the default
    # workspace, the recompute route with the minimum one), fp32 inputs and an odd head dim on
    # the fp32 kernels; the fp32 call's result still matches the oracle
    say("path queries")
    q, k, v = (torch.zeros((2, 256, 4, 128), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    assert sa.sdpa_fwd_path(q, k, v, is_causal=True) == "matrix_core"
    o = torch.zeros_like(q)
    assert sa.sdpa_bwd_path(q, k, v, o, o, is_causal=True) == "matrix_core_stored_ds"
    assert sa.sdpa_bwd_path(q, k, v, o, o, is_causal=True, store_ds=False) == "matrix_core"
    q96 = torch.zeros((2, 64, 4, 96), dtype=torch.bfloat16, device="cuda")
    assert sa.sdpa_fwd_path(q96, q96, q96) == "fp32"
    w = workloads.random_attention(4401, 1, 40, 50, 4, 2, 64, dtype="f32", is_causal=True)
    t = gpu_inputs(w)
    qf, kf, vf = t["q"], t["k"], t["v"]
    assert sa.sdpa_fwd_path(qf, kf, vf, is_causal=True) == "fp32"
    assert_close(run_gpu(w).cpu().numpy(), run_oracle(w), "f32", "fp32 path")
