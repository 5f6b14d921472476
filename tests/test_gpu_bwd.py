"""The gradient (sdpa_fwd_lse + sdpa_bwd) against the fp64 oracle gradient, on the GPU.

Page "Neural Network primitives from NNlib.jl", section "Fused implementation": the gradient
with respect to query, key, value and scale; rows with no allowed key take no part. The GPU
forward writes the log-sum-exp, the GPU backward starts from it; the oracle computes both from
the inputs alone. Bar: as for the output, with max-abs relative to the gradient's magnitude
(gpu_util.assert_grad_close).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import transformer_attention_sdpa_amd as sa
from gpu_util import say, dev, per_batch, gpu_inputs, assert_close, assert_grad_close, nan_like

pytestmark = pytest.mark.gpu


def run_bwd(w, dout, q_lengths=None, grad_dtype=torch.float32, use_mask_info=False, bq=128, bkv=128,
            out_dtype=torch.float32, mask=None, store_ds=True):
    # store_ds: a workspace with room for the stored dS (the dK/dV pass writes dS and the dQ pass
    # reads it) or the minimum one (the dQ pass forms the weights again); NaN-filled either way,
    # so a dS block the dQ pass reads without its having been written shows
    t = gpu_inputs(w)
    if mask is not None:
        t["mask"] = mask
    info = sa.build_block_mask_info(t["mask"], bq, bkv) if use_mask_info and t["mask"] is not None else None
    kw = dict(scale=w.scale, is_causal=w.is_causal, q_offset=per_batch(w.q_offset),
              kv_lengths=per_batch(w.kv_lengths), q_lengths=per_batch(q_lengths))
    out, lse = sa.sdpa(t["q"], t["k"], t["v"], None, None if info else t["mask"], mask_info=info,
                       return_lse=True, out_dtype=out_dtype, **kw)
    ws = nan_like((max(1, sa.bwd_workspace_bytes(t["q"], t["k"], t["v"], store_ds)),), torch.uint8)
    dq, dk, dv, dsc = sa.sdpa_bwd(t["q"], t["k"], t["v"], out, dev(dout, w.dtype), lse,
                                  None if info else t["mask"], mask_info=info, grad_dtype=grad_dtype,
                                  workspace=ws, **kw)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy()
    return dict(dq=f(dq), dk=f(dk), dv=f(dv), dscale=float(dsc.item()), lse=lse.cpu().numpy())


def run_ref(w, dout, q_lengths=None):
    kw = dict(mask=w.mask, scale=w.scale, is_causal=w.is_causal, q_offset=w.q_offset,
              kv_lengths=w.kv_lengths, q_lengths=q_lengths)
    g = oracle.sdpa_grad(w.values("q"), w.values("k"), w.values("v"), workloads.widen(dout, w.dtype), **kw)
    g["lse"] = oracle.sdpa_lse(w.values("q"), w.values("k"), w.values("v"), **kw)
    return g


def check(got, ref, dtype, label):
    for n in ("dq", "dk", "dv"):
        assert_grad_close(got[n], ref[n], dtype, f"{label} {n}")
    # dscale: the terms of a row cancel, so its error is bounded against the sum of their
    # magnitudes, at the max-abs bar (f32) or the rel-L2 bar (16-bit inputs)
    mag = max(1.0, ref["dscale_abs"])
    tol = 1e-5 if dtype == "f32" else 5e-3
    say(f"  {label} dscale gpu={got['dscale']:.6g} oracle={ref['dscale']:.6g} (terms {ref['dscale_abs']:.4g})")
    assert abs(got["dscale"] - ref["dscale"]) <= tol * mag
    fin = np.isfinite(ref["lse"])
    np.testing.assert_array_equal(np.isfinite(got["lse"]), fin)
    assert np.all(got["lse"][~fin] == -np.inf)
    assert_close(got["lse"][fin], ref["lse"][fin], dtype, f"{label} lse")


FEATURES = [
    dict(),
    dict(is_causal=True),
    dict(is_causal=True, q_offset=[37, -5]),
    dict(is_causal="bottom_right", kv_lengths=[150, 61]),
    dict(kv_lengths=[129, 3]),
    dict(mask_shape=(2, 4, 130, 150)),
    dict(mask_shape=(1, 1, 130, 150), is_causal="bottom_right"),
    dict(scale=-0.3, is_causal=True),
    dict(scale=0.0),
]


@pytest.mark.parametrize("store_ds", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("hkv", [4, 1])
@pytest.mark.parametrize("case", range(len(FEATURES)))
def test_grad_features(lib, case, hkv, D, dtype, store_ds):
    f = dict(FEATURES[case])
    kvl = f.pop("kv_lengths", None)
    qo = f.pop("q_offset", 0)
    w = workloads.random_attention(2000 + case * 7 + hkv + D, 2, 130, 150, 4, hkv, D, dtype=dtype,
                                   q_offset=np.array(qo, dtype=np.int32) if isinstance(qo, list) else qo,
                                   kv_lengths=None if kvl is None else np.array(kvl, dtype=np.int32), **f)
    dout = workloads.output_cotangent(w, 3000 + case)
    say(f"grad case={case} {FEATURES[case]} hkv={hkv} D={D} {dtype} store_ds={store_ds}")
    check(run_bwd(w, dout, store_ds=store_ds), run_ref(w, dout), dtype, f"case {case}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_q_lengths_and_empty_rows(lib, dtype):
    # rows past q_lengths and rows that attend nothing take no part, whatever dout holds there
    w = workloads.random_attention(2100, 2, 70, 90, 4, 2, 64, dtype=dtype, mask_shape=(2, 4, 70, 90))
    w.mask[0, 1, 5, :] = 0
    w.mask[1, :, 9, :] = 0
    ql = np.array([60, 33], dtype=np.int32)
    dout = workloads.output_cotangent(w, 3100)
    say(f"grad q_lengths + empty rows {dtype}")
    got, ref = run_bwd(w, dout, q_lengths=ql), run_ref(w, dout, q_lengths=ql)
    assert np.all(got["dq"][0, 5, 1] == 0) and np.all(got["dq"][1, 9] == 0) and np.all(got["dq"][1, 33:] == 0)
    check(got, ref, dtype, "q_lengths")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_value_head_dim_differs(lib, dtype):
    w = workloads.random_attention(2200, 2, 70, 90, 4, 2, 64, Dv=32, dtype=dtype, is_causal=True)
    dout = workloads.output_cotangent(w, 3200)
    say(f"grad Dv != D {dtype}")
    check(run_bwd(w, dout), run_ref(w, dout), dtype, "dv=32")


@pytest.mark.parametrize("Lkv,bq,bkv,D", [(272, 128, 64, 128), (272, 32, 32, 64), (496, 100, 96, 128), (496, 200, 160, 64)])
def test_grad_mask_info_equals_dense(lib, Lkv, bq, bkv, D):
    # byte rows of 16-byte runs: the dense mask and its block info both take the matrix-core
    # kernels and must agree bit for bit; blocks of every class, block edges off the 64-query and
    # 128-key steps of the kernels, ragged tails
    w = workloads.random_attention(2300 + bq, 2, 200, Lkv, 4, 2, D, dtype="bf16",
                                   mask_shape=(1, 4, 200, Lkv), is_causal="bottom_right")
    w.mask[..., :bq, :bkv] = 1                    # a full block
    w.mask[:, 1, bq:, :] = 0                      # empty blocks
    dout = workloads.output_cotangent(w, 3300)
    say(f"grad with block info Lkv={Lkv} bq={bq} bkv={bkv} D={D}")
    # one forward (its rounding depends on the tiles it visits) feeds both gradients
    t = gpu_inputs(w)
    kw = dict(scale=w.scale, is_causal=w.is_causal)
    out, lse = sa.sdpa(t["q"], t["k"], t["v"], None, t["mask"], return_lse=True, out_dtype=torch.float32, **kw)
    d_o = dev(dout, w.dtype)
    info = sa.build_block_mask_info(t["mask"], bq, bkv)
    # (the dense call on the same route as block info: the dQ pass forms the weights again)
    g_dense = sa.sdpa_bwd(t["q"], t["k"], t["v"], out, d_o, lse, t["mask"], store_ds=False, **kw)
    g_info = sa.sdpa_bwd(t["q"], t["k"], t["v"], out, d_o, lse, None, mask_info=info, **kw)
    torch.cuda.synchronize()
    for n, x, y in zip(("dq", "dk", "dv", "dscale"), g_info, g_dense):
        np.testing.assert_array_equal(x.float().cpu().numpy(), y.float().cpu().numpy(), err_msg=n)
    check(run_bwd(w, dout, use_mask_info=True, bq=bq, bkv=bkv), run_ref(w, dout), "bf16", "block info")


def test_grad_mask_info_unaligned_dense(lib):
    # 260-key byte rows take the generic kernels; the block info of the same mask the matrix-core
    # ones: both against the oracle
    w = workloads.random_attention(2350, 2, 200, 260, 4, 2, 128, dtype="bf16", mask_shape=(1, 4, 200, 260),
                                   is_causal="bottom_right")
    dout = workloads.output_cotangent(w, 3350)
    say("grad with block info, unaligned dense mask")
    ref = run_ref(w, dout)
    check(run_bwd(w, dout), ref, "bf16", "dense mask")
    check(run_bwd(w, dout, use_mask_info=True, bq=128, bkv=64), ref, "bf16", "block info")


@pytest.mark.parametrize("store_ds", [True, False])
@pytest.mark.parametrize("kind", ["u8", "u1"])
@pytest.mark.parametrize("dtype,D,mshape,causal", [("bf16", 128, (2, 8), False), ("f16", 64, (1, 1), "bottom_right"),
                                                   ("bf16", 64, (2, 1), True), ("f16", 128, (1, 8), True)])
def test_grad_mask_matrix_tiles(lib, kind, dtype, D, mshape, causal, store_ds):
    # masks whose rows suit the 16-bit matrix-core kernels (496 keys: 31 16-byte runs of bytes,
    # 16 words of bits) over several query and key tiles, ragged tails, GQA, per-batch kv_lengths,
    # and rows left with no allowed key; U1 padding bits are set, so a read of one would show
    w = workloads.random_attention(2800 + D, 2, 300, 496, 8, 2, D, dtype=dtype, is_causal=causal,
                                   mask_shape=mshape + (300, 496), mask_p=0.6,
                                   kv_lengths=np.array([496, 431], dtype=np.int32))
    w.mask[..., 7, :] = 0
    w.mask[0, ..., 150:260, 200:330] = 0
    dout = workloads.output_cotangent(w, 3800)
    m = None
    if kind == "u1":
        m = sa.PackedMask(torch.as_tensor(workloads.pack_mask_bits(w.mask, 1), device="cuda"), w.mask.shape[-1])
    say(f"grad mask {kind} {dtype} D={D} mask {mshape} causal={causal} store_ds={store_ds}")
    got = run_bwd(w, dout, mask=m, store_ds=store_ds)
    check(got, run_ref(w, dout), dtype, f"mask {kind}")
    if kind == "u1":
        dense = run_bwd(w, dout, store_ds=store_ds)
        for n in ("dq", "dk", "dv"):
            np.testing.assert_array_equal(got[n], dense[n])


@pytest.mark.parametrize("kind", ["u8", "u1"])
def test_grad_key_padding_mask(lib, kind):
    # a key-padding mask [B][1][1][Lkv] (query stride 0) in the matrix-core kernels, GQA, D 128
    w = workloads.random_attention(2900, 2, 260, 496, 8, 2, 128, dtype="bf16", mask_shape=(2, 1, 1, 496))
    w.mask[0, ..., 400:] = 0
    w.mask[1, ..., :37] = 0
    dout = workloads.output_cotangent(w, 3900)
    m = None
    if kind == "u1":
        m = sa.PackedMask(torch.as_tensor(workloads.pack_mask_bits(w.mask, 1), device="cuda"), w.mask.shape[-1])
    say(f"grad key-padding mask {kind}")
    check(run_bwd(w, dout, mask=m), run_ref(w, dout), "bf16", f"key padding {kind}")


@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float16])
def test_grad_16bit_outputs(lib, gdt):
    # 16-bit gradients from a 16-bit saved output (the forward's own dtype)
    w = workloads.random_attention(2400, 2, 130, 150, 4, 2, 128, dtype="bf16", is_causal=True)
    dout = workloads.output_cotangent(w, 3400)
    say(f"grad outputs {gdt}")
    check(run_bwd(w, dout, grad_dtype=gdt, out_dtype=None), run_ref(w, dout), "bf16", f"{gdt}")


def test_grad_is_deterministic(lib):
    w = workloads.random_attention(2500, 2, 300, 300, 8, 2, 128, dtype="bf16", is_causal=True)
    dout = workloads.output_cotangent(w, 3500)
    say("grad repeatable")
    a, b = run_bwd(w, dout), run_bwd(w, dout)
    for n in ("dq", "dk", "dv", "lse"):
        np.testing.assert_array_equal(a[n], b[n])
    assert a["dscale"] == b["dscale"]


@pytest.mark.parametrize("Lq,Lkv", [(0, 40), (40, 0), (1, 1)])
def test_grad_degenerate_lengths(lib, Lq, Lkv):
    w = workloads.random_attention(2600, 2, Lq, Lkv, 2, 1, 64, dtype="bf16")
    dout = workloads.output_cotangent(w, 3600)
    say(f"grad Lq={Lq} Lkv={Lkv}")
    got = run_bwd(w, dout)
    ref = run_ref(w, dout)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(got[n], ref[n], atol=2e-2, rtol=0)
    assert abs(got["dscale"] - ref["dscale"]) <= 2e-2


@pytest.mark.parametrize("store_ds", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_grad_gqa_ragged_several_tiles(lib, dtype, D, store_ds):
    # several 128-key and 128-query tiles with ragged tails, 4 query heads per K/V head,
    # bottom-right causal with per-batch kv_lengths
    w = workloads.random_attention(2700 + D, 2, 300, 777, 8, 2, D, dtype=dtype, is_causal="bottom_right",
                                   kv_lengths=np.array([700, 777], dtype=np.int32))
    dout = workloads.output_cotangent(w, 3700)
    say(f"grad GQA ragged {dtype} D={D} store_ds={store_ds}")
    check(run_bwd(w, dout, store_ds=store_ds), run_ref(w, dout), dtype, "gqa ragged")
