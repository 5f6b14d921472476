"""GPU parity at the five workloads' full sizes, in the launch configurations the benchmark
times. Every output element is compared with the fp64 oracle on the same values (the long
context chunk: eight whole heads, one per K/V group, every query tile of each). Outputs,
decode workspaces and gradient workspaces are NaN-filled before each call, so an element or a
split slot that a kernel fails to write fails the comparison instead of passing on stale data.

The oracle runs over (batch, head) slices on a thread pool (gpu_util.oracle_pool); each slice
is an independent attention problem, the K/V head of a query head being fixed by the grouping
rule.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev, gpu_inputs, assert_close, oracle_pool, nan_like
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu
f32 = workloads.bf16_to_f32


def _plane(a, b, h):
    """The [1][1][Lq][Lkv] plane of a [Bb][Hb][Lq][Lkv] bias or mask for (b, h) (size-1 dims
    broadcast)."""
    bb = b if a.shape[0] > 1 else 0
    hh = h if a.shape[1] > 1 else 0
    return a[bb:bb + 1, hh:hh + 1]


def _slices_oracle(w, heads=None):
    """Oracle output [B][Lq][Hq][Dv] of workload w (or of the listed query heads only, NaN
    elsewhere), one (batch, head) slice per pool job."""
    q, k, v = w.values("q"), w.values("k"), w.values("v")
    B, Lq, Lkv, Hq, Hkv, D, Dv = w.shape
    r = Hq // Hkv
    heads = range(Hq) if heads is None else heads

    def job(b, h):
        def run():
            g = h // r
            # the bias plane is widened inside the job, so only the running jobs hold one
            bias = None if w.bias is None else workloads.widen(_plane(w.bias, b, h), w.bias_dtype)
            mask = None if w.mask is None else _plane(w.mask, b, h)
            qo = w.q_offset if np.isscalar(w.q_offset) else int(w.q_offset[b])
            kvl = None if w.kv_lengths is None else int(w.kv_lengths[b])
            return oracle.sdpa(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
                               bias=bias, mask=mask, scale=w.scale, is_causal=w.is_causal, q_offset=qo,
                               kv_lengths=kvl)
        return run
    pairs = [(b, h) for b in range(B) for h in heads]
    res = oracle_pool([job(b, h) for b, h in pairs])
    out = np.full((B, Lq, Hq, Dv), np.nan)
    for (b, h), o in zip(pairs, res):
        out[b, :, h] = o[0, :, 0]
    return out


def test_causal_prefill_b4_h16_d128_l4096(lib):
    say("full size: causal prefill B4 H16 D128 L4096, whole output")
    w = workloads.causal_prefill()
    t = gpu_inputs(w)
    B, Lq, _, Hq, _, D, _ = w.shape
    ref = _slices_oracle(w)
    for out_dtype in (torch.float32, torch.bfloat16):      # bf16 is what the benchmark times
        out = nan_like((B, Lq, Hq, D), out_dtype)
        sa.sdpa(t["q"], t["k"], t["v"], is_causal=True, scale=w.scale, out=out)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy(), ref, "bf16", f"causal prefill, every element, out {out_dtype}")
        if out_dtype == torch.float32:
            # causal row 0 sees one key: p = 1, so the output is V's row 0 exactly
            assert torch.equal(out[:, 0], t["v"][:, 0].float())


def test_gqa_decode_b64_hq32_hkv8_cap8192(lib):
    say("full size: GQA decode B64 Hq32 Hkv8 D128 cap 8192, every sequence")
    d = workloads.gqa_decode()
    B, _, Hq, D = d.q.shape
    q = dev(d.q, "bf16")
    kc, vc = dev(d.k_cache, "bf16"), dev(d.v_cache, "bf16")
    kn, vn = dev(d.k_new, "bf16"), dev(d.v_new, "bf16")
    widx = dev(d.write_index, "i32")
    kvl = dev(d.kv_lengths, "i32")
    sa.kv_cache_update(kc, vc, kn, vn, widx)
    need = sa.decode_workspace_bytes(q, kc, 0)
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        outs[dt] = nan_like((B, 1, Hq, D), dt)
        sa.sdpa_decode(q, kc, vc, kvl, scale=d.scale, out=outs[dt], workspace=nan_like((need,), torch.uint8))
    torch.cuda.synchronize()
    # the written rows are the new rows, bit for bit
    bidx = torch.arange(B, device="cuda")
    wi = widx.long()
    assert torch.equal(kc[bidx, wi].view(torch.int16), kn[:, 0].view(torch.int16))
    assert torch.equal(vc[bidx, wi].view(torch.int16), vn[:, 0].view(torch.int16))
    lens = d.kv_lengths
    ekc, evc = oracle.kv_cache_update(d.k_cache, d.v_cache, d.k_new, d.v_new, d.write_index)
    jobs = [(lambda b=b: oracle.sdpa(f32(d.q[b:b + 1]), f32(ekc[b:b + 1, :lens[b]]), f32(evc[b:b + 1, :lens[b]]),
                                     scale=d.scale, is_causal="bottom_right")[0]) for b in range(B)]
    ref = np.stack(oracle_pool(jobs))
    for dt, o in outs.items():
        assert_close(o.float().cpu().numpy(), ref, "bf16", f"decode, all {B} sequences, out {dt}")


def test_bias_block_mask_b2_h16_d64_l8192(lib):
    say("full size: ALiBi bias + block-sparse mask B2 H16 D64 L8192, whole output")
    w = workloads.bias_block_mask()
    t = gpu_inputs(w)
    B, Lq, _, Hq, _, D, _ = w.shape
    info = sa.build_block_mask_info(t["mask"], 128, 128)
    out_info = nan_like((B, Lq, Hq, D), torch.float32)
    out_dense = nan_like((B, Lq, Hq, D), torch.float32)
    out_b16 = nan_like((B, Lq, Hq, D), torch.bfloat16)
    sa.sdpa(t["q"], t["k"], t["v"], t["bias"], None, mask_info=info, scale=w.scale, out=out_info)
    sa.sdpa(t["q"], t["k"], t["v"], t["bias"], t["mask"], scale=w.scale, out=out_dense)
    sa.sdpa(t["q"], t["k"], t["v"], t["bias"], None, mask_info=info, scale=w.scale, out=out_b16)
    torch.cuda.synchronize()
    # skipping empty blocks and dropping the per-element test on full blocks changes nothing
    assert torch.equal(torch.nan_to_num(out_info, nan=7.0), torch.nan_to_num(out_dense, nan=7.0))
    assert torch.equal(torch.isnan(out_info), torch.isnan(out_dense))
    ref = _slices_oracle(w)
    # rows whose mask row is all false are NaN in both (NaN positions must agree exactly)
    assert_close(out_info.cpu().numpy(), ref, "bf16", "bias + block mask, every element")
    assert_close(out_b16.float().cpu().numpy(), ref, "bf16", "bias + block mask, every element, bf16 out")


def test_chunked_prefill_b1_hq32_hkv8_kv131072(lib):
    say("full size: chunked prefill B1 Hq32 Hkv8 D128 kv 131072 q 2048 at offset 129024")
    w = workloads.chunked_prefill()
    t = gpu_inputs(w)
    B, Lq, _, Hq, _, D, _ = w.shape
    out = nan_like((B, Lq, Hq, D), torch.float32)
    sa.sdpa(t["q"], t["k"], t["v"], is_causal=True, q_offset=w.q_offset, scale=w.scale, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    # one query head of every K/V group (r = 4: heads 4g + g % 4), every query row of each
    heads = [4 * g + g % 4 for g in range(8)]
    ref = _slices_oracle(w, heads)
    assert_close(out[:, :, heads].cpu().numpy(), ref[:, :, heads], "bf16", f"chunked prefill heads {heads}")


def _poisoned_grads(q, k, v):
    return (nan_like(q.shape, q.dtype), nan_like(k.shape, k.dtype), nan_like(v.shape, v.dtype),
            nan_like((1,), torch.float32))


@pytest.mark.parametrize("store_ds", [True, False])
def test_causal_prefill_gradient_b4_h16_d128_l4096(lib, store_ds):
    # the gradient in the benchmark's configuration (bf16 inputs, saved output and gradients in
    # bf16): every row of two whole (batch, head) slices against the fp64 oracle gradient of the
    # slice (one K/V head per query head, so a slice is an independent attention); every entry
    # of all slices finite, with outputs and workspace NaN-filled first
    say(f"full size: gradient of the causal prefill B4 H16 D128 L4096, store_ds={store_ds}")
    from gpu_util import assert_grad_close
    w = workloads.causal_prefill()
    t = gpu_inputs(w)
    out, lse = sa.sdpa(t["q"], t["k"], t["v"], is_causal=True, scale=w.scale, out_dtype=torch.float32,
                       return_lse=True)
    dout_np = workloads.output_cotangent(w, 7)
    grads = _poisoned_grads(t["q"], t["k"], t["v"])
    ws = nan_like((sa.bwd_workspace_bytes(t["q"], t["k"], t["v"], store_ds),), torch.uint8)
    dq, dk, dv, dsc = sa.sdpa_bwd(t["q"], t["k"], t["v"], out.to(torch.bfloat16), dev(dout_np, "bf16"), lse,
                                  is_causal=True, scale=w.scale, grads=grads, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
    assert torch.isfinite(dsc).all()
    do64 = workloads.widen(dout_np, "bf16")
    for b, h in ((0, 0), (3, 15)):
        sl = lambda x: x[b:b + 1, :, h:h + 1]
        ref = oracle.sdpa_grad(sl(w.values("q")), sl(w.values("k")), sl(w.values("v")), sl(do64),
                               scale=w.scale, is_causal=True)
        for n, g_ in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert_grad_close(g_[b:b + 1, :, h:h + 1].float().cpu().numpy(), ref[n], "bf16", f"({b},{h}) {n}")
        # the lse of the slice
        lref = oracle.sdpa_lse(sl(w.values("q")), sl(w.values("k")), sl(w.values("v")), scale=w.scale,
                               is_causal=True)
        assert_close(lse[b:b + 1, h:h + 1].cpu().numpy(), lref, "bf16", f"({b},{h}) lse")


def test_causal_prefill_gradient_window_mask_b4_h16_d128_l4096(lib):
    # the gradient at the same size with a 1024-key sliding window on top of causal, given as a
    # byte mask and as its 128 x 128 block info (whose empty steps the kernels skip): the two agree
    # bit for bit; every row of one whole (batch, head) slice against the fp64 oracle gradient
    say("full size: gradient of the causal prefill B4 H16 D128 L4096 with a 1024-key window")
    from gpu_util import assert_grad_close
    w = workloads.causal_prefill()
    L = w.q.shape[1]
    band = ((np.arange(L)[:, None] - np.arange(L)[None, :]) < 1024).astype(np.uint8)[None, None]
    t = gpu_inputs(w)
    m8 = dev(band, "u8")
    info = sa.build_block_mask_info(m8, 128, 128)
    out, lse = sa.sdpa(t["q"], t["k"], t["v"], None, m8, is_causal=True, scale=w.scale,
                       out_dtype=torch.float32, return_lse=True)
    d_o = dev(workloads.output_cotangent(w, 9), "bf16")
    wsb = sa.bwd_workspace_bytes(t["q"], t["k"], t["v"])
    g8 = sa.sdpa_bwd(t["q"], t["k"], t["v"], out, d_o, lse, m8, is_causal=True, scale=w.scale,
                     grads=_poisoned_grads(t["q"], t["k"], t["v"]), workspace=nan_like((wsb,), torch.uint8))
    gi = sa.sdpa_bwd(t["q"], t["k"], t["v"], out, d_o, lse, None, mask_info=info, is_causal=True, scale=w.scale,
                     grads=_poisoned_grads(t["q"], t["k"], t["v"]), workspace=nan_like((wsb,), torch.uint8))
    torch.cuda.synchronize()
    for n, x, y in zip(("dq", "dk", "dv", "dscale"), gi, g8):
        assert torch.isfinite(x.float()).all(), n
        assert torch.equal(x, y), n
    b, h = 1, 7
    sl = lambda x: x[b:b + 1, :, h:h + 1]
    ref = oracle.sdpa_grad(sl(w.values("q")), sl(w.values("k")), sl(w.values("v")),
                           sl(workloads.widen(workloads.output_cotangent(w, 9), "bf16")), mask=band,
                           scale=w.scale, is_causal=True)
    for n, g_ in zip(("dq", "dk", "dv"), g8):
        assert_grad_close(g_[b:b + 1, :, h:h + 1].float().cpu().numpy(), ref[n], "bf16", f"window ({b},{h}) {n}")
