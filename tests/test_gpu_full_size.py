"""GPU parity at the five workloads' full sizes, in the launch configurations the benchmark
times, checked on sampled outputs the oracle computes row by row and on properties that hold
at any size.

Sampled query rows sit on the kernels' tile edges (128-row query tiles, 64-key K/V tiles), at
the first and last rows and in between. The oracle sees exactly the values the GPU sees.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev, gpu_inputs, assert_close
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu
f32 = workloads.bf16_to_f32


def _rows_oracle(w, rows):
    """Oracle output for query rows `rows` of every (batch, head) of workload w."""
    return oracle.sdpa(w.values("q"), w.values("k"), w.values("v"), bias=w.values("bias"), mask=w.mask,
                       scale=w.scale, is_causal=w.is_causal, q_offset=w.q_offset, kv_lengths=w.kv_lengths,
                       rows=rows)


def test_causal_prefill_b4_h16_d128_l4096(lib):
    say("full size: causal prefill B4 H16 D128 L4096")
    w = workloads.causal_prefill()
    t = gpu_inputs(w)
    rows = [0, 1, 63, 64, 127, 128, 129, 1000, 2047, 2048, 3333, 4094, 4095]
    ref = _rows_oracle(w, rows)
    for out_dtype in (torch.bfloat16, torch.float32):      # bf16 is what the benchmark times
        out = sa.sdpa(t["q"], t["k"], t["v"], is_causal=True, scale=w.scale, out_dtype=out_dtype)
        torch.cuda.synchronize()
        got = out[:, rows].float().cpu().numpy()
        assert_close(got, ref, "bf16", f"causal prefill rows, out {out_dtype}")
        assert torch.isfinite(out).all().item()
        if out_dtype == torch.float32:
            # causal row 0 sees one key: p = 1, so the output is V's row 0 exactly
            v0 = t["v"][:, 0].float()
            assert torch.equal(out[:, 0], v0)


def test_gqa_decode_b64_hq32_hkv8_cap8192(lib):
    say("full size: GQA decode B64 Hq32 Hkv8 D128 cap 8192")
    d = workloads.gqa_decode()
    B, _, Hq, D = d.q.shape
    q = dev(d.q, "bf16")
    kc, vc = dev(d.k_cache, "bf16"), dev(d.v_cache, "bf16")
    kn, vn = dev(d.k_new, "bf16"), dev(d.v_new, "bf16")
    widx = dev(d.write_index, "i32")
    kvl = dev(d.kv_lengths, "i32")
    sa.kv_cache_update(kc, vc, kn, vn, widx)
    outs = {dt: sa.sdpa_decode(q, kc, vc, kvl, scale=d.scale, out_dtype=dt) for dt in (torch.bfloat16, torch.float32)}
    torch.cuda.synchronize()
    # the written rows are the new rows, bit for bit
    bidx = torch.arange(B, device="cuda")
    wi = widx.long()
    assert torch.equal(kc[bidx, wi].view(torch.int16), kn[:, 0].view(torch.int16))
    assert torch.equal(vc[bidx, wi].view(torch.int16), vn[:, 0].view(torch.int16))
    # every output is finite: no slot past kv_lengths (NaN-filled) was read
    for o in outs.values():
        assert torch.isfinite(o).all().item()
    lens = d.kv_lengths
    sel = sorted({0, B // 2, B - 1, int(np.argmin(lens)), int(np.argmax(lens))})
    ekc, evc = oracle.kv_cache_update(d.k_cache[sel], d.v_cache[sel], d.k_new[sel], d.v_new[sel], d.write_index[sel])
    ref = np.stack([oracle.sdpa(f32(d.q[b:b + 1]), f32(ekc[i:i + 1, :lens[b]]), f32(evc[i:i + 1, :lens[b]]),
                                scale=d.scale, is_causal="bottom_right")[0] for i, b in enumerate(sel)])
    for dt, o in outs.items():
        assert_close(o[sel].float().cpu().numpy(), ref, "bf16", f"decode batches {sel}, out {dt}")


def test_bias_block_mask_b2_h16_d64_l8192(lib):
    say("full size: ALiBi bias + block-sparse mask B2 H16 D64 L8192")
    w = workloads.bias_block_mask()
    t = gpu_inputs(w)
    info = sa.build_block_mask_info(t["mask"], 128, 128)
    out_info = sa.sdpa(t["q"], t["k"], t["v"], t["bias"], None, mask_info=info, scale=w.scale,
                       out_dtype=torch.float32)
    out_dense = sa.sdpa(t["q"], t["k"], t["v"], t["bias"], t["mask"], scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # skipping empty blocks and dropping the per-element test on full blocks changes nothing
    assert torch.equal(torch.nan_to_num(out_info, nan=7.0), torch.nan_to_num(out_dense, nan=7.0))
    assert torch.equal(torch.isnan(out_info), torch.isnan(out_dense))
    rows = [0, 1, 127, 128, 4095, 4096, 8190, 8191]
    # not causal: the sampled rows form a problem of their own (bias and mask rows sliced alike)
    ref = oracle.sdpa(f32(w.q[:, rows]), w.values("k"), w.values("v"), bias=f32(w.bias[:, :, rows]),
                      mask=w.mask[..., rows, :], scale=w.scale)
    assert_close(out_info[:, rows].cpu().numpy(), ref, "bf16", "bias + block mask rows")
    # rows whose mask row is all false are NaN, the rest finite
    empty_rows = ~w.mask[0, 0].any(axis=1)
    got_nan = torch.isnan(out_info[0, :, 0, 0]).cpu().numpy()
    np.testing.assert_array_equal(got_nan, empty_rows)


def test_chunked_prefill_b1_hq32_hkv8_kv131072(lib):
    say("full size: chunked prefill B1 Hq32 Hkv8 D128 kv 131072 q 2048 at offset 129024")
    w = workloads.chunked_prefill()
    t = gpu_inputs(w)
    out = sa.sdpa(t["q"], t["k"], t["v"], is_causal=True, q_offset=w.q_offset, scale=w.scale,
                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    rows = [0, 1, 127, 128, 1024, 2046, 2047]
    ref = _rows_oracle(w, rows)
    assert_close(out[:, rows].cpu().numpy(), ref, "bf16", "chunked prefill rows")


def test_causal_prefill_gradient_b4_h16_d128_l4096(lib):
    # the gradient in the benchmark's configuration (bf16 inputs, saved output and gradients in
    # bf16): every row of two whole (batch, head) slices against the fp64 oracle gradient of the
    # slice (one K/V head per query head, so a slice is an independent attention); every entry
    # of all slices finite
    say("full size: gradient of the causal prefill B4 H16 D128 L4096")
    from gpu_util import assert_grad_close
    w = workloads.causal_prefill()
    t = gpu_inputs(w)
    out, lse = sa.sdpa(t["q"], t["k"], t["v"], is_causal=True, scale=w.scale, out_dtype=torch.float32,
                       return_lse=True)
    dout_np = workloads.output_cotangent(w, 7)
    dq, dk, dv, dsc = sa.sdpa_bwd(t["q"], t["k"], t["v"], out.to(torch.bfloat16), dev(dout_np, "bf16"), lse,
                                  is_causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
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
    g8 = sa.sdpa_bwd(t["q"], t["k"], t["v"], out, d_o, lse, m8, is_causal=True, scale=w.scale)
    gi = sa.sdpa_bwd(t["q"], t["k"], t["v"], out, d_o, lse, None, mask_info=info, is_causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for n, x, y in zip(("dq", "dk", "dv", "dscale"), gi, g8):
        assert torch.equal(x, y), n
    b, h = 1, 7
    sl = lambda x: x[b:b + 1, :, h:h + 1]
    ref = oracle.sdpa_grad(sl(w.values("q")), sl(w.values("k")), sl(w.values("v")),
                           sl(workloads.widen(workloads.output_cotangent(w, 9), "bf16")), mask=band,
                           scale=w.scale, is_causal=True)
    for n, g_ in zip(("dq", "dk", "dv"), g8):
        assert_grad_close(g_[b:b + 1, :, h:h + 1].float().cpu().numpy(), ref[n], "bf16", f"window ({b},{h}) {n}")
