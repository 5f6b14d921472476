"""Masks given as packed bits (U1), 8x smaller than a byte mask: the answer to the splash-attention
pull request's review of masks at 100k+ contexts ("packed bool values"). Block info and attention
from bits must equal the same from bytes, bit for bit, and the oracle (MI355X only).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev, assert_close
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu


def packed(mask, pad_bit=1):
    words = torch.as_tensor(workloads.pack_mask_bits(mask, pad_bit), device="cuda")
    return sa.PackedMask(words, mask.shape[-1])


@pytest.mark.parametrize("shape,bq,bkv,block", [((1, 1, 300, 260), 64, 64, 64), ((2, 3, 130, 100), 32, 32, 32),
                                                ((1, 2, 512, 384), 128, 128, 128), ((1, 1, 5, 33), 16, 32, 16),
                                                ((2, 1, 257, 1000), 128, 96, 32)])
def test_block_info_from_bits(lib, shape, bq, bkv, block):
    # padding bits past Lkv are set, so a read of them would show
    say(f"U1 mask info {shape} bq={bq} bkv={bkv}")
    Mb, Mh, Lq, Lkv = shape
    mask = workloads.block_sparse_mask(Lq, Lkv, block, k=13, shape_prefix=(Mb, Mh))
    got = sa.build_block_mask_info(packed(mask), bq, bkv).to_numpy()
    byt = sa.build_block_mask_info(dev(mask, "u8"), bq, bkv).to_numpy()
    ref = oracle.block_mask_info(mask, bq, bkv)
    for key in ("block_mask", "mask_next", "row_ptr", "data_next", "partial_bits"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
        np.testing.assert_array_equal(got[key], byt[key], err_msg=key)
    assert got["n_partial"] == ref["n_partial"]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 16)])
@pytest.mark.parametrize("mshape", [(1, 1), (2, 4), (2, 1)])
def test_attention_with_bit_mask(lib, dtype, D, mshape):
    say(f"U1 dense mask {mshape} {dtype} D={D}")
    w = workloads.random_attention(61 + D, 2, 130, 150, 4, 2, D, dtype=dtype, mask_shape=mshape + (130, 150),
                                   is_causal=True, kv_lengths=np.array([150, 97], dtype=np.int32))
    t = {n: dev(getattr(w, n), dtype) for n in ("q", "k", "v")}
    kvl = torch.as_tensor(w.kv_lengths, device="cuda")
    kw = dict(scale=w.scale, is_causal=True, kv_lengths=kvl, out_dtype=torch.float32)
    out_bits = sa.sdpa(t["q"], t["k"], t["v"], None, packed(w.mask), **kw)
    out_bytes = sa.sdpa(t["q"], t["k"], t["v"], None, dev(w.mask, "u8"), **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.nan_to_num(out_bits.cpu().numpy(), nan=7.0),
                                  np.nan_to_num(out_bytes.cpu().numpy(), nan=7.0))
    ref = oracle.sdpa(w.values("q"), w.values("k"), w.values("v"), mask=w.mask, scale=w.scale, is_causal=True,
                      kv_lengths=w.kv_lengths)
    assert_close(out_bits.cpu().numpy(), ref, dtype, "U1 mask vs oracle")
    # the combined allowed mask, exported from the kernel's predicate
    a_bits = sa.debug_allowed_mask(t["q"], t["k"], packed(w.mask), is_causal=True, kv_lengths=kvl)
    a_bytes = sa.debug_allowed_mask(t["q"], t["k"], dev(w.mask, "u8"), is_causal=True, kv_lengths=kvl)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a_bits.cpu().numpy(), a_bytes.cpu().numpy())


def test_per_head_bits_long_context(lib):
    # per-head masks over 16384 keys (a down-scaled long context): block info from bits, the
    # block-skipping path equal to the dense bit mask, sampled rows against the oracle
    say("U1 per-head mask, 2 heads x 256 x 16384")
    Lq, Lkv, H = 256, 16384, 2
    mask = workloads.block_sparse_mask(Lq, Lkv, 128, k=17, shape_prefix=(1, H))
    pm = packed(mask)
    info = sa.build_block_mask_info(pm, 128, 128)
    got = info.to_numpy()
    ref = oracle.block_mask_info(mask, 128, 128)
    for key in ("block_mask", "row_ptr", "data_next", "partial_bits"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    w = workloads.random_attention(71, 1, Lq, Lkv, H, 1, 128, dtype="bf16")
    t = {n: dev(getattr(w, n), "bf16") for n in ("q", "k", "v")}
    o_info = sa.sdpa(t["q"], t["k"], t["v"], mask_info=info, out_dtype=torch.float32)
    o_dense = sa.sdpa(t["q"], t["k"], t["v"], None, pm, out_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.nan_to_num(o_info.cpu().numpy(), nan=7.0), np.nan_to_num(o_dense.cpu().numpy(), nan=7.0))
    rows = [0, 1, 127, 128, 255]
    r = oracle.sdpa(workloads.bf16_to_f32(w.q[:, rows]), w.values("k"), w.values("v"), mask=mask[..., rows, :])
    assert_close(o_info[:, rows].cpu().numpy(), r, "bf16", "long-context rows")
