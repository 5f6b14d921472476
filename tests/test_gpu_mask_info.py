"""GPU build_block_mask_info against the oracle, bit for bit (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import say, dev
import transformer_attention_sdpa_amd as sa

pytestmark = pytest.mark.gpu


def check(mask, bq, bkv):
    info = sa.build_block_mask_info(dev(mask, "u8"), bq, bkv)
    got = info.to_numpy()
    ref = oracle.block_mask_info(mask, bq, bkv)
    for key in ("block_mask", "mask_next", "row_ptr", "data_next", "partial_bits"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    assert got["n_partial"] == ref["n_partial"]
    return got


@pytest.mark.parametrize("shape,bq,bkv,block", [((1, 1, 300, 260), 64, 64, 64), ((2, 3, 130, 100), 32, 32, 32),
                                                ((1, 2, 512, 384), 128, 128, 128), ((1, 1, 5, 33), 16, 32, 16),
                                                ((2, 1, 257, 1000), 128, 96, 32)])
def test_block_info_small(lib, shape, bq, bkv, block):
    say(f"mask info {shape} bq={bq} bkv={bkv}")
    Mb, Mh, Lq, Lkv = shape
    mask = workloads.block_sparse_mask(Lq, Lkv, block, k=11, shape_prefix=(Mb, Mh))
    check(mask, bq, bkv)


def test_block_info_all_empty_and_all_full(lib):
    say("mask info empty/full")
    z = np.zeros((1, 1, 256, 256), dtype=np.uint8)
    g = check(z, 128, 128)
    assert g["row_ptr"][-1] == 0 and g["n_partial"] == 0
    o = np.ones((1, 1, 256, 256), dtype=np.uint8)
    g = check(o, 128, 128)
    assert np.all(g["block_mask"] == 2) and g["n_partial"] == 0


def test_block_info_full_size_mask(lib):
    # the 8192 x 8192 runtime mask of the bias + block-sparse workload, 128 x 128 blocks
    say("mask info 8192x8192")
    mask = workloads.block_sparse_mask(8192, 8192, 128, k=3)
    got = check(mask, 128, 128)
    frac = np.bincount(got["block_mask"].ravel(), minlength=3) / got["block_mask"].size
    say(f"  block classes empty/partial/full = {frac}")
