"""Pins of the block-mask-info and KV-cache-update oracles (CPU only).

Block info follows the splash-attention pull request "Support dynamic masks in splash
attention #25213": blocks classed empty/full/partial, only non-empty blocks listed, partial
blocks stored. The cache update follows the keras issue on MultiHeadAttention's missing
position_bias (a cache-update index says where new keys/values go).
"""
import numpy as np
import pytest

from oracle import block_mask_info, unpack_block_mask, kv_cache_update, EMPTY, PARTIAL, FULL
import workloads


def test_block_info_hand_example():
    # Lq = 4, Lkv = 64, bq = 2, bkv = 32: a 2 x 2 grid of blocks
    m = np.zeros((1, 1, 4, 64), dtype=np.uint8)
    m[0, 0, 0:2, 32:64] = 1          # block (0, 1) full
    m[0, 0, 2, 5] = 1                # block (1, 0) partial: one element at row 0, col 5
    m[0, 0, 3, 31] = 1               #   and one at row 1, col 31
    # block (0, 0) and (1, 1) empty
    info = block_mask_info(m, 2, 32)
    np.testing.assert_array_equal(info["block_mask"][0, 0], [[EMPTY, FULL], [PARTIAL, EMPTY]])
    np.testing.assert_array_equal(info["row_ptr"], [0, 1, 2])
    np.testing.assert_array_equal(info["data_next"], [1, 0])
    np.testing.assert_array_equal(info["mask_next"][0, 0], [[0, 0], [0, 0]])
    assert info["n_partial"] == 1
    np.testing.assert_array_equal(info["partial_bits"][0], [[1 << 5], [1 << 31]])


def test_block_info_second_partial_gets_next_index_in_flat_order():
    m = np.zeros((2, 1, 2, 64), dtype=np.uint8)
    m[0, 0, 0, 40] = 1               # (b0, qb0, kb1) partial -> index 0
    m[1, 0, 1, 0] = 1                # (b1, qb0, kb0) partial -> index 1
    m[1, 0, :, 32:] = 1              # (b1, qb0, kb1) full
    info = block_mask_info(m, 2, 32)
    assert info["n_partial"] == 2
    assert info["mask_next"][0, 0, 0, 1] == 0 and info["mask_next"][1, 0, 0, 0] == 1
    np.testing.assert_array_equal(info["row_ptr"], [0, 1, 3])
    np.testing.assert_array_equal(info["data_next"], [1, 0, 1])
    np.testing.assert_array_equal(info["partial_bits"][0], [[1 << 8], [0]])   # row 0, col 40 - 32
    np.testing.assert_array_equal(info["partial_bits"][1], [[0], [1]])        # row 1, col 0


@pytest.mark.parametrize("shape,bq,bkv", [((1, 1, 300, 260), 64, 64), ((2, 3, 130, 100), 32, 32),
                                          ((1, 2, 256, 256), 128, 128), ((1, 1, 5, 33), 16, 32)])
def test_block_info_round_trip_and_invariants(shape, bq, bkv):
    Mb, Mh, Lq, Lkv = shape
    m = workloads.block_sparse_mask(Lq, Lkv, min(bq, bkv), k=7, shape_prefix=(Mb, Mh))
    info = block_mask_info(m, bq, bkv)
    np.testing.assert_array_equal(unpack_block_mask(info, shape, bq, bkv), m)
    bm = info["block_mask"]
    n_qb, n_kb = -(-Lq // bq), -(-Lkv // bkv)
    assert bm.shape == (Mb, Mh, n_qb, n_kb)
    assert ((bm == EMPTY).sum() + (bm == PARTIAL).sum() + (bm == FULL).sum()) == bm.size
    rp = info["row_ptr"]
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == (bm != EMPTY).sum()
    dn = info["data_next"]
    for r in range(Mb * Mh * n_qb):
        row = dn[rp[r]:rp[r + 1]]
        assert np.all(np.diff(row) > 0)
        np.testing.assert_array_equal(row, np.nonzero(bm.reshape(-1, n_kb)[r] != EMPTY)[0])
    # classes by a second route: counts of allowed elements per block via padding + reshape
    pad = np.zeros((Mb, Mh, n_qb * bq, n_kb * bkv), dtype=np.int64)
    pad[:, :, :Lq, :Lkv] = m
    cnt = pad.reshape(Mb, Mh, n_qb, bq, n_kb, bkv).sum(axis=(3, 5))
    rows_in = np.minimum(bq, Lq - np.arange(n_qb) * bq)[:, None]
    cols_in = np.minimum(bkv, Lkv - np.arange(n_kb) * bkv)[None, :]
    expect = np.where(cnt == 0, EMPTY, np.where(cnt == rows_in * cols_in, FULL, PARTIAL))
    np.testing.assert_array_equal(bm, expect)
    # mask_next: 0 on empty/full, consecutive indices on partials in flat order
    mn = info["mask_next"]
    assert np.all(mn[bm != PARTIAL] == 0)
    np.testing.assert_array_equal(mn[bm == PARTIAL], np.arange(info["n_partial"]))


def test_generated_mask_has_the_drawn_block_mix():
    m = workloads.block_sparse_mask(2048, 2048, 128, k=3)
    info = block_mask_info(m, 128, 128)
    frac = np.bincount(info["block_mask"].ravel(), minlength=3) / info["block_mask"].size
    assert abs(frac[EMPTY] - 0.3) < 0.06 and abs(frac[FULL] - 0.2) < 0.06 and abs(frac[PARTIAL] - 0.5) < 0.06


def test_kv_cache_update_hand_example():
    kc = np.arange(2 * 4 * 1 * 2, dtype=np.uint16).reshape(2, 4, 1, 2)
    vc = kc + 100
    kn = np.array([[[[901, 902]]], [[[911, 912]]]], dtype=np.uint16)
    vn = kn + 1000
    k2, v2 = kv_cache_update(kc, vc, kn, vn, np.array([3, 0]))
    expect_k = kc.copy()
    expect_k[0, 3, 0] = [901, 902]
    expect_k[1, 0, 0] = [911, 912]
    np.testing.assert_array_equal(k2, expect_k)
    np.testing.assert_array_equal(v2[0, 3, 0], [1901, 1902])
    np.testing.assert_array_equal(kc, np.arange(16, dtype=np.uint16).reshape(2, 4, 1, 2))   # inputs untouched


def test_kv_cache_update_skips_out_of_range_rows():
    kc = np.zeros((2, 4, 1, 1)); vc = np.zeros((2, 4, 1, 1))
    kn = np.ones((2, 3, 1, 1)); vn = np.ones((2, 3, 1, 1))
    k2, _ = kv_cache_update(kc, vc, kn, vn, np.array([2, -2]))
    np.testing.assert_array_equal(k2[0, :, 0, 0], [0, 0, 1, 1])      # rows 2, 3 written; 4 skipped
    np.testing.assert_array_equal(k2[1, :, 0, 0], [1, 0, 0, 0])      # -2, -1 skipped; 0 written


def test_pack_mask_bits_layout():
    # the U1 layout: element c of a row is bit c % 32 of word c // 32; padding bits as asked
    rng = np.random.default_rng(5)
    m = (rng.random((2, 3, 70)) < 0.5).astype(np.uint8)
    w = workloads.pack_mask_bits(m, pad_bit=1).view(np.uint32)
    assert w.shape == (2, 3, 3)
    for idx in np.ndindex(2, 3):
        for c in range(96):
            bit = (int(w[idx][c // 32]) >> (c % 32)) & 1
            assert bit == (m[idx][c] if c < 70 else 1)
