"""Block information of a runtime boolean mask (oracle; test infrastructure only).

Source: the pull request "Support dynamic masks in splash attention #25213" (its
description and review threads). A mask is cut into blocks of bq query rows by bkv key
columns. Every block is classed by its content as empty (no allowed element), full (all
allowed) or partial; only non-empty blocks are visited and only partial blocks carry
their elements. The PR's objects map onto ours as follows:

  block_mask          per-block class, values 0/1/2, stored as int8
                      (0 empty, 1 partial, 2 full -- the PR gives only the range);
  mask_next           per block, the index of its stored partial block; 0 for empty
                      and full blocks (the PR writes 0 there too);
  data_next, row_ptr  the non-empty key-block indices of every (batch, head, q-block)
                      row, listed row after row (a CSR: row r owns
                      data_next[row_ptr[r]:row_ptr[r+1]]);
  partial_bits        the partial blocks themselves, rows of queries by columns of keys
                      (the PR swaps the last two axes to get that order), bit-packed as the
                      review suggests: bit (c mod 32) of word r*(bkv/32) + c//32 is
                      element (r, c); 1 = attend.

Blocks are visited in ascending flat order (batch, head, q-block, kv-block), which makes
the result unique. A block at the ragged edge of the mask is classed over its in-range
elements; its out-of-range bits are 0.
"""
import numpy as np

EMPTY, PARTIAL, FULL = 0, 1, 2


def _pack_block(blk: np.ndarray, bq: int, bkv: int) -> np.ndarray:
    """bool [rows<=bq][cols<=bkv] -> uint32 [bq][bkv/32]; bit (c%32) of word c//32 of row r."""
    full = np.zeros((bq, bkv), dtype=np.uint64)
    full[:blk.shape[0], :blk.shape[1]] = blk
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    words = (full.reshape(bq, bkv // 32, 32) * weights).sum(axis=2)
    return words.astype(np.uint32)


def block_mask_info(mask, bq: int, bkv: int) -> dict:
    """mask: [Mb][Mh][Lq][Lkv] (nonzero = attend). Returns the block info arrays (numpy)."""
    mask = np.asarray(mask)
    if mask.ndim != 4:
        raise ValueError("mask must be [Mb][Mh][Lq][Lkv]")
    if bkv % 32:
        raise ValueError("bkv must be a multiple of 32 for bit packing")
    Mb, Mh, Lq, Lkv = mask.shape
    n_qb, n_kb = -(-Lq // bq), -(-Lkv // bkv)
    block_mask = np.zeros((Mb, Mh, n_qb, n_kb), dtype=np.int8)
    mask_next = np.zeros((Mb, Mh, n_qb, n_kb), dtype=np.int32)
    row_ptr = [0]
    data_next = []
    partial = []
    for b in range(Mb):
        for h in range(Mh):
            for qb in range(n_qb):
                for kb in range(n_kb):
                    blk = mask[b, h, qb * bq:(qb + 1) * bq, kb * bkv:(kb + 1) * bkv] != 0
                    n_true = int(blk.sum())
                    if n_true == 0:
                        cls = EMPTY
                    elif n_true == blk.size:
                        cls = FULL
                    else:
                        cls = PARTIAL
                    block_mask[b, h, qb, kb] = cls
                    if cls != EMPTY:
                        data_next.append(kb)
                    if cls == PARTIAL:
                        mask_next[b, h, qb, kb] = len(partial)
                        partial.append(_pack_block(blk, bq, bkv))
                row_ptr.append(len(data_next))
    bits = (np.stack(partial) if partial
            else np.zeros((0, bq, bkv // 32), dtype=np.uint32))
    return {
        "block_mask": block_mask,
        "mask_next": mask_next,
        "row_ptr": np.asarray(row_ptr, dtype=np.int32),
        "data_next": np.asarray(data_next, dtype=np.int32),
        "partial_bits": bits,
        "n_partial": len(partial),
        "n_qb": n_qb, "n_kb": n_kb,
    }


def unpack_block_mask(info: dict, shape, bq: int, bkv: int) -> np.ndarray:
    """Rebuild the uint8 mask [Mb][Mh][Lq][Lkv] from block info (inverse, for round trips)."""
    Mb, Mh, Lq, Lkv = shape
    out = np.zeros(shape, dtype=np.uint8)
    bm, mn, bits = info["block_mask"], info["mask_next"], info["partial_bits"]
    for b in range(Mb):
        for h in range(Mh):
            for qb in range(bm.shape[2]):
                for kb in range(bm.shape[3]):
                    r0, c0 = qb * bq, kb * bkv
                    r1, c1 = min(r0 + bq, Lq), min(c0 + bkv, Lkv)
                    cls = bm[b, h, qb, kb]
                    if cls == FULL:
                        out[b, h, r0:r1, c0:c1] = 1
                    elif cls == PARTIAL:
                        words = bits[mn[b, h, qb, kb]]
                        for r in range(r1 - r0):
                            for c in range(c1 - c0):
                                out[b, h, r0 + r, c0 + c] = (int(words[r, c // 32]) >> (c % 32)) & 1
    return out
