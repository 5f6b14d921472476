"""Plain, slow, obviously correct CPU oracle for scaled dot-product attention (fp64).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
package: only ``tests/``, the smoke check in ``__graft_entry__.py`` and the CPU
baseline leg of ``bench.py`` use it. It shares no code with the HIP library or its
Python binding, and imports numpy and the standard library only.

Contents (each function cites the passage it follows):

* ``sdpa``                 -- the materialized definition of attention, in fp64
                              (``oracle/sdpa.py``)
* ``sdpa_brute``           -- a second, independent pure-Python scalar version for tiny
                              shapes (``oracle/brute.py``)
* ``sdpa_packed``          -- attention over packed sequences: each segment as its own call
                              (``oracle/packed.py``)
* ``sdpa_grad``,
  ``sdpa_lse``             -- the gradient with respect to q, k, v, scale (and bias), and the
                              log-sum-exp of the logits (``oracle/grad.py``)
* ``block_mask_info``      -- block classification, CSR and bit-packed partial blocks of
                              a runtime boolean mask (``oracle/block_mask.py``)
* ``kv_cache_update``      -- cache rows written at a per-batch index (``oracle/kv_cache.py``)
* ``per_head_rms_norm``,
  ``rms_rows``             -- per-head RMS normalisation (``oracle/rms_norm.py``)
"""
from .sdpa import sdpa, kv_head_of, causal_offsets, allowed_matrix
from .brute import sdpa_brute
from .packed import sdpa_packed
from .grad import sdpa_grad, sdpa_lse
from .block_mask import block_mask_info, unpack_block_mask, EMPTY, PARTIAL, FULL
from .kv_cache import kv_cache_update
from .rms_norm import per_head_rms_norm, rms_rows, RMS_EPS

__all__ = [
    "sdpa", "kv_head_of", "causal_offsets", "allowed_matrix", "sdpa_brute", "sdpa_packed", "sdpa_grad", "sdpa_lse",
    "block_mask_info", "unpack_block_mask", "EMPTY", "PARTIAL", "FULL",
    "kv_cache_update", "per_head_rms_norm", "rms_rows", "RMS_EPS",
]
