"""MI355X-native scaled dot-product attention: a HIP library for gfx950 behind a C ABI
(include/sdpa.h), with this thin torch binding.

Entry points (same names as the C ABI): ``sdpa`` (sdpa_fwd, and sdpa_fwd_lse with
``return_lse=True``), ``sdpa_bwd``, ``sdpa_packed`` (sdpa_fwd_packed), ``sdpa_decode``,
``kv_cache_update``, ``build_block_mask_info``, ``head_rms_norm`` / ``per_head_rms_norm`` and
``debug_allowed_mask``; ``sdpa_fwd_path`` / ``sdpa_bwd_path`` name the kernels a call would
run (matrix-core or fp32); ``measure_mfma_bf16`` and ``measure_stream_read`` launch the two probes
that measure the roofline denominators. ``load()`` loads the shared library and raises when it is not built.
"""
from ._native import load, SdpaError, header_functions, LIB_PATH
from .api import (sdpa, sdpa_bwd, sdpa_packed, sdpa_decode, sdpa_decode_noalloc, decode_noalloc_max_scratch_bytes, kv_cache_update, build_block_mask_info, BlockMaskInfo, PackedMask,
                  head_rms_norm, per_head_rms_norm, debug_allowed_mask, decode_workspace_bytes, bwd_workspace_bytes,
                  desc, from_numpy, to_numpy_f32, measure_mfma_bf16, measure_stream_read,
                  sdpa_fwd_path, sdpa_bwd_path)

sdpa_fwd = sdpa
sdpa_fwd_lse = sdpa           # with return_lse=True
sdpa_fwd_packed = sdpa_packed

__all__ = ["load", "SdpaError", "header_functions", "LIB_PATH", "sdpa", "sdpa_fwd", "sdpa_fwd_lse", "sdpa_bwd", "sdpa_packed",
           "sdpa_fwd_packed", "sdpa_decode", "sdpa_decode_noalloc", "decode_noalloc_max_scratch_bytes",
           "kv_cache_update", "build_block_mask_info", "BlockMaskInfo", "PackedMask", "head_rms_norm",
           "per_head_rms_norm", "debug_allowed_mask", "decode_workspace_bytes", "bwd_workspace_bytes", "desc",
           "from_numpy", "to_numpy_f32", "measure_mfma_bf16", "measure_stream_read",
           "sdpa_fwd_path", "sdpa_bwd_path"]
