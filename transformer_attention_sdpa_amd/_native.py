"""ctypes view of include/sdpa.h and the loader of libsdpa_mi355x.so.

torch is imported first on purpose: it loads the HIP runtime (libamdhip64.so.7) that the
library then binds to, so the two share one runtime, one device context and one stream
namespace. The library must have been built (``python -m transformer_attention_sdpa_amd.build``
or ``__graft_entry__.build()``); there is no fallback of any kind when it is missing.
"""
import ctypes
import os
import re

import torch  # noqa: F401  (load order: torch's HIP runtime first)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsdpa_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "sdpa.h")

SDPA_OK, SDPA_ERR_NULL, SDPA_ERR_SHAPE, SDPA_ERR_DTYPE, SDPA_ERR_UNSUPPORTED, SDPA_ERR_WORKSPACE, SDPA_ERR_HIP = range(7)
SDPA_F32, SDPA_BF16, SDPA_U8, SDPA_F16, SDPA_U1 = 0, 1, 2, 3, 4
CAUSAL_NONE, CAUSAL_TRUE, CAUSAL_BOTTOM_RIGHT = 0, 1, 2
PATH_MATRIX_CORE, PATH_FP32, PATH_MATRIX_CORE_STORED_DS = 1, 2, 3
PATH_NAMES = {PATH_MATRIX_CORE: "matrix_core", PATH_FP32: "fp32", PATH_MATRIX_CORE_STORED_DS: "matrix_core_stored_ds"}


class SdpaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("dims", ctypes.c_int64 * 4),
        ("strides", ctypes.c_int64 * 4),
    ]


class BlockMaskInfoC(ctypes.Structure):
    _fields_ = [
        ("mask_batch", ctypes.c_int32), ("mask_heads", ctypes.c_int32),
        ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
        ("n_qb", ctypes.c_int32), ("n_kb", ctypes.c_int32),
        ("bq", ctypes.c_int32), ("bkv", ctypes.c_int32),
        ("block_mask", ctypes.c_void_p),
        ("mask_next", ctypes.c_void_p),
        ("row_ptr", ctypes.c_void_p),
        ("data_next", ctypes.c_void_p),
        ("partial_bits", ctypes.c_void_p),
        ("n_partial", ctypes.c_void_p),
    ]


T = ctypes.POINTER(SdpaTensor)
I32P = ctypes.c_void_p          # device int32 arrays are passed as raw addresses
VP = ctypes.c_void_p
I32 = ctypes.c_int32
SZ = ctypes.c_size_t

PROTOTYPES = {
    "sdpa_fwd": (I32, [T, T, T, T, T, ctypes.POINTER(BlockMaskInfoC), ctypes.c_float, I32,
                       I32P, I32, I32P, I32, I32P, I32, I32, T, VP, SZ, VP]),
    "sdpa_fwd_lse": (I32, [T, T, T, T, T, ctypes.POINTER(BlockMaskInfoC), ctypes.c_float, I32,
                           I32P, I32, I32P, I32, I32P, I32, I32, T, VP, VP, SZ, VP]),
    "sdpa_bwd": (I32, [T, T, T, T, T, VP, T, ctypes.POINTER(BlockMaskInfoC), ctypes.c_float, I32,
                       I32P, I32, I32P, I32, I32P, I32, T, T, T, VP, VP, SZ, VP]),
    "sdpa_bwd_workspace_bytes": (SZ, [T, T, T]),
    "sdpa_bwd_workspace_bytes_ds": (SZ, [T, T, T]),
    "sdpa_fwd_path": (I32, [T, T, T, T, T, ctypes.POINTER(BlockMaskInfoC), ctypes.c_float, I32, I32, T,
                            ctypes.POINTER(I32)]),
    "sdpa_bwd_path": (I32, [T, T, T, T, T, T, ctypes.POINTER(BlockMaskInfoC), ctypes.c_float, I32, T, T, T, SZ,
                            ctypes.POINTER(I32)]),
    "sdpa_fwd_packed": (I32, [T, T, T, I32P, I32P, I32, I32, ctypes.c_float, I32,
                              I32P, I32, I32P, I32, I32P, I32, I32, T, VP, SZ, VP]),
    "sdpa_fwd_workspace_bytes": (SZ, [T, T, T, I32]),
    "sdpa_decode": (I32, [T, T, T, I32P, ctypes.c_float, I32, T, VP, SZ, VP]),
    "sdpa_decode_workspace_bytes": (SZ, [T, T, I32]),
    "sdpa_decode_noalloc": (I32, [T, T, T, I32P, ctypes.c_float, I32, T, VP]),
    "sdpa_decode_noalloc_max_scratch_bytes": (SZ, []),
    "kv_cache_update": (I32, [T, T, T, T, I32P, VP]),
    "sdpa_block_mask_info_bytes": (I32, [T, I32, I32, ctypes.POINTER(SZ)]),
    "build_block_mask_info": (I32, [T, I32, I32, VP, SZ, ctypes.POINTER(BlockMaskInfoC), VP]),
    "head_rms_norm": (I32, [T, T, ctypes.c_float, VP]),
    "sdpa_debug_allowed_mask": (I32, [T, T, T, ctypes.POINTER(BlockMaskInfoC), I32, I32P, I32, I32P, I32,
                                      I32P, I32, T, VP]),
    "sdpa_measure_mfma_bf16": (I32, [I32, I32, VP, SZ, VP]),
    "sdpa_measure_stream_read": (I32, [VP, SZ, I32, VP, SZ, VP]),
    "sdpa_status_string": (ctypes.c_char_p, [I32]),
    "sdpa_last_error": (ctypes.c_char_p, []),
    "sdpa_version": (ctypes.c_char_p, []),
}


def header_functions():
    """Names of the functions include/sdpa.h declares (parsed from the header text)."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^SDPA_API\s+[\w\s\*]+?\b(\w+)\(", text, flags=re.M)))


class SdpaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load():
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m transformer_attention_sdpa_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status):
    if status != SDPA_OK:
        lib = load()
        msg = lib.sdpa_last_error().decode() or lib.sdpa_status_string(status).decode()
        raise SdpaError(status, msg)
