"""Torch-facing binding of libsdpa_mi355x.so: argument marshalling only.

Tensors use the C-order layout [batch][seq][heads][head_dim] for q/k/v/out and the caches,
and [batch][heads][q_len][kv_len] for bias/mask (size-1 dims broadcast). This is NNlib's
column-major (head_dim, heads, seq, batch) with the dims reversed, so each descriptor passed
to the library is the torch shape and strides read backwards. Every computation runs in the
HIP library on the caller's current stream; nothing here computes on the host or falls back
to another implementation.

``stream=``: every entry point takes an optional torch stream. The call then runs as if that
stream were current: the binding's own temporaries (int32 casts of per-batch arguments, the
workspace, a default output) are made on it, so the kernels never read a temporary that another
stream is still writing. Inputs the caller made on another stream are the caller's to order, as
with any torch operation.
"""
import contextlib
import ctypes
import functools
import math

import numpy as np
import torch

from . import _native as N

_DTYPE = {torch.float32: N.SDPA_F32, torch.bfloat16: N.SDPA_BF16, torch.float16: N.SDPA_F16,
          torch.uint8: N.SDPA_U8, torch.bool: N.SDPA_U8}
_CAUSAL = {False: N.CAUSAL_NONE, None: N.CAUSAL_NONE, True: N.CAUSAL_TRUE,
           "bottom_right": N.CAUSAL_BOTTOM_RIGHT}


def desc(t: torch.Tensor) -> N.SdpaTensor:
    """Descriptor of a tensor of up to 4 dims (leading dims are padded with 1)."""
    if t.dim() > 4:
        raise ValueError("at most 4 dims")
    if t.dtype not in _DTYPE:
        raise TypeError(f"dtype {t.dtype} is not accepted")
    shape = [1] * (4 - t.dim()) + list(t.shape)
    if t.numel() == 0:                      # no element is addressed: report contiguous strides
        stride, acc = [0] * 4, 1
        for i in range(3, -1, -1):
            stride[i] = acc
            acc *= max(shape[i], 1)
    else:
        stride = [0] * (4 - t.dim()) + list(t.stride())
    d = N.SdpaTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPE[t.dtype]
    for i in range(4):
        d.dims[i] = shape[3 - i]
        d.strides[i] = stride[3 - i]
    return d


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s, ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run ``fn`` with ``stream`` (a keyword argument, default the current stream) made current,
    so that every tensor the binding creates for the call is made on the stream the kernels run
    on."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, **kwargs)
    return wrapper


def _per_batch_arg(x, B, device, none_value):
    """int / None / [B] values -> (device int32 pointer or None, scalar, keep-alive tensor)."""
    if x is None:
        return None, none_value, None
    if isinstance(x, (int, np.integer)):
        return None, int(x), None
    t = torch.as_tensor(x, dtype=torch.int32, device=device).reshape(-1)
    if t.numel() == 1:
        t = t.expand(B)
    t = t.contiguous()
    if t.numel() != B:
        raise ValueError("per-batch argument needs one entry per batch element")
    return t.data_ptr(), 0, t


def _per_batch_tensor(x, B, device, name):
    """An int, a one-element or a [B] array/tensor -> contiguous int32 [B] device tensor. The
    count is checked before anything moves to the device: the kernels read entry b of every
    batch element b, so a shorter array would be read past its end."""
    if isinstance(x, (int, np.integer)):
        return torch.full((B,), int(x), dtype=torch.int32, device=device)
    t = x if isinstance(x, torch.Tensor) else torch.as_tensor(np.asarray(x, dtype=np.int32))
    t = t.reshape(-1)
    if t.numel() == 1:
        t = t.expand(B)
    if t.numel() != B:
        raise ValueError(f"{name} needs one entry per batch element ({B}), got {t.numel()}")
    return t.to(device=device, dtype=torch.int32).contiguous()


class PackedMask:
    """A boolean mask packed 32 elements per 32-bit word along the keys (the U1 layout of
    include/sdpa.h): element c of a row is bit c % 32 of word c // 32. ``words`` is an int32
    device tensor [Mb][Mh][Lq][ceil(kv_len / 32)] (leading dims may be 1 to broadcast);
    ``kv_len`` is the number of keys. The caller packs the bits."""

    def __init__(self, words: torch.Tensor, kv_len: int):
        if words.dtype != torch.int32:
            raise TypeError("packed mask words must be int32")
        if words.shape[-1] != (kv_len + 31) // 32:
            raise ValueError("packed mask rows need ceil(kv_len / 32) words")
        if words.stride(-1) != 1:
            raise ValueError("packed mask words must be contiguous along a row")
        self.words, self.kv_len = words, int(kv_len)
        self.device = words.device
        self.shape = tuple(words.shape[:-1]) + (self.kv_len,)

    def desc(self) -> N.SdpaTensor:
        d = desc(self.words.view(torch.float32))     # same 32-bit words; dims and strides in words
        d.data = self.words.data_ptr() if self.words.numel() > 0 else None
        d.dtype = N.SDPA_U1
        d.dims[0] = self.kv_len
        d.strides[0] = 1
        return d


def _mask_desc(m):
    return m.desc() if isinstance(m, PackedMask) else desc(m)


def _mask_u8(mask):
    if mask is None or isinstance(mask, PackedMask):
        return mask
    if mask.dtype == torch.bool:
        return mask.view(torch.uint8)
    if mask.dtype != torch.uint8:
        raise TypeError("mask must be bool or uint8")
    return mask


class BlockMaskInfo:
    """Block information of a runtime mask, held in one device buffer (see build_block_mask_info)."""

    def __init__(self, storage: torch.Tensor, c: N.BlockMaskInfoC, mask_shape):
        self.storage = storage
        self.c = c
        self.mask_shape = tuple(mask_shape)

    @property
    def n_blocks(self):
        c = self.c
        return c.mask_batch * c.mask_heads * c.n_qb * c.n_kb

    def _view(self, ptr, count, dtype):
        base = self.storage.data_ptr()
        off = ptr - base
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return self.storage[off:off + nbytes].view(dtype)

    def to_numpy(self) -> dict:
        """Copy the info to the host (synchronizes): the layout of ``oracle.block_mask_info``."""
        c = self.c
        shape = (c.mask_batch, c.mask_heads, c.n_qb, c.n_kb)
        nb = self.n_blocks
        nrows = c.mask_batch * c.mask_heads * c.n_qb
        row_ptr = self._view(c.row_ptr, nrows + 1, torch.int32).cpu().numpy()
        n_partial = int(self._view(c.n_partial, 1, torch.int32).cpu().item())
        words = c.bkv // 32
        return {
            "block_mask": self._view(c.block_mask, nb, torch.int8).cpu().numpy().reshape(shape),
            "mask_next": self._view(c.mask_next, nb, torch.int32).cpu().numpy().reshape(shape),
            "row_ptr": row_ptr,
            "data_next": self._view(c.data_next, int(row_ptr[-1]), torch.int32).cpu().numpy(),
            "partial_bits": self._view(c.partial_bits, n_partial * c.bq * words, torch.int32)
                                .cpu().numpy().view(np.uint32).reshape(n_partial, c.bq, words),
            "n_partial": n_partial, "n_qb": c.n_qb, "n_kb": c.n_kb,
        }


@_on_stream
def build_block_mask_info(mask: torch.Tensor, bq: int = 128, bkv: int = 128,
                          storage: torch.Tensor = None) -> BlockMaskInfo:
    """Block info of a runtime device mask [Mb][Mh][Lq][Lkv] (bool or uint8, or a PackedMask).

    ``storage``: a uint8 device tensor of at least sdpa_block_mask_info_bytes() to write into
    (allocated here when None); the returned info points into it.
    """
    lib = N.load()
    m = _mask_u8(mask)
    dm = _mask_desc(m)
    nbytes = ctypes.c_size_t()
    N.check(lib.sdpa_block_mask_info_bytes(ctypes.byref(dm), bq, bkv, ctypes.byref(nbytes)))
    if storage is None:
        storage = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=mask.device)
    elif storage.numel() < int(nbytes.value):
        raise ValueError(f"storage needs {int(nbytes.value)} bytes")
    info = N.BlockMaskInfoC()
    s, sp = _stream()
    N.check(lib.build_block_mask_info(ctypes.byref(dm), bq, bkv, ctypes.c_void_p(storage.data_ptr()),
                                      storage.numel(), ctypes.byref(info), sp))
    return BlockMaskInfo(storage, info, m.shape)


@_on_stream
def sdpa(q, k, v, bias=None, mask=None, *, mask_info: BlockMaskInfo = None, scale=None, is_causal=False,
         q_offset=0, kv_lengths=None, q_lengths=None, qk_norm=False, out=None, out_dtype=None, return_lse=False):
    """Scaled dot-product attention. q [B][Lq][Hq][D], k [B][Lkv][Hkv][D], v [B][Lkv][Hkv][Dv].

    is_causal: False, True or "bottom_right". q_offset, kv_lengths, q_lengths: int, None or a
    [B] int32 tensor on the device. scale: None = 1/sqrt(D). Returns out [B][Lq][Hq][Dv], or
    (out, lse) with return_lse (sdpa_fwd_lse): lse fp32 [B][Hq][Lq].
    """
    lib = N.load()
    B, Lq, Hq, _ = q.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, Lq, Hq, Dv), dtype=out_dtype or q.dtype, device=q.device)
    dq, dk, dv, do = desc(q), desc(k), desc(v), desc(out)
    db = desc(bias) if bias is not None else None
    m = _mask_u8(mask) if mask_info is None else None
    dm = _mask_desc(m) if m is not None else None
    qo_ptr, qo_all, qo_keep = _per_batch_arg(q_offset, B, q.device, 0)
    kv_ptr, kv_all, kv_keep = _per_batch_arg(kv_lengths, B, q.device, -1)
    ql_ptr, ql_all, ql_keep = _per_batch_arg(q_lengths, B, q.device, -1)
    ws_bytes = lib.sdpa_fwd_workspace_bytes(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(bool(qk_norm)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    s, sp = _stream()
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib.sdpa_fwd_lse(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                          ctypes.byref(db) if db is not None else None,
                          ctypes.byref(dm) if dm is not None else None,
                          ctypes.byref(mask_info.c) if mask_info is not None else None,
                          float("nan") if scale is None else float(scale), _CAUSAL[is_causal],
                          qo_ptr, qo_all, kv_ptr, kv_all, ql_ptr, ql_all, int(bool(qk_norm)),
                          ctypes.byref(do), ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
                          ctypes.c_void_p(ws.data_ptr()) if ws is not None else None, ws_bytes, sp)
    N.check(st)
    return (out, lse) if return_lse else out


@_on_stream
def sdpa_bwd(q, k, v, out, dout, lse, mask=None, *, mask_info: BlockMaskInfo = None, scale=None,
             is_causal=False, q_offset=0, kv_lengths=None, q_lengths=None, grad_dtype=None, grads=None,
             workspace=None, store_ds=True):
    """Gradient of ``sdpa`` with respect to q, k, v and scale (sdpa_bwd).

    out and lse come from ``sdpa(..., return_lse=True)`` of the same call; dout is the cotangent
    of out. Returns (dq, dk, dv, dscale): dq/dk/dv of q/k/v's shapes in grad_dtype (default
    q.dtype), dscale a one-element fp32 tensor. ``grads`` may pass those four tensors to be
    written instead, and ``workspace`` a uint8 device tensor of bwd_workspace_bytes() (its size
    picks the route: with bwd_workspace_bytes(store_ds=True) bytes the dK/dV pass stores dS for
    the dQ pass; with fewer the dQ pass forms the weights again). ``store_ds`` sizes the
    workspace allocated here when none is passed.
    """
    lib = N.load()
    B, Lq, Hq, _ = q.shape
    gd = grad_dtype or q.dtype
    if grads is not None:
        dq_t, dk_t, dv_t, dscale = grads
    else:
        dq_t = torch.empty(q.shape, dtype=gd, device=q.device)
        dk_t = torch.empty(k.shape, dtype=gd, device=q.device)
        dv_t = torch.empty(v.shape, dtype=gd, device=q.device)
        dscale = torch.empty(1, dtype=torch.float32, device=q.device)
    tq, tk, tv, to, tdo = desc(q), desc(k), desc(v), desc(out), desc(dout)
    gq, gk, gv = desc(dq_t), desc(dk_t), desc(dv_t)
    m = _mask_u8(mask) if mask_info is None else None
    dm = _mask_desc(m) if m is not None else None
    qo_ptr, qo_all, qo_keep = _per_batch_arg(q_offset, B, q.device, 0)
    kv_ptr, kv_all, kv_keep = _per_batch_arg(kv_lengths, B, q.device, -1)
    ql_ptr, ql_all, ql_keep = _per_batch_arg(q_lengths, B, q.device, -1)
    ws_bytes = lib.sdpa_bwd_workspace_bytes(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv))
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(q, k, v, store_ds), 1), dtype=torch.uint8, device=q.device)
    ws = workspace
    if ws.numel() < ws_bytes:
        raise ValueError(f"workspace needs {ws_bytes} bytes")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("lse must be a contiguous fp32 [B][Hq][Lq] tensor")
    s, sp = _stream()
    st = lib.sdpa_bwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(to), ctypes.byref(tdo),
                      ctypes.c_void_p(lse.data_ptr()), ctypes.byref(dm) if dm is not None else None,
                      ctypes.byref(mask_info.c) if mask_info is not None else None,
                      float("nan") if scale is None else float(scale), _CAUSAL[is_causal],
                      qo_ptr, qo_all, kv_ptr, kv_all, ql_ptr, ql_all,
                      ctypes.byref(gq), ctypes.byref(gk), ctypes.byref(gv), ctypes.c_void_p(dscale.data_ptr()),
                      ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp)
    N.check(st)
    return dq_t, dk_t, dv_t, dscale


@_on_stream
def sdpa_packed(q, k, v, q_segments, kv_segments=None, *, maxlen=None, scale=None, is_causal=False, q_offset=0,
                kv_lengths=None, q_lengths=None, qk_norm=False, out=None, out_dtype=None):
    """Attention over packed sequences. q [Lq_total][Hq][D], k [Lkv_total][Hkv][D], v [Lkv_total][Hkv][Dv]
    hold the segments one after the other; q_segments / kv_segments (device int32 tensors, kv =
    q when None) give their lengths. Segment s of q attends segment s of k/v only; is_causal,
    q_offset, kv_lengths and q_lengths apply per segment (an int, or one entry per segment).
    maxlen: None or a bound on every segment. Returns out [Lq_total][Hq][Dv].
    """
    lib = N.load()
    Lq, Hq, _ = q.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((Lq, Hq, Dv), dtype=out_dtype or q.dtype, device=q.device)
    qs = torch.as_tensor(q_segments, dtype=torch.int32, device=q.device).reshape(-1).contiguous()
    ks = None if kv_segments is None else torch.as_tensor(kv_segments, dtype=torch.int32,
                                                          device=q.device).reshape(-1).contiguous()
    S = qs.numel()
    if ks is not None and ks.numel() != S:
        raise ValueError("q_segments and kv_segments differ in count")
    dq, dk, dv, do = desc(q.unsqueeze(0)), desc(k.unsqueeze(0)), desc(v.unsqueeze(0)), desc(out.unsqueeze(0))
    qo_ptr, qo_all, qo_keep = _per_batch_arg(q_offset, S, q.device, 0)
    kv_ptr, kv_all, kv_keep = _per_batch_arg(kv_lengths, S, q.device, -1)
    ql_ptr, ql_all, ql_keep = _per_batch_arg(q_lengths, S, q.device, -1)
    ws_bytes = lib.sdpa_fwd_workspace_bytes(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(bool(qk_norm)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    s, sp = _stream()
    st = lib.sdpa_fwd_packed(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                             ctypes.c_void_p(qs.data_ptr()) if S else None,
                             ctypes.c_void_p(ks.data_ptr()) if ks is not None and S else None, S,
                             -1 if maxlen is None else int(maxlen),
                             float("nan") if scale is None else float(scale), _CAUSAL[is_causal],
                             qo_ptr, qo_all, kv_ptr, kv_all, ql_ptr, ql_all, int(bool(qk_norm)),
                             ctypes.byref(do), ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
                             ws_bytes, sp)
    N.check(st)
    return out


def sdpa_fwd_path(q, k, v, bias=None, mask=None, *, mask_info: BlockMaskInfo = None, scale=None, is_causal=False,
                  qk_norm=False, out=None, out_dtype=None) -> str:
    """Which kernels ``sdpa`` would run for these arguments (sdpa_fwd_path; nothing is launched):
    "matrix_core" (the bf16/f16 matrix-core kernels) or "fp32" (the fp32 vector kernels)."""
    lib = N.load()
    B, Lq, Hq, _ = q.shape
    if out is None:
        out = torch.empty((B, Lq, Hq, v.shape[-1]), dtype=out_dtype or q.dtype, device=q.device)
    dq, dk, dv, do = desc(q), desc(k), desc(v), desc(out)
    db = desc(bias) if bias is not None else None
    m = _mask_u8(mask) if mask_info is None else None
    dm = _mask_desc(m) if m is not None else None
    path = ctypes.c_int32(0)
    N.check(lib.sdpa_fwd_path(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                              ctypes.byref(db) if db is not None else None, ctypes.byref(dm) if dm is not None else None,
                              ctypes.byref(mask_info.c) if mask_info is not None else None,
                              float("nan") if scale is None else float(scale), _CAUSAL[is_causal],
                              int(bool(qk_norm)), ctypes.byref(do), ctypes.byref(path)))
    return N.PATH_NAMES[path.value]


def sdpa_bwd_path(q, k, v, out, dout, mask=None, *, mask_info: BlockMaskInfo = None, scale=None, is_causal=False,
                  grad_dtype=None, workspace_bytes=None, store_ds=True) -> str:
    """Which kernels ``sdpa_bwd`` would run (sdpa_bwd_path; nothing is launched): "matrix_core",
    "matrix_core_stored_ds" or "fp32". workspace_bytes defaults to what sdpa_bwd allocates
    itself (bwd_workspace_bytes(q, k, v, store_ds))."""
    lib = N.load()
    gd = grad_dtype or q.dtype
    gq = desc(torch.empty(q.shape, dtype=gd, device=q.device))
    gk = desc(torch.empty(k.shape, dtype=gd, device=q.device))
    gv = desc(torch.empty(v.shape, dtype=gd, device=q.device))
    tq, tk, tv, to, tdo = desc(q), desc(k), desc(v), desc(out), desc(dout)
    m = _mask_u8(mask) if mask_info is None else None
    dm = _mask_desc(m) if m is not None else None
    wb = bwd_workspace_bytes(q, k, v, store_ds) if workspace_bytes is None else int(workspace_bytes)
    path = ctypes.c_int32(0)
    N.check(lib.sdpa_bwd_path(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(to), ctypes.byref(tdo),
                              ctypes.byref(dm) if dm is not None else None,
                              ctypes.byref(mask_info.c) if mask_info is not None else None,
                              float("nan") if scale is None else float(scale), _CAUSAL[is_causal],
                              ctypes.byref(gq), ctypes.byref(gk), ctypes.byref(gv), wb, ctypes.byref(path)))
    return N.PATH_NAMES[path.value]


def bwd_workspace_bytes(q, k, v, store_ds=False) -> int:
    """Bytes of workspace sdpa_bwd needs for these tensors; with store_ds, the bytes with which
    it stores dS for its dQ pass where that route applies (else the same minimum)."""
    lib = N.load()
    tq, tk, tv = desc(q), desc(k), desc(v)
    n = int(lib.sdpa_bwd_workspace_bytes(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv)))
    if store_ds:
        n = max(n, int(lib.sdpa_bwd_workspace_bytes_ds(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv))))
    return n


def decode_workspace_bytes(q, k_cache, num_splits=0) -> int:
    lib = N.load()
    dq, dk = desc(q), desc(k_cache)
    return int(lib.sdpa_decode_workspace_bytes(ctypes.byref(dq), ctypes.byref(dk), int(num_splits)))


@_on_stream
def sdpa_decode(q, k_cache, v_cache, kv_lengths, *, scale=None, num_splits=0, out=None, out_dtype=None,
                workspace=None):
    """The newest T queries of each sequence, q [B][T][Hq][D], against caches [B][cap][Hkv][D]:
    query t attends keys [0, kv_lengths[b] - T + t] (bottom-right causal). kv_lengths: an int,
    or one entry per sequence (a one-element array broadcasts)."""
    lib = N.load()
    B, T, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    dq, dk, dv, do = desc(q), desc(k_cache), desc(v_cache), desc(out)
    kv = _per_batch_tensor(kv_lengths, B, q.device, "kv_lengths")
    need = int(lib.sdpa_decode_workspace_bytes(ctypes.byref(dq), ctypes.byref(dk), int(num_splits)))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    s, sp = _stream()
    N.check(lib.sdpa_decode(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.c_void_p(kv.data_ptr()),
                            float("nan") if scale is None else float(scale), int(num_splits), ctypes.byref(do),
                            ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), sp))
    return out


@_on_stream
def sdpa_decode_noalloc(q, k_cache, v_cache, kv_lengths, out, *, scale=None, num_splits=0):
    """sdpa_decode without a workspace (sdpa_decode_noalloc): the split partials go to the
    library's device scratch of sdpa_decode_noalloc_max_scratch_bytes(). Allocates nothing:
    ``kv_lengths`` must already be a contiguous int32 [B] device tensor and ``out`` is required.
    Calls that overlap on one GPU race on the shared scratch."""
    lib = N.load()
    B = q.shape[0]
    if not (isinstance(kv_lengths, torch.Tensor) and kv_lengths.dtype == torch.int32 and kv_lengths.is_contiguous()
            and kv_lengths.numel() == B and kv_lengths.device == q.device):
        raise ValueError("kv_lengths must be a contiguous int32 device tensor with one entry per sequence")
    dq, dk, dv, do = desc(q), desc(k_cache), desc(v_cache), desc(out)
    _, sp = _stream()
    N.check(lib.sdpa_decode_noalloc(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                    ctypes.c_void_p(kv_lengths.data_ptr()),
                                    float("nan") if scale is None else float(scale), int(num_splits),
                                    ctypes.byref(do), sp))
    return out


def decode_noalloc_max_scratch_bytes() -> int:
    """Bytes of the device scratch sdpa_decode_noalloc holds on each GPU."""
    return int(N.load().sdpa_decode_noalloc_max_scratch_bytes())


@_on_stream
def kv_cache_update(k_cache, v_cache, k_new, v_new, write_index):
    """In place: cache[b][write_index[b] + t] = new[b][t] for k and v (rows outside the cache skipped)."""
    lib = N.load()
    B = k_cache.shape[0]
    wi = _per_batch_tensor(write_index, B, k_cache.device, "write_index")
    dkc, dvc, dkn, dvn = desc(k_cache), desc(v_cache), desc(k_new), desc(v_new)
    s, sp = _stream()
    N.check(lib.kv_cache_update(ctypes.byref(dkc), ctypes.byref(dvc), ctypes.byref(dkn), ctypes.byref(dvn),
                                ctypes.c_void_p(wi.data_ptr()), sp))
    return k_cache, v_cache


@_on_stream
def head_rms_norm(x, eps=1e-6, out=None):
    """x [B][T][H][Dh] -> every head vector divided by sqrt(mean(v^2) + eps)."""
    lib = N.load()
    y = torch.empty_like(x) if out is None else out
    dx, dy = desc(x), desc(y)
    _, sp = _stream()
    N.check(lib.head_rms_norm(ctypes.byref(dx), ctypes.byref(dy), float(eps), sp))
    return y


def per_head_rms_norm(x, num_heads: int, eps=1e-6) -> dict:
    """The per-head RMS norm of the TensorTonic page "Static Arguments in jit": x (B, T, D) ->
    {"heads": (B, H, T, D/H), "merged": (B, T, D)}. The GPU computes the merged array; "heads" is
    a view of it with the head and token axes swapped."""
    B, T, D = x.shape
    if D % num_heads:
        raise ValueError("num_heads must divide D")
    merged = head_rms_norm(x.reshape(B, T, num_heads, D // num_heads), eps).reshape(B, T, D)
    heads = merged.view(B, T, num_heads, D // num_heads).transpose(1, 2)
    return {"heads": heads, "merged": merged}


@_on_stream
def debug_allowed_mask(q, k, mask=None, *, mask_info=None, is_causal=False, q_offset=0, kv_lengths=None,
                       q_lengths=None):
    """uint8 [B][Hq][Lq][Lkv]: 1 where the kernels let query i attend key j."""
    lib = N.load()
    B, Lq, Hq, _ = q.shape
    Lkv = k.shape[1]
    allowed = torch.empty((B, Hq, Lq, Lkv), dtype=torch.uint8, device=q.device)
    dq, dk, da = desc(q), desc(k), desc(allowed)
    m = _mask_u8(mask) if mask_info is None else None
    dm = _mask_desc(m) if m is not None else None
    qo_ptr, qo_all, _k1 = _per_batch_arg(q_offset, B, q.device, 0)
    kv_ptr, kv_all, _k2 = _per_batch_arg(kv_lengths, B, q.device, -1)
    ql_ptr, ql_all, _k3 = _per_batch_arg(q_lengths, B, q.device, -1)
    _, sp = _stream()
    N.check(lib.sdpa_debug_allowed_mask(ctypes.byref(dq), ctypes.byref(dk),
                                        ctypes.byref(dm) if dm is not None else None,
                                        ctypes.byref(mask_info.c) if mask_info is not None else None,
                                        _CAUSAL[is_causal], qo_ptr, qo_all, kv_ptr, kv_all, ql_ptr, ql_all,
                                        ctypes.byref(da), sp))
    return allowed


def from_numpy(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host array -> device tensor: ``dtype`` "bf16" takes uint16 bit patterns, "f16" float16,
    "f32" float32,
    "u8" uint8, "i32" int32 (a bit copy, no arithmetic)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16))
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    elif dtype == "u8":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8))
    elif dtype == "i32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
    else:
        raise ValueError(dtype)
    return t.to(device)


def to_numpy_f32(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float32 numpy (bf16 widened exactly; a copy, no other arithmetic)."""
    return t.detach().float().cpu().numpy()


@_on_stream
def measure_mfma_bf16(workgroups: int, iters: int, sink: torch.Tensor = None) -> float:
    """Launch the matrix-core rate probe (sdpa_measure_mfma_bf16) on the current stream; returns
    the flops it executes: workgroups * 4 waves * iters * 4 MFMAs * 32768."""
    lib = N.load()
    if sink is None:
        sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    _, sp = _stream()
    N.check(lib.sdpa_measure_mfma_bf16(int(workgroups), int(iters), ctypes.c_void_p(sink.data_ptr()),
                                       sink.numel() * 4, sp))
    return float(workgroups) * 4 * iters * 4 * 32768


@_on_stream
def measure_stream_read(buf: torch.Tensor, workgroups: int = 16384, sink: torch.Tensor = None) -> int:
    """Launch the streaming-read probe (sdpa_measure_stream_read) over the bytes of ``buf``;
    returns the bytes it reads."""
    lib = N.load()
    nbytes = (buf.numel() * buf.element_size()) & ~15
    if sink is None:
        sink = torch.empty(workgroups * 4, dtype=torch.int32, device=buf.device)
    _, sp = _stream()
    N.check(lib.sdpa_measure_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, int(workgroups),
                                         ctypes.c_void_p(sink.data_ptr()), sink.numel() * 4, sp))
    return nbytes
