"""The C ABI on the CPU: the library loads, exports every function include/sdpa.h declares,
and rejects every host-detectable bad argument with its status before touching the GPU.
No call here launches a kernel."""
import ctypes
import math

import pytest

import transformer_attention_sdpa_amd as sa
from transformer_attention_sdpa_amd import _native as N

FAKE = 0x1000   # a non-NULL address; validation fails before any pointer is used


@pytest.fixture(scope="module")
def lib():
    return sa.load()


def T(dims, dtype=N.SDPA_BF16, strides=None, data=FAKE):
    """Descriptor with NNlib-order dims (fastest first); contiguous strides by default."""
    t = N.SdpaTensor()
    t.data = data
    t.dtype = dtype
    st = strides
    if st is None:
        st, acc = [], 1
        for d in dims:
            st.append(acc)
            acc *= d
    for i in range(4):
        t.dims[i] = dims[i]
        t.strides[i] = st[i]
    return t


def fwd(lib, q, k, v, out, bias=None, mask=None, info=None, scale=math.nan, causal=0, qk_norm=0,
        ws=None, ws_bytes=0):
    r = lib.sdpa_fwd(ctypes.byref(q) if q else None, ctypes.byref(k) if k else None,
                     ctypes.byref(v) if v else None, ctypes.byref(bias) if bias else None,
                     ctypes.byref(mask) if mask else None, ctypes.byref(info) if info else None,
                     scale, causal, None, 0, None, -1, None, -1, qk_norm,
                     ctypes.byref(out) if out else None, ws, ws_bytes, None)
    return r, lib.sdpa_last_error().decode()


def test_every_declared_function_is_exported(lib):
    names = sa.header_functions()
    assert {"sdpa_fwd", "sdpa_decode", "kv_cache_update", "build_block_mask_info"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(N.PROTOTYPES), "binding prototypes and header disagree"


def test_status_strings(lib):
    assert lib.sdpa_status_string(0) == b"ok"
    assert lib.sdpa_status_string(N.SDPA_ERR_SHAPE) == b"shape mismatch"
    assert lib.sdpa_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.sdpa_version()


def good(D=64, Hq=8, Hkv=2, Lq=5, Lkv=7, B=3, dt=N.SDPA_BF16):
    return (T([D, Hq, Lq, B], dt), T([D, Hkv, Lkv, B], dt), T([D, Hkv, Lkv, B], dt), T([D, Hq, Lq, B], dt))


CASES = {
    "gqa_indivisible": (lambda: good(Hq=6, Hkv=4), N.SDPA_ERR_SHAPE, {}),
    "qk_dim_mismatch": (lambda: (T([64, 8, 5, 3]), T([32, 2, 7, 3]), T([64, 2, 7, 3]), T([64, 8, 5, 3])),
                        N.SDPA_ERR_SHAPE, {}),
    "kv_len_mismatch": (lambda: (T([64, 8, 5, 3]), T([64, 2, 7, 3]), T([64, 2, 6, 3]), T([64, 8, 5, 3])),
                        N.SDPA_ERR_SHAPE, {}),
    "batch_mismatch": (lambda: (T([64, 8, 5, 3]), T([64, 2, 7, 2]), T([64, 2, 7, 2]), T([64, 8, 5, 3])),
                       N.SDPA_ERR_SHAPE, {}),
    "out_shape": (lambda: good()[:3] + (T([64, 8, 6, 3]),), N.SDPA_ERR_SHAPE, {}),
    "inner_stride": (lambda: (T([64, 8, 5, 3], strides=[2, 128, 1024, 5120]),) + good()[1:], N.SDPA_ERR_SHAPE, {}),
    "mixed_dtype": (lambda: (T([64, 8, 5, 3], N.SDPA_F32),) + good()[1:], N.SDPA_ERR_DTYPE, {}),
    "u8_inputs": (lambda: good(dt=N.SDPA_U8), N.SDPA_ERR_DTYPE, {}),
    "f16_q_bf16_kv": (lambda: (T([64, 8, 5, 3], N.SDPA_F16),) + good()[1:], N.SDPA_ERR_DTYPE, {}),
    "unknown_dtype": (lambda: good(dt=7), N.SDPA_ERR_DTYPE, {}),
    "head_dim_too_big": (lambda: good(D=320), N.SDPA_ERR_UNSUPPORTED, {}),
    "bad_causal": (lambda: good(), N.SDPA_ERR_SHAPE, {"causal": 3}),
    "bad_qk_norm": (lambda: good(), N.SDPA_ERR_SHAPE, {"qk_norm": 2}),
    "bias_bad_dim": (lambda: good(), N.SDPA_ERR_SHAPE, {"bias": T([7, 5, 4, 3])}),
    "bias_u8": (lambda: good(), N.SDPA_ERR_DTYPE, {"bias": T([7, 5, 8, 3], N.SDPA_U8)}),
    "mask_bf16": (lambda: good(), N.SDPA_ERR_DTYPE, {"mask": T([7, 5, 1, 1], N.SDPA_BF16)}),
    "mask_u1_strided": (lambda: good(), N.SDPA_ERR_SHAPE, {"mask": T([7, 5, 1, 1], N.SDPA_U1, strides=[2, 1, 1, 1])}),
    "u1_inputs": (lambda: good(dt=N.SDPA_U1), N.SDPA_ERR_DTYPE, {}),
    "mask_bad_dim": (lambda: good(), N.SDPA_ERR_SHAPE, {"mask": T([7, 4, 1, 1], N.SDPA_U8)}),
    "qk_norm_no_workspace": (lambda: good(), N.SDPA_ERR_WORKSPACE, {"qk_norm": 1}),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fwd_validation(lib, name):
    make, status, kw = CASES[name]
    q, k, v, out = make()
    r, msg = fwd(lib, q, k, v, out, **kw)
    assert r == status, (name, r, msg)
    assert msg, "a failing call must leave a message"


def test_fwd_null_descriptors(lib):
    q, k, v, out = good()
    assert fwd(lib, None, k, v, out)[0] == N.SDPA_ERR_NULL
    assert fwd(lib, q, k, v, None)[0] == N.SDPA_ERR_NULL
    q0 = T([64, 8, 5, 3], data=None)
    assert fwd(lib, q0, k, v, out)[0] == N.SDPA_ERR_NULL


def test_fwd_empty_query_is_a_noop_without_a_gpu(lib):
    q, k, v, out = good(Lq=0)
    assert fwd(lib, q, k, v, out)[0] == N.SDPA_OK


def test_mask_info_validation(lib):
    q, k, v, out = good(Lq=300, Lkv=260)
    info = N.BlockMaskInfoC()
    info.mask_batch, info.mask_heads, info.q_len, info.kv_len = 1, 1, 300, 260
    info.bq, info.bkv, info.n_qb, info.n_kb = 128, 128, 3, 3
    for f in ("block_mask", "mask_next", "row_ptr", "data_next", "partial_bits", "n_partial"):
        setattr(info, f, FAKE)
    info.n_kb = 2                                        # wrong grid
    assert fwd(lib, q, k, v, out, info=info)[0] == N.SDPA_ERR_SHAPE
    info.n_kb = 3
    info.kv_len = 259                                    # built for another length
    assert fwd(lib, q, k, v, out, info=info)[0] == N.SDPA_ERR_SHAPE
    info.kv_len = 260
    info.mask_heads = 3                                  # neither 1 nor Hq
    assert fwd(lib, q, k, v, out, info=info)[0] == N.SDPA_ERR_SHAPE


def test_workspace_sizes(lib):
    q, k, v, _ = good(D=64, Hq=8, Hkv=2, Lq=5, Lkv=7, B=3)
    assert lib.sdpa_fwd_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0) == 0
    assert lib.sdpa_fwd_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 1) == 3 * 7 * 2 * 4
    qd = T([128, 32, 1, 64])
    kc = T([128, 8, 8192, 64])
    # 1024 keys per split by default -> 8 splits; (D + 2) floats per (b, head, split)
    assert lib.sdpa_decode_workspace_bytes(ctypes.byref(qd), ctypes.byref(kc), 0) == 64 * 32 * 8 * 130 * 4
    assert lib.sdpa_decode_workspace_bytes(ctypes.byref(qd), ctypes.byref(kc), 4) == 64 * 32 * 4 * 130 * 4
    # T query tokens: one partial per (b, token, head, split)
    q3 = T([128, 32, 3, 64])
    assert lib.sdpa_decode_workspace_bytes(ctypes.byref(q3), ctypes.byref(kc), 0) == 64 * 3 * 32 * 8 * 130 * 4


def test_decode_validation(lib):
    qd, kc, vc, od = T([128, 32, 1, 4]), T([128, 8, 64, 4]), T([128, 8, 64, 4]), T([128, 32, 1, 4])
    def call(q=qd, k=kc, v=vc, o=od, kvl=FAKE, splits=0, ws=FAKE, wsb=1 << 30):
        return lib.sdpa_decode(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), kvl, math.nan, splits,
                               ctypes.byref(o), ws, wsb, None)
    assert call(kvl=None) == N.SDPA_ERR_NULL
    assert call(q=T([128, 32, 65, 4]), o=T([128, 32, 65, 4])) == N.SDPA_ERR_SHAPE   # more tokens than capacity
    assert call(q=T([128, 32, 3, 4]), o=T([128, 32, 2, 4])) == N.SDPA_ERR_SHAPE    # out tokens != q tokens
    assert call(q=T([128, 32, 3, 4]), o=T([128, 32, 3, 4]), wsb=4 * 3 * 32 * 130 * 4 - 1) == N.SDPA_ERR_WORKSPACE
    assert call(splits=-1) == N.SDPA_ERR_SHAPE
    assert call(wsb=16) == N.SDPA_ERR_WORKSPACE
    assert call(k=T([64, 8, 64, 4])) == N.SDPA_ERR_SHAPE
    assert call(q=T([128, 30, 1, 4]), o=T([128, 30, 1, 4])) == N.SDPA_ERR_SHAPE      # 30 % 8


def test_kv_cache_update_validation(lib):
    kc, vc = T([128, 8, 64, 4]), T([128, 8, 64, 4])
    kn, vn = T([128, 8, 1, 4]), T([128, 8, 1, 4])
    def call(a=kc, b=vc, c=kn, d=vn, wi=FAKE):
        return lib.kv_cache_update(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), ctypes.byref(d), wi, None)
    assert call(wi=None) == N.SDPA_ERR_NULL
    assert call(c=T([128, 4, 1, 4]), d=T([128, 4, 1, 4])) == N.SDPA_ERR_SHAPE
    assert call(b=T([128, 8, 32, 4])) == N.SDPA_ERR_SHAPE
    assert call(c=T([128, 8, 1, 4], N.SDPA_F32)) == N.SDPA_ERR_DTYPE
    assert call(d=T([128, 8, 1, 4], N.SDPA_F16)) == N.SDPA_ERR_DTYPE     # f16 rows into bf16 caches


def test_block_mask_info_bytes(lib):
    m = T([8192, 8192, 1, 1], N.SDPA_U8)
    nb = ctypes.c_size_t()
    assert lib.sdpa_block_mask_info_bytes(ctypes.byref(m), 128, 128, ctypes.byref(nb)) == N.SDPA_OK
    blocks = 64 * 64
    assert nb.value >= blocks * (1 + 4 + 4) + 65 * 4 + 4 + blocks * 128 * 4 * 4
    assert lib.sdpa_block_mask_info_bytes(ctypes.byref(m), 128, 48, ctypes.byref(nb)) == N.SDPA_ERR_SHAPE
    assert lib.sdpa_block_mask_info_bytes(ctypes.byref(T([64, 64, 1, 1], N.SDPA_BF16)), 32, 32,
                                          ctypes.byref(nb)) == N.SDPA_ERR_DTYPE
    info = N.BlockMaskInfoC()
    assert lib.build_block_mask_info(ctypes.byref(m), 128, 128, FAKE, 16, ctypes.byref(info),
                                     None) == N.SDPA_ERR_WORKSPACE


def test_head_rms_norm_validation(lib):
    x = T([4, 2, 3, 1], N.SDPA_F32)
    assert lib.head_rms_norm(ctypes.byref(x), ctypes.byref(T([4, 2, 3, 2], N.SDPA_F32)), 1e-6, None) == N.SDPA_ERR_SHAPE
    assert lib.head_rms_norm(ctypes.byref(x), ctypes.byref(T([4, 2, 3, 1], N.SDPA_BF16)), 1e-6, None) == N.SDPA_ERR_DTYPE
    assert lib.head_rms_norm(ctypes.byref(x), ctypes.byref(T([4, 2, 3, 1], N.SDPA_F32)), -1.0, None) == N.SDPA_ERR_SHAPE


def test_packed_validation(lib):
    q, k, v, o = T([64, 8, 30, 1]), T([64, 2, 40, 1]), T([64, 2, 40, 1]), T([64, 8, 30, 1])
    def call(q=q, k=k, v=v, o=o, qs=FAKE, ks=None, n=3, maxlen=-1, norm=0, wsb=1 << 30, ws=FAKE):
        return lib.sdpa_fwd_packed(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), qs, ks, n, maxlen,
                                   math.nan, 0, None, 0, None, -1, None, -1, norm, ctypes.byref(o), ws, wsb, None)
    assert call(n=-1) == N.SDPA_ERR_SHAPE
    assert call(qs=None) == N.SDPA_ERR_NULL
    assert call(maxlen=-2) == N.SDPA_ERR_SHAPE
    assert call(q=T([64, 8, 15, 2]), o=T([64, 8, 15, 2])) == N.SDPA_ERR_SHAPE      # a batch dimension
    assert call(k=T([64, 2, 40, 2]), v=T([64, 2, 40, 2])) == N.SDPA_ERR_SHAPE
    assert call(norm=1, wsb=16) == N.SDPA_ERR_WORKSPACE
    assert call(q=T([64, 8, 30, 1], N.SDPA_F16)) == N.SDPA_ERR_DTYPE
    assert call(n=0) == N.SDPA_OK                                                    # nothing to do


def bwd(lib, ts, lse=FAKE, mask=None, scale=math.nan, causal=0, ws=FAKE, ws_bytes=1 << 20, dscale=None):
    q, k, v, out, dout, dq, dk, dv = ts
    ref = lambda t: ctypes.byref(t) if t else None
    r = lib.sdpa_bwd(ref(q), ref(k), ref(v), ref(out), ref(dout), lse, ref(mask), None, scale, causal,
                     None, 0, None, -1, None, -1, ref(dq), ref(dk), ref(dv), dscale, ws, ws_bytes, None)
    return r, lib.sdpa_last_error().decode()


def good_bwd(D=64, Hq=8, Hkv=2, Lq=5, Lkv=7, B=3, dt=N.SDPA_BF16):
    q, k, v, out = good(D, Hq, Hkv, Lq, Lkv, B, dt)
    return [q, k, v, out, T([D, Hq, Lq, B], dt), T([D, Hq, Lq, B], dt), T([D, Hkv, Lkv, B], dt),
            T([D, Hkv, Lkv, B], N.SDPA_F32)]


def test_bwd_validation(lib):
    def with_(i, t):
        ts = good_bwd()
        ts[i] = t
        return ts
    assert bwd(lib, with_(4, None))[0] == N.SDPA_ERR_NULL                           # no dout
    assert bwd(lib, with_(5, None))[0] == N.SDPA_ERR_NULL                           # no dq
    assert bwd(lib, with_(4, T([64, 8, 6, 3])))[0] == N.SDPA_ERR_SHAPE              # dout dims
    assert bwd(lib, with_(6, T([64, 2, 6, 3])))[0] == N.SDPA_ERR_SHAPE              # dk dims
    assert bwd(lib, with_(7, T([32, 2, 7, 3])))[0] == N.SDPA_ERR_SHAPE              # dv dims
    assert bwd(lib, with_(5, T([64, 8, 5, 3], N.SDPA_U8)))[0] == N.SDPA_ERR_DTYPE   # dq dtype
    assert bwd(lib, with_(4, T([64, 8, 5, 3], strides=[2, 128, 1024, 5120])))[0] == N.SDPA_ERR_SHAPE
    assert bwd(lib, good_bwd(), lse=None)[0] == N.SDPA_ERR_NULL
    r, msg = bwd(lib, good_bwd(), ws_bytes=16)
    assert r == N.SDPA_ERR_WORKSPACE and "workspace" in msg
    assert bwd(lib, good_bwd(), causal=3)[0] == N.SDPA_ERR_SHAPE
    assert bwd(lib, good_bwd(dt=N.SDPA_U8))[0] == N.SDPA_ERR_DTYPE


def test_bwd_workspace_bytes(lib):
    q, k, v = good_bwd()[:3]
    n = lib.sdpa_bwd_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v))
    rows = 3 * 8 * 5
    assert n == 3 * ((rows * 4 + 255) // 256 * 256) + 256      # + one chunk of first-stage dscale sums


def test_bwd_workspace_bytes_ds(lib):
    # the stored-dS route: the minimum, the dK/dV workgroups' dscale shares (8 each, one 128-key
    # block of 2 K/V heads in 3 batches), one chunk of their first-stage sums, and one 16 KiB dS
    # tile per (batch, query head, 64-query tile, 128-key block)
    f = lambda ts: lib.sdpa_bwd_workspace_bytes_ds(*(ctypes.byref(t) for t in ts[:3]))
    base = lib.sdpa_bwd_workspace_bytes(*(ctypes.byref(t) for t in good_bwd()[:3]))
    assert f(good_bwd()) == base + 256 + 256 + 3 * 8 * 1 * 1 * 16384
    assert f(good_bwd(Lq=65, Lkv=129)) == (lib.sdpa_bwd_workspace_bytes(*(ctypes.byref(t) for t in good_bwd(Lq=65, Lkv=129)[:3]))
                                          + 512 + 256 + 3 * 8 * 2 * 2 * 16384)   # 96 shares: 384 bytes
    assert f(good_bwd(D=128, dt=N.SDPA_F16)) > 0
    assert f(good_bwd(dt=N.SDPA_F32)) == 0                 # 16-bit inputs only
    assert f(good_bwd(D=32)) == 0                          # head dims 64 and 128 only
    assert f(good_bwd(Lq=0)) == 0
    # dS tiles above 8 GiB: the dQ pass forms the weights again
    assert f(good_bwd(D=128, Hq=16, Hkv=16, Lq=8192, Lkv=8192, B=5)) == 0
    assert f(good_bwd(D=128, Hq=16, Hkv=16, Lq=8192, Lkv=8192, B=4)) > 0


def test_decode_per_batch_lengths_are_checked_on_the_host(lib):
    # the kernels read kv_lengths[b] (and write_index[b]) for every batch element: a shorter
    # array is refused before anything reaches the device; an int or one entry broadcasts
    import numpy as np
    import torch
    from transformer_attention_sdpa_amd.api import _per_batch_tensor
    q = torch.zeros((3, 1, 4, 128), dtype=torch.bfloat16)
    kc = torch.zeros((3, 16, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="kv_lengths needs one entry per batch element"):
        sa.sdpa_decode(q, kc, kc, [5, 6])
    with pytest.raises(ValueError, match="kv_lengths needs one entry per batch element"):
        sa.sdpa_decode(q, kc, kc, np.array([5, 6, 7, 8], dtype=np.int32))
    with pytest.raises(ValueError, match="write_index needs one entry per batch element"):
        sa.kv_cache_update(kc, kc, q[:, :, :2], q[:, :, :2], [0, 1])
    assert _per_batch_tensor(5, 3, "cpu", "x").tolist() == [5, 5, 5]
    assert _per_batch_tensor([7], 3, "cpu", "x").tolist() == [7, 7, 7]
    assert _per_batch_tensor(np.array([1, 2, 3]), 3, "cpu", "x").dtype == torch.int32


def test_decode_noalloc_refuses_more_than_its_scratch(lib):
    # 64 sequences x 32 query heads x 128 splits of a 65536-slot cache need 136 MB of partials,
    # more than the 32 MiB scratch: refused on the host, before any launch
    import torch
    assert sa.decode_noalloc_max_scratch_bytes() == 32 << 20
    q = torch.zeros(128, dtype=torch.bfloat16).expand(64, 1, 32, 128)
    kc = torch.zeros(128, dtype=torch.bfloat16).expand(64, 65536, 8, 128)
    out = torch.zeros(128, dtype=torch.float32).expand(64, 1, 32, 128)
    kvl = torch.zeros(64, dtype=torch.int32)
    dq, dk, do = sa.desc(q), sa.desc(kc), sa.desc(out)
    st = lib.sdpa_decode_noalloc(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dk), ctypes.c_void_p(kvl.data_ptr()),
                                 math.nan, 0, ctypes.byref(do), None)
    assert st == N.SDPA_ERR_WORKSPACE
    assert "device scratch holds" in lib.sdpa_last_error().decode()
    assert sa.decode_workspace_bytes(q, kc, 0) > sa.decode_noalloc_max_scratch_bytes()


def fwd_path(lib, q, k, v, out, bias=None, scale=math.nan, causal=0, qk_norm=0):
    p = ctypes.c_int32(0)
    r = lib.sdpa_fwd_path(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(bias) if bias else None,
                          None, None, scale, causal, qk_norm, ctypes.byref(out), ctypes.byref(p))
    return r, p.value


def test_fwd_path_names_the_kernel_family(lib):
    # bf16 at D = 128 with aligned contiguous views: matrix cores; each thing the matrix-core
    # kernels decline moves the call to the fp32 kernels (nothing is launched)
    B, L, H, D = 2, 256, 4, 128
    q, k, v, o = (T([D, H, L, B]) for _ in range(4))
    assert fwd_path(lib, q, k, v, o) == (N.SDPA_OK, N.PATH_MATRIX_CORE)
    assert fwd_path(lib, q, k, v, o, causal=N.CAUSAL_TRUE) == (N.SDPA_OK, N.PATH_MATRIX_CORE)
    f32 = [T([D, H, L, B], N.SDPA_F32) for _ in range(4)]
    assert fwd_path(lib, *f32) == (N.SDPA_OK, N.PATH_FP32)
    q96, k96, v96, o96 = (T([96, H, L, B]) for _ in range(4))
    assert fwd_path(lib, q96, k96, v96, o96) == (N.SDPA_OK, N.PATH_FP32)
    assert fwd_path(lib, q, k, v, o, scale=-0.1) == (N.SDPA_OK, N.PATH_FP32)
    qmis = T([D, H, L, B], data=FAKE + 8)          # not 16-byte aligned
    assert fwd_path(lib, qmis, k, v, o) == (N.SDPA_OK, N.PATH_FP32)
    b16 = T([L, L, H, 1], N.SDPA_F16, strides=[1, L, L * L, 0])
    assert fwd_path(lib, q, k, v, o, bias=b16) == (N.SDPA_OK, N.PATH_FP32)
    bbf = T([L, L, H, 1], N.SDPA_BF16, strides=[1, L, L * L, 0])
    assert fwd_path(lib, q, k, v, o, bias=bbf) == (N.SDPA_OK, N.PATH_MATRIX_CORE)
    # invalid arguments: the call's own status
    kbad = T([D, H, L + 1, B + 1])
    assert fwd_path(lib, q, kbad, v, o)[0] == N.SDPA_ERR_SHAPE


def test_bwd_path_names_the_route(lib):
    B, L, H, D = 2, 256, 4, 128
    q, k, v, o, do, dq, dk, dv = (T([D, H, L, B]) for _ in range(8))
    need = lib.sdpa_bwd_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v))
    need_ds = lib.sdpa_bwd_workspace_bytes_ds(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v))
    assert need_ds > need > 0

    def path(ws, *t, scale=math.nan):
        p = ctypes.c_int32(0)
        r = lib.sdpa_bwd_path(*(ctypes.byref(x) for x in t[:5]), None, None, scale, N.CAUSAL_TRUE,
                              *(ctypes.byref(x) for x in t[5:]), ws, ctypes.byref(p))
        return r, p.value

    assert path(need_ds, q, k, v, o, do, dq, dk, dv) == (N.SDPA_OK, N.PATH_MATRIX_CORE_STORED_DS)
    assert path(need, q, k, v, o, do, dq, dk, dv) == (N.SDPA_OK, N.PATH_MATRIX_CORE)
    f32 = [T([D, H, L, B], N.SDPA_F32) for _ in range(8)]
    assert path(need_ds, *f32) == (N.SDPA_OK, N.PATH_FP32)
    assert path(need_ds, q, k, v, o, do, dq, dk, dv, scale=-1.0) == (N.SDPA_OK, N.PATH_FP32)
    dq_bad = T([D, H, L + 1, B])
    assert path(need_ds, q, k, v, o, do, dq_bad, dk, dv)[0] == N.SDPA_ERR_SHAPE
