"""Seeded synthetic inputs for the attention workloads.

This module holds no step of the attention method. It only draws random
numbers, rounds the draws to bfloat16, and lays them out in the shapes of the
workloads. Both sides read its arrays: the fp64 CPU oracle (through the tests
and the bench's CPU leg) and the HIP path (through the Python binding).

Layout (C order, which is the column-major NNlib order reversed, as the NNlib
reference page on ``scaled_dot_product_attention`` states in its "Attention"
section): q and out are [B][Lq][Hq][D]; k, v and the KV caches are
[B][Lkv][Hkv][D]; bias and mask are [B][H][Lq][Lkv], where a dimension of
size 1 broadcasts.

bfloat16 tensors are stored as their uint16 bit patterns. ``bf16_to_f32``
widens them exactly, so both sides see identical values. Float values are
drawn as float32 and rounded to bfloat16 with round-to-nearest-even.

Seeds: every tensor of workload ``k`` comes from
``numpy.random.default_rng([base + k, tag])`` with the tags below, so a
tensor can be regenerated on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_KNEW, TAG_VNEW, TAG_KVLEN, TAG_MCLASS, TAG_MBITS, TAG_BIAS, TAG_DOUT = range(10)
SEED_BASE = 1000

BF16_NAN_BITS = 0x7FC0  # quiet NaN, used to poison cache slots that must never be read


# ----------------------------------------------------------------------------------------------
# bfloat16 bit conversions (input representation only)
# ----------------------------------------------------------------------------------------------
def f32_to_bf16(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN_BITS
    return r


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16 with a single round-to-nearest-even.

    Goes through float32 with round-to-odd, which keeps the second rounding exact.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    # truncate toward zero: step back one ulp where float32 rounding moved away from zero
    away = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(away, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    inexact = f.astype(np.float64) != x
    bits = f.view(np.uint32).copy()
    bits[inexact] |= np.uint32(1)
    return f32_to_bf16(bits.view(np.float32))


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng_for(k: int, tag: int, *sub: int, base: int = SEED_BASE) -> np.random.Generator:
    return np.random.default_rng([base + k, tag, *sub])


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in the stored form of ``dtype``: "bf16" uint16 bits (RNE), "f16" numpy
    float16 (RNE), "f32" unchanged."""
    if dtype == "bf16":
        return f32_to_bf16(x)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    return x


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values of ``dtype`` as float32 (exact for all three)."""
    if dtype == "bf16":
        return bf16_to_f32(a)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    return a


def normal_tensor(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws as float32, in the stored form of ``dtype`` (see to_storage)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return to_storage(x, dtype)


# ----------------------------------------------------------------------------------------------
# A workload: the arrays plus the keyword arguments of one attention call
# ----------------------------------------------------------------------------------------------
@dataclass
class Attention:
    name: str
    dtype: str                       # "f32", "bf16" or "f16": storage of q, k, v (bf16 as uint16 bits)
    q: np.ndarray                    # [B][Lq][Hq][D]
    k: np.ndarray                    # [B][Lkv][Hkv][D]
    v: np.ndarray                    # [B][Lkv][Hkv][Dv]
    scale: Optional[float] = None    # None = 1/sqrt(D)
    is_causal: object = False        # False, True or "bottom_right"
    q_offset: object = 0             # int or int32 [B]
    kv_lengths: Optional[np.ndarray] = None  # None, or int32 [B]
    bias: Optional[np.ndarray] = None        # [Bb][Hb][Lq][Lkv], storage ``bias_dtype``
    bias_dtype: str = "f32"
    mask: Optional[np.ndarray] = None        # uint8 [Mb][Mh][Lq][Lkv], nonzero = attend
    qk_norm: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, Lq, Hq, D = self.q.shape
        _, Lkv, Hkv, Dv = self.v.shape
        return B, Lq, Lkv, Hq, Hkv, D, Dv

    def values(self, name: str) -> np.ndarray:
        """Float32 values of a stored tensor (16-bit storage widened exactly)."""
        a = getattr(self, name)
        if a is None:
            return None
        return widen(a, self.bias_dtype if name == "bias" else self.dtype)


# ----------------------------------------------------------------------------------------------
# Generic random workload (tests use it at small sizes)
# ----------------------------------------------------------------------------------------------
def random_attention(seed: int, B, Lq, Lkv, Hq, Hkv, D, Dv=None, dtype="f32", *, is_causal=False,
                     q_offset=0, kv_lengths=None, bias_shape=None, bias_dtype="f32",
                     mask_shape=None, mask_p=0.7, scale=None, qk_norm=False, dist="normal",
                     name="random") -> Attention:
    """Random q/k/v (and optional bias, mask) for the given shapes.

    ``dist`` is "normal" (N(0,1)) or "uniform" (U[0,1), as in the NNlib examples).
    ``bias_shape``/``mask_shape`` are 4-tuples over [B][H][Lq][Lkv] with 1 for broadcast dims.
    """
    Dv = D if Dv is None else Dv
    def draw(tag, shape):
        rng = np.random.default_rng([seed, tag])
        if dist == "uniform":
            x = rng.random(size=shape, dtype=np.float32)
        else:
            x = rng.standard_normal(size=shape, dtype=np.float32)
        return to_storage(x, dtype)
    q = draw(TAG_Q, (B, Lq, Hq, D))
    k = draw(TAG_K, (B, Lkv, Hkv, D))
    v = draw(TAG_V, (B, Lkv, Hkv, Dv))
    bias = None
    if bias_shape is not None:
        rng = np.random.default_rng([seed, TAG_BIAS])
        b = rng.standard_normal(size=bias_shape, dtype=np.float32)
        bias = to_storage(b, bias_dtype)
    mask = None
    if mask_shape is not None:
        rng = np.random.default_rng([seed, TAG_MBITS])
        mask = (rng.random(size=mask_shape) < mask_p).astype(np.uint8)
    return Attention(name, dtype, q, k, v, scale=scale, is_causal=is_causal, q_offset=q_offset,
                     kv_lengths=kv_lengths, bias=bias, bias_dtype=bias_dtype, mask=mask,
                     qk_norm=qk_norm)


def output_cotangent(w: Attention, seed: int) -> np.ndarray:
    """N(0,1) cotangent of the output of ``w`` ([B][Lq][Hq][Dv]), stored as ``w.dtype``."""
    B, Lq, _, Hq, _, _, Dv = w.shape
    return normal_tensor(np.random.default_rng([seed, TAG_DOUT]), (B, Lq, Hq, Dv), w.dtype)


# ----------------------------------------------------------------------------------------------
# The five workloads, with their sizes as parameters so tests can shrink them
# ----------------------------------------------------------------------------------------------
def tiny_f32(B=1, H=2, D=16, L=64, base=SEED_BASE) -> Attention:
    """Tiny fp32 attention: no GQA, no bias, no mask, not causal, scale 1/sqrt(D)."""
    k = 0
    return Attention(
        "tiny_f32", "f32",
        normal_tensor(rng_for(k, TAG_Q, base=base), (B, L, H, D), "f32"),
        normal_tensor(rng_for(k, TAG_K, base=base), (B, L, H, D), "f32"),
        normal_tensor(rng_for(k, TAG_V, base=base), (B, L, H, D), "f32"),
        scale=1.0 / math.sqrt(D))


def causal_prefill(B=4, H=16, D=128, L=4096, base=SEED_BASE) -> Attention:
    """Causal bf16 prefill: q_len = kv_len = L, is_causal=True, scale 1/sqrt(D)."""
    k = 1
    return Attention(
        "causal_prefill", "bf16",
        normal_tensor(rng_for(k, TAG_Q, base=base), (B, L, H, D), "bf16"),
        normal_tensor(rng_for(k, TAG_K, base=base), (B, L, H, D), "bf16"),
        normal_tensor(rng_for(k, TAG_V, base=base), (B, L, H, D), "bf16"),
        scale=1.0 / math.sqrt(D), is_causal=True)


@dataclass
class Decode:
    """One decode step: KV caches, the T new K/V rows, the write index and the T queries."""
    name: str
    q: np.ndarray            # bf16 bits [B][T][Hq][D]
    k_cache: np.ndarray      # bf16 bits [B][capacity][Hkv][D]
    v_cache: np.ndarray
    k_new: np.ndarray        # bf16 bits [B][T][Hkv][D]
    v_new: np.ndarray
    kv_lengths: np.ndarray   # int32 [B], lengths after the update
    scale: float
    dtype: str = "bf16"

    @property
    def write_index(self) -> np.ndarray:
        """The T new rows go to slots kv_lengths[b] - T .. kv_lengths[b] - 1."""
        return (self.kv_lengths - self.q.shape[1]).astype(np.int32)


def gqa_decode(B=64, Hq=32, Hkv=8, D=128, capacity=8192, kv_min=1024, kv_max=8192,
               base=SEED_BASE, q_len=1, dtype="bf16") -> Decode:
    """GQA decode with a KV cache; q_len new tokens per sequence (1: one decode step).

    kv_lengths[b] ~ U{kv_min..kv_max}. Cache slots [0, kv_lengths[b]-q_len) hold N(0,1) past
    rows (per-batch sub-streams, so one batch element can be regenerated alone); slots from
    kv_lengths[b]-q_len on hold a NaN, so a read of an unwritten slot shows in the output.
    ``dtype`` "bf16" (uint16 bits) or "f16" (numpy float16) storage.
    The new rows go to slots kv_lengths[b]-q_len .. kv_lengths[b]-1 (those below 0 are dropped
    by the cache update).
    """
    k = 2
    kvlen = rng_for(k, TAG_KVLEN, base=base).integers(kv_min, kv_max + 1, size=B).astype(np.int32)
    q = normal_tensor(rng_for(k, TAG_Q, base=base), (B, q_len, Hq, D), dtype)
    k_new = normal_tensor(rng_for(k, TAG_KNEW, base=base), (B, q_len, Hkv, D), dtype)
    v_new = normal_tensor(rng_for(k, TAG_VNEW, base=base), (B, q_len, Hkv, D), dtype)
    if dtype == "bf16":
        k_cache = np.full((B, capacity, Hkv, D), BF16_NAN_BITS, dtype=np.uint16)
    else:
        k_cache = np.full((B, capacity, Hkv, D), np.nan, dtype=np.float16)
    v_cache = k_cache.copy()
    for b in range(B):
        n = max(int(kvlen[b]) - q_len, 0)
        k_cache[b, :n] = decode_cache_rows(k, TAG_K, b, n, Hkv, D, base, dtype)
        v_cache[b, :n] = decode_cache_rows(k, TAG_V, b, n, Hkv, D, base, dtype)
    return Decode("gqa_decode", q, k_cache, v_cache, k_new, v_new, kvlen, 1.0 / math.sqrt(D), dtype)


def decode_cache_rows(k, tag, b, n, Hkv, D, base=SEED_BASE, dtype="bf16") -> np.ndarray:
    """The n past rows of batch element b's cache ([n][Hkv][D] in the stored form of dtype)."""
    return normal_tensor(rng_for(k, tag, b, base=base), (n, Hkv, D), dtype)


def alibi_slopes(H: int) -> np.ndarray:
    """slope_h = 2^(-8(h+1)/H), h = 0..H-1 (fp64)."""
    h = np.arange(H, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / H)


def alibi_bias_bf16(H: int, Lq: int, Lkv: int) -> np.ndarray:
    """Bias[0][h][i][j] = -slope_h * (i - j), computed in fp64, stored as bf16 bits [1][H][Lq][Lkv].

    Taken literally (no absolute value): keys after the query get a positive bias.
    """
    slopes = alibi_slopes(H)
    d = np.arange(-(Lkv - 1), Lq, dtype=np.float64)           # i - j from -(Lkv-1) to Lq-1
    out = np.empty((1, H, Lq, Lkv), dtype=np.uint16)
    ii = np.arange(Lq)[:, None]
    jj = np.arange(Lkv)[None, :]
    idx = (ii - jj) + (Lkv - 1)
    for h in range(H):
        table = f64_to_bf16(-slopes[h] * d)
        out[0, h] = table[idx]
    return out


def block_sparse_mask(Lq: int, Lkv: int, block: int, p_empty=0.3, p_full=0.2,
                      k: int = 3, base=SEED_BASE, shape_prefix=(1, 1)) -> np.ndarray:
    """uint8 mask [*shape_prefix][Lq][Lkv] drawn in block x block tiles.

    Each tile is all-false with probability p_empty, all-true with p_full, and otherwise
    partial with independent Bernoulli(0.5) elements. The mask is a runtime array.
    """
    nqb, nkb = -(-Lq // block), -(-Lkv // block)
    P = int(np.prod(shape_prefix))
    cls = rng_for(k, TAG_MCLASS, base=base).choice(
        3, size=(P, nqb, nkb), p=[p_empty, p_full, 1.0 - p_empty - p_full]).astype(np.int8)
    bits = rng_for(k, TAG_MBITS, base=base).integers(0, 2, size=(P, Lq, Lkv), dtype=np.uint8)
    cls_el = np.repeat(np.repeat(cls, block, axis=1), block, axis=2)[:, :Lq, :Lkv]
    mask = np.where(cls_el == 0, np.uint8(0), np.where(cls_el == 1, np.uint8(1), bits))
    return mask.astype(np.uint8).reshape(*shape_prefix, Lq, Lkv)


def bias_block_mask(B=2, H=16, D=64, L=8192, block=128, base=SEED_BASE) -> Attention:
    """bf16 attention with an ALiBi-style bias and a runtime block-sparse boolean mask."""
    k = 3
    return Attention(
        "bias_block_mask", "bf16",
        normal_tensor(rng_for(k, TAG_Q, base=base), (B, L, H, D), "bf16"),
        normal_tensor(rng_for(k, TAG_K, base=base), (B, L, H, D), "bf16"),
        normal_tensor(rng_for(k, TAG_V, base=base), (B, L, H, D), "bf16"),
        scale=1.0 / math.sqrt(D),
        bias=alibi_bias_bf16(H, L, L), bias_dtype="bf16",
        mask=block_sparse_mask(L, L, block, k=k, base=base),
        extra={"block": block})


def chunked_prefill(B=1, Hq=32, Hkv=8, D=128, Lkv=131072, Lq=2048, q_offset=129024,
                    base=SEED_BASE) -> Attention:
    """A causal chunk of Lq queries at q_offset over Lkv keys, with GQA."""
    k = 4
    return Attention(
        "chunked_prefill", "bf16",
        normal_tensor(rng_for(k, TAG_Q, base=base), (B, Lq, Hq, D), "bf16"),
        normal_tensor(rng_for(k, TAG_K, base=base), (B, Lkv, Hkv, D), "bf16"),
        normal_tensor(rng_for(k, TAG_V, base=base), (B, Lkv, Hkv, D), "bf16"),
        scale=1.0 / math.sqrt(D), is_causal=True, q_offset=q_offset)


def pack_mask_bits(mask: np.ndarray, pad_bit: int = 0) -> np.ndarray:
    """A boolean/uint8 mask [..., Lkv] as the 32-per-word U1 layout: int32 words [..., ceil(Lkv/32)],
    element c of a row in bit c % 32 of word c // 32. ``pad_bit`` fills the bits past Lkv in each
    row's last word (they must not matter).
    """
    m = np.asarray(mask) != 0
    Lkv = m.shape[-1]
    W = (Lkv + 31) // 32
    full = np.full(m.shape[:-1] + (W * 32,), bool(pad_bit))
    full[..., :Lkv] = m
    by = np.packbits(full, axis=-1, bitorder="little")            # 4 bytes per word, little-endian
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32).view(np.int32)
