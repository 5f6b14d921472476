// device_common.h -- device helpers shared by the attention kernels: element loads and stores,
// per-batch length/offset resolution and the allowed-key predicate.
//
// The predicate is the AND of the conditions of the page "Neural Network primitives from
// NNlib.jl", "Arguments" list: the boolean mask, the causal rule (query i attends keys
// j <= q_offset + i; bottom-right alignment takes q_offset = kv_len - q_len) and kv_lengths.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace sdpa {

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> IEEE binary16, round to nearest even (overflow to +-inf, NaN stays NaN).
__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == SDPA_BF16) return bf16_bits_to_float(static_cast<const uint16_t*>(base)[idx]);
  if (dtype == SDPA_F16) return f16_bits_to_float(static_cast<const uint16_t*>(base)[idx]);
  return static_cast<const float*>(base)[idx];
}

__device__ __forceinline__ void store_elem(void* base, int64_t idx, int dtype, float x) {
  if (dtype == SDPA_BF16) static_cast<uint16_t*>(base)[idx] = float_to_bf16_bits(x);
  else if (dtype == SDPA_F16) static_cast<uint16_t*>(base)[idx] = float_to_f16_bits(x);
  else static_cast<float*>(base)[idx] = x;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Valid keys of batch element b: kv_lengths clamped to [0, Lkv], or Lkv when none is given.
__device__ __forceinline__ int batch_kv_len(const AttnArgs& a, int b) {
  int n = a.kv_lengths ? a.kv_lengths[b] : (a.kv_length_all >= 0 ? a.kv_length_all : a.Lkv);
  return clampi(n, 0, a.Lkv);
}

// Valid queries of batch element b: q_lengths clamped to [0, Lq], or Lq when none is given.
__device__ __forceinline__ int batch_q_len(const AttnArgs& a, int b) {
  int n = a.q_lengths ? a.q_lengths[b] : (a.q_length_all >= 0 ? a.q_length_all : a.Lq);
  return clampi(n, 0, a.Lq);
}

// off_b of the causal rule j <= off_b + i (64-bit so extreme offsets cannot wrap).
__device__ __forceinline__ int64_t batch_causal_offset(const AttnArgs& a, int b) {
  if (a.causal == SDPA_CAUSAL_TRUE) return a.q_offset ? a.q_offset[b] : a.q_offset_all;
  if (a.causal == SDPA_CAUSAL_BOTTOM_RIGHT) return (int64_t)batch_kv_len(a, b) - batch_q_len(a, b);
  return 0;
}

// Mask element (b, h, i, j): dense array or block info; true when no mask is given.
__device__ __forceinline__ bool mask_allows(const AttnArgs& a, int b, int h, int i, int j) {
  if (a.bm_class) {
    const int mb = a.bm_batch > 1 ? b : 0, mh = a.bm_heads > 1 ? h : 0;
    const int qb = i / a.bm_bq, kb = j / a.bm_bkv;
    const int64_t blk = (((int64_t)mb * a.bm_heads + mh) * a.bm_nqb + qb) * a.bm_nkb + kb;
    const int c = a.bm_class[blk];
    if (c != 1) return c == 2;
    const int words = a.bm_bkv / 32;
    const int r = i - qb * a.bm_bq, col = j - kb * a.bm_bkv;
    const uint32_t w = a.bm_bits[((int64_t)a.bm_next[blk] * a.bm_bq + r) * words + col / 32];
    return (w >> (col & 31)) & 1u;
  }
  if (a.mask) {
    return a.mask[b * a.mask_sb + h * a.mask_sh + (int64_t)i * a.mask_sq + (int64_t)j * a.mask_sk] != 0;
  }
  return true;
}

// The combined predicate (mask AND causal AND kv_lengths) for query i and key j of (b, h).
__device__ __forceinline__ bool key_allowed(const AttnArgs& a, int b, int h, int i, int j, int nkv,
                                            int64_t off) {
  if (j >= nkv) return false;
  if (a.causal != SDPA_CAUSAL_NONE && (int64_t)j > off + i) return false;
  return mask_allows(a, b, h, i, j);
}

__device__ __forceinline__ float bias_at(const AttnArgs& a, int b, int h, int i, int j) {
  const int64_t idx = b * a.bias_sb + h * a.bias_sh + (int64_t)i * a.bias_sq + (int64_t)j * a.bias_sk;
  return load_elem(a.bias, idx, a.bias_dtype);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace sdpa
