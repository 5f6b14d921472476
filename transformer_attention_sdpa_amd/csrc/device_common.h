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

// ---- packed sequences (page "Neural Network primitives from NNlib.jl", "Packed sequences") --
// A workgroup of a packed launch handles one tile of `tile` query rows of one segment. The
// tiles are numbered segment by segment; a wave finds the segment of tile `item` by prefix sums
// of the segment lengths (64 segments per step, every lane one segment). Starts and lengths
// are cut to the arrays, so lengths that do not add up cannot reach past them.
struct SegView {
  int s;                       // segment
  int tile;                    // tile within the segment
  int64_t q_start, kv_start;   // first row of the segment in q and in k/v
  int q_len, kv_len;
};

__device__ __forceinline__ int64_t wave_incl_scan64(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ int64_t readfirstlane64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The chunk totals, the running bases and so the loop exit are made scalar: a loop whose exit
// the compiler must take as divergent would make every value leaving it divergent, and the
// buffer resources built from them would need waterfall loops.
__device__ __forceinline__ bool seg_locate(const AttnArgs& a, int item, int tile, SegView& sv) {
  const int lane = threadIdx.x & 63;
  const int32_t* kvs = a.kv_seg ? a.kv_seg : a.q_seg;
  int64_t qbase = 0, kbase = 0, tbase = 0;
  for (int c0 = 0; c0 < a.n_seg; c0 += 64) {
    const int s = c0 + lane;
    const int64_t ql = s < a.n_seg ? max(a.q_seg[s], 0) : 0;
    const int64_t kl = s < a.n_seg ? max(kvs[s], 0) : 0;
    const int64_t qi = wave_incl_scan64(ql), ki = wave_incl_scan64(kl);
    const int64_t q0 = min(qbase + qi - ql, (int64_t)a.Lq), k0 = min(kbase + ki - kl, (int64_t)a.Lkv);
    const int qn = (int)min(ql, (int64_t)a.Lq - q0), kn = (int)min(kl, (int64_t)a.Lkv - k0);
    const int64_t nt = (qn + tile - 1) / tile;
    const int64_t ti = wave_incl_scan64(nt);
    const int64_t tot = readfirstlane64(__shfl(ti, 63, 64));
    if (item < tbase + tot) {
      const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__builtin_amdgcn_ballot_w64(tbase + ti > item)));
      sv.s = c0 + l;
      sv.tile = __builtin_amdgcn_readfirstlane((int)(item - tbase - __shfl(ti - nt, l, 64)));
      sv.q_start = readfirstlane64(__shfl(q0, l, 64));
      sv.kv_start = readfirstlane64(__shfl(k0, l, 64));
      sv.q_len = __builtin_amdgcn_readfirstlane(__shfl(qn, l, 64));
      sv.kv_len = __builtin_amdgcn_readfirstlane(__shfl(kn, l, 64));
      return true;
    }
    tbase += tot;
    qbase += readfirstlane64(__shfl(qi, 63, 64));
    kbase += readfirstlane64(__shfl(ki, 63, 64));
  }
  return false;
}

// The arguments of segment sv as a batch of one: pointers moved to the segment's first rows,
// the segment's lengths as the array lengths, per-segment arrays moved to entry sv.s.
__device__ __forceinline__ AttnArgs seg_args(const AttnArgs& a, const SegView& sv) {
  AttnArgs r = a;
  const int ie = a.in_dtype == SDPA_F32 ? 4 : 2, oe = a.out_dtype == SDPA_F32 ? 4 : 2;
  r.q = static_cast<const char*>(a.q) + sv.q_start * a.q_ss * ie;
  r.k = static_cast<const char*>(a.k) + sv.kv_start * a.k_ss * ie;
  r.v = static_cast<const char*>(a.v) + sv.kv_start * a.v_ss * ie;
  r.out = static_cast<char*>(a.out) + sv.q_start * a.o_ss * oe;
  r.Lq = sv.q_len;
  r.Lkv = sv.kv_len;
  if (a.q_offset) r.q_offset = a.q_offset + sv.s;
  if (a.kv_lengths) r.kv_lengths = a.kv_lengths + sv.s;
  if (a.q_lengths) r.q_lengths = a.q_lengths + sv.s;
  if (a.k_rinv) r.k_rinv = a.k_rinv + sv.kv_start * a.Hkv;
  return r;
}

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

// Element of a dense mask: row at `row` (bytes for U8, 32-bit words for U1), element `col`
// within the row (already multiplied by the element stride).
__device__ __forceinline__ bool mask_bit(const uint8_t* mask, int u1, int64_t row, int64_t col) {
  if (u1) return (reinterpret_cast<const uint32_t*>(mask)[row + (col >> 5)] >> (col & 31)) & 1u;
  return mask[row + col] != 0;
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
    return mask_bit(a.mask, a.mask_u1, b * a.mask_sb + h * a.mask_sh + (int64_t)i * a.mask_sq, (int64_t)j * a.mask_sk);
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
