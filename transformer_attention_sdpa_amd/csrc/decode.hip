// decode.hip -- attention of one new query per sequence against a KV cache, split over keys.
//
// Cached attention is what makes generation practical (keras issue "MultiHeadAttention is
// missing a position_bias call argument, ...", its list of extensions); the result equals the
// bottom-right causal attention of a single query over kv_lengths[b] keys (page "Neural
// Network primitives from NNlib.jl", "Arguments": is_causal and kv_lengths, and the cache
// example under "Examples").
//
// The work is bound by streaming the cache from HBM (about 4 flops per byte), so the design
// is about bytes in flight and coalescing, not about matrix units:
//   pass 1 (decode_split): one workgroup per (K/V head g, key split s, sequence b). It streams
//     its split in tiles of 64 keys: 16-byte loads of whole K and V rows into LDS, the loads of
//     the next tile issued before the current one is consumed. Every query head that shares g
//     (grouped-query attention) is scored from the same tile: lane = key for q.k (bf16 dot2
//     with fp32 accumulate), lane = pair of head-dim elements for p*V. The online softmax is
//     kept in the exp2 domain (logits pre-multiplied by scale*log2 e). The split writes its
//     running max m, sum l and unnormalised output o in fp32.
//   pass 2 (decode_combine): per (query head, sequence), the splits merge by log-sum-exp:
//     M = max m_s, out = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s. This merge is exact because
//     the online softmax is associative (NNlib "Fused implementation": softmax taken online
//     over tiles of keys). No key at all gives NaN ("Fused implementation").
#include <algorithm>

#include "device_common.h"

namespace sdpa {

namespace {

constexpr int kDecD = 128;
constexpr int kDecTile = 64;
constexpr int kDecThreads = 256;
constexpr int kKRow = kDecD + 8;          // K row pitch in LDS (bf16): 272 B spreads rows over banks

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

template <int NH>   // query heads per wave: the group's r = Hq/Hkv heads spread over 4 waves
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeArgs a) {
  __shared__ __align__(16) uint16_t k_lds[kDecTile * kKRow];
  __shared__ __align__(16) uint16_t v_lds[kDecTile * kDecD];

  const int r = a.Hq / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int split = blockIdx.x / a.Hkv;
  const int b = blockIdx.y;
  const int nkv = clampi(a.kv_lengths[b], 0, a.cap);
  const int j_begin = split * a.split_len;
  if (j_begin >= nkv) return;                       // workgroup-uniform
  const int j_end = min(j_begin + a.split_len, nkv);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // query rows of this wave's heads, as packed bf16 pairs (wave-uniform)
  uint32_t qv[NH][kDecD / 2];
  bool active[NH];
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const int hl = wave + 4 * u;
    active[u] = hl < r;
    const int hq = g * r + (active[u] ? hl : 0);
    const uint32_t* qp = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + b * a.q_sb +
                                                           hq * a.q_sh);
#pragma unroll
    for (int t = 0; t < kDecD / 2; ++t) qv[u][t] = qp[t];
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.k_sb + g * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.v_sb + g * a.v_sh;

  uint4 kr[4], vr[4];
  auto gload = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kDecThreads * u;          // 16-byte chunk: row c/16, column (c%16)*8
      const int row = c >> 4, col = (c & 15) * 8;
      const int j = j0 + row;
      if (j < j_end) {
        kr[u] = *reinterpret_cast<const uint4*>(kbase + (int64_t)j * a.k_ss + col);
        vr[u] = *reinterpret_cast<const uint4*>(vbase + (int64_t)j * a.v_ss + col);
      } else {                                      // zero, never the poisoned tail: 0 * NaN = NaN
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kDecThreads * u;
      const int row = c >> 4, col = (c & 15) * 8;
      *reinterpret_cast<uint4*>(&k_lds[row * kKRow + col]) = kr[u];
      *reinterpret_cast<uint4*>(&v_lds[row * kDecD + col]) = vr[u];
    }
  };

  float m[NH], l[NH], o0[NH], o1[NH];
#pragma unroll
  for (int u = 0; u < NH; ++u) { m[u] = -INFINITY; l[u] = 0.f; o0[u] = 0.f; o1[u] = 0.f; }

  gload(j_begin);
  for (int j0 = j_begin; j0 < j_end; j0 += kDecTile) {
    sstore();
    __syncthreads();
    if (j0 + kDecTile < j_end) gload(j0 + kDecTile);

    // scores: lane = key
    const bool key_ok = j0 + lane < j_end;
    float s[NH];
#pragma unroll
    for (int u = 0; u < NH; ++u) s[u] = 0.f;
    const uint4* krow = reinterpret_cast<const uint4*>(&k_lds[lane * kKRow]);
#pragma unroll
    for (int c = 0; c < kDecD / 8; ++c) {
      const uint4 kk = krow[c];
#pragma unroll
      for (int u = 0; u < NH; ++u) {
        s[u] = dot2_bf16(kk.x, qv[u][4 * c + 0], s[u]);
        s[u] = dot2_bf16(kk.y, qv[u][4 * c + 1], s[u]);
        s[u] = dot2_bf16(kk.z, qv[u][4 * c + 2], s[u]);
        s[u] = dot2_bf16(kk.w, qv[u][4 * c + 3], s[u]);
      }
    }
    float p[NH];
#pragma unroll
    for (int u = 0; u < NH; ++u) {
      const float t = key_ok ? s[u] * a.scale_log2 : -INFINITY;
      const float m_new = fmaxf(m[u], wave_max(t));        // finite: the tile holds a valid key
      p[u] = __builtin_amdgcn_exp2f(t - m_new);
      const float alpha = __builtin_amdgcn_exp2f(m[u] - m_new);
      l[u] = l[u] * alpha + p[u];
      o0[u] *= alpha;
      o1[u] *= alpha;
      m[u] = m_new;
    }
    // p * V: lane = head-dim pair (2*lane, 2*lane+1)
    const uint32_t* vcol = reinterpret_cast<const uint32_t*>(v_lds) + lane;
#pragma unroll 16
    for (int jj = 0; jj < kDecTile; ++jj) {
      const uint32_t vv = vcol[jj * (kDecD / 2)];
      const float v_lo = __uint_as_float(vv << 16), v_hi = __uint_as_float(vv & 0xffff0000u);
#pragma unroll
      for (int u = 0; u < NH; ++u) {
        const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[u]), jj));
        o0[u] = fmaf(pj, v_lo, o0[u]);
        o1[u] = fmaf(pj, v_hi, o1[u]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const float lsum = wave_sum(l[u]);
    if (!active[u]) continue;
    const int hq = g * r + wave + 4 * u;
    const int64_t slot = ((int64_t)b * a.Hq + hq) * a.max_splits + split;
    if (lane == 0) {
      a.part_ml[2 * slot] = m[u];
      a.part_ml[2 * slot + 1] = lsum;
    }
    reinterpret_cast<float2*>(a.part_o + slot * kDecD)[lane] = make_float2(o0[u], o1[u]);
  }
}

__global__ __launch_bounds__(kDecD) void decode_combine_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int nkv = clampi(a.kv_lengths[b], 0, a.cap);
  const int nsp = (nkv + a.split_len - 1) / a.split_len;
  const int64_t slot0 = ((int64_t)b * a.Hq + hq) * a.max_splits;
  const float* ml = a.part_ml + 2 * slot0;
  const float* po = a.part_o + slot0 * kDecD + d;
  // four splits per round, so that the loads of a round are in flight together
  float M = -INFINITY;
  for (int s = 0; s < nsp; s += 4) {
    float t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = s + u < nsp ? ml[2 * (s + u)] : -INFINITY;
    M = fmaxf(M, fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
  }
  float L = 0.f, O = 0.f;
  for (int s = 0; s < nsp; s += 4) {
    float mm[4], ll[4], oo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = s + u < nsp;
      mm[u] = ok ? ml[2 * (s + u)] : -INFINITY;
      ll[u] = ok ? ml[2 * (s + u) + 1] : 0.f;
      oo[u] = ok ? po[(int64_t)(s + u) * kDecD] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = (s + u < nsp) ? __builtin_amdgcn_exp2f(mm[u] - M) : 0.f;
      L = fmaf(w, ll[u], L);
      O = fmaf(w, oo[u], O);
    }
  }
  const float res = (nsp > 0 && L > 0.f) ? O / L : NAN;
  store_elem(a.out, b * a.o_sb + hq * a.o_sh + d, a.out_dtype, res);
}

}  // namespace

bool decode_fast_supports(const DecodeArgs& a, int in_dtype) {
  if (in_dtype != SDPA_BF16 || a.D != kDecD) return false;
  const int r = a.Hq / a.Hkv;
  if (r > 8) return false;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  // 16-byte row loads: rows aligned, strides multiples of 8 elements; q rows 4-byte aligned
  if (!al16(a.k) || !al16(a.v)) return false;
  if ((a.k_sb | a.k_ss | a.k_sh | a.v_sb | a.v_ss | a.v_sh) & 7) return false;
  if ((reinterpret_cast<uintptr_t>(a.q) & 3) || ((a.q_sb | a.q_sh) & 1)) return false;
  return true;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int r = a.Hq / a.Hkv;
  dim3 grid(a.Hkv * a.max_splits, a.B);
  if (r <= 4) hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(kDecThreads), 0, s, a);
  else hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(kDecD), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdpa
