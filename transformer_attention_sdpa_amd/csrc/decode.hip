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
//   pass 1: one workgroup per (K/V head g, key split s, sequence b) scores every query head
//     that shares g (grouped-query attention) from the same K/V tiles and writes the split's
//     running max m, sum l and unnormalised output o in fp32. The online softmax is kept in
//     the exp2 domain (logits pre-multiplied by scale*log2 e).
//     - decode_split_mfma (head dim 128, 1024-key splits, up to 16 query heads per K/V head):
//       one wave streams 32-key tiles through a two-stage LDS ring filled by direct global ->
//       LDS loads and does q.k and p.V on the matrix cores (see that kernel). Its grid is
//       linear: all full splits first, then the partial ones, then idle workgroups (mf_locate).
//     - decode_split (the other bf16 shapes): 256 threads stream 64-key tiles through LDS with
//       16-byte loads, lane = key for q.k (bf16 dot2), lane = pair of head-dim elements for p.V.
//   pass 2 (decode_combine): per (query head, sequence), the splits merge by log-sum-exp:
//     M = max m_s, out = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s. This merge is exact because
//     the online softmax is associative (NNlib "Fused implementation": softmax taken online
//     over tiles of keys). No key at all gives NaN ("Fused implementation").
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
    const int64_t slot = ((int64_t)b * a.Hq + hq) * a.max_splits + split;   // one query token (T == 1)
    if (lane == 0) {
      a.part_ml[2 * slot] = m[u];
      a.part_ml[2 * slot + 1] = lsum;
    }
    reinterpret_cast<float2*>(a.part_o + slot * kDecD)[lane] = make_float2(o0[u], o1[u]);
  }
}

// ---- matrix-core variant of pass 1 --------------------------------------------------------
// One wave per (K/V head g, 1024-key split, sequence b). The split streams through LDS in
// 32-key tiles, filled by direct global -> LDS loads into a ring of two stages, so that one
// tile is in flight while the other is computed; there are no staging registers and no LDS
// stores. The 32 tiles of a split are unrolled into straight-line code: every stage is a
// distinct LDS array, which lets the compiler's wait-count tracking tell a read of one stage
// from a load in flight into another.
// Ring depth and split length were measured at the GQA decode workload once the loads carried
// the nontemporal policy (alternating builds, us per sdpa_decode call): 3 stages / 512 keys
// 237.8, 2 / 512 233.1, 4 / 512 247.0, 3 / 1024 235.5, 2 / 1024 229.9, 3 / 256 262.2, 2 / 768
// 233.8, 2 / 1536 240.3. Two stages of 16 KB let five waves share a CU's LDS instead of three.
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (or _f16): A = 16 keys x 32 head-dim values of K, B = Q^T with
//     the group's r query heads as columns (padded to 16 with zeros).
//   The 16x16 accumulator gives lane l the scores of keys 4*(l/16) + i (i = 0..3) of a 16-key
//     block for head l%16. For a 32-key chunk the lane's 8 probabilities, taken as the MFMA k
//     index 8*(l/16) + s (s < 4: block 0, s >= 4: block 1), are directly the B operand of
//     O^T += V^T P^T; the A operand V^T is read with ds_read_b64_tr_b16 for the same key order.
//   Softmax in the exp2 domain as in pass 1 above; row sums of the bf16 probabilities the
//     MFMA consumes.
constexpr int kMfTile = 32;                    // keys per tile
constexpr int kMfSplit = 1024;                 // keys per split (32 tiles)
constexpr int kMfTileElems = kMfTile * kDecD;  // 4096 bf16 = 8 KB

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void dec_lds_void;

// The 16-bit input type of the matrix-core pass 1: bf16 or IEEE f16 (MFMA and conversions).
template <bool F16> struct DecIn;
template <> struct DecIn<false> {
  typedef __bf16 x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  __device__ static f32x4_t mfma(x8 a, x8 b, f32x4_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
  __device__ static uint32_t pack(float a, float b) {
    const x2 p = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, p);
  }
  __device__ static float sum2(uint32_t p, float acc) {   // acc + both packed values
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(x2, p), __builtin_bit_cast(x2, 0x3f803f80u), acc, false);
  }
};
template <> struct DecIn<true> {
  typedef _Float16 x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  __device__ static f32x4_t mfma(x8 a, x8 b, f32x4_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
  __device__ static uint32_t pack(float a, float b) {
    const x2 p = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, p);
  }
  __device__ static float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(x2, p), __builtin_bit_cast(x2, 0x3c003c00u), acc, false);
  }
};

// One wave instruction of a direct load: lane l copies 16 bytes from byte offset voff of r into
// lds + 16*l. (Kept out of the kernel body: used there directly, the host pass drops the stub.)
// The cache rows are read exactly once per call, so the loads carry the nontemporal policy
// (kDecStream): on this GPU a streaming read with it sustains about 6.7 TB/s against about
// 6.0-6.3 TB/s without, and the split kernel went from 255 to 237 us at the GQA decode
// workload with identical results.
constexpr int kDecStream = 2;     // cache-policy operand of the buffer load: the NT bit
__device__ __forceinline__ void dec_dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (dec_lds_void*)lds, 16, voff, 0, 0, kDecStream);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dec_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
// 16-byte chunk positions of a 256-byte LDS row are XOR-swizzled: K fragment reads (16 rows,
// one chunk) and transposed V reads (8 rows, two chunks per 32 lanes) then hit distinct banks.
__device__ __forceinline__ int dec_kswz(int row) { return row & 15; }
__device__ __forceinline__ int dec_vswz(int row) { return 2 * (row & 7); }

// Per-lane state of one wave of the matrix-core pass 1. The loop-invariant offsets are set once;
// the softmax state and the output accumulators belong to the chunk being processed.
struct MfWave {
  int lane, col, grp;
  int kdo[8], vdo[8];          // direct-load byte offsets (K, V) of the lane's 8 slots per tile
  int vo_lo[8], vo_hi[8];      // element offsets of the two transposed V reads per 16-row block
  uint4 qf[4];                 // Q^T operand of the current (sequence, K/V head), 8 16-bit values each
  f32x4_t o[8];                // O^T accumulators, 16 head-dim rows each
  float m, lp0, lp1;           // running max (log2 units), two partial row sums
  bool cvalid;                 // this lane's column is a (query head, token) of the group
  int hq, tok;                 // its query head and token
  int jlim;                    // its keys end here (bottom-right causal), within the split
};

__device__ __forceinline__ void mf_init(MfWave& w, const DecodeArgs& a) {
  w.lane = threadIdx.x & 63;
  w.col = w.lane & 15;
  w.grp = w.lane >> 4;
  const int k_row_bytes = (int)(a.k_ss * 2), v_row_bytes = (int)(a.v_ss * 2);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int sl = 64 * u + w.lane, row = sl >> 4, pos = sl & 15;
    w.kdo[u] = row * k_row_bytes + ((pos ^ dec_kswz(row)) << 4);
    w.vdo[u] = row * v_row_bytes + ((pos ^ dec_vswz(row)) << 4);
  }
  const int vrow = 4 * w.grp + ((w.lane & 15) >> 2);
  const int vsw = dec_vswz(vrow);                   // rows vrow + 16 share it
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int c = 16 * db + 4 * (w.lane & 3);
    w.vo_lo[db] = vrow * kDecD + ((((c >> 3) ^ vsw) << 3) | (c & 7));
    w.vo_hi[db] = w.vo_lo[db] + 16 * kDecD;
    asm volatile("" : "+v"(w.vo_hi[db]));           // keeps each address one step from its buffer
  }
}

// Q^T (B operand) of sequence b, K/V head g, column group cg: the group's r*T (query head,
// token) pairs, token-minor, fill the 16 columns of each group; lane holds column col, head-dim
// 32*c + 8*grp + 0..7; columns past the pairs are zero. Query token t of a sequence with nkv
// keys attends keys below nkv - T + 1 + t (bottom-right causal); jlim is that limit cut to the
// split [.., j_end). Resets the chunk state.
__device__ __forceinline__ void mf_begin(MfWave& w, const DecodeArgs& a, int b, int g, int r, int cg, int nkv,
                                         int j_end) {
  const int pc = 16 * cg + w.col;
  w.cvalid = pc < r * a.T;
  const int hl = w.cvalid ? pc / a.T : 0;
  w.tok = w.cvalid ? pc - hl * a.T : 0;
  w.hq = g * r + hl;
  w.jlim = min(j_end, nkv - a.T + 1 + w.tok);
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_sb + (int64_t)w.tok * a.q_ss +
                       (int64_t)w.hq * a.q_sh;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 x = w.cvalid ? *reinterpret_cast<const uint4*>(qp + 32 * c + 8 * w.grp) : make_uint4(0, 0, 0, 0);
    w.qf[c] = x;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) w.o[db][e] = 0.f;
  w.m = -INFINITY;
  w.lp0 = 0.f;
  w.lp1 = 0.f;
}

// Direct loads of keys [j0, j0 + 32) of (b, g) into one ring stage; rows at or past j_end read 0.
__device__ __forceinline__ void mf_load(const MfWave& w, const DecodeArgs& a, int b, int g, int j0, int j_end,
                                        uint16_t* kd, uint16_t* vd) {
  const int64_t rows = (int64_t)j_end - j0;
  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + b * a.k_sb + g * a.k_sh + (int64_t)j0 * a.k_ss;
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + b * a.v_sb + g * a.v_sh + (int64_t)j0 * a.v_ss;
  const __amdgpu_buffer_rsrc_t rk = dec_rsrc(kb, rows * a.k_ss * 2);
  const __amdgpu_buffer_rsrc_t rv = dec_rsrc(vb, rows * a.v_ss * 2);
#pragma unroll
  for (int u = 0; u < 8; ++u) dec_dma16(rk, kd + 512 * u, w.kdo[u]);
#pragma unroll
  for (int u = 0; u < 8; ++u) dec_dma16(rv, vd + 512 * u, w.vdo[u]);
}

// One 32-key tile (keys j0.. of which those below j_end count) from a ring stage.
template <bool F16>
__device__ __forceinline__ void mf_tile(MfWave& w, const DecodeArgs& a, int j0, int j_end, const uint16_t* ks,
                                        const uint16_t* vs) {
  f32x4_t sc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[kb][e] = 0.f;
    const int row = 16 * kb + w.col;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      using x8 = typename DecIn<F16>::x8;
      const x8 ka = *reinterpret_cast<const x8*>(ks + row * kDecD + (((4 * c + w.grp) ^ dec_kswz(row)) << 3));
      sc[kb] = DecIn<F16>::mfma(ka, __builtin_bit_cast(x8, w.qf[c]), sc[kb]);
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 16 * kb + 4 * w.grp + i;
      const float x = j < w.jlim ? sc[kb][i] * a.scale_log2 : -INFINITY;
      sc[kb][i] = x;
      tmax = fmaxf(tmax, x);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  // a column may have no key in this tile yet (several tokens): its max stays -inf, and
  // m_use = 0 keeps alpha and the probabilities at 0 instead of NaN
  const float m_new = fmaxf(w.m, tmax);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(w.m - m_use);
  w.m = m_new;
  w.lp0 *= alpha;
  w.lp1 *= alpha;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) w.o[db][e] *= alpha;
  uint32_t pw[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    pw[2 * kb] = DecIn<F16>::pack(__builtin_amdgcn_exp2f(sc[kb][0] - m_use), __builtin_amdgcn_exp2f(sc[kb][1] - m_use));
    pw[2 * kb + 1] = DecIn<F16>::pack(__builtin_amdgcn_exp2f(sc[kb][2] - m_use), __builtin_amdgcn_exp2f(sc[kb][3] - m_use));
    w.lp0 = DecIn<F16>::sum2(pw[2 * kb], w.lp0);
    w.lp1 = DecIn<F16>::sum2(pw[2 * kb + 1], w.lp1);
  }
  using x8 = typename DecIn<F16>::x8;
  const x8 pb = __builtin_bit_cast(x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(vs + w.vo_lo[db]));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(vs + w.vo_hi[db]));
    const s16x8_t vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    w.o[db] = DecIn<F16>::mfma(__builtin_bit_cast(x8, vv), pb, w.o[db]);
  }
}

// Partials of one chunk: running max (log2 units), row sum, unnormalised output.
__device__ __forceinline__ void mf_store(const MfWave& w, const DecodeArgs& a, int b, int g, int r, int split) {
  float lsum = w.lp0 + w.lp1;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (!w.cvalid) return;
  const int64_t slot = (((int64_t)b * a.T + w.tok) * a.Hq + w.hq) * a.max_splits + split;
  if (w.grp == 0) {
    a.part_ml[2 * slot] = w.m;
    a.part_ml[2 * slot + 1] = lsum;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<float4*>(a.part_o + slot * kDecD + 16 * db + 4 * w.grp) =
        make_float4(w.o[db][0], w.o[db][1], w.o[db][2], w.o[db][3]);
}

constexpr int kMfTiles = kMfSplit / kMfTile;     // 16 tiles per chunk
// s_waitcnt immediate: lgkmcnt(0), vmcnt and expcnt not waited on
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

// Work order of the linear grid (batches up to kLinMaxB sequences): item i of K/V head g is
// workgroup Hkv*i + g; the items are the full splits of all sequences, sequence by sequence,
// then the partial last splits; workgroups past the last item exit at once. Compared with a
// (split, sequence) grid, the workgroups with nothing to do no longer hold slots in between the
// real ones (each keeps its LDS until it has read kv_lengths and left), and the shorter partial
// splits run last. Every lane reads the lengths of sequences lane, lane + 64, ... (all loads in
// flight together); a wave prefix sum of the split counts then locates the item.
constexpr int kLinMaxB = 256;

__device__ __forceinline__ bool mf_locate(const DecodeArgs& a, int item, int& b, int& split, int& nkv) {
  const int lane = threadIdx.x & 63;
  int len[kLinMaxB / 64];
#pragma unroll
  for (int c = 0; c < kLinMaxB / 64; ++c) {
    const int bb = 64 * c + lane;
    len[c] = bb < a.B ? clampi(a.kv_lengths[bb], 0, a.cap) : 0;
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {            // 0: full splits, 1: partial last splits
#pragma unroll
    for (int c = 0; c < kLinMaxB / 64; ++c) {
      const int cnt = pass == 0 ? len[c] / kMfSplit : (len[c] % kMfSplit != 0 ? 1 : 0);
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const int tot = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
      if (item < tot) {                             // scalar: a uniform branch
        const int l = __builtin_ctzll(__builtin_amdgcn_ballot_w64(incl > item));
        b = 64 * c + l;
        nkv = __shfl(len[c], l, 64);
        split = pass == 0 ? item - __shfl(incl - cnt, l, 64) : nkv / kMfSplit;
        return true;
      }
      item -= tot;
    }
  }
  return false;
}

// (query head, token) column groups of 16 per K/V head
__host__ __device__ __forceinline__ int mf_groups(const DecodeArgs& a) { return ((a.Hq / a.Hkv) * a.T + 15) / 16; }

// One workgroup (one wave) per (K/V head g, column group cg, split, sequence). The hardware
// deals consecutive workgroups round-robin over the 8 XCDs, so workgroup n runs on XCD n % 8;
// n is laid out so that each XCD takes all (head, group) pairs of one item back to back:
// hg = g + Hkv * cg = (n / 8) % HG and i = n % 8 + 8 * (n / (8 * HG)). The heads of one key
// range then leave one XCD close together, as whole 2 KB cache rows rather than 256-byte
// pieces at a 2 KB stride. LINEAR: i is an item of mf_locate; else i is the split and the
// sequence is blockIdx.y. Items past the end (the grid is padded to whole groups of 8) and
// splits past a sequence's length exit at once.
template <bool LINEAR, bool F16>
__global__ __launch_bounds__(64) void decode_split_mfma_kernel(DecodeArgs a) {
  __shared__ __align__(16) uint16_t k0s[kMfTileElems], k1s[kMfTileElems];
  __shared__ __align__(16) uint16_t v0s[kMfTileElems], v1s[kMfTileElems];
  const int r = a.Hq / a.Hkv;
  const int ng = mf_groups(a);
  const int HG = a.Hkv * ng;
  const int xk = blockIdx.x >> 3;
  const int hg = xk % HG;
  const int g = hg % a.Hkv, cg = hg / a.Hkv;
  const int item = (blockIdx.x & 7) + 8 * (xk / HG);
  int b, split, nkv;
  if constexpr (LINEAR) {
    if (!mf_locate(a, item, b, split, nkv)) return;
    b = __builtin_amdgcn_readfirstlane(b);
    split = __builtin_amdgcn_readfirstlane(split);
    nkv = __builtin_amdgcn_readfirstlane(nkv);
  } else {
    split = item;
    b = blockIdx.y;
    nkv = clampi(a.kv_lengths[b], 0, a.cap);
  }
  const int j_begin = split * kMfSplit;
  if (j_begin >= nkv) return;                       // wave-uniform
  const int j_end = min(j_begin + kMfSplit, nkv);
  MfWave w;
  mf_init(w, a);
  mf_begin(w, a, b, g, r, cg, nkv, j_end);
  uint16_t* const kst[2] = {k0s, k1s};
  uint16_t* const vst[2] = {v0s, v1s};
  mf_load(w, a, b, g, j_begin, j_end, kst[0], vst[0]);
#pragma unroll
  for (int t = 0; t < kMfTiles; ++t) {              // two stages: one tile in flight
    if (t + 1 < kMfTiles) {
      // the stage refilled here was read for tile t-1: those LDS reads must be complete before
      // the direct loads that overwrite it are issued (the compiler orders a direct load only
      // before later reads of its data, not after earlier reads of what it replaces)
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_sched_barrier(0);
      mf_load(w, a, b, g, j_begin + kMfTile * (t + 1), j_end, kst[(t + 1) % 2], vst[(t + 1) % 2]);
    }
    if (j_begin + kMfTile * t < j_end) mf_tile<F16>(w, a, j_begin + kMfTile * t, j_end, kst[t % 2], vst[t % 2]);
  }
  __builtin_amdgcn_s_waitcnt(0);                    // no direct load may land after the wave ends
  mf_store(w, a, b, g, r, split);
}

__global__ __launch_bounds__(kDecD) void decode_combine_kernel(DecodeArgs a) {
  const int hq = blockIdx.x % a.Hq, bt = blockIdx.x / a.Hq, d = threadIdx.x;   // bt = b * T + token
  const int b = bt / a.T, t = bt - b * a.T;
  const int nkv = clampi(a.kv_lengths[b], 0, a.cap);
  const int nsp = (nkv + a.split_len - 1) / a.split_len;
  const int64_t slot0 = ((int64_t)bt * a.Hq + hq) * a.max_splits;
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
  store_elem(a.out, b * a.o_sb + t * a.o_ss + hq * a.o_sh + d, a.out_dtype, res);
}

}  // namespace

// The matrix-core pass 1: 1024-key splits, up to 16 query tokens and 8 column groups, 16-byte
// aligned query rows (the K/V conditions of decode_fast_supports hold as well).
constexpr int kMfMaxT = 16, kMfMaxGroups = 8;
static bool decode_mfma_supports(const DecodeArgs& a) {
  if (a.split_len != kMfSplit || a.T < 1 || a.T > kMfMaxT || mf_groups(a) > kMfMaxGroups) return false;
  if ((reinterpret_cast<uintptr_t>(a.q) & 15) || ((a.q_sb | a.q_ss | a.q_sh) & 7)) return false;
  // byte offsets of 32 rows and the 32-bit buffer ranges
  if ((int64_t)kMfTile * a.k_ss * 2 > INT32_MAX || (int64_t)kMfTile * a.v_ss * 2 > INT32_MAX) return false;
  return true;
}

bool decode_fast_supports(const DecodeArgs& a, int in_dtype) {
  if ((in_dtype != SDPA_BF16 && in_dtype != SDPA_F16) || a.D != kDecD || a.in_dtype != in_dtype) return false;
  // grid limits: sequences in grid.y of the (split, sequence) grids, one combine workgroup per
  // (query head, sequence, token)
  if (a.B > 65535 || (int64_t)a.Hq * a.B * a.T > INT32_MAX) return false;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  // 16-byte row loads: rows aligned, strides multiples of 8 elements
  if (!al16(a.k) || !al16(a.v)) return false;
  if ((a.k_sb | a.k_ss | a.k_sh | a.v_sb | a.v_ss | a.v_sh) & 7) return false;
  if (decode_mfma_supports(a)) return true;
  // the vector pass 1: bf16, one query token, up to 8 query heads per K/V head, 4-byte aligned q rows
  if (in_dtype != SDPA_BF16 || a.T != 1 || a.Hq / a.Hkv > 8) return false;
  if ((reinterpret_cast<uintptr_t>(a.q) & 3) || ((a.q_sb | a.q_sh) & 1)) return false;
  return true;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int r = a.Hq / a.Hkv;
  dim3 grid(a.Hkv * a.max_splits, a.B);
  if (decode_mfma_supports(a)) {
    // grids padded to whole groups of 8 items per (head, group) pair (see the kernel)
    const int64_t hg = (int64_t)a.Hkv * mf_groups(a);
    const int64_t per_seq = hg * a.max_splits;
    const bool lin = a.B <= kLinMaxB && (per_seq * a.B + 8 * hg) <= INT32_MAX;
    const int64_t n_lin = hg * 8 * (((int64_t)a.max_splits * a.B + 7) / 8);
    const int64_t n_2d = hg * 8 * (((int64_t)a.max_splits + 7) / 8);
    const dim3 g1((unsigned)n_lin), g2((unsigned)n_2d, a.B);
    if (a.in_dtype == SDPA_F16) {
      if (lin) hipLaunchKernelGGL((decode_split_mfma_kernel<true, true>), g1, dim3(64), 0, s, a);
      else hipLaunchKernelGGL((decode_split_mfma_kernel<false, true>), g2, dim3(64), 0, s, a);
    } else {
      if (lin) hipLaunchKernelGGL((decode_split_mfma_kernel<true, false>), g1, dim3(64), 0, s, a);
      else hipLaunchKernelGGL((decode_split_mfma_kernel<false, false>), g2, dim3(64), 0, s, a);
    }
  }
  else if (r <= 4) hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(kDecThreads), 0, s, a);
  else hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((int64_t)a.Hq * a.B * a.T)), dim3(kDecD), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdpa
