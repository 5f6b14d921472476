// bwd_mfma.hip -- the dK/dV and dQ passes of the attention gradient on the gfx950 matrix cores
// (bf16 or f16 inputs, head dims 64 and 128, no bias, scale > 0; page "Neural Network primitives
// from NNlib.jl", section "Fused implementation": the weights are formed again tile by tile from
// q, k and the saved log-sum-exp, never stored). A boolean mask comes as U8 bytes, U1 bits or
// block info (the block-sparse scheme of the splash-attention pull request "Support dynamic
// masks in splash attention #25213"); each step's mask tile is staged in LDS next to the
// streamed tiles, and with block info only the steps that meet a non-empty block are visited.
//
// Both passes use v_mfma_f32_32x32x16 with one operand kept in registers for the whole loop
// and the other streamed through LDS, and they are mirror images of each other:
//
// * dK/dV: a workgroup of 8 waves owns 128 keys of one K/V head; K and V sit in LDS for the
//   whole kernel and are read as B operands. Waves w and w + 4 own the same 32 keys and take
//   the two 32-query blocks of each 64-query tile streamed from every query head of the group,
//   so each wave holds only its own accumulators and two waves share every SIMD. Per block a
//   wave forms S = Q K^T - lse/scale and dP = dO V^T - D, the row statistics being the MFMAs'
//   starting values. Its lanes then hold one key column each, with 16 consecutive queries per
//   lane half, because the A-operand rows of Q and dO are read in the permuted order perm32.
//   Next P = exp2(scale * log2 e * S) and dS = P dP. Finally P and dS are packed to 16 bits and
//   feed dV^T += dO^T P and dK^T += Q^T dS directly as B operands; dO^T and Q^T come from
//   transposed LDS reads (ds_read_b64_tr_b16). The two waves of a key block add their sums
//   through LDS at the end.
// * dQ: a workgroup owns 128 queries of one head (Q and dO in registers) and streams tiles of 64
//   keys. S^T = K Q^T and dP^T = V dO^T leave each lane one query column and 16 consecutive
//   keys per lane half; dS^T feeds dQ^T += K^T dS^T, with K^T read transposed. The lane also
//   sums dS * <q, k> for its row's share of dscale.
//
// Tiles sit in LDS row-major and unpermuted, 16-byte chunks XOR-swizzled by bswz so that both
// read patterns are free of bank conflicts: the permuted A-operand reads (rows perm32(0..15) of
// one chunk) and the transposed reads (4 consecutive rows x 64 bytes). Rows past the arrays
// arrive as zeros (buffer range checks); rows that take no part carry lse = +inf, so all their
// weights are 0; keys past kv_lengths, past the causal limit and masked out are set to weight
// 0 per element. No atomics: each workgroup writes its own rows.
#include <type_traits>

#include "mfma_common.h"

namespace sdpa {

namespace {

constexpr int NTB = 256;          // threads per workgroup (4 waves)
constexpr int RB = 128;           // rows a workgroup owns: keys (dK/dV) or queries (dQ)
constexpr int ST = 64;            // keys per streamed tile of the dQ pass

// MFMA row r of a 32-row A operand reads tile row perm32(r): accumulator entry 4*i + j of lane
// half h (MFMA row 8*i + 4*h + j) then belongs to tile row 16*h + 4*i + j.
__device__ __forceinline__ int perm32(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// Chunk swizzle of tile row `row` (chunk = 16 bytes): logical chunk c sits at position
// c ^ bswz(row). Bits 0-1 separate the rows perm32 reads together; bits 2-3 (D = 128) or bit
// 2 with the row's 128-byte half (D = 64) separate 4 consecutive rows for transposed reads.
template <int D>
__device__ __forceinline__ int bswz(int row) {
  const int f = ((row >> 2) & 1) | (((row >> 4) & 1) << 1);
  return D == 128 ? (((row & 3) << 2) | f) : ((((row >> 1) & 1) << 2) | f);
}

// Tile loader and readers for ST x D tiles of 16-bit elements in LDS.
template <int D, bool F16, int ST, int NTH = NTB>
struct Tiles {
  using x8 = typename In<F16>::x8;
  static constexpr int CPR = D / 8;                 // chunks per row
  static constexpr int SPT = ST * CPR / NTH;        // direct-load instructions per thread
  static constexpr int DB = D / 32;
  int doff[SPT];                                    // per-thread source offsets (row bytes applied)
  int nrow, nsw;                                    // permuted A-operand row of this lane, its swizzle
  int toff_lo[DB], toff_hi[DB];                     // transposed-read offsets (elements)

  __device__ void init(int row_bytes, int lane, int tid) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int sl = NTH * u + tid, row = sl / CPR, pos = sl % CPR;
      doff[u] = row * row_bytes + (pos ^ bswz<D>(row)) * 16;
    }
    nrow = perm32(lane & 31);
    nsw = bswz<D>(nrow);
    const int vr = 16 * (lane >> 5) + ((lane & 15) >> 2);
    const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const int col = 32 * d + vc;
      toff_lo[d] = vr * D + ((((col >> 3) ^ bswz<D>(vr)) << 3) | (col & 7));
      toff_hi[d] = (vr + 4) * D + ((((col >> 3) ^ bswz<D>(vr + 4)) << 3) | (col & 7));
      asm volatile("" : "+v"(toff_hi[d]));
    }
  }
  // rows [r0, r0 + ST) of the slice at `base` (row stride row_bytes), rows from `valid` on as zeros
  __device__ void load(const uint16_t* base, int64_t row_elems, int r0, int valid, int row_bytes,
                       uint16_t* dst, int wave) const {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)r0 * row_elems, (int64_t)(valid - r0) * row_bytes);
#pragma unroll
    for (int u = 0; u < SPT; ++u) dma16(r, dst + 8 * (NTH * u + 64 * wave), doff[u]);
  }
  // the same through a resource `r` over the whole slice (rows past its end read zeros), row r0
  // at byte r0_bytes of it (the caller keeps every offset within 32 bits)
  __device__ void load_at(__amdgpu_buffer_rsrc_t r, int r0_bytes, uint16_t* dst, int wave) const {
#pragma unroll
    for (int u = 0; u < SPT; ++u) dma16(r, dst + 8 * (NTH * u + 64 * wave), doff[u] + r0_bytes);
  }
  // A operand: 32-row block rb, head-dim chunk c (16 elements), rows in perm32 order
  __device__ x8 arow(const uint16_t* t, int rb, int c, int hh) const {
    const int row = 32 * rb + nrow;
    return *reinterpret_cast<const x8*>(t + row * D + (((2 * c + hh) ^ nsw) << 3));
  }
  // A operand, transposed: lane L gets tile[32*rb + 16*(L/32) + 8*sh + t][32*d + L%32], t = 0..7
  __device__ x8 atr(const uint16_t* t, int rb, int sh, int d) const {
    const int rows = (32 * rb + 8 * sh) * D;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(t + (rows + toff_lo[d])));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(t + (rows + toff_hi[d])));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(x8, v);
  }
};

// Workgroup n of a launch over n_t row tiles x HB (batch, head) slices -> (tile rank, slice).
// Rank-major, so that the heaviest tiles of every slice run first; with remap every XCD (the
// hardware deals workgroups round-robin over 8) gets a contiguous set of slices.
__device__ __forceinline__ void wg_map(int n, int HB, int remap, int& rank, int& slice) {
  if (remap) {
    const int per_x = HB >> 3, k = n >> 3;
    rank = k / per_x;
    slice = (n & 7) * per_x + k % per_x;
  } else {
    rank = n / HB;
    slice = n % HB;
  }
}

// 16-bit B operand from 8 fp32 values
template <bool F16>
__device__ __forceinline__ typename In<F16>::x8 pack8(const float* x) {
  using E = In<F16>;
  const uint4 u = make_uint4(E::pack(x[0], x[1]), E::pack(x[2], x[3]), E::pack(x[4], x[5]), E::pack(x[6], x[7]));
  return __builtin_bit_cast(typename E::x8, u);
}

// Four consecutive outputs (fp32, bf16 or f16) at element offset `off`
__device__ __forceinline__ void store4(void* base, int64_t off, int dtype, float r0, float r1, float r2, float r3) {
  if (dtype == SDPA_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = make_float4(r0, r1, r2, r3);
  } else if (dtype == SDPA_F16) {
    const uint32_t w0 = (uint32_t)float_to_f16_bits(r0) | ((uint32_t)float_to_f16_bits(r1) << 16);
    const uint32_t w1 = (uint32_t)float_to_f16_bits(r2) | ((uint32_t)float_to_f16_bits(r3) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) = make_uint2(w0, w1);
  } else {
    const uint32_t w0 = (uint32_t)float_to_bf16_bits(r0) | ((uint32_t)float_to_bf16_bits(r1) << 16);
    const uint32_t w1 = (uint32_t)float_to_bf16_bits(r2) | ((uint32_t)float_to_bf16_bits(r3) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) = make_uint2(w0, w1);
  }
}

// Masked variants: the mask tile of each step travels to LDS with the K/V or Q/dO tiles
// (direct loads, no registers held across the step). U8: one byte per key; U1: 32 keys a word.
constexpr int MK_NONE = 0, MK_U8 = 1, MK_U1 = 2, MK_BI = 3;

// cache-policy operand of a buffer access: the NT (streaming) bit
constexpr int kStreamPolicy = 2;
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);
// vmcnt(n) lgkmcnt(0), n < 64
constexpr int vm_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

// Buffer resource over the mask rows of (b, h): loads past its last row read 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mask_rsrc(const AttnArgs& a, int b, int h) {
  const int64_t eb = a.mask_u1 ? 4 : 1;
  const int64_t row_bytes = a.mask_u1 ? (int64_t)((a.Lkv + 31) / 32) * 4 : a.Lkv;
  const uint8_t* base = a.mask + (b * a.mask_sb + h * a.mask_sh) * eb;
  return make_rsrc(base, (int64_t)(a.Lq - 1) * a.mask_sq * eb + row_bytes);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}
// Block info (MK_BI): each of 256 threads owns one 32-key word of every step's mask tile, laid
// out in LDS as U1 words. The class and partial index of the word's block are loaded two steps
// ahead (bi_fetch), turned into the word's source one step ahead (bi_source: a byte offset into
// the partial bits, -1 for an empty block, -2 for a full one), and the word arrives by a direct
// 4-byte load; empty and full blocks load from past the end of the range, which writes 0, and a
// full block's word is set to all ones once the step's loads have landed. No load result is
// used before the step's own wait, so the tile prefetch is never stalled.
constexpr int kBiNone = 0x7ffffff0;               // past every partial-bits range (at most 2^30 bytes)
__device__ __forceinline__ void bi_fetch(const AttnArgs& a, int b, int h, int i, int j, int& cls, int& nxt) {
  cls = 0;
  nxt = 0;
  if (i < a.Lq && j < a.Lkv) {
    const int mb = a.bm_batch > 1 ? b : 0, mh = a.bm_heads > 1 ? h : 0;
    const int64_t blk = (((int64_t)mb * a.bm_heads + mh) * a.bm_nqb + i / a.bm_bq) * a.bm_nkb + j / a.bm_bkv;
    cls = a.bm_class[blk];
    nxt = a.bm_next[blk];
  }
}
__device__ __forceinline__ int bi_source(const AttnArgs& a, int cls, int nxt, int i, int j) {
  if (cls == 1) {
    const int r = i % a.bm_bq, c = j % a.bm_bkv;
    return (int)((((int64_t)nxt * a.bm_bq + r) * (a.bm_bkv >> 5) + (c >> 5)) * 4);
  }
  return cls == 2 ? -2 : -1;
}
// Block info: some block meeting rows [i0, i1) x keys [j0, j1) of head h is not empty.
// Rectangles of more than 16 blocks count as live without a look.
__device__ __forceinline__ bool bi_rect_live(const AttnArgs& a, int b, int h, int i0, int i1, int j0, int j1) {
  i1 = min(i1, a.Lq);
  j1 = min(j1, a.Lkv);
  if (i0 >= i1 || j0 >= j1) return false;
  const int qb0 = i0 / a.bm_bq, qb1 = (i1 - 1) / a.bm_bq, kb0 = j0 / a.bm_bkv, kb1 = (j1 - 1) / a.bm_bkv;
  if ((qb1 - qb0 + 1) * (kb1 - kb0 + 1) > 16) return true;
  const int mb = a.bm_batch > 1 ? b : 0, mh = a.bm_heads > 1 ? h : 0;
  const int64_t base = ((int64_t)mb * a.bm_heads + mh) * a.bm_nqb;
  for (int qb = qb0; qb <= qb1; ++qb)
    for (int kb = kb0; kb <= kb1; ++kb)
      if (a.bm_class[(base + qb) * a.bm_nkb + kb] != 0) return true;
  return false;
}
// Steps a workgroup can skip through its LDS bitmask of live steps (more: every step is visited)
constexpr int kLiveWords = 128;

__host__ __device__ __forceinline__ int64_t bi_bits_bytes(const AttnArgs& a) {
  return (int64_t)a.bm_batch * a.bm_heads * a.bm_nqb * a.bm_nkb * a.bm_bq * (a.bm_bkv / 32) * 4;
}

// 4 mask bytes to 4 bits (bit t: byte t nonzero). The high bit of ((x & 0x7f7f7f7f) + 0x7f7f7f7f)
// | x is set exactly in the nonzero bytes (no byte's sum carries into the next); the multiply
// moves the four flags, bits 7, 15, 23 and 31, to bits 28 .. 31 without overlapping carries.
__device__ __forceinline__ uint32_t nonzero_nibble4(uint32_t x) {
  const uint32_t hi = (((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;
  return (hi * 0x00204081u) >> 28;
}

// weight argument x where bit e of the 16-bit set `valid` is set, else -inf (a bit select)
__device__ __forceinline__ float keep_or_ninf(uint32_t valid, int e, float x) {
  const uint32_t keep = (uint32_t)((int32_t)(valid << (31 - e)) >> 31);
  return __uint_as_float((__float_as_uint(x) & keep) | (0xff800000u & ~keep));
}

// Byte offset, within a stored dS tile, of the 8 queries 8 * c .. + 7 (c = 0 .. 7) of key row
// r (0 .. 127): written by lane 32 * ((c >> 1) & 1) + r % 32 of the dK/dV wave owning keys
// 32 * (r / 32) .. and queries 32 * (c >> 2) .., as its operand sB[c & 1]
__device__ __forceinline__ int ds_offset(int r, int c) {
  return ((4 * (r >> 5) + 2 * (c >> 2) + (c & 1)) << 10) + ((((c >> 1) & 1) << 5) + (r & 31)) * 16;
}

// ================================ dK / dV ====================================================
// Eight waves: waves w and w + 4 own the same 32 keys and take the two 32-query blocks of each
// 64-query tile, so each holds only its accumulators and the S/dP pair, and two waves share
// every SIMD. K and V stay in LDS for the whole kernel (rows swizzled by kvswz for the B-operand
// reads, 16 consecutive rows per read). At the end the two waves of a key block add their
// partial dK/dV through LDS.
constexpr int NT8 = 512;
constexpr int QT8 = 64;

// chunk swizzle of the K/V rows read as B operands (16 consecutive rows, one chunk each)
template <int D>
__device__ __forceinline__ int kvswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }

// Quotient by a workgroup-invariant divisor 1 <= d < 2^31 for dividends below 2^31, by one
// multiply-high: the round-up method of Granlund and Montgomery ("Division by invariant integers
// using multiplication", 1994), with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1 and
// q = (t + ((n - t) >> 1)) >> (l - 1), t = mulhi(m, n); d = 1 is n itself.
struct DivU {
  uint32_t m;
  int l;
  __device__ void init(uint32_t d) {
    l = 0;
    while ((1u << l) < d) ++l;
    m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  }
  __device__ uint32_t div(uint32_t n) const {
    if (l == 0) return n;
    const uint32_t t = __umulhi(m, n);
    return (t + ((n - t) >> 1)) >> (l - 1);
  }
};

template <int D, bool F16, int MK, bool DS>
__global__ __launch_bounds__(NT8, 1) void bwd_dkdv8_kernel(BwdArgs g, int remap) {
  using E = In<F16>;
  using x8 = typename E::x8;
  constexpr int DC = D / 16, DB = D / 32, CPR = D / 8, TILE = QT8 * D;
  constexpr int KVSPT = RB * CPR / NT8;              // direct loads per thread for K (and V)
  __shared__ __align__(16) uint16_t kbuf[RB * D], vbuf[RB * D];
  __shared__ __align__(16) uint16_t qbuf0[TILE], qbuf1[TILE], obuf0[TILE], obuf1[TILE];
  // row statistics [-lse / scale, -D][query], one array per buffer: as one array, a read of one
  // buffer waited for the direct load in flight into the other at the start of every step
  __shared__ __align__(16) float stat0[2][QT8], stat1[2][QT8];
  // mask tile [buffer][query][key]: U8 128 bytes a query, U1 4 words a query
  __shared__ __align__(16) uint8_t mraw[MK ? 2 : 1][MK == MK_U8 ? QT8 * RB : QT8 * 16];
  __shared__ uint64_t live_bits[MK == MK_BI ? kLiveWords : 1];   // block info: bit s, step s is not empty
  const AttnArgs& a = g.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3, qp = wave >> 2;           // key block, query block of each tile
  const int ql = lane & 31, hh = lane >> 5;

  int kt, bg;
  wg_map(blockIdx.x, a.Hkv * a.B, remap, kt, bg);
  const int gk = bg % a.Hkv, b = bg / a.Hkv;
  const int grp = a.Hq / a.Hkv;
  const int k0 = kt * RB, wk0 = k0 + 32 * kw, key_me = wk0 + ql;
  const int nkv = batch_kv_len(a, b), nq = batch_q_len(a, b);
  const int64_t off = batch_causal_offset(a, b);
  const bool causal = a.causal != SDPA_CAUSAL_NONE;
  const float c2 = a.scale * LOG2E;

  int64_t i_lo = causal ? (int64_t)k0 - off : 0;
  i_lo = i_lo < 0 ? 0 : i_lo;
  const int n_qt = (nq + QT8 - 1) / QT8;
  const int qt0 = (k0 < nkv && i_lo < nq) ? (int)(i_lo / QT8) : n_qt;
  const int per_head = n_qt - qt0;
  const int n_it = per_head * grp;
  const int64_t wi_lo = causal ? (int64_t)wk0 - off : INT64_MIN / 2;
  const bool wave_live = wk0 < nkv;

  // K and V of the workgroup's 128 keys into LDS once (keys past kv_lengths as zeros)
  {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + gk * a.k_sh + (int64_t)k0 * a.k_ss;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + gk * a.v_sh + (int64_t)k0 * a.v_ss;
    const int kbytes = (int)(a.k_ss * 2), vbytes = (int)(a.v_ss * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp, (int64_t)(nkv - k0) * kbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp, (int64_t)(nkv - k0) * vbytes);
#pragma unroll
    for (int u = 0; u < KVSPT; ++u) {
      const int sl = NT8 * u + tid, row = sl / CPR, pos = sl % CPR;
      const int c = pos ^ kvswz<D>(row);
      dma16(rk, kbuf + 8 * (NT8 * u + 64 * wave), row * kbytes + c * 16);
      dma16(rv, vbuf + 8 * (NT8 * u + 64 * wave), row * vbytes + c * 16);
    }
  }
  // B operand from the K or V rows of this wave's keys: key column ql, head-dim chunk c
  const int kvrow = 32 * kw + ql, kvsw = kvswz<D>(kvrow);
  auto bkv = [&](const uint16_t* t, int c) -> x8 {
    return *reinterpret_cast<const x8*>(t + kvrow * D + (((2 * c + hh) ^ kvsw) << 3));
  };

  Tiles<D, F16, QT8, NT8> tq, to;
  tq.init((int)(a.q_ss * 2), lane, tid);
  to.init((int)(g.do_ss * 2), lane, tid);
  // step it = (head - gk * grp) * per_head + (query tile - qt0); the quotient by one multiply
  // (a runtime division costs some thirty scalar instructions, several times a step)
  DivU dph;
  dph.init(per_head > 0 ? per_head : 1);
  auto it_head = [&](int it) { return gk * grp + (int)dph.div((uint32_t)it); };
  auto it_q0 = [&](int it) { return (qt0 + it - (int)dph.div((uint32_t)it) * per_head) * QT8; };
  // buffer resources over one query head's Q and dO rows and its row statistics; with one
  // query head per K/V head (grp == 1) the workgroup's resources never change, else a step
  // builds those of its head. A step's first row enters the per-lane offsets (the host keeps
  // Lq + 64 rows within 32-bit offsets).
  auto q_rs = [&](int h) {
    return make_rsrc(static_cast<const uint16_t*>(a.q) + b * a.q_sb + (int64_t)h * a.q_sh, (int64_t)a.Lq * a.q_ss * 2);
  };
  auto o_rs = [&](int h) {
    return make_rsrc(static_cast<const uint16_t*>(g.dout) + b * g.do_sb + (int64_t)h * g.do_sh,
                     (int64_t)a.Lq * g.do_ss * 2);
  };
  auto st_rs = [&](int h) {
    return make_rsrc((wave == 0 ? g.w_lse : g.w_dsum) + ((int64_t)b * a.Hq + h) * a.Lq, (int64_t)a.Lq * 4);
  };
  const __amdgpu_buffer_rsrc_t rq0 = q_rs(gk * grp), ro0 = o_rs(gk * grp), rs0 = st_rs(gk * grp);
  const int q_row_bytes = (int)(a.q_ss * 2), o_row_bytes = (int)(g.do_ss * 2);
  auto load_tiles = [&](int it, uint16_t* qd, uint16_t* od) {
    const int h = it_head(it), i0 = it_q0(it);
    tq.load_at(grp == 1 ? rq0 : q_rs(h), i0 * q_row_bytes, qd, wave);
    to.load_at(grp == 1 ? ro0 : o_rs(h), i0 * o_row_bytes, od, wave);
  };
  // statistics of the step's queries into buffer buf by direct loads, like the tiles: wave 0
  // -lse / scale of queries it_q0 .. + 63, wave 1 their -D, the start values of S and dP as the
  // prep pass wrote them for this route (-inf and 0 for rows that take no part); rows past Lq
  // read 0 (buffer range), harmless there since their Q and dO tiles are zeros too. (Loaded into registers instead, the values made the compiler wait for every
  // load in flight where the branches on the thread index met, or spill.)
  auto dma_stat = [&](int it, int buf) {
    if (wave < 2) {
      float* dst = buf ? &stat1[wave][0] : &stat0[wave][0];
      dma4(grp == 1 ? rs0 : st_rs(it_head(it)), reinterpret_cast<uint32_t*>(dst), (lane + it_q0(it)) * 4);
    }
  };
  // mask rows of step it (queries it_q0 .. + 63, keys k0 .. k0 + 127) into mraw[buf]
  auto load_mask = [&](int it, int buf) {
    if constexpr (MK == MK_U8 || MK == MK_U1) {
      const __amdgpu_buffer_rsrc_t rm = mask_rsrc(a, b, it_head(it));
      const int64_t i0 = it_q0(it);
      if constexpr (MK == MK_U8) {                   // 16 bytes a thread: row 8 * wave + lane / 8
        const int64_t i = i0 + 8 * wave + (lane >> 3);
        dma16(rm, reinterpret_cast<uint16_t*>(mraw[buf] + 1024 * wave), (int)(i * a.mask_sq) + k0 + 16 * (lane & 7));
      } else if (wave == 0) {                        // 4 words a lane: row lane
        dma16(rm, reinterpret_cast<uint16_t*>(mraw[buf]), (int)(((i0 + lane) * a.mask_sq + (k0 >> 5)) * 4));
      }
    }
  };

  // block info: thread t < 256 owns word t % 4 of query row t / 4 of each step
  int bi_cls = 0, bi_nxt = 0, bi_src = -1;
  auto bi_load_raw = [&](int it) {
    if constexpr (MK == MK_BI) {
      if (tid < 256 && it < n_it) bi_fetch(a, b, it_head(it), it_q0(it) + (tid >> 2), k0 + 32 * (tid & 3), bi_cls, bi_nxt);
    }
  };
  auto bi_advance = [&](int it) {
    if constexpr (MK == MK_BI) {
      if (tid < 256) bi_src = bi_source(a, bi_cls, bi_nxt, it_q0(it) + (tid >> 2), k0 + 32 * (tid & 3));
    }
  };
  auto bi_dma = [&](int buf) {
    if constexpr (MK == MK_BI) {
      if (tid < 256) dma4(make_rsrc(a.bm_bits, bi_bits_bytes(a)), mraw[buf] + 256 * wave, bi_src >= 0 ? bi_src : kBiNone);
    }
  };
  auto bi_fix = [&](int buf) {
    if constexpr (MK == MK_BI) {
      if (tid < 256 && bi_src == -2) reinterpret_cast<uint32_t*>(mraw[buf])[tid] = 0xffffffffu;
    }
  };
  // block info: the steps that meet a non-empty block, found before the loop, and the loop
  // visits only those (the others would add exact zeros); other masks: every step
  bool scan = false;
  if constexpr (MK == MK_BI) {
    scan = n_it <= kLiveWords * 64;
    if (scan) {
      for (int s0 = 64 * wave; s0 < n_it; s0 += 64 * (NT8 / 64)) {
        const int st = s0 + lane;
        const bool lv = st < n_it && bi_rect_live(a, b, it_head(st), it_q0(st), it_q0(st) + QT8, k0, k0 + RB);
        const uint64_t m = __builtin_amdgcn_ballot_w64(lv);
        if (lane == 0) live_bits[s0 >> 6] = m;
      }
      __syncthreads();
    }
  }
  auto next_step = [&](int st) -> int {     // the first visited step after st, or n_it
    if constexpr (MK == MK_BI) {
      if (scan) {
        for (++st; st < n_it; st = (st | 63) + 1) {
          const uint64_t m = live_bits[st >> 6] >> (st & 63);
          if (m) return st + (int)__builtin_ctzll(m);
        }
        return n_it;
      }
    }
    return min(st + 1, n_it);
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[d][e] = dv[d][e] = 0.f;

  // stored-dS route: the step's dS tile (128 keys x 64 queries of one head, 16 KiB) goes to HBM
  // for the dQ pass, each store instruction of a wave writing 1 KiB in lane order: KiB
  // 4 * kw + 2 * qp + e holds, at 16 * lane, the entries of the lane's packed operand sB[e],
  // dS of key 32 * kw + ql and queries 32 * qp + 16 * hh + 8 * e .. + 7 (ds_offset). A wave that
  // skips its block (all weights 0) stores nothing: the dQ pass skips that block by the same test.
  const int ds_voff = (4 * kw + 2 * qp) * 1024 + 16 * lane;
  auto ds_store = [&](int it, x8 lo, x8 hi) {
    if constexpr (DS) {
      const int64_t tile = (((int64_t)b * a.Hq + it_head(it)) * ((a.Lq + QT8 - 1) / QT8) + it_q0(it) / QT8) *
                               ((a.Lkv + RB - 1) / RB) + kt;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(g.w_ds + tile * (RB * QT8), RB * QT8 * 2);
      // streaming stores (cache policy NT): the dQ pass reads them back only after this pass
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), r, ds_voff, 0, kStreamPolicy);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), r, ds_voff + 1024, 0, kStreamPolicy);
    }
  };

  const int first = next_step(-1), second = next_step(first);
  if (first < n_it) {
    dma_stat(first, 0);
    load_tiles(first, qbuf0, obuf0);
    load_mask(first, 0);
    if constexpr (MK == MK_BI) {
      bi_load_raw(first);
      __builtin_amdgcn_s_waitcnt(0);
      bi_advance(first);
      bi_dma(0);
      bi_load_raw(second);
    }
    __builtin_amdgcn_s_waitcnt(0);
    bi_fix(0);
    bi_advance(second);
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();

  // step it in buffer P; nx: the next visited step (prefetched here), nn: the one after it
  auto iter = [&](auto PAR_, int it, int nx, int nn) {
    constexpr int P = decltype(PAR_)::value;
    const uint16_t* qs = P ? qbuf1 : qbuf0;
    const uint16_t* os = P ? obuf1 : obuf0;
    if (nx < n_it) {
      dma_stat(nx, 1 - P);
      load_tiles(nx, P ? qbuf0 : qbuf1, P ? obuf0 : obuf1);
      load_mask(nx, 1 - P);
      bi_dma(1 - P);
      bi_load_raw(nn);
    }
    const int i0 = it_q0(it);
    // this wave's block: queries i0 + 32 * qp .. + 31 against keys wk0 .. wk0 + 31
    if (wave_live && (int64_t)i0 + 32 * qp + 31 >= wi_lo) {
      // entries below e_min: before this key's causal limit (or the key lies past kv_lengths)
      auto entry_min = [&]() {
        int em = 0;
        if (causal) {
          const int64_t m = (int64_t)key_me - off - (i0 + 32 * qp + 16 * hh);
          em = m < 0 ? 0 : (m > 16 ? 16 : (int)m);
        }
        return key_me >= nkv ? 16 : em;
      };
      const float* st = P ? &stat1[0][0] : &stat0[0][0];
      f32x16 s, dp;
      const float4* ls = reinterpret_cast<const float4*>(st + 32 * qp + 16 * hh);
      const float4* ds = reinterpret_cast<const float4*>(st + QT8 + 32 * qp + 16 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 l4 = ls[i], d4 = ds[i];
        s[4 * i] = l4.x; s[4 * i + 1] = l4.y; s[4 * i + 2] = l4.z; s[4 * i + 3] = l4.w;
        dp[4 * i] = d4.x; dp[4 * i + 1] = d4.y; dp[4 * i + 2] = d4.z; dp[4 * i + 3] = d4.w;
      }
      if constexpr (MK == MK_NONE) {
        // without a mask the limits enter as -inf start values (the products keep -inf, so the
        // weight is 0), and only in blocks that some lane does not keep whole (wave-uniform;
        // most blocks of a causal call are kept whole)
        const int e_min = entry_min();
        if (__builtin_amdgcn_ballot_w64(e_min != 0)) {
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] = e >= e_min ? s[e] : -INFINITY;
        }
      }
      if constexpr (MK == MK_NONE) {
        // the four operands of head-dim chunk c + 1 are read while chunk c's two products run
        // (the masked variants' extra registers would spill)
        x8 fa[2][4];
        auto rd = [&](int c, int buf) {
          fa[buf][0] = tq.arow(qs, qp, c, hh);
          fa[buf][1] = bkv(kbuf, c);
          fa[buf][2] = to.arow(os, qp, c, hh);
          fa[buf][3] = bkv(vbuf, c);
        };
        rd(0, 0);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          if (c + 1 < DC) rd(c + 1, (c + 1) & 1);
          s = E::mfma(fa[c & 1][0], fa[c & 1][1], s);
          dp = E::mfma(fa[c & 1][2], fa[c & 1][3], dp);
          __builtin_amdgcn_sched_barrier(0);           // keeps the next chunk's reads ahead
        }
      } else {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          s = E::mfma(tq.arow(qs, qp, c, hh), bkv(kbuf, c), s);
          dp = E::mfma(to.arow(os, qp, c, hh), bkv(vbuf, c), dp);
        }
      }
      uint32_t valid = 0;                             // masked: bit e set where query e keeps this key
      if constexpr (MK != MK_NONE) {
        const int e_min = entry_min();
        const int r0 = 32 * qp + 16 * hh;
        if constexpr (MK == MK_U8) {
          const uint8_t* mp = mraw[P] + r0 * RB + 32 * kw + ql;
#pragma unroll
          for (int e = 0; e < 16; ++e) valid |= (uint32_t)(mp[e * RB] != 0) << e;
        } else {
          const uint32_t* mp = reinterpret_cast<const uint32_t*>(mraw[P]) + 4 * r0 + kw;
#pragma unroll
          for (int e = 0; e < 16; ++e) valid |= ((mp[4 * e] >> ql) & 1u) << e;
        }
        valid &= 0xffffu << e_min;
      }
      float pv[16], sv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = s[e] * c2;
        float p;
        if constexpr (MK != MK_NONE) p = __builtin_amdgcn_exp2f(keep_or_ninf(valid, e, x));
        else p = __builtin_amdgcn_exp2f(x);           // the limit is in the start values
        pv[e] = p;
        sv[e] = p * dp[e];
      }
      // the four B operands packed first (the fp32 probabilities end here), then each pair of
      // transposed A operands read one MFMA pair ahead of its use
      const x8 pB[2] = {pack8<F16>(pv), pack8<F16>(pv + 8)}, sB[2] = {pack8<F16>(sv), pack8<F16>(sv + 8)};
      ds_store(it, sB[0], sB[1]);
      x8 ao = to.atr(os, qp, 0, 0), aq = tq.atr(qs, qp, 0, 0);
#pragma unroll
      for (int n = 0; n < 2 * DB; ++n) {
        const int sh = n / DB, d = n % DB;
        x8 ao_n = ao, aq_n = aq;
        if (n + 1 < 2 * DB) {
          ao_n = to.atr(os, qp, (n + 1) / DB, (n + 1) % DB);
          aq_n = tq.atr(qs, qp, (n + 1) / DB, (n + 1) % DB);
        }
        dv[d] = E::mfma(ao, pB[sh], dv[d]);
        dk[d] = E::mfma(aq, sB[sh], dk[d]);
        ao = ao_n;
        aq = aq_n;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (nx < n_it) {
      bi_fix(1 - P);
      bi_advance(nn);
    }
    __syncthreads();
  };
  std::integral_constant<int, 0> I0;
  std::integral_constant<int, 1> I1;
  for (int it = first, nx = second; it < n_it;) {
    int nn = next_step(nx);
    iter(I0, it, nx, nn);
    it = nx;
    nx = nn;
    if (it >= n_it) break;
    nn = next_step(nx);
    iter(I1, it, nx, nn);
    it = nx;
    nx = nn;
  }

  // the two waves of a key block add their partial sums: the second wave writes dV (then dK)
  // to LDS, lane-contiguous, and the first adds it to its own. Key blocks 0-1 use kbuf, 2-3 vbuf
  // (every read of K and V ended at the last barrier of the loop).
  float* xb = reinterpret_cast<float*>(kw < 2 ? kbuf : vbuf) + (kw & 1) * (DB * 16 * 64);
  auto merge = [&](f32x16 (&acc)[DB]) {
    if (qp == 1) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) xb[(d * 16 + e) * 64 + lane] = acc[d][e];
    }
    __syncthreads();
    if (qp == 0) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[d][e] += xb[(d * 16 + e) * 64 + lane];
    }
    __syncthreads();
  };
  if constexpr (DS) {
    // this wave's share of dscale = sum_ij dS_ij <q_i, k_j> = sum_j <dk_j, k_j>, dk_j being the
    // wave's sum_i dS_ij q_i (so the waves' shares add up), read before the merge overwrites K.
    // Lane (ql, hh) holds dk[d][4 i + t] of key kvrow at head-dim 32 d + 8 i + 4 hh + t.
    float part = 0.f;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 kk = *reinterpret_cast<const uint2*>(kbuf + kvrow * D + (((4 * d + i) ^ kvsw) << 3) + 4 * hh);
        part = fmaf(dk[d][4 * i], E::lo(kk.x), part);
        part = fmaf(dk[d][4 * i + 1], E::hi(kk.x), part);
        part = fmaf(dk[d][4 * i + 2], E::lo(kk.y), part);
        part = fmaf(dk[d][4 * i + 3], E::hi(kk.y), part);
      }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
    if (lane == 0 && g.w_dsp) g.w_dsp[(int64_t)blockIdx.x * (NT8 / 64) + wave] = part;
  }
  merge(dv);
  merge(dk);
  if (qp == 1 || key_me >= a.Lkv) return;
  const int64_t kr = b * g.dk_sb + (int64_t)key_me * g.dk_ss + gk * g.dk_sh;
  const int64_t vr = b * g.dv_sb + (int64_t)key_me * g.dv_ss + gk * g.dv_sh;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 32 * d + 8 * i + 4 * hh;
      store4(g.dk, kr + col, g.dk_dtype, dk[d][4 * i] * a.scale, dk[d][4 * i + 1] * a.scale,
             dk[d][4 * i + 2] * a.scale, dk[d][4 * i + 3] * a.scale);
      store4(g.dv, vr + col, g.dv_dtype, dv[d][4 * i], dv[d][4 * i + 1], dv[d][4 * i + 2], dv[d][4 * i + 3]);
    }
}

// ================================ dQ =========================================================
template <int D, bool F16, int MK>
__global__ __launch_bounds__(NTB, MK == MK_NONE ? 1 : 2) void bwd_dq_mfma_kernel(BwdArgs g, int n_qt, int remap) {
  using E = In<F16>;
  using x8 = typename E::x8;
  constexpr int DC = D / 16, DB = D / 32, TILE = ST * D;
  __shared__ __align__(16) uint16_t kbuf0[TILE], kbuf1[TILE], vbuf0[TILE], vbuf1[TILE];
  // mask tile [buffer][query][key]: U8 64 bytes a query, U1 2 words a query
  __shared__ __align__(16) uint8_t mraw[MK ? 2 : 1][MK == MK_U8 ? RB * ST : RB * 8];
  __shared__ uint64_t live_bits[MK == MK_BI ? kLiveWords : 1];   // block info: bit t, tile t is not empty
  const AttnArgs& a = g.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;

  int rank, bh;
  wg_map(blockIdx.x, a.Hq * a.B, remap, rank, bh);
  const int qt = n_qt - 1 - rank;                 // causal: the last query tiles are the heaviest
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int gk = h / (a.Hq / a.Hkv);
  const int q0 = qt * RB;
  const int nkv = batch_kv_len(a, b), nq = batch_q_len(a, b);
  const int64_t off = batch_causal_offset(a, b);
  const bool causal = a.causal != SDPA_CAUSAL_NONE;
  const float c2 = a.scale * LOG2E;
  const int i_me = q0 + 32 * wave + ql;
  const int64_t wrow = ((int64_t)b * a.Hq + h) * a.Lq + i_me;
  // the prep pass wrote -lse / scale and -D for this route (BwdArgs)
  const float lse2 = i_me < nq ? -g.w_lse[wrow] * c2 : INFINITY;
  const float dsum = i_me < nq ? -g.w_dsum[wrow] : 0.f;

  // keys the workgroup and this wave visit
  const int row_end = min(q0 + RB, nq);
  int64_t k_end = nkv;
  if (causal) { const int64_t l = off + row_end; if (l < k_end) k_end = l; }
  if (row_end <= q0 || k_end < 0) k_end = 0;
  const int w_last = min(q0 + 32 * wave + 31, row_end - 1);
  int64_t k_end_w = nkv;
  if (causal) { const int64_t l = off + w_last + 1; if (l < k_end_w) k_end_w = l; }
  if (w_last < q0 + 32 * wave || k_end_w < 0) k_end_w = 0;
  const int n_tiles = (int)((k_end + ST - 1) / ST);
  // per-entry key limit of this lane: keys below kv_lengths and (causal) at most off + i
  int64_t lim_me = nkv;
  if (causal) { const int64_t l = off + i_me + 1; if (l < lim_me) lim_me = l; }

  // Q and dO of this lane's query as B operands (rows past Lq as zeros)
  x8 qB[DC], oB[DC];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(a.q) + b * a.q_sb + h * a.q_sh,
                                                (int64_t)a.Lq * a.q_ss * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<const uint16_t*>(g.dout) + b * g.do_sb + h * g.do_sh,
                                                (int64_t)a.Lq * g.do_ss * 2);
    const int qo = i_me * (int)(a.q_ss * 2) + 16 * hh, oo = i_me * (int)(g.do_ss * 2) + 16 * hh;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      qB[c] = __builtin_bit_cast(x8, buf_load16(rq, qo + 32 * c));
      oB[c] = __builtin_bit_cast(x8, buf_load16(ro, oo + 32 * c));
    }
  }

  Tiles<D, F16, ST> tk, tv;
  tk.init((int)(a.k_ss * 2), lane, tid);
  tv.init((int)(a.v_ss * 2), lane, tid);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + gk * a.k_sh;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + gk * a.v_sh;
  auto load_tiles = [&](int t, uint16_t* kd, uint16_t* vd) {
    tk.load(kp, a.k_ss, t * ST, nkv, (int)(a.k_ss * 2), kd, wave);
    tv.load(vp, a.v_ss, t * ST, nkv, (int)(a.v_ss * 2), vd, wave);
  };

  f32x16 dq[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[d][e] = 0.f;
  float dsc = 0.f;
  // mask rows of tile t (queries q0 .. q0 + 127, keys t * 64 .. + 63) into mraw[buf]
  auto load_mask = [&](int t, int buf) {
    if constexpr (MK == MK_U8 || MK == MK_U1) {
      const __amdgpu_buffer_rsrc_t rm = mask_rsrc(a, b, h);
      if constexpr (MK == MK_U8) {                   // 16 bytes a thread and pass: row 64u + 16 * wave + lane / 4
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t i = q0 + 64 * u + 16 * wave + (lane >> 2);
          dma16(rm, reinterpret_cast<uint16_t*>(mraw[buf] + 4096 * u + 1024 * wave),
                (int)(i * a.mask_sq) + t * ST + 16 * (lane & 3));
        }
      } else {                                       // one word a thread: row tid / 2, word tid % 2
        const int64_t i = q0 + (tid >> 1);
        dma4(rm, mraw[buf] + 256 * wave, (int)((i * a.mask_sq + 2 * t + (tid & 1)) * 4));
      }
    }
  };

  // block info: thread t owns word t % 2 of query row t / 2 of each tile
  int bi_cls = 0, bi_nxt = 0, bi_src = -1;
  auto bi_load_raw = [&](int t) {
    if constexpr (MK == MK_BI) {
      if (t < n_tiles) bi_fetch(a, b, h, q0 + (tid >> 1), t * ST + 32 * (tid & 1), bi_cls, bi_nxt);
    }
  };
  auto bi_advance = [&](int t) {
    if constexpr (MK == MK_BI) bi_src = bi_source(a, bi_cls, bi_nxt, q0 + (tid >> 1), t * ST + 32 * (tid & 1));
  };
  auto bi_dma = [&](int buf) {
    if constexpr (MK == MK_BI)
      dma4(make_rsrc(a.bm_bits, bi_bits_bytes(a)), mraw[buf] + 256 * wave, bi_src >= 0 ? bi_src : kBiNone);
  };
  auto bi_fix = [&](int buf) {
    if constexpr (MK == MK_BI) {
      if (bi_src == -2) reinterpret_cast<uint32_t*>(mraw[buf])[tid] = 0xffffffffu;
    }
  };
  // block info: the tiles that meet a non-empty block (the loop visits only those)
  bool scan = false;
  if constexpr (MK == MK_BI) {
    scan = n_tiles <= kLiveWords * 64;
    if (scan) {
      for (int s0 = 64 * wave; s0 < n_tiles; s0 += 64 * (NTB / 64)) {
        const int st = s0 + lane;
        const bool lv = st < n_tiles && bi_rect_live(a, b, h, q0, q0 + RB, st * ST, st * ST + ST);
        const uint64_t m = __builtin_amdgcn_ballot_w64(lv);
        if (lane == 0) live_bits[s0 >> 6] = m;
      }
      __syncthreads();
    }
  }
  auto next_step = [&](int st) -> int {     // the first visited tile after st, or n_tiles
    if constexpr (MK == MK_BI) {
      if (scan) {
        for (++st; st < n_tiles; st = (st | 63) + 1) {
          const uint64_t m = live_bits[st >> 6] >> (st & 63);
          if (m) return st + (int)__builtin_ctzll(m);
        }
        return n_tiles;
      }
    }
    return min(st + 1, n_tiles);
  };

  const int first = next_step(-1), second = next_step(first);
  if (first < n_tiles) {
    load_tiles(first, kbuf0, vbuf0);
    load_mask(first, 0);
    if constexpr (MK == MK_BI) {
      bi_load_raw(first);
      __builtin_amdgcn_s_waitcnt(0);
      bi_advance(first);
      bi_dma(0);
      bi_load_raw(second);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (first < n_tiles) {
    bi_fix(0);
    bi_advance(second);
  }
  __syncthreads();

  // tile t in buffer P; nx: the next visited tile (prefetched here), nn: the one after it
  auto iter = [&](auto PAR_, int t, int nx, int nn) {
    constexpr int P = decltype(PAR_)::value;
    const uint16_t* ks = P ? kbuf1 : kbuf0;
    const uint16_t* vs = P ? vbuf1 : vbuf0;
    if (nx < n_tiles) {
      load_tiles(nx, P ? kbuf0 : kbuf1, P ? vbuf0 : vbuf1);
      load_mask(nx, 1 - P);
      bi_dma(1 - P);
      bi_load_raw(nn);
    }
    const int k0 = t * ST;
    if (k0 < k_end_w) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int jbase = k0 + 32 * kb + 16 * hh;     // entry e of this lane: key jbase + e
        f32x16 s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          s = E::mfma(tk.arow(ks, kb, c, hh), qB[c], s);
          dp = E::mfma(tv.arow(vs, kb, c, hh), oB[c], dp);
        }
        int e_end = 16;
        {
          const int64_t m = lim_me - jbase;
          e_end = m < 0 ? 0 : (m > 16 ? 16 : (int)m);
        }
        uint32_t valid = 0;                           // masked: bit e set where key jbase + e is kept
        if constexpr (MK == MK_U8) {
          const uint4 x = *reinterpret_cast<const uint4*>(mraw[P] + (32 * wave + ql) * ST + 32 * kb + 16 * hh);
          valid = nonzero_nibble4(x.x) | (nonzero_nibble4(x.y) << 4) | (nonzero_nibble4(x.z) << 8) |
                  (nonzero_nibble4(x.w) << 12);
        } else if constexpr (MK == MK_U1 || MK == MK_BI) {
          valid = reinterpret_cast<const uint32_t*>(mraw[P])[2 * (32 * wave + ql) + kb] >> (16 * hh);
        }
        if constexpr (MK != MK_NONE) valid &= (1u << e_end) - 1u;
        float sv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = fmaf(s[e], c2, -lse2);
          float p;
          if constexpr (MK != MK_NONE) p = __builtin_amdgcn_exp2f(keep_or_ninf(valid, e, x));
          else p = __builtin_amdgcn_exp2f(e < e_end ? x : -INFINITY);
          const float d_s = p * (dp[e] - dsum);
          sv[e] = d_s;
          dsc = fmaf(d_s, s[e], dsc);
        }
        if constexpr (D == 128) {
          // dS packed first, then each transposed K fragment read one MFMA ahead of its use
          // (at D = 64 the extra registers would cost a wave per SIMD)
          const x8 sB[2] = {pack8<F16>(sv), pack8<F16>(sv + 8)};
          x8 ak = tk.atr(ks, kb, 0, 0);
#pragma unroll
          for (int n = 0; n < 2 * DB; ++n) {
            x8 ak_n = ak;
            if (n + 1 < 2 * DB) ak_n = tk.atr(ks, kb, (n + 1) / DB, (n + 1) % DB);
            dq[n % DB] = E::mfma(ak, sB[n / DB], dq[n % DB]);
            ak = ak_n;
          }
        } else {
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            const x8 sB = pack8<F16>(sv + 8 * sh);
#pragma unroll
            for (int d = 0; d < DB; ++d) dq[d] = E::mfma(tk.atr(ks, kb, sh, d), sB, dq[d]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (nx < n_tiles) {
      bi_fix(1 - P);
      bi_advance(nn);
    }
    __syncthreads();
  };
  std::integral_constant<int, 0> I0;
  std::integral_constant<int, 1> I1;
  for (int t = first, nx = second; t < n_tiles;) {
    int nn = next_step(nx);
    iter(I0, t, nx, nn);
    t = nx;
    nx = nn;
    if (t >= n_tiles) break;
    nn = next_step(nx);
    iter(I1, t, nx, nn);
    t = nx;
    nx = nn;
  }

  if (i_me >= a.Lq) return;
  dsc += __shfl_xor(dsc, 32, 64);
  if (hh == 0) g.w_dsc[wrow] = dsc;
  const int64_t qr = b * g.dq_sb + (int64_t)i_me * g.dq_ss + h * g.dq_sh;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 32 * d + 8 * i + 4 * hh;
      store4(g.dq, qr + col, g.dq_dtype, dq[d][4 * i] * a.scale, dq[d][4 * i + 1] * a.scale,
             dq[d][4 * i + 2] * a.scale, dq[d][4 * i + 3] * a.scale);
    }
}

// ================================ dQ from the stored dS ======================================
// A workgroup of 8 waves owns 256 queries of one head and streams tiles of 64 keys. Wave w forms
// dQ^T += K^T dS^T for the 64 queries q0 + 64 (w / 2) .. + 63 and half of the head dim (32-wide
// blocks (w % 2) * DB / 2 ..), both operands by transposed LDS reads: K^T from the K tile, dS^T
// from the tile's four pieces of stored dS (queries q0 + 64 p .. + 63, 64 x 64 each, written to
// LDS row-major by key). The pass is bound by those LDS reads; 64 x D/2 per wave reads 20% less
// than 32 x D. The dS stream comes from HBM, whose latency is far longer than a tile's products,
// so it is loaded DQA tiles ahead into registers (each thread 16 bytes of each piece, in the order
// the dK/dV pass stored them) and written to LDS only when its tile comes up; K, read again by
// every query tile of the head and mostly found in L2, goes straight to LDS (a stage per tile in
// flight), requested once the stage's previous tile has been read. Loads past the last tile read
// an empty range, so every step issues the same loads and the waits are fixed counts. A piece the
// dK/dV pass did not write (no query of it sees a key of its block) is read from an empty range
// too: zeros. Within a written piece, a 32-key x 32-query block whose weights are all 0 holds
// stale bytes (the dK/dV wave skips it), and the same test skips it here.
constexpr int DQW = 256;          // queries of a dQ workgroup on this route
constexpr int DQA = 3;            // tiles of dS in flight (in registers)

template <int D, bool F16>
__global__ __launch_bounds__(NT8, 1) void bwd_dq_ds_kernel(BwdArgs g, int n_qt, int remap) {
  using E = In<F16>;
  using x8 = typename E::x8;
  constexpr int DB = D / 32, DW = DB / 2, TILE = ST * D, PIECE = 64 * 64, NP = DQW / 64, QT = 64;
  using TK = Tiles<D, F16, ST, NT8>;
  constexpr int LT = TK::SPT + NP;                    // loads per thread and tile
  // Each step issues the dS loads of the tile DQA ahead, then (after its barriers) the K loads
  // of the same tile. Waits, vmcnt(n) lgkmcnt(0): (a) the dS registers of the step's tile have
  // arrived (then issued: its K, and dS + K of the next DQA - 1 tiles); (c) its K has landed
  // (then issued: dS + K of the next DQA - 1 tiles, and the dS just requested)
  constexpr int kWaitA = vm_wait(TK::SPT + (DQA - 1) * LT);
  constexpr int kWaitC = vm_wait(NP + (DQA - 1) * LT);
  // one K array per stage: the compiler's wait analysis tells the direct loads into one array
  // from the reads of another only by the array (stages of one array look aliased)
  __shared__ __align__(16) uint16_t kbuf0[TILE], kbuf1[TILE], kbuf2[TILE], sbuf[NP * PIECE];
  auto kst = [&](auto S_) -> uint16_t* {
    constexpr int S = decltype(S_)::value % DQA;
    return S == 0 ? kbuf0 : (S == 1 ? kbuf1 : kbuf2);
  };
  const AttnArgs& a = g.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int wq = wave >> 1, wd = wave & 1;            // the wave's 64 queries (a piece), head-dim half

  int rank, bh;
  wg_map(blockIdx.x, a.Hq * a.B, remap, rank, bh);
  const int qt = n_qt - 1 - rank;                 // causal: the last query tiles are the heaviest
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int gk = h / (a.Hq / a.Hkv);
  const int q0 = qt * DQW;
  const int nkv = batch_kv_len(a, b), nq = batch_q_len(a, b);
  const int64_t off = batch_causal_offset(a, b);
  const bool causal = a.causal != SDPA_CAUSAL_NONE;

  // keys the workgroup visits, and the end of the keys each 32-query block of the wave sees
  // (past it the block's dS is all zeros)
  const int row_end = min(q0 + DQW, nq);
  int64_t k_end = nkv;
  if (causal) { const int64_t l = off + row_end; if (l < k_end) k_end = l; }
  if (row_end <= q0 || k_end < 0) k_end = 0;
  const int n_tiles = (int)((k_end + ST - 1) / ST);
  int64_t k_end_b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r0 = q0 + 64 * wq + 32 * j, last = min(r0 + 31, row_end - 1);
    int64_t e = nkv;
    if (causal) { const int64_t l = off + last + 1; if (l < e) e = l; }
    k_end_b[j] = (last < r0 || e < 0) ? 0 : e;
  }

  // the dK/dV pass wrote dS tile (query tile qt64, key block kb) iff the block starts before
  // kv_lengths (kb * RB < nkv), qt64 lies before q_lengths (qt64 < n_qt64), and qt64 is not
  // below the first query tile that sees the block: with i_lo = max(0, kb * RB - off) (causal,
  // else 0), i_lo < nq and qt64 >= i_lo / QT
  const int n_qt64 = (nq + QT - 1) / QT, ds_nqt = (a.Lq + QT - 1) / QT, ds_nkb = (a.Lkv + RB - 1) / RB;

  TK tk;
  tk.init((int)(a.k_ss * 2), lane, tid);
  // transposed-read offsets (the pattern of Tiles::atr, with the wave's column blocks fixed):
  // rows 16 * hh + (lane % 16) / 4 (+ 4), columns 16 * ((lane / 16) % 2) + 4 * (lane % 4) of
  // each 32-wide block; dS^T: query blocks 0 and 1 of the wave's piece, K^T: its head-dim blocks
  const int t_vr = 16 * hh + ((lane & 15) >> 2);
  const int t_vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int s_lo[2], s_hi[2], k_lo[DW], k_hi[DW];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 32 * j + t_vc;
    s_lo[j] = t_vr * 64 + ((((c >> 3) ^ bswz<64>(t_vr)) << 3) | (c & 7));
    s_hi[j] = (t_vr + 4) * 64 + ((((c >> 3) ^ bswz<64>(t_vr + 4)) << 3) | (c & 7));
  }
#pragma unroll
  for (int j = 0; j < DW; ++j) {
    const int c = 32 * (DW * wd + j) + t_vc;
    k_lo[j] = t_vr * D + ((((c >> 3) ^ bswz<D>(t_vr)) << 3) | (c & 7));
    k_hi[j] = (t_vr + 4) * D + ((((c >> 3) ^ bswz<D>(t_vr + 4)) << 3) | (c & 7));
  }
  auto tr = [&](const uint16_t* t, int lo, int hi) -> x8 {
    const s16x4 l = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(t + lo));
    const s16x4 u = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(t + hi));
    const s16x8 v = {l[0], l[1], l[2], l[3], u[0], u[1], u[2], u[3]};
    return __builtin_bit_cast(x8, v);
  };

  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + gk * a.k_sh;
  const uint16_t* dsp = g.w_ds + (((int64_t)b * a.Hq + h) * ds_nqt + NP * qt) * ds_nkb * (RB * QT);
  // thread tid reads bytes 16 * tid of a piece: KiB `wave`, lane `lane` of the dK/dV layout
  // (ds_offset), i.e. key row 32 * (wave >> 2) + ql, queries 8 * c .. + 7 with
  // c = 4 * ((wave >> 1) & 1) + 2 * hh + (wave & 1); it writes them to that row's swizzled chunk
  const int s_row = 32 * (wave >> 2) + ql;
  const int s_lds = s_row * 64 + (((4 * ((wave >> 1) & 1) + 2 * hh + (wave & 1)) ^ bswz<64>(s_row)) << 3);
  // Tile t of piece p is the PIECE at dsp + (p * ds_nkb + t / 2) * RB * QT + (t % 2) * PIECE,
  // i.e. at t * PIECE from the piece's first tile. The test above holds exactly for kb below
  // kb_lim(qt64) (the same test solved for kb), so each piece is read through one buffer range
  // that ends after its last written tile and before n_tiles: every other load returns zeros,
  // with no per-tile address or range arithmetic.
  auto kb_lim = [&](int qt64) -> int64_t {
    if (qt64 >= n_qt64 || nkv <= 0) return 0;
    int64_t lim = ((int64_t)nkv + RB - 1) / RB;
    if (causal) {
      const int64_t e = off + min((int64_t)nq, (int64_t)(qt64 + 1) * QT);
      const int64_t c = e > 0 ? (e + RB - 1) / RB : 0;
      lim = c < lim ? c : lim;
    }
    return lim;
  };
  __amdgpu_buffer_rsrc_t rds[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t nt = min(2 * kb_lim(NP * qt + p), (int64_t)n_tiles);
    rds[p] = make_rsrc(dsp + (int64_t)p * ds_nkb * (RB * QT), nt * (PIECE * 2));
  }
  auto load_ds = [&](int t, uint4 (&r)[NP]) {
    const int vo = 16 * tid + t * (PIECE * 2);
#pragma unroll
    for (int p = 0; p < NP; ++p) r[p] = buf_load16(rds[p], vo);
  };
  auto load_k = [&](int t, uint16_t* kd) { tk.load(kp, a.k_ss, t * ST, t < n_tiles ? nkv : t * ST, (int)(a.k_ss * 2), kd, wave); };
  auto put_ds = [&](const uint4 (&r)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) *reinterpret_cast<uint4*>(sbuf + p * PIECE + s_lds) = r[p];
  };

  f32x16 dq[2][DW];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int d = 0; d < DW; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[j][d][e] = 0.f;

  // prologue: dS and K of tiles 0 .. DQA - 1, in the order the steps issue them
  std::integral_constant<int, 0> I0;
  std::integral_constant<int, 1> I1;
  std::integral_constant<int, 2> I2;
  uint4 rb[DQA][NP];
  load_ds(0, rb[0]);
  load_k(0, kst(I0));
  load_ds(1, rb[1]);
  load_k(1, kst(I1));
  load_ds(2, rb[2]);
  load_k(2, kst(I2));

  // tile t: its dS in registers rb[t % DQA], its K in stage t % DQA
  auto iter = [&](auto S_, int t) {
    constexpr int S = decltype(S_)::value;
    __builtin_amdgcn_s_waitcnt(kWaitA);               // (a) dS of tile t has arrived
    put_ds(rb[S]);
    load_ds(t + DQA, rb[S]);
    __builtin_amdgcn_s_waitcnt(kWaitC);               // (c) K of tile t has landed, dS is in LDS
    __builtin_amdgcn_s_barrier();
    const uint16_t* ks = kst(S_);
    const uint16_t* ss = sbuf + wq * PIECE;
    // The tile's four (key block kb, 8-row step) sections in one branch-free chain, each
    // section's fragments read while the previous section's products run. The dK/dV wave of 32
    // keys and a 32-query block formed (and stored) its dS block iff the keys start before the
    // end of the keys the block sees; a block it skipped holds stale bytes in LDS, so its
    // operand is replaced by zeros (products of exact zeros, on edge tiles only).
    const int tk0 = t * ST;
    if (tk0 < k_end_b[0] || tk0 < k_end_b[1]) {
      x8 kA[2][DW], sB[2][2];
      auto rd = [&](int sc, int buf) {
        const int rows = 32 * (sc >> 1) + 8 * (sc & 1);
#pragma unroll
        for (int d = 0; d < DW; ++d) kA[buf][d] = tr(ks + rows * D, k_lo[d], k_hi[d]);
#pragma unroll
        for (int j = 0; j < 2; ++j) sB[buf][j] = tr(ss + rows * 64, s_lo[j], s_hi[j]);
      };
      rd(0, 0);
#pragma unroll
      for (int sc = 0; sc < 4; ++sc) {
        if (sc + 1 < 4) rd(sc + 1, (sc + 1) & 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bool live = tk0 + 32 * (sc >> 1) < k_end_b[j];
          const x8 bj = live ? sB[sc & 1][j] : x8{};
#pragma unroll
          for (int d = 0; d < DW; ++d) dq[j][d] = E::mfma(kA[sc & 1][d], bj, dq[j][d]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);           // this wave's reads of sbuf and stage S are done
    __builtin_amdgcn_s_barrier();
    load_k(t + DQA, kst(S_));
  };
  // whole periods of DQA steps, the last one's steps past n_tiles doing nothing but their
  // (empty) loads: every path into the loop head then carries the same loads in flight, which
  // the compiler's wait analysis needs to keep its counts exact across the back edge
  static_assert(DQA == 3, "the loop below is unrolled by DQA");
  for (int t = 0; t < n_tiles; t += DQA) {
    iter(I0, t);
    iter(I1, t + 1);
    iter(I2, t + 2);
  }
  __builtin_amdgcn_s_waitcnt(0);                      // the loads past the last tile

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i_me = q0 + 64 * wq + 32 * j + ql;
    if (i_me >= a.Lq) continue;
    const int64_t qr = b * g.dq_sb + (int64_t)i_me * g.dq_ss + h * g.dq_sh;
#pragma unroll
    for (int d = 0; d < DW; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = 32 * (DW * wd + d) + 8 * i + 4 * hh;
        store4(g.dq, qr + col, g.dq_dtype, dq[j][d][4 * i] * a.scale, dq[j][d][4 * i + 1] * a.scale,
               dq[j][d][4 * i + 2] * a.scale, dq[j][d][4 * i + 3] * a.scale);
      }
  }
}

bool al(const void* p, int n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

// The stored-dS route runs: the matrix-core kernels take the call (checked by the caller), the
// workspace holds the dS tiles, and no block info (whose skipped steps would leave tiles unwritten).
bool bwd_stores_ds(const BwdArgs& g) { return g.w_ds != nullptr && g.w_dsp != nullptr && !g.a.bm_class; }

namespace {

template <int D, bool F16>
hipError_t launch_dq_t(const BwdArgs& g, hipStream_t s) {
  const AttnArgs& a = g.a;
  const int n_qt = (a.Lq + RB - 1) / RB;
  const int HB = a.Hq * a.B;
  const dim3 grid((unsigned)((int64_t)n_qt * HB));
  const int remap = HB % 8 == 0 ? 1 : 0;
  if (bwd_stores_ds(g)) {
    const int n_qw = (a.Lq + DQW - 1) / DQW;
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, F16>), dim3((unsigned)((int64_t)n_qw * HB)), dim3(NT8), 0, s, g, n_qw,
                       remap);
  } else if (a.bm_class)
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<D, F16, MK_BI>), grid, dim3(NTB), 0, s, g, n_qt, remap);
  else if (!a.mask)
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<D, F16, MK_NONE>), grid, dim3(NTB), 0, s, g, n_qt, remap);
  else if (a.mask_u1)
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<D, F16, MK_U1>), grid, dim3(NTB), 0, s, g, n_qt, remap);
  else
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<D, F16, MK_U8>), grid, dim3(NTB), 0, s, g, n_qt, remap);
  return hipGetLastError();
}


}  // namespace

bool bwd_mfma_supports(const BwdArgs& g) {
  const AttnArgs& a = g.a;
  if ((a.in_dtype != SDPA_BF16 && a.in_dtype != SDPA_F16) || a.D != a.Dv || (a.D != 64 && a.D != 128)) return false;
  if (g.do_dtype != a.in_dtype) return false;            // dO streams through the same 16-bit tiles
  if (a.bias || a.qk_norm || a.q_seg) return false;
  if (a.bm_class && (bi_bits_bytes(a) > (1 << 30) || !al(a.bm_bits, 4))) return false;
  if (a.mask) {
    // 16-byte rows of the mask tiles: unit key stride, 16-byte aligned row starts; 32-bit offsets
    const int64_t eb = a.mask_u1 ? 4 : 1, q = 16 / eb;
    if (a.mask_sk != 1 || !al(a.mask, 16) || (a.mask_sb % q) || (a.mask_sh % q) || (a.mask_sq % q)) return false;
    if (a.mask_sb < 0 || a.mask_sh < 0 || a.mask_sq < 0) return false;
    const int64_t row_bytes = a.mask_u1 ? (int64_t)((a.Lkv + 31) / 32) * 4 : a.Lkv;
    if (((int64_t)a.Lq + 2 * RB) * a.mask_sq * eb + row_bytes + 2 * RB > INT32_MAX) return false;
  }
  if (!(a.scale > 0.f)) return false;    // the dK/dV pass folds lse / scale into its MFMAs
  if (!al(a.q, 16) || !al(a.k, 16) || !al(a.v, 16) || !al(g.dout, 16)) return false;
  if ((a.q_sb | a.q_ss | a.q_sh | a.k_sb | a.k_ss | a.k_sh | a.v_sb | a.v_ss | a.v_sh | g.do_sb | g.do_ss | g.do_sh) & 7)
    return false;
  const int64_t eq = g.dq_dtype == SDPA_F32 ? 4 : 2, ek = g.dk_dtype == SDPA_F32 ? 4 : 2, ev = g.dv_dtype == SDPA_F32 ? 4 : 2;
  if (!al(g.dq, (int)(4 * eq)) || !al(g.dk, (int)(4 * ek)) || !al(g.dv, (int)(4 * ev))) return false;
  if ((g.dq_sb | g.dq_ss | g.dq_sh | g.dk_sb | g.dk_ss | g.dk_sh | g.dv_sb | g.dv_ss | g.dv_sh) & 3) return false;
  if (a.q_ss < a.D || a.k_ss < a.D || a.v_ss < a.D || g.do_ss < a.D) return false;
  // (the dK/dV pass adds a step's first row to offsets within its 64-row tiles)
  if (((int64_t)a.Lq + QT8) * a.q_ss * 2 > INT32_MAX || (int64_t)a.Lkv * a.k_ss * 2 > INT32_MAX ||
      (int64_t)a.Lkv * a.v_ss * 2 > INT32_MAX || ((int64_t)a.Lq + QT8) * g.do_ss * 2 > INT32_MAX ||
      ((int64_t)a.Lq + QT8) * 4 > INT32_MAX)
    return false;
  const int64_t n1 = (int64_t)((a.Lkv + RB - 1) / RB) * a.Hkv * a.B, n2 = (int64_t)((a.Lq + RB - 1) / RB) * a.Hq * a.B;
  return n1 < (int64_t)INT32_MAX && n2 < (int64_t)INT32_MAX;
}

template <int D, bool F16>
hipError_t launch_dkdv8_t(const BwdArgs& g, hipStream_t s) {
  const AttnArgs& a = g.a;
  const int n_kt = (a.Lkv + RB - 1) / RB;
  const int HB = a.Hkv * a.B;
  const dim3 grid((unsigned)((int64_t)n_kt * HB));
  const int remap = HB % 8 == 0 ? 1 : 0;
  const bool ds = bwd_stores_ds(g);
  if (a.bm_class)
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, F16, MK_BI, false>), grid, dim3(NT8), 0, s, g, remap);
  else if (!a.mask && ds)
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, F16, MK_NONE, true>), grid, dim3(NT8), 0, s, g, remap);
  else if (!a.mask)
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, F16, MK_NONE, false>), grid, dim3(NT8), 0, s, g, remap);
  else if (a.mask_u1 && ds)
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, F16, MK_U1, true>), grid, dim3(NT8), 0, s, g, remap);
  else if (a.mask_u1)
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, F16, MK_U1, false>), grid, dim3(NT8), 0, s, g, remap);
  else if (ds)
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, F16, MK_U8, true>), grid, dim3(NT8), 0, s, g, remap);
  else
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, F16, MK_U8, false>), grid, dim3(NT8), 0, s, g, remap);
  return hipGetLastError();
}

hipError_t launch_bwd_mfma_dkdv(const BwdArgs& g, hipStream_t s) {
  const bool f16 = g.a.in_dtype == SDPA_F16;
  if (g.a.D == 128) return f16 ? launch_dkdv8_t<128, true>(g, s) : launch_dkdv8_t<128, false>(g, s);
  return f16 ? launch_dkdv8_t<64, true>(g, s) : launch_dkdv8_t<64, false>(g, s);
}

hipError_t launch_bwd_mfma_dq(const BwdArgs& g, hipStream_t s) {
  const bool f16 = g.a.in_dtype == SDPA_F16;
  if (g.a.D == 128) return f16 ? launch_dq_t<128, true>(g, s) : launch_dq_t<128, false>(g, s);
  return f16 ? launch_dq_t<64, true>(g, s) : launch_dq_t<64, false>(g, s);
}

}  // namespace sdpa
