// fwd_mfma.hip -- bf16 attention forward on the gfx950 matrix cores (head dims 64 and 128).
//
// What it computes is the "Fused implementation" of the page "Neural Network primitives from
// NNlib.jl": the output is built tile by tile with the softmax taken online over tiles of keys,
// so the weights are never materialized. Every option of that page's "Arguments" list that the
// ABI exposes is honoured: GQA, causal (top-left with q_offset, or bottom-right), kv_lengths,
// q_lengths, an additive bias and a boolean mask (dense, or as block info from
// build_block_mask_info so that empty blocks are never visited and full blocks skip the element
// test -- the block-sparse scheme of the splash-attention pull request "Support dynamic masks in
// splash attention #25213").
//
// Mapping onto CDNA4
// ------------------
// * One workgroup = 4 waves = a tile of 128 query rows of one (batch, head); each wave owns 32
//   rows; two workgroups share a CU (two waves per SIMD). The workgroup streams tiles of 64 keys
//   of the matching K/V head through LDS. Direct global -> LDS loads (no staging registers) of
//   K(t+2) and V(t+1) are issued as tile t starts and have landed by its end.
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16
//   head-dim values from LDS, B = the wave's Q^T kept in registers for the whole loop). K rows are
//   written to LDS in a permuted order so that the 16 accumulator entries a lane receives are 16
//   consecutive keys of one query row. That makes every row reduction mostly in-lane (one swap
//   with lane^32) and lets the probabilities P^T feed the next MFMA directly as its B operand, in
//   registers, with no LDS round trip.
// * O^T += V^T P^T with the same instruction; V stays row-major in LDS and its A operand is read
//   with ds_read_b64_tr_b16, which transposes 16-bit elements on the way out of LDS.
// * S(t+1) is formed while the probabilities of S(t) are taken, so that the matrix cores and the
//   VALU work on independent instructions.
// * The online softmax runs in the exp2 domain. Without bias and QK-norm, scale*log2(e) is
//   folded into Q once and the q.k MFMAs start from -m (the running max) instead of zero, so a
//   probability is a single v_exp_f32 of the accumulator; otherwise the logits are multiplied by
//   scale*log2(e) (and the bias by log2(e)) first. A row that has seen no allowed key
//   contributes nothing; if it ends with l = 0 it is written as NaN ("Fused implementation": a
//   query that attends no key).
// * Element masking (causal, kv_lengths, mask) is applied only on tiles that need it; tiles past
//   a wave's causal limit are skipped by that wave, tiles past the workgroup's limit are not
//   loaded. Keys past kv_lengths are loaded as zeros, so a poisoned cache tail never reaches
//   the arithmetic (0 * NaN would).
// * Grid: every XCD (the hardware deals consecutive workgroups round-robin over the 8 XCDs; each
//   has its own L2) gets a contiguous set of heads. Non-causal launches run one head's tiles
//   back to back (K/V reuse in L2), or, with a bias broadcast over the batch, the batches of one
//   head and tile back to back (bias reuse in L2); causal launches run longest tile first
//   within groups of 4 heads per XCD.
#include <type_traits>

#include "mfma_common.h"

namespace sdpa {

namespace {

constexpr int BM = 128;            // query rows per workgroup
constexpr int BN = 64;             // keys per tile
constexpr int NT = 256;            // threads per workgroup

// BIAS_F32: an fp32 bias, or a bf16 bias the fused path cannot stage (read element by element)
enum { BIAS_NONE = 0, BIAS_BF16 = 1, BIAS_F32 = 2 };
// MASK_INFO: block info whose rows hold at most 64 blocks (the host knows n_kb) of a power-of-two
// number of 64-key tiles, every CSR entry of a row in the lanes of one register; MASK_INFO_LONG:
// any other block info, entries from 64 on loaded from memory where they are used. (With such a load in one arm of a lookup, the
// compiler makes the common arm wait for every load in flight, prefetches included, so the
// short form has no such arm at all.)
enum { MASK_NONE = 0, MASK_DENSE = 1, MASK_INFO = 2, MASK_INFO_LONG = 3 };

// Key held by LDS row r (0..31) of a 32-key block of K: the A operand of S^T = K Q^T takes row
// r, and this order makes accumulator entry 4*i + j of lane half h hold key 16*h + 4*i + j.
__device__ __forceinline__ int k_row_key(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// LDS tiles hold whole 16-byte chunks (8 bf16) of D-element rows with no padding; the chunk
// positions within a row are XOR-swizzled so that the reads below hit distinct banks:
//   K: the 16 lanes of a half-wave read one chunk of 16 consecutive rows (b128 reads);
//   V: a transposed read covers 4 consecutive rows x 4 chunks per 32 lanes.
template <int D>
__device__ __forceinline__ int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// Heads an XCD runs together in a causal launch: 4 heads' K/V (8 MB at L4096 D128) against 8,
// 0.9% faster at the causal prefill than all of an XCD's heads at once, 2 heads slightly slower
constexpr int kGroupHeads = 4;

// Without a bias, once every row of a wave has its running max (the first tile holding one of
// its keys sets it), the per-tile row max is no longer taken: the max moves only when a tile's
// probabilities grow past kLazyBound, which the tile's probability sum shows (inf included)
// before any of them reaches the P.V products. Probabilities up to 2^64, sums of them over
// every key and the O accumulators all stay far inside fp32 and bf16 range.
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): lgkmcnt(0) only;
// vmcnt(4) and lgkmcnt(0)
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);
constexpr int kWaitVm4Lgkm0 = 0x4 | (0x7 << 4) | (0x0 << 8);
constexpr float kLazyBound = 18446744073709551616.0f;   // 2^64
constexpr float RESCALE_SLACK = 8.0f;   // log2 units: the running max moves only when a row's max grows by more
// With a bias (logits in natural units) a row's max can grow on every tile -- an ALiBi bias rises
// along the keys by its slope times the tile width -- and each move rescales O. There the max
// moves only when it grows by more than kNatSlack, and a move sets it kNatOver beyond the new
// maximum, so that the next move waits until the row has grown by kNatSlack + kNatOver. The
// largest probability stays below e^16 and the largest of a moved tile at e^-24, both far inside
// fp32 and bf16 range (the probabilities' relative precision does not depend on their scale);
// f16 probabilities have no such range, so f16 inputs keep the plain slack.
constexpr float kNatSlack = 16.0f;
constexpr float kNatOver = 24.0f;
// The fused bias path takes its probabilities against m_s = m_run clamped to [-kStartLim,
// kStartLim] (natural units), so that m_s * log2e is finite and one fma per score turns a logit
// into the exponent; a row max beyond the clamp (a bias at the dtype's most negative value) is
// handled by moving the scores explicitly.
constexpr float kStartLim = 16384.0f;

template <int D, int BIAS, int MASK, bool NORM, bool F16, bool PACKED>
__global__ __launch_bounds__(NT, 2) void fwd_mfma_kernel(AttnArgs args, int n_qt, int remap, int order) {
  using E = In<F16>;
  using bf16x8 = typename E::x8;     // the 16-bit operand vector (bf16 or f16)
  constexpr int DC = D / 16;         // 16-wide head-dim chunks (MFMA k steps for q.k)
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int SPT = BN * CPR / NT; // direct-load instructions per thread per tile (K or V)
  constexpr int TILE = BN * D;       // elements of one K or V tile in LDS
  // FUSED: the scale is folded into Q and each S MFMA chain starts from -m_run (plus the bias
  // for a bf16 bias at D = 64, FBIAS), so the accumulator holds the logit minus the running
  // max. Otherwise the logits are scaled (and biased) per element.
  // NAT: with a bias the logits are kept in natural units and turned into log2 units only
  // after the running max is subtracted. A finite bias below -FLT_MAX/log2(e) (an additive mask
  // filled with the dtype's most negative value) then stays finite, as the definition has it,
  // instead of overflowing to -inf and passing for a masked key. Without a bias the logits are
  // in log2 units from the start (scale*log2e folded into Q, or into the per-element scale).
  constexpr bool MI = MASK == MASK_INFO || MASK == MASK_INFO_LONG;
  constexpr bool FBIAS = BIAS == BIAS_BF16 && D == 64 && !NORM;
  constexpr bool FUSED = (BIAS == BIAS_NONE || FBIAS) && !NORM;
  constexpr bool NAT = BIAS != BIAS_NONE;
  // in the logits' units; f16 probabilities (largest 65504, smallest normal 2^-14) keep the
  // narrow slack and no overshoot
  constexpr float SLACK = NAT ? (F16 ? RESCALE_SLACK * LN2 : kNatSlack) : RESCALE_SLACK;
  constexpr float OVER = (NAT && !F16) ? kNatOver : 0.f;        // see kNatOver
  // Four statically distinct tile buffers, so that the compiler's wait-count tracking can tell a
  // read of one from a direct load in flight into another.
  __shared__ __align__(16) uint16_t kbuf0[TILE], kbuf1[TILE], vbuf0[TILE], vbuf1[TILE];
  __shared__ __align__(16) float krv_s[NORM ? 2 * BN : 1];
  // FBIAS: the bias of a tile (BM rows x BN keys) reaches LDS by direct loads, two tiles ahead
  // like K, in two buffers. MASK_INFO: the mask words of a partial block's tile, one tile ahead
  // like V, each wave its own 32 rows x 2 words, in two buffers.
  __shared__ __align__(16) uint16_t bbuf0[FBIAS ? BM * BN : 8], bbuf1[FBIAS ? BM * BN : 8];
  __shared__ __align__(16) uint32_t mbuf0[MI ? NT : 1], mbuf1[MI ? NT : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;

  // Workgroup -> (query tile, batch*head). The hardware deals workgroups round-robin over the
  // 8 XCDs (each with its own L2), so with remap every XCD gets a contiguous set of heads.
  // order 0 (head-major): one head's tiles back to back, heaviest causal tile first, so the
  // concurrently running workgroups of an XCD share few K/V heads. order 1 (rank-major, for
  // causal launches): heaviest tiles first, then the next rank, so no heavy tile starts at the
  // end and leaves the chip idle; an XCD takes its heads kGroupHeads at a time (all ranks of one
  // group, then the next group), which keeps fewer heads' K/V live in its L2 at once.
  // order 2: order 0 with the batch innermost (a bias shared by the batches).
  // PACKED: workgroup Hq * i + h takes query tile i of the segments (seg_locate) for head h,
  // and the segment is then a batch of one.
  AttnArgs a = args;
  const int HB = a.Hq * a.B;
  int qt, bh;
  if constexpr (PACKED) {
    SegView sv;
    if (!seg_locate(args, (int)(blockIdx.x / args.Hq), BM, sv)) return;     // workgroup-uniform
    a = seg_args(args, sv);
    // causal: a segment's last tiles attend the most keys, so they go first
    qt = args.causal != SDPA_CAUSAL_NONE ? (sv.q_len + BM - 1) / BM - 1 - sv.tile : sv.tile;
    bh = blockIdx.x % args.Hq;
  } else if (order == 1) {
    if (remap && ((HB >> 3) % kGroupHeads) == 0) {   // HB % 8 == 0, groups of kGroupHeads heads
      const int per_x = HB >> 3, k = blockIdx.x >> 3, gs = kGroupHeads * n_qt;
      const int g = k / gs, r = k % gs;
      qt = n_qt - 1 - r / kGroupHeads;
      bh = (blockIdx.x & 7) * per_x + g * kGroupHeads + r % kGroupHeads;
    } else if (remap) {                           // HB % 8 == 0
      const int per_x = HB >> 3, k = blockIdx.x >> 3;
      qt = n_qt - 1 - k / per_x;
      bh = (blockIdx.x & 7) * per_x + k % per_x;
    } else {
      qt = n_qt - 1 - (int)(blockIdx.x / HB);
      bh = blockIdx.x % HB;
    }
  } else {
    int n = blockIdx.x;
    if (remap) {                                  // gridDim % 8 == 0
      const int per = gridDim.x >> 3;
      n = (n & 7) * per + (n >> 3);
    }
    if (order == 2) {
      // batch innermost: the batches' workgroups of one (head, query tile) run back to back on
      // one XCD, so a bias shared by the batches is read from HBM once and then from L2
      const int bb = n % a.B, r = n / a.B;
      qt = n_qt - 1 - (r % n_qt);
      bh = bb * a.Hq + r / n_qt;
    } else {
      qt = n_qt - 1 - (n % n_qt);
      bh = n / n_qt;
    }
  }
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int q0 = qt * BM;
  const int g = h / (a.Hq / a.Hkv);
  const int nkv = batch_kv_len(a, b);
  const int nq = batch_q_len(a, b);
  const int64_t off = batch_causal_offset(a, b);
  const bool causal = a.causal != SDPA_CAUSAL_NONE;

  const int i_me = q0 + 32 * wave + ql;                  // this lane's query row
  const int row_end = min(q0 + BM, nq);                  // rows below this produce attention output
  const int wave_first = q0 + 32 * wave;
  const int wave_last = min(wave_first + 31, row_end - 1);

  // key limit of the workgroup and of this wave
  int64_t k_end = nkv;
  if (causal) { const int64_t lim = off + (int64_t)(row_end - 1) + 1; if (lim < k_end) k_end = lim; }
  if (row_end <= q0 || k_end < 0) k_end = 0;
  int64_t k_end_w = nkv;
  if (causal) { const int64_t lim = off + (int64_t)wave_last + 1; if (lim < k_end_w) k_end_w = lim; }
  if (wave_last < wave_first || k_end_w < 0) k_end_w = 0;

  // tiles to visit: all tiles below k_end, or the non-empty blocks of the mask info
  int n_tiles = 0, csr_begin = 0, sub_per_blk = 1, sub_shift = 0;
  int64_t info_row = 0;
  // MASK_INFO: lane l holds entry l of the row's CSR (its kv block, that block's class and, for a
  // partial block, its index among the partial blocks), so the tile loop reads them with
  // readlane instead of scalar loads, which would share their wait counter with the LDS reads.
  // Entries from 64 on are loaded where they are used.
  int dn_lane = 0, cls_lane = 0, nx_lane = 0;
  if constexpr (MI) {
    const int mb = a.bm_batch > 1 ? b : 0, mh = a.bm_heads > 1 ? h : 0;
    info_row = ((int64_t)mb * a.bm_heads + mh) * a.bm_nqb + qt;
    csr_begin = a.bm_row_ptr[info_row];
    const int csr_end = a.bm_row_ptr[info_row + 1];
    sub_per_blk = a.bm_bkv / BN;
    if constexpr (MASK == MASK_INFO) sub_shift = __builtin_ctz(sub_per_blk);   // a power of two (host)
    const bool in_row = csr_begin + lane < csr_end;
    if (in_row) {
      dn_lane = a.bm_data_next[csr_begin + lane];
      cls_lane = a.bm_class[info_row * a.bm_nkb + dn_lane];
      if (cls_lane == 1) nx_lane = a.bm_next[info_row * a.bm_nkb + dn_lane];
    }
    // the entries are ascending: those below k_end are a prefix
    int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(in_row && (int64_t)dn_lane * a.bm_bkv < k_end));
    if (MASK == MASK_INFO_LONG && cnt == 64) {
      for (int e = csr_begin + 64; e < csr_end; ++e) {
        if ((int64_t)a.bm_data_next[e] * a.bm_bkv >= k_end) break;
        ++cnt;
      }
    }
    n_tiles = cnt * sub_per_blk;
  } else {
    n_tiles = (int)((k_end + BN - 1) / BN);
  }
  // the CSR entry of tile t and the tile's place in that block (shifts in the short form,
  // where the host has made bkv / BN a power of two)
  auto tile_entry = [&](int t) -> int {
    if constexpr (MASK == MASK_INFO) return t >> sub_shift;
    return t / sub_per_blk;
  };
  auto tile_sub = [&](int t) -> int {
    if constexpr (MASK == MASK_INFO) return t & (sub_per_blk - 1);
    return t % sub_per_blk;
  };
  // kv block of the idx-th non-empty block of the row, and its class (MASK_INFO)
  auto blk_at = [&](int idx) -> int {
    if constexpr (MASK == MASK_INFO) return __builtin_amdgcn_readlane(dn_lane, idx);
    return idx < 64 ? __builtin_amdgcn_readlane(dn_lane, idx) : a.bm_data_next[csr_begin + idx];
  };
  auto cls_at = [&](int idx, int blk) -> int {
    if constexpr (MASK == MASK_INFO) return __builtin_amdgcn_readlane(cls_lane, idx);
    return idx < 64 ? __builtin_amdgcn_readlane(cls_lane, idx) : (int)a.bm_class[info_row * a.bm_nkb + blk];
  };
  auto next_at = [&](int idx, int blk) -> int {
    if constexpr (MASK == MASK_INFO) return __builtin_amdgcn_readlane(nx_lane, idx);
    return idx < 64 ? __builtin_amdgcn_readlane(nx_lane, idx) : a.bm_next[info_row * a.bm_nkb + blk];
  };
  auto tile_k0 = [&](int t) -> int {
    if constexpr (MI) return blk_at(tile_entry(t)) * a.bm_bkv + tile_sub(t) * BN;
    else return t * BN;
  };
  // staging runs ahead of the last tile without branches: past the end it reloads the last tile
  auto tile_k0c = [&](int t) -> int { return tile_k0(t < n_tiles ? t : (n_tiles > 0 ? n_tiles - 1 : 0)); };

  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + g * a.k_sh;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + g * a.v_sh;
  const int k_row_bytes = (int)(a.k_ss * 2), v_row_bytes = (int)(a.v_ss * 2);

  // ---- Q^T operand (stays in registers); rows past Lq load as zeros ------------------------
  bf16x8 qB[DC];
  float c_lane = NAT ? a.scale : a.scale * LOG2E;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(a.q) + b * a.q_sb + h * a.q_sh,
                                                (int64_t)a.Lq * a.q_ss * 2);
    const int qoff = i_me * (int)(a.q_ss * 2) + 16 * hh;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      uint4 x = buf_load16(rq, qoff + 32 * c);
      if constexpr (FUSED) {
        // the scale (times log2e without a bias) folded into Q, rounded to 16 bits once: the
        // q.k MFMAs then emit the logits, and the softmax needs no multiply per score
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w[t] = E::pack(E::lo(w[t]) * c_lane, E::hi(w[t]) * c_lane);
        }
        x = make_uint4(w[0], w[1], w[2], w[3]);
      }
      qB[c] = __builtin_bit_cast(bf16x8, x);
      if constexpr (NORM) {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float lo = E::lo(w[t]), hi = E::hi(w[t]);
          ss += lo * lo + hi * hi;
        }
      }
    }
    if constexpr (NORM) {
      ss += __shfl_xor(ss, 32, 64);
      c_lane *= 1.0f / sqrtf(ss / D + kRmsEps);
    }
    // Q must have landed before the loop: otherwise the wait-count analysis, which cannot tell
    // the loop-invariant Q loads from the per-tile K/V loads, makes every q.k MFMA wait for the
    // next tile's loads and the prefetch stops overlapping the compute.
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- K/V tiles: direct global -> LDS loads --------------------------------------------
  // Instruction u of wave w fills slots 256*u + 64*w + lane of a tile (slot = 16 bytes). K slot
  // (row R, position p) holds chunk p ^ k_swz(R) of key 32*(R/32) + k_row_key(R%32); V slot
  // (row r, position p) holds chunk p ^ v_swz(r) of key r. One buffer resource per operand spans
  // the keys below kv_len, so keys past kv_lengths arrive as zeros (never a poisoned tail); a
  // tile's first key enters the per-lane offset (the host keeps (Lkv + BN) rows of either
  // operand within 32-bit offsets), so a tile costs no address or range arithmetic.
  int kdoff[SPT], vdoff[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int sl = NT * u + tid, row = sl / CPR, pos = sl % CPR;
    kdoff[u] = ((row & ~31) + k_row_key(row & 31)) * k_row_bytes + (pos ^ k_swz<D>(row)) * 16;
    vdoff[u] = row * v_row_bytes + (pos ^ v_swz<D>(row)) * 16;
  }
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp, (int64_t)nkv * k_row_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp, (int64_t)nkv * v_row_bytes);
  auto dma_k = [&](int k0, uint16_t* dst) {
    const int ko = k0 * k_row_bytes;
#pragma unroll
    for (int u = 0; u < SPT; ++u) dma16(rk, dst + 8 * (NT * u + 64 * wave), kdoff[u] + ko);
  };
  auto dma_v = [&](int k0, uint16_t* dst) {
    const int vo = k0 * v_row_bytes;
#pragma unroll
    for (int u = 0; u < SPT; ++u) dma16(rv, dst + 8 * (NT * u + 64 * wave), vdoff[u] + vo);
  };
  // key factors 1/rms of the keys of a tile (QK-norm only): one per thread below BN
  float krv = 0.f;
  auto load_krv = [&](int k0) {
    if constexpr (NORM) {
      if (tid < BN) {
        const int j = k0 + tid;
        krv = j < nkv ? a.k_rinv[((int64_t)b * a.Lkv + j) * a.Hkv + g] : 0.f;
      }
    }
  };
  // K fragment (A operand of S^T = K Q^T): LDS row R = 32*kb + ql, head-dim elements 16*c + 8*hh
  auto kfrag_at = [&](const uint16_t* ks, int c, int kb) -> bf16x8 {
    const int row = 32 * kb + ql;
    return *reinterpret_cast<const bf16x8*>(ks + row * D + (((2 * c + hh) ^ k_swz<D>(row)) << 3));
  };
  // S^T = K Q^T for two 32-key blocks (two independent MFMA chains, interleaved)
  auto compute_s = [&](const uint16_t* ks, f32x16 (&sacc)[2]) {   // sacc holds the start values
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = E::mfma(kfrag_at(ks, c, kb), qB[c], sacc[kb]);
    }
  };
  // V^T fragment (A operand of O^T += V^T P^T) by two transposed reads: within each 16-lane
  // group the read hands lane i the values of 4 rows at the column lane i addresses, so lane L
  // receives V[32*kb + 16*(L/32) + 8*sh + t][32*d + L%32], t = 0..7 -- the keys whose
  // probabilities lane L holds as the B operand.
  const int vr_l = 16 * (lane >> 5) + ((lane & 15) >> 2);          // row within the 8-row step
  const int vc_l = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);        // column within 32 (elements)
  const int vsw = v_swz<D>(vr_l);                                    // same for rows vr_l + 4, + 8k
  // per-lane offsets of the two reads of a fragment, for each 32-column block d. The upper one
  // is hidden from the optimizer: folded back into "lower + 4 rows", its pointer chain grows
  // past what the compiler tracks to keep the buffer's alias information, and every such read
  // would then wait for all direct loads in flight.
  int voff_lo[DB], voff_hi[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    const int col = 32 * d + vc_l;
    voff_lo[d] = vr_l * D + ((((col >> 3) ^ vsw) << 3) | (col & 7));
    voff_hi[d] = voff_lo[d] + 4 * D;
    asm volatile("" : "+v"(voff_hi[d]));
  }
  auto vfrag_at = [&](const uint16_t* vt, int kb, int sh, int d) -> bf16x8 {
    const int rows = (32 * kb + 8 * sh) * D;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vt + (rows + voff_lo[d])));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vt + (rows + voff_hi[d])));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  // Running max m_run (in the logits' units, see NAT) and row sum l_run.
  //  * FUSED: the scores are kept relative to the running max -- the q.k MFMAs start from
  //    -m_run instead of zero, so they emit the logit minus m_run and a probability is one
  //    exp2 (NAT: of that times log2e). m_run starts at 0 with threshold thr = -inf: the first
  //    tile holding an allowed key of a row sets the row's max outright; after that the max
  //    moves only when it grows by more than SLACK.
  //  * otherwise: m_run starts at -inf; any finite logit grows it at once, and until one has
  //    come the probabilities are taken against 0 (every logit so far is -inf).
  float m_run = FUSED ? 0.f : -INFINITY, l_run = 0.f;
  float thr = -INFINITY;
  bool est = false;                                      // LAZY: every row of the wave has its max

  const int64_t bias_row = (BIAS != BIAS_NONE && i_me < a.Lq)
                               ? b * a.bias_sb + h * a.bias_sh + (int64_t)i_me * a.bias_sq : -1;
  const int64_t mask_row = (MASK == MASK_DENSE && i_me < a.Lq)
                               ? b * a.mask_sb + h * a.mask_sh + (int64_t)i_me * a.mask_sq : -1;

  // ---- FBIAS: the bias of a tile through LDS ---------------------------------------------
  // LDS row r holds the tile's 64 keys of query q0 + r, 16-byte chunk c at position c ^ (r & 7),
  // so that the reads below (lanes on consecutive rows, one chunk) hit distinct banks. Each wave
  // loads its own 32 rows (slot 64*u + lane of its 256, u < 4), so it can refill a buffer as
  // soon as its own reads of it are done, without waiting for the other waves: the bias of tile
  // t + 3 is requested in tile t, right after the bias of tile t + 1 has been read, and the
  // end-of-tile wait leaves those four loads in flight. Loads stop at the last element of the
  // last valid row (the buffer range), so rows past Lq and keys past the end read zeros; keys
  // past kv_len in other rows read the next row, and are masked like any key past kv_len.
  int bdoff[FBIAS ? 4 : 1];
  const int bias_row_bytes = (int)(a.bias_sq * 2);
  if constexpr (FBIAS) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sl = 64 * u + lane, row = 32 * wave + (sl >> 3), pos = sl & 7;
      bdoff[u] = row * bias_row_bytes + ((pos ^ (row & 7)) << 4);
    }
  }
  // one buffer resource over the workgroup's bias rows (the host keeps them within 32-bit
  // offsets); a tile's first key enters the per-lane offset
  const int rows_valid = min(BM, a.Lq - q0);
  const __amdgpu_buffer_rsrc_t rbias = [&]() {
    if constexpr (FBIAS)
      return make_rsrc(static_cast<const uint16_t*>(a.bias) + b * a.bias_sb + h * a.bias_sh + (int64_t)q0 * a.bias_sq,
                       (int64_t)(rows_valid - 1) * bias_row_bytes + (int64_t)a.Lkv * 2);
    else
      return make_rsrc(nullptr, 0);
  }();
  auto dma_bias = [&](int k0t, uint16_t* dst) {
    if constexpr (FBIAS) {
#pragma unroll
      for (int u = 0; u < 4; ++u) dma16(rbias, dst + 8 * (256 * wave + 64 * u), bdoff[u] + 2 * k0t);
    }
  };
  // the lane's bias of a tile from LDS: query i_me, keys 32*kb + 16*hh + 0..15 (two chunks)
  auto bias_lds = [&](const uint16_t* bb, uint4 (&x)[2][2]) {
    const int row = 32 * wave + ql;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int c = 4 * kb + 2 * hh;
      x[kb][0] = *reinterpret_cast<const uint4*>(bb + row * BN + ((c ^ (row & 7)) << 3));
      x[kb][1] = *reinterpret_cast<const uint4*>(bb + row * BN + (((c + 1) ^ (row & 7)) << 3));
    }
  };
  // ---- MASK_INFO: the mask words of a partial tile through LDS ------------------------------
  // Wave w's region of a buffer holds, in word ql + 32*k, word k of the tile in row 32*w + ql of
  // the block (its keys 32*k .. 32*k + 31); lane l loads word l of the region.
  auto dma_bits = [&](int u, uint32_t* dst) {
    if constexpr (MI) {
      const int idx = tile_entry(u);
      const int blk = blk_at(idx);
      if (cls_at(idx, blk) == 1) {                       // wave-uniform
        const int wpr = a.bm_bkv / 32;                   // words per block row
        const uint32_t* base = a.bm_bits + (int64_t)next_at(idx, blk) * a.bm_bq * wpr;
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(base, (int64_t)a.bm_bq * wpr * 4);
        const int row = 32 * wave + (lane & 31);
        const int word = tile_sub(u) * (BN / 32) + (lane >> 5);
        dma4(rm, dst + 64 * wave, (row * wpr + word) * 4);
      }
    }
  };
  // start values of an S chain: the bias (FBIAS), -m (other FUSED), 0
  auto s_start = [&](const uint4 (&src)[2][2], float m, f32x16 (&c)[2]) {   // src: the lane's raw bias
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (FBIAS) {
        const uint32_t w[8] = {src[kb][0].x, src[kb][0].y, src[kb][0].z, src[kb][0].w,
                               src[kb][1].x, src[kb][1].y, src[kb][1].z, src[kb][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          c[kb][2 * e] = __uint_as_float(w[e] << 16);
          c[kb][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) c[kb][e] = FUSED ? -m : 0.f;
      }
    }
  };

  // ---- pipeline prologue: K0, V0, K1 in LDS; S(0) formed ----------------------------------
  // K(t) lives in buffer t & 1, V(t) in buffer t & 1; S(t) in s_even (FUSED: s_odd for odd t).
  f32x16 s_even[2], s_odd[2];
  if (n_tiles > 0) {
    dma_bias(tile_k0(0), bbuf0);
    dma_bias(tile_k0c(1), bbuf1);
    dma_bits(0, mbuf0);
    dma_k(tile_k0(0), kbuf0);
    dma_v(tile_k0(0), vbuf0);
    dma_k(tile_k0c(1), kbuf1);
    load_krv(tile_k0(0));
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (NORM) {
      if (tid < BN) krv_s[tid] = krv;
    }
  }
  __syncthreads();
  {
    uint4 bx[2][2];
    if constexpr (FBIAS) {
      if (n_tiles > 0) {
        bias_lds(bbuf0, bx);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);          // this wave's reads of buffer 0 are done
        dma_bias(tile_k0c(2), bbuf0);                    // the bias of tile 2
      }
    }
    if (n_tiles > 0 && tile_k0(0) < k_end_w) {          // m_run = 0: from zero (or the bias)
      s_start(bx, 0.f, s_even);
      compute_s(kbuf0, s_even);
    }
  }
  __syncthreads();                                       // K buffer 0 is refilled in iteration 0

  // ---- one tile; P = t & 1 fixes every buffer's role at compile time -----------------------
  // At the start the direct loads of K(t+2) (into the K buffer freed by K(t), whose scores were
  // formed in the previous iteration) and V(t+1) (into the V buffer freed by V(t-1)) are
  // issued; they land while this tile is computed. The iteration ends with every load of this
  // wave complete and a barrier, so no load is pending across the loop header (the compiler's
  // wait-count tracking is conservative where the header merges its incoming states).
  auto iter = [&](auto PAR_, int t) {
    constexpr int P = decltype(PAR_)::value;
    // FUSED: the two score tiles swap roles every tile; otherwise (more live registers in the
    // bias and norm variants) S(t+1) is copied over S(t) at the end of the tile
    constexpr bool SWAP = FUSED && P;
    f32x16(&s_cur)[2] = SWAP ? s_odd : s_even;          // S(t)
    f32x16(&s_next)[2] = SWAP ? s_even : s_odd;         // S(t+1), formed in block A
    uint16_t* const kfree = P ? kbuf1 : kbuf0;
    const uint16_t* const knext = P ? kbuf0 : kbuf1;
    uint16_t* const vfree = P ? vbuf0 : vbuf1;
    const uint16_t* const vcur = P ? vbuf1 : vbuf0;
    // first keys of tiles t + 1 and t + 2 (with block info each is a CSR lookup): once each
    const int k1 = tile_k0c(t + 1), k2 = tile_k0c(t + 2);
    dma_k(k2, kfree);
    dma_v(k1, vfree);
    load_krv(k1);
    if (t + 1 < n_tiles) dma_bits(t + 1, P ? mbuf0 : mbuf1);   // the buffer tile t - 1's words were read from
    // the bias of tile t + 1 for the start values of S(t+1), requested in tile t - 2; once this
    // wave's reads of it are done, the buffer takes the bias of tile t + 3
    uint4 bx[2][2];
    if constexpr (FBIAS) {
      bias_lds(P ? bbuf0 : bbuf1, bx);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      dma_bias(tile_k0c(t + 3), P ? bbuf0 : bbuf1);
    }
    const int k0 = tile_k0(t);
    if (k0 < k_end_w) {
      // -- element masking, only on tiles that need it --------------------------------------
      // lane (ql, hh) holds, in s_cur[kb][e], the key k0 + 32*kb + 16*hh + e of query i_me
      // edge: some key of the tile lies past kv_lengths or past the causal limit of the wave's
      // first row (wave-uniform)
      const bool edge = (k0 + BN > nkv) || (causal && (int64_t)k0 + BN - 1 > off + wave_first);
      bool need_mask = edge || (MASK == MASK_DENSE);
      int blk_cls = 2;
      if constexpr (MI) {
        const int kb_blk = blk_at(tile_entry(t));          // the block tile t lies in
        blk_cls = cls_at(tile_entry(t), kb_blk);
        if (blk_cls == 1) need_mask = true;
      }
      // logits. FUSED: s is already the logit minus m_run; else s becomes
      // c*r_q*r_k*s + bias, with c = scale (NAT) or scale*log2e.
      if constexpr (!FUSED) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int jb = k0 + 32 * kb + 16 * hh;
#pragma unroll
          for (int e = 0; e < 16; ++e) s_cur[kb][e] *= c_lane;
          if constexpr (NORM) {
            const float4* kq = reinterpret_cast<const float4*>(krv_s + P * BN + 32 * kb + 16 * hh);
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
              const float4 r4 = kq[v4];
              s_cur[kb][4 * v4 + 0] *= r4.x; s_cur[kb][4 * v4 + 1] *= r4.y;
              s_cur[kb][4 * v4 + 2] *= r4.z; s_cur[kb][4 * v4 + 3] *= r4.w;
            }
          }
          if constexpr (BIAS != BIAS_NONE) {
            if (bias_row >= 0) {
              if (a.bias_vec && jb + 16 <= a.Lkv) {
                if constexpr (BIAS == BIAS_BF16) {
                  const uint4* bp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.bias) + bias_row + jb);
                  const uint4 b0 = bp[0], b1 = bp[1];
                  const uint32_t w[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                  for (int e = 0; e < 8; ++e) {
                    s_cur[kb][2 * e] += __uint_as_float(w[e] << 16);
                    s_cur[kb][2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
                  }
                } else {
                  const float4* bp = reinterpret_cast<const float4*>(static_cast<const float*>(a.bias) + bias_row + jb);
#pragma unroll
                  for (int v4 = 0; v4 < 4; ++v4) {
                    const float4 f = bp[v4];
                    s_cur[kb][4 * v4 + 0] += f.x;
                    s_cur[kb][4 * v4 + 1] += f.y;
                    s_cur[kb][4 * v4 + 2] += f.z;
                    s_cur[kb][4 * v4 + 3] += f.w;
                  }
                }
              } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                  if (jb + e < a.Lkv)
                    s_cur[kb][e] += load_elem(a.bias, bias_row + (int64_t)(jb + e) * a.bias_sk, a.bias_dtype);
              }
            }
          }
        }
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int jb = k0 + 32 * kb + 16 * hh;
          uint32_t bits = 0xffffu;
          if constexpr (MASK == MASK_DENSE) {
            bits = 0;
            if (mask_row >= 0 && a.mask_u1) {
              // U1: the 16 keys from jb (a multiple of 16) are 16 bits of one word of the row
              const uint32_t* mw = reinterpret_cast<const uint32_t*>(a.mask) + mask_row;
              if (a.mask_sk == 0) bits = (mw[0] & 1u) ? 0xffffu : 0u;
              else if (jb < a.Lkv) bits = (mw[jb >> 5] >> (jb & 31)) & 0xffffu;
            } else if (mask_row >= 0) {
              const uint8_t* mp = a.mask + mask_row + (int64_t)jb * a.mask_sk;
              if (a.mask_vec && jb + 16 <= a.Lkv) {
                // 16 mask bytes -> 16 bits: in a word x the high bit of each byte of
                // ((x & 0x7f7f7f7f) + 0x7f7f7f7f) | x is set exactly for the nonzero bytes (no
                // byte's sum carries), and the multiply gathers those 4 bits into bits 28..31
                const uint4 m4 = *reinterpret_cast<const uint4*>(mp);
                const uint32_t w[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                  const uint32_t hi8 = (((w[t4] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w[t4]) & 0x80808080u;
                  bits |= ((hi8 * 0x00204081u) >> 28) << (4 * t4);
                }
              } else {
                for (int e = 0; e < 16; ++e)
                  if (jb + e < a.Lkv) bits |= (mp[(int64_t)e * a.mask_sk] != 0) << e;
              }
            }
          } else if constexpr (MI) {
            if (blk_cls == 1) {
              // the tile's words arrived in LDS with the previous iteration's loads
              const uint32_t w = (P ? mbuf1 : mbuf0)[64 * wave + ql + 32 * kb];
              bits = (w >> (16 * hh)) & 0xffffu;
            }
          }
          if (edge) {
            // the keys this row may see are those below min(kv_len, its causal limit + 1): a
            // prefix of the 16 keys from jb
            const int64_t lim = causal ? off + i_me + 1 : (int64_t)nkv;
            const int64_t nk = (lim < nkv ? lim : (int64_t)nkv) - jb;
            bits &= nk >= 16 ? 0xffffu : (nk <= 0 ? 0u : (1u << nk) - 1u);
          }
          // bit e sign-extended is all ones (keep the score) or zero (take -inf): one bit select
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t keep = (uint32_t)((int32_t)(bits << (31 - e)) >> 31);
            const uint32_t x = __float_as_uint(s_cur[kb][e]);
            s_cur[kb][e] = __uint_as_float((x & keep) | (0xff800000u & ~keep));
          }
        }
      }

      // -- online softmax statistics (a row is the lane pair l, l^32) ------------------------
      // The running max m_run (shared by both halves of a row) only moves when a row's max grew
      // by more than RESCALE_SLACK; in between, probabilities may reach 2^RESCALE_SLACK, which
      // fp32 sums and bf16 probabilities hold without loss. Each lane first tests its own 32
      // scores; only when some lane exceeds the slack do the halves exchange maxima (a
      // cross-lane exchange goes through the LDS queue and would drain it every tile).
      // LAZY (fused, no bias, no mask): once the wave is established the max is left to the
      // check of the tile's probability sum below (kLazyBound)
      // (not with a mask: at D = 128 its registers would spill)
      constexpr bool LAZY = FUSED && !NAT && MASK == MASK_NONE;
      float mt = -INFINITY;
      float mL = 0.f;                                    // FBIAS: -m_s * log2e, see below
      if (!LAZY || !est) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s_cur[kb][e]);
      if constexpr (FUSED && NAT) {
        // s_cur holds the logits themselves (the chains start from the bias). Probabilities are
        // taken against m_s, m_run clamped to [-kStartLim, kStartLim], with one fma per score,
        // exp2(s * log2e - m_s * log2e), whose constant is finite because m_s is. off = m_run -
        // m_s is 0 unless the row max lies beyond the clamp; then every tile takes the branch
        // below and moves its scores by off (or to the new max), so that s - m_s is the logit
        // minus m_run. mt (after subtracting m_s) - off is the growth of the row max (thr: see
        // above).
        const float m_s = fminf(fmaxf(m_run, -kStartLim), kStartLim);
        const float off = m_run - m_s;
        mL = -m_s * LOG2E;
        mt -= m_s;
        if (__builtin_amdgcn_ballot_w64(mt - off > thr || off != 0.f)) {
          mt = fmaxf(mt, __shfl_xor(mt, 32, 64));        // row max over both halves
          const bool grow = mt - off > thr;              // thr and off are the same for both halves
          const float dlt = grow ? mt + OVER : off;      // the scores become relative to m_new
          const float m_new = grow ? m_s + mt + OVER : m_run;
          // a row's first keys: nothing accumulated yet (and the exp2 may overflow)
          const float alpha = thr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * LOG2E);
          l_run *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s_cur[kb][e] -= dlt;
          m_run = m_new;
          if (grow) thr = SLACK;
        }
      } else if constexpr (FUSED) {
        // s_cur holds scores minus m_run: mt is the growth of the row max (thr: see above)
        if (__builtin_amdgcn_ballot_w64(mt > thr)) {
          mt = fmaxf(mt, __shfl_xor(mt, 32, 64));        // row max over both halves
          const bool grow = mt > thr;                    // thr is the same for both halves
          const float dlt = grow ? mt : 0.f;
          // a row's first keys: nothing accumulated yet (and exp2(-dlt) may overflow)
          const float alpha = thr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(-dlt);
          l_run *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s_cur[kb][e] -= dlt;
          m_run += dlt;
          if (grow) thr = SLACK;
        }
      } else if (__builtin_amdgcn_ballot_w64(mt > m_run + SLACK)) {
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));          // row max over both halves
        const bool grow = mt > m_run + SLACK;
        const float m_new = grow ? mt + OVER : m_run;
        // 0 on a row's first finite logit (m_run = -inf)
        const float alpha = __builtin_amdgcn_exp2f(NAT ? (m_run - m_new) * LOG2E : m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
        m_run = m_new;
      }
      if constexpr (LAZY) est = __builtin_amdgcn_ballot_w64(thr == -INFINITY) == 0;
      }
      // no finite logit yet: every logit so far is -inf, and exp2(-inf - 0) = 0 (not NaN)
      const float m_use = m_run == -INFINITY ? 0.f : m_run;

      // -- the tile body, in chunks the compiler may not reorder across ---------------------
      // The matrix cores and the VALU only run side by side when their instructions alternate
      // in program order, so the body is cut into chunks fenced by sched_barrier(0):
      //   A  (DC chunks): 2 MFMAs of S(t+1) = K(t+1) Q^T, and 24 of the 32 probabilities of S(t)
      //   B1 (2*DB chunks): 1 MFMA of O += V P for keys 0..31 of the tile, and the last 8
      //      probabilities (keys 32..63, needed only by B2)
      //   B2 (2*DB chunks): 1 MFMA of O += V P for keys 32..63, and the staging of K(t+2),
      //      V(t+1) into LDS and the loads of K(t+3), V(t+2)
      // Each chunk also issues the LDS fragment read of the next chunk.
      constexpr int NA = DC, NB = 2 * DB;
      // LAZY: all 32 probabilities in block A, so that the tile's sum is checked before B1
      constexpr int EL_A = LAZY ? 32 : 24, EL_B = 32 - EL_A;
      float l_tile = 0.f;                                // LAZY: this tile's share of l_run
      float pf[32];                                      // probabilities of this lane's 32 keys
      uint32_t pw[16];                                   // the same, packed as bf16 pairs
      auto prob = [&](int f) {                           // element f = 16*kb + 8*sh + e
        const float xe = s_cur[f >> 4][f & 15];
        // NAT: the max is subtracted in natural units first (no overflow), then scaled
        float x2;
        if constexpr (FUSED) x2 = NAT ? fmaf(xe, LOG2E, mL) : xe;
        else x2 = NAT ? (xe - m_use) * LOG2E : xe - m_use;
        pf[f] = __builtin_amdgcn_exp2f(x2);
        if (f & 1) {
          pw[f >> 1] = E::pack(pf[f - 1], pf[f]);
          // row sum of the same 16-bit probabilities the MFMA consumes
          if constexpr (LAZY) l_tile = E::sum2(pw[f >> 1], l_tile);
          else l_run = E::sum2(pw[f >> 1], l_run);
        }
      };
      auto pb = [&](int kb, int sh) -> bf16x8 {
        const uint4 w = make_uint4(pw[8 * kb + 4 * sh + 0], pw[8 * kb + 4 * sh + 1], pw[8 * kb + 4 * sh + 2],
                                   pw[8 * kb + 4 * sh + 3]);
        return __builtin_bit_cast(bf16x8, w);
      };
      auto kfrag = [&](int c, int kb) { return kfrag_at(knext, c, kb); };
      auto vfrag = [&](int i) {                          // i = (kb*2 + sh)*DB + d
        return vfrag_at(vcur, i / (2 * DB), (i / DB) & 1, i % DB);
      };

      // LDS fragments are read PF chunks ahead of the MFMA that consumes them
      constexpr int PF = 2;
      bf16x8 kf[PF + 1][2];
#pragma unroll
      for (int c = 0; c < PF; ++c) {
        kf[c][0] = kfrag(c, 0);
        kf[c][1] = kfrag(c, 1);
      }
      // the C operand that starts S(t+1): zero, -m_run broadcast (FUSED), or the bias (FBIAS:
      // one start vector per 32-key block, the bias of tile t + 1). Built here, after the first
      // fragment reads are under way, from an opaque copy of m_run, so that its 16 registers
      // live only until the first two MFMAs.
      f32x16 c0[FBIAS ? 2 : 1];
      {
        float m0 = m_run;
        if constexpr (FUSED) asm volatile("" : "+v"(m0));
        if constexpr (FBIAS) {
          s_start(bx, m0, c0);
        } else if constexpr (FUSED) {
          // -m broadcast as eight 64-bit pairs (64-bit moves: half the instructions)
          const uint32_t nm = __float_as_uint(-m0);
          const uint64_t pr = ((uint64_t)nm << 32) | nm;
          uint64_t cu[8];
          cu[0] = pr;
#pragma unroll
          for (int e = 1; e < 8; ++e) asm volatile("v_mov_b64 %0, %1" : "=v"(cu[e]) : "v"(pr));
          c0[0] = __builtin_bit_cast(f32x16, cu);
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) c0[0][e] = 0.f;
        }
      }
      bf16x8 vf[PF + 1];
#pragma unroll
      for (int c = 0; c < NA; ++c) {                     // ---- block A
        if (c + PF < NA) {
          kf[(c + PF) % (PF + 1)][0] = kfrag(c + PF, 0);
          kf[(c + PF) % (PF + 1)][1] = kfrag(c + PF, 1);
        } else {
          vf[(c + PF - NA) % (PF + 1)] = vfrag(c + PF - NA);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (c == 0) {
            s_next[kb] = E::mfma(kf[0][kb], qB[0], c0[FBIAS ? kb : 0]);
          } else {
            s_next[kb] = E::mfma(kf[c % (PF + 1)][kb], qB[c], s_next[kb]);
          }
        }
#pragma unroll
        for (int f = c * EL_A / NA; f < (c + 1) * EL_A / NA; ++f) prob(f);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (LAZY) {
        // an established row's max moves only when a probability of this tile grew past 2^64
        // (the tile's sum shows it, inf included); the tile is then taken again against the
        // new max before its probabilities reach the P.V products, and S(t+1) is moved too
        if (est && __builtin_amdgcn_ballot_w64(!(l_tile <= kLazyBound))) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s_cur[kb][e]);
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float lt_row = l_tile + __shfl_xor(l_tile, 32, 64);
          const float dlt = !(lt_row <= kLazyBound) ? mx : 0.f;
          const float alpha = __builtin_amdgcn_exp2f(-dlt);
          l_run *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
          // S(t+1), formed in block A, started from the old max: it moves with it
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              s_cur[kb][e] -= dlt;
              s_next[kb][e] -= dlt;
            }
          m_run += dlt;
          l_tile = 0.f;
#pragma unroll
          for (int f = 0; f < 32; ++f) prob(f);
        }
        l_run += l_tile;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {                     // ---- block B1: keys 0..31
        vf[(i + PF) % (PF + 1)] = vfrag(i + PF);
        o[i % DB] = E::mfma(vf[i % (PF + 1)], pb(0, i / DB), o[i % DB]);
#pragma unroll
        for (int f = EL_A + i * EL_B / NB; f < EL_A + (i + 1) * EL_B / NB; ++f) prob(f);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {                     // ---- block B2: keys 32..63
        if (i + PF < NB) vf[(NB + i + PF) % (PF + 1)] = vfrag(NB + i + PF);
        o[i % DB] = E::mfma(vf[(NB + i) % (PF + 1)], pb(1, i / DB), o[i % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!FUSED) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_next[kb];
      }
    }
    // this wave's loads have landed, except (FBIAS) the four bias loads of tile t + 3, issued
    // after all others of this tile (a load's count retires in issue order); with those in
    // flight the barrier is a bare s_barrier, since a fenced one waits for every load
    if constexpr (FBIAS) {
      __builtin_amdgcn_s_waitcnt(kWaitVm4Lgkm0);
      __builtin_amdgcn_s_barrier();
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      if constexpr (NORM) {
        if (tid < BN) krv_s[(1 - P) * BN + tid] = krv;
      }
      __syncthreads();
    }
  };
  std::integral_constant<int, 0> I0;
  std::integral_constant<int, 1> I1;
  for (int t = 0; t < n_tiles; t += 2) {
    iter(I0, t);
    if (t + 1 >= n_tiles) break;
    iter(I1, t + 1);
  }
  // FBIAS: the last bias loads are still in flight; no direct load may land in LDS after the
  // workgroup has ended
  if constexpr (FBIAS) __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue: O / l; NaN for rows without keys; 0 past q_lengths -------------------------
  if (i_me >= a.Lq) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool zero_row = i_me >= nq;
  const float inv = zero_row ? 0.f : (l_tot > 0.f ? 1.0f / l_tot : NAN);
  if (a.lse && hh == 0) {
    // m_run is in the logits' units (natural with a bias, else log2), l_run relative to it
    a.lse[b * a.lse_sb + h * a.lse_sh + i_me] =
        (zero_row || !(l_tot > 0.f)) ? -INFINITY
                                     : (NAT ? m_run + __log2f(l_tot) * LN2 : (m_run + __log2f(l_tot)) * LN2);
  }
  const int64_t orow = b * a.o_sb + (int64_t)i_me * a.o_ss + h * a.o_sh;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dcol = 32 * d + 8 * i + 4 * hh;
      float r[4];
      // inv is NaN for a row without keys, so the product is too
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = zero_row ? 0.f : o[d][4 * i + j] * inv;
      if (a.out_dtype == SDPA_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + dcol) = make_float4(r[0], r[1], r[2], r[3]);
      } else if (a.out_dtype == SDPA_F16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + dcol) =
            make_uint2(In<true>::pack(r[0], r[1]), In<true>::pack(r[2], r[3]));
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + dcol) =
            make_uint2(In<false>::pack(r[0], r[1]), In<false>::pack(r[2], r[3]));
      }
    }
}

template <int D, int BIAS, int MASK, bool NORM, bool F16>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  if constexpr (BIAS == BIAS_NONE && MASK == MASK_NONE) {
    if (a.q_seg) {
      const int64_t nwg = packed_tiles_bound(a, BM) * a.Hq;
      if (nwg <= 0) return hipSuccess;
      hipLaunchKernelGGL((fwd_mfma_kernel<D, BIAS, MASK, NORM, F16, true>), dim3((unsigned)nwg), dim3(NT), 0, s,
                         a, 0, 0, 0);
      return hipGetLastError();
    }
  }
  const int n_qt = (a.Lq + BM - 1) / BM;
  const int64_t nwg = (int64_t)n_qt * a.Hq * a.B;
  // causal: longest tiles first across heads; a bias broadcast over several batches: batch
  // innermost (L2 sharing of the bias); otherwise one head's tiles back to back
  const int order = a.causal != SDPA_CAUSAL_NONE ? 1 : ((a.bias && a.bias_sb == 0 && a.B > 1) ? 2 : 0);
  const int remap = order == 1 ? ((a.Hq * a.B) % 8 == 0 ? 1 : 0) : (nwg % 8) == 0 ? 1 : 0;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, BIAS, MASK, NORM, F16, false>), dim3((unsigned)nwg), dim3(NT), 0, s, a, n_qt,
                     remap, order);
  return hipGetLastError();
}

template <int D, int BIAS, int MASK, bool NORM>
hipError_t launch_in(const AttnArgs& a, hipStream_t s) {
  if (a.in_dtype == SDPA_F16) return launch_t<D, BIAS, MASK, NORM, true>(a, s);
  return launch_t<D, BIAS, MASK, NORM, false>(a, s);
}

template <int D, int BIAS, int MASK>
hipError_t launch_norm(const AttnArgs& a, hipStream_t s) {
  if (a.qk_norm) return launch_in<D, BIAS, MASK, true>(a, s);
  return launch_in<D, BIAS, MASK, false>(a, s);
}

template <int D, int BIAS>
hipError_t launch_mask(const AttnArgs& a, hipStream_t s) {
  if (a.bm_class) {
    const int sub = a.bm_bkv / BN;
    if (a.bm_nkb <= 64 && (sub & (sub - 1)) == 0) return launch_norm<D, BIAS, MASK_INFO>(a, s);
    return launch_norm<D, BIAS, MASK_INFO_LONG>(a, s);
  }
  if (a.mask) return launch_norm<D, BIAS, MASK_DENSE>(a, s);
  return launch_norm<D, BIAS, MASK_NONE>(a, s);
}

template <int D>
hipError_t launch_bias(const AttnArgs& args, hipStream_t s) {
  if (!args.bias) return launch_mask<D, BIAS_NONE>(args, s);
  if (args.bias_dtype == SDPA_BF16) {
    // the fused bias at D = 64 (no QK-norm) reaches LDS by direct loads: it needs rows of
    // 16-byte runs and a 128-row span within 32-bit offsets; any other bf16 bias is read element
    // by element (the per-element path, which takes any dtype)
    const bool dma_ok = args.bias_vec && (int64_t)(BM - 1) * args.bias_sq * 2 + (int64_t)args.Lkv * 2 <= INT32_MAX;
    if (D != 64 || args.qk_norm || dma_ok) return launch_mask<D, BIAS_BF16>(args, s);
    AttnArgs a = args;
    a.bias_vec = 0;
    return launch_mask<D, BIAS_F32>(a, s);
  }
  return launch_mask<D, BIAS_F32>(args, s);
}

bool al(const void* p, int n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

bool fwd_mfma_supports(const AttnArgs& a) {
  if ((a.in_dtype != SDPA_BF16 && a.in_dtype != SDPA_F16) || a.D != a.Dv || (a.D != 64 && a.D != 128)) return false;
  if (a.bias && a.bias_dtype == SDPA_F16) return false;     // f16 bias: the general kernel
  if (!al(a.q, 16) || !al(a.k, 16) || !al(a.v, 16) || !al(a.out, 16)) return false;
  if ((a.q_sb | a.q_ss | a.q_sh | a.k_sb | a.k_ss | a.k_sh | a.v_sb | a.v_ss | a.v_sh) & 7) return false;
  if ((a.o_sb | a.o_ss | a.o_sh) & 3) return false;
  if (a.bm_class && (a.bm_bq != BM || a.bm_bkv % BN)) return false;
  // the softmax takes the row max on raw scores scaled once: the scale must be positive
  if (!(a.scale > 0.f)) return false;
  // buffer loads: rows at least head_dim long, 32-bit byte ranges per (batch, head) slice
  if (a.q_ss < a.D || a.k_ss < a.D || a.v_ss < a.D) return false;
  // (K and V: a tile's row offset is added to offsets within the tile, up to Lkv + BN rows)
  if ((int64_t)a.Lq * a.q_ss * 2 > INT32_MAX || ((int64_t)a.Lkv + BN) * a.k_ss * 2 > INT32_MAX ||
      ((int64_t)a.Lkv + BN) * a.v_ss * 2 > INT32_MAX)
    return false;
  if (a.q_seg && (a.bias || a.mask || a.bm_class)) return false;
  const int64_t nwg = (a.q_seg ? packed_tiles_bound(a, BM) : (int64_t)((a.Lq + BM - 1) / BM) * a.B) * a.Hq;
  return nwg > 0 && nwg < (int64_t)INT32_MAX;
}

hipError_t launch_fwd_mfma(const AttnArgs& args, hipStream_t s) {
  AttnArgs a = args;
  // 16-byte loads of 16 consecutive keys need unit key stride and 16-byte aligned runs
  const int per16 = a.bias_dtype == SDPA_BF16 ? 8 : 4;
  a.bias_vec = a.bias && a.bias_sk == 1 && al(a.bias, 16) && (a.bias_sb % per16) == 0 &&
               (a.bias_sh % per16) == 0 && (a.bias_sq % per16) == 0;
  a.mask_vec = a.mask && !a.mask_u1 && a.mask_sk == 1 && al(a.mask, 16) && (a.mask_sb % 16) == 0 &&
               (a.mask_sh % 16) == 0 && (a.mask_sq % 16) == 0;
  if (a.D == 128) return launch_bias<128>(a, s);
  return launch_bias<64>(a, s);
}

}  // namespace sdpa
