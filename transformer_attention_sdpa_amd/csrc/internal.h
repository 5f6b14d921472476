// internal.h -- argument blocks and launchers shared between the C-ABI layer (api.hip) and the
// kernel files. Not installed; the public interface is include/sdpa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "sdpa.h"

namespace sdpa {

// Everything an attention kernel reads, resolved on the host from the sdpa_tensor descriptors.
// Strides are in elements; head_dim has stride 1 for q/k/v/out. Broadcast dims of bias/mask
// carry stride 0.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int B, Lq, Lkv, Hq, Hkv, D, Dv;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int in_dtype, out_dtype;

  const void* bias;            // nullptr: no bias
  int bias_dtype;
  int64_t bias_sb, bias_sh, bias_sq, bias_sk;

  const uint8_t* mask;         // dense mask (nullptr: none, or block info in use)
  int64_t mask_sb, mask_sh, mask_sq, mask_sk;   // U1: sb/sh/sq in 32-bit words, sk 0 or 1 (bits)
  int mask_u1;                 // 1: the mask is U1 bits (see include/sdpa.h), 0: U8 bytes

  const int8_t* bm_class;      // block mask info (nullptr: none)
  const int32_t* bm_next;
  const int32_t* bm_row_ptr;
  const int32_t* bm_data_next;
  const uint32_t* bm_bits;
  int bm_batch, bm_heads, bm_nqb, bm_nkb, bm_bq, bm_bkv;

  float scale;
  int causal;                  // sdpa_causal
  int bias_vec, mask_vec;      // 1: bias/mask rows allow 16-byte vector loads (set by the MFMA launcher)
  const int32_t* q_offset;     int q_offset_all;
  const int32_t* kv_lengths;   int kv_length_all;   // < 0: none
  const int32_t* q_lengths;    int q_length_all;    // < 0: none
  int qk_norm;
  const float* k_rinv;         // [B][Lkv][Hkv]: 1/rms of each key head vector (qk_norm only)

  // packed sequences (B == 1): segment s of the queries attends segment s of the keys/values;
  // q_offset, q_lengths and kv_lengths then hold one entry per segment. nullptr: batched.
  const int32_t* q_seg;        // [n_seg] lengths along q
  const int32_t* kv_seg;       // [n_seg] lengths along k/v
  int n_seg;
  int seg_maxlen;              // bound on the segment lengths from the caller, or -1 (host use)

  // log-sum-exp output (natural log) of every query row, or nullptr: lse[b*lse_sb + h*lse_sh + i]
  float* lse;
  int64_t lse_sb, lse_sh;
};

struct DecodeArgs {
  const void* q;               // [B][T][Hq][D]
  const void* k;               // [B][cap][Hkv][D]
  const void* v;
  void* out;                   // [B][T][Hq][D]
  int B, T, Hq, Hkv, D, cap;   // T: query tokens per sequence (the last T of its kv_lengths[b] keys)
  int64_t q_sb, q_ss, q_sh, k_sb, k_ss, k_sh, v_sb, v_ss, v_sh, o_sb, o_ss, o_sh;
  int in_dtype, out_dtype;
  const int32_t* kv_lengths;
  float scale_log2;            // scale * log2(e)
  int split_len, max_splits;
  float* part_o;               // [B][T][Hq][max_splits][D]
  float* part_ml;              // [B][T][Hq][max_splits][2]: running max (log2 units), sum
};

struct MaskInfoArgs {
  const uint8_t* mask;
  int64_t sb, sh, sq, sk;      // U1: sb/sh/sq in 32-bit words, sk 0 or 1 (bits)
  int u1;                      // 1: U1 bits, 0: U8 bytes
  int vec16;                   // U8 rows allow 16-byte loads (aligned base and strides, unit column stride)
  int Mb, Mh, Lq, Lkv, bq, bkv, n_qb, n_kb;
  int8_t* cls;
  int32_t* next;
  int32_t* row_ptr;
  int32_t* data_next;
  uint32_t* bits;
  int32_t* n_partial;
};

// The backward pass: the forward's arguments (a.out is the forward output O, read only) plus
// the output cotangent, the saved log-sum-exp, the gradients and the workspace rows.
struct BwdArgs {
  AttnArgs a;
  const void* dout;            // [B][Lq][Hq][Dv]
  int64_t do_sb, do_ss, do_sh;
  int do_dtype;
  const float* lse;            // [B][Hq][Lq] natural log, from the forward
  void* dq;                    // [B][Lq][Hq][D]
  void* dk;                    // [B][Lkv][Hkv][D]
  void* dv;                    // [B][Lkv][Hkv][Dv]
  int64_t dq_sb, dq_ss, dq_sh, dk_sb, dk_ss, dk_sh, dv_sb, dv_ss, dv_sh;
  int dq_dtype, dk_dtype, dv_dtype;
  float* dscale;               // one float, or nullptr
  // workspace rows, [B][Hq][Lq] each: D = rowsum(dO * O) (0 for rows that take no part), the lse
  // of rows that take part (+inf for the others, so that every weight of such a row is 0), and
  // each row's share of dscale. On the matrix-core route (stat_mfma) the first two hold -D and
  // -lse / scale (-inf for rows that take no part; scale > 0 there): the start values of that
  // route's S and dP products, taken as they are.
  float* w_dsum;
  float* w_lse;
  float* w_dsc;
  double* w_dsc2;              // first-stage sums of w_dsc (or of w_dsp)
  // Stored-dS route (matrix-core kernels, no block info), else nullptr: the dK/dV pass writes
  // every dS tile it forms, 16-bit, as tiles of 128 keys x 64 queries (queries contiguous, key
  // rows of 128 bytes) indexed [B][Hq][ceil(Lq/64)][ceil(Lkv/128)], and its workgroups' shares
  // of dscale (8 floats each, w_dsp); the dQ pass then reads dS instead of forming S and dP again.
  uint16_t* w_ds;
  float* w_dsp;
  double* w_dsc2_ds;           // first-stage sums of w_dsp
};

// Workgroups of the dK/dV pass (128 keys of one K/V head each) and their dscale shares (8 each)
inline int64_t bwd_dkdv_workgroups(int64_t B, int64_t Hkv, int64_t Lkv) { return B * Hkv * ((Lkv + 127) / 128); }

// Stored-dS route: bytes of the dS tiles (0 where the route does not apply: 16-bit inputs,
// D == Dv in {64, 128}) and the cap above which the gradient forms S and dP again in its dQ pass
constexpr int64_t kDsCapBytes = (int64_t)8 << 30;
inline int64_t bwd_ds_tile_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t Lkv, int64_t D, int64_t Dv, int dtype) {
  if ((dtype != SDPA_BF16 && dtype != SDPA_F16) || D != Dv || (D != 64 && D != 128) || B <= 0 || Hq <= 0 ||
      Lq <= 0 || Lkv <= 0)
    return 0;
  // the dQ pass reads a query tile's row of dS tiles with 32-bit offsets (at most 65536 tiles)
  if ((Lkv + 127) / 128 > 65536) return 0;
  const int64_t n = B * Hq * ((Lq + 63) / 64) * ((Lkv + 127) / 128) * (64 * 128 * 2);
  return n <= kDsCapBytes ? n : 0;
}

constexpr float kRmsEps = 1e-6f;

// Query tiles of `tile` rows over all segments of a packed launch, at most: every segment adds
// at most one partial tile, and none has more than the caller's maxlen rows. Host only.
inline int64_t packed_tiles_bound(const AttnArgs& a, int tile) {
  int64_t n = ((int64_t)a.Lq + tile - 1) / tile + a.n_seg;
  if (a.seg_maxlen >= 0) {
    const int64_t m = (int64_t)a.n_seg * ((a.seg_maxlen + tile - 1) / tile);
    if (m < n) n = m;
  }
  return n;
}

// Launchers (each returns hipSuccess or the launch error).
hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t s);
bool fwd_mfma_supports(const AttnArgs& a);
hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_row_rinv(const void* x, int dtype, int64_t sb, int64_t ss, int64_t sh, int B, int L,
                           int H, int D, float eps, float* rinv, hipStream_t s);
hipError_t launch_head_rms_norm(const void* x, void* y, int dtype, int64_t xsb, int64_t xss, int64_t xsh,
                                int64_t ysb, int64_t yss, int64_t ysh, int B, int T, int H, int Dh,
                                float eps, hipStream_t s);
bool decode_fast_supports(const DecodeArgs& a, int in_dtype);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_kv_cache_update(void* kc, void* vc, const void* kn, const void* vn, int elem_bytes,
                                  int B, int T, int H, int D, int cap,
                                  int64_t kc_sb, int64_t kc_ss, int64_t kc_sh,
                                  int64_t vc_sb, int64_t vc_ss, int64_t vc_sh,
                                  int64_t kn_sb, int64_t kn_ss, int64_t kn_sh,
                                  int64_t vn_sb, int64_t vn_ss, int64_t vn_sh,
                                  const int32_t* write_index, hipStream_t s);
hipError_t launch_mask_info(const MaskInfoArgs& m, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& g, hipStream_t s);
// whether the gradient runs on the matrix-core kernels (else the fp32 ones)
bool bwd_mfma_supports(const BwdArgs& g);
hipError_t launch_measure_mfma(int workgroups, int iters, float* sink, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s);
hipError_t launch_debug_allowed(const AttnArgs& a, uint8_t* out, int64_t sb, int64_t sh, int64_t sq,
                                int64_t sk, hipStream_t s);

}  // namespace sdpa
