// api.hip -- the extern "C" entry points of include/sdpa.h: argument validation on the host,
// resolution of the sdpa_tensor descriptors into kernel argument blocks, and dispatch.
//
// Validation touches no GPU state, so every error path can be exercised without a device.
// Nothing here allocates, synchronizes or reads a device array.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "internal.h"

using namespace sdpa;

namespace {

thread_local std::string g_err;

sdpa_status fail(sdpa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

sdpa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SDPA_OK;
  return fail(SDPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_float(int dt) { return dt == SDPA_F32 || dt == SDPA_BF16 || dt == SDPA_F16; }

bool dims_ok(const sdpa_tensor* t) {
  for (int i = 0; i < 4; ++i)
    if (t->dims[i] < 0 || t->dims[i] > INT32_MAX) return false;
  return true;
}

int64_t numel(const sdpa_tensor* t) { return t->dims[0] * t->dims[1] * t->dims[2] * t->dims[3]; }

// A bias/mask descriptor {Lkv|1, Lq|1, H|1, B|1}: checks the dims and returns strides with 0
// on broadcast dims, in (b, h, q, k) order.
sdpa_status bcast_strides(const sdpa_tensor* t, const char* name, int64_t Lkv, int64_t Lq, int64_t H,
                          int64_t B, int64_t st[4]) {
  const int64_t full[4] = {Lkv, Lq, H, B};
  for (int i = 0; i < 4; ++i) {
    if (t->dims[i] != 1 && t->dims[i] != full[i])
      return fail(SDPA_ERR_SHAPE, "%s dim %d is %lld; it must be 1 or %lld", name, i, (long long)t->dims[i],
                  (long long)full[i]);
  }
  st[0] = t->dims[3] == 1 ? 0 : t->strides[3];
  st[1] = t->dims[2] == 1 ? 0 : t->strides[2];
  st[2] = t->dims[1] == 1 ? 0 : t->strides[1];
  st[3] = t->dims[0] == 1 ? 0 : t->strides[0];
  return SDPA_OK;
}

// Shared resolution of sdpa_fwd / sdpa_debug_allowed_mask arguments. `v` and `out` may be NULL
// (debug export).
sdpa_status resolve_attention(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                              const sdpa_tensor* bias, const sdpa_tensor* mask,
                              const sdpa_block_mask_info* mi, float scale, int32_t is_causal,
                              const int32_t* q_offset, int32_t q_offset_all, const int32_t* kv_lengths,
                              int32_t kv_length_all, const int32_t* q_lengths, int32_t q_length_all,
                              int32_t qk_norm, const sdpa_tensor* out, AttnArgs& a) {
  std::memset(&a, 0, sizeof a);
  if (!q || !k) return fail(SDPA_ERR_NULL, "q and k descriptors are required");
  if (!dims_ok(q) || !dims_ok(k) || (v && !dims_ok(v)) || (out && !dims_ok(out)))
    return fail(SDPA_ERR_SHAPE, "a dim is negative or exceeds int32");
  if (!is_float(q->dtype) || k->dtype != q->dtype || (v && v->dtype != q->dtype))
    return fail(SDPA_ERR_DTYPE, "q, k and v must share one dtype: F32, BF16 or F16");
  if (out && !is_float(out->dtype)) return fail(SDPA_ERR_DTYPE, "out must be F32, BF16 or F16");
  const int64_t D = q->dims[0], Hq = q->dims[1], Lq = q->dims[2], B = q->dims[3];
  const int64_t Hkv = k->dims[1], Lkv = k->dims[2];
  if (D < 1) return fail(SDPA_ERR_SHAPE, "head_dim must be at least 1");
  if (k->dims[0] != D) return fail(SDPA_ERR_SHAPE, "q and k head dims differ (%lld vs %lld)", (long long)D,
                                   (long long)k->dims[0]);
  if (k->dims[3] != B) return fail(SDPA_ERR_SHAPE, "q and k batch sizes differ");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv)
    return fail(SDPA_ERR_SHAPE, "query heads (%lld) must be a positive multiple of key/value heads (%lld)",
                (long long)Hq, (long long)Hkv);
  int64_t Dv = D;
  if (v) {
    Dv = v->dims[0];
    if (Dv < 1) return fail(SDPA_ERR_SHAPE, "v head_dim must be at least 1");
    if (v->dims[1] != Hkv || v->dims[2] != Lkv || v->dims[3] != B)
      return fail(SDPA_ERR_SHAPE, "k and v must agree in heads, length and batch");
    if (v->strides[0] != 1) return fail(SDPA_ERR_SHAPE, "v needs head_dim stride 1");
  }
  if (out) {
    if (out->dims[0] != Dv || out->dims[1] != Hq || out->dims[2] != Lq || out->dims[3] != B)
      return fail(SDPA_ERR_SHAPE, "out must be {v_head_dim, Hq, Lq, B}");
    if (out->strides[0] != 1) return fail(SDPA_ERR_SHAPE, "out needs head_dim stride 1");
  }
  if (q->strides[0] != 1 || k->strides[0] != 1) return fail(SDPA_ERR_SHAPE, "q and k need head_dim stride 1");
  if (is_causal < SDPA_CAUSAL_NONE || is_causal > SDPA_CAUSAL_BOTTOM_RIGHT)
    return fail(SDPA_ERR_SHAPE, "is_causal must be 0, 1 or 2");
  if (qk_norm != 0 && qk_norm != 1) return fail(SDPA_ERR_SHAPE, "qk_norm must be 0 or 1");
  if (D > 256 || Dv > 256) return fail(SDPA_ERR_UNSUPPORTED, "head dims above 256 have no kernel");

  a.q = q->data; a.k = k->data; a.v = v ? v->data : nullptr; a.out = out ? out->data : nullptr;
  a.B = (int)B; a.Lq = (int)Lq; a.Lkv = (int)Lkv; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.D = (int)D; a.Dv = (int)Dv;
  a.q_sb = q->strides[3]; a.q_ss = q->strides[2]; a.q_sh = q->strides[1];
  a.k_sb = k->strides[3]; a.k_ss = k->strides[2]; a.k_sh = k->strides[1];
  if (v) { a.v_sb = v->strides[3]; a.v_ss = v->strides[2]; a.v_sh = v->strides[1]; }
  if (out) { a.o_sb = out->strides[3]; a.o_ss = out->strides[2]; a.o_sh = out->strides[1]; a.out_dtype = out->dtype; }
  a.in_dtype = q->dtype;

  if (bias) {
    if (!is_float(bias->dtype)) return fail(SDPA_ERR_DTYPE, "bias must be F32, BF16 or F16");
    if (!dims_ok(bias)) return fail(SDPA_ERR_SHAPE, "bias dims out of range");
    int64_t st[4];
    sdpa_status s = bcast_strides(bias, "bias", Lkv, Lq, Hq, B, st);
    if (s != SDPA_OK) return s;
    a.bias = bias->data; a.bias_dtype = bias->dtype;
    a.bias_sb = st[0]; a.bias_sh = st[1]; a.bias_sq = st[2]; a.bias_sk = st[3];
    if (!a.bias && numel(bias) > 0) return fail(SDPA_ERR_NULL, "bias data is NULL");
  }
  if (mi) {
    if (mi->mask_batch != 1 && mi->mask_batch != B) return fail(SDPA_ERR_SHAPE, "mask_info batch must be 1 or B");
    if (mi->mask_heads != 1 && mi->mask_heads != Hq) return fail(SDPA_ERR_SHAPE, "mask_info heads must be 1 or Hq");
    if (mi->q_len != Lq || mi->kv_len != Lkv) return fail(SDPA_ERR_SHAPE, "mask_info was built for other lengths");
    if (mi->bq < 1 || mi->bkv < 32 || mi->bkv % 32 ||
        mi->n_qb != (Lq + mi->bq - 1) / mi->bq || mi->n_kb != (Lkv + mi->bkv - 1) / mi->bkv)
      return fail(SDPA_ERR_SHAPE, "mask_info block grid is inconsistent");
    if (!mi->block_mask || !mi->mask_next || !mi->row_ptr || !mi->data_next || !mi->partial_bits)
      return fail(SDPA_ERR_NULL, "mask_info pointers are NULL");
    a.bm_class = mi->block_mask; a.bm_next = mi->mask_next; a.bm_row_ptr = mi->row_ptr;
    a.bm_data_next = mi->data_next; a.bm_bits = mi->partial_bits;
    a.bm_batch = mi->mask_batch; a.bm_heads = mi->mask_heads; a.bm_nqb = mi->n_qb; a.bm_nkb = mi->n_kb;
    a.bm_bq = mi->bq; a.bm_bkv = mi->bkv;
  } else if (mask) {
    if (mask->dtype != SDPA_U8 && mask->dtype != SDPA_U1) return fail(SDPA_ERR_DTYPE, "mask must be U8 or U1");
    if (!dims_ok(mask)) return fail(SDPA_ERR_SHAPE, "mask dims out of range");
    if (mask->dtype == SDPA_U1 && mask->dims[0] != 1 && mask->strides[0] != 1)
      return fail(SDPA_ERR_SHAPE, "a U1 mask needs its elements contiguous (strides[0] == 1)");
    int64_t st[4];
    sdpa_status s = bcast_strides(mask, "mask", Lkv, Lq, Hq, B, st);
    if (s != SDPA_OK) return s;
    a.mask = static_cast<const uint8_t*>(mask->data);
    a.mask_u1 = mask->dtype == SDPA_U1;
    a.mask_sb = st[0]; a.mask_sh = st[1]; a.mask_sq = st[2]; a.mask_sk = st[3];
    if (!a.mask && numel(mask) > 0) return fail(SDPA_ERR_NULL, "mask data is NULL");
  }
  a.scale = std::isnan(scale) ? (float)(1.0 / std::sqrt((double)D)) : scale;
  a.causal = is_causal;
  a.q_offset = q_offset; a.q_offset_all = q_offset_all;
  a.kv_lengths = kv_lengths; a.kv_length_all = kv_length_all;
  a.q_lengths = q_lengths; a.q_length_all = q_length_all;
  a.qk_norm = qk_norm;
  return SDPA_OK;
}

int decode_split_len(int64_t cap, int32_t num_splits) {
  int64_t len = 1024;                                  // library choice: 1024 keys per split
  if (num_splits > 0) len = (cap + num_splits - 1) / num_splits;
  len = ((len + 63) / 64) * 64;
  if (len < 64) len = 64;
  if (len > INT32_MAX) len = INT32_MAX & ~63;
  return (int)len;
}

}  // namespace

namespace {

struct MaskLayout {
  int64_t nblk, nrows, words;
  size_t off_cls, off_next, off_rowptr, off_data, off_np, off_bits, total;
};

sdpa_status mask_layout(const sdpa_tensor* mask, int32_t bq, int32_t bkv, MaskLayout& L) {
  if (!mask) return fail(SDPA_ERR_NULL, "mask descriptor is required");
  if (mask->dtype != SDPA_U8 && mask->dtype != SDPA_U1) return fail(SDPA_ERR_DTYPE, "mask must be U8 or U1");
  if (!dims_ok(mask)) return fail(SDPA_ERR_SHAPE, "mask dims out of range");
  if (mask->dtype == SDPA_U1 && mask->dims[0] != 1 && mask->strides[0] != 1)
    return fail(SDPA_ERR_SHAPE, "a U1 mask needs its elements contiguous (strides[0] == 1)");
  if (bq < 1 || bkv < 32 || bkv % 32) return fail(SDPA_ERR_SHAPE, "bq >= 1 and bkv a positive multiple of 32");
  const int64_t Lkv = mask->dims[0], Lq = mask->dims[1], Mh = mask->dims[2], Mb = mask->dims[3];
  const int64_t n_qb = (Lq + bq - 1) / bq, n_kb = (Lkv + bkv - 1) / bkv;
  L.nblk = Mb * Mh * n_qb * n_kb;
  L.nrows = Mb * Mh * n_qb;
  L.words = bkv / 32;
  if (L.nblk > INT32_MAX) return fail(SDPA_ERR_UNSUPPORTED, "too many blocks");
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o = 0;
  L.off_cls = o;    o = up(o + (size_t)L.nblk);
  L.off_next = o;   o = up(o + (size_t)L.nblk * 4);
  L.off_rowptr = o; o = up(o + (size_t)(L.nrows + 1) * 4);
  L.off_data = o;   o = up(o + (size_t)L.nblk * 4);
  L.off_np = o;     o = up(o + 4);
  L.off_bits = o;   o = up(o + (size_t)L.nblk * bq * L.words * 4);
  L.total = o;
  return SDPA_OK;
}

}  // namespace

extern "C" {

const char* sdpa_status_string(int32_t s) {
  switch (s) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_NULL: return "null pointer";
    case SDPA_ERR_SHAPE: return "shape mismatch";
    case SDPA_ERR_DTYPE: return "unsupported dtype";
    case SDPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SDPA_ERR_WORKSPACE: return "workspace too small";
    case SDPA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* sdpa_last_error(void) { return g_err.c_str(); }

const char* sdpa_version(void) { return "sdpa_mi355x 0.1 gfx950"; }

sdpa_status sdpa_measure_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, size_t sink_bytes, void* stream) {
  g_err.clear();
  if (!sink) return fail(SDPA_ERR_NULL, "sink is required");
  if (workgroups < 1 || iters < 1) return fail(SDPA_ERR_SHAPE, "workgroups and iters must be positive");
  if (sink_bytes < (size_t)workgroups * 256 * sizeof(float))
    return fail(SDPA_ERR_WORKSPACE, "sink needs %zu bytes", (size_t)workgroups * 256 * sizeof(float));
  return hip_status(launch_measure_mfma(workgroups, iters, sink, static_cast<hipStream_t>(stream)),
                    "sdpa_measure_mfma_bf16");
}

sdpa_status sdpa_measure_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                     size_t sink_bytes, void* stream) {
  g_err.clear();
  if (!src || !sink) return fail(SDPA_ERR_NULL, "src and sink are required");
  if (workgroups < 1 || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15))
    return fail(SDPA_ERR_SHAPE, "need workgroups >= 1, bytes a positive multiple of 16, src 16-byte aligned");
  if (sink_bytes < (size_t)workgroups * 4 * sizeof(uint32_t))
    return fail(SDPA_ERR_WORKSPACE, "sink needs %zu bytes", (size_t)workgroups * 4 * sizeof(uint32_t));
  return hip_status(launch_stream_read(src, bytes, sink, workgroups, static_cast<hipStream_t>(stream)),
                    "sdpa_measure_stream_read");
}

sdpa_status sdpa_fwd_packed(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                            const int32_t* q_segments, const int32_t* kv_segments, int32_t n_segments, int32_t maxlen,
                            float scale, int32_t is_causal, const int32_t* q_offset, int32_t q_offset_all,
                            const int32_t* kv_lengths, int32_t kv_length_all, const int32_t* q_lengths,
                            int32_t q_length_all, int32_t qk_norm, sdpa_tensor* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!v || !out) return fail(SDPA_ERR_NULL, "v and out descriptors are required");
  if (n_segments < 0) return fail(SDPA_ERR_SHAPE, "n_segments must be >= 0");
  if (n_segments > 0 && !q_segments) return fail(SDPA_ERR_NULL, "q_segments is required");
  if (maxlen < -1) return fail(SDPA_ERR_SHAPE, "maxlen must be -1 (none) or a length");
  if (!q || !k || q->dims[3] != 1 || k->dims[3] != 1 || out->dims[3] != 1)
    return fail(SDPA_ERR_SHAPE, "packed sequences have no batch dimension (dims[3] == 1)");
  AttnArgs a;
  sdpa_status st = resolve_attention(q, k, v, nullptr, nullptr, nullptr, scale, is_causal, q_offset, q_offset_all,
                                     kv_lengths, kv_length_all, q_lengths, q_length_all, qk_norm, out, a);
  if (st != SDPA_OK) return st;
  const size_t need = sdpa_fwd_workspace_bytes(q, k, v, qk_norm);
  if (workspace_bytes < need || (need && !workspace))
    return fail(SDPA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (a.Lq == 0 || n_segments == 0) return SDPA_OK;
  if (!a.q || !a.out || (a.Lkv > 0 && (!a.k || !a.v))) return fail(SDPA_ERR_NULL, "a tensor's data is NULL");
  a.q_seg = q_segments;
  a.kv_seg = kv_segments;
  a.n_seg = n_segments;
  a.seg_maxlen = maxlen;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (qk_norm && a.Lkv > 0) {
    a.k_rinv = static_cast<const float*>(workspace);
    sdpa_status hs = hip_status(launch_row_rinv(a.k, a.in_dtype, a.k_sb, a.k_ss, a.k_sh, 1, a.Lkv, a.Hkv, a.D,
                                                kRmsEps, static_cast<float*>(workspace), s),
                                "key RMS factors");
    if (hs != SDPA_OK) return hs;
  }
  if (fwd_mfma_supports(a)) return hip_status(launch_fwd_mfma(a, s), "sdpa_fwd_packed (mfma)");
  return hip_status(launch_fwd_generic(a, s), "sdpa_fwd_packed (generic)");
}

size_t sdpa_fwd_workspace_bytes(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v, int32_t qk_norm) {
  (void)q; (void)v;
  if (!qk_norm || !k) return 0;
  return (size_t)(k->dims[3] * k->dims[2] * k->dims[1]) * sizeof(float);
}

sdpa_status sdpa_fwd(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v, const sdpa_tensor* bias,
                     const sdpa_tensor* mask, const sdpa_block_mask_info* mask_info, float scale, int32_t is_causal,
                     const int32_t* q_offset, int32_t q_offset_all, const int32_t* kv_lengths,
                     int32_t kv_length_all, const int32_t* q_lengths, int32_t q_length_all, int32_t qk_norm,
                     sdpa_tensor* out, void* workspace, size_t workspace_bytes, void* stream) {
  return sdpa_fwd_lse(q, k, v, bias, mask, mask_info, scale, is_causal, q_offset, q_offset_all, kv_lengths,
                      kv_length_all, q_lengths, q_length_all, qk_norm, out, nullptr, workspace, workspace_bytes,
                      stream);
}

sdpa_status sdpa_fwd_lse(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v, const sdpa_tensor* bias,
                         const sdpa_tensor* mask, const sdpa_block_mask_info* mask_info, float scale,
                         int32_t is_causal, const int32_t* q_offset, int32_t q_offset_all,
                         const int32_t* kv_lengths, int32_t kv_length_all, const int32_t* q_lengths,
                         int32_t q_length_all, int32_t qk_norm, sdpa_tensor* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!v || !out) return fail(SDPA_ERR_NULL, "v and out descriptors are required");
  AttnArgs a;
  sdpa_status st = resolve_attention(q, k, v, bias, mask, mask_info, scale, is_causal, q_offset, q_offset_all,
                                     kv_lengths, kv_length_all, q_lengths, q_length_all, qk_norm, out, a);
  if (st != SDPA_OK) return st;
  const size_t need = sdpa_fwd_workspace_bytes(q, k, v, qk_norm);
  if (workspace_bytes < need || (need && !workspace))
    return fail(SDPA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (a.B == 0 || a.Lq == 0) return SDPA_OK;
  if (!a.q || !a.out || (a.Lkv > 0 && (!a.k || !a.v))) return fail(SDPA_ERR_NULL, "a tensor's data is NULL");
  a.lse = lse;
  a.lse_sh = a.Lq;
  a.lse_sb = (int64_t)a.Hq * a.Lq;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (qk_norm && a.Lkv > 0) {
    a.k_rinv = static_cast<const float*>(workspace);
    sdpa_status hs = hip_status(launch_row_rinv(a.k, a.in_dtype, a.k_sb, a.k_ss, a.k_sh, a.B, a.Lkv, a.Hkv, a.D,
                                                kRmsEps, static_cast<float*>(workspace), s),
                                "key RMS factors");
    if (hs != SDPA_OK) return hs;
  }
  if (fwd_mfma_supports(a)) return hip_status(launch_fwd_mfma(a, s), "sdpa_fwd (mfma)");
  return hip_status(launch_fwd_generic(a, s), "sdpa_fwd (generic)");
}

size_t sdpa_bwd_workspace_bytes(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v) {
  (void)k; (void)v;
  if (!q) return 0;
  const size_t rows = (size_t)(q->dims[3] * q->dims[1] * q->dims[2]);
  const size_t chunks = (rows + 4095) / 4096;
  return 3 * ((rows * sizeof(float) + 255) & ~(size_t)255) + ((chunks * sizeof(double) + 255) & ~(size_t)255);
}

// the stored-dS extension, after the bytes above: dK/dV workgroup shares of dscale, their
// first-stage sums, the dS tiles
size_t sdpa_bwd_workspace_bytes_ds(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v) {
  if (!q || !k || !v) return 0;
  const int64_t tiles = bwd_ds_tile_bytes(q->dims[3], q->dims[1], q->dims[2], k->dims[2], q->dims[0], v->dims[0],
                                          q->dtype);
  if (tiles <= 0 || k->dims[3] <= 0 || k->dims[1] <= 0) return 0;
  const size_t n_dsp = (size_t)bwd_dkdv_workgroups(k->dims[3], k->dims[1], k->dims[2]) * 8;
  const size_t chunks = (n_dsp + 4095) / 4096;
  return sdpa_bwd_workspace_bytes(q, k, v) + ((n_dsp * sizeof(float) + 255) & ~(size_t)255) +
         ((chunks * sizeof(double) + 255) & ~(size_t)255) + (size_t)tiles;
}

// The gradient's arguments (everything but lse, dscale and the workspace) into g, validated.
static sdpa_status resolve_bwd(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                               const sdpa_tensor* out, const sdpa_tensor* dout, const sdpa_tensor* mask,
                               const sdpa_block_mask_info* mask_info, float scale, int32_t is_causal,
                               const int32_t* q_offset, int32_t q_offset_all, const int32_t* kv_lengths,
                               int32_t kv_length_all, const int32_t* q_lengths, int32_t q_length_all,
                               const sdpa_tensor* dq, const sdpa_tensor* dk, const sdpa_tensor* dv, BwdArgs& g) {
  if (!v || !out || !dout || !dq || !dk || !dv)
    return fail(SDPA_ERR_NULL, "v, out, dout, dq, dk and dv descriptors are required");
  std::memset(&g, 0, sizeof g);
  sdpa_status st = resolve_attention(q, k, v, nullptr, mask, mask_info, scale, is_causal, q_offset, q_offset_all,
                                     kv_lengths, kv_length_all, q_lengths, q_length_all, 0, out, g.a);
  if (st != SDPA_OK) return st;
  auto same = [](const sdpa_tensor* x, const sdpa_tensor* y) {
    for (int i = 0; i < 4; ++i)
      if (x->dims[i] != y->dims[i]) return false;
    return true;
  };
  if (!same(dout, out)) return fail(SDPA_ERR_SHAPE, "dout must have the dims of out");
  if (!same(dq, q) || !same(dk, k) || !same(dv, v)) return fail(SDPA_ERR_SHAPE, "dq, dk, dv must have the dims of q, k, v");
  if (!dims_ok(dout) || !dims_ok(dq) || !dims_ok(dk) || !dims_ok(dv)) return fail(SDPA_ERR_SHAPE, "a dim is out of range");
  if (!is_float(dout->dtype) || !is_float(dq->dtype) || !is_float(dk->dtype) || !is_float(dv->dtype))
    return fail(SDPA_ERR_DTYPE, "dout, dq, dk and dv must be F32, BF16 or F16");
  if (dout->strides[0] != 1 || dq->strides[0] != 1 || dk->strides[0] != 1 || dv->strides[0] != 1)
    return fail(SDPA_ERR_SHAPE, "dout, dq, dk and dv need head_dim stride 1");
  g.dout = dout->data; g.do_sb = dout->strides[3]; g.do_ss = dout->strides[2]; g.do_sh = dout->strides[1];
  g.do_dtype = dout->dtype;
  g.dq = dq->data; g.dq_sb = dq->strides[3]; g.dq_ss = dq->strides[2]; g.dq_sh = dq->strides[1];
  g.dk = dk->data; g.dk_sb = dk->strides[3]; g.dk_ss = dk->strides[2]; g.dk_sh = dk->strides[1];
  g.dv = dv->data; g.dv_sb = dv->strides[3]; g.dv_ss = dv->strides[2]; g.dv_sh = dv->strides[1];
  g.dq_dtype = dq->dtype; g.dk_dtype = dk->dtype; g.dv_dtype = dv->dtype;
  return SDPA_OK;
}

sdpa_status sdpa_bwd(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v, const sdpa_tensor* out,
                     const sdpa_tensor* dout, const float* lse, const sdpa_tensor* mask,
                     const sdpa_block_mask_info* mask_info, float scale, int32_t is_causal,
                     const int32_t* q_offset, int32_t q_offset_all, const int32_t* kv_lengths,
                     int32_t kv_length_all, const int32_t* q_lengths, int32_t q_length_all, sdpa_tensor* dq,
                     sdpa_tensor* dk, sdpa_tensor* dv, float* dscale, void* workspace, size_t workspace_bytes,
                     void* stream) {
  g_err.clear();
  BwdArgs g;
  sdpa_status st = resolve_bwd(q, k, v, out, dout, mask, mask_info, scale, is_causal, q_offset, q_offset_all,
                               kv_lengths, kv_length_all, q_lengths, q_length_all, dq, dk, dv, g);
  if (st != SDPA_OK) return st;
  const AttnArgs& a = g.a;
  const size_t need = sdpa_bwd_workspace_bytes(q, k, v);
  if (workspace_bytes < need || (need && !workspace))
    return fail(SDPA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  const int64_t rows = (int64_t)a.B * a.Hq * a.Lq;
  if (rows > 0 && !lse) return fail(SDPA_ERR_NULL, "lse is required");
  if ((rows > 0 && (!a.q || !a.out || !dout->data || !dq->data)) ||
      ((int64_t)a.B * a.Lkv > 0 && (!a.k || !a.v || !dk->data || !dv->data)))
    return fail(SDPA_ERR_NULL, "a tensor's data is NULL");
  g.lse = lse;
  g.dscale = dscale;
  const size_t seg = ((size_t)rows * sizeof(float) + 255) & ~(size_t)255;
  g.w_dsum = static_cast<float*>(workspace);
  g.w_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + seg);
  g.w_dsc = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * seg);
  g.w_dsc2 = reinterpret_cast<double*>(static_cast<char*>(workspace) + 3 * seg);
  const size_t need_ds = sdpa_bwd_workspace_bytes_ds(q, k, v);
  if (need_ds && workspace_bytes >= need_ds) {
    const size_t n_dsp = (size_t)bwd_dkdv_workgroups(k->dims[3], k->dims[1], k->dims[2]) * 8;
    char* x = static_cast<char*>(workspace) + need;
    g.w_dsp = reinterpret_cast<float*>(x);
    x += (n_dsp * sizeof(float) + 255) & ~(size_t)255;
    g.w_dsc2_ds = reinterpret_cast<double*>(x);
    x += (((n_dsp + 4095) / 4096) * sizeof(double) + 255) & ~(size_t)255;
    g.w_ds = reinterpret_cast<uint16_t*>(x);
  }
  return hip_status(launch_bwd(g, static_cast<hipStream_t>(stream)), "sdpa_bwd");
}

sdpa_status sdpa_fwd_path(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v, const sdpa_tensor* bias,
                          const sdpa_tensor* mask, const sdpa_block_mask_info* mask_info, float scale,
                          int32_t is_causal, int32_t qk_norm, const sdpa_tensor* out, int32_t* path) {
  g_err.clear();
  if (!path) return fail(SDPA_ERR_NULL, "path is required");
  if (!v || !out) return fail(SDPA_ERR_NULL, "v and out descriptors are required");
  AttnArgs a;
  const sdpa_status st = resolve_attention(q, k, v, bias, mask, mask_info, scale, is_causal, nullptr, 0, nullptr, -1,
                                           nullptr, -1, qk_norm, out, a);
  if (st != SDPA_OK) return st;
  *path = fwd_mfma_supports(a) ? SDPA_PATH_MATRIX_CORE : SDPA_PATH_FP32;
  return SDPA_OK;
}

sdpa_status sdpa_bwd_path(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v, const sdpa_tensor* out,
                          const sdpa_tensor* dout, const sdpa_tensor* mask, const sdpa_block_mask_info* mask_info,
                          float scale, int32_t is_causal, const sdpa_tensor* dq, const sdpa_tensor* dk,
                          const sdpa_tensor* dv, size_t workspace_bytes, int32_t* path) {
  g_err.clear();
  if (!path) return fail(SDPA_ERR_NULL, "path is required");
  BwdArgs g;
  const sdpa_status st = resolve_bwd(q, k, v, out, dout, mask, mask_info, scale, is_causal, nullptr, 0, nullptr, -1,
                                     nullptr, -1, dq, dk, dv, g);
  if (st != SDPA_OK) return st;
  if (!bwd_mfma_supports(g)) {
    *path = SDPA_PATH_FP32;
    return SDPA_OK;
  }
  // sdpa_bwd hands the dS tiles a workspace of sdpa_bwd_workspace_bytes_ds() bytes; block info
  // keeps the route that forms the weights again
  const size_t need_ds = sdpa_bwd_workspace_bytes_ds(q, k, v);
  *path = (need_ds && workspace_bytes >= need_ds && !g.a.bm_class) ? SDPA_PATH_MATRIX_CORE_STORED_DS
                                                                    : SDPA_PATH_MATRIX_CORE;
  return SDPA_OK;
}

size_t sdpa_decode_workspace_bytes(const sdpa_tensor* q, const sdpa_tensor* k_cache, int32_t num_splits) {
  if (!q || !k_cache) return 0;
  const int64_t cap = k_cache->dims[2];
  const int64_t len = decode_split_len(cap, num_splits);
  const int64_t max_splits = (cap + len - 1) / len;
  const int64_t T = q->dims[2] > 0 ? q->dims[2] : 0;
  return (size_t)(q->dims[3] * T * q->dims[1] * max_splits * (q->dims[0] + 2)) * sizeof(float);
}

namespace {

// ---- the allocation-free decode's device scratch -------------------------------------------
// One array per GPU (each device that loads the code object holds its own copy, at its own
// address, until the process ends). Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, taken once per device with that device
// current, and kept here.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sdpa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SDPA_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SDPA_OK;
}

// sdpa_decode and sdpa_decode_noalloc: with use_scratch the split partials go to the device
// scratch instead of the caller's workspace.
sdpa_status decode_call(const sdpa_tensor* q, const sdpa_tensor* kc, const sdpa_tensor* vc, const int32_t* kv_lengths,
                        float scale, int32_t num_splits, sdpa_tensor* out, void* workspace, size_t workspace_bytes,
                        void* stream, bool use_scratch);

}  // namespace

sdpa_status sdpa_decode(const sdpa_tensor* q, const sdpa_tensor* kc, const sdpa_tensor* vc, const int32_t* kv_lengths,
                        float scale, int32_t num_splits, sdpa_tensor* out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  g_err.clear();
  return decode_call(q, kc, vc, kv_lengths, scale, num_splits, out, workspace, workspace_bytes, stream, false);
}

sdpa_status sdpa_decode_noalloc(const sdpa_tensor* q, const sdpa_tensor* kc, const sdpa_tensor* vc,
                                const int32_t* kv_lengths, float scale, int32_t num_splits, sdpa_tensor* out,
                                void* stream) {
  g_err.clear();
  return decode_call(q, kc, vc, kv_lengths, scale, num_splits, out, nullptr, 0, stream, true);
}

size_t sdpa_decode_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

namespace {

sdpa_status decode_call(const sdpa_tensor* q, const sdpa_tensor* kc, const sdpa_tensor* vc, const int32_t* kv_lengths,
                        float scale, int32_t num_splits, sdpa_tensor* out, void* workspace, size_t workspace_bytes,
                        void* stream, bool use_scratch) {
  if (!q || !kc || !vc || !out) return fail(SDPA_ERR_NULL, "q, k_cache, v_cache and out are required");
  if (!kv_lengths) return fail(SDPA_ERR_NULL, "kv_lengths is required for decode");
  if (q->dims[2] < 0 || q->dims[2] > kc->dims[2])
    return fail(SDPA_ERR_SHAPE, "decode takes 0 to capacity query positions (q dims[2])");
  if (num_splits < 0) return fail(SDPA_ERR_SHAPE, "num_splits must be >= 0");
  if (kc->dims[0] != vc->dims[0] || q->dims[0] != vc->dims[0])
    return fail(SDPA_ERR_SHAPE, "decode needs equal q, k and v head dims");
  AttnArgs a;
  sdpa_status st = resolve_attention(q, kc, vc, nullptr, nullptr, nullptr, scale, SDPA_CAUSAL_BOTTOM_RIGHT,
                                     nullptr, 0, kv_lengths, -1, nullptr, -1, 0, out, a);
  if (st != SDPA_OK) return st;
  const size_t need = sdpa_decode_workspace_bytes(q, kc, num_splits);
  if (use_scratch) {
    if (need > kNoAllocScratchBytes)
      return fail(SDPA_ERR_WORKSPACE,
                  "sdpa_decode_noalloc: this call needs %zu bytes of split partials; the device scratch holds %zu "
                  "(fewer sequences, query heads, tokens or splits fit; sdpa_decode takes any size)",
                  need, kNoAllocScratchBytes);
  } else if (workspace_bytes < need || (need && !workspace)) {
    return fail(SDPA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  }
  if (a.B == 0 || a.Lq == 0) return SDPA_OK;
  if (use_scratch && need) {
    st = scratch_address(&workspace);
    if (st != SDPA_OK) return st;
  }
  if (!a.q || !a.out || (a.Lkv > 0 && (!a.k || !a.v))) return fail(SDPA_ERR_NULL, "a tensor's data is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);

  DecodeArgs d;
  std::memset(&d, 0, sizeof d);
  d.q = a.q; d.k = a.k; d.v = a.v; d.out = a.out;
  d.B = a.B; d.T = a.Lq; d.Hq = a.Hq; d.Hkv = a.Hkv; d.D = a.D; d.cap = a.Lkv;
  d.q_sb = a.q_sb; d.q_ss = a.q_ss; d.q_sh = a.q_sh; d.k_sb = a.k_sb; d.k_ss = a.k_ss; d.k_sh = a.k_sh;
  d.v_sb = a.v_sb; d.v_ss = a.v_ss; d.v_sh = a.v_sh; d.o_sb = a.o_sb; d.o_ss = a.o_ss; d.o_sh = a.o_sh;
  d.in_dtype = a.in_dtype;
  d.out_dtype = a.out_dtype;
  d.kv_lengths = kv_lengths;
  d.scale_log2 = a.scale * 1.4426950408889634f;
  d.split_len = decode_split_len(a.Lkv, num_splits);
  d.max_splits = (int)((a.Lkv + d.split_len - 1) / d.split_len);
  if (d.max_splits > 0 && decode_fast_supports(d, a.in_dtype)) {
    d.part_o = static_cast<float*>(workspace);
    d.part_ml = d.part_o + (size_t)a.B * a.Lq * a.Hq * d.max_splits * a.D;
    return hip_status(launch_decode(d, s), "sdpa_decode");
  }
  // any other shape: the general kernel at these T queries, bottom-right causal, these kv_lengths
  return hip_status(launch_fwd_generic(a, s), "sdpa_decode (generic)");
}

}  // namespace

sdpa_status kv_cache_update(sdpa_tensor* kc, sdpa_tensor* vc, const sdpa_tensor* kn, const sdpa_tensor* vn,
                            const int32_t* write_index, void* stream) {
  g_err.clear();
  if (!kc || !vc || !kn || !vn) return fail(SDPA_ERR_NULL, "cache and new-row descriptors are required");
  if (!write_index) return fail(SDPA_ERR_NULL, "write_index is required");
  if (!dims_ok(kc) || !dims_ok(vc) || !dims_ok(kn) || !dims_ok(vn)) return fail(SDPA_ERR_SHAPE, "dims out of range");
  if (!is_float(kc->dtype) || vc->dtype != kc->dtype || kn->dtype != kc->dtype || vn->dtype != kc->dtype)
    return fail(SDPA_ERR_DTYPE, "caches and new rows must share one dtype, F32, BF16 or F16");
  for (int i = 0; i < 4; ++i)
    if (vc->dims[i] != kc->dims[i] || vn->dims[i] != kn->dims[i])
      return fail(SDPA_ERR_SHAPE, "k and v caches (and new rows) must have equal dims");
  if (kn->dims[0] != kc->dims[0] || kn->dims[1] != kc->dims[1] || kn->dims[3] != kc->dims[3])
    return fail(SDPA_ERR_SHAPE, "new rows must be {D, Hkv, T, B} of the cache");
  if (kc->strides[0] != 1 || vc->strides[0] != 1 || kn->strides[0] != 1 || vn->strides[0] != 1)
    return fail(SDPA_ERR_SHAPE, "head_dim stride must be 1");
  const int D = (int)kc->dims[0], H = (int)kc->dims[1], cap = (int)kc->dims[2], B = (int)kc->dims[3];
  const int T = (int)kn->dims[2];
  if ((int64_t)B * T * H * D == 0) return SDPA_OK;
  if (!kc->data || !vc->data || !kn->data || !vn->data) return fail(SDPA_ERR_NULL, "a tensor's data is NULL");
  const int eb = kc->dtype == SDPA_F32 ? 4 : 2;
  return hip_status(launch_kv_cache_update(kc->data, vc->data, kn->data, vn->data, eb, B, T, H, D, cap,
                                           kc->strides[3], kc->strides[2], kc->strides[1],
                                           vc->strides[3], vc->strides[2], vc->strides[1],
                                           kn->strides[3], kn->strides[2], kn->strides[1],
                                           vn->strides[3], vn->strides[2], vn->strides[1],
                                           write_index, static_cast<hipStream_t>(stream)),
                    "kv_cache_update");
}


sdpa_status sdpa_block_mask_info_bytes(const sdpa_tensor* mask, int32_t bq, int32_t bkv, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(SDPA_ERR_NULL, "bytes is NULL");
  MaskLayout L;
  sdpa_status s = mask_layout(mask, bq, bkv, L);
  if (s != SDPA_OK) return s;
  *bytes = L.total;
  return SDPA_OK;
}

sdpa_status build_block_mask_info(const sdpa_tensor* mask, int32_t bq, int32_t bkv, void* storage,
                                  size_t storage_bytes, sdpa_block_mask_info* info, void* stream) {
  g_err.clear();
  if (!info) return fail(SDPA_ERR_NULL, "info is NULL");
  MaskLayout L;
  sdpa_status s = mask_layout(mask, bq, bkv, L);
  if (s != SDPA_OK) return s;
  if (!storage || storage_bytes < L.total)
    return fail(SDPA_ERR_WORKSPACE, "storage needs %zu bytes, got %zu", L.total, storage_bytes);
  if (!mask->data && numel(mask) > 0) return fail(SDPA_ERR_NULL, "mask data is NULL");
  char* base = static_cast<char*>(storage);
  std::memset(info, 0, sizeof *info);
  info->mask_batch = (int32_t)mask->dims[3];
  info->mask_heads = (int32_t)mask->dims[2];
  info->q_len = (int32_t)mask->dims[1];
  info->kv_len = (int32_t)mask->dims[0];
  info->bq = bq; info->bkv = bkv;
  info->n_qb = (int32_t)((mask->dims[1] + bq - 1) / bq);
  info->n_kb = (int32_t)((mask->dims[0] + bkv - 1) / bkv);
  info->block_mask = reinterpret_cast<int8_t*>(base + L.off_cls);
  info->mask_next = reinterpret_cast<int32_t*>(base + L.off_next);
  info->row_ptr = reinterpret_cast<int32_t*>(base + L.off_rowptr);
  info->data_next = reinterpret_cast<int32_t*>(base + L.off_data);
  info->n_partial = reinterpret_cast<int32_t*>(base + L.off_np);
  info->partial_bits = reinterpret_cast<uint32_t*>(base + L.off_bits);

  MaskInfoArgs m;
  std::memset(&m, 0, sizeof m);
  m.mask = static_cast<const uint8_t*>(mask->data);
  m.u1 = mask->dtype == SDPA_U1;
  m.sb = mask->strides[3]; m.sh = mask->strides[2]; m.sq = mask->strides[1]; m.sk = mask->dims[0] == 1 ? 0 : mask->strides[0];
  // 16-byte loads of U8 rows: unit column stride, aligned base, and every row start aligned
  m.vec16 = !m.u1 && m.sk == 1 && (reinterpret_cast<uintptr_t>(m.mask) & 15) == 0 &&
            ((mask->dims[3] <= 1 || m.sb % 16 == 0) && (mask->dims[2] <= 1 || m.sh % 16 == 0) &&
             (mask->dims[1] <= 1 || m.sq % 16 == 0));
  m.Mb = info->mask_batch; m.Mh = info->mask_heads; m.Lq = info->q_len; m.Lkv = info->kv_len;
  m.bq = bq; m.bkv = bkv; m.n_qb = info->n_qb; m.n_kb = info->n_kb;
  m.cls = info->block_mask; m.next = info->mask_next; m.row_ptr = info->row_ptr; m.data_next = info->data_next;
  m.bits = info->partial_bits; m.n_partial = info->n_partial;
  return hip_status(launch_mask_info(m, static_cast<hipStream_t>(stream)), "build_block_mask_info");
}

sdpa_status head_rms_norm(const sdpa_tensor* x, sdpa_tensor* y, float eps, void* stream) {
  g_err.clear();
  if (!x || !y) return fail(SDPA_ERR_NULL, "x and y descriptors are required");
  if (!dims_ok(x) || !dims_ok(y)) return fail(SDPA_ERR_SHAPE, "dims out of range");
  if (!is_float(x->dtype) || y->dtype != x->dtype) return fail(SDPA_ERR_DTYPE, "x and y must share F32, BF16 or F16");
  for (int i = 0; i < 4; ++i)
    if (x->dims[i] != y->dims[i]) return fail(SDPA_ERR_SHAPE, "x and y dims differ");
  if (x->strides[0] != 1 || y->strides[0] != 1) return fail(SDPA_ERR_SHAPE, "head_dim stride must be 1");
  if (!(eps >= 0.f)) return fail(SDPA_ERR_SHAPE, "eps must be >= 0");
  if (numel(x) == 0) return SDPA_OK;
  if (!x->data || !y->data) return fail(SDPA_ERR_NULL, "a tensor's data is NULL");
  return hip_status(launch_head_rms_norm(x->data, y->data, x->dtype, x->strides[3], x->strides[2], x->strides[1],
                                         y->strides[3], y->strides[2], y->strides[1], (int)x->dims[3],
                                         (int)x->dims[2], (int)x->dims[1], (int)x->dims[0], eps,
                                         static_cast<hipStream_t>(stream)),
                    "head_rms_norm");
}

sdpa_status sdpa_debug_allowed_mask(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* mask,
                                    const sdpa_block_mask_info* mask_info, int32_t is_causal, const int32_t* q_offset,
                                    int32_t q_offset_all, const int32_t* kv_lengths, int32_t kv_length_all,
                                    const int32_t* q_lengths, int32_t q_length_all, sdpa_tensor* allowed,
                                    void* stream) {
  g_err.clear();
  if (!allowed) return fail(SDPA_ERR_NULL, "allowed descriptor is required");
  AttnArgs a;
  sdpa_status st = resolve_attention(q, k, nullptr, nullptr, mask, mask_info, NAN, is_causal, q_offset,
                                     q_offset_all, kv_lengths, kv_length_all, q_lengths, q_length_all, 0, nullptr,
                                     a);
  if (st != SDPA_OK) return st;
  if (allowed->dtype != SDPA_U8) return fail(SDPA_ERR_DTYPE, "allowed must be U8");
  if (allowed->dims[0] != a.Lkv || allowed->dims[1] != a.Lq || allowed->dims[2] != a.Hq || allowed->dims[3] != a.B)
    return fail(SDPA_ERR_SHAPE, "allowed must be {Lkv, Lq, Hq, B}");
  if ((int64_t)a.B * a.Hq * a.Lq * a.Lkv == 0) return SDPA_OK;
  if (!allowed->data) return fail(SDPA_ERR_NULL, "allowed data is NULL");
  return hip_status(launch_debug_allowed(a, static_cast<uint8_t*>(allowed->data), allowed->strides[3],
                                         allowed->strides[2], allowed->strides[1], allowed->strides[0],
                                         static_cast<hipStream_t>(stream)),
                    "sdpa_debug_allowed_mask");
}

}  // extern "C"
