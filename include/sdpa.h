/*
 * sdpa.h -- C ABI of libsdpa_mi355x.so: multi-head scaled dot-product attention on MI355X (gfx950).
 *
 * The operation and its arguments follow the page "Neural Network primitives from NNlib.jl"
 * (Flux documentation), section "Attention" and its "Arguments" list:
 *
 *     out = softmax(scale * q^T k + bias, where allowed) * v
 *
 * with grouped-query K/V heads, is_causal (true, or bottom-right aligned), q_offset,
 * kv_lengths, q_lengths, an additive bias and a boolean mask that combine by AND. A query that
 * may attend no key gets NaN ("Fused implementation" section); a query at or past q_lengths
 * gets 0 ("Arguments": q_lengths).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are described by sdpa_tensor: dims and strides (in elements) in NNlib order,
 *   fastest first. q/k/v/out are {head_dim, heads, seq, batch}; bias/mask are
 *   {kv_len, q_len, heads, batch}, where a dim of size 1 broadcasts ("Arguments": bias, mask).
 *   This is C-order [batch][seq][heads][head_dim] for contiguous q/k/v/out. Extra NNlib batch
 *   dims are flattened into dims[3] by the caller; an unbatched array has dims[3] == 1.
 * - All data pointers are DEVICE pointers unless stated; the caller owns every buffer. The
 *   library never allocates, frees or retains memory, never synchronizes, and never reads a
 *   device array on the host (the NNlib page notes, under maxlen, that such a read waits for
 *   the device). Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *   default stream).
 * - Device-resident integers are not validated: kv_lengths and q_lengths are clamped to
 *   [0, kv_len] and [0, q_len]; a negative q_offset is legal; cache rows outside the cache are
 *   not written.
 * - Every host-detectable error returns a status without touching the GPU; the thread-local
 *   sdpa_last_error() tells what failed. The library is stateless and thread-safe.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points keep default visibility; the library builds everything else hidden. */
#if defined(__GNUC__) || defined(__clang__)
#define SDPA_API __attribute__((visibility("default")))
#else
#define SDPA_API
#endif

typedef enum {
  SDPA_OK = 0,
  SDPA_ERR_NULL = 1,         /* a required pointer is NULL */
  SDPA_ERR_SHAPE = 2,        /* dims/strides disagree with the operation */
  SDPA_ERR_DTYPE = 3,        /* a dtype the argument does not accept */
  SDPA_ERR_UNSUPPORTED = 4,  /* legal request with no kernel (e.g. head_dim > 256) */
  SDPA_ERR_WORKSPACE = 5,    /* workspace / storage too small */
  SDPA_ERR_HIP = 6           /* a HIP launch failed */
} sdpa_status;

/* F16 is IEEE binary16, the other 16-bit input NNlib's fused implementation takes ("Fused
 * implementation": bf16/f16 GPU arrays). */
typedef enum { SDPA_F32 = 0, SDPA_BF16 = 1, SDPA_U8 = 2, SDPA_F16 = 3, SDPA_U1 = 4 } sdpa_dtype;
/* SDPA_U1: a boolean mask packed 32 elements per 32-bit word, 8x smaller than U8 (the
 * splash-attention pull request's review asks for packed booleans where a 100k+ context makes a
 * byte mask too large). Element c of a row is bit (c mod 32) of word c/32 of that row; dims[0]
 * counts elements with strides[0] == 1 (or dims[0] == 1 to broadcast); strides[1..3] count
 * 32-bit words, each row starting on a word. Bits past dims[0] in a row's last word are ignored. */

/* "Arguments": is_causal. TRUE: query i attends keys j <= q_offset + i. BOTTOM_RIGHT: the
 * same with q_offset = kv_len_b - q_len_b, each the given length or else the array size. */
typedef enum { SDPA_CAUSAL_NONE = 0, SDPA_CAUSAL_TRUE = 1, SDPA_CAUSAL_BOTTOM_RIGHT = 2 } sdpa_causal;

typedef struct {
  void* data;
  int32_t dtype;        /* sdpa_dtype */
  int32_t reserved;
  int64_t dims[4];      /* NNlib order, fastest first */
  int64_t strides[4];   /* elements; q/k/v/out need strides[0] == 1 */
} sdpa_tensor;

/* Block information of a runtime boolean mask (pull request "Support dynamic masks in splash
 * attention #25213": blocks classed empty/partial/full, only non-empty blocks visited, partial
 * blocks stored). Filled by build_block_mask_info; every pointer points into the caller's
 * storage. Blocks are ordered by flat index (mask batch, mask head, q-block, kv-block). */
typedef struct {
  int32_t mask_batch, mask_heads;   /* 1 (broadcast) or the full size */
  int32_t q_len, kv_len;            /* mask size the info was built from */
  int32_t n_qb, n_kb, bq, bkv;      /* block grid and block size */
  int8_t* block_mask;               /* [mask_batch][mask_heads][n_qb][n_kb]: 0 empty, 1 partial, 2 full */
  int32_t* mask_next;               /* same shape: partial -> index into partial_bits, else 0 */
  int32_t* row_ptr;                 /* [mask_batch*mask_heads*n_qb + 1]: CSR row starts */
  int32_t* data_next;               /* [row_ptr[last]]: kv-block index of each non-empty block, ascending per row */
  uint32_t* partial_bits;           /* [n_partial][bq][bkv/32]: bit (c%32) of word r*(bkv/32)+c/32 = element (r,c); 1 = attend */
  int32_t* n_partial;               /* device scalar */
} sdpa_block_mask_info;

/* ---------------------------------------------------------------------------------------
 * sdpa_fwd -- attention forward ("Attention", "Arguments", "Fused implementation").
 *
 * q    {Dqk, Hq, Lq, B}; k {Dqk, Hkv, Lkv, B}; v {Dv, Hkv, Lkv, B}; Hq % Hkv == 0, and query head h
 *      reads K/V head h / (Hq/Hkv) ("Attention": grouped-query attention). F32, BF16 or F16, all
 *      three the same dtype. out {Dv, Hq, Lq, B}, F32, BF16 or F16. Arithmetic is fp32 (16-bit
 *      products accumulate in fp32).
 * bias NULL, or F32/BF16/F16 {Lkv|1, Lq|1, Hq|1, B|1}; added to the scaled logits, not scaled.
 * mask NULL, or U8 {Lkv|1, Lq|1, Hq|1, B|1}, nonzero = may attend; or the same as U1 bits.
 * mask_info  NULL, or block info built from the mask by build_block_mask_info. When given it
 *      replaces `mask` (which is then not read), lets the kernel skip empty blocks and skip the
 *      element test on full blocks. Its mask_batch/mask_heads must be 1 or B/Hq and its
 *      q_len/kv_len must be Lq/Lkv.
 * scale  multiplier of q.k; NaN selects 1/sqrt(Dqk). 0 and negative values are legal.
 * is_causal  sdpa_causal. q_offset: device int32 [B], or NULL to use q_offset_all.
 * kv_lengths device int32 [B], or NULL to use kv_length_all (< 0 means none).
 * q_lengths  device int32 [B], or NULL to use q_length_all (< 0 means none).
 * qk_norm  0 off; 1 normalizes every q and k head vector by its RMS with eps 1e-6 before the
 *      dot product (TensorTonic page "Static Arguments in jit", its normalisation formula).
 * workspace  device scratch of at least sdpa_fwd_workspace_bytes(); may be NULL when that is 0.
 * Lq == 0 does nothing. Lkv == 0 gives NaN rows.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_fwd(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                     const sdpa_tensor* bias, const sdpa_tensor* mask,
                     const sdpa_block_mask_info* mask_info,
                     float scale, int32_t is_causal,
                     const int32_t* q_offset, int32_t q_offset_all,
                     const int32_t* kv_lengths, int32_t kv_length_all,
                     const int32_t* q_lengths, int32_t q_length_all,
                     int32_t qk_norm,
                     sdpa_tensor* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * sdpa_fwd_lse -- sdpa_fwd that also writes the log-sum-exp of every query row, which the
 * gradient (sdpa_bwd) starts from (page "Neural Network primitives from NNlib.jl", section
 * "Fused implementation": the fused gradient forms the weights again, as exp(s_ij - lse_i)).
 *
 * lse  device fp32 [B][Hq][Lq] (contiguous, row i of head h of batch b at (b*Hq + h)*Lq + i),
 *      or NULL (then this is sdpa_fwd): the natural log of the sum of exp over the row's
 *      allowed logits (scale and bias included). -inf for a row with no allowed key and for
 *      the rows at or past q_lengths. Every other argument as for sdpa_fwd.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_fwd_lse(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                                  const sdpa_tensor* bias, const sdpa_tensor* mask,
                                  const sdpa_block_mask_info* mask_info,
                                  float scale, int32_t is_causal,
                                  const int32_t* q_offset, int32_t q_offset_all,
                                  const int32_t* kv_lengths, int32_t kv_length_all,
                                  const int32_t* q_lengths, int32_t q_length_all,
                                  int32_t qk_norm,
                                  sdpa_tensor* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ---------------------------------------------------------------------------------------
 * sdpa_bwd -- the gradient of sdpa_fwd with respect to query, key, value and scale (page
 * "Neural Network primitives from NNlib.jl", section "Fused implementation"). The weights are
 * formed again from q, k and lse, never stored. A query with no allowed key (NaN output) and
 * the queries at or past q_lengths (zero output) take no part: their dq rows are 0 and they
 * add nothing to dk, dv or dscale. Under grouped-query attention dk and dv of a K/V head sum
 * over the query heads that read it.
 *
 * q, k, v, mask, mask_info, scale, is_causal, q_offset, kv_lengths, q_lengths: those of the
 *      forward call (no bias and no qk_norm: the page sends a call with a bias to the
 *      materialized path, whose gradient is not this one).
 * out  the forward output {Dv, Hq, Lq, B}; dout its cotangent, same dims; each F32, BF16 or F16.
 *      dout must be finite everywhere, also on rows that take no part: the matrix-core kernels
 *      multiply it by their zero weights, and a NaN or Inf there would reach dk and dv.
 * lse  device fp32 [B][Hq][Lq] as written by sdpa_fwd_lse for this call.
 * dq {D, Hq, Lq, B}, dk {D, Hkv, Lkv, B}, dv {Dv, Hkv, Lkv, B}: outputs, each F32, BF16 or F16,
 *      head_dim stride 1; every element is written (0 for keys that no query attends).
 * dscale  device fp32 scalar, or NULL: sum over all pairs of dS_ij * <q_i, k_j>.
 * workspace  device scratch of at least sdpa_bwd_workspace_bytes(); results are deterministic
 *      (no atomics, fixed reduction order). With at least sdpa_bwd_workspace_bytes_ds() bytes
 *      (when that is not 0) and neither block info nor a call the matrix-core kernels decline,
 *      the dK/dV pass also stores every dS tile it forms, and the dQ pass reads them instead of
 *      forming the weights a second time; the results agree to rounding (the dQ products take
 *      a 16-bit dS either way), and dscale is then summed over the keys j as
 *      <sum_i dS_ij q_i, k_j>.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_bwd(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                              const sdpa_tensor* out, const sdpa_tensor* dout, const float* lse,
                              const sdpa_tensor* mask, const sdpa_block_mask_info* mask_info,
                              float scale, int32_t is_causal,
                              const int32_t* q_offset, int32_t q_offset_all,
                              const int32_t* kv_lengths, int32_t kv_length_all,
                              const int32_t* q_lengths, int32_t q_length_all,
                              sdpa_tensor* dq, sdpa_tensor* dk, sdpa_tensor* dv, float* dscale,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace sdpa_bwd needs for these shapes. Host only. */
SDPA_API size_t sdpa_bwd_workspace_bytes(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v);

/* Bytes of workspace with which sdpa_bwd stores dS for its dQ pass: the bytes above plus
 * B*Hq*ceil(Lq/64)*ceil(Lkv/128)*16 KiB of dS tiles and the dK/dV workgroups' dscale shares.
 * 0 where that route does not apply (inputs other than bf16/f16, D != Dv, D not 64 or 128),
 * Lkv is above 8M keys, or the dS tiles would exceed 8 GiB. Host only. */
SDPA_API size_t sdpa_bwd_workspace_bytes_ds(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v);

/* ---------------------------------------------------------------------------------------
 * sdpa_fwd_path / sdpa_bwd_path -- which kernels sdpa_fwd (sdpa_fwd_lse) or sdpa_bwd would run
 * for these arguments. Nothing is launched and no device memory is read; the descriptors'
 * data pointers count only for their alignment. The arguments mean what they mean for
 * sdpa_fwd and sdpa_bwd (q_offset, kv_lengths and q_lengths do not change the choice);
 * workspace_bytes is the size the gradient call would be given. On success *path is:
 *   SDPA_PATH_MATRIX_CORE           the bf16/f16 matrix-core kernels;
 *   SDPA_PATH_MATRIX_CORE_STORED_DS the gradient's matrix-core kernels with dS kept in the
 *                                   workspace for the dQ pass (sdpa_bwd_workspace_bytes_ds());
 *   SDPA_PATH_FP32                  the fp32 vector kernels, which take every other accepted
 *                                   call (fp32 inputs, head dims other than 64/128, D != Dv, an
 *                                   f16 bias, scale <= 0, unaligned or oddly strided views,
 *                                   per-(batch, head) slices beyond 32-bit offsets) and are many
 *                                   times slower.
 * Errors are those the call itself would return for invalid arguments; *path is then unset.
 * Host only. */
typedef enum { SDPA_PATH_MATRIX_CORE = 1, SDPA_PATH_FP32 = 2, SDPA_PATH_MATRIX_CORE_STORED_DS = 3 } sdpa_path;
SDPA_API sdpa_status sdpa_fwd_path(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                                   const sdpa_tensor* bias, const sdpa_tensor* mask,
                                   const sdpa_block_mask_info* mask_info, float scale, int32_t is_causal,
                                   int32_t qk_norm, const sdpa_tensor* out, int32_t* path);
SDPA_API sdpa_status sdpa_bwd_path(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                                   const sdpa_tensor* out, const sdpa_tensor* dout, const sdpa_tensor* mask,
                                   const sdpa_block_mask_info* mask_info, float scale, int32_t is_causal,
                                   const sdpa_tensor* dq, const sdpa_tensor* dk, const sdpa_tensor* dv,
                                   size_t workspace_bytes, int32_t* path);

/* ---------------------------------------------------------------------------------------
 * sdpa_fwd_packed -- attention over packed sequences (page "Neural Network primitives from
 * NNlib.jl", section "Packed sequences"; "Arguments": q_segments, kv_segments, maxlen). The
 * inputs hold n_segments sequences one after the other with no batch dimension: q
 * {Dqk, Hq, Lq_total, 1}, k {Dqk, Hkv, Lkv_total, 1}, v {Dv, Hkv, Lkv_total, 1}, out
 * {Dv, Hq, Lq_total, 1}; dtypes as for sdpa_fwd. Segment s of the queries attends segment s
 * of the keys and values only, as batch element s of a padded batch would.
 *
 * q_segments  device int32 [n_segments]: segment lengths along q.
 * kv_segments device int32 [n_segments] along k/v, or NULL: the same as q_segments.
 * maxlen      -1, or a bound on every segment length (no segment may exceed it). The lengths
 *             are never read on the host; maxlen only narrows the launch.
 * is_causal, q_offset, kv_lengths, q_lengths, qk_norm, scale: as for sdpa_fwd, applied within
 *             each segment; the per-batch arrays take one entry per segment.
 * The lengths have to add up to Lq_total and Lkv_total; the kernels cut any segment at the end
 * of the arrays, and rows of q outside every segment are not written. No bias or mask (the
 * page allows none with segments). workspace: sdpa_fwd_workspace_bytes() of the same tensors.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_fwd_packed(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                                     const int32_t* q_segments, const int32_t* kv_segments,
                                     int32_t n_segments, int32_t maxlen,
                                     float scale, int32_t is_causal,
                                     const int32_t* q_offset, int32_t q_offset_all,
                                     const int32_t* kv_lengths, int32_t kv_length_all,
                                     const int32_t* q_lengths, int32_t q_length_all,
                                     int32_t qk_norm,
                                     sdpa_tensor* out, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace sdpa_fwd needs for these shapes (0 when none). Host only. */
SDPA_API size_t sdpa_fwd_workspace_bytes(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                                int32_t qk_norm);

/* ---------------------------------------------------------------------------------------
 * sdpa_decode -- the newest T query positions of each sequence against a KV cache: the cached
 * attention of the keras issue on MultiHeadAttention (its list of extensions puts cached
 * attention first) and the decode loop of the Flax discussion on nnx.MultiHeadAttention with
 * decode=True (T = 1); T > 1 is the NNlib "Examples" cache case with several new queries.
 * Same result as sdpa_fwd with Lq == T, is_causal = BOTTOM_RIGHT and these kv_lengths (page
 * "Neural Network primitives from NNlib.jl", "Arguments": is_causal and kv_lengths): query t
 * (0-based) of sequence b attends keys [0, kv_lengths[b] - T + t].
 *
 * q {D, Hq, T, B} F32, BF16 or F16, 0 <= T <= capacity; k_cache, v_cache {D, Hkv, capacity, B}, same
 * dtype; kv_lengths device int32 [B] (required), clamped to [0, capacity];
 * out {D, Hq, T, B} F32, BF16 or F16. num_splits: key splits per sequence (0 = library choice);
 * the partial results are merged by a log-sum-exp pass. workspace: at least
 * sdpa_decode_workspace_bytes(), which grows with T. A query with no key to attend
 * (kv_lengths[b] - T + t < 0) gives a NaN row.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_decode(const sdpa_tensor* q, const sdpa_tensor* k_cache, const sdpa_tensor* v_cache,
                        const int32_t* kv_lengths, float scale, int32_t num_splits,
                        sdpa_tensor* out, void* workspace, size_t workspace_bytes, void* stream);

SDPA_API size_t sdpa_decode_workspace_bytes(const sdpa_tensor* q, const sdpa_tensor* k_cache, int32_t num_splits);

/* ---------------------------------------------------------------------------------------
 * sdpa_decode_noalloc -- sdpa_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation). Same arguments,
 * result and kernels as sdpa_decode, minus the workspace: the split partials go to a device
 * array the library holds, sdpa_decode_noalloc_max_scratch_bytes() bytes (32 MiB) on every GPU
 * the library runs on, kept until the process ends. A call whose partials need more
 * (sdpa_decode_workspace_bytes() of the same arguments) returns SDPA_ERR_WORKSPACE without
 * launching anything. The call allocates nothing. All calls on one GPU share its array, so
 * calls that overlap on one GPU (on different streams, or from different threads without
 * ordering) race; calls ordered on one stream do not. Nothing in the array needs clearing
 * between calls: every partial a call reads it has written first.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_decode_noalloc(const sdpa_tensor* q, const sdpa_tensor* k_cache, const sdpa_tensor* v_cache,
                                         const int32_t* kv_lengths, float scale, int32_t num_splits,
                                         sdpa_tensor* out, void* stream);
SDPA_API size_t sdpa_decode_noalloc_max_scratch_bytes(void);

/* ---------------------------------------------------------------------------------------
 * kv_cache_update -- writes row t of k_new/v_new of batch b at cache position
 * write_index[b] + t (keras issue: a cache-update index says where new keys/values go; Flax
 * discussion: the cache grows one position per decode step). A bit-exact copy. Rows whose
 * position falls outside [0, capacity) are skipped.
 * k_cache, v_cache {D, Hkv, capacity, B}, in place; k_new, v_new {D, Hkv, T, B}; all four of one
 * dtype (F32, BF16 or F16). write_index device int32 [B].
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status kv_cache_update(sdpa_tensor* k_cache, sdpa_tensor* v_cache,
                            const sdpa_tensor* k_new, const sdpa_tensor* v_new,
                            const int32_t* write_index, void* stream);

/* ---------------------------------------------------------------------------------------
 * build_block_mask_info -- block information of a runtime (device) boolean mask (pull request
 * "Support dynamic masks in splash attention #25213"). mask U8 or U1 {Lkv, Lq, Hm|1, Bm|1};
 * bq >= 1, bkv a multiple of 32. A block is classed by its in-range elements; bits of a ragged
 * edge block past the mask are 0. storage: device memory of at least
 * sdpa_block_mask_info_bytes(); info: HOST struct, filled with pointers into storage. The
 * result is deterministic and bit-exact.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_block_mask_info_bytes(const sdpa_tensor* mask, int32_t bq, int32_t bkv, size_t* bytes);
SDPA_API sdpa_status build_block_mask_info(const sdpa_tensor* mask, int32_t bq, int32_t bkv,
                                  void* storage, size_t storage_bytes,
                                  sdpa_block_mask_info* info, void* stream);

/* ---------------------------------------------------------------------------------------
 * head_rms_norm -- per-head RMS normalisation (TensorTonic page "Static Arguments in jit"):
 * every head vector v becomes v / sqrt(mean(v^2) + eps). x, y {Dh, H, T, B}, F32, BF16 or F16 (same
 * dtype); fp32 arithmetic. y may alias x.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status head_rms_norm(const sdpa_tensor* x, sdpa_tensor* y, float eps, void* stream);

/* ---------------------------------------------------------------------------------------
 * sdpa_debug_allowed_mask -- writes allowed[b][h][i][j] (U8 {Lkv, Lq, Hq, B}) as the attention
 * kernels decide it: mask AND causal rule AND kv_lengths ("Arguments", the AND rule). For
 * bit-exact tests of the masking logic; arguments as in sdpa_fwd.
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_debug_allowed_mask(const sdpa_tensor* q, const sdpa_tensor* k,
                                    const sdpa_tensor* mask, const sdpa_block_mask_info* mask_info,
                                    int32_t is_causal, const int32_t* q_offset, int32_t q_offset_all,
                                    const int32_t* kv_lengths, int32_t kv_length_all,
                                    const int32_t* q_lengths, int32_t q_length_all,
                                    sdpa_tensor* allowed, void* stream);

/* ---------------------------------------------------------------------------------------
 * Measurement probes. They are not part of the attention operation: they measure the two
 * roofline denominators (the bf16 matrix-core rate and the HBM streaming-read rate) on the
 * device the library runs on, so that a kernel's fraction can be stated against the measured
 * rates as well as against the vendor's published peaks.
 *
 * sdpa_measure_mfma_bf16: `workgroups` workgroups of 256 threads (two per CU at most); every
 *   wave issues iters x 4 v_mfma_f32_32x32x16_bf16 on four independent accumulator chains and
 *   nothing else. Work = workgroups * 4 * iters * 4 * 32768 flops. sink: device float array of
 *   at least workgroups * 256 elements, overwritten with meaningless sums.
 * sdpa_measure_stream_read: reads `bytes` of device memory at src (16-byte aligned, bytes a
 *   multiple of 16) once, with 16-byte loads spread over `workgroups` workgroups of 256
 *   threads. sink: device uint32 array of at least workgroups * 4 elements, overwritten.
 * Both are asynchronous on `stream`; host-detectable errors: NULL pointers (NULL), sizes out of
 *   range or a misaligned src (SHAPE), a sink too small (WORKSPACE).
 * ------------------------------------------------------------------------------------- */
SDPA_API sdpa_status sdpa_measure_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, size_t sink_bytes,
                                            void* stream);
SDPA_API sdpa_status sdpa_measure_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                              size_t sink_bytes, void* stream);

/* Status text; detail of the last non-OK status on this thread (empty if none). */
SDPA_API const char* sdpa_status_string(int32_t status);
SDPA_API const char* sdpa_last_error(void);

/* Library version string, e.g. "sdpa_mi355x 0.1 gfx950". */
SDPA_API const char* sdpa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SDPA_MI355X_H */
