// fwd_generic.hip -- attention forward for any shape the ABI accepts (head dims up to 256,
// fp32, bf16 or f16 inputs, every masking option, packed sequences), with fp32 arithmetic and
// an accurate expf.
//
// The softmax is taken online over tiles of 64 keys, so the weights are never materialized
// (page "Neural Network primitives from NNlib.jl", section "Fused implementation"): one wave
// owns one query row; lanes score 64 keys at a time, the wave keeps the running max m and
// sum l, and rescales its output accumulator by exp(m_old - m_new) whenever the max grows.
// A row with no allowed key ends with l == 0 and is written as NaN (same section).
//
// This kernel serves the fp32 configurations and every shape the MFMA kernel does not take.
#include "device_common.h"

namespace sdpa {

namespace {

constexpr int kGenThreads = 256;                 // 4 waves = 4 query rows per workgroup
constexpr int kGenRows = kGenThreads / 64;
constexpr int kGenMaxD = 256;                    // largest head dim accepted

__global__ __launch_bounds__(kGenThreads) void fwd_generic_kernel(AttnArgs args) {
  __shared__ float q_lds[kGenRows][kGenMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y;
  // packed sequences: workgroup x takes tile x (kGenRows rows) of the segments (seg_locate),
  // and the segment is then a batch of one
  AttnArgs a = args;
  int i, b;
  if (args.q_seg) {
    SegView sv;
    if (!seg_locate(args, blockIdx.x, kGenRows, sv)) return;
    a = seg_args(args, sv);
    i = sv.tile * kGenRows + wave;
    b = 0;
  } else {
    i = blockIdx.x * kGenRows + wave;
    b = blockIdx.z;
  }
  if (i >= a.Lq) return;                         // whole wave leaves together; no block barriers below

  const int g = h / (a.Hq / a.Hkv);
  const int nkv = batch_kv_len(a, b);
  const int nq = batch_q_len(a, b);
  const int64_t off = batch_causal_offset(a, b);
  const int64_t o_row = b * a.o_sb + (int64_t)i * a.o_ss + h * a.o_sh;

  float* lse = a.lse ? a.lse + b * a.lse_sb + h * a.lse_sh + i : nullptr;
  if (i >= nq) {                                 // past q_lengths: output 0, attends nothing
    for (int d = lane; d < a.Dv; d += 64) store_elem(a.out, o_row + d, a.out_dtype, 0.f);
    if (lse && lane == 0) *lse = -INFINITY;
    return;
  }

  const int64_t q_row = b * a.q_sb + (int64_t)i * a.q_ss + h * a.q_sh;
  float ss = 0.f;
  for (int d = lane; d < a.D; d += 64) {
    const float x = load_elem(a.q, q_row + d, a.in_dtype);
    q_lds[wave][d] = x;
    ss += x * x;
  }
  if (a.qk_norm) {
    const float r = 1.0f / sqrtf(wave_sum(ss) / a.D + kRmsEps);
    for (int d = lane; d < a.D; d += 64) q_lds[wave][d] *= r;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int64_t k_base = b * a.k_sb + g * a.k_sh;
  const int64_t v_base = b * a.v_sb + g * a.v_sh;
  float m = -INFINITY, l = 0.f;
  float o[kGenMaxD / 64];
#pragma unroll
  for (int t = 0; t < kGenMaxD / 64; ++t) o[t] = 0.f;

  for (int j0 = 0; j0 < nkv; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (key_allowed(a, b, h, i, j, nkv, off)) {
      const int64_t k_row = k_base + (int64_t)j * a.k_ss;
      float dot = 0.f;
      for (int d = 0; d < a.D; ++d) dot += q_lds[wave][d] * load_elem(a.k, k_row + d, a.in_dtype);
      if (a.qk_norm) dot *= a.k_rinv[((int64_t)b * a.Lkv + j) * a.Hkv + g];
      s = dot * a.scale;
      if (a.bias) s += bias_at(a, b, h, i, j);
    }
    const float m_new = fmaxf(m, wave_max(s));
    if (m_new == -INFINITY) continue;            // nothing allowed yet (wave-uniform)
    const float p = (s == -INFINITY) ? 0.f : expf(s - m_new);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int t = 0; t < kGenMaxD / 64; ++t) o[t] *= alpha;
    const int n_here = min(64, nkv - j0);
    for (int jj = 0; jj < n_here; ++jj) {
      const float pj = __shfl(p, jj, 64);
      if (pj == 0.f) continue;                   // never touch the value row of a skipped key
      const int64_t v_row = v_base + (int64_t)(j0 + jj) * a.v_ss;
#pragma unroll
      for (int t = 0; t < kGenMaxD / 64; ++t) {
        const int d = lane + 64 * t;
        if (d < a.Dv) o[t] += pj * load_elem(a.v, v_row + d, a.in_dtype);
      }
    }
    m = m_new;
  }

  const float inv_l = (l > 0.f) ? 1.0f / l : NAN;
  if (lse && lane == 0) *lse = (l > 0.f) ? m + logf(l) : -INFINITY;
#pragma unroll
  for (int t = 0; t < kGenMaxD / 64; ++t) {
    const int d = lane + 64 * t;
    if (d < a.Dv) store_elem(a.out, o_row + d, a.out_dtype, (l > 0.f) ? o[t] * inv_l : inv_l);
  }
}

__global__ void debug_allowed_kernel(AttnArgs a, uint8_t* out, int64_t sb, int64_t sh, int64_t sq,
                                     int64_t sk) {
  const int64_t total = (int64_t)a.B * a.Hq * a.Lq * a.Lkv;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(e % a.Lkv);
    const int i = (int)((e / a.Lkv) % a.Lq);
    const int h = (int)((e / ((int64_t)a.Lkv * a.Lq)) % a.Hq);
    const int b = (int)(e / ((int64_t)a.Lkv * a.Lq * a.Hq));
    const int nkv = batch_kv_len(a, b);
    const int64_t off = batch_causal_offset(a, b);
    out[b * sb + h * sh + (int64_t)i * sq + (int64_t)j * sk] = key_allowed(a, b, h, i, j, nkv, off) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t s) {
  if (a.q_seg) {
    const int64_t n = packed_tiles_bound(a, kGenRows);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fwd_generic_kernel, dim3((unsigned)n, a.Hq, 1), dim3(kGenThreads), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid((a.Lq + kGenRows - 1) / kGenRows, a.Hq, a.B);
  hipLaunchKernelGGL(fwd_generic_kernel, grid, dim3(kGenThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_debug_allowed(const AttnArgs& a, uint8_t* out, int64_t sb, int64_t sh, int64_t sq,
                                int64_t sk, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.Hq * a.Lq * a.Lkv;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(debug_allowed_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                     a, out, sb, sh, sq, sk);
  return hipGetLastError();
}

}  // namespace sdpa
