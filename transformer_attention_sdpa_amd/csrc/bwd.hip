// bwd.hip -- the gradient of attention with respect to query, key, value and scale (page
// "Neural Network primitives from NNlib.jl", section "Fused implementation": the fused call's
// gradient forms the weights again tile by tile instead of storing them, and a query with no
// allowed key takes no part).
//
// With the log-sum-exp lse_i saved by the forward, the weight of a pair is
// P_ij = exp(s_ij - lse_i), and with D_i = <dO_i, O_i> (= sum_j P_ij <dO_i, v_j>) the chain rule
// gives dS_ij = P_ij (<dO_i, v_j> - D_i), dv_j = sum_i P_ij dO_i, dq_i = scale sum_j dS_ij k_j,
// dk_j = scale sum_i dS_ij q_i and dscale = sum_ij dS_ij <q_i, k_j>. Four passes, all
// deterministic (no atomics):
//   1. prep: D_i, and the lse of the rows that take part (+inf for the others);
//   2. dK/dV: a key's gradients, summed over the query heads of its group and all queries;
//   3. dQ: a query's gradient and its row share of dscale;
//   4. dscale: a fixed-order sum of the row shares.
// Passes 2 and 3 have a matrix-core form for bf16/f16 at head dims 64 and 128 (bwd_mfma.hip);
// the kernels here take every other case, in fp32 with an accurate expf.
#include "device_common.h"

namespace sdpa {

namespace {

constexpr int kBwdThreads = 256;                 // 4 waves
constexpr int kBwdMaxD = 256;

// ---- 1. prep: one wave per (b, h, i) ---------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(BwdArgs g) {
  const AttnArgs& a = g.a;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6);
  const int64_t n_rows = (int64_t)a.B * a.Hq * a.Lq;
  if (row >= n_rows) return;
  const int i = (int)(row % a.Lq);
  const int h = (int)((row / a.Lq) % a.Hq);
  const int b = (int)(row / ((int64_t)a.Lq * a.Hq));
  const float lse = g.lse[row];
  const bool part = i < batch_q_len(a, b) && lse > -INFINITY && lse < INFINITY;
  float acc = 0.f;
  if (part) {
    const int64_t o = b * a.o_sb + (int64_t)i * a.o_ss + h * a.o_sh;
    const int64_t d_ = b * g.do_sb + (int64_t)i * g.do_ss + h * g.do_sh;
    for (int d = lane; d < a.Dv; d += 64)
      acc += load_elem(a.out, o + d, a.out_dtype) * load_elem(g.dout, d_ + d, g.do_dtype);
    acc = wave_sum(acc);
  }
  if (lane == 0) {
    g.w_dsum[row] = part ? acc : 0.f;
    g.w_lse[row] = part ? lse : INFINITY;
  }
}

// ---- 2. dK/dV: one wave per key (b, kv head, j); lanes hold head-dim columns ------------------
// For 64 queries at a time every lane scores one query against the wave's key; the weights and
// dS values are then broadcast one query at a time and accumulated into the columns.
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_generic_kernel(BwdArgs g) {
  const AttnArgs& a = g.a;
  __shared__ float kv_lds[kBwdThreads / 64][2][kBwdMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kBwdThreads / 64) + wave;
  const int gk = blockIdx.y, b = blockIdx.z;
  if (j >= a.Lkv) return;                        // whole wave leaves; no block barriers below
  const int nkv = batch_kv_len(a, b), nq = batch_q_len(a, b);
  const int64_t off = batch_causal_offset(a, b);
  const int grp = a.Hq / a.Hkv;
  float* kl = kv_lds[wave][0];
  float* vl = kv_lds[wave][1];
  const int64_t k_row = b * a.k_sb + (int64_t)j * a.k_ss + gk * a.k_sh;
  const int64_t v_row = b * a.v_sb + (int64_t)j * a.v_ss + gk * a.v_sh;
  for (int d = lane; d < a.D; d += 64) kl[d] = load_elem(a.k, k_row + d, a.in_dtype);
  for (int d = lane; d < a.Dv; d += 64) vl[d] = load_elem(a.v, v_row + d, a.in_dtype);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  float dk[kBwdMaxD / 64], dv[kBwdMaxD / 64];
#pragma unroll
  for (int t = 0; t < kBwdMaxD / 64; ++t) dk[t] = dv[t] = 0.f;

  if (j < nkv) {
    for (int h = gk * grp; h < (gk + 1) * grp; ++h) {
      const int64_t wrow = ((int64_t)b * a.Hq + h) * a.Lq;
      for (int i0 = 0; i0 < nq; i0 += 64) {
        const int i = i0 + lane;
        float p = 0.f, ds = 0.f;
        if (i < nq && key_allowed(a, b, h, i, j, nkv, off)) {
          const float lse = g.w_lse[wrow + i];
          if (lse < INFINITY) {
            const int64_t q_row = b * a.q_sb + (int64_t)i * a.q_ss + h * a.q_sh;
            const int64_t d_row = b * g.do_sb + (int64_t)i * g.do_ss + h * g.do_sh;
            float dot = 0.f, dp = 0.f;
            for (int d = 0; d < a.D; ++d) dot += load_elem(a.q, q_row + d, a.in_dtype) * kl[d];
            for (int d = 0; d < a.Dv; ++d) dp += load_elem(g.dout, d_row + d, g.do_dtype) * vl[d];
            p = expf(dot * a.scale - lse);
            ds = p * (dp - g.w_dsum[wrow + i]);
          }
        }
        const int n_here = min(64, nq - i0);
        for (int r = 0; r < n_here; ++r) {
          const float pr = __shfl(p, r, 64), dsr = __shfl(ds, r, 64);
          if (pr == 0.f && dsr == 0.f) continue;  // wave-uniform
          const int ir = i0 + r;
          const int64_t q_row = b * a.q_sb + (int64_t)ir * a.q_ss + h * a.q_sh;
          const int64_t d_row = b * g.do_sb + (int64_t)ir * g.do_ss + h * g.do_sh;
#pragma unroll
          for (int t = 0; t < kBwdMaxD / 64; ++t) {
            const int d = lane + 64 * t;
            if (d < a.D) dk[t] += dsr * load_elem(a.q, q_row + d, a.in_dtype);
            if (d < a.Dv) dv[t] += pr * load_elem(g.dout, d_row + d, g.do_dtype);
          }
        }
      }
    }
  }
  const int64_t dk_row = b * g.dk_sb + (int64_t)j * g.dk_ss + gk * g.dk_sh;
  const int64_t dv_row = b * g.dv_sb + (int64_t)j * g.dv_ss + gk * g.dv_sh;
#pragma unroll
  for (int t = 0; t < kBwdMaxD / 64; ++t) {
    const int d = lane + 64 * t;
    if (d < a.D) store_elem(g.dk, dk_row + d, g.dk_dtype, dk[t] * a.scale);
    if (d < a.Dv) store_elem(g.dv, dv_row + d, g.dv_dtype, dv[t]);
  }
}

// ---- 3. dQ: one wave per query (b, h, i); lanes score 64 keys at a time ----------------------
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_generic_kernel(BwdArgs g) {
  const AttnArgs& a = g.a;
  __shared__ float qd_lds[kBwdThreads / 64][2][kBwdMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kBwdThreads / 64) + wave;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= a.Lq) return;
  const int gk = h / (a.Hq / a.Hkv);
  const int nkv = batch_kv_len(a, b);
  const int64_t off = batch_causal_offset(a, b);
  const int64_t wrow = ((int64_t)b * a.Hq + h) * a.Lq + i;
  const float lse = g.w_lse[wrow], dsum = g.w_dsum[wrow];
  float* ql = qd_lds[wave][0];
  float* dl = qd_lds[wave][1];
  const int64_t q_row = b * a.q_sb + (int64_t)i * a.q_ss + h * a.q_sh;
  const int64_t d_row = b * g.do_sb + (int64_t)i * g.do_ss + h * g.do_sh;
  for (int d = lane; d < a.D; d += 64) ql[d] = load_elem(a.q, q_row + d, a.in_dtype);
  for (int d = lane; d < a.Dv; d += 64) dl[d] = load_elem(g.dout, d_row + d, g.do_dtype);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  float dq[kBwdMaxD / 64];
#pragma unroll
  for (int t = 0; t < kBwdMaxD / 64; ++t) dq[t] = 0.f;
  float dsc = 0.f;
  const int64_t k_base = b * a.k_sb + gk * a.k_sh;
  const int64_t v_base = b * a.v_sb + gk * a.v_sh;
  if (lse < INFINITY) {                          // the row takes part (wave-uniform)
    for (int j0 = 0; j0 < nkv; j0 += 64) {
      const int j = j0 + lane;
      float ds = 0.f;
      if (key_allowed(a, b, h, i, j, nkv, off)) {
        float dot = 0.f, dp = 0.f;
        for (int d = 0; d < a.D; ++d) dot += ql[d] * load_elem(a.k, k_base + (int64_t)j * a.k_ss + d, a.in_dtype);
        for (int d = 0; d < a.Dv; ++d) dp += dl[d] * load_elem(a.v, v_base + (int64_t)j * a.v_ss + d, a.in_dtype);
        const float p = expf(dot * a.scale - lse);
        ds = p * (dp - dsum);
        dsc += ds * dot;
      }
      const int n_here = min(64, nkv - j0);
      for (int r = 0; r < n_here; ++r) {
        const float dsr = __shfl(ds, r, 64);
        if (dsr == 0.f) continue;                // wave-uniform
        const int64_t k_row = k_base + (int64_t)(j0 + r) * a.k_ss;
#pragma unroll
        for (int t = 0; t < kBwdMaxD / 64; ++t) {
          const int d = lane + 64 * t;
          if (d < a.D) dq[t] += dsr * load_elem(a.k, k_row + d, a.in_dtype);
        }
      }
    }
  }
  dsc = wave_sum(dsc);
  if (lane == 0) g.w_dsc[wrow] = dsc;
  const int64_t dq_row = b * g.dq_sb + (int64_t)i * g.dq_ss + h * g.dq_sh;
#pragma unroll
  for (int t = 0; t < kBwdMaxD / 64; ++t) {
    const int d = lane + 64 * t;
    if (d < a.D) store_elem(g.dq, dq_row + d, g.dq_dtype, dq[t] * a.scale);
  }
}

// ---- 4. dscale: one workgroup, a fixed order of fp64 sums --------------------------------------
__global__ __launch_bounds__(kBwdThreads) void bwd_dscale_kernel(const float* part, int64_t n, float* out) {
  __shared__ double red[kBwdThreads];
  double acc = 0.0;
  for (int64_t e = threadIdx.x; e < n; e += kBwdThreads) acc += (double)part[e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kBwdThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = (float)red[0];
}

}  // namespace

bool bwd_mfma_supports(const BwdArgs& g);
hipError_t launch_bwd_mfma_dkdv(const BwdArgs& g, hipStream_t s);
hipError_t launch_bwd_mfma_dq(const BwdArgs& g, hipStream_t s);

hipError_t launch_bwd(const BwdArgs& g, hipStream_t s) {
  const AttnArgs& a = g.a;
  const int64_t n_rows = (int64_t)a.B * a.Hq * a.Lq;
  const int rpw = kBwdThreads / 64;
  if (n_rows > 0) {
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((n_rows + rpw - 1) / rpw)), dim3(kBwdThreads), 0, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool mf = bwd_mfma_supports(g);
  if (a.Lkv > 0 && a.B > 0) {
    if (mf) {
      hipError_t e = launch_bwd_mfma_dkdv(g, s);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(bwd_dkdv_generic_kernel, dim3((a.Lkv + rpw - 1) / rpw, a.Hkv, a.B), dim3(kBwdThreads), 0, s,
                         g);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (a.Lq > 0 && a.B > 0) {
    if (mf) {
      hipError_t e = launch_bwd_mfma_dq(g, s);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(bwd_dq_generic_kernel, dim3((a.Lq + rpw - 1) / rpw, a.Hq, a.B), dim3(kBwdThreads), 0, s, g);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (g.dscale) {
    hipLaunchKernelGGL(bwd_dscale_kernel, dim3(1), dim3(kBwdThreads), 0, s, g.w_dsc, n_rows, g.dscale);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace sdpa
