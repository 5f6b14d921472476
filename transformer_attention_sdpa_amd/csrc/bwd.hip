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
//   4. dscale: a fixed-order sum of the row shares, in two stages.
// Passes 2 and 3 have a matrix-core form for bf16/f16 at head dims 64 and 128 (bwd_mfma.hip);
// the kernels here take every other case, in fp32 with an accurate expf.
#include "device_common.h"

namespace sdpa {

namespace {

constexpr int kBwdThreads = 256;                 // 4 waves
constexpr int kBwdMaxD = 256;

// ---- 1. prep: 16 lanes per (b, h, i) row, 16 rows per workgroup ------------------------------
// Each lane takes 8 consecutive head-dim elements at a time (one 16-byte load of 16-bit data,
// two of fp32) when the rows allow vector loads (vec), else single elements.
__device__ __forceinline__ void load8(const void* base, int64_t idx, int dtype, float* x) {
  if (dtype == SDPA_F32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    return;
  }
  const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (dtype == SDPA_BF16) {
      x[2 * t] = bf16_bits_to_float((uint16_t)w[t]);
      x[2 * t + 1] = bf16_bits_to_float((uint16_t)(w[t] >> 16));
    } else {
      x[2 * t] = f16_bits_to_float((uint16_t)w[t]);
      x[2 * t + 1] = f16_bits_to_float((uint16_t)(w[t] >> 16));
    }
  }
}

constexpr int kPrepRows = 4;                     // rows per 16-lane group
constexpr int kPastRange = 0x7ffffff0;           // a buffer offset past every range used here

// The 16-lane sums of a group's rows, then the row statistics (BwdArgs) by lane 0 of the group
__device__ __forceinline__ void prep_store(const BwdArgs& g, float (&acc)[kPrepRows], const float (&lse)[kPrepRows],
                                           int i0, int64_t row0, int nq, int l16, int stat_mfma) {
  const AttnArgs& a = g.a;
#pragma unroll
  for (int r = 0; r < kPrepRows; ++r) {
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) acc[r] += __shfl_xor(acc[r], m, 64);
    const bool in = i0 + r < a.Lq;
    const bool part = in && i0 + r < nq && lse[r] > -INFINITY && lse[r] < INFINITY;
    if (in && l16 == 0) {
      if (stat_mfma) {                     // the matrix-core route's form (BwdArgs)
        g.w_dsum[row0 + r] = part ? -acc[r] : 0.f;
        g.w_lse[row0 + r] = part ? -lse[r] / a.scale : -INFINITY;
      } else {
        g.w_dsum[row0 + r] = part ? acc[r] : 0.f;
        g.w_lse[row0 + r] = part ? lse[r] : INFINITY;
      }
    }
  }
}

__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(BwdArgs g, int vec, int stat_mfma) {
  const AttnArgs& a = g.a;
  const int l16 = threadIdx.x & 15;
  // grid: x = block of kPrepRows * 16 queries * Hq + head, y = batch (a scalar division per
  // workgroup, none per row); rows of the stats are [b][h][i]. Head innermost: workgroups that
  // run together read the heads of the same rows, i.e. whole contiguous rows of O and dO.
  const int ib = (int)blockIdx.x / a.Hq, h = (int)blockIdx.x - ib * a.Hq, b = blockIdx.y;
  const int i0 = (ib * (kBwdThreads / 16) + (threadIdx.x >> 4)) * kPrepRows;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.Lq + i0;
  const int nq = batch_q_len(a, b);
  // O and dO are read for every row in range, in parallel with lse, and for the group's rows
  // together (one memory latency for all of them); a row that takes no part discards its sum
  // (the 16-lane sums stay within one row). No early exit: shuffles below.
  float lse[kPrepRows], acc[kPrepRows];
#pragma unroll
  for (int r = 0; r < kPrepRows; ++r) {
    lse[r] = i0 + r < a.Lq ? g.lse[row0 + r] : 0.f;
    acc[r] = 0.f;
  }
  const int64_t ob = b * a.o_sb + h * a.o_sh, db = b * g.do_sb + h * g.do_sh;
  if (vec && a.Dv <= 128) {                        // one 8-element run per lane and row
    float x[kPrepRows][8], y[kPrepRows][8];
#pragma unroll
    for (int r = 0; r < kPrepRows; ++r) {
      if (i0 + r < a.Lq && 8 * l16 < a.Dv) {
        load8(a.out, ob + (int64_t)(i0 + r) * a.o_ss + 8 * l16, a.out_dtype, x[r]);
        load8(g.dout, db + (int64_t)(i0 + r) * g.do_ss + 8 * l16, g.do_dtype, y[r]);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) x[r][t] = y[r][t] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < kPrepRows; ++r)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[r] = fmaf(x[r][t], y[r][t], acc[r]);
  } else {
#pragma unroll
    for (int r = 0; r < kPrepRows; ++r) {
      if (i0 + r >= a.Lq) continue;
      const int64_t o = ob + (int64_t)(i0 + r) * a.o_ss;
      const int64_t d_ = db + (int64_t)(i0 + r) * g.do_ss;
      if (vec) {
        for (int d = 8 * l16; d < a.Dv; d += 128) {
          float x[8], y[8];
          load8(a.out, o + d, a.out_dtype, x);
          load8(g.dout, d_ + d, g.do_dtype, y);
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[r] = fmaf(x[t], y[t], acc[r]);
        }
      } else {
        for (int d = l16; d < a.Dv; d += 16)
          acc[r] += load_elem(a.out, o + d, a.out_dtype) * load_elem(g.dout, d_ + d, g.do_dtype);
      }
    }
  }
  prep_store(g, acc, lse, i0, row0, nq, l16, stat_mfma);
}

// 16-bit O and dO, Dv <= 128, rows of whole 16-byte runs: the rows of bwd_prep_kernel by buffer
// loads whose range checks stand in for the row and head-dim limits (a load past them reads 0),
// so the lse and all 8 row loads of a lane go out together, with no branch between them
template <int OD, int DD>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep16_kernel(BwdArgs g, int stat_mfma) {
  const AttnArgs& a = g.a;
  const int l16 = threadIdx.x & 15;
  const int ib = (int)blockIdx.x / a.Hq, h = (int)blockIdx.x - ib * a.Hq, b = blockIdx.y;
  const int i0 = (ib * (kBwdThreads / 16) + (threadIdx.x >> 4)) * kPrepRows;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.Lq + i0;
  const int nq = batch_q_len(a, b);
  auto rsrc = [](const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t ro = rsrc(static_cast<const uint16_t*>(a.out) + b * a.o_sb + h * a.o_sh,
                                         (int64_t)a.Lq * a.o_ss * 2);
  const __amdgpu_buffer_rsrc_t rd = rsrc(static_cast<const uint16_t*>(g.dout) + b * g.do_sb + h * g.do_sh,
                                         (int64_t)a.Lq * g.do_ss * 2);
  const __amdgpu_buffer_rsrc_t rl = rsrc(g.lse + ((int64_t)b * a.Hq + h) * a.Lq, (int64_t)a.Lq * 4);
  const bool lane_in = 8 * l16 < a.Dv;
  uint4 xo[kPrepRows], xd[kPrepRows];
  float lse[kPrepRows], acc[kPrepRows];
#pragma unroll
  for (int r = 0; r < kPrepRows; ++r) {
    const int i = i0 + r;
    lse[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * i, 0, 0));
    const int oo = lane_in ? i * (int)(a.o_ss * 2) + 16 * l16 : kPastRange;
    const int od = lane_in ? i * (int)(g.do_ss * 2) + 16 * l16 : kPastRange;
    xo[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ro, oo, 0, 0));
    xd[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, od, 0, 0));
  }
  auto f = [](uint32_t w, bool hi, int dt) {
    const uint16_t x = hi ? (uint16_t)(w >> 16) : (uint16_t)w;
    return dt == SDPA_BF16 ? bf16_bits_to_float(x) : f16_bits_to_float(x);
  };
#pragma unroll
  for (int r = 0; r < kPrepRows; ++r) {
    const uint32_t wo[4] = {xo[r].x, xo[r].y, xo[r].z, xo[r].w}, wd[4] = {xd[r].x, xd[r].y, xd[r].z, xd[r].w};
    float s_ = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s_ = fmaf(f(wo[t], false, OD), f(wd[t], false, DD), s_);
      s_ = fmaf(f(wo[t], true, OD), f(wd[t], true, DD), s_);
    }
    acc[r] = s_;
  }
  prep_store(g, acc, lse, i0, row0, nq, l16, stat_mfma);
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

// ---- 4. dscale: a fixed-order sum in two stages ----------------------------------------------
// Stage 1: workgroup c sums rows [c * kDscChunk, (c + 1) * kDscChunk) (each thread 16 of them,
// then a tree in LDS) into part2[c]; stage 2: one workgroup sums part2 the same way. The order
// of every addition is fixed by the sizes alone, so the result is repeatable.
constexpr int kDscChunk = kBwdThreads * 16;

__device__ __forceinline__ double block_sum(double acc) {
  __shared__ double red[kBwdThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kBwdThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}

__global__ __launch_bounds__(kBwdThreads) void bwd_dscale_stage1(const float* part, int64_t n, double* part2) {
  const int64_t base = (int64_t)blockIdx.x * kDscChunk + threadIdx.x;
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t e = base + (int64_t)u * kBwdThreads;
    if (e < n) acc += (double)part[e];
  }
  const double t = block_sum(acc);
  if (threadIdx.x == 0) part2[blockIdx.x] = t;
}

// One workgroup over at most kDscSmall float shares (fixed order, fp64 sums)
constexpr int64_t kDscSmall = 65536;
__global__ __launch_bounds__(kBwdThreads) void bwd_dscale_small(const float* part, int64_t n, float* out) {
  double acc = 0.0;
  // buffer loads: past n they read 0, so the 16 loads go out together with no branch between
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(part), (short)0,
                                                                      (int)(n * 4), 0x00020000);
  for (int base = threadIdx.x; base < n; base += 16 * kBwdThreads) {
    float v[16];                                   // 16 loads in flight at once
#pragma unroll
    for (int u = 0; u < 16; ++u)
      v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 4 * (base + u * kBwdThreads), 0, 0));
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += (double)v[u];
  }
  const double t = block_sum(acc);
  if (threadIdx.x == 0) *out = (float)t;
}

__global__ __launch_bounds__(kBwdThreads) void bwd_dscale_stage2(const double* part2, int64_t n, float* out) {
  double acc = 0.0;
  for (int64_t e = threadIdx.x; e < n; e += kBwdThreads) acc += part2[e];
  const double t = block_sum(acc);
  if (threadIdx.x == 0) *out = (float)t;
}

}  // namespace

bool bwd_stores_ds(const BwdArgs& g);
hipError_t launch_bwd_mfma_dkdv(const BwdArgs& g, hipStream_t s);
hipError_t launch_bwd_mfma_dq(const BwdArgs& g, hipStream_t s);

hipError_t launch_bwd(const BwdArgs& g, hipStream_t s) {
  const AttnArgs& a = g.a;
  const int64_t n_rows = (int64_t)a.B * a.Hq * a.Lq;
  const int rpw = kBwdThreads / 64;
  const bool mf = bwd_mfma_supports(g);
  if (n_rows > 0) {
    const int pe = a.out_dtype == SDPA_F32 ? 4 : 8, de = g.do_dtype == SDPA_F32 ? 4 : 8;   // elements per 16 B
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const int vec = (a.Dv % 8 == 0) && al16(a.out) && al16(g.dout) && ((a.o_sb | a.o_ss | a.o_sh) % pe == 0) &&
                    ((g.do_sb | g.do_ss | g.do_sh) % de == 0);
    const int rpb = kBwdThreads / 16 * kPrepRows;
    const dim3 grid((unsigned)((int64_t)((a.Lq + rpb - 1) / rpb) * a.Hq), (unsigned)a.B);
    auto is16 = [](int dt) { return dt == SDPA_BF16 || dt == SDPA_F16; };
    // 32-bit buffer offsets: every row start and the past-range offset stay apart
    const int64_t lim = kPastRange - 256;
    if (vec && a.Dv <= 128 && is16(a.out_dtype) && is16(g.do_dtype) && (int64_t)(a.Lq + rpb) * a.o_ss * 2 < lim &&
        (int64_t)(a.Lq + rpb) * g.do_ss * 2 < lim && (int64_t)(a.Lq + rpb) * 4 < lim) {
      const bool ob = a.out_dtype == SDPA_BF16, db = g.do_dtype == SDPA_BF16;
      if (ob && db)
        hipLaunchKernelGGL((bwd_prep16_kernel<SDPA_BF16, SDPA_BF16>), grid, dim3(kBwdThreads), 0, s, g, mf ? 1 : 0);
      else if (ob)
        hipLaunchKernelGGL((bwd_prep16_kernel<SDPA_BF16, SDPA_F16>), grid, dim3(kBwdThreads), 0, s, g, mf ? 1 : 0);
      else if (db)
        hipLaunchKernelGGL((bwd_prep16_kernel<SDPA_F16, SDPA_BF16>), grid, dim3(kBwdThreads), 0, s, g, mf ? 1 : 0);
      else
        hipLaunchKernelGGL((bwd_prep16_kernel<SDPA_F16, SDPA_F16>), grid, dim3(kBwdThreads), 0, s, g, mf ? 1 : 0);
    } else {
      hipLaunchKernelGGL(bwd_prep_kernel, grid, dim3(kBwdThreads), 0, s, g, vec, mf ? 1 : 0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
    // the stored-dS route sums the dK/dV workgroups' shares, the other the dQ rows' shares
    const bool ds = mf && bwd_stores_ds(g);
    const int64_t n = ds ? (a.Lkv > 0 ? bwd_dkdv_workgroups(a.B, a.Hkv, a.Lkv) * 8 : 0) : n_rows;
    const float* part = ds ? g.w_dsp : g.w_dsc;
    double* part2 = ds ? g.w_dsc2_ds : g.w_dsc2;
    if (n <= kDscSmall) {
      hipLaunchKernelGGL(bwd_dscale_small, dim3(1), dim3(kBwdThreads), 0, s, part, n, g.dscale);
      return hipGetLastError();
    }
    const int64_t n2 = (n + kDscChunk - 1) / kDscChunk;
    if (n2 > 0) {
      hipLaunchKernelGGL(bwd_dscale_stage1, dim3((unsigned)n2), dim3(kBwdThreads), 0, s, part, n, part2);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bwd_dscale_stage2, dim3(1), dim3(kBwdThreads), 0, s, part2, n2, g.dscale);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace sdpa
