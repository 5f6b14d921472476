// mask_info.hip -- block information of a runtime boolean mask.
//
// The pull request "Support dynamic masks in splash attention #25213" preprocesses a mask into
// per-block classes (empty / partial / full, int8), the list of blocks a kernel must visit, the
// index of each partial block's stored elements, and the partial blocks themselves; with a
// runtime mask the number of partial blocks is unknown in advance, so room for every block is
// reserved. The review suggests packing the 0/1 elements to save memory; here every partial
// block is stored as bits.
//
// Three stream-ordered passes, all deterministic:
//   1. classify: one workgroup per block counts the allowed in-range elements;
//   2. scan: one workgroup walks the blocks in flat order (mask batch, mask head, q-block,
//      kv-block) with an exclusive scan, writing row_ptr, data_next, mask_next and n_partial;
//   3. pack: one workgroup per partial block turns each row into bits with wave ballots and
//      writes them at its compacted index.
#include "device_common.h"

namespace sdpa {

namespace {

__device__ __forceinline__ void block_coords(const MaskInfoArgs& m, int64_t blk, int& bb, int& hh, int& qb,
                                             int& kb) {
  kb = (int)(blk % m.n_kb);
  qb = (int)((blk / m.n_kb) % m.n_qb);
  const int64_t bh = blk / ((int64_t)m.n_kb * m.n_qb);
  hh = (int)(bh % m.Mh);
  bb = (int)(bh / m.Mh);
}

__global__ __launch_bounds__(256) void mask_classify_kernel(MaskInfoArgs m) {
  __shared__ int partial_counts[4];
  const int64_t blk = blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
  const int64_t nblk = (int64_t)m.Mb * m.Mh * m.n_qb * m.n_kb;
  if (blk >= nblk) return;
  int bb, hh, qb, kb;
  block_coords(m, blk, bb, hh, qb, kb);
  const int r0 = qb * m.bq, c0 = kb * m.bkv;
  const int nr = min(m.bq, m.Lq - r0), nc = min(m.bkv, m.Lkv - c0);
  int count = 0;
  const int n = nr * nc;
  const int64_t row0 = bb * m.sb + hh * m.sh + (int64_t)r0 * m.sq;    // bytes (U8) or words (U1)
  if (m.u1 && m.sk == 1) {
    // whole words: the block's columns start on a word (bkv is a multiple of 32)
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(m.mask) + row0 + (c0 >> 5);
    const int nw = (nc + 31) >> 5, tail = nc & 31;
    for (int e = threadIdx.x; e < nr * nw; e += blockDim.x) {
      const int r = e / nw, w = e - r * nw;
      uint32_t bits = w0[(int64_t)r * m.sq + w];
      if (tail && w == nw - 1) bits &= (1u << tail) - 1u;
      count += __builtin_popcount(bits);
    }
  } else {
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
      const int r = e / nc, c = e - r * nc;
      count += mask_bit(m.mask, m.u1, row0 + (int64_t)r * m.sq, (int64_t)(c0 + c) * m.sk);
    }
  }
  // workgroup sum
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) count += __shfl_xor(count, o, 64);
  if ((threadIdx.x & 63) == 0) partial_counts[threadIdx.x >> 6] = count;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tot = partial_counts[0] + partial_counts[1] + partial_counts[2] + partial_counts[3];
    m.cls[blk] = (int8_t)(tot == 0 ? 0 : (tot == n ? 2 : 1));
  }
}

constexpr int kScanThreads = 1024;

// Exclusive scan of two 0/1 flags across the workgroup; returns prefixes and totals.
__device__ __forceinline__ void block_scan2(int a, int b, int& a_ex, int& b_ex, int& a_tot, int& b_tot) {
  __shared__ int wa[kScanThreads / 64], wb[kScanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ia = a, ib = b;                                  // inclusive wave scan
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ta = __shfl_up(ia, o, 64), tb = __shfl_up(ib, o, 64);
    if (lane >= o) { ia += ta; ib += tb; }
  }
  if (lane == 63) { wa[wave] = ia; wb[wave] = ib; }
  __syncthreads();
  int pa = 0, pb = 0;
  a_tot = 0; b_tot = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wave) { pa += wa[w]; pb += wb[w]; }
    a_tot += wa[w]; b_tot += wb[w];
  }
  a_ex = pa + ia - a;
  b_ex = pb + ib - b;
  __syncthreads();                                     // wa/wb reused by the next call
}

__global__ __launch_bounds__(kScanThreads) void mask_scan_kernel(MaskInfoArgs m) {
  const int64_t nblk = (int64_t)m.Mb * m.Mh * m.n_qb * m.n_kb;
  int run_ne = 0, run_pa = 0;
  for (int64_t base = 0; base < nblk; base += kScanThreads) {
    const int64_t idx = base + threadIdx.x;
    const int c = idx < nblk ? m.cls[idx] : 0;
    const int ne = c != 0, pa = c == 1;
    int ne_ex, pa_ex, ne_tot, pa_tot;
    block_scan2(ne, pa, ne_ex, pa_ex, ne_tot, pa_tot);
    if (idx < nblk) {
      const int kb = (int)(idx % m.n_kb);
      const int64_t row = idx / m.n_kb;
      if (kb == 0) m.row_ptr[row] = run_ne + ne_ex;
      if (ne) m.data_next[run_ne + ne_ex] = kb;
      m.next[idx] = pa ? run_pa + pa_ex : 0;
    }
    run_ne += ne_tot;
    run_pa += pa_tot;
  }
  if (threadIdx.x == 0) {
    m.row_ptr[(int64_t)m.Mb * m.Mh * m.n_qb] = run_ne;
    *m.n_partial = run_pa;
  }
}

__global__ __launch_bounds__(256) void mask_pack_kernel(MaskInfoArgs m) {
  const int64_t blk = blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
  const int64_t nblk = (int64_t)m.Mb * m.Mh * m.n_qb * m.n_kb;
  if (blk >= nblk || m.cls[blk] != 1) return;
  int bb, hh, qb, kb;
  block_coords(m, blk, bb, hh, qb, kb);
  const int r0 = qb * m.bq, c0 = kb * m.bkv;
  const int nr = min(m.bq, m.Lq - r0), nc = min(m.bkv, m.Lkv - c0);
  const int words = m.bkv / 32;
  uint32_t* dst = m.bits + (int64_t)m.next[blk] * m.bq * words;
  const int64_t row0 = bb * m.sb + hh * m.sh + (int64_t)r0 * m.sq;    // bytes (U8) or words (U1)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (m.u1 && m.sk == 1) {
    // the block's words as they are, bits past the mask cleared; one word per lane
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(m.mask) + row0 + (c0 >> 5);
    const int nw = (nc + 31) >> 5, tail = nc & 31;
    for (int r = wave; r < m.bq; r += blockDim.x >> 6) {
      for (int w = lane; w < words; w += 64) {
        uint32_t bits = (r < nr && w < nw) ? w0[(int64_t)r * m.sq + w] : 0u;
        if (tail && w == nw - 1) bits &= (1u << tail) - 1u;
        dst[(int64_t)r * words + w] = bits;
      }
    }
    return;
  }
  for (int r = wave; r < m.bq; r += blockDim.x >> 6) {
    for (int c = 0; c < m.bkv; c += 64) {
      const int col = c + lane;
      const bool bit = r < nr && col < nc && mask_bit(m.mask, m.u1, row0 + (int64_t)r * m.sq, (int64_t)(c0 + col) * m.sk);
      const uint64_t bal = __ballot(bit);
      if (lane == 0) dst[(int64_t)r * words + c / 32] = (uint32_t)bal;
      if (lane == 1 && c / 32 + 1 < words) dst[(int64_t)r * words + c / 32 + 1] = (uint32_t)(bal >> 32);
    }
  }
}

dim3 block_grid(int64_t nblk) {
  const int64_t x = nblk < 65535 ? nblk : 65535;
  return dim3((unsigned)x, (unsigned)((nblk + x - 1) / x));
}

}  // namespace

hipError_t launch_mask_info(const MaskInfoArgs& m, hipStream_t s) {
  const int64_t nblk = (int64_t)m.Mb * m.Mh * m.n_qb * m.n_kb;
  if (nblk == 0) {
    hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, m);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(mask_classify_kernel, block_grid(nblk), dim3(256), 0, s, m);
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, m);
  hipLaunchKernelGGL(mask_pack_kernel, block_grid(nblk), dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace sdpa
