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
//   1. classify: one workgroup per block counts the allowed in-range elements (16 mask bytes
//      per load where the rows allow it);
//   2. scan: one workgroup walks the blocks in flat order (mask batch, mask head, q-block,
//      kv-block), 4 consecutive blocks per thread and round, with an exclusive scan, writing
//      row_ptr, data_next, mask_next and n_partial;
//   3. pack: one workgroup per partial block turns each row into bits (16 bytes to 16 bits per
//      thread, or with wave ballots where rows do not allow 16-byte loads) and writes them at
//      its compacted index.
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

// U8 16-byte paths: a byte's high bit in ((x & 0x7f7f7f7f) + 0x7f7f7f7f) | x is set exactly
// when the byte is nonzero.
__device__ __forceinline__ uint32_t nonzero_bytes_hi(uint32_t x) {
  return (((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;
}
// the four byte flags of a word as a nibble (bit k = byte k nonzero): the multiply moves bit
// 7 + 8k to bit 28 + k, and no other product lands in bits 28..31
__device__ __forceinline__ uint32_t nonzero_nibble(uint32_t x) { return (nonzero_bytes_hi(x) * 0x00204081u) >> 28; }

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
  } else if (m.vec16 && (nc & 15) == 0) {
    // 16 bytes per load: rows of nc / 16 chunks
    const int cpr = nc >> 4;
    const uint8_t* b0 = m.mask + row0 + c0;
    for (int e = threadIdx.x; e < nr * cpr; e += blockDim.x) {
      const int r = e / cpr, ch = e - r * cpr;
      const uint4 x = *reinterpret_cast<const uint4*>(b0 + (int64_t)r * m.sq + 16 * ch);
      count += __builtin_popcount(nonzero_bytes_hi(x.x)) + __builtin_popcount(nonzero_bytes_hi(x.y)) +
               __builtin_popcount(nonzero_bytes_hi(x.z)) + __builtin_popcount(nonzero_bytes_hi(x.w));
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

constexpr int kScanPer = 4;                          // consecutive blocks per thread and round

__global__ __launch_bounds__(kScanThreads) void mask_scan_kernel(MaskInfoArgs m) {
  const int64_t nblk = (int64_t)m.Mb * m.Mh * m.n_qb * m.n_kb;
  int run_ne = 0, run_pa = 0;
  for (int64_t base = 0; base < nblk; base += (int64_t)kScanThreads * kScanPer) {
    // each thread sums its kScanPer blocks, the workgroup scans the sums, and each thread then
    // walks its blocks from its own starting offsets
    const int64_t i0 = base + (int64_t)threadIdx.x * kScanPer;
    int cl[kScanPer], ne_sum = 0, pa_sum = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      cl[j] = i0 + j < nblk ? m.cls[i0 + j] : 0;
      ne_sum += cl[j] != 0;
      pa_sum += cl[j] == 1;
    }
    int ne_ex, pa_ex, ne_tot, pa_tot;
    block_scan2(ne_sum, pa_sum, ne_ex, pa_ex, ne_tot, pa_tot);
    int ne_at = run_ne + ne_ex, pa_at = run_pa + pa_ex;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t idx = i0 + j;
      if (idx < nblk) {
        const int kb = (int)(idx % m.n_kb);
        const int64_t row = idx / m.n_kb;
        if (kb == 0) m.row_ptr[row] = ne_at;
        if (cl[j] != 0) m.data_next[ne_at] = kb;
        m.next[idx] = cl[j] == 1 ? pa_at : 0;
        ne_at += cl[j] != 0;
        pa_at += cl[j] == 1;
      }
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
    // every thread takes (row, word) pairs, so all lanes load at once
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(m.mask) + row0 + (c0 >> 5);
    const int nw = (nc + 31) >> 5, tail = nc & 31;
    for (int e = threadIdx.x; e < m.bq * words; e += blockDim.x) {
      const int r = e / words, w = e - r * words;
      uint32_t bits = (r < nr && w < nw) ? w0[(int64_t)r * m.sq + w] : 0u;
      if (tail && w == nw - 1) bits &= (1u << tail) - 1u;
      dst[(int64_t)r * words + w] = bits;
    }
    return;
  }
  if (m.vec16 && (nc & 15) == 0) {
    // 16 bytes -> 16 bits per thread, written as the low or high half of a word
    const int cpr = m.bkv >> 4;                        // 16-column chunks of a stored row
    const uint8_t* b0 = m.mask + row0 + c0;
    uint16_t* dst16 = reinterpret_cast<uint16_t*>(dst);
    for (int e = threadIdx.x; e < m.bq * cpr; e += blockDim.x) {
      const int r = e / cpr, ch = e - r * cpr;
      uint32_t bits = 0;
      if (r < nr && 16 * ch < nc) {
        const uint4 x = *reinterpret_cast<const uint4*>(b0 + (int64_t)r * m.sq + 16 * ch);
        bits = nonzero_nibble(x.x) | (nonzero_nibble(x.y) << 4) | (nonzero_nibble(x.z) << 8) |
               (nonzero_nibble(x.w) << 12);
      }
      dst16[(int64_t)r * words * 2 + ch] = (uint16_t)bits;
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
