// measure.hip -- the two probes that measure the roofline denominators on the device the
// library runs on: the bf16 matrix-core rate and the HBM streaming-read rate. They are not part
// of the attention operation; the benchmark reports every attention kernel's fraction against
// both these measured rates and the vendor's published peaks.
//
// * measure_mfma_kernel: 256 threads (4 waves) per workgroup, two workgroups per CU, so every
//   SIMD runs two waves, as the attention kernels do. Each wave issues only
//   v_mfma_f32_32x32x16_bf16 on four independent accumulator chains (an MFMA occupies the
//   matrix pipe for 8 passes; four chains keep each dependent issue that far apart). Work:
//   workgroups * 4 waves * iters * 4 chains * 32768 flops.
// * stream_read_kernel: a grid-stride read of 16-byte chunks with the nontemporal policy, four
//   chunks in flight per lane, consecutive lanes on consecutive chunks (1 KiB per wave
//   instruction), folded by XOR into one word per wave so that nothing is optimised away. The
//   buffer is meant to be much larger than the 256 MiB last-level cache, so the rate is the
//   HBM's. Of the read patterns tried on this GPU (grid-stride or one slab per workgroup, 4 or 8
//   loads in flight, 1024 to 16384 workgroups, with and without the nontemporal policy) this
//   one at 16384 workgroups of 256 was the fastest, at about 6.7 TB/s.
#include "mfma_common.h"

namespace sdpa {

namespace {

__global__ __launch_bounds__(256, 2) void measure_mfma_kernel(int iters, float* sink) {
  using E = In<false>;
  const int lane = threadIdx.x & 63;
  // operands that the compiler cannot treat as constants
  const float fa = 1.0f + 1e-3f * (float)lane, fb = 1.0f - 1e-3f * (float)(lane ^ 5);
  E::x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(fa * (float)(e + 1) * 1e-2f);
    b[e] = static_cast<__bf16>(fb * (float)(8 - e) * 1e-2f);
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = E::mfma(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u* s4 = reinterpret_cast<const v4u*>(src);
  for (; i + 3 * stride < n16; i += 4 * stride) {
    // nontemporal: each byte is read once, as the decode's cache rows are
    const v4u c0 = __builtin_nontemporal_load(s4 + i), c1 = __builtin_nontemporal_load(s4 + i + stride);
    const v4u c2 = __builtin_nontemporal_load(s4 + i + 2 * stride), c3 = __builtin_nontemporal_load(s4 + i + 3 * stride);
    x ^= c0.x ^ c0.y ^ c0.z ^ c0.w ^ c1.x ^ c1.y ^ c1.z ^ c1.w;
    x ^= c2.x ^ c2.y ^ c2.z ^ c2.w ^ c3.x ^ c3.y ^ c3.z ^ c3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 c0 = src[i];
    x ^= c0.x ^ c0.y ^ c0.z ^ c0.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

}  // namespace

hipError_t launch_measure_mfma(int workgroups, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(measure_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, s,
                     static_cast<const uint4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace sdpa
