// norm.hip -- per-head RMS normalisation (TensorTonic page "Static Arguments in jit", its
// normalisation formula): a head vector v of width Dh becomes v / sqrt(mean(v^2) + eps).
//
// Two kernels: head_rms_norm writes the normalised vectors; row_rinv writes only the factor
// 1/sqrt(mean(v^2) + eps) of every key head vector, which the attention kernels apply to the
// logits (s = scale * r_q * r_k * <q, k>), the same number as normalising both vectors first.
// One wave per vector; fp32 arithmetic.
#include "device_common.h"

namespace sdpa {

namespace {

__global__ __launch_bounds__(256) void head_rms_norm_kernel(const void* x, void* y, int dtype, int64_t xsb,
                                                            int64_t xss, int64_t xsh, int64_t ysb, int64_t yss,
                                                            int64_t ysh, int B, int T, int H, int Dh, float eps) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;        // over (b, t, h)
  if (row >= (int64_t)B * T * H) return;
  const int h = (int)(row % H);
  const int t = (int)((row / H) % T);
  const int b = (int)(row / ((int64_t)H * T));
  const int64_t xo = b * xsb + (int64_t)t * xss + h * xsh;
  const int64_t yo = b * ysb + (int64_t)t * yss + h * ysh;
  float ss = 0.f;
  for (int d = lane; d < Dh; d += 64) {
    const float v = load_elem(x, xo + d, dtype);
    ss += v * v;
  }
  const float r = 1.0f / sqrtf(wave_sum(ss) / Dh + eps);
  for (int d = lane; d < Dh; d += 64) store_elem(y, yo + d, dtype, load_elem(x, xo + d, dtype) * r);
}

__global__ __launch_bounds__(256) void row_rinv_kernel(const void* x, int dtype, int64_t sb, int64_t ss_,
                                                       int64_t sh, int B, int L, int H, int D, float eps,
                                                       float* rinv) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;        // over (b, l, h), output [B][L][H]
  if (row >= (int64_t)B * L * H) return;
  const int h = (int)(row % H);
  const int l = (int)((row / H) % L);
  const int b = (int)(row / ((int64_t)H * L));
  const int64_t xo = b * sb + (int64_t)l * ss_ + h * sh;
  float ss = 0.f;
  for (int d = lane; d < D; d += 64) {
    const float v = load_elem(x, xo + d, dtype);
    ss += v * v;
  }
  ss = wave_sum(ss);
  if (lane == 0) rinv[row] = 1.0f / sqrtf(ss / D + eps);
}

}  // namespace

hipError_t launch_head_rms_norm(const void* x, void* y, int dtype, int64_t xsb, int64_t xss, int64_t xsh,
                                int64_t ysb, int64_t yss, int64_t ysh, int B, int T, int H, int Dh,
                                float eps, hipStream_t s) {
  const int64_t rows = (int64_t)B * T * H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(head_rms_norm_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, y, dtype, xsb,
                     xss, xsh, ysb, yss, ysh, B, T, H, Dh, eps);
  return hipGetLastError();
}

hipError_t launch_row_rinv(const void* x, int dtype, int64_t sb, int64_t ss, int64_t sh, int B, int L, int H,
                           int D, float eps, float* rinv, hipStream_t s) {
  const int64_t rows = (int64_t)B * L * H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(row_rinv_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, dtype, sb, ss, sh,
                     B, L, H, D, eps, rinv);
  return hipGetLastError();
}

}  // namespace sdpa
