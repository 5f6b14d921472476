// kv_cache.hip -- KV-cache update at a per-sequence write index.
//
// The keras issue "MultiHeadAttention is missing a position_bias call argument, ..." proposes
// separate key and value caches plus an index that says where new keys and values are
// written; the Flax discussion on nnx.MultiHeadAttention with decode=True shows the cache
// growing by one position per step. Row t of the new keys/values of sequence b lands at
// position write_index[b] + t; positions outside the cache are skipped. A pure copy of the
// element bits, so the result is bit-exact.
//
// One thread moves one 16-byte chunk when the rows are 16-byte aligned and a multiple of 16
// bytes long, else one element.
#include "device_common.h"

namespace sdpa {

namespace {

struct CacheArgs {
  char* kc; char* vc; const char* kn; const char* vn;
  int elem, B, T, H, D, cap;
  int64_t kc_sb, kc_ss, kc_sh, vc_sb, vc_ss, vc_sh, kn_sb, kn_ss, kn_sh, vn_sb, vn_ss, vn_sh;  // bytes
  const int32_t* widx;
};

template <int CHUNK>
__global__ __launch_bounds__(256) void kv_cache_update_kernel(CacheArgs c) {
  const int per_row = (c.D * c.elem) / CHUNK;
  const int64_t total = (int64_t)c.B * c.T * c.H * per_row;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int part = (int)(e % per_row);
    const int h = (int)((e / per_row) % c.H);
    const int t = (int)((e / ((int64_t)per_row * c.H)) % c.T);
    const int b = (int)(e / ((int64_t)per_row * c.H * c.T));
    const int64_t pos = (int64_t)c.widx[b] + t;
    if (pos < 0 || pos >= c.cap) continue;
    const int64_t off = (int64_t)part * CHUNK;
    const char* ks = c.kn + b * c.kn_sb + t * c.kn_ss + h * c.kn_sh + off;
    const char* vs = c.vn + b * c.vn_sb + t * c.vn_ss + h * c.vn_sh + off;
    char* kd = c.kc + b * c.kc_sb + pos * c.kc_ss + h * c.kc_sh + off;
    char* vd = c.vc + b * c.vc_sb + pos * c.vc_ss + h * c.vc_sh + off;
    if constexpr (CHUNK == 16) {
      *reinterpret_cast<uint4*>(kd) = *reinterpret_cast<const uint4*>(ks);
      *reinterpret_cast<uint4*>(vd) = *reinterpret_cast<const uint4*>(vs);
    } else if constexpr (CHUNK == 4) {
      *reinterpret_cast<uint32_t*>(kd) = *reinterpret_cast<const uint32_t*>(ks);
      *reinterpret_cast<uint32_t*>(vd) = *reinterpret_cast<const uint32_t*>(vs);
    } else {
      *reinterpret_cast<uint16_t*>(kd) = *reinterpret_cast<const uint16_t*>(ks);
      *reinterpret_cast<uint16_t*>(vd) = *reinterpret_cast<const uint16_t*>(vs);
    }
  }
}

}  // namespace

hipError_t launch_kv_cache_update(void* kc, void* vc, const void* kn, const void* vn, int elem_bytes,
                                  int B, int T, int H, int D, int cap,
                                  int64_t kc_sb, int64_t kc_ss, int64_t kc_sh,
                                  int64_t vc_sb, int64_t vc_ss, int64_t vc_sh,
                                  int64_t kn_sb, int64_t kn_ss, int64_t kn_sh,
                                  int64_t vn_sb, int64_t vn_ss, int64_t vn_sh,
                                  const int32_t* write_index, hipStream_t s) {
  const int64_t e = elem_bytes;
  CacheArgs c{static_cast<char*>(kc), static_cast<char*>(vc), static_cast<const char*>(kn),
              static_cast<const char*>(vn), elem_bytes, B, T, H, D, cap,
              kc_sb * e, kc_ss * e, kc_sh * e, vc_sb * e, vc_ss * e, vc_sh * e,
              kn_sb * e, kn_ss * e, kn_sh * e, vn_sb * e, vn_ss * e, vn_sh * e, write_index};
  const int64_t rows = (int64_t)B * T * H;
  if (rows == 0 || D == 0) return hipSuccess;
  // 16-byte chunks only when every row start is 16-byte aligned
  auto al = [](const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  auto strides_al = [&](int64_t a) {
    const int64_t st[] = {c.kc_sb, c.kc_ss, c.kc_sh, c.vc_sb, c.vc_ss, c.vc_sh,
                          c.kn_sb, c.kn_ss, c.kn_sh, c.vn_sb, c.vn_ss, c.vn_sh};
    for (int64_t x : st) if (x % a) return false;
    return al(kc, a) && al(vc, a) && al(kn, a) && al(vn, a) && ((int64_t)D * e) % a == 0;
  };
  const int chunk = strides_al(16) ? 16 : (elem_bytes == 4 || strides_al(4)) ? 4 : 2;
  const int64_t total = rows * ((int64_t)D * e / chunk);
  const int64_t blocks = (total + 255) / 256;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  if (chunk == 16) hipLaunchKernelGGL(kv_cache_update_kernel<16>, grid, dim3(256), 0, s, c);
  else if (chunk == 4) hipLaunchKernelGGL(kv_cache_update_kernel<4>, grid, dim3(256), 0, s, c);
  else hipLaunchKernelGGL(kv_cache_update_kernel<2>, grid, dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace sdpa
