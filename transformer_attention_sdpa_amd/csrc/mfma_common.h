// mfma_common.h -- pieces shared by the matrix-core kernels (forward and gradient): the 16-bit
// input traits (bf16 or f16 MFMAs and conversions), buffer resources with hardware range
// checks, and direct global -> LDS loads.
#pragma once

#include "device_common.h"

namespace sdpa {

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// The 16-bit input type: bf16 or IEEE f16. What differs is the MFMA, the operand vectors and
// the conversions; everything else (loads, LDS layout, transposed reads) moves 16-bit words.
template <bool F16> struct In;
template <> struct In<false> {
  typedef __bf16 x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  __device__ static f32x16 mfma(x8 a, x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
  __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }          // element 0 of a pair
  __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }  // element 1
  __device__ static uint16_t bits(float f) { return float_to_bf16_bits(f); }
  __device__ static uint32_t pack(float a, float b) {
    const x2 p = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, p);
  }
  // acc + the two packed values (a dot product with 1, 1)
  __device__ static float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(x2, p), __builtin_bit_cast(x2, 0x3f803f80u), acc, false);
  }
};
template <> struct In<true> {
  typedef _Float16 x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  __device__ static f32x16 mfma(x8 a, x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
  __device__ static float lo(uint32_t w) { return f16_bits_to_float(static_cast<uint16_t>(w)); }
  __device__ static float hi(uint32_t w) { return f16_bits_to_float(static_cast<uint16_t>(w >> 16)); }
  __device__ static uint16_t bits(float f) { return float_to_f16_bits(f); }
  __device__ static uint32_t pack(float a, float b) {
    const x2 p = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, p);
  }
  __device__ static float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(x2, p), __builtin_bit_cast(x2, 0x3c003c00u), acc, false);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// One wave instruction of a direct global -> LDS load: lane l copies 16 bytes from byte offset
// voff of r into lds + 16*l (M0 holds lds). (Kept out of the kernel body: used there
// directly, the host pass drops the kernel's stub.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// The same with one 32-bit word per lane: lane l copies 4 bytes from byte offset voff of r into
// lds + 4*l.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}

// Buffer resource over `bytes` bytes from `base`: loads past the end return 0 (the hardware's
// range check), which zero-fills ragged tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;

}  // namespace

}  // namespace sdpa
