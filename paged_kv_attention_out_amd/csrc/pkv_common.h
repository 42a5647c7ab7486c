// Shared device helpers for the paged-KV attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kNegInf = -__builtin_huge_valf();

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// One fp32 -> bf16 bit pattern, round to nearest even.
__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane 4q+e receives element e (16-bit) of the 8-byte chunks that
// lanes q, q+4, q+8 and q+12 address.  `p` must point into LDS.
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform broadcast of lane 0's value.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace pkv

// Host-side helpers shared by the entry points.
namespace pkv_host {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool is_pow2_page(int ps) {
  return ps == 16 || ps == 32 || ps == 64 || ps == 128 || ps == 256;
}
inline int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}
inline bool finite_positive(float x) { return x > 0.0f && x <= 3.4028234e38f; }

// Launch a kernel whose only argument is a parameter struct; the status
// reported is this launch's own (hipLaunchKernel's return value).
template <typename P>
inline int launch(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t stream, P params,
                  size_t dynamic_lds = 0) {
  void* args[] = {&params};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args,
                                 dynamic_lds, stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace pkv_host
