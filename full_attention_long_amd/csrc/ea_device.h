// ea_device.h -- small gfx950 device helpers shared by libea's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource (gfx9 word 3 = 0x00020000): loads past `bytes` return zero and
// stores past it are dropped, which makes ragged tails and padding keys free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, unsigned v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

// `x` read from the first active lane: tells the compiler a wavefront-uniform value is
// uniform, so it can live in a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Value of `x` held by lane (lane ^ 32) of the wavefront.
__device__ __forceinline__ float xor32(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  // lanes 0..31: s[1] holds the upper half's value; lanes 32..63: s[0] holds the lower's.
  return __uint_as_float((threadIdx.x & 32) ? s[0] : s[1]);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

}  // namespace ea
