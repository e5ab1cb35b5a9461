// Device helpers shared by the libskipattn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace skipattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;    // decision tile edge (queries and keys)
constexpr int kSplit = 4096; // decode split length in keys
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_exp_f32: 2^x, exact 0 for -inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Round two floats to bf16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Value of x held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }
__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16); }

// Four rows (keys) of eight bf16 (columns) -> for each column e, the four
// keys' values packed as 2 dwords (key 0,1 in .x, key 2,3 in .y).
__device__ __forceinline__ u32x2 column_of_4x8(const u32x4 (&r)[4], int e) {
  const int w = e >> 1;
  uint32_t lo, hi;
  if ((e & 1) == 0) {
    lo = (r[0][w] & 0xffffu) | (r[1][w] << 16);
    hi = (r[2][w] & 0xffffu) | (r[3][w] << 16);
  } else {
    lo = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
    hi = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
  }
  u32x2 out;
  out[0] = lo;
  out[1] = hi;
  return out;
}

}  // namespace skipattn
