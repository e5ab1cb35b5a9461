// Device helpers shared by the 4-bit and 2-bit KV-cache kernels: the block
// parameters and codes of the quantisers, the parameter word, and raw buffer
// loads with a chosen cache policy.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace skipattn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

namespace kvq {

constexpr uint32_t kCfg = 0x00020000u;     // raw 32-bit buffer, range-checked
constexpr uint32_t kNoRead = 0x80000000u;  // tile offset of a load that reads nothing
constexpr int kNT = 2;                     // non-temporal cache policy
constexpr int kRT = 0;                     // default cache policy

// Head numbering of a cache that holds some of the KV heads (a hybrid
// cache's heads of one width): (b, head) slice b * n + i of the cache comes
// from slice b * n_in + g[i] of the full set (the quantisers' src_slice),
// and its query heads are rows of the full set's query heads: KV head i of
// the cache is head full_head(i) of the full set.
__device__ __forceinline__ int full_head(int g, const KvHeadMap& hm) {
  return hm.n ? hm.g[g] : g;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Non-negative finite fp32 rounded up to the bf16 grid.
__device__ __forceinline__ float bf16_round_up(float x) {
  uint32_t b = __builtin_bit_cast(uint32_t, x);
  if (b & 0xffffu) b = (b + 0x10000u) & 0xffff0000u;
  return __builtin_bit_cast(float, b);
}

// Block parameters and codes for codes 0 .. CMAX. The fp32 subtract and
// divide are rounded to nearest even and are not fused with anything: they
// decide integers.
template <int CMAX>
__device__ __forceinline__ float block_scale(float lo, float hi) {
  return bf16_round_up(__fdiv_rn(__fsub_rn(hi, lo), (float)CMAX));
}
template <int CMAX>
__device__ __forceinline__ uint32_t code_of(float x, float s, float z) {
  if (!(s > 0.f)) return 0u;
  const float r = rintf(__fdiv_rn(__fsub_rn(x, z), s));
  return (uint32_t)fminf(fmaxf(r, 0.f), (float)CMAX);
}

// Parameter word: bf16 s in the low half, bf16 z in the high half.
__device__ __forceinline__ uint32_t pack_params(float s, float z) {
  return (__builtin_bit_cast(uint32_t, s) >> 16) | (__builtin_bit_cast(uint32_t, z) & 0xffff0000u);
}
__device__ __forceinline__ float param_s(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float param_z(uint32_t p) { return __builtin_bit_cast(float, p & 0xffff0000u); }

template <int AUX>
__device__ __forceinline__ u32x4 ld4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ uint32_t ld1(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ u32x2 ld2(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, AUX));
}

}  // namespace kvq
}  // namespace skipattn
