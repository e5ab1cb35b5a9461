// Block-quantised fp8 (E4M3) codes of Q and K for the 8-bit QK^T prefill.
//
// Method: the TurboAttention talk page ("Technical Deep Dive", "Key
// Findings"; its pre-fill workflow) runs the products of blockwise attention
// on symmetric 8-bit operands quantised block by block inside the flash
// blocks. gfx950's 8-bit matrix cores take fp8; the block is a 64-row tile
// (a query tile of Q, a key tile of K), the decision tile of the skip rule.
//
// Per block: m = largest |x| over its rows (rows past N take no part);
// scale s = m / 448 in fp32 (1 for a block of zeros); code = E4M3 of
// clamp(x / s, -448, 448), the division in fp32, rounded to the nearest E4M3
// value with ties to the even mantissa; a value that rounds to zero is
// code 0. Codes [X, N, D] uint8 (row-major like the input), scales
// [X, ceil(N/64)] fp32.
//
// One workgroup of 256 threads per block: thread t owns row t / 4 of the
// block and D / 4 consecutive elements of it (16-byte loads and stores).
#include "common.hpp"
#include "launch.hpp"

namespace skipattn {
namespace {
// Exact widening of a bf16 bit pattern.
__device__ __forceinline__ float bf16_bits_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
}  // namespace
}  // namespace skipattn

namespace skipattn {

namespace {

// E4M3 code of |y| <= 448: below 2^-6 the values are multiples of 2^-9
// (exact scaling, rint rounds ties to even); above, the fp32 mantissa is
// rounded to 3 bits (ties to even, a carry moves into the exponent) and the
// exponent rebiased from 127 to 7 (960 = 120 << 3).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const float a = fabsf(y);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const uint32_t bits = __builtin_bit_cast(uint32_t, a);
    mag = ((bits + 0x7FFFFu + ((bits >> 20) & 1u)) >> 20) - 960u;
  }
  return mag == 0u ? 0u : (mag | ((__builtin_bit_cast(uint32_t, y) >> 24) & 0x80u));
}

template <int D>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales, int N,
                                                        int nt) {
  constexpr int E = D / 4;  // elements per thread
  static_assert(E % 16 == 0, "16-byte pieces");
  __shared__ float wmax[4];
  const int blk = blockIdx.x;
  const long long xi = blk / nt;  // which (batch, head)
  const int t = blk % nt;
  const int tid = threadIdx.x;
  const int r = tid >> 2;          // row in the block
  const int row = t * kTile + r;
  const bool ok = row < N;
  const uint16_t* src = x + ((size_t)xi * N + (ok ? row : 0)) * D + (tid & 3) * E;

  float v[E];
#pragma unroll
  for (int p = 0; p < E / 8; ++p) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (ok) w = ldg16(src + 8 * p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * p + 2 * i] = bf16_bits_f32(w[i] & 0xffffu);
      v[8 * p + 2 * i + 1] = bf16_bits_f32(w[i] >> 16);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float sc = m > 0.f ? m / 448.f : 1.f;
  if (tid == 0) scales[(size_t)xi * nt + t] = sc;
  if (!ok) return;
  uint8_t* dst = codes + ((size_t)xi * N + row) * D + (tid & 3) * E;
#pragma unroll
  for (int p = 0; p < E / 16; ++p) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = fminf(fmaxf(v[16 * p + 4 * i + j] / sc, -448.f), 448.f);
        word |= e4m3_code(y) << (8 * j);
      }
      w[i] = word;
    }
    *reinterpret_cast<u32x4*>(dst + 16 * p) = w;
  }
}

}  // namespace

int launch_quantize_fp8(const void* x, uint8_t* codes, float* scales, long long X, int N, int D,
                        void* stream) {
  const int nt = (N + kTile - 1) / kTile;
  const long long blocks = X * nt;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  if (D == 128)
    hipLaunchKernelGGL((quant_fp8_kernel<128>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (const uint16_t*)x, codes, scales, N, nt);
  else
    hipLaunchKernelGGL((quant_fp8_kernel<64>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (const uint16_t*)x, codes, scales, N, nt);
  return 0;
}

}  // namespace skipattn
