// Block-quantised 8-bit codes of Q and K for the 8-bit QK^T prefills (fp8
// E4M3, or symmetric int8), and the V codes of the 8-bit P.V prefill.
//
// Method: the TurboAttention talk page ("Technical Deep Dive", "Key
// Findings"; its pre-fill workflow) runs the products of blockwise attention
// on symmetric 8-bit operands quantised block by block inside the flash
// blocks. gfx950's 8-bit matrix cores take fp8 and int8; the block is a 64-row tile
// (a query tile of Q, a key tile of K), the decision tile of the skip rule.
//
// Per block: m = largest |x| over its rows (rows past N take no part);
// scale s = m / 448 in fp32 (1 for a block of zeros); code = E4M3 of
// clamp(x / s, -448, 448), the division in fp32, rounded to the nearest E4M3
// value with ties to the even mantissa; a value that rounds to zero is
// code 0. Codes [X, N, D] uint8 (row-major like the input), scales
// [X, ceil(N/64)] fp32.
//
// The int8 reading (the pages name symmetric int8 for these operands):
// scale s = m / 127, code = clamp(rint(x / s), -127, 127) (fp32 division,
// rint ties to even; -128 unused), stored as two's complement bytes, for the
// int8 matrix cores.
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

// One 64-row block per workgroup. I8 = false: E4M3 codes, scale m / 448;
// I8 = true: symmetric int8 codes clamp(rint(x / s), -127, 127) (two's
// complement bytes), scale m / 127; both with the division in fp32.
template <int D, bool I8>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x,
                                            uint8_t* __restrict__ codes,
                                            float* __restrict__ scales, int N, int nt) {
  constexpr int E = D / 4;  // elements per thread
  static_assert(E % 16 == 0, "16-byte pieces");
  constexpr float kMax = I8 ? 127.f : 448.f;
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
  const float sc = m > 0.f ? m / kMax : 1.f;
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
        const float y = v[16 * p + 4 * i + j] / sc;
        uint32_t code;
        if constexpr (I8)
          code = (uint32_t)(int)fminf(fmaxf(__builtin_rintf(y), -kMax), kMax) & 0xffu;
        else
          code = e4m3_code(fminf(fmaxf(y, -kMax), kMax));
        word |= code << (8 * j);
      }
      w[i] = word;
    }
    *reinterpret_cast<u32x4*>(dst + 16 * p) = w;
  }
}

template <int D>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales, int N,
                                                        int nt) {
  quant_block<D, false>(x, codes, scales, N, nt);
}

template <int D>
__global__ __launch_bounds__(256) void quant_i8_kernel(const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales, int N,
                                                       int nt) {
  quant_block<D, true>(x, codes, scales, N, nt);
}

// ---- V for the 8-bit P.V product: one scale per (sequence, KV head) ----
// (TurboAttention talk page, "Technical Deep Dive": the PV product on 8-bit
// operands too.) A per-tile scale would not factor out of P.V, whose sum
// runs over every key tile into one accumulator, so V takes one scale per
// head: s = (largest |v| of the head) / 448, 1 for a head of zeros. Three
// passes: the tiles' largest |v|, the head's scale, the codes.
//
// Code layout, per head and 64-key tile t: D rows of 64 bytes; row c holds
// channel c's codes in the order of the P.V contraction index j (j = 32 h +
// 16 a + 4 i + e holds key 32 a + 8 i + 4 h + e of the tile: the order in
// which a lane's probabilities come out of the S^T accumulators), with the
// row's 16-byte chunk x stored at chunk x ^ ((c >> 2) & 3) so that the
// kernel's 16-lane reads of 16 consecutive rows hit distinct LDS banks.
// Keys past N have code 0.

// Largest |v| of each 64-key tile: thread t reads row t / 4 of the tile.
template <int D>
__global__ __launch_bounds__(256) void v8_tile_max_kernel(const uint16_t* __restrict__ x,
                                                          float* __restrict__ tmax, int N,
                                                          int nt) {
  constexpr int E = D / 4;
  __shared__ float wmax[4];
  const long long xi = blockIdx.x / nt;
  const int t = blockIdx.x % nt;
  const int tid = threadIdx.x;
  const int row = t * kTile + (tid >> 2);
  float m = 0.f;
  if (row < N) {
    const uint16_t* src = x + ((size_t)xi * N + row) * D + (tid & 3) * E;
#pragma unroll
    for (int p = 0; p < E / 8; ++p) {
      const u32x4 w = ldg16(src + 8 * p);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m = fmaxf(m, fmaxf(fabsf(bf16_bits_f32(w[i] & 0xffffu)), fabsf(bf16_bits_f32(w[i] >> 16))));
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) tmax[blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// The head's scale from its tiles' maxima.
__global__ __launch_bounds__(256) void v8_head_scale_kernel(const float* __restrict__ tmax,
                                                            float* __restrict__ vscale, int nt) {
  __shared__ float wmax[4];
  const int tid = threadIdx.x;
  const float* src = tmax + (size_t)blockIdx.x * nt;
  float m = 0.f;
  for (int t = tid; t < nt; t += 256) m = fmaxf(m, src[t]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    vscale[blockIdx.x] = m > 0.f ? m / 448.f : 1.f;
  }
}

// Codes of one tile: the tile's bf16 rows go to LDS (rows past N as zeros),
// then thread t writes 64 D / 256 bytes of the tile's code block, gathering
// each byte's key and channel from LDS.
template <int D>
__global__ __launch_bounds__(256) void v8_quant_kernel(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ vscale,
                                                       uint8_t* __restrict__ codes, int N,
                                                       int nt) {
  constexpr int E = D / 4;
  constexpr int BPT = 64 * D / 256;  // code bytes per thread: 32 (D = 128) or 16
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile][D];
  const long long xi = blockIdx.x / nt;
  const int t = blockIdx.x % nt;
  const int tid = threadIdx.x;
  {
    const int r = tid >> 2;
    const int row = t * kTile + r;
    const uint16_t* src = x + ((size_t)xi * N + (row < N ? row : 0)) * D + (tid & 3) * E;
#pragma unroll
    for (int p = 0; p < E / 8; ++p) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < N) w = ldg16(src + 8 * p);
      *reinterpret_cast<u32x4*>(&tile[r][(tid & 3) * E + 8 * p]) = w;
    }
  }
  __syncthreads();
  const float sc = vscale[xi];
  const int c = tid / (256 / D);                 // channel (code row)
  const int p0 = (tid % (256 / D)) * BPT;        // first byte of this thread in the row
  const int sw = (c >> 2) & 3;
  uint8_t* dst = codes + ((size_t)xi * nt + t) * (64 * D) + c * 64 + p0;
#pragma unroll
  for (int q = 0; q < BPT / 16; ++q) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int p = p0 + 16 * q + 4 * i + b;             // stored byte position
        const int j = 16 * ((p >> 4) ^ sw) + (p & 15);     // contraction index
        const int key = 32 * ((j >> 4) & 1) + 8 * ((j >> 2) & 3) + 4 * (j >> 5) + (j & 3);
        const float v = bf16_bits_f32(tile[key][c]);
        const float y = fminf(fmaxf(v / sc, -448.f), 448.f);
        word |= e4m3_code(y) << (8 * b);
      }
      w[i] = word;
    }
    *reinterpret_cast<u32x4*>(dst + 16 * q) = w;
  }
}

}  // namespace

int launch_quantize_v8(const void* v, uint8_t* codes, float* tmax, float* vscale, long long X,
                       int N, int D, void* stream) {
  const int nt = (N + kTile - 1) / kTile;
  const long long blocks = X * nt;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  hipStream_t st = (hipStream_t)stream;
  const uint16_t* x = (const uint16_t*)v;
  if (D == 128) {
    hipLaunchKernelGGL((v8_tile_max_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                       tmax, N, nt);
    hipLaunchKernelGGL(v8_head_scale_kernel, dim3((unsigned)X), dim3(256), 0, st, tmax, vscale,
                       nt);
    hipLaunchKernelGGL((v8_quant_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                       vscale, codes, N, nt);
  } else {
    hipLaunchKernelGGL((v8_tile_max_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                       tmax, N, nt);
    hipLaunchKernelGGL(v8_head_scale_kernel, dim3((unsigned)X), dim3(256), 0, st, tmax, vscale,
                       nt);
    hipLaunchKernelGGL((v8_quant_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                       vscale, codes, N, nt);
  }
  return 0;
}

int launch_quantize_i8(const void* x, uint8_t* codes, float* scales, long long X, int N, int D,
                       void* stream) {
  const int nt = (N + kTile - 1) / kTile;
  const long long blocks = X * nt;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  if (D == 128)
    hipLaunchKernelGGL((quant_i8_kernel<128>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (const uint16_t*)x, codes, scales, N, nt);
  else
    hipLaunchKernelGGL((quant_i8_kernel<64>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (const uint16_t*)x, codes, scales, N, nt);
  return 0;
}

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
