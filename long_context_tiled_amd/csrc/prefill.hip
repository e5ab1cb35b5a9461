// Prefill: exact tiled softmax attention with the Skip-Softmax tile test,
// bf16 MFMA on gfx950.
//
// Method: blockwise attention (TurboAttention talk page, "Technical Deep
// Dive") with the Skip-Softmax rule (TensorRT-LLM Skip Softmax summary page,
// "Key Points", "Detailed Analysis"): for every 64-query x 64-key tile,
// visited in ascending key order, the scores are formed, each row's tile
// maximum t_r is compared with its running maximum m_r, and the exp and PV
// work of the tile is dropped when t_r < m_r - tau for every valid row.
//
// Work decomposition
//   A workgroup is 4 waves. Wave w owns one 64-row query tile of one head,
//   so the skip vote of a decision tile is a single wave ballot. The waves of
//   a workgroup are HPW heads of one grouped-query KV group x (4 / HPW)
//   consecutive query tiles, and share every K/V tile through LDS.
//   Grid order is longest-first for causal attention.
//
// Data movement
//   K and V tiles (64 keys x d, bf16) go from HBM/L2 straight into LDS with
//   buffer_load_dwordx4 ... lds (no VGPR staging). Keys past N read as zero
//   through the buffer descriptor's range check. Rows are stored unpadded,
//   with the 16-byte chunk c of row r at slot c ^ (r & (chunks - 1)) so that
//   the fragment reads below hit distinct LDS banks. STAGES tiles are in
//   flight; one workgroup barrier per key tile.
//
// Per wave and key tile:
//   S^T (64 keys x 64 queries) = K . Q^T with v_mfma_f32_32x32x16_bf16:
//   lane l owns query column (l & 31) of each 32-query half and 16 key rows
//   of each 32-key half, so a query's tile max is an in-lane max over 32
//   values plus one exchange between lane halves (v_permlane32_swap).
//   P^T, rounded to bf16, is already the B operand of O^T = V^T . P^T (the
//   MFMA contraction index is permuted consistently on both sides). The
//   V^T operand is read from the row-major V tile with ds_read_b64_tr_b16.
//   O^T accumulates in fp32; lane l owns query (l & 31), so the online
//   rescale is one multiplier per lane, and it is skipped (exactly, since
//   the multiplier would be 1) when no row's maximum grew.
//
// Units: scores stay raw (q.k) in registers. The test compares
// t < m - tau * sqrt(d); exponentials use exp2 with log2(e)/sqrt(d) folded
// into one FMA per score.
#include "common.hpp"
#include "launch.hpp"

namespace skipattn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr uint32_t kBufferCfg = 0x00020000u;  // raw 32-bit buffer, range-checked

template <int D>
struct PrefillTile {
  static constexpr int rowBytes = 2 * D;
  static constexpr int chunks = D / 8;               // 16-byte chunks per row
  static constexpr int bytes = kTile * rowBytes;      // one K or V tile
  static constexpr int rowsPerInstr = 1024 / rowBytes;
  static constexpr int instrPerWave = kTile / rowsPerInstr / 4;
};

// Byte offset, inside a swizzled tile, of 16-byte chunk c of row r.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return r * PrefillTile<D>::rowBytes + 16 * (c ^ (r & (PrefillTile<D>::chunks - 1)));
}

// Lane l gets the pair (x[l % 32], x[32 + l % 32]) from one
// v_permlane32_swap on two copies of x. (The builtin, given the same value
// twice, is folded as if both results were equal, so the swap is written
// out; the s_nop covers the VALU-write-to-permlane read hazard.)
__device__ __forceinline__ void swap_halves(float x, float& lo, float& hi) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}

__device__ __forceinline__ float swap_halves_max(float x) {
  float a, b;
  swap_halves(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  float a, b;
  swap_halves(x, a, b);
  return a + b;
}

// V^T fragments of one 16-key step for MB 32-d blocks: two transpose reads
// per block (keys +0..3 and +8..11 of each lane half) at the per-lane LDS
// addresses ad[] plus the immediate KOFF. The reads and the wait for them are
// one asm block, so no load is left in flight past it and the compiler adds
// no wait on the tile copies still in flight.
template <int MB, int KOFF>
__device__ __forceinline__ void read_vt(bf16x8 (&vf)[MB], const uint32_t (&ad)[2 * MB]) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  u32x2v r[2 * MB];
  if constexpr (MB == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%c16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%c16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%c16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%c16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%c16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%c16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%c16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%c16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7]), "i"(KOFF)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%c8\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%c8\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%c8\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%c8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(KOFF)
        : "memory");
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    u32x4 w;
    w[0] = r[2 * mb][0];
    w[1] = r[2 * mb][1];
    w[2] = r[2 * mb + 1][0];
    w[3] = r[2 * mb + 1][1];
    vf[mb] = as_bf16x8(w);
  }
}

// The O^T accumulators live in fixed AGPRs: block (mb, nb) of the 128-d
// kernel is a[32 mb + 16 nb : +15] (a[0:63] for d = 64). Every asm statement
// that touches them names those registers, so the register allocator keeps
// them there for the whole key loop. (Written as builtins inside the
// kept-tile branch, the allocator parks them in VGPRs between iterations and
// copies all of them on every tile.)
#define SKA_ACC8                                                                   \
  "+{a[0:15]}"(acc[0][0]), "+{a[16:31]}"(acc[0][1]), "+{a[32:47]}"(acc[1][0]),     \
      "+{a[48:63]}"(acc[1][1]), "+{a[64:79]}"(acc[2][0]), "+{a[80:95]}"(acc[2][1]), \
      "+{a[96:111]}"(acc[3][0]), "+{a[112:127]}"(acc[3][1])
#define SKA_ACC4 \
  "+{a[0:15]}"(acc[0][0]), "+{a[16:31]}"(acc[0][1]), "+{a[32:47]}"(acc[1][0]), "+{a[48:63]}"(acc[1][1])

// O^T += V^T . P^T for one 16-key step. The leading s_nop covers the
// VALU-write to MFMA-read wait states of the P and V operands.
__device__ __forceinline__ void pv_step(f32x16 (&acc)[4][2], const bf16x8 (&vf)[4],
                                        const bf16x8 (&pf)[2]) {
  asm volatile(
      "s_nop 4\n\t"
      "v_mfma_f32_32x32x16_bf16 a[0:15], %8, %12, a[0:15]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[16:31], %8, %13, a[16:31]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[32:47], %9, %12, a[32:47]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[48:63], %9, %13, a[48:63]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[64:79], %10, %12, a[64:79]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[80:95], %10, %13, a[80:95]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[96:111], %11, %12, a[96:111]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[112:127], %11, %13, a[112:127]"
      : SKA_ACC8
      : "v"(vf[0]), "v"(vf[1]), "v"(vf[2]), "v"(vf[3]), "v"(pf[0]), "v"(pf[1]));
}

__device__ __forceinline__ void pv_step(f32x16 (&acc)[2][2], const bf16x8 (&vf)[2],
                                        const bf16x8 (&pf)[2]) {
  asm volatile(
      "s_nop 4\n\t"
      "v_mfma_f32_32x32x16_bf16 a[0:15], %4, %6, a[0:15]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[16:31], %4, %7, a[16:31]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[32:47], %5, %6, a[32:47]\n\t"
      "v_mfma_f32_32x32x16_bf16 a[48:63], %5, %7, a[48:63]"
      : SKA_ACC4
      : "v"(vf[0]), "v"(vf[1]), "v"(pf[0]), "v"(pf[1]));
}

// Wait states after the last accumulating MFMA (16 passes) before its result
// registers may be read by other instructions.
__device__ __forceinline__ void drain_mfma() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Zero the pinned accumulators.
#define SKA_Z4(a, b, c, d)                                                     \
  "v_accvgpr_write_b32 a" #a ", 0\n\tv_accvgpr_write_b32 a" #b ", 0\n\t"        \
  "v_accvgpr_write_b32 a" #c ", 0\n\tv_accvgpr_write_b32 a" #d ", 0\n\t"

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][2]) {
  asm volatile(
      SKA_Z4(0, 1, 2, 3) SKA_Z4(4, 5, 6, 7) SKA_Z4(8, 9, 10, 11) SKA_Z4(12, 13, 14, 15)
      SKA_Z4(16, 17, 18, 19) SKA_Z4(20, 21, 22, 23) SKA_Z4(24, 25, 26, 27) SKA_Z4(28, 29, 30, 31)
      SKA_Z4(32, 33, 34, 35) SKA_Z4(36, 37, 38, 39) SKA_Z4(40, 41, 42, 43) SKA_Z4(44, 45, 46, 47)
      SKA_Z4(48, 49, 50, 51) SKA_Z4(52, 53, 54, 55) SKA_Z4(56, 57, 58, 59) SKA_Z4(60, 61, 62, 63)
      SKA_Z4(64, 65, 66, 67) SKA_Z4(68, 69, 70, 71) SKA_Z4(72, 73, 74, 75) SKA_Z4(76, 77, 78, 79)
      SKA_Z4(80, 81, 82, 83) SKA_Z4(84, 85, 86, 87) SKA_Z4(88, 89, 90, 91) SKA_Z4(92, 93, 94, 95)
      SKA_Z4(96, 97, 98, 99) SKA_Z4(100, 101, 102, 103) SKA_Z4(104, 105, 106, 107)
      SKA_Z4(108, 109, 110, 111) SKA_Z4(112, 113, 114, 115) SKA_Z4(116, 117, 118, 119)
      SKA_Z4(120, 121, 122, 123) SKA_Z4(124, 125, 126, 127)
      "s_nop 1"
      : "={a[0:15]}"(acc[0][0]), "={a[16:31]}"(acc[0][1]), "={a[32:47]}"(acc[1][0]),
        "={a[48:63]}"(acc[1][1]), "={a[64:79]}"(acc[2][0]), "={a[80:95]}"(acc[2][1]),
        "={a[96:111]}"(acc[3][0]), "={a[112:127]}"(acc[3][1]));
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[2][2]) {
  asm volatile(
      SKA_Z4(0, 1, 2, 3) SKA_Z4(4, 5, 6, 7) SKA_Z4(8, 9, 10, 11) SKA_Z4(12, 13, 14, 15)
      SKA_Z4(16, 17, 18, 19) SKA_Z4(20, 21, 22, 23) SKA_Z4(24, 25, 26, 27) SKA_Z4(28, 29, 30, 31)
      SKA_Z4(32, 33, 34, 35) SKA_Z4(36, 37, 38, 39) SKA_Z4(40, 41, 42, 43) SKA_Z4(44, 45, 46, 47)
      SKA_Z4(48, 49, 50, 51) SKA_Z4(52, 53, 54, 55) SKA_Z4(56, 57, 58, 59) SKA_Z4(60, 61, 62, 63)
      "s_nop 1"
      : "={a[0:15]}"(acc[0][0]), "={a[16:31]}"(acc[0][1]), "={a[32:47]}"(acc[1][0]),
        "={a[48:63]}"(acc[1][1]));
}

// Copy one pinned accumulator block into 16 VGPR floats.
#define SKA_RD1(i, n) "v_accvgpr_read_b32 %" #i ", a" #n "\n\t"
#define SKA_READ16(RANGE, blk, out, n0, n1, n2, n3, n4, n5, n6, n7, n8, n9, n10, n11, n12, n13, \
                   n14, n15)                                                                   \
  asm volatile(SKA_RD1(0, n0) SKA_RD1(1, n1) SKA_RD1(2, n2) SKA_RD1(3, n3) SKA_RD1(4, n4)       \
                   SKA_RD1(5, n5) SKA_RD1(6, n6) SKA_RD1(7, n7) SKA_RD1(8, n8) SKA_RD1(9, n9)   \
                       SKA_RD1(10, n10) SKA_RD1(11, n11) SKA_RD1(12, n12) SKA_RD1(13, n13)      \
                           SKA_RD1(14, n14) SKA_RD1(15, n15) "s_nop 1"                          \
               : "=v"(out[0]), "=v"(out[1]), "=v"(out[2]), "=v"(out[3]), "=v"(out[4]),         \
                 "=v"(out[5]), "=v"(out[6]), "=v"(out[7]), "=v"(out[8]), "=v"(out[9]),         \
                 "=v"(out[10]), "=v"(out[11]), "=v"(out[12]), "=v"(out[13]), "=v"(out[14]),    \
                 "=v"(out[15])                                                                  \
               : RANGE(blk))

// Block (mb, nb) of the pinned accumulators, as 16 floats in VGPRs.
template <int MBX>
__device__ __forceinline__ void read_acc(const f32x16 (&acc)[MBX][2], int mb, int nb, float (&o)[16]) {
  const int id = 2 * mb + nb;
  if (id == 0) SKA_READ16("{a[0:15]}", acc[0][0], o, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  if (id == 1) SKA_READ16("{a[16:31]}", acc[0][1], o, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31);
  if (id == 2) SKA_READ16("{a[32:47]}", acc[1][0], o, 32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43, 44, 45, 46, 47);
  if (id == 3) SKA_READ16("{a[48:63]}", acc[1][1], o, 48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63);
  if constexpr (MBX == 4) {
    if (id == 4) SKA_READ16("{a[64:79]}", acc[2][0], o, 64, 65, 66, 67, 68, 69, 70, 71, 72, 73, 74, 75, 76, 77, 78, 79);
    if (id == 5) SKA_READ16("{a[80:95]}", acc[2][1], o, 80, 81, 82, 83, 84, 85, 86, 87, 88, 89, 90, 91, 92, 93, 94, 95);
    if (id == 6) SKA_READ16("{a[96:111]}", acc[3][0], o, 96, 97, 98, 99, 100, 101, 102, 103, 104, 105, 106, 107, 108, 109, 110, 111);
    if (id == 7) SKA_READ16("{a[112:127]}", acc[3][1], o, 112, 113, 114, 115, 116, 117, 118, 119, 120, 121, 122, 123, 124, 125, 126, 127);
  }
}

// acc[.][nb] *= alpha in place, on the pinned AGPRs.
#define SKA_R1(n)                                                                \
  "v_accvgpr_read_b32 %[t], a" #n "\n\ts_nop 1\n\tv_mul_f32 %[t], %[t], %[al]\n\t" \
  "s_nop 1\n\tv_accvgpr_write_b32 a" #n ", %[t]\n\t"
#define SKA_R4(a, b, c, d) SKA_R1(a) SKA_R1(b) SKA_R1(c) SKA_R1(d)
#define SKA_R16(a0, a1, a2, a3, a4, a5, a6, a7, a8, a9, a10, a11, a12, a13, a14, a15) \
  SKA_R4(a0, a1, a2, a3) SKA_R4(a4, a5, a6, a7) SKA_R4(a8, a9, a10, a11) SKA_R4(a12, a13, a14, a15)

__device__ __forceinline__ void rescale_acc(f32x16 (&acc)[4][2], float alpha0, float alpha1) {
  float t;
  asm volatile(
      SKA_R16(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15)
      SKA_R16(32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43, 44, 45, 46, 47)
      SKA_R16(64, 65, 66, 67, 68, 69, 70, 71, 72, 73, 74, 75, 76, 77, 78, 79)
      SKA_R16(96, 97, 98, 99, 100, 101, 102, 103, 104, 105, 106, 107, 108, 109, 110, 111)
      "s_nop 1"
      : SKA_ACC8, [t] "=&v"(t)
      : [al] "v"(alpha0));
  asm volatile(
      SKA_R16(16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31)
      SKA_R16(48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63)
      SKA_R16(80, 81, 82, 83, 84, 85, 86, 87, 88, 89, 90, 91, 92, 93, 94, 95)
      SKA_R16(112, 113, 114, 115, 116, 117, 118, 119, 120, 121, 122, 123, 124, 125, 126, 127)
      "s_nop 1"
      : SKA_ACC8, [t] "=&v"(t)
      : [al] "v"(alpha1));
}

__device__ __forceinline__ void rescale_acc(f32x16 (&acc)[2][2], float alpha0, float alpha1) {
  float t;
  asm volatile(
      SKA_R16(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15)
      SKA_R16(32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43, 44, 45, 46, 47)
      "s_nop 1"
      : SKA_ACC4, [t] "=&v"(t)
      : [al] "v"(alpha0));
  asm volatile(
      SKA_R16(16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31)
      SKA_R16(48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63)
      "s_nop 1"
      : SKA_ACC4, [t] "=&v"(t)
      : [al] "v"(alpha1));
}

// One 16-byte-per-lane copy from a buffer straight into LDS: lane i writes
// bytes [16 i, 16 i + 16) after the wave-uniform LDS address lds. (Kept out
// of the kernel body: used there directly, the builtin stops the host pass
// from emitting the kernel's launch stub.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, lds_void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0);
}

template <int D, bool CAUSAL, int HPW, int STAGES>
__global__ __launch_bounds__(256, 1) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, uint8_t* __restrict__ mask, int Hq, int Hkv,
    int N, float tau_raw, float c, int nqg, int ny) {
  constexpr int QPW = 4 / HPW;   // query tiles per workgroup
  constexpr int KS = D / 16;     // MFMA k-steps over d for S^T
  constexpr int MB = D / 32;     // 32-row d blocks of O^T
  using T = PrefillTile<D>;
  constexpr int STAGE_BYTES = 2 * T::bytes;
  // K/V stages, then one 64-row Q tile per wave.
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES + 4 * T::bytes];
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char*)smem;  // LDS byte address

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int G = Hq / Hkv;
  const int gper = G / HPW;

  const int lin = blockIdx.x;
  const int y = lin % ny;
  const int qg = CAUSAL ? (nqg - 1 - lin / ny) : lin / ny;
  const int b = y / (Hkv * gper);
  const int rem = y % (Hkv * gper);
  const int g = rem / gper;
  const int h = g * G + (rem % gper) * HPW + (wave % HPW);
  const int qb = qg * QPW + wave / HPW;
  const int nqb = (N + kTile - 1) / kTile;
  const bool wave_valid = qb < nqb;
  const int nkb_wg = CAUSAL ? min(nqb, qg * QPW + QPW) : nqb;
  const int nkb_w = wave_valid ? (CAUSAL ? qb + 1 : nqb) : 0;

  const int head_bytes = N * D * 2;
  const size_t kv_off = (size_t)(b * Hkv + g) * N * D;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + kv_off), (short)0, head_bytes, kBufferCfg);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + kv_off), (short)0, head_bytes, kBufferCfg);
  const size_t bh = (size_t)b * Hq + h;
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(q + bh * N * D), (short)0, head_bytes, kBufferCfg);

  // Q^T fragments (B operand of S^T = K . Q^T): query row (l & 31) of each
  // 32-query half, d = 16 ks + 8 (l >> 5) .. + 7. Rows past N read as 0.
  // Per-lane load geometry for the direct-to-LDS copies: instruction i of
  // wave w fills LDS bytes [1024 (w * IPW + i), +1024) of the tile.
  constexpr int IPW = T::instrPerWave;
  int ld_goff[IPW];   // global byte offset within the head, relative to key 0
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * T::rowsPerInstr + lane / T::chunks;
    const int slot = lane % T::chunks;
    const int cc = slot ^ (r & (T::chunks - 1));
    ld_goff[i] = r * T::rowBytes + cc * 16;
  }

  auto issue_tile = [&](int kb) {
    char* st = smem + (kb % STAGES) * STAGE_BYTES;
    const int base = kb * kTile * T::rowBytes;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      lds_void* dk = (lds_void*)(st + 1024 * (wave * IPW + i));
      dma16(krs, dk, base + ld_goff[i]);
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      lds_void* dv = (lds_void*)(st + T::bytes + 1024 * (wave * IPW + i));
      dma16(vrs, dv, base + ld_goff[i]);
    }
  };

  // The wave's 64 query rows go to its own swizzled LDS tile once (rows past
  // N read as zero); Q^T fragments are read from there for every key tile.
  char* qs_ = smem + STAGES * STAGE_BYTES + wave * T::bytes;
  if (wave_valid) {
    constexpr int QI = T::bytes / 1024;  // 1 KB copy instructions per Q tile
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int r = i * T::rowsPerInstr + lane / T::chunks;
      const int slot = lane % T::chunks;
      const int cc = slot ^ (r & (T::chunks - 1));
      dma16(qrs, (lds_void*)(qs_ + 1024 * i), (qb * kTile + r) * T::rowBytes + cc * 16);
    }
  }

  // ds_read_b64_tr_b16 geometry for the V^T operand: lane k of a 16-lane
  // group fetches 4 consecutive d of key row (16 ks + key_base + k / 4); the
  // instruction hands lane i of the group element (i % 4) of the chunks of
  // lanes 4e + i / 4, e = 0..3, i.e. 4 keys of one d column. For each 32-d
  // block mb, the swizzled address is A ^ (64 mb) with A fixed per lane.
  const int grp16 = lane >> 4;
  const int k16 = lane & 15;
  uint32_t tr_off[2 * MB];  // LDS address (stage 0) of each (mb, 4-key half) read
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 4 * (grp16 >> 1) + (k16 >> 2) + 8 * half;
    const int d = 16 * (grp16 & 1) + 4 * (k16 & 3);
    const uint32_t a = (uint32_t)(swz<D>(row, d >> 3) + 2 * (d & 7));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tr_off[2 * mb + half] = smem_lds + (a ^ (64u * mb));
  }

  f32x16 acc[MB][2];  // O^T accumulators, pinned to AGPRs (see pv_step)
  zero_acc(acc);
  float m[2] = {-INFINITY, -INFINITY};     // running max over kept tiles (skip test)
  float mref[2] = {-INFINITY, -INFINITY};  // reference max of what acc / lsum hold
  float lsum[2] = {0.f, 0.f};
  const float lazy_raw = 8.0f / c;         // 8 in log2 units, as a raw-score gap

  // Prologue: tiles 0 .. STAGES-2 in flight.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nkb_wg) issue_tile(s);

  for (int kb = 0; kb < nkb_wg; ++kb) {
    // Wait for this wave's copies of tile kb (later tiles may stay in flight),
    // then make every wave's copies visible.
    if (STAGES == 3 && kb + 1 < nkb_wg)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * IPW));   // vmcnt(2 * IPW)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
    __syncthreads();
    if (kb + STAGES - 1 < nkb_wg) issue_tile(kb + STAGES - 1);

    if (kb < nkb_w) {
      const char* ks_ = smem + (kb % STAGES) * STAGE_BYTES;
      const char* vs_ = ks_ + T::bytes;

      // ---- S^T = K . Q^T (raw scores, fp32) ----
      f32x16 s[2][2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int row = a * 32 + l32;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks_ + swz<D>(row, 2 * ks + hh));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const bf16x8 qf =
                *reinterpret_cast<const bf16x8*>(qs_ + swz<D>(nb * 32 + l32, 2 * ks + hh));
            if (ks == 0) {
              const f32x16 zero = {};
              s[a][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, zero, 0, 0, 0);
            } else {
              s[a][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, s[a][nb], 0, 0, 0);
            }
          }
        }
      }

      // ---- causal diagonal and ragged-tail masking ----
      const int key0 = kb * kTile;
      if ((CAUSAL && kb == qb) || key0 + kTile > N) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int qrow = qb * kTile + nb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + a * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
              if (key >= N || (CAUSAL && key > qrow)) s[a][nb][r] = -INFINITY;
            }
          }
      }

      // ---- per-row tile maximum ----
      float t[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float x = s[0][nb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) x = fmaxf(x, s[0][nb][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) x = fmaxf(x, s[1][nb][r]);
        t[nb] = swap_halves_max(x);
      }

      // ---- Skip-Softmax vote: skip iff every valid row has t < m - tau ----
      bool blocks = false;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int qrow = qb * kTile + nb * 32 + l32;
        if (qrow < N && !(t[nb] < m[nb] - tau_raw)) blocks = true;
      }
      const bool skip = __ballot(blocks) == 0ull;
      if (mask != nullptr && lane == 0)
        mask[(bh * nqb + qb) * nqb + kb] = skip ? 1 : 0;

      if (!skip) {
        // ---- online softmax update ----
        // m is the running max of the skip test. The exponentials use a
        // reference mref <= m that is only raised (with a rescale of acc and
        // lsum) once some row's max exceeds it by more than 2^8 in weight,
        // so the rescale is rare; the final O = acc / l and LSE = mref / sqrt(d)
        // + ln l do not depend on which reference was used.
        bool grow = false;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          m[nb] = fmaxf(m[nb], t[nb]);
          grow |= m[nb] > mref[nb] + lazy_raw;
        }
        if (__ballot(grow) != 0ull) {
          drain_mfma();
          float alpha[2];
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            alpha[nb] = m[nb] > mref[nb] ? exp2_fast((mref[nb] - m[nb]) * c) : 1.0f;
            lsum[nb] *= alpha[nb];
            mref[nb] = fmaxf(mref[nb], m[nb]);
          }
          rescale_acc(acc, alpha[0], alpha[1]);
        }
        bf16x8 pf[4][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float nmc = -mref[nb] * c;
          float l = lsum[nb];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            u32x4 w;
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
              const int r0 = 8 * (ks & 1) + 2 * i2;
              const float p0 = exp2_fast(__builtin_fmaf(s[ks >> 1][nb][r0], c, nmc));
              const float p1 = exp2_fast(__builtin_fmaf(s[ks >> 1][nb][r0 + 1], c, nmc));
              w[i2] = pack_bf16x2(p0, p1);
              l += p0 + p1;  // fp32 row sum of the unrounded weights
            }
            pf[ks][nb] = as_bf16x8(w);
          }
          lsum[nb] = l;
        }

        // ---- O^T += V^T . P^T ----
        const uint32_t vstage = (uint32_t)(vs_ - smem);
        uint32_t ad[2 * MB];
#pragma unroll
        for (int i = 0; i < 2 * MB; ++i) ad[i] = tr_off[i] + vstage;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 vf[MB];
          if (ks == 0) read_vt<MB, 0 * 16 * T::rowBytes>(vf, ad);
          if (ks == 1) read_vt<MB, 1 * 16 * T::rowBytes>(vf, ad);
          if (ks == 2) read_vt<MB, 2 * 16 * T::rowBytes>(vf, ad);
          if (ks == 3) read_vt<MB, 3 * 16 * T::rowBytes>(vf, ad);
          pv_step(acc, vf, pf[ks]);
        }
      }
    }
  }

  if (!wave_valid) return;
  drain_mfma();

  // ---- epilogue: O = O^T / l, LSE = m / sqrt(d) + ln l ----
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float ltot = swap_halves_sum(lsum[nb]);
    const float inv = 1.f / ltot;
    const int row = qb * kTile + nb * 32 + l32;
    if (row < N) {
      float* orow = o + (bh * N + row) * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float ov[16];
        read_acc<MB>(acc, mb, nb, ov);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 val;
#pragma unroll
          for (int i = 0; i < 4; ++i) val[i] = ov[4 * r4 + i] * inv;
          *reinterpret_cast<f32x4*>(orow + mb * 32 + 8 * r4 + 4 * hh) = val;
        }
      }
      if (hh == 0) lse[bh * N + row] = (mref[nb] * c + __log2f(ltot)) * kLn2;
    }
  }
  if (CAUSAL && mask != nullptr) {
    for (int kb = qb + 1 + lane; kb < nqb; kb += 64)
      mask[(bh * nqb + qb) * nqb + kb] = 2;
  }
}

constexpr int kStages = 3;

template <int D, bool CAUSAL, int HPW>
static int launch_one(const PrefillArgs& a) {
  const int nqb = (a.N + kTile - 1) / kTile;
  constexpr int QPW = 4 / HPW;
  const int nqg = (nqb + QPW - 1) / QPW;
  const int G = a.Hq / a.Hkv;
  const int ny = a.B * a.Hkv * (G / HPW);
  const long long blocks = (long long)nqg * ny;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, HPW, kStages>), dim3((unsigned)blocks), dim3(256),
                     0, (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.o, a.lse, a.mask, a.Hq, a.Hkv, a.N,
                     a.tau_raw, a.c, nqg, ny);
  return 0;
}

template <int D, bool CAUSAL>
static int launch_h(const PrefillArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (G % 4 == 0) return launch_one<D, CAUSAL, 4>(a);
  if (G % 2 == 0) return launch_one<D, CAUSAL, 2>(a);
  return launch_one<D, CAUSAL, 1>(a);
}

int launch_prefill(const PrefillArgs& a) {
  if (a.d == 128) return a.causal ? launch_h<128, true>(a) : launch_h<128, false>(a);
  return a.causal ? launch_h<64, true>(a) : launch_h<64, false>(a);
}

}  // namespace skipattn
