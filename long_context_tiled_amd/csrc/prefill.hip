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
//   A work item is one such workgroup's share (a query tile group of a head
//   group). Items are numbered longest-first for causal attention; the grid
//   holds one workgroup per compute unit, each starting on item blockIdx.x
//   and then taking the next unclaimed item from a device-wide counter, so
//   that compute units (and XCDs, whose clocks differ) that finish early
//   take more of the work.
//
// Data movement
//   K and V tiles (64 keys x d, bf16) go from HBM/L2 straight into LDS with
//   buffer_load_dwordx4 ... lds (no VGPR staging). Keys past N read as zero
//   through the buffer descriptor's range check. Rows are stored unpadded,
//   with their 16-byte chunks permuted per row (swz_k / swz_v below) so that
//   the fragment reads hit distinct LDS banks. There are five tile slots
//   (tile t in slot t % 5); the Q tiles pass through slots 3-4 on their way
//   to AGPRs. The loop takes one workgroup barrier per two key tiles and
//   copies tiles three ahead.
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
//   rescale is one multiplier per lane. It is lazy: the reference maximum
//   behind O and the row sums only moves when a row's maximum has grown by
//   more than 2^8 in exp2 units, which keeps every weight below 2^8.
//
// Schedule: the key loop is software-pipelined over two tiles. The per-tile
// steps (S^T MFMAs of tile n + 1 beside the exponentials of tile n, PV MFMAs
// of tile n beside the row maxima of tile n + 1) are hand-scheduled
// instruction blocks written by gen_prefill_steps.py into prefill_steps.inc,
// which also fixes the register plan: O^T and Q^T live in AGPRs, the scores
// of two tiles in v[128:255], fragments and P^T in v[48:127]; the compiler
// gets v[0:40) for everything else (amdgpu_num_vgpr below), so none of that
// state is ever an SSA value it could move or spill.
//
// Units: scores stay raw (q.k) in registers. The test compares
// t < m - tau * sqrt(d); exponentials use exp2 with log2(e)/sqrt(d) folded
// into one FMA per score.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "sas.hpp"

namespace skipattn {

typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kBufferCfg = 0x00020000u;  // raw 32-bit buffer, range-checked

// Tile geometry: V rows are bf16 (2 D bytes), or with the 8-bit P.V (V8) a
// V tile is a block of D rows of 64 E4M3 codes (one row per channel, in the
// contraction order of the P.V product); K and Q rows are bf16 too, or fp8
// codes (D bytes) when QK^T runs on 8-bit operands.
template <int D, bool F8, bool V8 = false>
struct PrefillTile {
  static constexpr int rowBytes = 2 * D;              // V (bf16)
  static constexpr int chunks = rowBytes / 16;        // 16-byte chunks per V row
  static constexpr int bytes = V8 ? kTile * D : kTile * rowBytes;  // one V tile
  static constexpr int rowsPerInstr = 1024 / rowBytes;
  static constexpr int instrPerWave = bytes / 1024 / 4;
  static constexpr int kRowBytes = F8 ? D : 2 * D;    // K and Q
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = kTile * kRowBytes;    // one K (or Q) tile
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;
  static constexpr int kInstrPerWave = kTile / kRowsPerInstr / 4;
};

// Tiles sit in LDS unpadded; the 16-byte chunk c of row r is stored at
// slot c ^ g(r) of its row, with g chosen so that the fragment reads hit
// distinct banks (64 banks of 4 bytes; a 128-bit read is served 16 lanes at
// a time, a 64-bit read 32 lanes at a time).
//   K and Q (read by ds_read_b128: 16 lanes = 16 consecutive rows, one
//   chunk): g must be one-to-one on 16 consecutive rows, modulo the 256-byte
//   bank period: g = r & 15 for d = 128, g = (r >> 1) & 7 for d = 64 (two
//   128-byte rows share a bank period).
//   V (read by ds_read_b64_tr_b16: 32 lanes = 4 consecutive rows x 4 chunks
//   4 mb .. 4 mb + 3): the 16 (row, chunk) pairs must fill all 16 bank
//   quads: g = 4 (r & 3) for d = 128, g = 4 ((r >> 1) & 1) for d = 64.
// XOR by g keeps chunk blocks 4 mb aligned, so the V^T address of block mb
// is that of block 0 XOR 64 mb.
// The K / Q swizzle by row size in bytes: 256-byte rows (bf16, d = 128),
// 128-byte rows (bf16 d = 64, fp8 d = 128) and 64-byte rows (fp8 d = 64),
// one-to-one on the rows that share a 16-lane read.
template <int RB>
__device__ __forceinline__ int swz_row(int r) {
  return RB == 256 ? (r & 15) : RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return swz_row<2 * D>(r);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
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

// Wait states after the last MFMA (8 passes) before its result registers
// may be read by other instructions.
__device__ __forceinline__ void drain_mfma() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// One 16-byte-per-lane copy from a buffer straight into LDS: lane i writes
// bytes [16 i, 16 i + 16) after the wave-uniform LDS address lds. (Kept out
// of the kernel body: used there directly, the builtin stops the host pass
// from emitting the kernel's launch stub.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, lds_void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0);
}

// The blocks name registers the compiler is told it may not allocate; the
// warning for such clobbers is expected.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#include "prefill_steps.inc"
#pragma clang diagnostic pop

// Calls the d = 128 or d = 64 version of a generated block (bf16 QK^T, or
// fp8 QK^T when F8_ is set, int8 when I8_ is set too; P.V on fp8 codes when
// V8_ is set).
#define SKA_CALL(D_, F8_, SAS_, V8_, I8_, fn, ...)                               \
  do {                                                                           \
    if constexpr ((I8_) && (D_) == 128) d128i8::fn(__VA_ARGS__);                 \
    else if constexpr (I8_) d64i8::fn(__VA_ARGS__);                              \
    else if constexpr ((V8_) && (D_) == 128 && (F8_)) d128f8v8::fn(__VA_ARGS__); \
    else if constexpr ((V8_) && (D_) == 128) d128v8::fn(__VA_ARGS__);            \
    else if constexpr ((V8_) && (F8_)) d64f8v8::fn(__VA_ARGS__);                 \
    else if constexpr (V8_) d64v8::fn(__VA_ARGS__);                              \
    else if constexpr ((SAS_) == 2 && (D_) == 128) d128s2::fn(__VA_ARGS__);      \
    else if constexpr ((SAS_) == 2) d64s2::fn(__VA_ARGS__);                      \
    else if constexpr ((SAS_) == 3 && (D_) == 128) d128s3::fn(__VA_ARGS__);      \
    else if constexpr ((SAS_) == 3) d64s3::fn(__VA_ARGS__);                      \
    else if constexpr ((D_) == 128 && !(F8_)) d128::fn(__VA_ARGS__);             \
    else if constexpr ((D_) == 64 && !(F8_)) d64::fn(__VA_ARGS__);              \
    else if constexpr ((D_) == 128) d128f8::fn(__VA_ARGS__);                    \
    else d64f8::fn(__VA_ARGS__);                                                \
  } while (0)

template <int D, bool F8, int SAS, bool V8, bool I8>
struct LoopArgsOf;
template <> struct LoopArgsOf<128, false, 0, false, false> { using type = d128::LoopArgs; };
template <> struct LoopArgsOf<64, false, 0, false, false> { using type = d64::LoopArgs; };
template <> struct LoopArgsOf<128, true, 0, false, false> { using type = d128f8::LoopArgs; };
template <> struct LoopArgsOf<64, true, 0, false, false> { using type = d64f8::LoopArgs; };
template <> struct LoopArgsOf<128, false, 2, false, false> { using type = d128s2::LoopArgs; };
template <> struct LoopArgsOf<64, false, 2, false, false> { using type = d64s2::LoopArgs; };
template <> struct LoopArgsOf<128, false, 3, false, false> { using type = d128s3::LoopArgs; };
template <> struct LoopArgsOf<64, false, 3, false, false> { using type = d64s3::LoopArgs; };
template <> struct LoopArgsOf<128, false, 0, true, false> { using type = d128v8::LoopArgs; };
template <> struct LoopArgsOf<64, false, 0, true, false> { using type = d64v8::LoopArgs; };
template <> struct LoopArgsOf<128, true, 0, true, false> { using type = d128f8v8::LoopArgs; };
template <> struct LoopArgsOf<64, true, 0, true, false> { using type = d64f8v8::LoopArgs; };
template <> struct LoopArgsOf<128, true, 0, false, true> { using type = d128i8::LoopArgs; };
template <> struct LoopArgsOf<64, true, 0, false, true> { using type = d64i8::LoopArgs; };

// I8 (with F8, whole-sequence only): Q and K are symmetric int8 codes with
// the same tile scales; S^T runs on v_mfma_i32_32x32x32_i8 (two per fp8
// MFMA: the contraction halves of the same operand registers), exact in
// int32. The sums start from the bits of 1/(2 pi), so each score s leaves
// the MFMA as the exact float 1/(2 pi) + s 2^-26 with no conversion; the Q
// scale carries the 2^26 back (sqv below).
// F8: Q and K are fp8 (E4M3) codes with one fp32 scale per 64-row Q tile
// (qsc, [B, Hq, ceil(Nq/64)]) and per 64-key K tile (ksc, [B, Hkv,
// ceil(cap/64)]); S^T = K . Q^T runs on v_mfma_f32_32x32x64_f8f6f4 in code
// units and each tile's scores are scaled by q scale x k scale where they
// are used (the skip test's tile maxima and the exponent input). V and PV
// stay bf16.
// SAS (2 or 3, bf16 QK^T only): every exponential of the online softmax, the
// probabilities and the rescale factor, is the SAS exponential of that
// degree (T[floor x] p(x - floor x), x the logit gap), with the reference
// maximum kept equal to the running maximum (no deferred rescale: SAS of a
// product is not the product of SAS values).
// V8 (whole-sequence only): P.V runs on v_mfma_f32_32x32x64_f8f6f4 with V as
// E4M3 code blocks (vsc: one fp32 scale per KV head, [B, Hkv]) and the
// probabilities rounded to E4M3 as they are packed: relative to the
// reference maximum they stay below 2^8, inside E4M3's range, so they take
// no scale. The row sums stay over the unrounded probabilities, and the
// head's V scale multiplies O with 1 / l.
template <int D, bool CAUSAL, int HPW, int STAGES, bool CHUNK, bool F8, int SAS, bool V8,
          bool I8>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_num_vgpr(40))) void prefill_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, uint8_t* __restrict__ mask, const float* __restrict__ qsc,
    const float* __restrict__ ksc, const float* __restrict__ vsc, int Hq, int Hkv,
    int Nq_arg, int N, int q0t_arg, int cap_arg, float tau_raw, float c, int nqg, int ny,
    uint32_t* __restrict__ queue, int total) {
  // Nq queries (the chunk) at key positions 64 q0t .. 64 q0t + Nq - 1 of N
  // keys: query tile qb of the chunk is tile qb + q0t of the key axis. The
  // whole-sequence instance (CHUNK false) has Nq = N and q0t = 0 as
  // constants (same per-wave code; measured, about 40% fewer L2 misses than
  // the same values passed at run time).
  const int Nq = CHUNK ? Nq_arg : N;
  const int q0t = CHUNK ? q0t_arg : 0;
  const int cap = CHUNK ? cap_arg : N;  // rows allocated per K/V head
  constexpr int QPW = 4 / HPW;   // query tiles per workgroup
  constexpr int MB = D / 32;     // 32-row d blocks of O^T
  using T = PrefillTile<D, F8, V8>;
  constexpr int KRB = T::kRowBytes;
  constexpr int STAGE_BYTES = T::kBytes + T::bytes;  // K tile then V tile
  // STAGES K/V slots, tile t in slot t % STAGES. The four Q tiles are
  // staged from slot 3 on before the loop (with 8-bit V tiles and bf16 Q
  // they run past the slots).
  constexpr int SMEM_BYTES = std::max(STAGES * STAGE_BYTES, 3 * STAGE_BYTES + 4 * T::kBytes);
  static_assert(STAGES == 5 && SMEM_BYTES <= 160 * 1024, "slot plan");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char*)smem;  // LDS byte address

  const int G = Hq / Hkv;
  const int gper = G / HPW;

  auto run_item = [&](const int lin, uint32_t& nxt) __attribute__((always_inline)) {
    // The lane geometry is re-derived for every item from an opaque copy of
    // the thread index: hoisted out of the item loop, it would stay live
    // through the key loop and the epilogue, and the compiler's registers
    // would no longer fit below the key loop's fixed register plan.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int y = lin % ny;
    const int qg = CAUSAL ? (nqg - 1 - lin / ny) : lin / ny;
    const int b = y / (Hkv * gper);
    const int rem = y % (Hkv * gper);
    const int g = rem / gper;
    const int h = g * G + (rem % gper) * HPW + (wave % HPW);
    const int qb = qg * QPW + wave / HPW;   // query tile within the chunk
    const int qbg = qb + q0t;               // the same tile on the key axis
    const int nqb = (Nq + kTile - 1) / kTile;
    const int nkb = (N + kTile - 1) / kTile;
    const bool wave_valid = qb < nqb;
    const int nkb_wg = CAUSAL ? min(nkb, qg * QPW + QPW + q0t) : nkb;
    const int nkb_w = wave_valid ? (CAUSAL ? qbg + 1 : nkb) : 0;

    const int k_head_bytes = N * KRB;
    // V8: the head's code blocks, nkb of them (N = cap for the V8 instances)
    const int v_head_bytes = V8 ? nkb * T::bytes : N * D * 2;
    const size_t kv_row0 = (size_t)(b * Hkv + g) * cap;  // first row of the head's K/V
    const uint8_t* kh = k + kv_row0 * KRB;
    const uint8_t* vh = V8 ? v + (size_t)(b * Hkv + g) * nkb * T::bytes : v + kv_row0 * D * 2;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)kh, (short)0, k_head_bytes, kBufferCfg);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)vh, (short)0, v_head_bytes, kBufferCfg);
    const size_t bh = (size_t)b * Hq + h;
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q + bh * Nq * KRB), (short)0, Nq * KRB, kBufferCfg);

    // Per-lane load geometry for the direct-to-LDS copies: instruction i of
    // wave w fills LDS bytes [1024 (w * IPW + i), +1024) of the tile (K and V
    // tiles each; their instruction counts differ when K is fp8).
    constexpr int IPW = T::instrPerWave;
    constexpr int KIPW = T::kInstrPerWave;
    int ld_gk[KIPW], ld_gv[IPW];  // global byte offsets within the head, relative to key 0
  #pragma unroll
    for (int i = 0; i < KIPW; ++i) {
      const int r = (wave * KIPW + i) * T::kRowsPerInstr + lane / T::kChunks;
      const int slot = lane % T::kChunks;
      ld_gk[i] = r * KRB + 16 * (slot ^ swz_row<KRB>(r));
    }
  #pragma unroll
    for (int i = 0; i < IPW; ++i) {
      if constexpr (V8) {
        // code blocks are stored as they sit in LDS: a linear copy
        ld_gv[i] = (wave * IPW + i) * 1024 + 16 * lane;
      } else {
        const int r = (wave * IPW + i) * T::rowsPerInstr + lane / T::chunks;
        const int slot = lane % T::chunks;
        ld_gv[i] = r * T::rowBytes + 16 * (slot ^ swz_v<D>(r));
      }
    }

    auto issue_tile = [&](int kb) __attribute__((always_inline)) {
      char* st = smem + (kb % STAGES) * STAGE_BYTES;
  #pragma unroll
      for (int i = 0; i < KIPW; ++i) {
        lds_void* dk = (lds_void*)(st + 1024 * (wave * KIPW + i));
        dma16(krs, dk, kb * T::kBytes + ld_gk[i]);
      }
  #pragma unroll
      for (int i = 0; i < IPW; ++i) {
        lds_void* dv = (lds_void*)(st + T::kBytes + 1024 * (wave * IPW + i));
        dma16(vrs, dv, kb * T::bytes + ld_gv[i]);
      }
    };

    // The wave's 64 query rows go to its own swizzled LDS tile once (rows past
    // N read as zero), and from there into AGPRs.
    const uint32_t q_lds = (uint32_t)(3 * STAGE_BYTES + wave * T::kBytes);
    if (wave_valid) {
      constexpr int QI = T::kBytes / 1024;  // 1 KB copy instructions per Q tile
  #pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int r = i * T::kRowsPerInstr + lane / T::kChunks;
        const int slot = lane % T::kChunks;
        const int cc = slot ^ swz_row<KRB>(r);
        dma16(qrs, (lds_void*)(smem + q_lds + 1024 * i), (qb * kTile + r) * KRB + cc * 16);
      }
    }

    // K / Q fragment reads (A / B operands of S^T = K . Q^T): lane l reads row
    // (32 a + l32) of a swizzled tile. bf16: 16-byte chunk 2 ks + hh; fp8: the
    // chunks 4 ks + 2 hh and 4 ks + 2 hh + 1. With rows 32 apart sharing the
    // swizzle, the second row half is an immediate offset, and the chunk XOR
    // moves only address bits below the row: the k-step address is frag ^
    // (32 ks) (bf16) or frag ^ (64 ks) with the second chunk at ^ 16 (fp8),
    // for a 1 KB-aligned tile base.
    const uint32_t frag =
        (uint32_t)(l32 * KRB + 16 * ((F8 ? 2 * hh : hh) ^ swz_row<KRB>(l32)));

    // ds_read_b64_tr_b16 geometry for the V^T operand: lane k of a 16-lane
    // group fetches 4 consecutive d of key row (16 ks + key_base + k / 4); the
    // instruction hands lane i of the group element (i % 4) of the chunks of
    // lanes 4e + i / 4, e = 0..3, i.e. 4 keys of one d column. For 32-d block
    // mb the swizzled address is (that of block 0) ^ (64 mb).
    const int grp16 = lane >> 4;
    const int k16 = lane & 15;
    uint32_t tr0[2];  // block-0 address of each 4-key half, within a tile
  #pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 4 * (grp16 >> 1) + (k16 >> 2) + 8 * half;
      const int d = 16 * (grp16 & 1) + 4 * (k16 & 3);
      tr0[half] = (uint32_t)(row * T::rowBytes + 16 * ((d >> 3) ^ swz_v<D>(row)) + 2 * (d & 7));
    }
    if constexpr (V8) {
      // V^T operand of the 8-bit P.V: lane l reads code row l32 of each
      // 32-row block, contraction indices 32 hh .. 32 hh + 31: chunks 2 hh
      // and 2 hh + 1, stored at chunk (x ^ ((row >> 2) & 3)); the second
      // is the first's address ^ 16, block mb 2 KB further
      tr0[0] = (uint32_t)(l32 * 64 + 16 * ((2 * hh) ^ ((l32 >> 2) & 3)));
      tr0[1] = tr0[0] ^ 16u;
    }

    // Prologue: Q tiles (slots 3-4) and K/V tiles 0-2 copied; Q^T into AGPRs.
    SKA_CALL(D, F8, SAS, V8, I8, zero_o);
    for (int t = 0; t < 3; ++t)
      if (t < nkb_wg) issue_tile(t);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (0 < nkb_w) SKA_CALL(D, F8, SAS, V8, I8, load_q, smem_lds + q_lds + frag);
    __syncthreads();  // slots 3-4 are K/V slots from here on

    // The key loop runs as one generated block (barriers, tile copies, the
    // pipelined steps, votes, rescales, masks). Its scalar operands must be
    // wave-uniform.
    const float lazy_raw = 8.0f / c;  // 8 in log2 units, as a raw-score gap
    typename LoopArgsOf<D, F8, SAS, V8, I8>::type la;
    la.frag = frag;
    la.tr0 = tr0[0];
    la.tr1 = tr0[1];
  #pragma unroll
    for (int i = 0; i < KIPW; ++i) la.gk[i] = (uint32_t)ld_gk[i];
  #pragma unroll
    for (int i = 0; i < IPW; ++i) la.gv[i] = (uint32_t)ld_gv[i];
  #pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int qrow = qb * kTile + nb * 32 + l32;  // row within the chunk
      const int qpos = qbg * kTile + nb * 32 + l32; // its key position
      const int last = CAUSAL ? min(N - 1, qpos) : N - 1;  // last key this row may see
      la.lim_base[nb] = last - 4 * hh;
      la.val[nb] = __ballot(qrow < Nq);
    }
    la.lazy = lazy_raw;
    la.nkb_wg = nkb_wg;
    la.nkb_w = __builtin_amdgcn_readfirstlane(nkb_w);
    la.qb = __builtin_amdgcn_readfirstlane(qbg);  // the diagonal tile
    la.N = N;
    la.tau = tau_raw;
    la.c = c;
    if constexpr (SAS != 0) {
      la.c = c * kLn2;  // 1 / sqrt(d): the SAS argument is in logits
      la.lazy = 0.f;
#pragma unroll
      for (int j = 0; j <= SAS; ++j) la.sa[j] = SAS == 2 ? kSasPoly2[j] : kSasPoly3[j];
      la.c6 = 6.f;
      la.c7 = 7.f;
    }
    auto rsrc = [&](const void* p, int bytes) {
      const uint64_t a = (uint64_t)(uintptr_t)p;
      u32x4 r;
      r[0] = (uint32_t)a;
      r[1] = (uint32_t)(a >> 32) & 0xffffu;  // stride 0
      r[2] = (uint32_t)bytes;
      r[3] = kBufferCfg;
      return r;
    };
    la.krs = rsrc(kh, k_head_bytes);
    la.vrs = rsrc(vh, v_head_bytes);
    la.wl = smem_lds + (uint32_t)(wave * KIPW * 1024);
    la.smem = smem_lds;
    la.mask_row = mask != nullptr ? (uint64_t)(uintptr_t)(mask + (bh * nqb + qb) * nkb) : 0ull;
    if constexpr (F8) {
      const int nkbc = (cap + kTile - 1) / kTile;  // K scales per head
      la.ksp = (uint64_t)(uintptr_t)(ksc + (size_t)(b * Hkv + g) * nkbc);
      // int8: times 2^26 (exact), the unit of the scores as the int8 key
      // loops read them
      la.sqv = (wave_valid ? qsc[bh * nqb + qb] : 1.f) * (I8 ? 0x1p26f : 1.f);
      la.nkbm1 = nkb - 1;
      la.wlv = smem_lds + (uint32_t)(T::kBytes + wave * IPW * 1024);
    } else if constexpr (V8) {
      la.wlv = smem_lds + (uint32_t)(T::kBytes + wave * IPW * 1024);
    }
    float m[2], mref[2], lsum[2];
    if constexpr (CAUSAL) SKA_CALL(D, F8, SAS, V8, I8, key_loop_causal, la, m, mref, lsum);
    else SKA_CALL(D, F8, SAS, V8, I8, key_loop_full, la, m, mref, lsum);
    (void)m;

    // Claim the next item as this one's key loop ends: a claim made earlier
    // would bind a workgroup to its next item before it is known to be
    // among the first free, which undoes the longest-first balance when
    // there are few items per workgroup.
    uint32_t claim = 0;
    if (tid == 0) claim = atomicAdd(queue, 1u);
    nxt = __builtin_amdgcn_readfirstlane(claim) + gridDim.x;  // meaningful in wave 0
    if (!wave_valid) return;
    drain_mfma();

    // ---- epilogue: O = O^T / l (V8: times the head's V scale), LSE = m / sqrt(d) + ln l ----
    const float oscale = V8 ? vsc[b * Hkv + g] : 1.f;
  #pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float ltot = swap_halves_sum(lsum[nb]);
      const float inv = oscale / ltot;
      const int row = qb * kTile + nb * 32 + l32;
  #pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float ov[16];
        const int id = 2 * mb + nb;
        if (id == 0) SKA_CALL(D, F8, SAS, V8, I8, read_o_00, ov);
        if (id == 1) SKA_CALL(D, F8, SAS, V8, I8, read_o_01, ov);
        if (id == 2) SKA_CALL(D, F8, SAS, V8, I8, read_o_10, ov);
        if (id == 3) SKA_CALL(D, F8, SAS, V8, I8, read_o_11, ov);
        if constexpr (MB == 4 && !F8) {
          if (id == 4) d128::read_o_20(ov);
          if (id == 5) d128::read_o_21(ov);
          if (id == 6) d128::read_o_30(ov);
          if (id == 7) d128::read_o_31(ov);
        } else if constexpr (MB == 4 && I8) {
          if (id == 4) d128i8::read_o_20(ov);
          if (id == 5) d128i8::read_o_21(ov);
          if (id == 6) d128i8::read_o_30(ov);
          if (id == 7) d128i8::read_o_31(ov);
        } else if constexpr (MB == 4) {
          if (id == 4) d128f8::read_o_20(ov);
          if (id == 5) d128f8::read_o_21(ov);
          if (id == 6) d128f8::read_o_30(ov);
          if (id == 7) d128f8::read_o_31(ov);
        }
        if (row < Nq) {
          float* orow = o + (bh * Nq + row) * D;
  #pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 val;
  #pragma unroll
            for (int i = 0; i < 4; ++i) val[i] = ov[4 * r4 + i] * inv;
            *reinterpret_cast<f32x4*>(orow + mb * 32 + 8 * r4 + 4 * hh) = val;
          }
        }
      }
      if (row < Nq && hh == 0) lse[bh * Nq + row] = (mref[nb] * c + __log2f(ltot)) * kLn2;
    }
    if (CAUSAL && mask != nullptr) {
      for (int kb = qbg + 1 + lane; kb < nkb; kb += 64)
        mask[(bh * nqb + qb) * nkb + kb] = 2;
    }
  };

  uint32_t* const bcast = reinterpret_cast<uint32_t*>(smem);
  int item = blockIdx.x;
  while (item < total) {
    uint32_t nxt = 0;
    run_item(item, nxt);
    __syncthreads();  // every wave is done with the LDS tiles
    if (threadIdx.x == 0) bcast[0] = nxt;
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(bcast[0]);
    __syncthreads();  // read before the next item's copies overwrite slot 0
  }
  // The last workgroup out returns the counter pair to zero for the next
  // call that uses this slot. Every claim of every workgroup (its result
  // consumed above) precedes that workgroup's count.
  if (threadIdx.x == 0) {
    __threadfence();
    if (atomicAdd(queue + 1, 1u) == gridDim.x - 1) {
      __threadfence();
      atomicExch(queue, 0u);
      atomicExch(queue + 1, 0u);
    }
  }
}

constexpr int kStages = 5;

// Work-item counters of the persistent prefill grid: kQueueSlots pairs
// (next item, workgroups finished), each in its own 64-byte line, zero at
// load and returned to zero by the last workgroup of every call. A call
// takes the next slot in turn, so calls in flight at the same time on
// different streams share a slot only when kQueueSlots - 1 other prefill
// calls were made between them. Each GPU holds its own copy; host code uses
// the address from hipGetSymbolAddress, taken once per device.
constexpr int kQueueSlots = 1024;
static __device__ __align__(256) uint32_t prefill_queue[kQueueSlots * 16];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<uint32_t*> g_queue_addr[kMaxDevices];
std::atomic<int> g_num_cu[kMaxDevices];
std::atomic<uint32_t> g_next_slot{0};

// The current device's counter array and compute-unit count.
int queue_and_cus(uint32_t** q, int* ncu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -2;
  uint32_t* p = g_queue_addr[dev].load(std::memory_order_acquire);
  int n = g_num_cu[dev].load(std::memory_order_acquire);
  if (p == nullptr || n <= 0) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(prefill_queue)) != hipSuccess || a == nullptr)
      return -2;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return -2;
    p = static_cast<uint32_t*>(a);
    g_queue_addr[dev].store(p, std::memory_order_release);
    g_num_cu[dev].store(n, std::memory_order_release);
  }
  *q = p;
  *ncu = n;
  return 0;
}
}  // namespace

template <int D, bool CAUSAL, int HPW, bool CHUNK, bool F8, int SAS, bool V8 = false,
          bool I8 = false>
static int launch_one(const PrefillArgs& a) {
  const int nqb = (a.Nq + kTile - 1) / kTile;
  constexpr int QPW = 4 / HPW;
  const int nqg = (nqb + QPW - 1) / QPW;
  const int G = a.Hq / a.Hkv;
  const int ny = a.B * a.Hkv * (G / HPW);
  const long long items = (long long)nqg * ny;
  if (items > 0x7fffffffLL) return -1;
  if (items == 0) return 0;
  uint32_t* queue = nullptr;
  int ncu = 0;
  if (queue_and_cus(&queue, &ncu) != 0) return -2;
  queue += 16 * (g_next_slot.fetch_add(1, std::memory_order_relaxed) % kQueueSlots);
  // one workgroup per compute unit (the tile slots fill the LDS)
  const int grid = (int)std::min<long long>(items, ncu);
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, HPW, kStages, CHUNK, F8, SAS, V8, I8>),
                     dim3((unsigned)grid), dim3(256), 0, (hipStream_t)a.stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.o, a.lse,
                     a.mask, a.qscale, a.kscale, a.vscale, a.Hq, a.Hkv,
                     a.Nq, a.N, a.q0t, a.cap, a.tau_raw, a.c, nqg, ny, queue, (int)items);
  return 0;
}

template <int D, bool CAUSAL, bool CHUNK, bool F8, int SAS, bool V8 = false, bool I8 = false>
static int launch_g(const PrefillArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (G % 4 == 0) return launch_one<D, CAUSAL, 4, CHUNK, F8, SAS, V8, I8>(a);
  if (G % 2 == 0) return launch_one<D, CAUSAL, 2, CHUNK, F8, SAS, V8, I8>(a);
  return launch_one<D, CAUSAL, 1, CHUNK, F8, SAS, V8, I8>(a);
}

template <int D, bool CAUSAL, bool F8>
static int launch_h(const PrefillArgs& a) {
  if (a.Nq != a.N || a.q0t != 0 || a.cap != a.N) return launch_g<D, CAUSAL, true, F8, 0>(a);
  return launch_g<D, CAUSAL, false, F8, 0>(a);
}

template <bool F8>
static int launch_f(const PrefillArgs& a) {
  if (a.d == 128) return a.causal ? launch_h<128, true, F8>(a) : launch_h<128, false, F8>(a);
  return a.causal ? launch_h<64, true, F8>(a) : launch_h<64, false, F8>(a);
}

// The SAS key loops exist for the whole-sequence bf16 prefill only.
template <int SAS>
static int launch_s(const PrefillArgs& a) {
  if (a.d == 128)
    return a.causal ? launch_g<128, true, false, false, SAS>(a)
                    : launch_g<128, false, false, false, SAS>(a);
  return a.causal ? launch_g<64, true, false, false, SAS>(a)
                  : launch_g<64, false, false, false, SAS>(a);
}

// The 8-bit P.V key loops exist for the whole-sequence prefill (QK^T in bf16
// or fp8).
template <bool F8>
static int launch_v8(const PrefillArgs& a) {
  if (a.d == 128)
    return a.causal ? launch_g<128, true, false, F8, 0, true>(a)
                    : launch_g<128, false, false, F8, 0, true>(a);
  return a.causal ? launch_g<64, true, false, F8, 0, true>(a)
                  : launch_g<64, false, false, F8, 0, true>(a);
}

// The int8 QK^T key loops exist for the whole-sequence prefill (P.V in bf16).
static int launch_i8(const PrefillArgs& a) {
  if (a.d == 128)
    return a.causal ? launch_g<128, true, false, true, 0, false, true>(a)
                    : launch_g<128, false, false, true, 0, false, true>(a);
  return a.causal ? launch_g<64, true, false, true, 0, false, true>(a)
                  : launch_g<64, false, false, true, 0, false, true>(a);
}

int launch_prefill(const PrefillArgs& a) {
  if (a.qk_int8) {
    if (a.qscale == nullptr || a.vscale != nullptr || a.sas != 0 || a.Nq != a.N || a.q0t != 0 ||
        a.cap != a.N)
      return -3;
    return launch_i8(a);
  }
  if (a.vscale != nullptr) {
    if (a.sas != 0 || a.Nq != a.N || a.q0t != 0 || a.cap != a.N) return -3;
    return a.qscale != nullptr ? launch_v8<true>(a) : launch_v8<false>(a);
  }
  if (a.sas != 0) {
    if (a.qscale != nullptr || a.Nq != a.N || a.q0t != 0 || a.cap != a.N) return -3;
    return a.sas == 2 ? launch_s<2>(a) : launch_s<3>(a);
  }
  return a.qscale != nullptr ? launch_f<true>(a) : launch_f<false>(a);
}

}  // namespace skipattn
