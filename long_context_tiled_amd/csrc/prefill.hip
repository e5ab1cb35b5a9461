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
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace skipattn {

typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kBufferCfg = 0x00020000u;  // raw 32-bit buffer, range-checked

template <int D>
struct PrefillTile {
  static constexpr int rowBytes = 2 * D;
  static constexpr int chunks = D / 8;               // 16-byte chunks per row
  static constexpr int bytes = kTile * rowBytes;      // one K or V tile
  static constexpr int rowsPerInstr = 1024 / rowBytes;
  static constexpr int instrPerWave = kTile / rowsPerInstr / 4;
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
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
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

// Calls the d = 128 or d = 64 version of a generated block.
#define SKA_CALL(D_, fn, ...)                \
  do {                                       \
    if constexpr ((D_) == 128) d128::fn(__VA_ARGS__); \
    else d64::fn(__VA_ARGS__);               \
  } while (0)

template <int D, bool CAUSAL, int HPW, int STAGES, bool CHUNK>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_num_vgpr(40))) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, uint8_t* __restrict__ mask, int Hq, int Hkv,
    int Nq_arg, int N, int q0t_arg, float tau_raw, float c, int nqg, int ny) {
  // Nq queries (the chunk) at key positions 64 q0t .. 64 q0t + Nq - 1 of N
  // keys: query tile qb of the chunk is tile qb + q0t of the key axis. The
  // whole-sequence instance (CHUNK false) has Nq = N and q0t = 0 as
  // constants (same per-wave code; measured, about 40% fewer L2 misses than
  // the same values passed at run time).
  const int Nq = CHUNK ? Nq_arg : N;
  const int q0t = CHUNK ? q0t_arg : 0;
  constexpr int QPW = 4 / HPW;   // query tiles per workgroup
  constexpr int MB = D / 32;     // 32-row d blocks of O^T
  using T = PrefillTile<D>;
  constexpr int STAGE_BYTES = 2 * T::bytes;
  // STAGES K/V slots, tile t in slot t % STAGES. The four Q tiles are
  // staged in slots 3-4 before the loop.
  static_assert(STAGES == 5 && 4 * T::bytes == 2 * STAGE_BYTES, "slot plan");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
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
  const int qb = qg * QPW + wave / HPW;   // query tile within the chunk
  const int qbg = qb + q0t;               // the same tile on the key axis
  const int nqb = (Nq + kTile - 1) / kTile;
  const int nkb = (N + kTile - 1) / kTile;
  const bool wave_valid = qb < nqb;
  const int nkb_wg = CAUSAL ? min(nkb, qg * QPW + QPW + q0t) : nkb;
  const int nkb_w = wave_valid ? (CAUSAL ? qbg + 1 : nkb) : 0;

  const int head_bytes = N * D * 2;
  const size_t kv_off = (size_t)(b * Hkv + g) * N * D;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + kv_off), (short)0, head_bytes, kBufferCfg);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + kv_off), (short)0, head_bytes, kBufferCfg);
  const size_t bh = (size_t)b * Hq + h;
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(q + bh * Nq * D), (short)0, Nq * D * 2, kBufferCfg);

  // Per-lane load geometry for the direct-to-LDS copies: instruction i of
  // wave w fills LDS bytes [1024 (w * IPW + i), +1024) of the tile.
  constexpr int IPW = T::instrPerWave;
  int ld_gk[IPW], ld_gv[IPW];  // global byte offsets within the head, relative to key 0
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * T::rowsPerInstr + lane / T::chunks;
    const int slot = lane % T::chunks;
    ld_gk[i] = r * T::rowBytes + 16 * (slot ^ swz_k<D>(r));
    ld_gv[i] = r * T::rowBytes + 16 * (slot ^ swz_v<D>(r));
  }

  auto issue_tile = [&](int kb) __attribute__((always_inline)) {
    char* st = smem + (kb % STAGES) * STAGE_BYTES;
    const int base = kb * kTile * T::rowBytes;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      lds_void* dk = (lds_void*)(st + 1024 * (wave * IPW + i));
      dma16(krs, dk, base + ld_gk[i]);
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      lds_void* dv = (lds_void*)(st + T::bytes + 1024 * (wave * IPW + i));
      dma16(vrs, dv, base + ld_gv[i]);
    }
  };

  // The wave's 64 query rows go to its own swizzled LDS tile once (rows past
  // N read as zero), and from there into AGPRs.
  const uint32_t q_lds = (uint32_t)(3 * STAGE_BYTES + wave * T::bytes);
  if (wave_valid) {
    constexpr int QI = T::bytes / 1024;  // 1 KB copy instructions per Q tile
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int r = i * T::rowsPerInstr + lane / T::chunks;
      const int slot = lane % T::chunks;
      const int cc = slot ^ swz_k<D>(r);
      dma16(qrs, (lds_void*)(smem + q_lds + 1024 * i), (qb * kTile + r) * T::rowBytes + cc * 16);
    }
  }

  // K / Q fragment reads (A / B operands of S^T = K . Q^T): lane l reads row
  // (32 a + l32) of a swizzled tile, 16-byte chunk 2 ks + hh. With rows 32
  // apart sharing the swizzle, the second row half is the immediate offset
  // 32 rowBytes, and the chunk XOR (2 ks + hh) ^ g moves only address bits
  // 4..7 (bits below the row): the k-step ks address is frag ^ (32 ks) for a
  // 1 KB-aligned tile base.
  const uint32_t frag = (uint32_t)(l32 * T::rowBytes + 16 * (hh ^ swz_k<D>(l32)));

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

  // Prologue: Q tiles (slots 3-4) and K/V tiles 0-2 copied; Q^T into AGPRs.
  SKA_CALL(D, zero_o);
  for (int t = 0; t < 3; ++t)
    if (t < nkb_wg) issue_tile(t);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (0 < nkb_w) SKA_CALL(D, load_q, smem_lds + q_lds + frag);
  __syncthreads();  // slots 3-4 are K/V slots from here on

  // The key loop runs as one generated block (barriers, tile copies, the
  // pipelined steps, votes, rescales, masks). Its scalar operands must be
  // wave-uniform.
  const float lazy_raw = 8.0f / c;  // 8 in log2 units, as a raw-score gap
  typename std::conditional<D == 128, d128::LoopArgs, d64::LoopArgs>::type la;
  la.frag = frag;
  la.tr0 = tr0[0];
  la.tr1 = tr0[1];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    la.gk[i] = (uint32_t)ld_gk[i];
    la.gv[i] = (uint32_t)ld_gv[i];
  }
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
  auto rsrc = [&](const uint16_t* p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    u32x4 r;
    r[0] = (uint32_t)a;
    r[1] = (uint32_t)(a >> 32) & 0xffffu;  // stride 0
    r[2] = (uint32_t)head_bytes;
    r[3] = kBufferCfg;
    return r;
  };
  la.krs = rsrc(k + kv_off);
  la.vrs = rsrc(v + kv_off);
  la.wl = smem_lds + (uint32_t)(wave * IPW * 1024);
  la.smem = smem_lds;
  la.mask_row = mask != nullptr ? (uint64_t)(uintptr_t)(mask + (bh * nqb + qb) * nkb) : 0ull;
  float m[2], mref[2], lsum[2];
  if constexpr (CAUSAL) SKA_CALL(D, key_loop_causal, la, m, mref, lsum);
  else SKA_CALL(D, key_loop_full, la, m, mref, lsum);
  (void)m;

  if (!wave_valid) return;
  drain_mfma();

  // ---- epilogue: O = O^T / l, LSE = m / sqrt(d) + ln l ----
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float ltot = swap_halves_sum(lsum[nb]);
    const float inv = 1.f / ltot;
    const int row = qb * kTile + nb * 32 + l32;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float ov[16];
      const int id = 2 * mb + nb;
      if (id == 0) SKA_CALL(D, read_o_00, ov);
      if (id == 1) SKA_CALL(D, read_o_01, ov);
      if (id == 2) SKA_CALL(D, read_o_10, ov);
      if (id == 3) SKA_CALL(D, read_o_11, ov);
      if constexpr (MB == 4) {
        if (id == 4) d128::read_o_20(ov);
        if (id == 5) d128::read_o_21(ov);
        if (id == 6) d128::read_o_30(ov);
        if (id == 7) d128::read_o_31(ov);
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
}

constexpr int kStages = 5;

template <int D, bool CAUSAL, int HPW, bool CHUNK>
static int launch_one(const PrefillArgs& a) {
  const int nqb = (a.Nq + kTile - 1) / kTile;
  constexpr int QPW = 4 / HPW;
  const int nqg = (nqb + QPW - 1) / QPW;
  const int G = a.Hq / a.Hkv;
  const int ny = a.B * a.Hkv * (G / HPW);
  const long long blocks = (long long)nqg * ny;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, HPW, kStages, CHUNK>), dim3((unsigned)blocks), dim3(256),
                     0, (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.o, a.lse, a.mask, a.Hq, a.Hkv, a.Nq, a.N, a.q0t,
                     a.tau_raw, a.c, nqg, ny);
  return 0;
}

template <int D, bool CAUSAL, bool CHUNK>
static int launch_g(const PrefillArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (G % 4 == 0) return launch_one<D, CAUSAL, 4, CHUNK>(a);
  if (G % 2 == 0) return launch_one<D, CAUSAL, 2, CHUNK>(a);
  return launch_one<D, CAUSAL, 1, CHUNK>(a);
}

template <int D, bool CAUSAL>
static int launch_h(const PrefillArgs& a) {
  if (a.Nq != a.N || a.q0t != 0) return launch_g<D, CAUSAL, true>(a);
  return launch_g<D, CAUSAL, false>(a);
}

int launch_prefill(const PrefillArgs& a) {
  if (a.d == 128) return a.causal ? launch_h<128, true>(a) : launch_h<128, false>(a);
  return a.causal ? launch_h<64, true>(a) : launch_h<64, false>(a);
}

}  // namespace skipattn
