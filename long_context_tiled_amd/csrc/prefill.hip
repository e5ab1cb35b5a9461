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
// per block (keys +0..3 and +8..11 of each lane half). The reads and the wait
// for them are one asm block, so no load is left in flight past it and the
// compiler adds no wait on the tile copies still in flight.
template <int MB>
__device__ __forceinline__ void read_vt(bf16x8 (&vf)[MB], uint32_t base, uint32_t a0, uint32_t a1) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  u32x2v r[2 * MB];
  uint32_t ad[2 * MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    ad[2 * mb] = base + (a0 ^ (64u * mb));
    ad[2 * mb + 1] = base + (a1 ^ (64u * mb));
  }
  if constexpr (MB == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
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
  bf16x8 qf[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = wave_valid ? qb * kTile + nb * 32 + l32 : N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(qrs, (row * D + ks * 16 + 8 * hh) * 2, 0, 0);
      qf[nb][ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

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

  // ds_read_b64_tr_b16 geometry for the V^T operand: lane k of a 16-lane
  // group fetches 4 consecutive d of key row (16 ks + key_base + k / 4); the
  // instruction hands lane i of the group element (i % 4) of the chunks of
  // lanes 4e + i / 4, e = 0..3, i.e. 4 keys of one d column. For each 32-d
  // block mb, the swizzled address is A ^ (64 mb) with A fixed per lane.
  const int grp16 = lane >> 4;
  const int k16 = lane & 15;
  uint32_t tr_addr[2];  // rows tr_row and tr_row + 8 of key step 0, mb = 0
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 4 * (grp16 >> 1) + (k16 >> 2) + 8 * half;
    const int d = 16 * (grp16 & 1) + 4 * (k16 & 3);
    tr_addr[half] = (uint32_t)(swz<D>(row, d >> 3) + 2 * (d & 7));
  }

  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
  float m[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

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
            if (ks == 0) {
              const f32x16 zero = {};
              s[a][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][0], zero, 0, 0, 0);
            } else {
              s[a][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][ks], s[a][nb], 0, 0, 0);
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
        float mn[2];
        bool grow = false;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          mn[nb] = fmaxf(m[nb], t[nb]);
          grow |= mn[nb] > m[nb];
        }
        if (__ballot(grow) != 0ull) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const float alpha = exp2_fast((m[nb] - mn[nb]) * c);
            lsum[nb] *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[mb][nb][r] *= alpha;
          }
        }
        bf16x8 pf[4][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          m[nb] = mn[nb];
          const float nmc = -mn[nb] * c;
          float part = 0.f;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            u32x4 w;
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
              const int r0 = 8 * (ks & 1) + 2 * i2;
              const float p0 = exp2_fast(__builtin_fmaf(s[ks >> 1][nb][r0], c, nmc));
              const float p1 = exp2_fast(__builtin_fmaf(s[ks >> 1][nb][r0 + 1], c, nmc));
              part += p0 + p1;
              w[i2] = pack_bf16x2(p0, p1);
            }
            pf[ks][nb] = as_bf16x8(w);
          }
          lsum[nb] += part;
        }

        // ---- O^T += V^T . P^T ----
        const uint32_t vbase = smem_lds + (uint32_t)(vs_ - smem);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 vf[MB];
          read_vt<MB>(vf, vbase + 16 * ks * T::rowBytes, tr_addr[0], tr_addr[1]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[mb], pf[ks][nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
  }

  if (!wave_valid) return;

  // ---- epilogue: O = O^T / l, LSE = m / sqrt(d) + ln l ----
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float ltot = swap_halves_sum(lsum[nb]);
    const float inv = 1.f / ltot;
    const int row = qb * kTile + nb * 32 + l32;
    if (row < N) {
      float* orow = o + (bh * N + row) * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 val;
#pragma unroll
          for (int i = 0; i < 4; ++i) val[i] = acc[mb][nb][4 * r4 + i] * inv;
          *reinterpret_cast<f32x4*>(orow + mb * 32 + 8 * r4 + 4 * hh) = val;
        }
      if (hh == 0) lse[bh * N + row] = (m[nb] * c + __log2f(ltot)) * kLn2;
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
