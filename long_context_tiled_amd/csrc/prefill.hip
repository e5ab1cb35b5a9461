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
// Per wave and key tile (d = D):
//   S^T (64 keys x 64 queries) = K . Q^T with v_mfma_f32_32x32x16_bf16:
//   lane l owns query column (l & 31) of each 32-query half, and 16 key rows
//   of each 32-key half. A query's tile max is an in-lane max over 32 values
//   and one exchange between lane halves (l, l ^ 32).
//   P^T, rounded to bf16, is already the B operand of O^T = V^T . P^T: the
//   MFMA contraction index is permuted consistently on both sides, and V^T is
//   written to LDS in that permuted key order.
//   O^T accumulates in fp32: lane l owns query (l & 31), so the online
//   rescale is one multiplier per lane.
//
// Units: scores stay raw (q.k) in registers. The test compares
// t < m - tau * sqrt(d); exponentials use exp2 with log2(e)/sqrt(d) folded
// into one FMA per score.
#include "common.hpp"
#include "launch.hpp"

namespace skipattn {

template <int D>
struct PrefillLds {
  static constexpr int kStride = D * 2 + 16;    // bytes per K row (padded)
  static constexpr int vStride = kTile * 2 + 16; // bytes per V^T row (padded)
  static constexpr int kBytes = kTile * kStride;
  static constexpr int vBytes = D * vStride;
  static constexpr int stage = kBytes + vBytes;
  static constexpr int total = 2 * stage;
};

// Position, inside V^T's LDS row, of key j of the tile: bits 2 and 3 of j are
// swapped, which is the order in which the S^T accumulator registers hand
// keys to the PV MFMA's contraction index.
__device__ __forceinline__ int vt_pos(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

template <int D, bool CAUSAL, int HPW>
__global__ __launch_bounds__(256, 1) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, uint8_t* __restrict__ mask, int Hq, int Hkv,
    int N, float tau_raw, float c, int nqg, int ny) {
  constexpr int QPW = 4 / HPW;   // query tiles per workgroup
  constexpr int KS = D / 16;     // MFMA k-steps over d for S^T
  constexpr int MB = D / 32;     // 32-row d blocks of O^T
  constexpr int NK = D / 32;     // 16-byte K chunks per thread per tile
  constexpr int C8 = D / 8;      // 16-byte chunks per row
  using Lds = PrefillLds<D>;
  __shared__ __attribute__((aligned(16))) char smem[Lds::total];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  const size_t kv_off = (size_t)(b * Hkv + g) * N * D;
  const uint16_t* kbase = k + kv_off;
  const uint16_t* vbase = v + kv_off;
  const size_t bh = (size_t)b * Hq + h;
  const uint16_t* qbase = q + bh * N * D;

  // Q^T fragments (B operand of S^T = K . Q^T): query row (l & 31) of each
  // 32-query half, d = 16 ks + 8 (l >> 5) .. + 7.
  bf16x8 qf[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = qb * kTile + nb * 32 + l32;
    const bool ok = wave_valid && row < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = ldg16(qbase + (size_t)row * D + ks * 16 + 8 * hh);
      qf[nb][ks] = as_bf16x8(x);
    }
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

  // Global -> register staging of one K/V tile.
  u32x4 kst[NK];
  u32x4 vst[4];
  const bool v_owner = tid < 2 * D;        // owns a 4-key x 8-d block of V
  const int v_kg = tid / C8;               // key group (4 keys)
  const int v_dc = tid % C8;               // 8-column chunk

  auto gload = [&](int kb) {
    const int key0 = kb * kTile;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / C8, col = cidx % C8;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key0 + row < N) x = ldg16(kbase + (size_t)(key0 + row) * D + col * 8);
      kst[i] = x;
    }
    if (v_owner) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * v_kg + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key0 + row < N) x = ldg16(vbase + (size_t)(key0 + row) * D + v_dc * 8);
        vst[j] = x;
      }
    }
  };

  auto swrite = [&](int st) {
    char* ks_ = smem + st * Lds::stage;
    char* vs_ = ks_ + Lds::kBytes;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / C8, col = cidx % C8;
      *reinterpret_cast<u32x4*>(ks_ + row * Lds::kStride + col * 16) = kst[i];
    }
    if (v_owner) {
      const int pos = vt_pos(4 * v_kg);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<u32x2*>(vs_ + (v_dc * 8 + e) * Lds::vStride + pos * 2) =
            column_of_4x8(vst, e);
    }
  };

  const float nc_tau = tau_raw;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int kb = 0; kb < nkb_wg; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nkb_wg) gload(kb + 1);

    if (kb < nkb_w) {
      const char* ks_ = smem + st * Lds::stage;
      const char* vs_ = ks_ + Lds::kBytes;

      // ---- S^T = K . Q^T (raw scores, fp32) ----
      f32x16 s[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[a][nb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              ks_ + (a * 32 + l32) * Lds::kStride + (ks * 16 + 8 * hh) * 2);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            s[a][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][ks], s[a][nb], 0, 0, 0);
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
        t[nb] = fmaxf(x, xor32(x));
      }

      // ---- Skip-Softmax vote: skip iff every valid row has t < m - tau ----
      bool blocks = false;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int qrow = qb * kTile + nb * 32 + l32;
        if (qrow < N && !(t[nb] < m[nb] - nc_tau)) blocks = true;
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
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                vs_ + (mb * 32 + l32) * Lds::vStride + (ks * 16 + 8 * hh) * 2);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks][nb], acc[mb][nb], 0, 0, 0);
          }
        }
      }
    }

    if (kb + 1 < nkb_wg) swrite(st ^ 1);
    __syncthreads();
  }

  if (!wave_valid) return;

  // ---- epilogue: O = O^T / l, LSE = m / sqrt(d) + ln l ----
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float ltot = lsum[nb] + xor32(lsum[nb]);
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

template <int D, bool CAUSAL, int HPW>
static int launch_one(const PrefillArgs& a) {
  const int nqb = (a.N + kTile - 1) / kTile;
  constexpr int QPW = 4 / HPW;
  const int nqg = (nqb + QPW - 1) / QPW;
  const int G = a.Hq / a.Hkv;
  const int ny = a.B * a.Hkv * (G / HPW);
  const long long blocks = (long long)nqg * ny;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, HPW>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
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
