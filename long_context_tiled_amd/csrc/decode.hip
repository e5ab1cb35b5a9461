// Decode: one query token per sequence against a contiguous bf16 KV cache,
// split-K over fixed 4096-key splits, then a log-sum-exp merge.
//
// Method: blockwise attention (TurboAttention talk page, "Technical Deep
// Dive"; its profile in "Background" puts decode attention behind the
// KV-cache memory traffic) with the Skip-Softmax rule (TensorRT-LLM Skip
// Softmax summary page, "Key Points", "Detailed Analysis"). Each split runs
// the rule over its 64-key tiles in ascending order with its own running
// maximum per query head; the decision tile is one query x 64 keys.
//
// Split kernel: one wave per (sequence b, KV head g, split). The G query
// heads of g ride in the N dimension of v_mfma_f32_16x16x32_bf16 (16 slots):
//   S^T (16 keys x 16 heads) = K . q^T, K fragments loaded straight from HBM
//   as 16-byte row segments (K is read exactly once), next tile prefetched.
//   Lane l owns head (l & 15) and 16 keys of the tile; the tile max per head
//   is an in-lane max and two lane exchanges.
//   The V tile is loaded only when at least one head keeps the tile: 16-byte
//   coalesced row loads, transposed in registers into V^T in the wave's own
//   LDS region, in the key order that P^T's registers hand to the PV MFMA.
// The split writes its normalised partial output and LSE to the workspace.
//
// Merge kernel: one wave per (b, query head): LSE = log sum_s e^lse_s and
// O = sum_s e^(lse_s - LSE) O_s.
#include "common.hpp"
#include "launch.hpp"

namespace skipattn {

constexpr int kDecodeVStride = kTile * 2 + 16;  // bytes per V^T row (padded)

// Position, inside a V^T LDS row, of key j of the tile: within each 32-key
// group, key 16a + 4g + c sits at 8g + 4a + c.
__device__ __forceinline__ int dec_vt_pos(int j) {
  const int kap = j & 31;
  return (j & ~31) | (((kap >> 2) & 3) << 3) | (((kap >> 4) & 1) << 2) | (kap & 3);
}

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, uint8_t* __restrict__ mask, int Hq, int Hkv,
    int L, int nsplit, float tau_raw, float c, int nwork) {
  constexpr int KS = D / 32;  // k-steps over d (32 each) for S^T
  constexpr int DB = D / 16;  // 16-row d blocks of O^T
  constexpr int C8 = D / 8;   // 16-byte chunks per row
  constexpr int VB = (2 * D) / 64;  // 4-key x 8-d V blocks per lane
  __shared__ __attribute__((aligned(16))) char smem[4][D * kDecodeVStride];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int work = blockIdx.x * 4 + wave;
  if (work >= nwork) return;  // whole wave leaves; the kernel has no barrier
  const int sp = work % nsplit;
  const int bg = work / nsplit;
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  const int G = Hq / Hkv;
  const int hl = lane & 15;   // head slot
  const int grp = lane >> 4;  // lane group 0..3
  char* vs_ = smem[wave];

  const size_t kv_off = (size_t)(b * Hkv + g) * L * D;
  const uint16_t* kbase = k + kv_off;
  const uint16_t* vbase = v + kv_off;
  const int ntile_all = (L + kTile - 1) / kTile;
  const int key_begin = sp * kSplit;
  const int key_end = min(L, key_begin + kSplit);
  const int ntile = (key_end - key_begin + kTile - 1) / kTile;
  const bool head_ok = hl < G;
  const size_t bh = (size_t)b * Hq + g * G + hl;

  // q^T fragments: B[k = d][n = head].
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (head_ok) x = ldg16(q + bh * D + ks * 32 + 8 * grp);
    qf[ks] = as_bf16x8(x);
  }

  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[db][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  // K fragments: A[m = key][k = d], key 16 mb + hl, d = 32 ks + 8 grp.
  u32x4 kcur[4][KS], knext[4][KS];
  auto kload = [&](int t, u32x4 (&dst)[4][KS]) {
    const int key0 = key_begin + t * kTile;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int key = key0 + 16 * mb + hl;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < L) x = ldg16(kbase + (size_t)key * D + ks * 32 + 8 * grp);
        dst[mb][ks] = x;
      }
    }
  };

  kload(0, kcur);
  for (int t = 0; t < ntile; ++t) {
    if (t + 1 < ntile) kload(t + 1, knext);
    const int key0 = key_begin + t * kTile;

    // ---- S^T = K . q^T ----
    f32x4 s[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[mb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[mb][ks]), qf[ks], s[mb], 0, 0, 0);
    }
    if (key0 + kTile > L) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * mb + 4 * grp + r >= L) s[mb][r] = -INFINITY;
    }

    // ---- tile max per head, skip test per head ----
    float tmax = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[mb][r]);
    tmax = fmaxf(tmax, xor16(tmax));
    tmax = fmaxf(tmax, xor32(tmax));
    const bool keep = !(tmax < m - tau_raw);
    if (mask != nullptr && lane < G)
      mask[bh * ntile_all + key0 / kTile] = keep ? 0 : 1;
    const bool any = __ballot(keep && head_ok) != 0ull;

    if (any) {
      // ---- V tile -> V^T in this wave's LDS region ----
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const int blk = lane + 64 * j;
        const int kg = blk / C8, dc = blk % C8;
        u32x4 rows[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 4 * kg + i;
          u32x4 x = {0u, 0u, 0u, 0u};
          if (key < L) x = ldg16(vbase + (size_t)key * D + dc * 8);
          rows[i] = x;
        }
        const int pos = dec_vt_pos(4 * kg);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<u32x2*>(vs_ + (dc * 8 + e) * kDecodeVStride + pos * 2) =
              column_of_4x8(rows, e);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();

      // ---- online softmax for the heads that keep the tile ----
      const float mn = keep ? fmaxf(m, tmax) : m;
      if (mn > m) {
        const float alpha = exp2_fast((m - mn) * c);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[db][r] *= alpha;
      }
      m = mn;
      const float nmc = -mn * c;
      bf16x8 pf[2];
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 w;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int mb = 2 * ks + (i2 >> 1);
          const int r0 = 2 * (i2 & 1);
          float p0 = exp2_fast(__builtin_fmaf(s[mb][r0], c, nmc));
          float p1 = exp2_fast(__builtin_fmaf(s[mb][r0 + 1], c, nmc));
          if (!keep) { p0 = 0.f; p1 = 0.f; }
          part += p0 + p1;
          w[i2] = pack_bf16x2(p0, p1);
        }
        pf[ks] = as_bf16x8(w);
      }
      lsum += part;

      // ---- O^T += V^T . P^T ----
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
              vs_ + (16 * db + hl) * kDecodeVStride + (32 * ks + 8 * grp) * 2);
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ks], acc[db], 0, 0, 0);
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }

#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kcur[mb][ks] = knext[mb][ks];
  }

  // ---- split epilogue: normalised partial output and its LSE ----
  float ltot = lsum + xor16(lsum);
  ltot += xor32(ltot);
  if (head_ok) {
    const float inv = 1.f / ltot;
    float* dst = ws_o + (bh * nsplit + sp) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x4 val;
#pragma unroll
      for (int r = 0; r < 4; ++r) val[r] = acc[db][r] * inv;
      *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * grp) = val;
    }
    if (grp == 0) ws_lse[bh * nsplit + sp] = (m * c + __log2f(ltot)) * kLn2;
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    float* __restrict__ o, float* __restrict__ lse, int nbh, int nsplit) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= nbh) return;
  const float* ls = ws_lse + (size_t)bh * nsplit;
  float big = -INFINITY;
  for (int s = 0; s < nsplit; ++s) big = fmaxf(big, ls[s]);
  float wsum = 0.f;
  float out[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) out[i] = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float w = expf(ls[s] - big);
    wsum += w;
    const float* os = ws_o + ((size_t)bh * nsplit + s) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] += w * os[lane + 64 * i];
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[(size_t)bh * D + lane + 64 * i] = out[i] * inv;
  if (lane == 0) lse[bh] = big + logf(wsum);
}

template <int D>
static int launch_d(const DecodeArgs& a) {
  const long long nwork = (long long)a.B * a.Hkv * a.nsplit;
  const long long nbh = (long long)a.B * a.Hq;
  if (nwork > 0x7fffffffLL || nbh > 0x7fffffffLL) return -1;
  const unsigned g1 = (unsigned)((nwork + 3) / 4);
  const unsigned g2 = (unsigned)((nbh + 3) / 4);
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3(g1), dim3(256), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     a.ws_o, a.ws_lse, a.mask, a.Hq, a.Hkv, a.L, a.nsplit, a.tau_raw,
                     a.c, (int)nwork);
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(g2), dim3(256), 0, (hipStream_t)a.stream,
                     a.ws_o, a.ws_lse, a.o, a.lse, (int)nbh, a.nsplit);
  return 0;
}

int launch_decode(const DecodeArgs& a) {
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

}  // namespace skipattn
