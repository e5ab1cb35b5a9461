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
//   (K is read exactly once), next tile prefetched.
//   Lane l owns head (l & 15) and 16 keys of the tile; the tile max per head
//   is an in-lane max and two lane exchanges.
//   The V tile is read from memory only when at least one head keeps the
//   tile; it is transposed in registers into V^T in the wave's own LDS
//   region, in the key order that P^T's registers hand to the PV MFMA.
//   Every K and V load instruction reads 8 rows x 128 contiguous bytes (whole
//   128-byte lines) as a streaming (non-temporal) load: the cache keeps no
//   line that is read once, and no line is split between two instructions.
//   The fragment layouts above hold only 4 lanes per key row, so each pair of
//   loads is dealt out to its lanes by one exchange between lanes l and l ^ 8
//   (pair_fix).
// The split writes its normalised partial output and LSE to the workspace,
// and the skip bits of its tiles to the optional mask after its loop.
//
// Merge kernel: one wave per (b, query head): LSE = log sum_s e^lse_s and
// O = sum_s e^(lse_s - LSE) O_s.
#include <atomic>

#include "common.hpp"
#include "lane_max.hpp"
#include "sas.hpp"
#include "launch.hpp"

namespace skipattn {

constexpr int kDecodeVStride = kTile * 2 + 16;  // bytes per V^T row (padded)
constexpr uint32_t kBufferCfg = 0x00020000u;    // raw 32-bit buffer, range-checked

// Position, inside a V^T LDS row, of key j of the tile: within each 32-key
// group, key 16a + 4g + c sits at 8g + 4a + c (the order in which the S^T
// accumulator registers hand keys to the PV MFMA's contraction index).
__device__ __forceinline__ int dec_vt_pos(int j) {
  const int kap = j & 31;
  return (j & ~31) | (((kap >> 2) & 3) << 3) | (((kap >> 4) & 1) << 2) | (kap & 3);
}

// 16-byte raw buffer load with the non-temporal cache policy (bit 1 of the
// cache-policy operand): the KV cache is streamed once per call.
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 2));
}
// Tile base offset of a load that must read nothing: at or above 2^31, past
// every head's byte range (the host keeps head slices below 2^31 - 2^16), so
// the range check returns zeros without a memory access. Every iteration of
// the tile loop issues the same loads, wanted or not: the wait counts that the
// compiler derives then hold on every path and never drain loads still needed
// in flight.
constexpr uint32_t kNoLoad = 0x80000000u;

// A pair of loads I0, I1 covers 16 rows x 8 chunks (I0 the first 8 rows, I1
// the last 8). Lane (hl, grp) read chunk grp of its rows if hl < 8 ("lo"),
// chunk grp + 4 if not. The fragments want row hl with chunk grp in r0 and
// chunk grp + 4 in r1, so a lo lane keeps I0 as r0 and takes r1 from lane
// hl + 8's I0, and a hi lane keeps I1 as r1 and takes r0 from lane hl - 8's
// I1. The exchange is a rotate by 8 lanes within each 16-lane row (DPP
// row_ror:8, control 0x128).
__device__ __forceinline__ void pair_fix(u32x4& r0, u32x4& r1, bool lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t y0 = __builtin_amdgcn_mov_dpp((int)r0[e], 0x128, 0xf, 0xf, false);
    const uint32_t y1 = __builtin_amdgcn_mov_dpp((int)r1[e], 0x128, 0xf, 0xf, false);
    r0[e] = lo ? r0[e] : y1;
    r1[e] = lo ? y0 : r1[e];
  }
}

// SAS = 0: exact exponentials; SAS = 2 or 3: every exponential of the
// split's online softmax (the probabilities and the rescale factor) is
// sas_exp<SAS> of the distance below the running maximum in logits.
template <int D, int SAS>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, uint8_t* __restrict__ mask, int Hq, int Hkv,
    int L, int cap, int nhs, int nsplit, float tau_raw, float c, int nwork) {
  constexpr int KS = D / 32;        // k-steps over d (32 each) for S^T
  constexpr int DB = D / 16;        // 16-row d blocks of O^T
  constexpr int VB = (2 * D) / 64;  // 4-key x 8-d V blocks per lane
  static_assert(kSplit / kTile <= 64, "the per-lane skip bits hold one split");
  __shared__ __attribute__((aligned(16))) char smem[4][D * kDecodeVStride];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int work = blockIdx.x * 4 + wave;
  if (work >= nwork) return;  // whole wave leaves; the kernel has no barrier
  const int sp = work % nsplit;
  const int hs = (work / nsplit) % nhs;  // which 16 query heads of the group
  const int bg = work / nsplit / nhs;
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  const int G = Hq / Hkv;
  const int hoff = 16 * hs;  // first head of this wave's slice, within the group
  const int hl = lane & 15;   // head slot
  const int grp = lane >> 4;  // lane group 0..3
  char* vs_ = smem[wave];

  const size_t kv_off = (size_t)(b * Hkv + g) * cap * D;  // heads are cap rows apart
  const int head_bytes = L * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + kv_off), (short)0, head_bytes, kBufferCfg);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + kv_off), (short)0, head_bytes, kBufferCfg);
  const int ntile_all = (L + kTile - 1) / kTile;
  const int key_begin = sp * kSplit;
  const int key_end = min(L, key_begin + kSplit);
  const int ntile = (key_end - key_begin + kTile - 1) / kTile;
  const bool head_ok = hoff + hl < G;
  const size_t bh = (size_t)b * Hq + g * G + hoff + hl;

  // q^T fragments: B[k = d][n = head].
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (head_ok) x = ldg16(q + bh * D + ks * 32 + 8 * grp);
    qf[ks] = as_bf16x8(x);
  }

  const bool lo = hl < 8;
  const int h7 = hl & 7, hi4 = 4 * (hl >> 3);
  // K fragments: A[m = key][k = d], key 16 mb + hl, d = 32 ks + 8 grp (chunk
  // 4 ks + grp); keys past L read as zero. Loaded as pairs (2p, 2p + 1): load
  // s of the pair reads rows 16 mb + 8 s + (hl & 7), chunk 8 p + grp + 4 (hl >> 3).
  u32x4 kreg[4][KS];
  auto kload = [&](int t) {
    const uint32_t tb = t < ntile ? (uint32_t)(key_begin + t * kTile) * (D * 2) : kNoLoad;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kreg[mb][ks] = bload16(
            krs, tb + ((16 * mb + 8 * (ks & 1) + h7) * D + 8 * (8 * (ks >> 1) + grp + hi4)) * 2);
  };
  auto kfix = [&]() {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int p = 0; p < KS / 2; ++p) pair_fix(kreg[mb][2 * p], kreg[mb][2 * p + 1], lo);
  };
  // V blocks of 4 keys x 8 d: lane l takes key group (l & 15), d chunk
  // (l >> 4) + 4 j, so that the transposed LDS writes of one instruction
  // cover whole V^T rows (no bank conflicts). Loaded as pairs (2q, 2q + 1):
  // load j reads key group (hl & 7) + 8 (j & 1), chunk grp + 4 (hl >> 3) + 8 (j >> 1).
  u32x4 vreg[VB][4];
  auto vload = [&](int t, bool want) {
    const uint32_t tb = want && t < ntile ? (uint32_t)(key_begin + t * kTile) * (D * 2) : kNoLoad;
#pragma unroll
    for (int j = 0; j < VB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vreg[j][i] = bload16(
            vrs, tb + ((4 * (h7 + 8 * (j & 1)) + i) * D + 8 * (grp + hi4 + 8 * (j >> 1))) * 2);
  };
  auto vfix = [&]() {
#pragma unroll
    for (int q2 = 0; q2 < VB / 2; ++q2)
#pragma unroll
      for (int i = 0; i < 4; ++i) pair_fix(vreg[2 * q2][i], vreg[2 * q2 + 1][i], lo);
  };

  // Scores of one tile, masked past L, and the per-head tile maximum.
  auto scores = [&](int t, f32x4 (&s)[4]) -> float {
    const int key0 = key_begin + t * kTile;
    kfix();
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 zero = {};
      s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kreg[mb][0]), qf[0], zero, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < KS; ++ks)
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kreg[mb][ks]), qf[ks], s[mb], 0, 0, 0);
    }
    if (key0 + kTile > L) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * mb + 4 * grp + r >= L) s[mb][r] = -INFINITY;
    }
    float x = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) x = fmaxf(x, s[mb][r]);
    return max_over_row_groups(x);
  };

  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[db][r] = 0.f;
  float m_run = -INFINITY;  // running max over kept tiles: the skip test's reference
  float m_ref = -INFINITY;  // reference max of the exponentials accumulated so far
  float lsum = 0.f;

  // The decision of tile t+1 is taken while tile t's V is still in flight:
  // scores run one tile ahead of the exp/PV work.
  // Skipped tiles of this lane's head, bit t for tile t of the split (a split
  // holds at most 64 tiles); written to the mask after the loop.
  uint64_t skipped = 0;
  auto decide = [&](float tmax, int t, bool& keep) -> bool {
    keep = !(tmax < m_run - tau_raw);
    if (keep) m_run = fmaxf(m_run, tmax);
    else skipped |= 1ull << t;
    return __ballot(keep && head_ok) != 0ull;
  };

  kload(0);
  f32x4 s_cur[4];
  float t_cur = scores(0, s_cur);
  bool keep_cur;
  bool any_cur = decide(t_cur, 0, keep_cur);
  // K of the next tile is always issued before V of the current one (here and
  // in the loop), and the scheduler may not swap them: the loop's wait for K
  // then leaves the 16 V loads behind it in flight.
  kload(1);
  __builtin_amdgcn_sched_barrier(0);
  vload(0, any_cur);

  for (int t = 0; t < ntile; ++t) {
    f32x4 s_nx[4];
    float t_nx = -INFINITY;
    bool keep_nx = false, any_nx = false;
    if (t + 1 < ntile) {
      t_nx = scores(t + 1, s_nx);
      any_nx = decide(t_nx, t + 1, keep_nx);
    }
    kload(t + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (any_cur) {
      // ---- V tile t -> V^T in this wave's LDS region ----
      vfix();
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const int dc = grp + 4 * j;
        const int pos = dec_vt_pos(4 * hl);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<u32x2*>(vs_ + (dc * 8 + e) * kDecodeVStride + pos * 2) =
              column_of_4x8(vreg[j], e);
      }
    }
    vload(t + 1, any_nx);
    if (any_cur) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();

      // ---- online softmax for the heads that keep tile t ----
      const float mn = keep_cur ? fmaxf(m_ref, t_cur) : m_ref;
      if (mn > m_ref) {
        float alpha;
        if constexpr (SAS == 0)
          alpha = exp2_fast((m_ref - mn) * c);
        else
          alpha = sas_exp<SAS>((mn - m_ref) * (c * kLn2));
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[db][r] *= alpha;
        m_ref = mn;
      }
      const float nmc = -m_ref * c;
      bf16x8 pf[2];
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 w;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int mb = 2 * ks + (i2 >> 1);
          const int r0 = 2 * (i2 & 1);
          float p0, p1;
          if constexpr (SAS == 0) {
            p0 = exp2_fast(__builtin_fmaf(s_cur[mb][r0], c, nmc));
            p1 = exp2_fast(__builtin_fmaf(s_cur[mb][r0 + 1], c, nmc));
          } else {
            // x = (m_ref - s) c ln 2, logits below the running maximum; the
            // difference first, so that x >= 0 exactly (a fused form can
            // round the maximum's own x below 0, across SAS's step at 0)
            const float cn = c * kLn2;
            p0 = sas_exp<SAS>((m_ref - s_cur[mb][r0]) * cn);
            p1 = sas_exp<SAS>((m_ref - s_cur[mb][r0 + 1]) * cn);
          }
          if (!keep_cur) { p0 = 0.f; p1 = 0.f; }
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
    for (int mb = 0; mb < 4; ++mb) s_cur[mb] = s_nx[mb];
    t_cur = t_nx;
    keep_cur = keep_nx;
    any_cur = any_nx;
  }

  if (mask != nullptr && lane < 16 && head_ok) {  // grp 0: head slot hl = lane
    uint8_t* mrow = mask + bh * ntile_all + key_begin / kTile;
    for (int t = 0; t < ntile; ++t) mrow[t] = (uint8_t)((skipped >> t) & 1u);
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
    if (grp == 0) ws_lse[bh * nsplit + sp] = (m_ref * c + __log2f(ltot)) * kLn2;
  }
}

// One wave per (sequence, query head): the partials of all splits are merged
// with weights exp(lse_s - max lse). A wave reads 64 / (D / 4) splits at a
// time, one 16-byte piece of a partial row per lane, eight such rounds in
// flight before the first use.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    float* __restrict__ o, float* __restrict__ lse, int nbh, int nsplit) {
  constexpr int CL = D / 4;    // lanes per partial row
  constexpr int SW = 64 / CL;  // splits per round
  constexpr int U = 8;         // rounds per batch of loads
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= nbh) return;
  const int c4 = lane % CL;
  const int sl = lane / CL;
  const float* ls = ws_lse + (size_t)bh * nsplit;
  const float* os = ws_o + (size_t)bh * nsplit * D + 4 * c4;
  float big = -INFINITY;
  for (int s = lane; s < nsplit; s += 64) big = fmaxf(big, ls[s]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) big = fmaxf(big, __shfl_xor(big, m));
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s0 = sl; s0 < nsplit; s0 += SW * U) {
    f32x4 x[U];
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + SW * u;
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      l[u] = -INFINITY;
      if (s < nsplit) {
        x[u] = *reinterpret_cast<const f32x4*>(os + (size_t)s * D);
        l[u] = ls[s];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = expf(l[u] - big);  // 0 for a split past the end
      wsum += w;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(w, x[u][i], acc[i]);
    }
  }
#pragma unroll
  for (int m = CL; m < 64; m <<= 1) {
    wsum += __shfl_xor(wsum, m);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], m);
  }
  const float inv = 1.f / wsum;
  if (sl == 0) {
    f32x4 val;
#pragma unroll
    for (int i = 0; i < 4; ++i) val[i] = acc[i] * inv;
    *reinterpret_cast<f32x4*>(o + (size_t)bh * D + 4 * c4) = val;
    if (lane == 0) lse[bh] = big + logf(wsum);
  }
}

template <int D>
static int launch_d(const DecodeArgs& a) {
  // one wave per (sequence, KV head, slice of up to 16 query heads, split)
  const int nhs = (a.Hq / a.Hkv + 15) / 16;
  const long long nwork = (long long)a.B * a.Hkv * nhs * a.nsplit;
  const long long nbh = (long long)a.B * a.Hq;
  if (nwork > 0x7fffffffLL || nbh > 0x7fffffffLL) return -1;
  const unsigned g1 = (unsigned)((nwork + 3) / 4);
  const unsigned g2 = (unsigned)((nbh + 3) / 4);
  auto kern = a.sas == 2 ? decode_split_kernel<D, 2>
              : a.sas == 3 ? decode_split_kernel<D, 3> : decode_split_kernel<D, 0>;
  hipLaunchKernelGGL(kern, dim3(g1), dim3(256), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     a.ws_o, a.ws_lse, a.mask, a.Hq, a.Hkv, a.L, a.cap, nhs, a.nsplit, a.tau_raw,
                     a.c, (int)nwork);
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(g2), dim3(256), 0, (hipStream_t)a.stream,
                     a.ws_o, a.ws_lse, a.o, a.lse, (int)nbh, a.nsplit);
  return 0;
}

int launch_decode(const DecodeArgs& a) {
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

// Device scratch for callers that cannot allocate (attn_decode_noalloc):
// the per-split partials live in this file-scope array instead of a
// caller's workspace. Each GPU the library runs on holds its own copy for
// the life of the process. In host code `scratch` is only a stand-in for
// the symbol; its device address comes from hipGetSymbolAddress, taken once
// per device and kept below.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

int decode_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with `dev` current: the address of this device's copy of the array
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -2;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return 0;
}

int launch_decode_merge(const float* ws_o, const float* ws_lse, float* o, float* lse, int nbh,
                        int d, int nsplit, void* stream) {
  const unsigned g = (unsigned)((nbh + 3) / 4);
  if (d == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3(g), dim3(256), 0, (hipStream_t)stream,
                       ws_o, ws_lse, o, lse, nbh, nsplit);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3(g), dim3(256), 0, (hipStream_t)stream,
                       ws_o, ws_lse, o, lse, nbh, nsplit);
  return 0;
}

}  // namespace skipattn
