// 2-bit asymmetric KV cache: the stored format and the split-K decode that
// reads it directly (the quantisers that write it are in kvq_quant.hip).
//
// Method: the TurboAttention talk page ("Technical Deep Dive", the pre-fill /
// decoding workflow and the trade-offs it lists) stores the KV cache as
// low-bit asymmetric integers with a floating zero point per block, with a
// near-lossless 4-bit and a lossy, faster 2-bit option; this file is the
// 2-bit option (kvq4.hip the 4-bit one). Decoding runs the Skip-Softmax rule
// (TensorRT-LLM Skip Softmax summary page, "Key Points", "Detailed Analysis")
// per query head over 64-key tiles, each 4096-key split with its own running
// maximum, exactly as the other decodes do.
//
// Format (readings where the pages are silent): blocks as for 4-bit (a K
// block is one key row, a V block one channel of one 64-key tile); z = block
// minimum, s = (max - z) / 3 in fp32 rounded up to bf16, code =
// clamp(rint((x - z) / s), 0, 3) in fp32. A 32-bit word holds 16 consecutive
// elements: the even ones in the 2-bit fields of bits 0-15, the odd ones in
// those of bits 16-31. kq [B,Hkv,L,d/4] u8, kp [B,Hkv,L] u32, vq
// [B,Hkv,T,d,16] u8 (64 keys of a channel per tile, keys past L code 0),
// vp [B,Hkv,T,d] u32, T = ceil(L/64).
//
// Decode split kernel: one wave per (sequence, KV head, split), the layout
// of the 4-bit decode (P the A operand of the PV product, O head-major, two
// register sets per operand, no LDS memory):
//   q.K on v_mfma_f32_16x16x32_bf16: each code expanded by a mask and an
//   or into 0x4300 to the exact bf16 value 128 + F c, F = 1, 4 or 16 by the
//   element's place in its word (three shifted copies of a word hold all its
//   fields at bits 0..5 of each half); q enters divided by F (exact), the
//   accumulator starts at -128 sum(q / F), so q.k^ = s (q.c) + z sum(q).
//   P.V on v_mfma_f32_16x16x32_f16: codes expanded by masks alone to the
//   exact fp16 values 1024 + 4^f c, f the field's place in its byte (fp16
//   1024 has 10 mantissa bits, so 64 c fits), and the factor moved to P:
//   P' = (64 / 4^f) P (exponent input + 6 - 2f), rounded to fp16 (<= 64).
//   Then P'.(expanded) = 64 P.c + 1024 sum(P'); with the accumulator started
//   at -1024 sum(P'), sum_j p_j v^_jc = (s_c / 64) (64 P.c) + z_c sum(P),
//   where sum(P) (also the row sum) and -1024 sum(P') come from MFMAs over
//   the same fp16 P'.
//   Key order inside a tile as for 4-bit: lane (head, grp) owns keys
//   16 grp .. 16 grp + 15, which are word grp of every V code row (its two
//   halves the two PV k-steps), and its K rows are 16 (hl >> 2) + 4 mb +
//   (hl & 3) with lane group grp reading the d range [grp d/4, (grp+1) d/4),
//   word ks / 2, half ks % 2 for k-step ks. Every code load covers whole
//   128-byte lines with the non-temporal policy.
#include "kvq_common.hpp"
#include "lane_max.hpp"
#include "sas.hpp"
#include "launch.hpp"

namespace skipattn {

namespace {

using namespace kvq;

// ------------------------------------------------------------ decode kernel
// The constants of the code expansions, in registers so that each
// shift-free mask-and-or is one v_and_or_b32 (gfx9 VOP3 takes no literal):
// the four 2-bit field masks of both 16-bit halves in SGPRs, the bf16 and
// fp16 magics in VGPRs.
struct Expand2Consts {
  uint32_t m[4];    // 0x00030003 << 2 f
  uint32_t bmagic;  // 0x43004300: bf16 128 in both halves
  uint32_t hmagic;  // 0x64006400: fp16 1024 in both halves
};
__device__ __forceinline__ Expand2Consts expand2_consts() {
  Expand2Consts k;
  asm volatile("s_mov_b32 %0, 0x00030003" : "=s"(k.m[0]));
  asm volatile("s_mov_b32 %0, 0x000c000c" : "=s"(k.m[1]));
  asm volatile("s_mov_b32 %0, 0x00300030" : "=s"(k.m[2]));
  asm volatile("s_mov_b32 %0, 0x00c000c0" : "=s"(k.m[3]));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.bmagic));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.hmagic));
  return k;
}

// Half h of a storage word (elements 8 h .. 8 h + 7) -> bf16 values
// 128 + F c by masks alone: element pair p (elements 2 p, 2 p + 1, field p of
// each 16-bit half) is read from w, w >> 6 or w >> 12 with its field left at
// bit 0, 2 or 4 (bf16 128 has 7 mantissa bits), so F = kScaleK[p]. The q
// fragment is divided by the same F (a power of two: exact in bf16).
constexpr int kScaleK[8] = {1, 4, 16, 1, 4, 16, 1, 4};
__device__ __forceinline__ bf16x8 expand2_bf16(uint32_t w, int h, const Expand2Consts& k) {
  const uint32_t x6 = w >> 6;
  u32x4 r;
  if (h == 0) {
    r[0] = (w & k.m[0]) | k.bmagic;
    r[1] = (w & k.m[1]) | k.bmagic;
    r[2] = (w & k.m[2]) | k.bmagic;
    r[3] = (x6 & k.m[0]) | k.bmagic;
  } else {
    const uint32_t x12 = w >> 12;
    r[0] = (x6 & k.m[1]) | k.bmagic;
    r[1] = (x6 & k.m[2]) | k.bmagic;
    r[2] = (x12 & k.m[0]) | k.bmagic;
    r[3] = (x12 & k.m[1]) | k.bmagic;
  }
  return __builtin_bit_cast(bf16x8, r);
}

// bf16 pair word x with both halves divided by f (1, 4 or 16): exact.
__device__ __forceinline__ uint32_t bf16x2_div(uint32_t x, int f) {
  const float inv = 1.f / (float)f;
  const uint32_t lo = __builtin_bit_cast(uint32_t, bf16_to_f32(x & 0xffffu) * inv) >> 16;
  const uint32_t hi = __builtin_bit_cast(uint32_t, bf16_to_f32(x >> 16) * inv) & 0xffff0000u;
  return lo | hi;
}

// Half h of a storage word -> fp16 values 1024 + 4^f c (field f in place).
__device__ __forceinline__ f16x8 expand2_f16(uint32_t w, int h, const Expand2Consts& k) {
  const uint32_t x = h ? (w >> 8) : w;
  u32x4 r;
#pragma unroll
  for (int f = 0; f < 4; ++f) r[f] = (x & k.m[f]) | k.hmagic;
  return __builtin_bit_cast(f16x8, r);
}

// SAS = 0: exact exponentials; 2 or 3: the SAS exponential of that degree
// for every exponential of the split's online softmax.
template <int D, int SAS>
__global__ __launch_bounds__(256, 2) void decode_q2_split_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kq,
    const uint32_t* __restrict__ kp, const uint8_t* __restrict__ vq,
    const uint32_t* __restrict__ vp, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    uint8_t* __restrict__ mask, int Hq, int Hkv, int L, int cap, int nhs, int nsplit, float tau_raw, float c,
    int nwork, const KvHeadMap hm) {
  constexpr int KS = D / 32;  // QK k-steps
  constexpr int KW = D / 64;  // code words per lane per K row
  constexpr int DB = D / 16;  // 16-channel blocks of O and of V code rows
  constexpr int RB = D / 4;   // bytes of codes per K row
  static_assert(kSplit / kTile <= 64, "the per-lane skip bits hold one split");

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
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int T = (L + kTile - 1) / kTile;
  const int Tc = (cap + kTile - 1) / kTile;  // tiles the arrays are sized for

  const size_t head = (size_t)(b * Hkv + g);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kq + head * cap * RB), (short)0, L * RB, kCfg);
  const __amdgpu_buffer_rsrc_t kprs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kp + head * cap), (short)0, L * 4, kCfg);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vq + head * Tc * D * 16), (short)0, T * D * 16, kCfg);
  const __amdgpu_buffer_rsrc_t vprs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vp + head * Tc * D), (short)0, T * D * 4, kCfg);

  const int key_begin = sp * kSplit;
  const int key_end = min(L, key_begin + kSplit);
  const int ntile = (key_end - key_begin + kTile - 1) / kTile;
  const int tile_begin = key_begin / kTile;
  const bool head_ok = hoff + hl < G;
  // rows of q, the partials and the mask: those of the full set of heads
  const int Hqo = hm.n ? hm.n_in * G : Hq;
  const size_t bh = (size_t)b * Hqo + full_head(g, hm) * G + hoff + hl;

  // q^T fragments (B operand, n = head): lane group grp holds d range
  // [grp D/4, (grp + 1) D/4), k-step ks its elements 8 ks .. 8 ks + 7; qf
  // as given, qs divided by the expansion's factors (element pair p of word
  // half ks & 1 by kScaleK[4 (ks & 1) + p]).
  bf16x8 qf[KS], qs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (head_ok) x = ldg16(q + bh * D + grp * (D / 4) + 8 * ks);
    qf[ks] = as_bf16x8(x);
#pragma unroll
    for (int p = 0; p < 4; ++p) x[p] = bf16x2_div(x[p], kScaleK[4 * (ks & 1) + p]);
    qs[ks] = as_bf16x8(x);
  }
  const Expand2Consts xk = expand2_consts();
  // sum_d q_d and sum_d q_d / F_d per head from the MFMA itself (A = ones);
  // the score MFMAs start from -128 sum(q / F), so they return q.c directly
  float qsum, nqc;
  {
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, as = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), qf[ks], a, 0, 0, 0);
      as = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), qs[ks], as, 0, 0, 0);
    }
    qsum = a[0];
    nqc = -128.f * as[0];
  }
  // fp16 weights for sums over P' (P' = (64 / 4^f) P for the keys of field
  // f): sum(P) with 4^f / 64 = 1/64, 1/16, 1/4, 1; -1024 sum(P') with -1024.
  const u32x4 wp = {0x24002400u, 0x2c002c00u, 0x34003400u, 0x3c003c00u};
  const u32x4 wneg = {0xe400e400u, 0xe400e400u, 0xe400e400u, 0xe400e400u};

  // Per-tile registers: K codes (block mb: KW words of row 16 (hl >> 2) +
  // 4 mb + (hl & 3)), K parameters (keys 16 grp + 4 j .. + 3), V codes (word
  // grp of channel row 16 db + hl) and the V parameter of that channel; two
  // register sets each, as in the 4-bit decode.
  struct KSet {
    uint32_t c[4][KW];
    u32x4 p[4];
  };
  struct VSet {
    uint32_t c[DB];
    uint32_t p[DB];
  };
  KSet ka, kb;
  VSet va, vb;
  const int krow = 16 * (hl >> 2) + (hl & 3);
  auto kload = [&](KSet& ks_, int t) {
    const uint32_t tb = t < ntile ? (uint32_t)(key_begin + t * kTile) : 0u;
    const uint32_t no = t < ntile ? 0u : kNoRead;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint32_t off = no + (tb + krow + 4 * mb) * RB + grp * (RB / 4);
      if constexpr (KW == 2) {
        const u32x2 x = ld2<kNT>(krs, off);
        ks_.c[mb][0] = x[0];
        ks_.c[mb][1] = x[1];
      } else {
        ks_.c[mb][0] = ld1<kNT>(krs, off);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ks_.p[j] = ld4<kRT>(kprs, no + (tb + 16 * grp + 4 * j) * 4);
  };
  // the lane's byte in a tile's V code rows and parameter words; the
  // channel blocks follow at constant offsets (the loads' immediate field)
  const uint32_t vcl = 16 * hl + 4 * grp;
  const uint32_t vpl = 4 * hl;
  auto vload = [&](VSet& vs, int t, bool want) {
    const bool rd = want && t < ntile;
    const uint32_t tile = rd ? (uint32_t)(tile_begin + t) : 0u;
    const uint32_t no = rd ? 0u : kNoRead;
    const uint32_t cb = no + tile * (D * 16) + vcl;
    const uint32_t pb = no + tile * (D * 4) + vpl;
#pragma unroll
    for (int db = 0; db < DB; ++db) vs.c[db] = ld1<kNT>(vrs, cb + 256 * db);
#pragma unroll
    for (int db = 0; db < DB; ++db) vs.p[db] = ld1<kRT>(vprs, pb + 64 * db);
  };

  // Scores of one tile (raw q.k^ units), masked past L, and the tile max.
  auto scores = [&](const KSet& ks_, int t, f32x4 (&s)[4]) -> float {
    const int key0 = key_begin + t * kTile;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x4 a = {nqc, nqc, nqc, nqc};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(expand2_bf16(ks_.c[mb][ks >> 1], ks & 1, xk),
                                                    qs[ks], a, 0, 0, 0);
      // q.k^ = s (q.c) + z sum(q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t p = ks_.p[mb][r];
        s[mb][r] = __builtin_fmaf(param_s(p), a[r], param_z(p) * qsum);
      }
    }
    if (key0 + kTile > L) {
      asm volatile("");  // keeps this a branch taken on the last tile only
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * grp + 4 * mb + r >= L) s[mb][r] = -INFINITY;
    }
    float x = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) x = fmaxf(x, s[mb][r]);
    return max_over_row_groups(x);
  };

  // O: acc[db][r] = O[head 4 grp + r][channel 16 db + hl]; lr[r] the row sum
  // of that head over the same fp16 P the product multiplies. The running
  // max and the skip state stay per head hl.
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[db][r] = 0.f;
  f32x4 lr = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max over kept tiles: the skip test's reference
  float m_ref = -INFINITY;  // reference max of the exponentials accumulated so far
  uint64_t skipped = 0;
  auto decide = [&](float tmax, int t, bool& keep) -> bool {
    keep = !(tmax < m_run - tau_raw);
    if (keep) m_run = fmaxf(m_run, tmax);
    else skipped |= 1ull << t;
    return __ballot(keep && head_ok) != 0ull;
  };
  // value of head 4 grp + r, from the lane of grp 0 that holds it per head
  const int hsrc = 16 * grp;  // byte address of lane 4 grp, for ds_bpermute
  auto of_head = [&](float x, int r) -> float {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                         hsrc + 4 * r, __builtin_bit_cast(int, x)));
  };

  // K runs two tiles ahead of the scores and V one tile ahead of the PV, with
  // the same load order and no-read loads as the 4-bit decode.
  kload(ka, 0);
  kload(kb, 1);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s_cur[4];
  float t_cur = scores(ka, 0, s_cur);
  bool keep_cur;
  bool any_cur = decide(t_cur, 0, keep_cur);
  vload(va, 0, any_cur);
  __builtin_amdgcn_sched_barrier(0);
  kload(ka, 2);
  __builtin_amdgcn_sched_barrier(0);

  auto step = [&](int t, KSet& kn, const VSet& vc, VSet& vn) {
    f32x4 s_nx[4];
    float t_nx = -INFINITY;
    bool keep_nx = false, any_nx = false;
    if (t + 1 < ntile) {
      t_nx = scores(kn, t + 1, s_nx);
      any_nx = decide(t_nx, t + 1, keep_nx);
    }
    vload(vn, t + 1, any_nx);
    __builtin_amdgcn_sched_barrier(0);
    kload(kn, t + 3);
    __builtin_amdgcn_sched_barrier(0);
    if (any_cur) {
      const float mn = keep_cur ? fmaxf(m_ref, t_cur) : m_ref;
      if (__ballot(mn > m_ref) != 0ull) {
        float alpha;
        if constexpr (SAS == 0)
          alpha = mn > m_ref ? exp2_fast((m_ref - mn) * c) : 1.f;
        else
          alpha = mn > m_ref ? sas_exp<SAS>((mn - m_ref) * (c * kLn2)) : 1.f;
        m_ref = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = of_head(alpha, r);
          lr[r] *= ar;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db][r] *= ar;
        }
      }
      // P' = (64 / 4^f) P, f = the field of the key's code (element e of a
      // k-step: f = e / 2), i.e. exponent input + 6 - 2 f; a skipped head's
      // exponentials are exp2(-inf) = 0
      const float nmc = keep_cur ? -m_ref * c : -INFINITY;
      f16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if constexpr (SAS == 0)
            pf[ks][e] = (_Float16)exp2_fast(__builtin_fmaf(
                s_cur[2 * ks + (e >> 2)][e & 3], c, nmc + (float)(6 - 2 * (e >> 1))));
          else  // x from the difference, so x >= 0 exactly
            pf[ks][e] = keep_cur ? (_Float16)sas_exp_scaled<SAS>(
                                       (m_ref - s_cur[2 * ks + (e >> 2)][e & 3]) * (c * kLn2),
                                       (float)(6 - 2 * (e >> 1)))
                                 : (_Float16)0.f;
      // sum_j p_j (pt) and -1024 sum_j p'_j (u0) of head 4 grp + r
      f32x4 pt = {0.f, 0.f, 0.f, 0.f}, u0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pt = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ks], __builtin_bit_cast(f16x8, wp), pt, 0, 0,
                                                    0);
        u0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ks], __builtin_bit_cast(f16x8, wneg), u0, 0,
                                                    0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) lr[r] += pt[r];
      // P'.(expanded codes) = 64 P.c + 1024 sum(P'); from -1024 sum(P'):
      // O += (s_c / 64) (64 P.c) + z_c sum_j p_j
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 u = u0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          u = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ks], expand2_f16(vc.c[db], ks, xk), u, 0, 0,
                                                     0);
        const float sc64 = 0.015625f * param_s(vc.p[db]);
        const float zc = param_z(vc.p[db]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[db][r] = __builtin_fmaf(sc64, u[r], __builtin_fmaf(zc, pt[r], acc[db][r]));
      }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) s_cur[mb] = s_nx[mb];
    t_cur = t_nx;
    keep_cur = keep_nx;
    any_cur = any_nx;
  };
  for (int t = 0; t < ntile; t += 2) {
    step(t, kb, va, vb);
    step(t + 1, ka, vb, va);
  }

  if (mask != nullptr && lane < 16 && head_ok) {  // grp 0: head slot hl = lane
    uint8_t* mrow = mask + bh * T + tile_begin;
    for (int t = 0; t < ntile; ++t) mrow[t] = (uint8_t)((skipped >> t) & 1u);
  }

  const size_t bh0 = (size_t)b * Hqo + full_head(g, hm) * G + hoff;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float mr = of_head(m_ref, r);
    const int h = 4 * grp + r;
    if (hoff + h < G) {
      const float ir = 1.f / lr[r];
      float* dst = ws_o + ((bh0 + h) * nsplit + sp) * D + hl;
#pragma unroll
      for (int db = 0; db < DB; ++db) dst[16 * db] = acc[db][r] * ir;
      if (hl == 0) ws_lse[(bh0 + h) * nsplit + sp] = (mr * c + __log2f(lr[r])) * kLn2;
    }
  }
}

// Two KV groups per wave (group sizes G <= 8): the 16 head columns of every
// MFMA hold the heads of groups gA = 2 pr (columns 0-7) and gB = 2 pr + 1
// (columns 8-15), so the per-head work (scores, maxima, exponentials, the O
// update) runs on useful lanes only. q.K: each MFMA's 32-long contraction
// holds 16 d of group A (k-slots 0-15, lane groups 0-1) and 16 d of group B
// (k-slots 16-31, lane groups 2-3); the q fragment of a head column is zero
// in the other group's half, so column h gets its own group's scores. Lane
// group grp reads d range [(grp & 1) D/2, +D/2) of its group's key rows.
// P.V: per k-step two MFMAs into the same accumulator, one on group A's V
// codes with P kept in columns 0-7 (head rows 0-7) and zero elsewhere, one on
// group B's with P kept in rows 8-15; the key order, the expansions, the
// parameter arithmetic and the merge are those of the kernel above.
template <int D, int SAS>
__global__ __launch_bounds__(256, 2) void decode_q2_pair_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kq,
    const uint32_t* __restrict__ kp, const uint8_t* __restrict__ vq,
    const uint32_t* __restrict__ vp, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    uint8_t* __restrict__ mask, int Hq, int Hkv, int L, int cap, int nsplit, float tau_raw,
    float c, int nwork, const KvHeadMap hm) {
  constexpr int KS = D / 16;  // q.K k-steps per 16-key block (16 d of each group)
  constexpr int KW = D / 32;  // code words per lane per K row (half a row)
  constexpr int DB = D / 16;  // 16-channel blocks of O and of V code rows
  constexpr int RB = D / 4;   // bytes of codes per K row
  static_assert(kSplit / kTile <= 64, "the per-lane skip bits hold one split");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int work = blockIdx.x * 4 + wave;
  if (work >= nwork) return;  // whole wave leaves; the kernel has no barrier
  const int npair = (Hkv + 1) / 2;
  const int sp = work % nsplit;
  const int pr = (work / nsplit) % npair;
  const int b = work / nsplit / npair;
  const int G = Hq / Hkv;
  const int gA = 2 * pr;
  const bool b_ok = gA + 1 < Hkv;   // an odd last group has no partner
  const int gB = b_ok ? gA + 1 : gA;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int gh = grp >> 1;          // group of this lane's k-slots (q.K) / head rows (O)
  const int col_g = hl >> 3;        // group of this lane's head column
  const int T = (L + kTile - 1) / kTile;
  const int Tc = (cap + kTile - 1) / kTile;

  // Buffer descriptors must be wave-uniform (a per-lane descriptor makes the
  // compiler loop over its distinct values for every load): the K codes, K
  // parameters and V parameters of both groups sit behind one descriptor
  // from group A's start over both groups' arrays (adjacent KV heads), and a
  // lane reaches its group's by a per-lane offset. Keys past L are masked in
  // the scores (their K bytes are never used) and the V codes of a tile past
  // L are zero, so the range check of one group inside the span is not needed.
  const size_t hA = (size_t)(b * Hkv + gA);
  const int ngrp = b_ok ? 2 : 1;
  // (sizes through readfirstlane: computed on the vector unit they would put
  // the descriptors in VGPRs)
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kq + hA * cap * RB), (short)0, uni(ngrp * cap * RB), kCfg);
  const __amdgpu_buffer_rsrc_t kprs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kp + hA * cap), (short)0, uni(ngrp * cap * 4), kCfg);
  const __amdgpu_buffer_rsrc_t vrsA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vq + hA * Tc * D * 16), (short)0, T * D * 16, kCfg);
  const __amdgpu_buffer_rsrc_t vrsB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vq + (hA + (b_ok ? 1 : 0)) * Tc * D * 16), (short)0, T * D * 16, kCfg);
  const __amdgpu_buffer_rsrc_t vprs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vp + hA * Tc * D), (short)0, uni(ngrp * Tc * D * 4), kCfg);
  // per-lane byte offsets of the lane's group within those spans
  const uint32_t k_off = (b_ok && gh) ? (uint32_t)(cap * RB) : 0u;     // K codes: k-slot group
  const uint32_t kp_off = (b_ok && col_g) ? (uint32_t)(cap * 4) : 0u;  // K params: column group
  const uint32_t vp_off = (b_ok && gh) ? (uint32_t)(Tc * D * 4) : 0u;  // V params: head-row group

  const int key_begin = sp * kSplit;
  const int key_end = min(L, key_begin + kSplit);
  const int ntile = (key_end - key_begin + kTile - 1) / kTile;
  const int tile_begin = key_begin / kTile;
  const int hcol = hl & 7;                          // head of the column within its group
  const bool head_ok = hcol < G && (col_g == 0 || b_ok);
  // rows of q, the partials and the mask: those of the full set of heads
  const int Hqo = hm.n ? hm.n_in * G : Hq;
  const int gAo = full_head(gA, hm), gBo = full_head(gB, hm);
  const size_t bh = (size_t)b * Hqo + (col_g ? gBo : gAo) * G + hcol;
  const bool q_on = col_g == gh && head_ok;         // this lane's q fragment is the column's

  // q^T fragments (B operand, n = head column): k-step ks holds elements
  // (grp & 1) D/2 + 8 ks .. + 7 of the column's q if its group owns the
  // lane's k-slots, else zeros; qs divided by the expansion's factors.
  bf16x8 qs[KS];
  float qsum, nqc;
  {
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, as = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (q_on) x = ldg16(q + bh * D + (grp & 1) * (D / 2) + 8 * ks);
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), as_bf16x8(x), a, 0, 0, 0);
#pragma unroll
      for (int p = 0; p < 4; ++p) x[p] = bf16x2_div(x[p], kScaleK[4 * (ks & 1) + p]);
      qs[ks] = as_bf16x8(x);
      as = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), qs[ks], as, 0, 0, 0);
    }
    qsum = a[0];
    nqc = -128.f * as[0];
  }
  const Expand2Consts xk = expand2_consts();
  const u32x4 wp = {0x24002400u, 0x2c002c00u, 0x34003400u, 0x3c003c00u};
  const u32x4 wneg = {0xe400e400u, 0xe400e400u, 0xe400e400u, 0xe400e400u};
  // P kept in head columns 0-7 (group A's MFMA) or 8-15 (group B's)
  const uint32_t keepA = col_g == 0 ? 0xffffffffu : 0u;
  const uint32_t keepB = ~keepA;

  struct KSet {
    uint32_t c[4][KW];
    u32x4 p[4];
  };
  struct VSet {
    uint32_t ca[DB], cb[DB];
    uint32_t p[DB];
  };
  // One K register set (its loads run one tile ahead of the scores: with two
  // groups per wave that keeps as many K bytes in flight as two tiles ahead
  // of a one-group wave), two V sets.
  KSet kset;
  VSet va, vb;
  const int krow = 16 * (hl >> 2) + (hl & 3);
  auto kload = [&](KSet& ks_, int t) {
    const uint32_t tb = t < ntile ? (uint32_t)(key_begin + t * kTile) : 0u;
    const uint32_t no = t < ntile ? 0u : kNoRead;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint32_t off = no + k_off + (tb + krow + 4 * mb) * RB + (grp & 1) * (RB / 2);
      if constexpr (KW == 4) {
        const u32x4 x = ld4<kNT>(krs, off);
#pragma unroll
        for (int i = 0; i < 4; ++i) ks_.c[mb][i] = x[i];
      } else {
        const u32x2 x = ld2<kNT>(krs, off);
        ks_.c[mb][0] = x[0];
        ks_.c[mb][1] = x[1];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ks_.p[j] = ld4<kRT>(kprs, no + kp_off + (tb + 16 * grp + 4 * j) * 4);
  };
  const uint32_t vcl = 16 * hl + 4 * grp;
  const uint32_t vpl = 4 * hl;
  auto vload = [&](VSet& vs, int t, bool wantA, bool wantB) {
    const bool in = t < ntile;
    const uint32_t tile = in ? (uint32_t)(tile_begin + t) : 0u;
    const uint32_t noA = in && wantA ? 0u : kNoRead;
    const uint32_t noB = in && wantB ? 0u : kNoRead;
    const uint32_t noP = in && (gh ? wantB : wantA) ? 0u : kNoRead;
    const uint32_t cb = tile * (D * 16) + vcl;
    const uint32_t pb = vp_off + tile * (D * 4) + vpl;
#pragma unroll
    for (int db = 0; db < DB; ++db) vs.ca[db] = ld1<kNT>(vrsA, noA + cb + 256 * db);
#pragma unroll
    for (int db = 0; db < DB; ++db) vs.cb[db] = ld1<kNT>(vrsB, noB + cb + 256 * db);
#pragma unroll
    for (int db = 0; db < DB; ++db) vs.p[db] = ld1<kRT>(vprs, noP + pb + 64 * db);
  };

  auto scores = [&](const KSet& ks_, int t, f32x4 (&s)[4]) -> float {
    const int key0 = key_begin + t * kTile;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x4 a = {nqc, nqc, nqc, nqc};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(expand2_bf16(ks_.c[mb][ks >> 1], ks & 1, xk),
                                                    qs[ks], a, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t p = ks_.p[mb][r];
        s[mb][r] = __builtin_fmaf(param_s(p), a[r], param_z(p) * qsum);
      }
    }
    if (key0 + kTile > L) {
      asm volatile("");
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * grp + 4 * mb + r >= L) s[mb][r] = -INFINITY;
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
  f32x4 lr = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float m_ref = -INFINITY;
  uint64_t skipped = 0;
  constexpr uint64_t kColsA = 0x00ff00ff00ff00ffull;  // lanes of head columns 0-7
  // keep flags per group: any kept head column of group A / group B
  auto decide = [&](float tmax, int t, bool& keep, bool& anyA, bool& anyB) {
    keep = !(tmax < m_run - tau_raw);
    if (keep) m_run = fmaxf(m_run, tmax);
    else skipped |= 1ull << t;
    const uint64_t k = __ballot(keep && head_ok);
    anyA = (k & kColsA) != 0ull;
    anyB = (k & ~kColsA) != 0ull;
  };
  const int hsrc = 16 * grp;
  auto of_head = [&](float x, int r) -> float {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                         hsrc + 4 * r, __builtin_bit_cast(int, x)));
  };

  kload(kset, 0);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s_cur[4];
  float t_cur = scores(kset, 0, s_cur);
  bool keep_cur, anyA_cur, anyB_cur;
  decide(t_cur, 0, keep_cur, anyA_cur, anyB_cur);
  kload(kset, 1);
  vload(va, 0, anyA_cur, anyB_cur);
  __builtin_amdgcn_sched_barrier(0);

  auto step = [&](int t, const VSet& vc, VSet& vn) {
    f32x4 s_nx[4];
    float t_nx = -INFINITY;
    bool keep_nx = false, anyA_nx = false, anyB_nx = false;
    if (t + 1 < ntile) {
      t_nx = scores(kset, t + 1, s_nx);
      decide(t_nx, t + 1, keep_nx, anyA_nx, anyB_nx);
    }
    kload(kset, t + 2);
    vload(vn, t + 1, anyA_nx, anyB_nx);
    __builtin_amdgcn_sched_barrier(0);
    if (anyA_cur || anyB_cur) {
      const float mn = keep_cur ? fmaxf(m_ref, t_cur) : m_ref;
      if (__ballot(mn > m_ref) != 0ull) {
        float alpha;
        if constexpr (SAS == 0)
          alpha = mn > m_ref ? exp2_fast((m_ref - mn) * c) : 1.f;
        else
          alpha = mn > m_ref ? sas_exp<SAS>((mn - m_ref) * (c * kLn2)) : 1.f;
        m_ref = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = of_head(alpha, r);
          lr[r] *= ar;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db][r] *= ar;
        }
      }
      const float nmc = keep_cur ? -m_ref * c : -INFINITY;
      f16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if constexpr (SAS == 0)
            pf[ks][e] = (_Float16)exp2_fast(__builtin_fmaf(
                s_cur[2 * ks + (e >> 2)][e & 3], c, nmc + (float)(6 - 2 * (e >> 1))));
          else
            pf[ks][e] = keep_cur ? (_Float16)sas_exp_scaled<SAS>(
                                       (m_ref - s_cur[2 * ks + (e >> 2)][e & 3]) * (c * kLn2),
                                       (float)(6 - 2 * (e >> 1)))
                                 : (_Float16)0.f;
      f32x4 pt = {0.f, 0.f, 0.f, 0.f}, u0 = {0.f, 0.f, 0.f, 0.f};
      f16x8 pa[2], pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pt = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ks], __builtin_bit_cast(f16x8, wp), pt, 0, 0,
                                                    0);
        u0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ks], __builtin_bit_cast(f16x8, wneg), u0, 0,
                                                    0, 0);
        const u32x4 w = __builtin_bit_cast(u32x4, pf[ks]);
        u32x4 wa, wb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wa[i] = w[i] & keepA;
          wb[i] = w[i] & keepB;
        }
        pa[ks] = __builtin_bit_cast(f16x8, wa);
        pb[ks] = __builtin_bit_cast(f16x8, wb);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) lr[r] += pt[r];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 u = u0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[ks], expand2_f16(vc.ca[db], ks, xk), u, 0,
                                                     0, 0);
          u = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb[ks], expand2_f16(vc.cb[db], ks, xk), u, 0,
                                                     0, 0);
        }
        const float sc64 = 0.015625f * param_s(vc.p[db]);
        const float zc = param_z(vc.p[db]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[db][r] = __builtin_fmaf(sc64, u[r], __builtin_fmaf(zc, pt[r], acc[db][r]));
      }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) s_cur[mb] = s_nx[mb];
    t_cur = t_nx;
    keep_cur = keep_nx;
    anyA_cur = anyA_nx;
    anyB_cur = anyB_nx;
  };
  for (int t = 0; t < ntile; t += 2) {
    step(t, va, vb);
    step(t + 1, vb, va);
  }

  if (mask != nullptr && lane < 16 && head_ok) {  // grp 0: head column hl
    uint8_t* mrow = mask + bh * T + tile_begin;
    for (int t = 0; t < ntile; ++t) mrow[t] = (uint8_t)((skipped >> t) & 1u);
  }

  // O rows: head column 4 grp + r, i.e. group grp >> 1, head 4 (grp & 1) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float mr = of_head(m_ref, r);
    const int hh = 4 * (grp & 1) + r;
    const int go = gh ? gBo : gAo;
    if (hh < G && (gh == 0 || b_ok)) {
      const size_t bhr = (size_t)b * Hqo + go * G + hh;
      const float ir = 1.f / lr[r];
      float* dst = ws_o + (bhr * nsplit + sp) * D + hl;
#pragma unroll
      for (int db = 0; db < DB; ++db) dst[16 * db] = acc[db][r] * ir;
      if (hl == 0) ws_lse[bhr * nsplit + sp] = (mr * c + __log2f(lr[r])) * kLn2;
    }
  }
}

template <int D>
int launch_dq2_d(const DecodeQ4Args& a) {
  const int G = a.Hq / a.Hkv;
  if (G <= 8) {
    // one wave per (sequence, pair of KV heads, split)
    const long long nwork = (long long)a.B * ((a.Hkv + 1) / 2) * a.nsplit;
    if (nwork > 0x7fffffffLL) return -1;
    const unsigned g1 = (unsigned)((nwork + 3) / 4);
    auto kern = a.sas == 2 ? decode_q2_pair_kernel<D, 2>
                : a.sas == 3 ? decode_q2_pair_kernel<D, 3> : decode_q2_pair_kernel<D, 0>;
    hipLaunchKernelGGL(kern, dim3(g1), dim3(256), 0, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, a.kq, a.kp, a.vq, a.vp, a.ws_o, a.ws_lse, a.mask,
                       a.Hq, a.Hkv, a.L, a.cap, a.nsplit, a.tau_raw, a.c, (int)nwork, a.map);
    if (!a.merge) return 0;
    return launch_decode_merge(a.ws_o, a.ws_lse, a.o, a.lse, a.B * a.Hq, a.d, a.nsplit, a.stream);
  }
  // one wave per (sequence, KV head, slice of up to 16 query heads, split)
  const int nhs = (a.Hq / a.Hkv + 15) / 16;
  const long long nwork = (long long)a.B * a.Hkv * nhs * a.nsplit;
  if (nwork > 0x7fffffffLL) return -1;
  const unsigned g1 = (unsigned)((nwork + 3) / 4);
  auto kern = a.sas == 2 ? decode_q2_split_kernel<D, 2>
              : a.sas == 3 ? decode_q2_split_kernel<D, 3> : decode_q2_split_kernel<D, 0>;
  hipLaunchKernelGGL(kern, dim3(g1), dim3(256), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, a.kq, a.kp, a.vq, a.vp, a.ws_o, a.ws_lse, a.mask, a.Hq,
                     a.Hkv, a.L, a.cap, nhs, a.nsplit, a.tau_raw, a.c, (int)nwork, a.map);
  if (!a.merge) return 0;
  return launch_decode_merge(a.ws_o, a.ws_lse, a.o, a.lse, a.B * a.Hq, a.d, a.nsplit, a.stream);
}

}  // namespace

int launch_decode_q2(const DecodeQ4Args& a) {
  return a.d == 128 ? launch_dq2_d<128>(a) : launch_dq2_d<64>(a);
}

}  // namespace skipattn
