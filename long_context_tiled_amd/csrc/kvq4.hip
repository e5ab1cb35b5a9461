// 4-bit asymmetric KV cache: the stored format and the split-K decode that
// reads it directly (the quantisers that write it are in kvq_quant.hip).
//
// Method: the TurboAttention talk page ("Technical Deep Dive" and the
// pre-fill / decoding workflow) stores and moves the KV cache as low-bit
// asymmetric integers with a floating zero point per block, and turns them
// back into numbers inside the attention kernel, next to the products. The
// 4-bit width is the one the talk calls near-lossless. Decoding runs the
// Skip-Softmax rule (TensorRT-LLM Skip Softmax summary page, "Key Points",
// "Detailed Analysis") per query head over 64-key tiles, each 4096-key split
// with its own running maximum, exactly as the bf16 decode does.
//
// Format (readings where the pages are silent):
//   K block = one key row of d values; V block = one channel of one 64-key
//   tile. Each block runs along the contraction index of the product that
//   consumes it (d for q.K, keys for P.V), so its scale s and zero z factor
//   out of the matrix product: q.k^ = s (q.c) + z sum(q), and
//   sum_j p_j v^_jc = s_c (sum_j p_j c_jc) + z_c sum_j p_j.
//   z = block minimum; s = (max - z) / 15 in fp32, rounded up to bf16;
//   code = clamp(rint((x - z) / s), 0, 15) in fp32 (0 if s == 0).
//   A 32-bit word holds 8 consecutive elements, even ones in nibbles 0-3, odd
//   ones in nibbles 4-7. Parameter word: bf16 s (low half), bf16 z (high).
//   kq [B,Hkv,L,d/2] u8, kp [B,Hkv,L] u32, vq [B,Hkv,T,d,32] u8 (64 keys of a
//   channel per tile, keys past L code 0), vp [B,Hkv,T,d] u32, T = ceil(L/64).
//
// Decode split kernel: one wave per (sequence, KV head, split), no LDS
// memory (only ds_bpermute lane exchanges).
//   q.K on v_mfma_f32_16x16x32_bf16: q exact in bf16, each code c expanded to
//   the exact bf16 value 128 + c (bits 0x4300 | c, one and-or per pair of
//   codes), the MFMA accumulator started at -128 sum(q) so that it returns
//   q.c, and q.k^ = s (q.c) + z sum(q), with sum(q) from the same MFMA on a
//   row of ones.
//   P.V on v_mfma_f32_16x16x32_f16: codes expanded by masks alone to the exact
//   fp16 values 1024 + c (word positions 0, 1, 4, 5) and 1024 + 16 c
//   (positions 2, 3, 6, 7), and P' = 16 P on the keys of the first kind
//   (exponent + 4), P on the others, rounded to fp16. Then
//   P'.(expanded) = 16 P.c + 1024 sum(P'); with the accumulator started at
//   -1024 sum(P'), sum_j p_j v^_jc = (s_c / 16) (16 P.c) + z_c sum(P). sum(P)
//   and sum(P') come from MFMAs over the same fp16 P' (B = per-position
//   weights 1/16 and 1, then ones), so the offset cancels up to fp32 rounding
//   and sum(P) is also the row sum l. P is that product's A operand and the
//   codes its B operand, so O comes out head-major and each lane needs the
//   parameter of one channel per 16-channel block.
//   Key order inside a tile: S^T row 4 grp + r of block mb holds key
//   16 grp + 4 mb + r, so lane (head, grp) owns keys 16 grp .. 16 grp + 15 and
//   its P fragment for PV k-step ks is keys 16 grp + 8 ks .. + 7, which is
//   word 2 grp + ks of every V code row. The K fragment row m of block mb is
//   then key 16 (m >> 2) + 4 mb + (m & 3), and lane group grp reads d range
//   [grp d/4, (grp + 1) d/4) of it, k-step ks taking word ks of that range.
//   Every load instruction reads whole 128-byte lines of codes (K: 4 runs of
//   4 rows; V: 16 rows of 32 bytes) with the non-temporal policy; the small
//   parameter words use the default policy.
#include "kvq_common.hpp"
#include "lane_max.hpp"
#include "sas.hpp"
#include "launch.hpp"

namespace skipattn {

namespace {

using namespace kvq;

// ------------------------------------------------------------ decode kernel

// The constants of the expand_word functions, held in registers: gfx9 VOP3 encodings
// take no literal, so with the mask in an SGPR and the magic in a VGPR the
// compiler can fuse each mask-and-or into one v_and_or_b32 (and it still
// sees every register it writes, for the MFMA read hazards).
struct ExpandConsts {
  uint32_t mask;     // 0x000f000f
  uint32_t mask4;    // 0x00f000f0
  uint32_t bmagic;   // 0x43004300: bf16 128 in both halves
  uint32_t hmagic;   // 0x64006400: fp16 1024 in both halves
};
__device__ __forceinline__ ExpandConsts expand_consts() {
  ExpandConsts k;
  asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(k.mask));
  asm volatile("s_mov_b32 %0, 0x00f000f0" : "=s"(k.mask4));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.bmagic));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.hmagic));
  return k;
}

// One storage word -> its 8 codes as bf16 values 128 + c, element order:
// nibble n of each 16-bit half, moved to bits 0..3 and or-ed into 0x4300.
// (bf16 has 7 mantissa bits, so a nibble cannot stay at bits 4..7.)
__device__ __forceinline__ bf16x8 expand_word_bf16(uint32_t w, const ExpandConsts& k) {
  u32x4 r;
  r[0] = (w & k.mask) | k.bmagic;
  r[1] = ((w >> 4) & k.mask) | k.bmagic;
  r[2] = ((w >> 8) & k.mask) | k.bmagic;
  r[3] = ((w >> 12) & k.mask) | k.bmagic;
  return __builtin_bit_cast(bf16x8, r);
}

// One storage word -> its 8 codes as exact fp16 values, element order, by
// masks alone (one shift, four and-ors): elements 0, 1, 4, 5 (nibbles 0 and
// 2 of each 16-bit half) become 1024 + c, elements 2, 3, 6, 7 (nibbles 1 and
// 3) become 1024 + 16 c: fp16 1024 (0x6400) has 10 mantissa bits and a unit
// in the last place of 1, so mantissa bits 4..7 add 16 c. The other operand
// carries the factor 16 on the first kind instead (see the decode kernel).
__device__ __forceinline__ f16x8 expand_word_f16(uint32_t w, const ExpandConsts& k) {
  const uint32_t w8 = w >> 8;
  u32x4 r;
  r[0] = (w & k.mask) | k.hmagic;
  r[1] = (w & k.mask4) | k.hmagic;
  r[2] = (w8 & k.mask) | k.hmagic;
  r[3] = (w8 & k.mask4) | k.hmagic;
  return __builtin_bit_cast(f16x8, r);
}



// SAS = 0: exact exponentials; 2 or 3: the SAS exponential of that degree
// for every exponential of the split's online softmax.
template <int D, int SAS>
__global__ __launch_bounds__(256, 2) void decode_q4_split_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kq,
    const uint32_t* __restrict__ kp, const uint8_t* __restrict__ vq,
    const uint32_t* __restrict__ vp, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    uint8_t* __restrict__ mask, int Hq, int Hkv, int L, int cap, int nhs, int nsplit, float tau_raw, float c,
    int nwork, const KvHeadMap hm) {
  constexpr int KS = D / 32;  // QK k-steps; words per lane per K row
  constexpr int DB = D / 16;  // 16-channel blocks of O^T and of V code rows
  constexpr int RB = D / 2;   // bytes of codes per K row
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
      (void*)(vq + head * Tc * D * 32), (short)0, T * D * 32, kCfg);
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
  // [grp D/4, (grp + 1) D/4), k-step ks its elements 8 ks .. 8 ks + 7.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (head_ok) x = ldg16(q + bh * D + grp * (D / 4) + 8 * ks);
    qf[ks] = as_bf16x8(x);
  }
  const ExpandConsts xk = expand_consts();
  // sum_d q_d per head, accumulated by the MFMA itself (A = ones); the score
  // MFMAs start from -128 sum(q), so they return q.c directly
  float qsum, nqc;
  {
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), qf[ks], a, 0, 0, 0);
    qsum = a[0];
    nqc = -128.f * qsum;
  }
  // fp16 weights for sums over P' (P' = 16 P on positions 0, 1, 4, 5 of each
  // key word, P elsewhere): sum(P) with 1/16 and 1, -1024 sum(P') with -1024.
  const u32x4 wp = {0x2c002c00u, 0x3c003c00u, 0x2c002c00u, 0x3c003c00u};
  const u32x4 wneg = {0xe400e400u, 0xe400e400u, 0xe400e400u, 0xe400e400u};

  // Per-tile registers: K codes (block mb: KS words of row 16 (hl >> 2) +
  // 4 mb + (hl & 3)), K parameters (keys 16 grp + 4 j .. + 3), V codes and
  // the V parameter of channel 16 db + hl. V codes come as one 16-byte load
  // per pair of blocks (2 dp, 2 dp + 1): lane (hl, grp) reads half grp >> 1
  // of channel row 32 dp + 16 (grp & 1) + hl (the pair's 32 rows, 1 KB, in
  // one instruction); swapping rows between lane groups 2i and 2i + 1
  // (v_permlane16_swap) then leaves every lane words 2 grp, 2 grp + 1 of
  // both rows 32 dp + hl and 32 dp + 16 + hl, the B fragments of the pair.
  // V has two register sets, so the V of tile t + 1 is in flight while the
  // PV of tile t waits for its own.
  struct KSet {
    uint32_t c[4][KS];
    u32x4 p[4];
  };
  struct VSet {
    u32x4 c[DB / 2];
    uint32_t p[DB];
  };
  KSet ka, kb;  // K of even tiles in ka, of odd tiles in kb
  VSet va, vb;  // V of even tiles in va, of odd tiles in vb
  const int krow = 16 * (hl >> 2) + (hl & 3);
  auto kload = [&](KSet& ks_, int t) {
    const uint32_t tb = t < ntile ? (uint32_t)(key_begin + t * kTile) : 0u;
    const uint32_t no = t < ntile ? 0u : kNoRead;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint32_t off = no + (tb + krow + 4 * mb) * RB + grp * (RB / 4);
      if constexpr (KS == 4) {
        const u32x4 x = ld4<kNT>(krs, off);
#pragma unroll
        for (int w = 0; w < 4; ++w) ks_.c[mb][w] = x[w];
      } else {
        const u32x2 x = ld2<kNT>(krs, off);
#pragma unroll
        for (int w = 0; w < 2; ++w) ks_.c[mb][w] = x[w];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ks_.p[j] = ld4<kRT>(kprs, no + (tb + 16 * grp + 4 * j) * 4);
  };
  // the lane's byte in a tile's V code rows and parameter words; the
  // channel blocks follow at constant offsets (the loads' immediate field)
  const uint32_t vcl = (16 * (grp & 1) + hl) * 32 + 16 * (grp >> 1);
  const uint32_t vpl = 4 * hl;
  auto vload = [&](VSet& vs, int t, bool want) {
    const bool rd = want && t < ntile;
    const uint32_t tile = rd ? (uint32_t)(tile_begin + t) : 0u;
    const uint32_t no = rd ? 0u : kNoRead;
    const uint32_t cb = no + tile * (D * 32) + vcl;
    const uint32_t pb = no + tile * (D * 4) + vpl;
#pragma unroll
    for (int dp = 0; dp < DB / 2; ++dp) vs.c[dp] = ld4<kNT>(vrs, cb + 1024 * dp);
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
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(expand_word_bf16(ks_.c[mb][ks], xk), qf[ks], a,
                                                    0, 0, 0);
      // q.k^ = s (q.c) + z sum(q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t p = ks_.p[mb][r];
        s[mb][r] = __builtin_fmaf(param_s(p), a[r], param_z(p) * qsum);
      }
    }
    if (key0 + kTile > L) {
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

  // O accumulator: acc[db][r] = O[head 4 grp + r][channel 16 db + hl]
  // (P is the A operand of the PV product, the V codes the B operand), and
  // the row sum of that head in lr[r]: the sum of the same fp16 P the
  // product multiplies, so O is an exact weighted mean of the dequantised V
  // (fp16 rounding moves the LSE by at most 2^-12 relative in l). The running
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

  // K runs two tiles ahead of the scores and V one tile ahead of the PV; in
  // every step the V of tile t + 1 and the K of tile t + 3 go out before the
  // PV of tile t waits for its V, and every step issues the same loads
  // (kNoRead for the unwanted ones), so the compiler's wait counts keep the
  // later loads in flight.
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

  // One tile: scores and decision of tile t + 1 (K in kn, which then takes
  // tile t + 3, V into vn), exp/PV of tile t (V in vc). A step past the last
  // tile issues only loads that read nothing.
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
      // P' = 16 P on the keys whose V codes expand to 1024 + c (positions
      // 0, 1, 4, 5 of each key word: exponent + 4), P on the others; a
      // skipped head's exponentials are exp2(-inf) = 0
      const float nmc = keep_cur ? -m_ref * c : -INFINITY;
      const float nmc4 = nmc + 4.f;
      f16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if constexpr (SAS == 0)
            pf[ks][e] = (_Float16)exp2_fast(
                __builtin_fmaf(s_cur[2 * ks + (e >> 2)][e & 3], c, (e & 2) ? nmc : nmc4));
          else  // x from the difference, so x >= 0 exactly
            pf[ks][e] = keep_cur ? (_Float16)sas_exp_scaled<SAS>(
                                       (m_ref - s_cur[2 * ks + (e >> 2)][e & 3]) * (c * kLn2),
                                       (e & 2) ? 0.f : 4.f)
                                 : (_Float16)0.f;
      // sum_j p_j (pt) and -1024 sum_j p'_j (u0) of head 4 grp + r, from
      // MFMAs over the same fp16 P' (B = per-position weights, then -1024)
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
      // P'.(expanded codes) = 16 P.c + 1024 sum(P'), so with the MFMA
      // accumulator started at -1024 sum(P'):
      // O += (s_c / 16) (16 P.c) + z_c sum_j p_j
#pragma unroll
      for (int dp = 0; dp < DB / 2; ++dp) {
        // odd lane groups' words 0, 1 <-> even lane groups' words 2, 3
        const u32x2 s0 = __builtin_amdgcn_permlane16_swap(vc.c[dp][0], vc.c[dp][2], false, false);
        const u32x2 s1 = __builtin_amdgcn_permlane16_swap(vc.c[dp][1], vc.c[dp][3], false, false);
        const uint32_t w[2][2] = {{s0[0], s1[0]}, {s0[1], s1[1]}};  // [block of the pair][ks]
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int db = 2 * dp + h;
          f32x4 u = u0;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            u = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ks], expand_word_f16(w[h][ks], xk), u, 0,
                                                       0, 0);
          const float sc16 = 0.0625f * param_s(vc.p[db]);
          const float zc = param_z(vc.p[db]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[db][r] = __builtin_fmaf(sc16, u[r], __builtin_fmaf(zc, pt[r], acc[db][r]));
        }
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

template <int D>
int launch_dq_d(const DecodeQ4Args& a) {
  // one wave per (sequence, KV head, slice of up to 16 query heads, split)
  const int nhs = (a.Hq / a.Hkv + 15) / 16;
  const long long nwork = (long long)a.B * a.Hkv * nhs * a.nsplit;
  if (nwork > 0x7fffffffLL) return -1;
  const unsigned g1 = (unsigned)((nwork + 3) / 4);
  auto kern = a.sas == 2 ? decode_q4_split_kernel<D, 2>
              : a.sas == 3 ? decode_q4_split_kernel<D, 3> : decode_q4_split_kernel<D, 0>;
  hipLaunchKernelGGL(kern, dim3(g1), dim3(256), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, a.kq, a.kp, a.vq, a.vp, a.ws_o, a.ws_lse, a.mask, a.Hq,
                     a.Hkv, a.L, a.cap, nhs, a.nsplit, a.tau_raw, a.c, (int)nwork, a.map);
  if (!a.merge) return 0;
  return launch_decode_merge(a.ws_o, a.ws_lse, a.o, a.lse, a.B * a.Hq, a.d, a.nsplit, a.stream);
}

}  // namespace

int launch_decode_q4(const DecodeQ4Args& a) {
  return a.d == 128 ? launch_dq_d<128>(a) : launch_dq_d<64>(a);
}

}  // namespace skipattn
