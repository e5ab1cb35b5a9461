// Quantisers of the 4-bit and 2-bit KV caches: bf16 K and V -> codes and
// parameter words in the formats that kvq4.hip (4 bits) and kvq2.hip
// (2 bits) document. Blocks: a K block is one key row of d values, a V block
// one channel of one 64-key tile (TurboAttention talk page, "Technical Deep
// Dive": low-bit asymmetric integers with a floating zero point per block).
// Every element's arithmetic (block minimum and maximum, the scale rounded up
// to bf16, the code by an fp32 subtract, divide and rint) is kvq_common.hpp's.
//
// Both kernels are streams: every input byte is read once and every output
// byte written once, so HBM bounds them, with the vector arithmetic (about
// 11 instructions per value) close behind. A wave first issues all of its loads
// (8 KB of K rows, or a whole 64-key V tile), then does the arithmetic.
//   K: a lane holds two code words of a row (16 values for 4 bits, 32 for 2):
//   words w and w + W of the row for the row's W = d / (2 x values per word)
//   lanes, so each 16-byte load instruction reads W x 16 contiguous bytes of
//   every row it touches; a wave takes S slots of 64 / W consecutive rows.
//   V: one wave per tile. Lane (c, g) loads channels C c .. C c + C - 1
//   (C = 8, or 4 for 2-bit codes at d = 64) of the K_L = d / C consecutive
//   keys g K_L .. g K_L + K_L - 1, one row piece per load (each load
//   instruction reads 64 / K_L whole rows). The keys of a lane are then the
//   K_L / (values per word) whole code words of each of its channels, so
//   codes are packed in registers.
//   A block's minimum and maximum meet across its lanes by DPP operand
//   permutations and the gfx950 lane swaps; the codes use no division
//   instruction sequence (block_div below).
#include "kvq_common.hpp"
#include "launch.hpp"

namespace skipattn {

namespace {

using namespace kvq;

// Storage word of BITS-wide codes: 32 / BITS consecutive elements, the even
// ones in the fields of bits 0-15 and the odd ones in those of bits 16-31,
// lowest field first.
template <int BITS>
struct Fmt {
  static constexpr int CMAX = (1 << BITS) - 1;
  static constexpr int EPW = 32 / BITS;  // elements per word
};

// Element e of a run of bf16 values held as dwords (even elements in the
// low halves).
template <int N>
__device__ __forceinline__ float elem(const uint32_t (&w)[N], int e) {
  const uint32_t d = w[e >> 1];
  return __builtin_bit_cast(float, (e & 1) ? (d & 0xffff0000u) : (d << 16));
}

// v_min_f32 / v_max_f32 as they are: the inputs are finite bf16 values, so
// the compiler's NaN canonicalisation of each operand is not needed.
__device__ __forceinline__ float vmin(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Minimum and maximum over lane groups. Within a row of 16 lanes by DPP
// operand permutations (quad_perm, row_half_mirror, row_mirror, row_ror:8):
// each step pairs every lane with one of the other half of its group, so
// after log2 W steps every lane of a group of W holds the group's result.
// Across rows by the gfx950 lane swaps (l ^ 16, l ^ 32) on two copies. The
// s_nop covers the wait states a DPP or swap read needs after a vector
// write of its operand.
#define SKA_MINMAX_DPP(ctrl)                                                        \
  asm("s_nop 1\n\tv_min_f32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:0xf\n\t" \
      "v_max_f32_dpp %1, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf"                 \
      : "+v"(lo), "+v"(hi))
__device__ __forceinline__ void minmax_xor1(float& lo, float& hi) { SKA_MINMAX_DPP("quad_perm:[1,0,3,2]"); }
__device__ __forceinline__ void minmax_xor2(float& lo, float& hi) { SKA_MINMAX_DPP("quad_perm:[2,3,0,1]"); }
__device__ __forceinline__ void minmax_half(float& lo, float& hi) { SKA_MINMAX_DPP("row_half_mirror"); }
__device__ __forceinline__ void minmax_row(float& lo, float& hi) { SKA_MINMAX_DPP("row_mirror"); }
__device__ __forceinline__ void minmax_xor8(float& lo, float& hi) { SKA_MINMAX_DPP("row_ror:8"); }
#undef SKA_MINMAX_DPP
__device__ __forceinline__ void minmax_xor16(float& lo, float& hi) {
  float a = lo, b = lo, c = hi, d = hi;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\ts_nop 1"
      : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
  lo = vmin(a, b);
  hi = vmax(c, d);
}
__device__ __forceinline__ void minmax_xor32(float& lo, float& hi) {
  float a = lo, b = lo, c = hi, d = hi;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\ts_nop 1"
      : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
  lo = vmin(a, b);
  hi = vmax(c, d);
}
// Groups of W consecutive lanes (W = 2, 4, 8, 16).
template <int W>
__device__ __forceinline__ void minmax_lanes(float& lo, float& hi) {
  if constexpr (W >= 2) minmax_xor1(lo, hi);
  if constexpr (W >= 4) minmax_xor2(lo, hi);
  if constexpr (W >= 8) minmax_half(lo, hi);
  if constexpr (W >= 16) minmax_row(lo, hi);
}
// Lanes l, l + LG, l + 2 LG, ... (LG = 8 or 16).
template <int LG>
__device__ __forceinline__ void minmax_strided(float& lo, float& hi) {
  if constexpr (LG == 8) minmax_xor8(lo, hi);
  minmax_xor16(lo, hi);
  minmax_xor32(lo, hi);
}

// Codes of one block: code(x) = clamp(rint(fl(fl(x - z) / s)), 0, CMAX) with
// s = bf16_round_up(fl(fl(max - z) / CMAX)), bit for bit as block_scale and
// code_of compute them, without a division instruction sequence:
//   fl(a / b) = RN(q0 + e y) for q0 = RN(a y), e = a - b q0 (exact in one
//   fma) and y = RN(1 / b) (Markstein's correction step), while no step
//   leaves the normal range; an exhaustive check over every fp32 significand
//   confirms it for b = 15 and 3.
//   y = RN(1 / s) from v_rcp_f32 and one Newton step, y0 + y0 (1 - s y0),
//   exact for every bf16 significand from any start within 3 ulp (also
//   checked exhaustively); s is a bf16 value.
//   For 2^-60 <= s <= 2^60 every quotient that can round to a code >= 1 has
//   x - z >= s / 2, well inside the normal range, and max - z >= 2^-59, so
//   the steps are exact. The code is the low field of the bits of
//   RN(q + 2^23) = 2^23 + rint(q) (ties to even); no clamp is needed, as
//   0 <= q <= CMAX (1 + 2^-23) (z is the minimum, and s >= fl((max - z) /
//   CMAX)). max = z (s = 0) divides by 1, which gives code 0 as code_of does;
//   blocks with other scales outside the range take block_scale and code_of.
struct BlockDiv {
  float s;    // the block's scale (valid when fast)
  float sd;   // divisor: s, or 1 when s = 0
  float inv;  // RN(1 / sd)
  bool fast;
};
template <int CMAX>
__device__ __forceinline__ BlockDiv block_div(float lo, float hi) {
  constexpr float c = 1.0f / CMAX;  // RN(1 / CMAX)
  const float d = __fsub_rn(hi, lo);
  const float q0 = __fmul_rn(d, c);
  const float q = __fmaf_rn(__fmaf_rn(-(float)CMAX, q0, d), c, q0);
  BlockDiv b;
  b.s = bf16_round_up(q);
  b.fast = d == 0.f || (b.s >= 0x1p-60f && b.s <= 0x1p60f);
  b.sd = b.s > 0.f ? b.s : 1.f;
  const float y0 = __builtin_amdgcn_rcpf(b.sd);
  b.inv = __fmaf_rn(__fmaf_rn(-b.sd, y0, 1.f), y0, y0);
  return b;
}
constexpr uint32_t kCodeBase = 0x4b000000u;  // bits of 2^23
__device__ __forceinline__ uint32_t code_bits(float x, float z, const BlockDiv& b) {
  const float r = __fsub_rn(x, z);
  const float q0 = __fmul_rn(r, b.inv);
  const float e = __fmaf_rn(-b.sd, q0, r);
  const float q = __fmaf_rn(e, b.inv, q0);
  return __builtin_bit_cast(uint32_t, __fadd_rn(q, 8388608.f));
}

// One storage word from 32 / BITS values kCodeBase + code (element order):
// b << (BITS f) + ... keeps the codes in bits 0-15 (kCodeBase has its low
// 24 bits clear), and v_perm_b32 joins the two halves.
template <int BITS>
__device__ __forceinline__ uint32_t pack_bits(const uint32_t* b) {
  uint32_t lo = b[0], hi = b[1];
#pragma unroll
  for (int f = 1; f < 16 / BITS; ++f) {
    lo = (b[2 * f] << (BITS * f)) + lo;
    hi = (b[2 * f + 1] << (BITS * f)) + hi;
  }
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

template <int D, int BITS>
struct KPlan {
  static constexpr int EPW = Fmt<BITS>::EPW;
  static constexpr int NW = 2;                       // code words per lane and row
  static constexpr int W = D / (EPW * NW);           // lanes per key row
  static constexpr int RPS = 64 / W;                 // rows per slot
  static constexpr int LD = EPW / 8;                 // 16-byte loads per word
  static constexpr int S = 8 * 1024 / (64 * NW * EPW * 2);  // slots per wave: 8 KB of rows
  static constexpr int ROWS = RPS * S;               // rows per wave
  static constexpr int DW = NW * EPW / 2;            // dwords of a lane's part of a row
};

// Slice of the full set of heads that cache slice sl is quantised from (the
// head map of a hybrid cache), in scalar arithmetic: sl is uniform.
__device__ __forceinline__ uint32_t src_slice(uint32_t sl, const KvHeadMap& hm) {
  if (hm.n == 0) return sl;
  const uint32_t n = (uint32_t)hm.n;
  return (sl / n) * (uint32_t)hm.n_in + hm.g[sl % n];
}

// The wave's number in the grid (uniform, in a scalar register).
__device__ __forceinline__ uint32_t wave_id() {
  return __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
}

// K rows k0 .. k1 - 1 (nk of them) of every (b, g) of a cache of L keys.
// Wave w takes keys k0 + ROWS (w % cpw) .. of slice w / cpw (cpw = chunks
// per slice); rows past k1 are loaded from the slice's last row and not
// stored.
template <int D, int BITS, bool FULL>
__device__ __forceinline__ void quant_k_rows(const uint16_t* __restrict__ src,
                                             uint8_t* __restrict__ kq, uint32_t* __restrict__ kp,
                                             int krow, int nk, long long dst0) {
  using P = KPlan<D, BITS>;
  constexpr int CMAX = Fmt<BITS>::CMAX;
  const int lane = threadIdx.x & 63;
  const int w = lane % P::W;
  const int r0 = krow + lane / P::W;  // this lane's row of slot 0, from the slice's key k0
  uint32_t x[P::S][P::DW];
#pragma unroll
  for (int s = 0; s < P::S; ++s) {
    const int r = FULL ? r0 + s * P::RPS : min(r0 + s * P::RPS, nk - 1);
#pragma unroll
    for (int j = 0; j < P::NW; ++j) {
      const u32x4* p =
          reinterpret_cast<const u32x4*>(src + (long long)r * D + P::EPW * (w + P::W * j));
#pragma unroll
      for (int i = 0; i < P::LD; ++i) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
#pragma unroll
        for (int t = 0; t < 4; ++t) x[s][P::EPW / 2 * j + 4 * i + t] = v[t];
      }
    }
  }
#pragma unroll
  for (int s = 0; s < P::S; ++s) {
    float lo = elem(x[s], 0), hi = lo;
#pragma unroll
    for (int e = 1; e < P::NW * P::EPW; ++e) {
      lo = vmin(lo, elem(x[s], e));
      hi = vmax(hi, elem(x[s], e));
    }
    minmax_lanes<P::W>(lo, hi);
    const int r = r0 + s * P::RPS;
    if (!FULL && r >= nk) continue;
    const BlockDiv bd = block_div<CMAX>(lo, hi);
    uint32_t c[P::NW * P::EPW];
#pragma unroll
    for (int e = 0; e < P::NW * P::EPW; ++e) c[e] = code_bits(elem(x[s], e), lo, bd);
    float sc = bd.s;
    if (!bd.fast) {  // rare: one value at a time, indexing registers by a uniform counter
      sc = block_scale<CMAX>(lo, hi);
#pragma unroll 1
      for (int e = 0; e < P::NW * P::EPW; ++e)
        c[e] = kCodeBase + code_of<CMAX>(elem(x[s], e), sc, lo);
    }
    const long long row = dst0 + r;
    // a row's code words and parameter words come from several lanes and
    // stores: through L2, which joins the pieces of a line
    uint32_t* dst = reinterpret_cast<uint32_t*>(kq + row * (D * BITS / 8)) + w;
#pragma unroll
    for (int j = 0; j < P::NW; ++j) dst[P::W * j] = pack_bits<BITS>(c + P::EPW * j);
    if (w == 0) kp[row] = pack_params(sc, lo);
  }
}

template <int D, int BITS>
__global__ __launch_bounds__(256) void quant_k_kernel(const uint16_t* __restrict__ k,
                                                      uint8_t* __restrict__ kq,
                                                      uint32_t* __restrict__ kp, uint32_t slices,
                                                      uint32_t cpw, int L, int k0, int nk,
                                                      const KvHeadMap hm) {
  using P = KPlan<D, BITS>;
  const uint32_t wv = wave_id();
  const uint32_t sl = wv / cpw;
  if (sl >= slices) return;  // whole waves
  const int krow = (int)(wv % cpw) * P::ROWS;
  const uint16_t* src = k + ((long long)src_slice(sl, hm) * L + k0) * D;
  const long long dst0 = (long long)sl * L + k0;
  if (krow + P::ROWS <= nk)
    quant_k_rows<D, BITS, true>(src, kq, kp, krow, nk, dst0);
  else
    quant_k_rows<D, BITS, false>(src, kq, kp, krow, nk, dst0);
}

template <int D, int BITS>
struct VPlan {
  static constexpr int EPW = Fmt<BITS>::EPW;
  static constexpr int C = (BITS == 2 && D == 64) ? 4 : 8;  // channels per lane
  static constexpr int LG = D / C;                          // lanes per key row
  static constexpr int KL = 64 / (64 / LG);                 // keys per lane (= LG)
  static constexpr int WPC = KL / EPW;                      // code words per channel and lane
  static constexpr int RB = 64 * BITS / 8;                  // bytes of a channel's code row
  static_assert(KL % EPW == 0, "a lane's keys must be whole code words");
};

// The codes of one tile's lane: nl valid keys of KL (FULL: all of them).
template <int D, int BITS, bool FULL>
__device__ __forceinline__ void quant_v_lane(const uint32_t (&x)[VPlan<D, BITS>::KL][VPlan<D, BITS>::C / 2],
                                             int nl, int kg, long long blk,
                                             uint8_t* __restrict__ vq, uint32_t* __restrict__ vp) {
  using P = VPlan<D, BITS>;
  constexpr int CMAX = Fmt<BITS>::CMAX;
  uint32_t params[P::C];
#pragma unroll
  for (int e = 0; e < P::C; ++e) {
    float lo = elem(x[0], e), hi = lo;  // key 0 of a lane: valid whenever any is
#pragma unroll
    for (int i = 1; i < P::KL; ++i) {
      if (FULL || i < nl) {
        lo = vmin(lo, elem(x[i], e));
        hi = vmax(hi, elem(x[i], e));
      }
    }
    if (!FULL && nl == 0) {
      lo = __builtin_inff();
      hi = -__builtin_inff();
    }
    minmax_strided<P::LG>(lo, hi);
    const BlockDiv bd = block_div<CMAX>(lo, hi);
    uint32_t c[P::KL];
#pragma unroll
    for (int i = 0; i < P::KL; ++i)
      c[i] = (FULL || i < nl) ? code_bits(elem(x[i], e), lo, bd) : kCodeBase;
    float sc = bd.s;
    if (!bd.fast) {
      sc = block_scale<CMAX>(lo, hi);
#pragma unroll
      for (int i = 0; i < P::KL; ++i)
        c[i] = kCodeBase + ((FULL || i < nl) ? code_of<CMAX>(elem(x[i], e), sc, lo) : 0u);
    }
    params[e] = pack_params(sc, lo);
    uint32_t words[P::WPC];
#pragma unroll
    for (int wd = 0; wd < P::WPC; ++wd) words[wd] = pack_bits<BITS>(c + P::EPW * wd);
    uint8_t* row = vq + (blk + e) * P::RB + kg * P::WPC * 4;
    // a few bytes of each of 16 code rows per store: through L2, which joins
    // the pieces of a line before it is written back
    if constexpr (P::WPC == 2) {
      *reinterpret_cast<u32x2*>(row) = u32x2{words[0], words[1]};
    } else {
      *reinterpret_cast<uint32_t*>(row) = words[0];
    }
  }
  if (kg == 0) {
    u32x4* dst = reinterpret_cast<u32x4*>(vp + blk);
#pragma unroll
    for (int h = 0; h < P::C / 4; ++h)
      __builtin_nontemporal_store(
          u32x4{params[4 * h], params[4 * h + 1], params[4 * h + 2], params[4 * h + 3]}, dst + h);
  }
}

// V tiles t0 .. t0 + nt - 1 of every (b, g) of a cache of T tiles; a tile
// holds its keys below k1 (keys at or past k1 get code 0 and take no part
// in the block's minimum and maximum). One wave per tile, four per block.
// The V tile's loads: key i of the lane from row (i < nl ? i : 0) - kg KL
// of src (the tile's key 0 stands in for keys past its end).
template <int D, int BITS, bool FULL>
__device__ __forceinline__ void load_v_lane(const uint16_t* __restrict__ src, int nl, int kg,
                                            uint32_t (&x)[VPlan<D, BITS>::KL][VPlan<D, BITS>::C / 2]) {
  using P = VPlan<D, BITS>;
#pragma unroll
  for (int i = 0; i < P::KL; ++i) {
    const int r = FULL ? i : (i < nl ? i : -kg * P::KL);
    if constexpr (P::C == 8) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r * D));
#pragma unroll
      for (int j = 0; j < 4; ++j) x[i][j] = v[j];
    } else {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src + r * D));
#pragma unroll
      for (int j = 0; j < 2; ++j) x[i][j] = v[j];
    }
  }
}

// V tiles t0 .. t0 + nt - 1 of every (b, g) of a cache of T tiles; a tile
// holds its keys below k1 (keys at or past k1 get code 0 and take no part
// in the block's minimum and maximum). One wave per tile, four per block.
template <int D, int BITS>
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ v,
                                                      uint8_t* __restrict__ vq,
                                                      uint32_t* __restrict__ vp, int L, int T,
                                                      int t0, int nt, int k1, uint32_t tiles,
                                                      const KvHeadMap hm) {
  using P = VPlan<D, BITS>;
  const uint32_t tile = wave_id();
  if (tile >= tiles) return;  // whole waves
  const int lane = threadIdx.x & 63;
  const int lc = lane % P::LG, kg = lane / P::LG;
  const uint32_t bg = tile / (uint32_t)nt;
  const int t = t0 + (int)(tile % (uint32_t)nt);
  const int n = min(kTile, k1 - kTile * t);  // keys of the tile, >= 1
  const uint16_t* src = v + ((long long)src_slice(bg, hm) * L + (long long)kTile * t + kg * P::KL) * D +
                        P::C * lc;
  const long long blk = ((long long)bg * T + t) * D + P::C * lc;  // first channel's block
  uint32_t x[P::KL][P::C / 2];
  if (n == kTile) {
    load_v_lane<D, BITS, true>(src, P::KL, kg, x);
    quant_v_lane<D, BITS, true>(x, P::KL, kg, blk, vq, vp);
  } else {
    const int nl = max(0, min(P::KL, n - kg * P::KL));  // valid keys of this lane
    load_v_lane<D, BITS, false>(src, nl, kg, x);
    quant_v_lane<D, BITS, false>(x, nl, kg, blk, vq, vp);
  }
}

template <int D, int BITS>
int launch_quant_d(const QuantArgs& a) {
  using KP = KPlan<D, BITS>;
  const int nk = a.k1 - a.k0;
  const long long slices = (long long)a.B * a.Hkv;
  const long long cpw = (nk + KP::ROWS - 1) / KP::ROWS;  // K chunks per slice
  const long long kwaves = slices * cpw;
  const int T = (a.L + kTile - 1) / kTile;
  const int t0 = a.k0 / kTile;
  const int nt = (a.k1 + kTile - 1) / kTile - t0;
  const long long tiles = slices * nt;
  // wave numbers in 32 bits (a cache past 2^31 tiles would exceed HBM)
  if (kwaves > 0x7fffffffLL || tiles > 0x7fffffffLL) return -1;
  if (kwaves > 0)
    hipLaunchKernelGGL((quant_k_kernel<D, BITS>), dim3((unsigned)((kwaves + 3) / 4)), dim3(256), 0,
                       (hipStream_t)a.stream, (const uint16_t*)a.k, a.kq, a.kp, (uint32_t)slices,
                       (uint32_t)cpw, a.L, a.k0, nk, a.map);
  if (tiles > 0)
    hipLaunchKernelGGL((quant_v_kernel<D, BITS>), dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0,
                       (hipStream_t)a.stream, (const uint16_t*)a.v, a.vq, a.vp, a.L, T, t0, nt,
                       a.k1, (uint32_t)tiles, a.map);
  return 0;
}

}  // namespace

int launch_kv_quantize_q4(const QuantArgs& a) {
  return a.d == 128 ? launch_quant_d<128, 4>(a) : launch_quant_d<64, 4>(a);
}

int launch_kv_quantize_q2(const QuantArgs& a) {
  return a.d == 128 ? launch_quant_d<128, 2>(a) : launch_quant_d<64, 2>(a);
}

}  // namespace skipattn
