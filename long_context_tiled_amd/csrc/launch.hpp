// Host-side launch interfaces between the C ABI (api.hip) and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace skipattn {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  uint8_t* mask;
  int B, Hq, Hkv, N, d, causal;
  int Nq;         // queries: key positions N - Nq .. N - 1 (Nq == N: self-attention)
  int q0t;        // (N - Nq) / 64
  int cap;        // rows allocated per K/V head (>= N; N for a cache of exactly N keys)
  float tau_raw;  // tau * sqrt(d): threshold in raw q.k units (+inf = dense)
  float c;        // log2(e) / sqrt(d)
  void* stream;
  // fp8 QK^T: q and k are E4M3 codes (uint8, same shapes) with per-tile
  // scales qscale [B, Hq, ceil(Nq/64)], kscale [B, Hkv, ceil(cap/64)];
  // both null for bf16 q and k
  const float* qscale = nullptr;
  const float* kscale = nullptr;
  // 0: exact exponentials; 2 or 3: the SAS exponential of that degree (bf16
  // whole-sequence prefill only)
  int sas = 0;
  // 8-bit P.V (whole-sequence prefill only): v holds E4M3 code blocks
  // [B, Hkv, ceil(N/64), d, 64] (launch_quantize_v8) and vscale [B, Hkv]
  // their scales; null for bf16 V
  const float* vscale = nullptr;
  // int8 QK^T (whole-sequence prefill only, P.V in bf16): q and k hold
  // symmetric int8 codes with the fp8 path's tile scales (launch_quantize_i8)
  bool qk_int8 = false;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  uint8_t* mask;
  float* ws_o;    // [B, Hq, nsplit, d] per-split normalised outputs
  float* ws_lse;  // [B, Hq, nsplit] per-split natural-log LSE
  int B, Hq, Hkv, L, d, nsplit;
  int cap;        // rows allocated per K/V head (>= L)
  float tau_raw;
  float c;
  void* stream;
  int sas;        // 0: exact exponentials; 2 or 3: SAS polynomial degree
};

// The KV heads of one width of a hybrid cache (heads of different widths in
// arrays of their own): head i of such a sub-cache is head g[i] of the n_in
// heads of the full set. n = 0: no map (the cache holds every head).
constexpr int kMaxMappedHeads = 256;
struct KvHeadMap {
  int n = 0;
  int n_in = 0;
  uint8_t g[kMaxMappedHeads] = {};
};

struct QuantArgs {
  const void* k;  // bf16 [B, Hkv, L, d]
  const void* v;
  uint8_t* kq;    // codes and parameter words, layout in kvq4.hip / kvq2.hip
  uint32_t* kp;
  uint8_t* vq;
  uint32_t* vp;
  int B, Hkv, L, d;
  int k0, k1;     // keys written: k0 .. k1 - 1 (k0 a multiple of 64)
  void* stream;
  // map.n: the cache holds map.n (= Hkv) heads, head i quantised from head
  // map.g[i] of the map.n_in heads of k and v ([B, map.n_in, L, d])
  KvHeadMap map = {};
};

struct DecodeQ4Args {
  const void* q;
  const uint8_t* kq;
  const uint32_t* kp;
  const uint8_t* vq;
  const uint32_t* vp;
  float* o;
  float* lse;
  uint8_t* mask;
  float* ws_o;
  float* ws_lse;
  int B, Hq, Hkv, L, d, nsplit;
  int cap;        // keys the cache arrays are sized for (>= L)
  float tau_raw;
  float c;
  void* stream;
  int sas;        // 0: exact exponentials; 2 or 3: SAS polynomial degree
  // map.n: the cache holds map.n (= Hkv) of the map.n_in KV heads; q, the
  // per-split partials and the mask then hold the rows of all of them
  // ([B, map.n_in * Hq / Hkv, ...]), and this call touches its heads' rows
  KvHeadMap map = {};
  bool merge = true;  // false: the split kernel only (the caller merges)
};

// Each returns 0 when the kernels were enqueued, nonzero if the grid cannot
// be expressed (launch_prefill: -1, -2 when the device's work-queue address
// or compute-unit count cannot be read, -3 for an SAS or 8-bit P.V request
// outside their whole-sequence prefills); launch errors are read back by the
// caller.
int launch_prefill(const PrefillArgs& a);
int launch_decode(const DecodeArgs& a);
int launch_kv_quantize_q4(const QuantArgs& a);
int launch_decode_q4(const DecodeQ4Args& a);
// The 2-bit cache (layout in kvq2.hip) takes the same arguments.
int launch_kv_quantize_q2(const QuantArgs& a);
int launch_decode_q2(const DecodeQ4Args& a);
// Block-quantised fp8 (E4M3) codes of a bf16 tensor [X, N, D]: codes uint8
// [X, N, D] and one fp32 scale per 64-row block, scales [X, ceil(N/64)]
// (fp8.hip). Returns nonzero if the grid cannot be expressed.
int launch_quantize_fp8(const void* x, uint8_t* codes, float* scales, long long X, int N, int D,
                        void* stream);
// The same blocks as symmetric int8 codes (scale m / 127; fp8.hip).
int launch_quantize_i8(const void* x, uint8_t* codes, float* scales, long long X, int N, int D,
                       void* stream);
// V codes for the 8-bit P.V prefill (fp8.hip): bf16 V [X, N, D] -> E4M3
// codes in the kernel's tile blocks [X, ceil(N/64), D, 64] with one fp32
// scale per head, vscale [X]; tmax [X, ceil(N/64)] is scratch.
int launch_quantize_v8(const void* v, uint8_t* codes, float* tmax, float* vscale, long long X,
                       int N, int D, void* stream);
// Bytes of the device-resident decode scratch (decode.hip), and its address
// on the current device (0 on success; the first call on a device looks it
// up with that device current).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
int decode_scratch(void** ptr);
// The log-sum-exp merge of per-split partials (shared by both decodes).
int launch_decode_merge(const float* ws_o, const float* ws_lse, float* o, float* lse, int nbh,
                        int d, int nsplit, void* stream);

}  // namespace skipattn
