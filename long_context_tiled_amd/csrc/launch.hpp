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
  float tau_raw;  // tau * sqrt(d): threshold in raw q.k units (+inf = dense)
  float c;        // log2(e) / sqrt(d)
  void* stream;
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
  float tau_raw;
  float c;
  void* stream;
  int sas;        // 0: exact exponentials; 2 or 3: SAS polynomial degree
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
  float tau_raw;
  float c;
  void* stream;
  int sas;        // 0: exact exponentials; 2 or 3: SAS polynomial degree
};

// Each returns 0 when the kernels were enqueued, nonzero if the grid cannot
// be expressed; launch errors are read back by the caller.
int launch_prefill(const PrefillArgs& a);
int launch_decode(const DecodeArgs& a);
int launch_kv_quantize_q4(const QuantArgs& a);
int launch_decode_q4(const DecodeQ4Args& a);
// The 2-bit cache (layout in kvq2.hip) takes the same arguments.
int launch_kv_quantize_q2(const QuantArgs& a);
int launch_decode_q2(const DecodeQ4Args& a);
// The log-sum-exp merge of per-split partials (shared by both decodes).
int launch_decode_merge(const float* ws_o, const float* ws_lse, float* o, float* lse, int nbh,
                        int d, int nsplit, void* stream);

}  // namespace skipattn
