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
};

// Each returns 0 when the kernels were enqueued, nonzero if the grid cannot
// be expressed; launch errors are read back by the caller.
int launch_prefill(const PrefillArgs& a);
int launch_decode(const DecodeArgs& a);

}  // namespace skipattn
