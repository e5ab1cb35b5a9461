// C ABI of libskipattn: argument validation and kernel launches.
// The operations and their readings are documented in include/skipattn.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/skipattn.h"
#include "launch.hpp"

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr long long kMaxElems = 1LL << 40;
// The kernels address one (b, head) slice of K, V (and Q) through a buffer
// resource with a 32-bit byte range and 32-bit offsets, with up to one tile of
// padding rows past its end and offsets at or above 2^31 reserved for loads
// that must read nothing; a slice must stay below 2^31 - 2^16 bytes.
constexpr long long kMaxHeadBytes = (1LL << 31) - (1LL << 16);

int check_tau(float tau) {
  if (isnan(tau)) return fail(SKIPATTN_EINVAL, "tau is NaN");
  if (tau < 0.f) return fail(SKIPATTN_EINVAL, "tau must be >= 0 (got %g)", (double)tau);
  return SKIPATTN_OK;
}

int check_heads(int Hq, int Hkv) {
  if (Hq < 1 || Hkv < 1) return fail(SKIPATTN_EINVAL, "Hq and Hkv must be >= 1 (got %d, %d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(SKIPATTN_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  return SKIPATTN_OK;
}

float tau_raw(float tau, int d) {
  return isinf(tau) ? INFINITY : (float)((double)tau * sqrt((double)d));
}

float exp2_scale(int d) { return (float)(1.4426950408889634 / sqrt((double)d)); }

int check_d(int d) {
  if (d != 64 && d != 128) return fail(SKIPATTN_EINVAL, "d must be 64 or 128 (got %d)", d);
  return SKIPATTN_OK;
}

// Prefill arguments; K and V heads are `cap` rows apart (cap >= N).
int prefill_check(const void* q, const void* k, const void* v, const float* o, const float* lse,
                  int B, int Hq, int Hkv, int Nq, int N, int cap, int d, int causal, float tau,
                  const uint8_t* skip_mask) {
  (void)skip_mask;
  g_err[0] = '\0';
  if (!q || !k || !v || !o || !lse) return fail(SKIPATTN_EINVAL, "NULL tensor pointer");
  if (B < 0 || N < 0 || Nq < 0 || d < 0)
    return fail(SKIPATTN_EINVAL, "negative size (B=%d Nq=%d N=%d d=%d)", B, Nq, N, d);
  if (Nq > N) return fail(SKIPATTN_EINVAL, "Nq (%d) exceeds N (%d)", Nq, N);
  if (cap < N) return fail(SKIPATTN_EINVAL, "cap (%d) is below N (%d)", cap, N);
  if (int e = check_heads(Hq, Hkv)) return e;
  if (causal != 0 && causal != 1) return fail(SKIPATTN_EINVAL, "causal must be 0 or 1 (got %d)", causal);
  if (int e = check_tau(tau)) return e;
  if (int e = check_d(d)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SKIPATTN_EINVAL, "q, k, v and o must be 16-byte aligned");
  if ((long long)B * Hq * N * (long long)d > kMaxElems ||
      (long long)B * Hkv * cap * (long long)d > kMaxElems)
    return fail(SKIPATTN_EINVAL, "tensor too large");
  if ((long long)N * d * 2 > kMaxHeadBytes)
    return fail(SKIPATTN_EUNSUPPORTED, "N * d * 2 = %lld bytes per head exceeds %lld", (long long)N * d * 2,
                kMaxHeadBytes);
  if (causal && (N - Nq) % SKIPATTN_TILE != 0)
    return fail(SKIPATTN_EUNSUPPORTED, "causal chunk must start on a 64-key boundary (N - Nq = %d)",
                N - Nq);
  return SKIPATTN_OK;
}

// Decode arguments; K and V heads (or the quantised cache's arrays) are
// sized for `cap` keys, of which the first L are attended.
int decode_check(const void* q, const void* k, const void* v, const float* o, const float* lse,
                 int B, int Hq, int Hkv, int L, int cap, int d, float tau,
                 const void* workspace, size_t workspace_bytes) {
  g_err[0] = '\0';
  if (!q || !k || !v || !o || !lse) return fail(SKIPATTN_EINVAL, "NULL tensor pointer");
  if (B < 0 || L < 0 || d < 0) return fail(SKIPATTN_EINVAL, "negative size (B=%d L=%d d=%d)", B, L, d);
  if (cap < L) return fail(SKIPATTN_EINVAL, "cap (%d) is below L (%d)", cap, L);
  if (int e = check_heads(Hq, Hkv)) return e;
  if (int e = check_tau(tau)) return e;
  if (int e = check_d(d)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SKIPATTN_EINVAL, "q, k, v and o must be 16-byte aligned");
  if ((long long)B * Hkv * cap * (long long)d > kMaxElems || (long long)B * Hq * (long long)d > kMaxElems)
    return fail(SKIPATTN_EINVAL, "tensor too large");
  if ((long long)L * d * 2 > kMaxHeadBytes)
    return fail(SKIPATTN_EUNSUPPORTED, "L * d * 2 = %lld bytes per head exceeds %lld", (long long)L * d * 2,
                kMaxHeadBytes);
  if (B == 0 || L == 0) return SKIPATTN_OK;
  const size_t need = attn_decode_workspace_bytes(B, Hq, L, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SKIPATTN_EWORKSPACE, "decode workspace needs %zu bytes (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(SKIPATTN_EINVAL, "workspace must be 16-byte aligned");
  return SKIPATTN_OK;
}

int check_degree(int degree) {
  if (degree != 0 && degree != 2 && degree != 3)
    return fail(SKIPATTN_EINVAL, "SAS degree must be 2 or 3, or 0 for exact (got %d)", degree);
  return SKIPATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err; }

int attn_prefill_chunk_check(const void* q, const void* k, const void* v, const float* o,
                             const float* lse, int B, int Hq, int Hkv, int Nq, int N, int d,
                             int causal, float tau, const uint8_t* skip_mask) {
  return prefill_check(q, k, v, o, lse, B, Hq, Hkv, Nq, N, N, d, causal, tau, skip_mask);
}

int attn_prefill_check(const void* q, const void* k, const void* v, const float* o,
                       const float* lse, int B, int Hq, int Hkv, int N, int d,
                       int causal, float tau, const uint8_t* skip_mask) {
  return attn_prefill_chunk_check(q, k, v, o, lse, B, Hq, Hkv, N, N, d, causal, tau, skip_mask);
}

}  // extern "C"

namespace {

int prefill_launch(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int N, int cap, int d, int causal, float tau,
                   uint8_t* skip_mask, void* stream, int sas = 0) {
  if (int e = prefill_check(q, k, v, o, lse, B, Hq, Hkv, Nq, N, cap, d, causal, tau, skip_mask))
    return e;
  if (B == 0 || Nq == 0) return SKIPATTN_OK;
  skipattn::PrefillArgs a{q,  k,     v,  o,  lse, skip_mask, B,
                          Hq, Hkv,   N,  d,  causal,
                          Nq, causal ? (N - Nq) / SKIPATTN_TILE : 0,
                          cap, tau_raw(tau, d), exp2_scale(d), stream};
  a.sas = sas;
  const int lr = skipattn::launch_prefill(a);
  if (lr == -1) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  if (lr == -3) return fail(SKIPATTN_EUNSUPPORTED, "SAS prefill: whole-sequence bf16 only");
  if (lr != 0) return fail(SKIPATTN_EHIP, "prefill: device query for the work queue failed");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "prefill launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

// Workspace of attn_prefill_qk8: fp8 codes of Q and K, then their tile
// scales, each part 256-byte aligned.
struct Qk8Layout {
  size_t qc, kc, qs, ks, total;
};
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
Qk8Layout qk8_layout(int B, int Hq, int Hkv, int N, int d) {
  Qk8Layout l;
  const size_t nt = ((size_t)N + SKIPATTN_TILE - 1) / SKIPATTN_TILE;
  l.qc = 0;
  l.kc = l.qc + align256((size_t)B * Hq * N * d);
  l.qs = l.kc + align256((size_t)B * Hkv * N * d);
  l.ks = l.qs + align256((size_t)B * Hq * nt * 4);
  l.total = l.ks + align256((size_t)B * Hkv * nt * 4);
  return l;
}

// Workspace of attn_prefill_pv8: the V code blocks, the V tiles' largest
// |v| (scratch), the V scales, then (qk8) the parts of attn_prefill_qk8.
struct Pv8Layout {
  size_t vc, vt, vs, qk, total;
};
Pv8Layout pv8_layout(int B, int Hq, int Hkv, int N, int d, int qk8) {
  Pv8Layout l;
  const size_t nt = ((size_t)N + SKIPATTN_TILE - 1) / SKIPATTN_TILE;
  l.vc = 0;
  l.vt = l.vc + align256((size_t)B * Hkv * nt * SKIPATTN_TILE * d);
  l.vs = l.vt + align256((size_t)B * Hkv * nt * 4);
  l.qk = l.vs + align256((size_t)B * Hkv * 4);
  l.total = l.qk + (qk8 ? qk8_layout(B, Hq, Hkv, N, d).total : 0);
  return l;
}

int decode_launch(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                  int Hq, int Hkv, int L, int cap, int d, float tau, int degree,
                  uint8_t* skip_mask, void* workspace, size_t workspace_bytes, void* stream) {
  if (int e = decode_check(q, k, v, o, lse, B, Hq, Hkv, L, cap, d, tau, workspace,
                           workspace_bytes))
    return e;
  if (int e = check_degree(degree)) return e;
  if (B == 0 || L == 0) return SKIPATTN_OK;
  const int nsplit = (L + SKIPATTN_SPLIT - 1) / SKIPATTN_SPLIT;
  float* ws_o = (float*)workspace;
  float* ws_lse = ws_o + (size_t)B * Hq * nsplit * d;
  skipattn::DecodeArgs a{q,  k,   v, o, lse, skip_mask, ws_o, ws_lse, B, Hq, Hkv, L, d, nsplit,
                         cap, tau_raw(tau, d), exp2_scale(d), stream, degree};
  if (skipattn::launch_decode(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "decode launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

int cache_ptrs_check(const uint8_t* kq, const uint32_t* kp, const uint8_t* vq, const uint32_t* vp) {
  g_err[0] = '\0';
  if (!kq || !kp || !vq || !vp) return fail(SKIPATTN_EINVAL, "NULL cache pointer");
  if (!aligned16(kq) || !aligned16(kp) || !aligned16(vq) || !aligned16(vp))
    return fail(SKIPATTN_EINVAL, "kq, kp, vq and vp must be 16-byte aligned");
  return SKIPATTN_OK;
}

// The shared body of the 4-bit and 2-bit cache decodes: both take the same
// arguments and differ only in the kernels.
int decode_quantized(int (*launch)(const skipattn::DecodeQ4Args&), const char* what,
                     const void* q, const uint8_t* kq, const uint32_t* kp, const uint8_t* vq,
                     const uint32_t* vp, float* o, float* lse, int B, int Hq, int Hkv, int L,
                     int cap, int d, float tau, int degree, uint8_t* skip_mask, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (int e = cache_ptrs_check(kq, kp, vq, vp)) return e;
  // The bf16 checks cover every other argument; kq stands in for k and v.
  if (int e = decode_check(q, kq, kq, o, lse, B, Hq, Hkv, L, cap, d, tau, workspace,
                           workspace_bytes))
    return e;
  if (int e = check_degree(degree)) return e;
  if (B == 0 || L == 0) return SKIPATTN_OK;
  const int nsplit = (L + SKIPATTN_SPLIT - 1) / SKIPATTN_SPLIT;
  float* ws_o = (float*)workspace;
  float* ws_lse = ws_o + (size_t)B * Hq * nsplit * d;
  skipattn::DecodeQ4Args a{q,    kq,     kp, vq, vp,  o, lse, skip_mask, ws_o,
                           ws_lse, B,    Hq, Hkv, L, d, nsplit, cap,
                           tau_raw(tau, d), exp2_scale(d), stream, degree};
  if (launch(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "%s launch: %s", what, hipGetErrorString(err));
  return SKIPATTN_OK;
}

// The checks of the 4-bit and 2-bit quantisers (Hkv: heads of k and v).
int quantize_check(const void* k, const void* v, const uint8_t* kq, const uint32_t* kp,
                   const uint8_t* vq, const uint32_t* vp, int B, int Hkv, int L, int d, int k0,
                   int k1) {
  g_err[0] = '\0';
  if (!k || !v || !kq || !kp || !vq || !vp) return fail(SKIPATTN_EINVAL, "NULL tensor pointer");
  if (B < 0 || L < 0 || d < 0) return fail(SKIPATTN_EINVAL, "negative size (B=%d L=%d d=%d)", B, L, d);
  if (Hkv < 1) return fail(SKIPATTN_EINVAL, "Hkv must be >= 1 (got %d)", Hkv);
  if (k0 < 0 || k1 < k0 || k1 > L)
    return fail(SKIPATTN_EINVAL, "key range [%d, %d) outside [0, %d]", k0, k1, L);
  if (int e = check_d(d)) return e;
  if (!aligned16(k) || !aligned16(v) || !aligned16(kq) || !aligned16(kp) || !aligned16(vq) ||
      !aligned16(vp))
    return fail(SKIPATTN_EINVAL, "every pointer must be 16-byte aligned");
  if ((long long)B * Hkv * L * (long long)d > kMaxElems)
    return fail(SKIPATTN_EINVAL, "tensor too large");
  if ((long long)L * d * 2 > kMaxHeadBytes)
    return fail(SKIPATTN_EUNSUPPORTED, "L * d * 2 = %lld bytes per head exceeds %lld", (long long)L * d * 2,
                kMaxHeadBytes);
  if (k0 % SKIPATTN_TILE != 0)
    return fail(SKIPATTN_EUNSUPPORTED, "k0 (%d) must be a multiple of 64", k0);
  return SKIPATTN_OK;
}

// Enqueue a checked quantiser call; with map.n the cache holds those heads.
int quantize_launch(int (*launch)(const skipattn::QuantArgs&), const void* k, const void* v,
                    uint8_t* kq, uint32_t* kp, uint8_t* vq, uint32_t* vp, int B, int Hkv, int L,
                    int d, int k0, int k1, void* stream, const skipattn::KvHeadMap& map) {
  if (B == 0 || k1 == k0) return SKIPATTN_OK;
  skipattn::QuantArgs a{k, v, kq, kp, vq, vp, B, Hkv, L, d, k0, k1, stream};
  if (map.n) {
    a.Hkv = map.n;
    a.map = map;
  }
  if (launch(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "quantize launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

// The shared body of the 4-bit and 2-bit quantisers.
int quantize_range(int (*launch)(const skipattn::QuantArgs&), const void* k, const void* v,
                   uint8_t* kq, uint32_t* kp, uint8_t* vq, uint32_t* vp, int B, int Hkv, int L,
                   int d, int k0, int k1, void* stream) {
  if (int e = quantize_check(k, v, kq, kp, vq, vp, B, Hkv, L, d, k0, k1)) return e;
  return quantize_launch(launch, k, v, kq, kp, vq, vp, B, Hkv, L, d, k0, k1, stream,
                         skipattn::KvHeadMap{});
}

// The head maps of a hybrid cache's two widths from the per-head widths
// (host array of Hkv entries, each 4 or 2): each width's heads in
// increasing order.
int hybrid_maps(const uint8_t* kv_bits, int Hkv, skipattn::KvHeadMap& m4,
                skipattn::KvHeadMap& m2) {
  g_err[0] = '\0';
  if (!kv_bits) return fail(SKIPATTN_EINVAL, "NULL kv_bits");
  if (Hkv < 1) return fail(SKIPATTN_EINVAL, "Hkv must be >= 1 (got %d)", Hkv);
  if (Hkv > skipattn::kMaxMappedHeads)
    return fail(SKIPATTN_EUNSUPPORTED, "a hybrid cache holds at most %d KV heads (got %d)",
                skipattn::kMaxMappedHeads, Hkv);
  m4 = skipattn::KvHeadMap{};
  m2 = skipattn::KvHeadMap{};
  m4.n_in = m2.n_in = Hkv;
  for (int g = 0; g < Hkv; ++g) {
    if (kv_bits[g] == 4) {
      m4.g[m4.n++] = (uint8_t)g;
    } else if (kv_bits[g] == 2) {
      m2.g[m2.n++] = (uint8_t)g;
    } else {
      return fail(SKIPATTN_EINVAL, "kv_bits[%d] must be 4 or 2 (got %d)", g, (int)kv_bits[g]);
    }
  }
  return SKIPATTN_OK;
}

int hybrid_quantize(const void* k, const void* v, const uint8_t* kv_bits, uint8_t* kq4,
                    uint32_t* kp4, uint8_t* vq4, uint32_t* vp4, uint8_t* kq2, uint32_t* kp2,
                    uint8_t* vq2, uint32_t* vp2, int B, int Hkv, int L, int d, int k0, int k1,
                    void* stream) {
  skipattn::KvHeadMap m4, m2;
  if (int e = hybrid_maps(kv_bits, Hkv, m4, m2)) return e;
  // every check before the first launch
  if (m4.n)
    if (int e = quantize_check(k, v, kq4, kp4, vq4, vp4, B, Hkv, L, d, k0, k1)) return e;
  if (m2.n)
    if (int e = quantize_check(k, v, kq2, kp2, vq2, vp2, B, Hkv, L, d, k0, k1)) return e;
  if (m4.n)
    if (int e = quantize_launch(skipattn::launch_kv_quantize_q4, k, v, kq4, kp4, vq4, vp4, B, Hkv,
                                L, d, k0, k1, stream, m4))
      return e;
  if (m2.n)
    if (int e = quantize_launch(skipattn::launch_kv_quantize_q2, k, v, kq2, kp2, vq2, vp2, B, Hkv,
                                L, d, k0, k1, stream, m2))
      return e;
  return SKIPATTN_OK;
}

// Decode over a hybrid cache: each width's split kernel writes its heads'
// rows of one set of partials (and of the mask), then one merge.
int hybrid_decode(const void* q, const uint8_t* kv_bits, const uint8_t* kq4,
                  const uint32_t* kp4, const uint8_t* vq4, const uint32_t* vp4,
                  const uint8_t* kq2, const uint32_t* kp2, const uint8_t* vq2,
                  const uint32_t* vp2, float* o, float* lse, int B, int Hq, int Hkv, int L,
                  int cap, int d, float tau, int degree, uint8_t* skip_mask, void* workspace,
                  size_t workspace_bytes, void* stream) {
  skipattn::KvHeadMap m4, m2;
  if (int e = hybrid_maps(kv_bits, Hkv, m4, m2)) return e;
  if (m4.n)
    if (int e = cache_ptrs_check(kq4, kp4, vq4, vp4)) return e;
  if (m2.n)
    if (int e = cache_ptrs_check(kq2, kp2, vq2, vp2)) return e;
  // The bf16 checks cover every other argument; a code array stands in for k and v.
  const uint8_t* any = m4.n ? kq4 : kq2;
  if (int e = decode_check(q, any, any, o, lse, B, Hq, Hkv, L, cap, d, tau, workspace,
                           workspace_bytes))
    return e;
  if (int e = check_degree(degree)) return e;
  if (B == 0 || L == 0) return SKIPATTN_OK;
  const int nsplit = (L + SKIPATTN_SPLIT - 1) / SKIPATTN_SPLIT;
  const int G = Hq / Hkv;
  float* ws_o = (float*)workspace;
  float* ws_lse = ws_o + (size_t)B * Hq * nsplit * d;
  struct Part {
    int (*launch)(const skipattn::DecodeQ4Args&);
    const skipattn::KvHeadMap* map;
    const uint8_t* kq;
    const uint32_t* kp;
    const uint8_t* vq;
    const uint32_t* vp;
  } parts[2] = {{skipattn::launch_decode_q4, &m4, kq4, kp4, vq4, vp4},
                {skipattn::launch_decode_q2, &m2, kq2, kp2, vq2, vp2}};
  for (const Part& p : parts) {
    if (p.map->n == 0) continue;
    skipattn::DecodeQ4Args a{q,      p.kq,     p.kp, p.vq, p.vp,  o, lse, skip_mask, ws_o,
                             ws_lse, B,        Hq,   Hkv,  L,     d, nsplit, cap,
                             tau_raw(tau, d), exp2_scale(d), stream, degree};
    a.Hq = p.map->n * G;
    a.Hkv = p.map->n;
    a.map = *p.map;
    a.merge = false;
    if (p.launch(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  }
  if (skipattn::launch_decode_merge(ws_o, ws_lse, o, lse, B * Hq, d, nsplit, stream) != 0)
    return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "decode_hybrid launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

// The 8-bit QK^T prefills: Q and K quantised into the workspace (fp8 E4M3,
// or symmetric int8), then the prefill on their codes.
int prefill_qk8_impl(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                     int Hq, int Hkv, int N, int d, int causal, float tau, uint8_t* skip_mask,
                     void* workspace, size_t workspace_bytes, void* stream, bool i8) {
  const char* name = i8 ? "prefill_qki8" : "prefill_qk8";
  if (int e = prefill_check(q, k, v, o, lse, B, Hq, Hkv, N, N, N, d, causal, tau, skip_mask))
    return e;
  if (B == 0 || N == 0) return SKIPATTN_OK;
  const Qk8Layout l = qk8_layout(B, Hq, Hkv, N, d);
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(SKIPATTN_EWORKSPACE, "%s workspace needs %zu bytes (got %zu)", name, l.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(SKIPATTN_EINVAL, "workspace must be 16-byte aligned");
  char* ws = (char*)workspace;
  uint8_t* qc = (uint8_t*)(ws + l.qc);
  uint8_t* kc = (uint8_t*)(ws + l.kc);
  float* qs = (float*)(ws + l.qs);
  float* ks = (float*)(ws + l.ks);
  auto quant = i8 ? skipattn::launch_quantize_i8 : skipattn::launch_quantize_fp8;
  if (quant(q, qc, qs, (long long)B * Hq, N, d, stream) != 0 ||
      quant(k, kc, ks, (long long)B * Hkv, N, d, stream) != 0)
    return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  skipattn::PrefillArgs a{qc, kc, v, o, lse, skip_mask, B, Hq, Hkv, N, d, causal,
                          N,  0,  N, tau_raw(tau, d), exp2_scale(d), stream, qs, ks};
  a.qk_int8 = i8;
  const int lr = skipattn::launch_prefill(a);
  if (lr == -1) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  if (lr != 0) return fail(SKIPATTN_EHIP, "%s: device query for the work queue failed", name);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "%s launch: %s", name, hipGetErrorString(err));
  return SKIPATTN_OK;
}
}  // namespace

extern "C" {

int attn_prefill_chunk(const void* q, const void* k, const void* v, float* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int N, int d, int causal, float tau,
                       uint8_t* skip_mask, void* stream) {
  return prefill_launch(q, k, v, o, lse, B, Hq, Hkv, Nq, N, N, d, causal, tau, skip_mask, stream);
}

int attn_prefill_chunk_cap(const void* q, const void* k, const void* v, float* o, float* lse,
                           int B, int Hq, int Hkv, int Nq, int N, int cap, int d, int causal,
                           float tau, uint8_t* skip_mask, void* stream) {
  return prefill_launch(q, k, v, o, lse, B, Hq, Hkv, Nq, N, cap, d, causal, tau, skip_mask,
                        stream);
}

int attn_prefill(const void* q, const void* k, const void* v, float* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float tau,
                 uint8_t* skip_mask, void* stream) {
  return prefill_launch(q, k, v, o, lse, B, Hq, Hkv, N, N, N, d, causal, tau, skip_mask, stream);
}

int attn_prefill_sas(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                     int Hq, int Hkv, int N, int d, int causal, float tau, int degree,
                     uint8_t* skip_mask, void* stream) {
  if (degree != 0 && degree != 2 && degree != 3)
    return fail(SKIPATTN_EINVAL, "SAS degree must be 0, 2 or 3 (got %d)", degree);
  return prefill_launch(q, k, v, o, lse, B, Hq, Hkv, N, N, N, d, causal, tau, skip_mask, stream,
                        degree);
}

size_t attn_prefill_pv8_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int qk8) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  return pv8_layout(B, Hq, Hkv, N, d, qk8 != 0).total;
}

int attn_prefill_pv8(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                     int Hq, int Hkv, int N, int d, int causal, float tau, int qk8,
                     uint8_t* skip_mask, void* workspace, size_t workspace_bytes, void* stream) {
  if (int e = prefill_check(q, k, v, o, lse, B, Hq, Hkv, N, N, N, d, causal, tau, skip_mask))
    return e;
  if (qk8 != 0 && qk8 != 1) return fail(SKIPATTN_EINVAL, "qk8 must be 0 or 1 (got %d)", qk8);
  if (B == 0 || N == 0) return SKIPATTN_OK;
  const Pv8Layout l = pv8_layout(B, Hq, Hkv, N, d, qk8);
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(SKIPATTN_EWORKSPACE, "prefill_pv8 workspace needs %zu bytes (got %zu)", l.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(SKIPATTN_EINVAL, "workspace must be 16-byte aligned");
  char* ws = (char*)workspace;
  uint8_t* vc = (uint8_t*)(ws + l.vc);
  float* vt = (float*)(ws + l.vt);
  float* vs = (float*)(ws + l.vs);
  if (skipattn::launch_quantize_v8(v, vc, vt, vs, (long long)B * Hkv, N, d, stream) != 0)
    return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  skipattn::PrefillArgs a{q,  k,  vc, o, lse, skip_mask, B, Hq, Hkv, N, d, causal,
                          N,  0,  N, tau_raw(tau, d), exp2_scale(d), stream};
  a.vscale = vs;
  if (qk8) {
    const Qk8Layout lq = qk8_layout(B, Hq, Hkv, N, d);
    char* wq = ws + l.qk;
    uint8_t* qc = (uint8_t*)(wq + lq.qc);
    uint8_t* kc = (uint8_t*)(wq + lq.kc);
    float* qs = (float*)(wq + lq.qs);
    float* ks = (float*)(wq + lq.ks);
    if (skipattn::launch_quantize_fp8(q, qc, qs, (long long)B * Hq, N, d, stream) != 0 ||
        skipattn::launch_quantize_fp8(k, kc, ks, (long long)B * Hkv, N, d, stream) != 0)
      return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
    a.q = qc;
    a.k = kc;
    a.qscale = qs;
    a.kscale = ks;
  }
  const int lr = skipattn::launch_prefill(a);
  if (lr == -1) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  if (lr != 0) return fail(SKIPATTN_EHIP, "prefill_pv8: device query for the work queue failed");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "prefill_pv8 launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

size_t attn_prefill_qk8_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  return qk8_layout(B, Hq, Hkv, N, d).total;
}

int attn_prefill_qk8(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                     int Hq, int Hkv, int N, int d, int causal, float tau, uint8_t* skip_mask,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_qk8_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, tau, skip_mask, workspace,
                          workspace_bytes, stream, false);
}

int attn_prefill_qki8(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                      int Hq, int Hkv, int N, int d, int causal, float tau, uint8_t* skip_mask,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_qk8_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, tau, skip_mask, workspace,
                          workspace_bytes, stream, true);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int L, int d) {
  if (B <= 0 || Hq <= 0 || L <= 0 || d <= 0) return 0;
  const size_t nsplit = ((size_t)L + SKIPATTN_SPLIT - 1) / SKIPATTN_SPLIT;
  return (size_t)B * Hq * nsplit * ((size_t)d + 1) * sizeof(float);
}

int attn_decode_check(const void* q, const void* k, const void* v, const float* o,
                      const float* lse, int B, int Hq, int Hkv, int L, int d, float tau,
                      const uint8_t* skip_mask, const void* workspace, size_t workspace_bytes) {
  (void)skip_mask;
  return decode_check(q, k, v, o, lse, B, Hq, Hkv, L, L, d, tau, workspace, workspace_bytes);
}

int attn_decode(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                int Hq, int Hkv, int L, int d, float tau, uint8_t* skip_mask, void* workspace,
                size_t workspace_bytes, void* stream) {
  return decode_launch(q, k, v, o, lse, B, Hq, Hkv, L, L, d, tau, 0, skip_mask, workspace,
                       workspace_bytes, stream);
}

int attn_decode_sas(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                    int Hq, int Hkv, int L, int d, float tau, int degree, uint8_t* skip_mask,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_launch(q, k, v, o, lse, B, Hq, Hkv, L, L, d, tau, degree, skip_mask, workspace,
                       workspace_bytes, stream);
}

int attn_decode_cap(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                    int Hq, int Hkv, int L, int cap, int d, float tau, int degree,
                    uint8_t* skip_mask, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_launch(q, k, v, o, lse, B, Hq, Hkv, L, cap, d, tau, degree, skip_mask, workspace,
                       workspace_bytes, stream);
}

int attn_decode_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                        int B, int Hq, int Hkv, int L, int d, float tau, uint8_t* skip_mask,
                        void* stream) {
  // attn_decode's checks, with the device scratch in place of the workspace
  // (a non-null, aligned stand-in address: the checks never dereference it)
  const void* stand_in = reinterpret_cast<const void*>(uintptr_t(256));
  const int e = decode_check(q, k, v, o, lse, B, Hq, Hkv, L, L, d, tau, stand_in,
                             skipattn::kDecodeScratchBytes);
  if (e == SKIPATTN_EWORKSPACE)
    return fail(SKIPATTN_EWORKSPACE,
                "attn_decode_noalloc: the per-split partials need %zu bytes, more than the "
                "%zu-byte device scratch (attn_decode takes a workspace of any size)",
                attn_decode_workspace_bytes(B, Hq, L, d), skipattn::kDecodeScratchBytes);
  if (e) return e;
  if (B == 0 || L == 0) return SKIPATTN_OK;
  void* ws = nullptr;
  if (skipattn::decode_scratch(&ws) != 0)
    return fail(SKIPATTN_EHIP, "attn_decode_noalloc: no device address for the scratch");
  return decode_launch(q, k, v, o, lse, B, Hq, Hkv, L, L, d, tau, 0, skip_mask, ws,
                       skipattn::kDecodeScratchBytes, stream);
}

int attn_decode_q4_check(const void* q, const uint8_t* kq, const uint32_t* kp,
                         const uint8_t* vq, const uint32_t* vp, const float* o,
                         const float* lse, int B, int Hq, int Hkv, int L, int d, float tau,
                         const uint8_t* skip_mask, const void* workspace,
                         size_t workspace_bytes) {
  (void)skip_mask;
  if (int e = cache_ptrs_check(kq, kp, vq, vp)) return e;
  return decode_check(q, kq, kq, o, lse, B, Hq, Hkv, L, L, d, tau, workspace, workspace_bytes);
}

int attn_decode_q2_check(const void* q, const uint8_t* kq, const uint32_t* kp,
                         const uint8_t* vq, const uint32_t* vp, const float* o,
                         const float* lse, int B, int Hq, int Hkv, int L, int d, float tau,
                         const uint8_t* skip_mask, const void* workspace,
                         size_t workspace_bytes) {
  return attn_decode_q4_check(q, kq, kp, vq, vp, o, lse, B, Hq, Hkv, L, d, tau, skip_mask,
                              workspace, workspace_bytes);
}

int attn_decode_q4(const void* q, const uint8_t* kq, const uint32_t* kp, const uint8_t* vq,
                   const uint32_t* vp, float* o, float* lse, int B, int Hq, int Hkv, int L, int d,
                   float tau, uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return decode_quantized(skipattn::launch_decode_q4, "decode_q4", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, L, d, tau, 0, skip_mask, workspace, workspace_bytes, stream);
}

int attn_decode_q4_sas(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o, float* lse, int B,
                       int Hq, int Hkv, int L, int d, float tau, int degree,
                       uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_quantized(skipattn::launch_decode_q4, "decode_q4", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, L, d, tau, degree, skip_mask, workspace, workspace_bytes,
                          stream);
}

int attn_decode_q4_cap(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o, float* lse, int B,
                       int Hq, int Hkv, int L, int cap, int d, float tau, int degree,
                       uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_quantized(skipattn::launch_decode_q4, "decode_q4", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, cap, d, tau, degree, skip_mask, workspace,
                          workspace_bytes, stream);
}

int attn_decode_q2(const void* q, const uint8_t* kq, const uint32_t* kp, const uint8_t* vq,
                   const uint32_t* vp, float* o, float* lse, int B, int Hq, int Hkv, int L, int d,
                   float tau, uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return decode_quantized(skipattn::launch_decode_q2, "decode_q2", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, L, d, tau, 0, skip_mask, workspace, workspace_bytes, stream);
}

int attn_decode_q2_sas(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o, float* lse, int B,
                       int Hq, int Hkv, int L, int d, float tau, int degree,
                       uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_quantized(skipattn::launch_decode_q2, "decode_q2", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, L, d, tau, degree, skip_mask, workspace, workspace_bytes,
                          stream);
}

int attn_decode_q2_cap(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o, float* lse, int B,
                       int Hq, int Hkv, int L, int cap, int d, float tau, int degree,
                       uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_quantized(skipattn::launch_decode_q2, "decode_q2", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, cap, d, tau, degree, skip_mask, workspace,
                          workspace_bytes, stream);
}

int attn_kv_quantize_q4_range(const void* k, const void* v, uint8_t* kq, uint32_t* kp,
                              uint8_t* vq, uint32_t* vp, int B, int Hkv, int L, int d, int k0,
                              int k1, void* stream) {
  return quantize_range(skipattn::launch_kv_quantize_q4, k, v, kq, kp, vq, vp, B, Hkv, L, d, k0,
                        k1, stream);
}

int attn_kv_quantize_q4(const void* k, const void* v, uint8_t* kq, uint32_t* kp, uint8_t* vq,
                        uint32_t* vp, int B, int Hkv, int L, int d, void* stream) {
  return attn_kv_quantize_q4_range(k, v, kq, kp, vq, vp, B, Hkv, L, d, 0, L < 0 ? 0 : L, stream);
}

int attn_kv_quantize_q2_range(const void* k, const void* v, uint8_t* kq, uint32_t* kp,
                              uint8_t* vq, uint32_t* vp, int B, int Hkv, int L, int d, int k0,
                              int k1, void* stream) {
  return quantize_range(skipattn::launch_kv_quantize_q2, k, v, kq, kp, vq, vp, B, Hkv, L, d, k0,
                        k1, stream);
}

int attn_kv_quantize_q2(const void* k, const void* v, uint8_t* kq, uint32_t* kp, uint8_t* vq,
                        uint32_t* vp, int B, int Hkv, int L, int d, void* stream) {
  return attn_kv_quantize_q2_range(k, v, kq, kp, vq, vp, B, Hkv, L, d, 0, L < 0 ? 0 : L, stream);
}

int attn_kv_quantize_hybrid_range(const void* k, const void* v, const uint8_t* kv_bits,
                                  uint8_t* kq4, uint32_t* kp4, uint8_t* vq4, uint32_t* vp4,
                                  uint8_t* kq2, uint32_t* kp2, uint8_t* vq2, uint32_t* vp2,
                                  int B, int Hkv, int L, int d, int k0, int k1, void* stream) {
  return hybrid_quantize(k, v, kv_bits, kq4, kp4, vq4, vp4, kq2, kp2, vq2, vp2, B, Hkv, L, d,
                         k0, k1, stream);
}

int attn_kv_quantize_hybrid(const void* k, const void* v, const uint8_t* kv_bits, uint8_t* kq4,
                            uint32_t* kp4, uint8_t* vq4, uint32_t* vp4, uint8_t* kq2,
                            uint32_t* kp2, uint8_t* vq2, uint32_t* vp2, int B, int Hkv, int L,
                            int d, void* stream) {
  return hybrid_quantize(k, v, kv_bits, kq4, kp4, vq4, vp4, kq2, kp2, vq2, vp2, B, Hkv, L, d, 0,
                         L < 0 ? 0 : L, stream);
}

int attn_decode_hybrid(const void* q, const uint8_t* kv_bits, const uint8_t* kq4,
                       const uint32_t* kp4, const uint8_t* vq4, const uint32_t* vp4,
                       const uint8_t* kq2, const uint32_t* kp2, const uint8_t* vq2,
                       const uint32_t* vp2, float* o, float* lse, int B, int Hq, int Hkv, int L,
                       int d, float tau, uint8_t* skip_mask, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return hybrid_decode(q, kv_bits, kq4, kp4, vq4, vp4, kq2, kp2, vq2, vp2, o, lse, B, Hq, Hkv, L,
                       L, d, tau, 0, skip_mask, workspace, workspace_bytes, stream);
}

int attn_decode_hybrid_cap(const void* q, const uint8_t* kv_bits, const uint8_t* kq4,
                           const uint32_t* kp4, const uint8_t* vq4, const uint32_t* vp4,
                           const uint8_t* kq2, const uint32_t* kp2, const uint8_t* vq2,
                           const uint32_t* vp2, float* o, float* lse, int B, int Hq, int Hkv,
                           int L, int cap, int d, float tau, int degree, uint8_t* skip_mask,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return hybrid_decode(q, kv_bits, kq4, kp4, vq4, vp4, kq2, kp2, vq2, vp2, o, lse, B, Hq, Hkv, L,
                       cap, d, tau, degree, skip_mask, workspace, workspace_bytes, stream);
}

}  // extern "C"
