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

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err; }

int attn_prefill_chunk_check(const void* q, const void* k, const void* v, const float* o,
                             const float* lse, int B, int Hq, int Hkv, int Nq, int N, int d,
                             int causal, float tau, const uint8_t* skip_mask) {
  (void)skip_mask;
  g_err[0] = '\0';
  if (!q || !k || !v || !o || !lse) return fail(SKIPATTN_EINVAL, "NULL tensor pointer");
  if (B < 0 || N < 0 || Nq < 0 || d < 0)
    return fail(SKIPATTN_EINVAL, "negative size (B=%d Nq=%d N=%d d=%d)", B, Nq, N, d);
  if (Nq > N) return fail(SKIPATTN_EINVAL, "Nq (%d) exceeds N (%d)", Nq, N);
  if (int e = check_heads(Hq, Hkv)) return e;
  if (causal != 0 && causal != 1) return fail(SKIPATTN_EINVAL, "causal must be 0 or 1 (got %d)", causal);
  if (int e = check_tau(tau)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SKIPATTN_EINVAL, "q, k, v and o must be 16-byte aligned");
  if ((long long)B * Hq * N * (long long)(d > 0 ? d : 1) > kMaxElems)
    return fail(SKIPATTN_EINVAL, "tensor too large");
  if (d != 64 && d != 128) return fail(SKIPATTN_EUNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  if ((long long)N * d * 2 > kMaxHeadBytes)
    return fail(SKIPATTN_EUNSUPPORTED, "N * d * 2 = %lld bytes per head exceeds %lld", (long long)N * d * 2,
                kMaxHeadBytes);
  if (causal && (N - Nq) % SKIPATTN_TILE != 0)
    return fail(SKIPATTN_EUNSUPPORTED, "causal chunk must start on a 64-key boundary (N - Nq = %d)",
                N - Nq);
  return SKIPATTN_OK;
}

int attn_prefill_check(const void* q, const void* k, const void* v, const float* o,
                       const float* lse, int B, int Hq, int Hkv, int N, int d,
                       int causal, float tau, const uint8_t* skip_mask) {
  return attn_prefill_chunk_check(q, k, v, o, lse, B, Hq, Hkv, N, N, d, causal, tau, skip_mask);
}

int attn_prefill_chunk(const void* q, const void* k, const void* v, float* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int N, int d, int causal, float tau,
                       uint8_t* skip_mask, void* stream) {
  if (int e = attn_prefill_chunk_check(q, k, v, o, lse, B, Hq, Hkv, Nq, N, d, causal, tau,
                                       skip_mask))
    return e;
  if (B == 0 || Nq == 0) return SKIPATTN_OK;
  skipattn::PrefillArgs a{q,         k,      v, o, lse, skip_mask, B, Hq, Hkv, N, d, causal,
                          Nq,        causal ? (N - Nq) / SKIPATTN_TILE : 0,
                          tau_raw(tau, d), exp2_scale(d), stream};
  if (skipattn::launch_prefill(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "prefill launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

int attn_prefill(const void* q, const void* k, const void* v, float* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float tau,
                 uint8_t* skip_mask, void* stream) {
  return attn_prefill_chunk(q, k, v, o, lse, B, Hq, Hkv, N, N, d, causal, tau, skip_mask, stream);
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
  g_err[0] = '\0';
  if (!q || !k || !v || !o || !lse) return fail(SKIPATTN_EINVAL, "NULL tensor pointer");
  if (B < 0 || L < 0 || d < 0) return fail(SKIPATTN_EINVAL, "negative size (B=%d L=%d d=%d)", B, L, d);
  if (int e = check_heads(Hq, Hkv)) return e;
  if (int e = check_tau(tau)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SKIPATTN_EINVAL, "q, k, v and o must be 16-byte aligned");
  if ((long long)B * Hkv * L * (long long)(d > 0 ? d : 1) > kMaxElems)
    return fail(SKIPATTN_EINVAL, "tensor too large");
  if (d != 64 && d != 128) return fail(SKIPATTN_EUNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  if (Hq / Hkv > 16) return fail(SKIPATTN_EUNSUPPORTED, "decode supports at most 16 query heads per KV head (got %d)", Hq / Hkv);
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

int attn_decode(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                int Hq, int Hkv, int L, int d, float tau, uint8_t* skip_mask, void* workspace,
                size_t workspace_bytes, void* stream) {
  return attn_decode_sas(q, k, v, o, lse, B, Hq, Hkv, L, d, tau, 0, skip_mask, workspace,
                         workspace_bytes, stream);
}

int attn_decode_sas(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                    int Hq, int Hkv, int L, int d, float tau, int degree, uint8_t* skip_mask,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (int e = attn_decode_check(q, k, v, o, lse, B, Hq, Hkv, L, d, tau, skip_mask, workspace,
                                workspace_bytes))
    return e;
  if (degree != 0 && degree != 2 && degree != 3)
    return fail(SKIPATTN_EINVAL, "SAS degree must be 2 or 3, or 0 for exact (got %d)", degree);
  if (B == 0 || L == 0) return SKIPATTN_OK;
  const int nsplit = (L + SKIPATTN_SPLIT - 1) / SKIPATTN_SPLIT;
  float* ws_o = (float*)workspace;
  float* ws_lse = ws_o + (size_t)B * Hq * nsplit * d;
  skipattn::DecodeArgs a{q, k, v, o, lse, skip_mask, ws_o, ws_lse, B, Hq, Hkv, L, d, nsplit,
                         tau_raw(tau, d), exp2_scale(d), stream, degree};
  if (skipattn::launch_decode(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "decode launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

int attn_decode_q4_check(const void* q, const uint8_t* kq, const uint32_t* kp,
                         const uint8_t* vq, const uint32_t* vp, const float* o,
                         const float* lse, int B, int Hq, int Hkv, int L, int d, float tau,
                         const uint8_t* skip_mask, const void* workspace,
                         size_t workspace_bytes) {
  g_err[0] = '\0';
  if (!kq || !kp || !vq || !vp) return fail(SKIPATTN_EINVAL, "NULL cache pointer");
  if (!aligned16(kq) || !aligned16(kp) || !aligned16(vq) || !aligned16(vp))
    return fail(SKIPATTN_EINVAL, "kq, kp, vq and vp must be 16-byte aligned");
  // The bf16 checks cover every other argument; kq stands in for k and v.
  return attn_decode_check(q, kq, kq, o, lse, B, Hq, Hkv, L, d, tau, skip_mask, workspace,
                           workspace_bytes);
}

}  // extern "C"

namespace {

// The shared body of the 4-bit and 2-bit cache decodes: both take the same
// arguments and differ only in the kernels.
int decode_quantized(int (*launch)(const skipattn::DecodeQ4Args&), const char* what,
                     const void* q, const uint8_t* kq, const uint32_t* kp, const uint8_t* vq,
                     const uint32_t* vp, float* o, float* lse, int B, int Hq, int Hkv, int L,
                     int d, float tau, int degree, uint8_t* skip_mask, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (degree != 0 && degree != 2 && degree != 3) {
    g_err[0] = '\0';
    return fail(SKIPATTN_EINVAL, "SAS degree must be 2 or 3, or 0 for exact (got %d)", degree);
  }
  if (int e = attn_decode_q4_check(q, kq, kp, vq, vp, o, lse, B, Hq, Hkv, L, d, tau, skip_mask,
                                   workspace, workspace_bytes))
    return e;
  if (B == 0 || L == 0) return SKIPATTN_OK;
  const int nsplit = (L + SKIPATTN_SPLIT - 1) / SKIPATTN_SPLIT;
  float* ws_o = (float*)workspace;
  float* ws_lse = ws_o + (size_t)B * Hq * nsplit * d;
  skipattn::DecodeQ4Args a{q,         kq,   kp,     vq, vp,     o,  lse,      skip_mask,
                           ws_o,      ws_lse, B,   Hq, Hkv, L, d, nsplit,
                           tau_raw(tau, d), exp2_scale(d), stream, degree};
  if (launch(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "%s launch: %s", what, hipGetErrorString(err));
  return SKIPATTN_OK;
}

// The shared body of the 4-bit and 2-bit quantisers.
int quantize_range(int (*launch)(const skipattn::QuantArgs&), const void* k, const void* v,
                   uint8_t* kq, uint32_t* kp, uint8_t* vq, uint32_t* vp, int B, int Hkv, int L,
                   int d, int k0, int k1, void* stream) {
  g_err[0] = '\0';
  if (!k || !v || !kq || !kp || !vq || !vp) return fail(SKIPATTN_EINVAL, "NULL tensor pointer");
  if (B < 0 || L < 0 || d < 0) return fail(SKIPATTN_EINVAL, "negative size (B=%d L=%d d=%d)", B, L, d);
  if (Hkv < 1) return fail(SKIPATTN_EINVAL, "Hkv must be >= 1 (got %d)", Hkv);
  if (k0 < 0 || k1 < k0 || k1 > L)
    return fail(SKIPATTN_EINVAL, "key range [%d, %d) outside [0, %d]", k0, k1, L);
  if (!aligned16(k) || !aligned16(v) || !aligned16(kq) || !aligned16(kp) || !aligned16(vq) ||
      !aligned16(vp))
    return fail(SKIPATTN_EINVAL, "every pointer must be 16-byte aligned");
  if ((long long)B * Hkv * L * (long long)(d > 0 ? d : 1) > kMaxElems)
    return fail(SKIPATTN_EINVAL, "tensor too large");
  if (d != 64 && d != 128) return fail(SKIPATTN_EUNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  if ((long long)L * d * 2 > kMaxHeadBytes)
    return fail(SKIPATTN_EUNSUPPORTED, "L * d * 2 = %lld bytes per head exceeds %lld", (long long)L * d * 2,
                kMaxHeadBytes);
  if (k0 % SKIPATTN_TILE != 0)
    return fail(SKIPATTN_EUNSUPPORTED, "k0 (%d) must be a multiple of 64", k0);
  if (B == 0 || k1 == k0) return SKIPATTN_OK;
  skipattn::QuantArgs a{k, v, kq, kp, vq, vp, B, Hkv, L, d, k0, k1, stream};
  if (launch(a) != 0) return fail(SKIPATTN_EUNSUPPORTED, "grid too large");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SKIPATTN_EHIP, "quantize launch: %s", hipGetErrorString(err));
  return SKIPATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_q4(const void* q, const uint8_t* kq, const uint32_t* kp, const uint8_t* vq,
                   const uint32_t* vp, float* o, float* lse, int B, int Hq, int Hkv, int L, int d,
                   float tau, uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return decode_quantized(skipattn::launch_decode_q4, "decode_q4", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, d, tau, 0, skip_mask, workspace, workspace_bytes, stream);
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

int attn_decode_q2_check(const void* q, const uint8_t* kq, const uint32_t* kp,
                         const uint8_t* vq, const uint32_t* vp, const float* o,
                         const float* lse, int B, int Hq, int Hkv, int L, int d, float tau,
                         const uint8_t* skip_mask, const void* workspace,
                         size_t workspace_bytes) {
  return attn_decode_q4_check(q, kq, kp, vq, vp, o, lse, B, Hq, Hkv, L, d, tau, skip_mask,
                              workspace, workspace_bytes);
}

int attn_decode_q2(const void* q, const uint8_t* kq, const uint32_t* kp, const uint8_t* vq,
                   const uint32_t* vp, float* o, float* lse, int B, int Hq, int Hkv, int L, int d,
                   float tau, uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return decode_quantized(skipattn::launch_decode_q2, "decode_q2", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, d, tau, 0, skip_mask, workspace, workspace_bytes, stream);
}

int attn_decode_q4_sas(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o, float* lse, int B,
                       int Hq, int Hkv, int L, int d, float tau, int degree,
                       uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_quantized(skipattn::launch_decode_q4, "decode_q4", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, d, tau, degree, skip_mask, workspace, workspace_bytes,
                          stream);
}

int attn_decode_q2_sas(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o, float* lse, int B,
                       int Hq, int Hkv, int L, int d, float tau, int degree,
                       uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_quantized(skipattn::launch_decode_q2, "decode_q2", q, kq, kp, vq, vp, o, lse, B,
                          Hq, Hkv, L, d, tau, degree, skip_mask, workspace, workspace_bytes,
                          stream);
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

}  // extern "C"
