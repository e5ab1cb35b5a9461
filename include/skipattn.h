/*
 * skipattn.h - C ABI of libskipattn: exact tiled softmax attention with the
 * Skip-Softmax tile-skip rule, for long-context prefill and split-K decode,
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed
 * ----------------
 * Blockwise ("Flash") attention: scores, softmax and the value product are
 * formed one key block at a time and the N x N score matrix is never stored
 * (TurboAttention talk page, "Technical Deep Dive").
 *
 * Skip-Softmax (TensorRT-LLM Skip Softmax summary page, "Key Points" and
 * "Detailed Analysis"): key blocks are visited in ascending order, and a
 * block is skipped when its local maximum score lies below the running
 * maximum minus a user threshold tau. Readings fixed by this library:
 *   - scores are s = q.k / sqrt(d); tau is in the same (natural-logit) units;
 *   - the decision tile is 64 query rows x 64 keys; the running maximum is
 *     per query row, over the tiles kept so far; the tile is skipped iff
 *     EVERY valid row r has t_r < m_r - tau (strict), t_r = the row's
 *     maximum score inside the tile;
 *   - a skipped tile contributes nothing to the output, to the normaliser or
 *     to the running maximum; its scores are still formed for the test;
 *   - the first visited tile (running max -inf) is never skipped;
 *   - tau = +INFINITY gives dense exact attention; tau must be >= 0.
 * Query head h reads key/value head h / (Hq / Hkv) (grouped-query attention).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers to dense row-major arrays.
 *   q, k, v are bfloat16 (passed as void*); o and lse are float32.
 * - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *   null stream) and returns; results are valid once the stream has
 *   synchronised. The library never allocates, frees or synchronises.
 *   The caller owns every buffer, including the decode workspace.
 * - Arguments are validated on the host before anything is launched: a
 *   nonzero return leaves every output untouched.
 * - Calls on different streams may overlap; calls that share output or
 *   workspace buffers must be ordered by the caller.
 * - Empty work (B == 0, or N / L == 0) is valid and launches nothing.
 *
 * Return codes
 *   SKIPATTN_OK           0
 *   SKIPATTN_EINVAL       1  NULL q/k/v/o/lse pointer; negative size;
 *                            Hq or Hkv < 1 or Hq % Hkv != 0; d not in
 *                            {64, 128}; causal not 0/1; tau NaN or < 0; a
 *                            pointer not 16-byte aligned; an element count
 *                            beyond 2^40; a cache capacity below the
 *                            attended length (the _cap entry points)
 *   SKIPATTN_EUNSUPPORTED 2  one head of K/V over 2^31 - 2^16 bytes
 *                            (N * d * 2, L * d * 2); a causal chunk that
 *                            does not start on a 64-key boundary; a
 *                            quantiser key range starting off a tile
 *   SKIPATTN_EWORKSPACE   3  decode workspace NULL or smaller than
 *                            attn_decode_workspace_bytes()
 *   SKIPATTN_EHIP         4  a kernel launch failed (hipGetLastError)
 * attn_last_error() returns a description of the last nonzero return on
 * the calling thread.
 */
#ifndef SKIPATTN_H
#define SKIPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKIPATTN_OK 0
#define SKIPATTN_EINVAL 1
#define SKIPATTN_EUNSUPPORTED 2
#define SKIPATTN_EWORKSPACE 3
#define SKIPATTN_EHIP 4

/* Tile edge of the skip decision (queries and keys), and the decode split. */
#define SKIPATTN_TILE 64
#define SKIPATTN_SPLIT 4096

/* Mask byte values. */
#define SKIPATTN_KEPT 0
#define SKIPATTN_SKIPPED 1
#define SKIPATTN_NOT_VISITED 2

/*
 * attn_prefill - causal or full self-attention over N tokens.
 *
 *   q    bf16 [B, Hq,  N, d]
 *   k    bf16 [B, Hkv, N, d]
 *   v    bf16 [B, Hkv, N, d]
 *   o    fp32 [B, Hq,  N, d]  out: softmax over the kept keys, times V
 *   lse  fp32 [B, Hq,  N]     out: natural-log sum of e^s over kept keys
 *   causal     1: query i attends keys j <= i; tiles wholly above the
 *              diagonal are not visited. 0: every key.
 *   tau        skip threshold in logit units, >= 0; +INFINITY = dense.
 *   skip_mask  NULL, or uint8 [B, Hq, ceil(N/64), ceil(N/64)], written for
 *              every (query tile, key tile): SKIPATTN_KEPT, SKIPATTN_SKIPPED,
 *              or SKIPATTN_NOT_VISITED (causal tiles above the diagonal).
 * N need not be a multiple of 64: missing keys of the last tile are masked
 * and missing rows of the last query tile take no part in the vote.
 */
int attn_prefill(const void* q, const void* k, const void* v, float* o,
                 float* lse, int B, int Hq, int Hkv, int N, int d, int causal,
                 float tau, uint8_t* skip_mask, void* stream);

/*
 * attn_prefill_chunk - chunked prefill: the last Nq of N positions attend
 * to the N keys (the rows N - Nq .. N - 1 of attn_prefill over N positions,
 * with the same decisions and results; attn_prefill is the case Nq == N).
 *
 *   q    bf16 [B, Hq,  Nq, d]  the chunk's queries
 *   k    bf16 [B, Hkv, N,  d]  every key up to the chunk's end
 *   v    bf16 [B, Hkv, N,  d]
 *   o    fp32 [B, Hq,  Nq, d]  out
 *   lse  fp32 [B, Hq,  Nq]     out
 *   skip_mask  NULL, or uint8 [B, Hq, ceil(Nq/64), ceil(N/64)].
 * causal == 1 requires N - Nq to be a multiple of 64 (the chunk starts on a
 * decision-tile boundary; SKIPATTN_EUNSUPPORTED otherwise); 0 <= Nq <= N.
 */
int attn_prefill_chunk(const void* q, const void* k, const void* v, float* o,
                       float* lse, int B, int Hq, int Hkv, int Nq, int N, int d,
                       int causal, float tau, uint8_t* skip_mask, void* stream);

/*
 * attn_prefill_chunk_cap - attn_prefill_chunk over K and V held in a cache
 * allocated for `cap` keys per (sequence, KV head), of which the first N
 * exist (chunked prefill into a preallocated cache):
 *   k, v  bf16 [B, Hkv, cap, d]   rows N .. cap - 1 are not read
 * cap >= N (SKIPATTN_EINVAL otherwise); every other argument, result and
 * error as for attn_prefill_chunk, which is the case cap == N.
 */
int attn_prefill_chunk_cap(const void* q, const void* k, const void* v, float* o,
                           float* lse, int B, int Hq, int Hkv, int Nq, int N,
                           int cap, int d, int causal, float tau,
                           uint8_t* skip_mask, void* stream);

/*
 * attn_prefill_sas - attn_prefill with the Sparse Activated SoftMax
 * exponential (TurboAttention talk page, "Technical Deep Dive", its Sparse
 * Activated SoftMax part): every exponential of each query row's online
 * softmax, the probabilities e^-(m - s) and the rescale factor when a kept
 * tile raises the row's running maximum m, is taken as T[n] p(f), with
 * n = floor(x), f = x - n for the gap x in logits, T[n] = e^-n for n < 6 and
 * 0 from 6 on, and p the least-squares polynomial of degree `degree` (2 or
 * 3) for e^-f on [0, 1] (the exponential of attn_decode_sas). The skip
 * decisions, outputs and mask are those of attn_prefill; `degree` 0 is
 * attn_prefill itself. Results depend on the order in which the running
 * maximum rises (ascending key tiles, as for the rule). It computes more
 * vector instructions per score than the exact exponential (the exponential
 * unit still gives e^-n), so it is slower; it exists as the pages' option.
 * Errors as for attn_prefill, and SKIPATTN_EINVAL for another degree.
 */
int attn_prefill_sas(const void* q, const void* k, const void* v, float* o,
                     float* lse, int B, int Hq, int Hkv, int N, int d,
                     int causal, float tau, int degree, uint8_t* skip_mask,
                     void* stream);

/*
 * attn_prefill_qk8 - attn_prefill with QK^T on block-quantised 8-bit
 * operands (TurboAttention talk page, "Technical Deep Dive" and "Key
 * Findings": symmetric 8-bit quantisation of the matrix-product operands,
 * block-wise inside the flash blocks). Q and K are quantised to fp8 E4M3
 * per 64-row tile (a query tile of Q, a key tile of K) and S = Q K^T runs on
 * the fp8 matrix cores; V, P V, the softmax and the skip rule are as in
 * attn_prefill. Per tile: scale s = (largest |x| in the tile) / 448 in fp32
 * (1 for a tile of zeros); code = the E4M3 value nearest clamp(x / s, -448,
 * 448) (fp32 division; ties to the even mantissa; a value that rounds to
 * zero is code 0). The scores are those of the dequantised q^ = code * s_q,
 * k^ = code * s_k.
 *
 *   q, k, v, o, lse, causal, tau, skip_mask  as for attn_prefill
 *   workspace  device scratch of at least attn_prefill_qk8_workspace_bytes();
 *              on return (once the stream has synchronised) it holds, each
 *              part starting on a 256-byte boundary: Q codes uint8 [B, Hq,
 *              N, d], K codes uint8 [B, Hkv, N, d], Q scales fp32 [B, Hq,
 *              ceil(N/64)], K scales fp32 [B, Hkv, ceil(N/64)].
 * Errors as for attn_prefill; SKIPATTN_EWORKSPACE if the workspace is NULL
 * or too small.
 */
size_t attn_prefill_qk8_workspace_bytes(int B, int Hq, int Hkv, int N, int d);
int attn_prefill_qk8(const void* q, const void* k, const void* v, float* o,
                     float* lse, int B, int Hq, int Hkv, int N, int d,
                     int causal, float tau, uint8_t* skip_mask,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_prefill_qki8 - attn_prefill_qk8 with symmetric int8 operands, the
 * pages' own 8-bit format for the QK^T product (TurboAttention talk page,
 * "Technical Deep Dive": symmetric int8 quantisation block-wise inside the
 * flash blocks). Q and K are quantised per 64-row tile: scale s = (largest
 * |x| in the tile) / 127 in fp32 (1 for a tile of zeros), code =
 * clamp(rint(x / s), -127, 127) (fp32 division, rint ties to even), and
 * S = Q K^T runs on the int8 matrix cores, exact in int32, before the tile's
 * scales apply. The scores are those of q^ = code * s_q, k^ = code * s_k.
 * Arguments, outputs and errors as for attn_prefill_qk8, whole sequences
 * only; the workspace is attn_prefill_qk8_workspace_bytes() bytes with the
 * same parts, the codes as two's complement int8 bytes.
 */
int attn_prefill_qki8(const void* q, const void* k, const void* v, float* o,
                      float* lse, int B, int Hq, int Hkv, int N, int d,
                      int causal, float tau, uint8_t* skip_mask,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_prefill_pv8 - attn_prefill with the P.V product on 8-bit operands too
 * (TurboAttention talk page, "Technical Deep Dive" and "Key Findings": both
 * products of blockwise attention on block-quantised 8-bit operands), QK^T
 * in bf16 (qk8 = 0) or as in attn_prefill_qk8 (qk8 = 1; any other value:
 * SKIPATTN_EINVAL). V is quantised by the call into E4M3 codes with one fp32
 * scale per (sequence, KV head), s = (largest |v| of the head) / 448 (1 for
 * a head of zeros), code = E4M3 of v / s (fp32 division, ties to even). Each
 * probability, taken relative to the row's reference maximum (the running
 * maximum as of the last rescale, which moves once some row of the 64-row
 * block has grown past it by more than 8 ln 2, taking every grown row to its
 * running maximum), is rounded to E4M3 without a scale (it stays below 2^8)
 * before it multiplies V's codes; the row sums stay over the unrounded
 * probabilities. O = s (sum of E4M3(p) codes) / l, LSE = m_ref + ln l.
 * Skip decisions follow the rule on the (bf16 or 8-bit) scores. Arguments,
 * outputs and errors as for attn_prefill, whole sequences only, plus the
 * workspace: attn_prefill_pv8_workspace_bytes(B, Hq, Hkv, N, d, qk8) bytes,
 * 16-byte aligned (SKIPATTN_EWORKSPACE if smaller or NULL), holding the V
 * code blocks, their scales and (qk8) the parts of attn_prefill_qk8's.
 */
size_t attn_prefill_pv8_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int qk8);
int attn_prefill_pv8(const void* q, const void* k, const void* v, float* o,
                     float* lse, int B, int Hq, int Hkv, int N, int d,
                     int causal, float tau, int qk8, uint8_t* skip_mask,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_workspace_bytes - bytes of device scratch attn_decode needs:
 * B * Hq * ceil(L / 4096) * (d + 1) * 4 (per-split partial outputs and
 * log-sum-exps). Returns 0 for invalid or empty sizes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int L, int d);

/*
 * attn_decode - one query token per sequence against a contiguous KV cache,
 * split-K over fixed 4096-key splits.
 *
 *   q    bf16 [B, Hq, d]
 *   k    bf16 [B, Hkv, L, d]
 *   v    bf16 [B, Hkv, L, d]
 *   o    fp32 [B, Hq, d]   out
 *   lse  fp32 [B, Hq]      out, natural log
 *   tau        as for attn_prefill. The decision tile is one query x 64 keys,
 *              per query head. Each split [4096 s, 4096 (s+1)) runs the rule
 *              over its own tiles with its own running maximum, starting at
 *              -inf, so the first tile of every split is kept.
 *   skip_mask  NULL, or uint8 [B, Hq, ceil(L/64)]: SKIPATTN_KEPT or
 *              SKIPATTN_SKIPPED per (head, key tile).
 *   workspace  device scratch of at least attn_decode_workspace_bytes();
 *              its contents on entry do not matter.
 * The query attends all L cached keys (no mask). The per-split partial
 * results are merged by log-sum-exp in a second kernel on the same stream.
 */
int attn_decode(const void* q, const void* k, const void* v, float* o,
                float* lse, int B, int Hq, int Hkv, int L, int d, float tau,
                uint8_t* skip_mask, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * attn_prefill_check / attn_prefill_chunk_check / attn_decode_check - the
 * host-side argument validation of those entry points on its own: the same return code the
 * entry point would give before launching, with no HIP call at all.
 */
int attn_prefill_check(const void* q, const void* k, const void* v,
                       const float* o, const float* lse, int B, int Hq,
                       int Hkv, int N, int d, int causal, float tau,
                       const uint8_t* skip_mask);
int attn_prefill_chunk_check(const void* q, const void* k, const void* v,
                             const float* o, const float* lse, int B, int Hq,
                             int Hkv, int Nq, int N, int d, int causal,
                             float tau, const uint8_t* skip_mask);
int attn_decode_check(const void* q, const void* k, const void* v,
                      const float* o, const float* lse, int B, int Hq,
                      int Hkv, int L, int d, float tau,
                      const uint8_t* skip_mask, const void* workspace,
                      size_t workspace_bytes);

/*
 * attn_decode_sas - attn_decode with the Sparse Activated SoftMax
 * exponential (TurboAttention talk page, "Technical Deep Dive", its Sparse
 * Activated SoftMax part): inside each split every exponential of the
 * online softmax, the probabilities e^-(m - s) and the rescale factor when
 * a kept tile raises the running maximum m, is taken as T[n] p(f), with
 * n = floor(x), f = x - n for x = m - s in logits, T[n] = e^-n for n < 6
 * and 0 from 6 on, and p the least-squares polynomial of degree `degree`
 * (2 or 3) for e^-f on [0, 1]. The skip decisions, splits, merge, outputs,
 * mask and workspace are those of attn_decode; `degree` 0 is attn_decode
 * itself. Results depend on the order in which the running maximum rises
 * (the tiles are taken in ascending key order, as for the rule).
 * Errors as for attn_decode, and SKIPATTN_EINVAL for another degree.
 */
int attn_decode_sas(const void* q, const void* k, const void* v, float* o,
                    float* lse, int B, int Hq, int Hkv, int L, int d,
                    float tau, int degree, uint8_t* skip_mask,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_cap - attn_decode_sas over a KV cache allocated for `cap` keys
 * per (sequence, KV head), of which the first L are attended (a cache that
 * is appended to between decode steps):
 *   k, v  bf16 [B, Hkv, cap, d]   rows L .. cap - 1 are not read
 * cap >= L (SKIPATTN_EINVAL otherwise); `degree` 0 for exact exponentials,
 * 2 or 3 for SAS; the mask is [B, Hq, ceil(L/64)] and the workspace that of
 * attn_decode_workspace_bytes(B, Hq, L, d). attn_decode is the case
 * cap == L, degree == 0.
 */
int attn_decode_cap(const void* q, const void* k, const void* v, float* o,
                    float* lse, int B, int Hq, int Hkv, int L, int cap, int d,
                    float tau, int degree, uint8_t* skip_mask,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * 4-bit asymmetric KV cache (TurboAttention talk page, "Technical Deep Dive"
 * and its pre-fill / decoding workflow: the cache is stored and moved as
 * low-bit asymmetric integers with a floating zero point per block and is
 * turned back into numbers inside the attention kernel). The 4-bit width is
 * the one the talk calls near-lossless. Readings fixed by this library:
 *   - a K block is one key's row of d values; a V block is one channel of one
 *     64-key tile (the keys of that tile that exist);
 *   - per block: z = minimum; s = (maximum - z) / 15 in fp32, rounded up to
 *     the next bf16 value; code = clamp(rint((x - z) / s), 0, 15), subtract
 *     and divide in fp32 rounded to nearest even (0 when s == 0); the value
 *     the decode attends to is code * s + z, within s / 2 of x;
 *   - a 32-bit word holds 8 consecutive elements (consecutive d for K,
 *     consecutive keys for V): elements 0, 2, 4, 6 in nibbles 0..3 and
 *     elements 1, 3, 5, 7 in nibbles 4..7; a parameter word holds the bf16
 *     bits of s in its low half and of z in its high half.
 * Arrays (T = ceil(L / 64)), all 16-byte aligned:
 *   kq  uint8  [B, Hkv, L, d/2]       K codes, row by row
 *   kp  uint32 [B, Hkv, L]            K parameter word per key
 *   vq  uint8  [B, Hkv, T, d, 32]     V codes: per tile and channel, the 64
 *                                     keys' codes (keys past L: code 0)
 *   vp  uint32 [B, Hkv, T, d]         V parameter word per (tile, channel)
 * Inputs must be finite with |x| < 2^127.
 */

/*
 * attn_kv_quantize_q4 - K, V bf16 [B, Hkv, L, d] -> kq, kp, vq, vp (every
 * byte of the outputs is written). Errors as for attn_decode.
 */
int attn_kv_quantize_q4(const void* k, const void* v, uint8_t* kq, uint32_t* kp,
                        uint8_t* vq, uint32_t* vp, int B, int Hkv, int L,
                        int d, void* stream);

/*
 * attn_kv_quantize_q4_range - the same for keys k0 .. k1 - 1 only, into
 * arrays sized for a cache of L keys (K, V bf16 [B, Hkv, L, d] hold the
 * cache's bf16 keys and values; rows outside the range are not read).
 * k0 must be a multiple of 64. Every V tile that holds a key of the range
 * is written from its keys below k1, so appending a chunk and later
 * rewriting a partial tile with more keys gives the same bytes as one call
 * over the whole cache. 0 <= k0 <= k1 <= L.
 */
int attn_kv_quantize_q4_range(const void* k, const void* v, uint8_t* kq,
                              uint32_t* kp, uint8_t* vq, uint32_t* vp, int B,
                              int Hkv, int L, int d, int k0, int k1,
                              void* stream);

/*
 * attn_decode_q4 - attn_decode over a 4-bit cache: the same rule, splits,
 * outputs, mask and workspace (attn_decode_workspace_bytes), with the keys
 * and values taken as code * s + z from kq/kp and vq/vp (layout above).
 * Both products run on the exact codes with fp32 accumulation: q.K in bf16
 * (q as given), P.V in fp16 with the probabilities rounded to fp16 (times 16
 * on half of the keys, an exact scaling), and the row sum taken over the
 * same fp16 probabilities, so O is an exact weighted mean of the dequantised
 * values and the LSE moves by at most about 4e-4 from that rounding.
 */
int attn_decode_q4(const void* q, const uint8_t* kq, const uint32_t* kp,
                   const uint8_t* vq, const uint32_t* vp, float* o,
                   float* lse, int B, int Hq, int Hkv, int L, int d,
                   float tau, uint8_t* skip_mask, void* workspace,
                   size_t workspace_bytes, void* stream);
int attn_decode_q4_check(const void* q, const uint8_t* kq, const uint32_t* kp,
                         const uint8_t* vq, const uint32_t* vp,
                         const float* o, const float* lse, int B, int Hq,
                         int Hkv, int L, int d, float tau,
                         const uint8_t* skip_mask, const void* workspace,
                         size_t workspace_bytes);

/*
 * 2-bit asymmetric KV cache: the same talk's lossy but faster width. The
 * blocks, parameters and rounding are those of the 4-bit cache with 3 in
 * place of 15 (s = (maximum - z) / 3 rounded up to bf16, code = clamp(rint(
 * (x - z) / s), 0, 3)). A 32-bit word holds 16 consecutive elements:
 * elements 0, 2, .., 14 in the 2-bit fields 0..7 of bits 0-15 and elements
 * 1, 3, .., 15 in those of bits 16-31. Arrays (T = ceil(L / 64)), all
 * 16-byte aligned:
 *   kq  uint8  [B, Hkv, L, d/4]       K codes, row by row
 *   kp  uint32 [B, Hkv, L]            K parameter word per key
 *   vq  uint8  [B, Hkv, T, d, 16]     V codes: per tile and channel, the 64
 *                                     keys' codes (keys past L: code 0)
 *   vp  uint32 [B, Hkv, T, d]         V parameter word per (tile, channel)
 * The quantisers and the decode take the arguments, follow the rules and
 * return the errors of their 4-bit counterparts. In the decode, P.V runs on
 * fp16 probabilities scaled by 64, 16, 4 or 1 (exact) per key, with the
 * same bound on the LSE.
 */
int attn_kv_quantize_q2(const void* k, const void* v, uint8_t* kq, uint32_t* kp,
                        uint8_t* vq, uint32_t* vp, int B, int Hkv, int L,
                        int d, void* stream);
int attn_kv_quantize_q2_range(const void* k, const void* v, uint8_t* kq,
                              uint32_t* kp, uint8_t* vq, uint32_t* vp, int B,
                              int Hkv, int L, int d, int k0, int k1,
                              void* stream);
int attn_decode_q2(const void* q, const uint8_t* kq, const uint32_t* kp,
                   const uint8_t* vq, const uint32_t* vp, float* o,
                   float* lse, int B, int Hq, int Hkv, int L, int d,
                   float tau, uint8_t* skip_mask, void* workspace,
                   size_t workspace_bytes, void* stream);
int attn_decode_q2_check(const void* q, const uint8_t* kq, const uint32_t* kp,
                         const uint8_t* vq, const uint32_t* vp,
                         const float* o, const float* lse, int B, int Hq,
                         int Hkv, int L, int d, float tau,
                         const uint8_t* skip_mask, const void* workspace,
                         size_t workspace_bytes);

/*
 * attn_decode_q4_sas, attn_decode_q2_sas - attn_decode_q4 and
 * attn_decode_q2 with the SAS exponential of attn_decode_sas (the quantised
 * KV cache and SAS together, as in the talk's decoding workflow); `degree`
 * 2 or 3, 0 for exact exponentials. Arguments and errors as for the
 * quantised decodes, and SKIPATTN_EINVAL for another degree.
 */
int attn_decode_q4_sas(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o,
                       float* lse, int B, int Hq, int Hkv, int L, int d,
                       float tau, int degree, uint8_t* skip_mask,
                       void* workspace, size_t workspace_bytes, void* stream);
int attn_decode_q2_sas(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o,
                       float* lse, int B, int Hq, int Hkv, int L, int d,
                       float tau, int degree, uint8_t* skip_mask,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_q4_cap, attn_decode_q2_cap - the quantised decodes over cache
 * arrays sized for `cap` keys (the shapes above with cap in place of L, as
 * written by attn_kv_quantize_q4_range / _q2_range with L = cap), of which
 * the first L keys are attended: a cache appended to chunk by chunk and
 * decoded at its current length. cap >= L (SKIPATTN_EINVAL otherwise);
 * `degree` as for attn_decode_q4_sas; other arguments, results and errors as
 * for attn_decode_q4 / attn_decode_q2 (the case cap == L).
 */
int attn_decode_q4_cap(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o,
                       float* lse, int B, int Hq, int Hkv, int L, int cap,
                       int d, float tau, int degree, uint8_t* skip_mask,
                       void* workspace, size_t workspace_bytes, void* stream);
int attn_decode_q2_cap(const void* q, const uint8_t* kq, const uint32_t* kp,
                       const uint8_t* vq, const uint32_t* vp, float* o,
                       float* lse, int B, int Hq, int Hkv, int L, int cap,
                       int d, float tau, int degree, uint8_t* skip_mask,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Hybrid 2/4-bit KV cache (TurboAttention talk page, "Technical Deep Dive":
 * the cache keeps its less critical parts at 2 bits and its more important
 * parts at 4). The talk gives no rule for which parts are which; here the
 * unit is the KV head and the caller chooses: kv_bits is a HOST array of
 * Hkv bytes, kv_bits[g] = 4 or 2 the width of KV head g (any other value:
 * SKIPATTN_EINVAL). Hkv <= 256 (SKIPATTN_EUNSUPPORTED beyond). The heads of
 * each width live in arrays of their own, in increasing head order: with
 * H4 heads at 4 bits and H2 at 2 bits, (kq4, kp4, vq4, vp4) is a 4-bit
 * cache of H4 heads (layout of attn_kv_quantize_q4 with Hkv = H4) and
 * (kq2, kp2, vq2, vp2) a 2-bit cache of H2 heads (Hkv = H2); a width with
 * no head takes NULL pointers. Every head's codes are byte-identical to
 * those of the single-width quantiser of its width.
 *
 * attn_kv_quantize_hybrid(_range) - K, V bf16 [B, Hkv, L, d] -> the two
 * caches; key ranges, errors and the rewriting of partial tiles as for
 * attn_kv_quantize_q4(_range). Every check is made before the first launch.
 *
 * attn_decode_hybrid - attn_decode over a hybrid cache: q, o, lse, the mask
 * and the workspace (attn_decode_workspace_bytes(B, Hq, L, d)) are those of
 * attn_decode over all Hq query heads; the query heads of KV head g attend
 * to its keys and values as stored at kv_bits[g] bits, with the products,
 * rule and rounding of attn_decode_q4 or attn_decode_q2. The two widths run
 * as two split launches into one set of per-split partials, then one merge.
 * attn_decode_hybrid_cap - the same over arrays sized for `cap` keys, of
 * which the first L are attended, with `degree` as for attn_decode_q4_sas.
 */
int attn_kv_quantize_hybrid(const void* k, const void* v, const uint8_t* kv_bits,
                            uint8_t* kq4, uint32_t* kp4, uint8_t* vq4,
                            uint32_t* vp4, uint8_t* kq2, uint32_t* kp2,
                            uint8_t* vq2, uint32_t* vp2, int B, int Hkv, int L,
                            int d, void* stream);
int attn_kv_quantize_hybrid_range(const void* k, const void* v,
                                  const uint8_t* kv_bits, uint8_t* kq4,
                                  uint32_t* kp4, uint8_t* vq4, uint32_t* vp4,
                                  uint8_t* kq2, uint32_t* kp2, uint8_t* vq2,
                                  uint32_t* vp2, int B, int Hkv, int L, int d,
                                  int k0, int k1, void* stream);
int attn_decode_hybrid(const void* q, const uint8_t* kv_bits,
                       const uint8_t* kq4, const uint32_t* kp4,
                       const uint8_t* vq4, const uint32_t* vp4,
                       const uint8_t* kq2, const uint32_t* kp2,
                       const uint8_t* vq2, const uint32_t* vp2, float* o,
                       float* lse, int B, int Hq, int Hkv, int L, int d,
                       float tau, uint8_t* skip_mask, void* workspace,
                       size_t workspace_bytes, void* stream);
int attn_decode_hybrid_cap(const void* q, const uint8_t* kv_bits,
                           const uint8_t* kq4, const uint32_t* kp4,
                           const uint8_t* vq4, const uint32_t* vp4,
                           const uint8_t* kq2, const uint32_t* kp2,
                           const uint8_t* vq2, const uint32_t* vp2, float* o,
                           float* lse, int B, int Hq, int Hkv, int L, int cap,
                           int d, float tau, int degree, uint8_t* skip_mask,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * attn_decode_noalloc - attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, kernels, results and errors, with
 * no workspace argument. The per-split partials go to a device scratch array
 * inside the library, SKIPATTN_DECODE_SCRATCH_BYTES (32 MiB) on each GPU it
 * runs on, held until the process ends; a call whose partials would need
 * more (attn_decode_workspace_bytes(B, Hq, L, d) > 32 MiB; decode at B = 16,
 * Hq = 64, L = 131072, d = 128 needs 16.9 MB) returns SKIPATTN_EWORKSPACE
 * before any launch. The call allocates and frees nothing. Every call on a
 * GPU shares that GPU's scratch: calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller. No
 * scratch content carries over between calls (each call writes every
 * partial it reads). The first call on a device looks up the scratch's
 * address there (SKIPATTN_EHIP if that fails).
 */
#define SKIPATTN_DECODE_SCRATCH_BYTES (32u << 20)
int attn_decode_noalloc(const void* q, const void* k, const void* v, float* o,
                        float* lse, int B, int Hq, int Hkv, int L, int d,
                        float tau, uint8_t* skip_mask, void* stream);

/* Text for the last nonzero return on this thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SKIPATTN_H */
