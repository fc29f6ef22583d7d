/* kv8 -- fp8 e4m3 latent KV cache for multi-head latent attention on MI355X.
 *
 * C ABI of libkv8.so (hand-written HIP for gfx950).  The operations follow
 * the page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
 * (colibri pull request #299), cited below as [colibri#299]:
 *
 *   commit message, first paragraph: the MLA latent rows -- Lc (kv_lora) and
 *     Rc (qk_rope) -- are stored as fp8 e4m3 bytes with a per-row f32
 *     amax/448 scale; the latent is both key and value of the absorbed
 *     attention.
 *   commit message, kv_fp8.h item: round-to-nearest-even encoder saturating
 *     at +-448, keeping the sign of zero and storing NaN as an inert 0; the
 *     per-row quantizer guards an amax so small that 448/amax overflows.
 *   commit message, attention_rows item: the producer quantizes each fresh
 *     row instead of copying f32; the absorbed score and context loops
 *     dequantize inline with the row scale applied outside the dot product.
 *   PR description: one f32 scale each for the Lc and the Rc row; a follow-up
 *     adds split-T kernels for long slots.
 *
 * Element format: OCP 8-bit floating point, E4M3 (bias 7, no infinities,
 * NaN = S.1111.111, largest finite 448, subnormals m * 2^-9).
 *
 * Cache layout (device memory, owned by the caller):
 *   codes  uint8 [n_cache_rows][kv_lora + rope], row-major, one token row per
 *          cache row: the kv_lora Lc codes, then the rope Rc codes;
 *   scales f32   [n_cache_rows][2]: scales[r][0] for Lc, scales[r][1] for Rc.
 *   A token occupies kv_lora + rope + 8 bytes per layer (584 for 512 + 64).
 *
 * Conventions for every call:
 *   - every pointer argument is a DEVICE pointer owned by the caller, except
 *     where stated; buffers must stay valid until the stream has finished;
 *   - `stream` is a hipStream_t (NULL = the default stream); calls are
 *     asynchronous on it and never synchronize the host;
 *   - bf16 values are passed as their uint16_t bit patterns;
 *   - the kernel calls keep no results between calls.  One call allocates:
 *     kv8_absorb_decode takes stream-ordered device memory for its split
 *     partials from a memory pool of the library's own (one per device,
 *     created on the first such call on it) and returns it to that pool on
 *     the same stream before returning (its signature has no workspace); the
 *     pool keeps that memory for later calls until the process ends.  Every
 *     other call runs on caller memory only; kv8_absorb_decode_splitT, the
 *     two-stage form and kv8_absorb_decode_noalloc are the allocation-free
 *     decode calls;
 *   - argument errors are reported synchronously through the return value
 *     and nothing is launched; data is never an error (NaN, inf, zero and
 *     subnormal values have defined results); nothing aborts or prints.
 *
 * Supported shapes: kv_lora = 512, rope = 64, Q*H <= 2^21 query rows per
 * sequence (other values return KV8_EUNSUPPORTED).
 */
#ifndef KV8_H
#define KV8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KV8_OK = 0,
    KV8_EINVAL = -1,        /* bad argument: null pointer, negative size, bad alignment */
    KV8_EUNSUPPORTED = -2,  /* valid but unsupported shape (kv_lora != 512, rope != 64) */
    KV8_ELAUNCH = -3,       /* a HIP launch or runtime call failed */
    KV8_EWORKSPACE = -4,    /* split-T workspace missing or too small */
    KV8_ENOMEM = -5,        /* a device allocation failed */
    KV8_EIO = -6,           /* a file system call failed (kv8_pool.h stores) */
    KV8_EFORMAT = -7        /* not a kv8 store, torn header, or other dimensions */
} kv8_status;

/* Quantize f32 latent token rows into the fp8 cache ([colibri#299] commit
 * message, kv_fp8.h and attention_rows items; PR description).
 *
 * src            f32 [n_rows][src_row_stride]; row i holds kv_lora Lc values
 *                then rope Rc values (further columns are ignored).  src must
 *                be 16-byte aligned and src_row_stride a multiple of 4,
 *                >= kv_lora + rope.
 * n_rows         rows to quantize (0 is a no-op).
 * codes, scales  the cache (layout above); row i is written to cache row
 *                dst_rows[i], or to row i when dst_rows is NULL.  codes must
 *                be 4-byte and scales 8-byte aligned.
 * dst_rows       int64 [n_rows] device array or NULL.  Rows must be distinct
 *                and inside the cache (not checked: they are device data).
 *
 * Per segment x (Lc, then Rc): amax = max |x_j| over finite entries (0 if
 * none); inv = fl32(448 / amax); if inv is +inf the segment is guarded:
 * scale = +0 and inv = 0; otherwise scale = fl32(amax / 448).  Each code is
 * the saturating round-to-nearest-even e4m3 encoding of fl32(x_j * inv):
 * |q| >= 448 (and +-inf) -> +-448 (0x7E | sign), sign of zero kept, NaN ->
 * 0x00.  Results are bit-identical to this definition. */
int kv8_quantize_rows(const float* src, int64_t src_row_stride, int64_t n_rows,
                      int32_t kv_lora, int32_t rope,
                      uint8_t* codes, float* scales, const int64_t* dst_rows,
                      void* stream);

/* Block-scaled (MX) variant of the quantizer: e4m3 elements with one
 * power-of-two scale per 32 values instead of one f32 scale per segment (the
 * e4m3 bytes + ue8m0 exponents of the mxfp8 format on the page "Phase 0
 * toward V4.1 on a 128 GB Mac: lossless mxfp8 residents and kill-test
 * tooling" (keep PR #3), mxfp8 residents paragraph): 594 bytes per token and
 * layer, 8.25 bits per value.
 *
 * src, src_row_stride, n_rows, codes, dst_rows   as kv8_quantize_rows.
 * exps     uint8 [*][(kv_lora + rope) / 32]: block b of cache row r has the
 *          scale 2^(exps[r][b] - 127) (a ue8m0 byte).
 * Per block of 32 values: amax over finite entries (0 if none); E = the
 * smallest integer with amax <= 448 * 2^E, clamped to [-127, 127] (no finite
 * value saturates); each code is the encoder of kv8_quantize_rows applied to
 * x * 2^-E.  Results are bit-identical to this definition. */
int kv8_quantize_rows_mx(const float* src, int64_t src_row_stride, int64_t n_rows,
                         int32_t kv_lora, int32_t rope, uint8_t* codes, uint8_t* exps,
                         const int64_t* dst_rows, void* stream);

/* The producer step fused with the quantizer ([colibri#299] commit message,
 * attention_rows item: the producer quantizes the fresh normalised and
 * rotary-embedded latent row in place of the f32 copy).  The page names the
 * two steps but not their form; this call takes the standard ones:
 *
 *   Lc: y_j = w_j x_j / sqrt(mean_k x_k^2 + eps)   (RMS normalisation);
 *   Rc: the interleaved pairs (2i, 2i+1), i < rope/2, are rotated by the angle
 *       a_i = fl32(fl32(pos) f_i), f_i = fl32(rope_theta^(-2i/rope)):
 *       y_2i = x_2i cos a_i - x_2i+1 sin a_i, y_2i+1 = x_2i sin a_i + x_2i+1 cos a_i;
 *
 * and y is then quantized and stored exactly as kv8_quantize_rows does with
 * y for the source row.  y is computed in f32 (sum of squares reduced in f32,
 * f32 sincos), so a code may differ by one step from the quantization of the
 * exact y where that value lies next to a rounding boundary.
 *
 * src, src_row_stride, n_rows, codes, scales, dst_rows   as kv8_quantize_rows.
 * norm_weight    f32 [kv_lora] device array, 16-byte aligned.
 * eps            >= 0 and finite.
 * positions      int64 [n_rows] device array, 8-byte aligned: the token
 *                position of each row.
 * rope_theta     > 0 and finite (e.g. 10000).
 * Returns KV8_EINVAL for a bad argument, KV8_EUNSUPPORTED unless kv_lora is
 * 512 and rope 64, KV8_ELAUNCH when the launch fails. */
int kv8_norm_rope_quantize_rows(const float* src, int64_t src_row_stride, int64_t n_rows,
                                int32_t kv_lora, int32_t rope, const float* norm_weight,
                                float eps, const int64_t* positions, float rope_theta,
                                uint8_t* codes, float* scales, const int64_t* dst_rows,
                                void* stream);

/* Absorbed-MLA decode straight from the fp8 rows ([colibri#299] commit
 * message, first paragraph and attention_rows item).
 *
 * q_lat          bf16 [B][Q][H][kv_lora]  (queries already absorbed into the
 *                latent space), 16-byte aligned.
 * q_rope         bf16 [B][Q][H][rope], 16-byte aligned.
 * codes, scales  the cache; codes 16-byte aligned.
 * kv_start       int64 [B]: first cache row of sequence b.
 * kv_len         int32 [B]: rows of sequence b, including its Q newest ones;
 *                0 <= kv_len[b] <= max_len.
 * max_len        host-side upper bound of kv_len (sizes the launch).
 * B, Q, H        sequences, query positions per sequence, heads (>= 1).
 * softmax_scale  f32 multiplier of the scores (e.g. 1/sqrt(576)).
 * out            f32 [B][Q][H][kv_lora], 16-byte aligned: the normalised
 *                latent context (before any value up-projection).
 *
 * Query i of sequence b attends its first n = kv_len[b] - (Q-1) + i rows
 * (causal multi-token decode); n <= 0 gives a zero output.  For every
 * visible row t: s_t = softmax_scale * (scale_Lc[t] * (q_lat . dec(Lc_t)) +
 * scale_Rc[t] * (q_rope . dec(Rc_t))); out = sum_t softmax(s)_t *
 * scale_Lc[t] * dec(Lc_t).  Long sequences are split internally and merged
 * by log-sum-exp.
 *
 * Accuracy (every finite cache and query, any row magnitude): the score
 * products are exact products of the dequantized rows and the queries,
 * summed in f32, where each query row enters as two e4m3 terms whose sum
 * equals every bf16 element of at least 2^-9 of the row's largest magnitude
 * (every element of rows below 2^-119) and is within 2^-17 of that largest
 * magnitude for the others; scores are formed relative to the largest row
 * scale of the token range, so they stay finite for rows up to the f32
 * maximum.  A query row with a NaN or infinite element gives a NaN output
 * row (other rows are unaffected).
 * The probabilities enter the context pass as fp16 relative to the range's
 * largest Lc scale; a range whose Lc scales differ by more than 2^6 is run
 * watched, and a query row whose largest probability operand falls below
 * 2^-6 is run again with its operands shifted by up to 2^100, so precision is
 * lost only when the rows carrying a query's weight have Lc scales more than
 * 2^100 below the largest one of their range.  Each row's probability
 * operand is rounded to fp16 once (relative error <= 2^-11); these errors
 * average out over rows, except when many rows with the same scale and weight
 * cancel each other in the weighted average, where the error relative to the
 * output grows with the cancellation factor sum_t w_t |V_t| / |sum_t w_t V_t|.
 * Weights below 2^-149 of a query row's largest weight are dropped (f32
 * underflow).  A split adds one 16-bit rounding of each range's normalised
 * context (see the two-stage form below). */
int kv8_absorb_decode(const uint16_t* q_lat, const uint16_t* q_rope,
                      const uint8_t* codes, const float* scales,
                      const int64_t* kv_start, const int32_t* kv_len, int32_t max_len,
                      int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                      float softmax_scale, float* out, void* stream);

/* Size of the static device array kv8_absorb_decode_noalloc keeps its split
 * partials in (64 MiB per device the library runs on, held until the process
 * ends). */
#define KV8_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kv8_absorb_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, split plan, kernels and results, but the
 * split partials live in a static device array of KV8_NOALLOC_SCRATCH_BYTES
 * instead of stream-ordered memory; the call allocates nothing.  The array's
 * device address is looked up on the first call on each device (with that
 * device current; `stream` must belong to the current device).
 * Returns KV8_EWORKSPACE when the plan's partials,
 * kv8_partials_bytes(B, Q, H, kv_lora, n) with n from kv8_decode_plan, exceed
 * KV8_NOALLOC_SCRATCH_BYTES (e.g. B*Q*H*n above 64,527 rows x ranges), and
 * KV8_ELAUNCH when the address lookup fails.  Every call on one device shares
 * its array: calls that overlap on one device (different streams, or host
 * threads) race and must be serialised by the caller.  No part of the array
 * needs clearing between calls (every value a call reads was written by the
 * same call, or is given weight 0). */
int kv8_absorb_decode_noalloc(const uint16_t* q_lat, const uint16_t* q_rope,
                              const uint8_t* codes, const float* scales,
                              const int64_t* kv_start, const int32_t* kv_len, int32_t max_len,
                              int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                              float softmax_scale, float* out, void* stream);

/* Bytes of workspace kv8_absorb_decode_splitT needs for these shapes. */
size_t kv8_splitT_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t kv_lora,
                                  int32_t num_splits);

/* Split-T decode ([colibri#299] PR description, follow-up paragraph: split-T
 * kernels for long slots).  Same arguments and result as kv8_absorb_decode;
 * the rows [0, kv_len[b]) of every sequence are cut into num_splits equal
 * ranges of ceil(kv_len[b] / num_splits) rows (the last ones may be short or
 * empty), each range yields a partial softmax (reference maximum, sum,
 * weighted context), and the partials are merged by log-sum-exp.  When
 * B * ceil(Q*H/128) * num_splits is below the number of compute units, each
 * range is further cut into equal sub-ranges so that every compute unit has
 * one; their partials enter the same merge.  workspace is a
 * caller-owned device buffer of at least
 * kv8_splitT_workspace_bytes(B, Q, H, kv_lora, num_splits) bytes, 256-byte
 * aligned; its contents on entry do not matter. */
int kv8_absorb_decode_splitT(const uint16_t* q_lat, const uint16_t* q_rope,
                             const uint8_t* codes, const float* scales,
                             const int64_t* kv_start, const int32_t* kv_len, int32_t max_len,
                             int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                             float softmax_scale, float* out,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Absorbed decode over block-scaled (MX) rows (codes and exponents from
 * kv8_quantize_rows_mx): the same arguments, ranges, workspace and result as
 * kv8_absorb_decode_splitT, with exps (uint8 [*][(kv_lora + rope) / 32],
 * 4-byte aligned, block b of row r scaled by 2^(exps[r][b] - 127)) in place
 * of the scales: s_t = softmax_scale * (q_lat . xhat_Lc[t] + q_rope .
 * xhat_Rc[t]), out = sum_t softmax(s)_t xhat_Lc[t], xhat = decode(code) *
 * 2^(exp - 127).  The kernel of kv8_absorb_decode runs it: each row's largest
 * Lc and Rc block exponents act as its two scales, and its codes enter the
 * fp16 operands times 2^(E_block - E_largest), exact for blocks within 2^15
 * of their segment's largest (smaller blocks round to fp16 subnormals, an
 * error below 2^-15 of that segment's largest values); everything else,
 * accuracy included, is as for the per-row scales.  The copies read the
 * exponent array's last 4-byte word whole.  workspace: kv8_mx_workspace_bytes
 * (the same partials as kv8_absorb_decode_splitT). */
size_t kv8_mx_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t kv_lora,
                              int32_t num_splits);
int kv8_absorb_decode_mx(const uint16_t* q_lat, const uint16_t* q_rope,
                         const uint8_t* codes, const uint8_t* exps,
                         const int64_t* kv_start, const int32_t* kv_len, int32_t max_len,
                         int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                         float softmax_scale, float* out,
                         int32_t num_splits, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---- Two-stage form of the decode (used by kv8_absorb_decode itself) ----
 * Stage 1 writes one partial softmax per (token range, sequence, query row);
 * stage 2 merges the partials by log-sum-exp.  Partials of several devices
 * holding different token ranges of one sequence can be merged the same way.
 *
 * Partials buffer (device, caller-owned, 256-byte aligned), R = Q*H:
 *   V  int16 [num_splits][B][R][kv_lora]  codes of the range's normalised
 *                                         context V = O / l, with
 *                                         O = sum_t 2^(c (x_t - m)) scale_Lc[t] dec(Lc_t)
 *   st 16-byte records [num_splits][B][R] { double m; float l; float v_scale; }:
 *                                         m = reference score (f64),
 *                                         l = sum_t 2^(c (x_t - m)),
 *                                         v_scale = scale of the codes
 * (st follows V directly).  V of a row is code * v_scale, with the codes
 * rounded from 32767 V / max |V| over the row (max |V| = 32767 v_scale; a
 * row with V = 0 has v_scale = 0): 16 bits per value with an absolute error
 * of at most max |V| / 65534 on each.  V stays within the range of the rows'
 * values, so every field is finite for every finite cache.  With
 * x_t = q_lat . xhat_Lc[t] + q_rope . xhat_Rc[t] (before softmax_scale),
 * c = softmax_scale * log2(e); a range with no visible row has m = l =
 * v_scale = 0 and its codes are not written (the merge gives it weight 0).
 * The merge passes the codes' error on as at most max_s max|V_s| / 65534 per
 * output value: below 1e-3 of the largest output as long as no range's
 * normalised context exceeds the largest output by more than 65x (that only
 * happens when ranges cancel each other in the merged average). */

/* Bytes of a partials buffer for these shapes. */
size_t kv8_partials_bytes(int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t num_splits);

/* The split kv8_absorb_decode chooses for these shapes: *num_splits ranges of
 * *split_tokens rows each (num_splits == 1: no split, direct output). */
int kv8_decode_plan(int32_t B, int32_t Q, int32_t H, int32_t max_len,
                    int32_t* split_tokens, int32_t* num_splits);

/* Stage 1.  Range s of sequence b is rows [s*k, (s+1)*k) of the sequence with
 * k = split_tokens, or k = ceil(kv_len[b] / num_splits) when split_tokens is
 * 0.  A fixed split must cover max_len (split_tokens * num_splits >= max_len,
 * else KV8_EINVAL).  Other arguments as kv8_absorb_decode. */
int kv8_absorb_decode_partials(const uint16_t* q_lat, const uint16_t* q_rope,
                               const uint8_t* codes, const float* scales,
                               const int64_t* kv_start, const int32_t* kv_len, int32_t max_len,
                               int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                               float softmax_scale, int32_t split_tokens, int32_t num_splits,
                               void* partials, size_t partials_bytes, void* stream);

/* Stage 2 ([colibri#299] PR description, follow-up: split-T kernels):
 * out[b][r] = sum_s w_s l_s V_s / sum_s w_s l_s over ranges with l_s > 0,
 * w_s = 2^(c (m_s - m*)), m* the reference with the largest c m_s; zero when
 * no range saw a row.  partials_bytes (the buffer's size) must be at least
 * kv8_partials_bytes(B, Q, H, kv_lora, num_splits), else KV8_EWORKSPACE. */
int kv8_lse_merge(const void* partials, size_t partials_bytes, int32_t B, int32_t Q, int32_t H,
                  int32_t kv_lora, int32_t num_splits, float softmax_scale, float* out,
                  void* stream);

/* The non-absorbed consumer of the cache rows ([colibri#299] commit message,
 * attention_rows item: the non-absorbed prefill dequantizes Lc into a staging
 * row for the kv_b matmul and reads Rc via the decode table):
 *
 *   out[m][n]      = bf16( s_Lc[m] * sum_k decode(codes[m][k]) * W[n][k] ),  k < kv_lora
 *   rope_out[m][j] = s_Rc[m] * decode(codes[m][kv_lora + j]),               j < rope
 *
 * codes, scales  n_rows consecutive cache rows (layout above), codes 16-byte
 *                aligned (pass the cache pointers offset to the first row).
 * w_kv_b         bf16 [N][kv_lora] device array, 16-byte aligned: row n holds
 *                output column n's weights (a linear layer's weight layout).
 * N              output columns, a multiple of 128 (KV8_EUNSUPPORTED otherwise).
 * out            bf16 [n_rows][N], 16-byte aligned; the products are summed in f32 (bf16 MFMA;
 *                every e4m3 value is exact in bf16) and the scaled sum is
 *                rounded to nearest even.
 * rope_out       f32 [n_rows][rope], 16-byte aligned, or NULL to skip.
 * Returns KV8_EINVAL for a bad argument, KV8_EUNSUPPORTED unless kv_lora is 512,
 * rope 64 and N a multiple of 128, KV8_ELAUNCH when the launch fails. */
int kv8_project_rows(const uint8_t* codes, const float* scales, int64_t n_rows, int32_t kv_lora,
                     int32_t rope, const uint16_t* w_kv_b, int32_t N, uint16_t* out,
                     float* rope_out, void* stream);

/* kv8_project_rows with f32 output, the f32 staging the page's kv_b matmul
 * takes: out[m][n] = s_Lc[m] * sum_k decode(codes[m][k]) * W[n][k], the f32
 * sum of the exact bf16 products times the row scale, not rounded further.
 * out f32 [n_rows][N], 16-byte aligned; every other argument, the rope
 * output and the status codes as kv8_project_rows. */
int kv8_project_rows_f32(const uint8_t* codes, const float* scales, int64_t n_rows, int32_t kv_lora,
                         int32_t rope, const uint16_t* w_kv_b, int32_t N, float* out,
                         float* rope_out, void* stream);

/* Human-readable name of a kv8_status value (static string, never NULL). */
const char* kv8_status_string(int status);

/* ---- Verification entry points (same device code as the calls above) ---- */

/* out[k] = e4m3 code of the f32 value whose bit pattern is first + k, for
 * k < count (count <= 2^32 - first).  encoder 0: the encoder kv8_quantize_rows
 * uses (the gfx950 fp8 conversion after a clamp to +-448 and NaN -> +0);
 * encoder 1: an integer bit-math encoder of the same rules ([colibri#299]
 * commit message, kv_fp8.h item: round-to-nearest-even bit-math encoder),
 * kept as a second, independent device implementation.  out must be 4-byte
 * aligned; other encoder values return KV8_EINVAL. */
int kv8_encode_bits(uint32_t first, uint64_t count, int32_t encoder, uint8_t* out, void* stream);

/* Decode n codes with the exact conversions the decode kernels use:
 * out_bf16[k], out_f16[k] = bit patterns of dec(codes[k]) as bf16 and fp16. */
int kv8_decode_codes(const uint8_t* codes, int64_t n, uint16_t* out_bf16, uint16_t* out_f16,
                     void* stream);

/* ---- Measurement ---- */

/* The shader clock, in MHz, of the current device while every SIMD runs a
 * chain of fp16 MFMAs for about busy_us microseconds (1..100000): the median
 * over blocks of (shader-clock counter delta / wall-clock counter delta) times
 * the wall clock's rate.  MI355X's dense MFMA peaks are quoted at its 2.4 GHz
 * peak engine clock; this is the clock matrix-core-bound kernels actually get.
 * Allocates and frees a small device buffer, synchronizes the stream.
 * KV8_EINVAL for a bad argument, KV8_ENOMEM, KV8_ELAUNCH. */
int kv8_shader_clock_mhz(int32_t busy_us, double* mhz, void* stream);

/* HBM floor of a kernel's traffic: one launch that reads bytes0 at src0 and
 * bytes1 at src1 and writes dst_bytes at dst (content unspecified) with plain
 * 16-byte grid-stride loads and stores, nothing else.  Sizes multiples of 16,
 * pointers 16-byte aligned when their size is non-zero (else KV8_EINVAL).
 * Asynchronous on stream; KV8_ELAUNCH when the launch fails. */
int kv8_stream_floor(const void* src0, uint64_t bytes0, const void* src1, uint64_t bytes1,
                     void* dst, uint64_t dst_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KV8_H */
