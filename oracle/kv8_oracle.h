/* kv8 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of what the fp8 e4m3 latent
 * KV cache computes.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library; the product path never does.  It
 * shares no code, header, table or constant generator with the HIP library.
 *
 * Subject page: "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
 * (colibri pull request #299), cited below as [colibri#299].  The element
 * format is OCP 8-bit floating point, E4M3 variant (no infinities, one NaN
 * mantissa pattern per sign, max finite 448), cited as [OFP8 E4M3].
 *
 * Every function here is pinned by CPU tests against closed forms, invariants,
 * a library conversion routine and brute force; none is "parity unpinned".
 */
#ifndef KV8_ORACLE_H
#define KV8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Value of one e4m3 code, from the [OFP8 E4M3] formula (not a typed table).
 * Codes 0x7F and 0xFF are NaN. */
double orc_decode(uint8_t code);

/* Saturating round-to-nearest-even encoder, [colibri#299] commit message,
 * kv_fp8.h item: nearest finite e4m3 value, ties to the even code, magnitudes
 * >= 448 (and +-inf) give +-448, the sign of zero is kept, NaN gives 0x00. */
uint8_t orc_encode(float q);

/* Encode the f32 values whose bit patterns are first, first+1, ...,
 * first+count-1 (count may reach 2^32).  threads <= 0: all hardware threads. */
void orc_encode_bits_range(uint64_t first, uint64_t count, uint8_t* out, int threads);

/* Encode n arbitrary f32 values. */
void orc_encode_array(const float* in, int64_t n, uint8_t* out, int threads);

/* Per-segment quantizer of one row segment (amax over finite entries,
 * inv = 448/amax in f32, guard when inv overflows to +inf, scale = amax/448,
 * codes = E(x*inv)).  Writes w codes and returns the scale. */
float orc_quantize_segment(const float* x, int32_t w, uint8_t* codes);

/* Token rows: [kv_lora | rope] floats each, with row stride src_row_stride
 * floats.  Row i goes to cache row dst_rows[i] (or i when dst_rows is NULL):
 * codes[dst][0..kv_lora+rope), scales[dst][0] = Lc scale, [1] = Rc scale. */
void orc_quantize_rows(const float* src, int64_t src_row_stride, int64_t n_rows,
                       int32_t kv_lora, int32_t rope, uint8_t* codes, float* scales,
                       const int64_t* dst_rows, int threads);

/* Absorbed-MLA decode over the dequantized fp8 rows, f64 throughout.
 * q_lat bf16 bits [B,Q,H,kv_lora], q_rope bf16 bits [B,Q,H,rope];
 * sequence b owns cache rows kv_start[b] .. kv_start[b]+kv_len[b]-1; query i
 * of sequence b sees its first kv_len[b]-(Q-1)+i rows (zero output when that
 * count is <= 0).  out f64 [B,Q,H,kv_lora] = softmax(s * q . xhat) . xhat_Lc,
 * xhat = decode(code) * segment scale.
 * sel: optional list of n_sel flat (b*Q+i)*H+h indices; when given, only those
 * output rows are computed and written compactly to out[n_sel][kv_lora].
 * num_splits > 1 evaluates each output row as num_splits partial softmaxes over
 * equal token ranges merged by log-sum-exp (the split-T decomposition).
 * Returns 0, or -1 on bad arguments. */
int orc_attention(const uint16_t* q_lat, const uint16_t* q_rope,
                  const uint8_t* codes, const float* scales,
                  const int64_t* kv_start, const int32_t* kv_len,
                  int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                  float softmax_scale, int32_t num_splits,
                  const int64_t* sel, int64_t n_sel, double* out, int threads);

/* The same attention over raw f32 rows (the KV8=0 path of [colibri#299]):
 * rows [*, row_stride] floats, first kv_lora are Lc, next rope are Rc. */
int orc_attention_f32rows(const uint16_t* q_lat, const uint16_t* q_rope,
                          const float* rows, int64_t row_stride,
                          const int64_t* kv_start, const int32_t* kv_len,
                          int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                          float softmax_scale, int32_t num_splits,
                          const int64_t* sel, int64_t n_sel, double* out, int threads);

/* The producer step in front of the quantizer ([colibri#299] commit message,
 * attention_rows item: the producer quantizes the fresh normalised and
 * rotary-embedded latent row).  The page names both steps but not their form;
 * this takes the standard ones, computed in f64 and rounded to f32 once:
 *   Lc (kv_lora values): RMS normalisation with a per-channel weight,
 *     y_j = w_j x_j / sqrt(mean_k x_k^2 + eps);
 *   Rc (rope values, even): rotary embedding of the interleaved pairs
 *     (2i, 2i+1), i < rope/2, by the angle a_i = fl32(fl32(pos) f_i) with the
 *     f32 frequency f_i = fl32(theta^(-2i/rope)):
 *     y_2i = x_2i cos a_i - x_2i+1 sin a_i,  y_2i+1 = x_2i sin a_i + x_2i+1 cos a_i.
 * src rows have stride src_row_stride floats; out is [n_rows][kv_lora+rope]
 * f32.  The row then goes to orc_quantize_rows unchanged. */
void orc_norm_rope_rows(const float* src, int64_t src_row_stride, int64_t n_rows,
                        int32_t kv_lora, int32_t rope, const float* norm_weight, float eps,
                        const int64_t* positions, float rope_theta, float* out, int threads);

/* The non-absorbed consumer of the same rows ([colibri#299] commit message,
 * attention_rows item: the non-absorbed prefill dequantizes Lc into a staging
 * row for the kv_b matmul and reads Rc through the decode table), in f64:
 *   out[m][n]  = s_Lc[m] * sum_k decode(code[m][k]) * W[n][k],  k < kv_lora,
 *   rope[m][j] = s_Rc[m] * decode(code[m][kv_lora + j]),       j < rope,
 * for the n_rows cache rows codes[0..n_rows), scales[0..n_rows) and a bf16
 * weight W[N][kv_lora] (bits; row n holds output column n's weights, the
 * layout of a linear layer's weight). */
void orc_project_rows(const uint8_t* codes, const float* scales, int64_t n_rows,
                      int32_t kv_lora, int32_t rope, const uint16_t* w_bf16, int32_t N,
                      double* out, double* rope_out, int threads);

/* Block-scaled (MX) variant of the row quantizer: the row is cut into blocks of
 * 32 values (kv_lora and rope multiples of 32), each with one power-of-two
 * scale 2^E stored as the ue8m0 byte E + 127 (the e4m3 bytes + ue8m0 exponents
 * of the mxfp8 format named on the page "Phase 0 toward V4.1 on a 128 GB Mac:
 * lossless mxfp8 residents and kill-test tooling" (keep PR #3), mxfp8
 * residents paragraph).  Per block: amax over finite entries; E is the
 * smallest integer with amax <= 448 * 2^E, clamped to [-127, 127] (so a
 * finite value never saturates, as in the per-row quantizer); codes are
 * E(x * 2^-E) with the saturating encoder.  Row i goes to cache row
 * dst_rows[i] (or i): codes[dst][0..kv_lora+rope), exps[dst][0..(kv_lora+rope)/32). */
void orc_quantize_rows_mx(const float* src, int64_t src_row_stride, int64_t n_rows,
                          int32_t kv_lora, int32_t rope, uint8_t* codes, uint8_t* exps,
                          const int64_t* dst_rows, int threads);

/* orc_attention over block-scaled rows: xhat = decode(code) * 2^(exp byte - 127). */
int orc_attention_mx(const uint16_t* q_lat, const uint16_t* q_rope,
                     const uint8_t* codes, const uint8_t* exps,
                     const int64_t* kv_start, const int32_t* kv_len,
                     int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                     float softmax_scale, int32_t num_splits,
                     const int64_t* sel, int64_t n_sel, double* out, int threads);

/* Bytes one token occupies per layer: kv_lora + rope code bytes plus the two
 * f32 scales ([colibri#299] PR description: one f32 scale each for Lc, Rc). */
int64_t orc_bytes_per_token_layer(int32_t kv_lora, int32_t rope);

/* The same for the block-scaled variant: one exponent byte per 32 values. */
int64_t orc_bytes_per_token_layer_mx(int32_t kv_lora, int32_t rope);

#ifdef __cplusplus
}
#endif
#endif
