// Launch helpers shared by the C ABI (kv8_api.hip) and the kernel files.
// Each returns 0 on success or -1 when the launch failed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kv8 {

constexpr int kKvLora = 512;  // supported Lc width
constexpr int kRope = 64;     // supported Rc width

int launch_quantize_rows(const float* src, int64_t stride, int64_t n_rows, uint8_t* codes,
                         float* scales, const int64_t* dst_rows, hipStream_t stream);
// the producer step (RMS-normalised Lc, rotary-embedded Rc) fused with the quantizer
int launch_norm_rope_quantize_rows(const float* src, int64_t stride, int64_t n_rows,
                                   const float* norm_weight, float eps, const int64_t* positions,
                                   float theta, uint8_t* codes, float* scales,
                                   const int64_t* dst_rows, hipStream_t stream);
// encoder 0: the quantizer's conversion; 1: the integer bit-math encoder
// block-scaled variant: codes [rows][576], ue8m0 exponents [rows][18]
int launch_quantize_rows_mx(const float* src, int64_t stride, int64_t n_rows, uint8_t* codes,
                            uint8_t* exps, const int64_t* dst_rows, hipStream_t stream);
int launch_encode_bits(uint32_t first, uint64_t count, int encoder, uint8_t* out, hipStream_t stream);
// non-absorbed projection of cache rows (see kv8_project.hip); N a multiple of 128
int launch_project_rows(const uint8_t* codes, const float* scales, int64_t n_rows,
                        const uint16_t* w_kv_b, int N, void* out, bool out_f32, float* rope_out,
                        hipStream_t stream);
// One absorbed-decode launch (see kv8_decode.hip).  Token ranges: with
// split_chunk > 0 range s of a sequence is [s * split_chunk, (s+1) * split_chunk);
// otherwise the sequence is cut into n_outer equal ranges of ceil(L / n_outer)
// rows and each of those into n_sub equal sub-ranges; n_splits = n_outer * n_sub.
// n_splits > 1 needs workspace of splitT_workspace_bytes(B, Q, H, n_splits).
struct DecodeLaunch {
    const uint16_t* q_lat;
    const uint16_t* q_rope;
    const uint8_t* codes;
    const float* scales;            // per-row scales, or
    const uint8_t* exps = nullptr;  // block exponents of block-scaled rows
    const int64_t* kv_start;
    const int32_t* kv_len;
    int B, Q, H;
    int n_splits;
    int split_chunk;
    int n_sub;
    float softmax_scale;
    float* out;
    void* workspace;
};

size_t splitT_workspace_bytes(int B, int Q, int H, int n_splits);
// decode kernel (+ merge when n_splits > 1 and `merge` is set)
int launch_absorb_decode(const DecodeLaunch& d, hipStream_t stream, bool merge = true);
int launch_lse_merge(const void* partials, int B, int QH, int n_splits, float softmax_scale,
                     float* out, hipStream_t stream);

int launch_decode_codes(const uint8_t* codes, int64_t n, uint16_t* bf, uint16_t* hf,
                        hipStream_t stream);

}  // namespace kv8
