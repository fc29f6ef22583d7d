// Row quantizer of the fp8 e4m3 latent cache, plus the encoder sweep and
// decode check used to verify the device conversions.  gfx950.
//
// Page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
// (colibri PR #299): commit message, kv_fp8.h item (per-row f32 amax/448
// scale, guard when 448/amax overflows, saturating RNE encoder) and
// attention_rows item (the producer quantizes each fresh row); PR
// description (one scale each for the Lc and Rc rows).
//
// One wave64 quantizes one 576-value token row held in registers, so HBM is
// read once and written once:
//   lane l reads Lc[4l..4l+3] and Lc[256+4l..256+4l+3] (two 1 KiB coalesced
//   float4 loads per wave) and, for l < 16, Rc[4l..4l+3];
//   the Lc and Rc amax are integer maxima of finite |x| bit patterns reduced
//   over the wave (exact and order-free);
//   scale and inverse use correctly rounded f32 division;
//   each lane packs its 4-value groups into one 32-bit word of codes.
#include "kv8_device.hpp"
#include "kv8_internal.hpp"

#pragma clang fp contract(off)

namespace kv8 {
namespace {

struct SegScale {
    float scale;
    float inv;
};

// scale = fl32(amax / 448), inv = fl32(448 / amax); guarded (both 0) when the
// inverse overflows to +inf.
__device__ __forceinline__ SegScale segment_scale(uint32_t amax_bits) {
    const float amax = __uint_as_float(amax_bits);
    const float inv = __fdiv_rn(448.0f, amax);
    SegScale s;
    if (__float_as_uint(inv) == 0x7F800000u) {
        s.scale = 0.0f;
        s.inv = 0.0f;
    } else {
        s.scale = __fdiv_rn(amax, 448.0f);
        s.inv = inv;
    }
    return s;
}

__device__ __forceinline__ uint32_t encode4(float4 v, float inv) {
    return pack4(encode_e4m3(__fmul_rn(v.x, inv)), encode_e4m3(__fmul_rn(v.y, inv)),
                 encode_e4m3(__fmul_rn(v.z, inv)), encode_e4m3(__fmul_rn(v.w, inv)));
}

__device__ __forceinline__ uint32_t amax4(float4 v) {
    uint32_t a = max(finite_abs_bits(v.x), finite_abs_bits(v.y));
    uint32_t b = max(finite_abs_bits(v.z), finite_abs_bits(v.w));
    return max(a, b);
}

constexpr int kQuantWaves = 4;  // rows per 256-thread block

__global__ __launch_bounds__(64 * kQuantWaves) void quantize_rows_kernel(
    const float* __restrict__ src, int64_t stride, int64_t n_rows,
    uint8_t* __restrict__ codes, float* __restrict__ scales,
    const int64_t* __restrict__ dst_rows) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const float* x = src + row * stride;
    const float4 a = *reinterpret_cast<const float4*>(x + 4 * lane);
    const float4 b = *reinterpret_cast<const float4*>(x + 256 + 4 * lane);
    float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < 16) c = *reinterpret_cast<const float4*>(x + kKvLora + 4 * lane);

    const uint32_t mL = wave_max_u32(max(amax4(a), amax4(b)));
    const uint32_t mR = wave_max_u32(amax4(c));
    const SegScale sL = segment_scale(mL);
    const SegScale sR = segment_scale(mR);

    const int64_t d = dst_rows ? dst_rows[row] : row;
    uint8_t* out = codes + d * kRowBytes;
    reinterpret_cast<uint32_t*>(out)[lane] = encode4(a, sL.inv);
    reinterpret_cast<uint32_t*>(out + 256)[lane] = encode4(b, sL.inv);
    if (lane < 16) reinterpret_cast<uint32_t*>(out + kKvLora)[lane] = encode4(c, sR.inv);
    if (lane == 0) reinterpret_cast<float2*>(scales)[d] = make_float2(sL.scale, sR.scale);
}

// out[k] = encode(f32 with bit pattern first + k), 4 codes per thread.
__global__ __launch_bounds__(256) void encode_bits_kernel(uint32_t first, uint64_t count,
                                                          uint8_t* __restrict__ out) {
    const uint64_t n4 = (count + 3) / 4;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
         i += static_cast<uint64_t>(gridDim.x) * 256) {
        const uint64_t k = 4 * i;
        uint32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c[j] = encode_e4m3(__uint_as_float(static_cast<uint32_t>(first + k + j)));
        if (k + 4 <= count) {
            reinterpret_cast<uint32_t*>(out)[i] = pack4(c[0], c[1], c[2], c[3]);
        } else {
            for (int j = 0; j < 4 && k + j < count; ++j) out[k + j] = static_cast<uint8_t>(c[j]);
        }
    }
}

__global__ __launch_bounds__(256) void decode_codes_kernel(const uint8_t* __restrict__ codes,
                                                           int64_t n, uint16_t* __restrict__ bf,
                                                           uint16_t* __restrict__ hf) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    // the code in byte 2 exercises the high-half selector, byte 0 the low one
    const uint32_t c = codes[i];
    const uint32_t w = c | (c << 16);
    const uint32_t lo_b = dec2_bf16<false>(w), hi_b = dec2_bf16<true>(w);
    const uint32_t lo_h = dec2_f16<false>(w), hi_h = dec2_f16<true>(w);
    // both selectors must agree; a mismatch is reported as 0xFFFF (not a decode of any code)
    bf[i] = (lo_b & 0xFFFFu) == (hi_b & 0xFFFFu) ? static_cast<uint16_t>(lo_b) : 0xFFFFu;
    hf[i] = (lo_h & 0xFFFFu) == (hi_h & 0xFFFFu) ? static_cast<uint16_t>(lo_h) : 0xFFFFu;
}

}  // namespace

int launch_quantize_rows(const float* src, int64_t stride, int64_t n_rows, uint8_t* codes,
                         float* scales, const int64_t* dst_rows, hipStream_t stream) {
    const int64_t blocks = (n_rows + kQuantWaves - 1) / kQuantWaves;
    hipLaunchKernelGGL(quantize_rows_kernel, dim3(static_cast<uint32_t>(blocks)),
                       dim3(64 * kQuantWaves), 0, stream, src, stride, n_rows, codes, scales,
                       dst_rows);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_encode_bits(uint32_t first, uint64_t count, uint8_t* out, hipStream_t stream) {
    const uint64_t n4 = (count + 3) / 4;
    uint64_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return 0;
    hipLaunchKernelGGL(encode_bits_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, first, count, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode_codes(const uint8_t* codes, int64_t n, uint16_t* bf, uint16_t* hf,
                        hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(decode_codes_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, codes, n, bf, hf);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
