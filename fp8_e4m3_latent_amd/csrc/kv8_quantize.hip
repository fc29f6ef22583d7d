// Row quantizer of the fp8 e4m3 latent cache, plus the encoder sweep and
// decode check used to verify the device conversions.  gfx950.
//
// Page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
// (colibri PR #299): commit message, kv_fp8.h item (per-row f32 amax/448
// scale, guard when 448/amax overflows, saturating RNE encoder) and
// attention_rows item (the producer quantizes each fresh row); PR
// description (one scale each for the Lc and Rc rows).
//
// One wave64 quantizes eight 576-value token rows held in registers, so HBM
// is read once and written once:
//   lane l reads Lc[4l..4l+3] and Lc[256+4l..256+4l+3] (two 1 KiB coalesced
//   float4 loads per row) and, for l < 16, Rc[4l..4l+3], for all eight rows
//   before any arithmetic (streaming loads: the source is read once);
//   the Lc and Rc amax are integer maxima of |x| bit patterns reduced over
//   the wave with DPP row reductions and four lane reads (exact and
//   order-free); a segment whose maximum is inf or NaN is reduced again over
//   its finite values only;
//   the 2 x 16 correctly rounded divisions (scale and inverse of every
//   segment) run in one pass, one per lane;
//   codes come from the gfx950 fp8 conversion (round to nearest even) after
//   the clamp to [-448, 448] and NaN -> +0, which reproduces the encoder
//   rules exactly for every f32 value;
//   the eight scale pairs of a wave are written by eight lanes at once.
//
// The producer variant (same page, attention_rows item: the producer
// quantizes the fresh normalised and rotary-embedded row) first turns the
// loaded row into y and quantizes y exactly as above:
//   Lc: y_j = w_j (x_j r), r = 1 / sqrt(sum_k x_k^2 / 512 + eps) from the
//   hardware reciprocal square root, the sum of squares reduced over the wave
//   in f32;
//   Rc: pairs (2i, 2i+1) rotated by a_i = fl32(fl32(pos) f_i), with the f32
//   frequency f_i = fl32(theta^(-2i/64)) evaluated in f64 on the host (lane
//   l < 16 holds pairs 2l and 2l+1); a_i is reduced modulo 2 pi in f64 and
//   cos and sin come from the f32 sincos of the reduced angle (with eight rows
//   a wave, every lane computes four of the wave's 256 rotations and passes
//   them on through LDS).
#include <cmath>

#include "kv8_device.hpp"
#include "kv8_internal.hpp"

#pragma clang fp contract(off)

namespace kv8 {
namespace {

__device__ __forceinline__ uint32_t amax4(float4 v) {
    uint32_t a = max(finite_abs_bits(v.x), finite_abs_bits(v.y));
    uint32_t b = max(finite_abs_bits(v.z), finite_abs_bits(v.w));
    return max(a, b);
}
// max of |x| bit patterns including inf and NaN (NaN patterns sort above inf)
__device__ __forceinline__ uint32_t rawmax4(float4 v) {
    const uint32_t m = 0x7FFFFFFFu;
    return max(max(__float_as_uint(v.x) & m, __float_as_uint(v.y) & m),
               max(__float_as_uint(v.z) & m, __float_as_uint(v.w) & m));
}

// Unsigned max over the wave, returned wave-uniform: DPP steps within each
// row of 16 lanes (xor 1, xor 2, half-row mirror, row mirror), then the four
// row results read into scalars.
__device__ __forceinline__ uint32_t wave_max_uniform(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
    const uint32_t r0 = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
    const uint32_t r1 = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
    const uint32_t r3 = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
    return max(max(r0, r1), max(r2, r3));
}

// f32 sum over the wave, returned wave-uniform (DPP steps within each row of
// 16 lanes, then the four row sums)
__device__ __forceinline__ float wave_sum_uniform(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// a - 2 pi k in [-pi, pi] for an f32 angle a, reduced in f64 (2 pi as a sum of
// two doubles, so the reduction is exact to ~1e-16 for |a| < 2^40) and rounded
// to f32: sincosf then stays on its short path.  The f32 rounding of the
// reduced angle adds at most 2^-23 to it.
__device__ __forceinline__ float reduce_angle(float a) {
    const double two_pi_hi = 6.283185307179586232;    // fl64(2 pi)
    const double two_pi_lo = 2.4492935982947064e-16;  // 2 pi - two_pi_hi
    const double x = static_cast<double>(a);
    const double k = rint(x * (1.0 / 6.283185307179586232));
    double r = fma(-k, two_pi_hi, x);
    r = fma(-k, two_pi_lo, r);
    return static_cast<float>(r);
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {  // read-once data
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

// Codes of 4 values q = fl32(x * inv).  `finite` (wave-uniform): the row
// segment holds no inf or NaN and inv is finite, so q is finite and
// |q| <= fl32(amax * fl32(448 / amax)) < 464, which round-to-nearest-even
// takes to at most 448: only the clamp of encode4_e4m3_hw is kept.
__device__ __forceinline__ uint32_t encode4(float4 v, float inv, bool finite) {
    const float q0 = __fmul_rn(v.x, inv), q1 = __fmul_rn(v.y, inv);
    const float q2 = __fmul_rn(v.z, inv), q3 = __fmul_rn(v.w, inv);
    if (finite) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q0, -448.0f, 448.0f),
                                                       __builtin_amdgcn_fmed3f(q1, -448.0f, 448.0f), 0, false);
        return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(
            __builtin_amdgcn_fmed3f(q2, -448.0f, 448.0f), __builtin_amdgcn_fmed3f(q3, -448.0f, 448.0f), lo, true));
    }
    return encode4_e4m3_hw(q0, q1, q2, q3);
}

constexpr int kQuantWaves = 4;    // waves per 256-thread block
constexpr int64_t kFewRows = 8192;  // below: one row per wave

// producer step inputs (unused by the plain quantizer)
struct ProducerArgs {
    const float* norm_weight;   // [512]
    const int64_t* positions;   // [n_rows]
    float eps;
    float freq[kRope / 2];      // f_i = fl32(theta^(-2i/64)), from the host
};

// kRowsPerWave rows per wave: 8 for bulk work (eight rows of loads in flight
// per wave), 1 for a few rows (the per-token append of a decode step, where
// the kernel's latency is what counts: one row per wave spreads the rows
// over more compute units and shortens each wave's chain).
template <int kRowsPerWave, bool kProducer>
__global__ __launch_bounds__(64 * kQuantWaves) void quantize_rows_kernel(
    const float* __restrict__ src, int64_t stride, int64_t n_rows,
    uint8_t* __restrict__ codes, float* __restrict__ scales,
    const int64_t* __restrict__ dst_rows, ProducerArgs pa) {
    constexpr int kSegs = 2 * kRowsPerWave;  // (row, Lc/Rc) segments of a wave
    const int lane = threadIdx.x & 63;
    const int64_t row0 =
        (static_cast<int64_t>(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6)) * kRowsPerWave;
    if (row0 >= n_rows) return;
    // destination rows, loaded first: a load where the codes are stored would
    // add a dependent round trip at the end of the wave's chain
    int64_t drow[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t row = row0 + r < n_rows ? row0 + r : row0;
        drow[r] = dst_rows ? dst_rows[row] : row;
    }
    // producer: the positions are loaded before the rows, so that the
    // rotation factors (which need only them) are computed while the row
    // loads are in flight (vector loads complete in order)
    float rpos = 0.0f;
    float fq[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // this lane's frequencies (lane-indexed)
    if constexpr (kProducer) {
        const int64_t rrow = kRowsPerWave == 8 ? row0 + (lane >> 3) : row0;
        rpos = static_cast<float>(pa.positions[rrow < n_rows ? rrow : row0]);
        if constexpr (kRowsPerWave == 8) {  // pairs 4 (lane % 8) .. +3
#pragma unroll
            for (int t = 0; t < 4; ++t) fq[t] = pa.freq[4 * (lane & 7) + t];
        } else {  // pairs 2 (lane % 16), +1
            fq[0] = pa.freq[2 * (lane & 15)];
            fq[1] = pa.freq[2 * (lane & 15) + 1];
        }
        // keep these loads ahead of the row loads
        asm volatile("" ::: "memory");
    }
    float4 a[kRowsPerWave], b[kRowsPerWave], c[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        // (a missing second row repeats the first; it is not stored)
        const int64_t row = row0 + r < n_rows ? row0 + r : row0;
        const float* x = src + row * stride;
        a[r] = load_stream(x + 4 * lane);
        b[r] = load_stream(x + 256 + 4 * lane);
        // Rc: every lane loads (lanes 16-63 repeat the 256 bytes of lanes
        // 0-15, the same lines) and lanes 16-63 then hold zeros.  A load
        // under a lane branch would end in a wait for every load in flight.
        const float4 rc = load_stream(x + kKvLora + 4 * (lane & 15));
        c[r] = lane < 16 ? rc : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // producer: nothing that waits for the position moves between the row loads
    if constexpr (kProducer) __builtin_amdgcn_sched_barrier(0);

    if constexpr (kProducer) {
        // Lc weights of the lane's columns
        const float4 wa = *reinterpret_cast<const float4*>(pa.norm_weight + 4 * lane);
        const float4 wb = *reinterpret_cast<const float4*>(pa.norm_weight + 256 + 4 * lane);
        // With eight rows, the 8 x 32 rotations of the wave are spread over all
        // lanes: lane L computes (cos, sin) of pairs 4 (L % 8) .. +3 of row L / 8
        // into this wave's LDS area, [row][pair][cos, sin], where lane l < 16
        // (the Rc holder of pairs 2 l, 2 l + 1) reads them.
        float* rot = nullptr;
        if constexpr (kRowsPerWave == 8) {
            __shared__ __attribute__((aligned(16))) float s_rot[kQuantWaves][8 * 32 * 2];
            rot = &s_rot[threadIdx.x >> 6][0];
            float cv[4], sv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                sincosf(reduce_angle(rpos * fq[t]), &sv[t], &cv[t]);
            *reinterpret_cast<float4*>(rot + 8 * lane) = make_float4(cv[0], sv[0], cv[1], sv[1]);
            *reinterpret_cast<float4*>(rot + 8 * lane + 4) = make_float4(cv[2], sv[2], cv[3], sv[3]);
        }
        // one row per wave: the row's own two pairs, before its loads are waited for
        float s0r = 0.0f, c0r = 0.0f, s1r = 0.0f, c1r = 0.0f;
        if constexpr (kRowsPerWave == 1) {
            if (lane < 16) {
                sincosf(reduce_angle(rpos * fq[0]), &s0r, &c0r);
                sincosf(reduce_angle(rpos * fq[1]), &s1r, &c1r);
            }
        }
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
            float4& u = a[r];
            float4& v = b[r];
            float ss = u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
            ss = wave_sum_uniform(ss);
            const float rr = __builtin_amdgcn_rsqf(ss * (1.0f / kKvLora) + pa.eps);  // (~1 ulp)
            u = make_float4(wa.x * (u.x * rr), wa.y * (u.y * rr), wa.z * (u.z * rr), wa.w * (u.w * rr));
            v = make_float4(wb.x * (v.x * rr), wb.y * (v.y * rr), wb.z * (v.z * rr), wb.w * (v.w * rr));
            if (lane < 16) {
                float s0, c0, s1, c1;
                if constexpr (kRowsPerWave == 8) {
                    const float4 t = *reinterpret_cast<const float4*>(rot + 64 * r + 4 * lane);
                    c0 = t.x; s0 = t.y; c1 = t.z; s1 = t.w;
                } else {
                    c0 = c0r; s0 = s0r; c1 = c1r; s1 = s1r;
                }
                const float4 q = c[r];
                c[r] = make_float4(q.x * c0 - q.y * s0, q.x * s0 + q.y * c0,
                                   q.z * c1 - q.w * s1, q.z * s1 + q.w * c1);
            }
        }
    }

    // segment k = 2 r + (0: Lc, 1: Rc): amax over finite |x|; the plain
    // maximum of |x| patterns is that value unless it is inf or NaN
    uint32_t amax[kSegs];
    bool finite[kSegs];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        uint32_t mL = wave_max_uniform(max(rawmax4(a[r]), rawmax4(b[r])));
        uint32_t mR = wave_max_uniform(rawmax4(c[r]));
        finite[2 * r] = mL < 0x7F800000u;
        finite[2 * r + 1] = mR < 0x7F800000u;
        if (!finite[2 * r]) mL = wave_max_uniform(max(amax4(a[r]), amax4(b[r])));
        if (!finite[2 * r + 1]) mR = wave_max_uniform(amax4(c[r]));
        amax[2 * r] = mL;
        amax[2 * r + 1] = mR;
    }

    // All 2 kSegs correctly rounded divisions in one pass: lane k < kSegs
    // computes inv_k = 448 / amax_k, lane kSegs + k computes amax_k / 448.
    const int k = lane & (kSegs - 1);
    uint32_t am = amax[0];
#pragma unroll
    for (int j = 1; j < kSegs; ++j) am = k == j ? amax[j] : am;
    const bool is_inv = (lane & kSegs) == 0;
    const float quot = __fdiv_rn(is_inv ? 448.0f : __uint_as_float(am),
                                 is_inv ? __uint_as_float(am) : 448.0f);
    float inv[kSegs], scl[kSegs];
#pragma unroll
    for (int j = 0; j < kSegs; ++j) {
        inv[j] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_int(quot), j));
        scl[j] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_int(quot), kSegs + j));
        if (__float_as_uint(inv[j]) == 0x7F800000u) {  // guarded: 448 / amax overflows
            inv[j] = 0.0f;
            scl[j] = 0.0f;
            finite[j] = false;
        }
    }

    // the wave's scale pairs: lane r < kRowsPerWave holds row r's
    float2 sp = make_float2(scl[0], scl[1]);
#pragma unroll
    for (int r = 1; r < kRowsPerWave; ++r)
        if (lane == r) sp = make_float2(scl[2 * r], scl[2 * r + 1]);
    const int64_t nw = n_rows - row0 < kRowsPerWave ? n_rows - row0 : kRowsPerWave;  // rows stored
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t row = row0 + r;
        if (row >= n_rows) break;
        const int64_t d = drow[r];
        uint32_t* out = reinterpret_cast<uint32_t*>(codes + d * kRowBytes);
        __builtin_nontemporal_store(encode4(a[r], inv[2 * r], finite[2 * r]), out + lane);
        __builtin_nontemporal_store(encode4(b[r], inv[2 * r], finite[2 * r]), out + 64 + lane);
        if (lane < 16)
            __builtin_nontemporal_store(encode4(c[r], inv[2 * r + 1], finite[2 * r + 1]),
                                        out + kKvLora / 4 + lane);
        if (dst_rows && r == 0 && lane == 0) reinterpret_cast<float2*>(scales)[d] = sp;
    }
    if (dst_rows) {
        // rows 1.. of a scattered wave: one lane each
#pragma unroll
        for (int r = 1; r < kRowsPerWave; ++r)
            if (r < nw && lane == r) reinterpret_cast<float2*>(scales)[drow[r]] = sp;
    } else if (lane < nw) {
        reinterpret_cast<float2*>(scales)[row0 + lane] = sp;  // contiguous rows: one store
    }
}

// ---------------------------------------------------------------------------
// Block-scaled (MX) variant: one power-of-two scale per 32 values (page
// "Phase 0 toward V4.1 on a 128 GB Mac: lossless mxfp8 residents and
// kill-test tooling", mxfp8 residents paragraph: e4m3 bytes and ue8m0
// exponents per 32-wide group).  The block exponent is the smallest E with
// amax <= 448 * 2^E, read off the bit pattern of amax = m 2^k: 448 = 1.75 *
// 2^8, so E = k - 8 when m <= 1.75 (mantissa field <= 0x600000) and k - 7
// otherwise, within [-127, 127]; a zero or subnormal amax gives -127.  Codes
// are E(x * 2^-E) (an exact power-of-two scaling wherever the code can be
// nonzero).  Stored as the ue8m0 byte E + 127.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
    const int ef = static_cast<int>(amax_bits >> 23);
    if (ef == 0) return -127;
    const int E = ef - 127 - 8 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return E < -127 ? -127 : (E > 127 ? 127 : E);
}
// max over the 8 lanes of each lane octet (every lane gets its octet's maximum)
__device__ __forceinline__ uint32_t octet_max(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
    return v;
}
__device__ __forceinline__ uint32_t encode4_scaled(float4 v, int E) {
    return encode4_e4m3_hw(__builtin_ldexpf(v.x, -E), __builtin_ldexpf(v.y, -E),
                           __builtin_ldexpf(v.z, -E), __builtin_ldexpf(v.w, -E));
}

// One wave quantizes one 576-value row: lane l holds Lc[4l..4l+3],
// Lc[256+4l..] and (l < 16) Rc[4l..]; octet k of lanes holds block k of each
// part (Lc blocks k and 8 + k, Rc blocks 16 + k).
__global__ __launch_bounds__(256) void quantize_rows_mx_kernel(
    const float* __restrict__ src, int64_t stride, int64_t n_rows, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ exps, const int64_t* __restrict__ dst_rows) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const float* x = src + row * stride;
    const float4 a = load_stream(x + 4 * lane);
    const float4 b = load_stream(x + 256 + 4 * lane);
    float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < 16) c = load_stream(x + kKvLora + 4 * lane);
    const int Ea = mx_exponent(octet_max(amax4(a)));
    const int Eb = mx_exponent(octet_max(amax4(b)));
    const int Ec = mx_exponent(octet_max(amax4(c)));
    const int64_t d = dst_rows ? dst_rows[row] : row;
    uint32_t* out = reinterpret_cast<uint32_t*>(codes + d * kRowBytes);
    __builtin_nontemporal_store(encode4_scaled(a, Ea), out + lane);
    __builtin_nontemporal_store(encode4_scaled(b, Eb), out + 64 + lane);
    if (lane < 16) __builtin_nontemporal_store(encode4_scaled(c, Ec), out + kKvLora / 4 + lane);
    uint8_t* e = exps + d * (kRowBytes / 32);
    if ((lane & 7) == 0) {
        e[lane >> 3] = static_cast<uint8_t>(Ea + 127);
        e[8 + (lane >> 3)] = static_cast<uint8_t>(Eb + 127);
        if (lane < 16) e[16 + (lane >> 3)] = static_cast<uint8_t>(Ec + 127);
    }
}

// out[k] = encode(f32 with bit pattern first + k), 4 codes per thread, with
// the quantizer's conversion (kBitMath false) or the integer encoder.
template <bool kBitMath>
__global__ __launch_bounds__(256) void encode_bits_kernel(uint32_t first, uint64_t count,
                                                          uint8_t* __restrict__ out) {
    const uint64_t n4 = (count + 3) / 4;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
         i += static_cast<uint64_t>(gridDim.x) * 256) {
        const uint64_t k = 4 * i;
        const float f0 = __uint_as_float(static_cast<uint32_t>(first + k));
        const float f1 = __uint_as_float(static_cast<uint32_t>(first + k + 1));
        const float f2 = __uint_as_float(static_cast<uint32_t>(first + k + 2));
        const float f3 = __uint_as_float(static_cast<uint32_t>(first + k + 3));
        const uint32_t w = kBitMath ? pack4(encode_e4m3(f0), encode_e4m3(f1), encode_e4m3(f2), encode_e4m3(f3))
                                    : encode4_e4m3_hw(f0, f1, f2, f3);
        if (k + 4 <= count) {
            reinterpret_cast<uint32_t*>(out)[i] = w;
        } else {
            for (int j = 0; j < 4 && k + j < count; ++j) out[k + j] = static_cast<uint8_t>(w >> (8 * j));
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

template <bool kProducer>
int launch_rows(const float* src, int64_t stride, int64_t n_rows, uint8_t* codes, float* scales,
                const int64_t* dst_rows, const ProducerArgs& pa, hipStream_t stream) {
    if (n_rows < kFewRows) {
        const int64_t blocks = (n_rows + kQuantWaves - 1) / kQuantWaves;
        hipLaunchKernelGGL((quantize_rows_kernel<1, kProducer>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(64 * kQuantWaves), 0, stream, src, stride, n_rows, codes, scales,
                           dst_rows, pa);
    } else {
        const int64_t rows_per_block = static_cast<int64_t>(kQuantWaves) * 8;
        const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
        hipLaunchKernelGGL((quantize_rows_kernel<8, kProducer>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(64 * kQuantWaves), 0, stream, src, stride, n_rows, codes, scales,
                           dst_rows, pa);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize_rows(const float* src, int64_t stride, int64_t n_rows, uint8_t* codes,
                         float* scales, const int64_t* dst_rows, hipStream_t stream) {
    return launch_rows<false>(src, stride, n_rows, codes, scales, dst_rows,
                              ProducerArgs{nullptr, nullptr, 0.0f, {}}, stream);
}

int launch_norm_rope_quantize_rows(const float* src, int64_t stride, int64_t n_rows,
                                   const float* norm_weight, float eps, const int64_t* positions,
                                   float theta, uint8_t* codes, float* scales,
                                   const int64_t* dst_rows, hipStream_t stream) {
    ProducerArgs pa{norm_weight, positions, eps, {}};
    for (int i = 0; i < kRope / 2; ++i)
        pa.freq[i] = static_cast<float>(std::pow(static_cast<double>(theta), -2.0 * i / kRope));
    return launch_rows<true>(src, stride, n_rows, codes, scales, dst_rows, pa, stream);
}

int launch_quantize_rows_mx(const float* src, int64_t stride, int64_t n_rows, uint8_t* codes,
                            uint8_t* exps, const int64_t* dst_rows, hipStream_t stream) {
    const int64_t blocks = (n_rows + 3) / 4;
    hipLaunchKernelGGL(quantize_rows_mx_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       src, stride, n_rows, codes, exps, dst_rows);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_encode_bits(uint32_t first, uint64_t count, int encoder, uint8_t* out, hipStream_t stream) {
    const uint64_t n4 = (count + 3) / 4;
    uint64_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return 0;
    if (encoder == 1)
        hipLaunchKernelGGL(encode_bits_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                           stream, first, count, out);
    else
        hipLaunchKernelGGL(encode_bits_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
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
