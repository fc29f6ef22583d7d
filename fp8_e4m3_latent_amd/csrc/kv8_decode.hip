// Absorbed-MLA decode straight from the fp8 e4m3 latent cache.  gfx950.
//
// Page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
// (colibri PR #299): commit message, first paragraph (the latent row is both
// key and value of the absorbed attention) and attention_rows item (score
// and context loops over fp8 rows, dequantized inline, row scale applied
// outside the dot product); PR description, follow-up paragraph (split-T
// kernels for long slots).
//
// One block = 4 waves = 128 query rows (q, h) of one sequence x one token
// range.  Wave w owns rows 32w..32w+31 for the whole computation:
//
//   tiles of 32 tokens are copied global -> LDS by the direct-to-LDS loads
//   (three raw fp8 buffers, two tiles in flight); while the MFMAs work on
//   tile i, all 256 threads decode tile i+1 once, exactly, into an fp16
//   staging tile (rows padded to 1168 bytes so that the operand reads below
//   hit distinct banks);
//
//   score pass  S^T[token, row] = dec(KV)[token, 0:576] . q[row, 0:576]
//               36 MFMA 32x32x16 f16 per tile, A = staged fp16 rows
//               (ds_read_b128), B = the wave's 32 query rows resident in VGPRs
//               as fp16 (each row scaled by a power of two so its largest
//               element sits in [2^14, 2^15): every bf16 input is then exact
//               in fp16 unless it is 2^32 times smaller than the row maximum);
//               separate accumulators for the Lc (512) and Rc (64) columns so
//               the two row scales are applied after the dot product;
//
//   softmax     per row, with weights 2^(c (x - m)), c = softmax_scale log2(e);
//               a lane holds one row and 16 of the tile's tokens, so row maxima
//               need one cross-half exchange.  Each row's reference m is its
//               largest score in the first tile with a visible token and is
//               only raised when a later tile exceeds it by more than 15 (in
//               log2 units; p < 2^15 still fits fp16).  Raising it makes the
//               block finish the pass and run its token range once more with
//               the final references, so the context accumulator is never
//               rescaled and lives untouched in AGPRs; the result is the exact
//               softmax either way;
//
//   context     O[row, 0:512] += (p * s_Lc / 2^e)[row, token] . dec(Lc)[token, :]
//               32 MFMA 32x32x16 f16 per tile; the probabilities come straight
//               from the score accumulator registers (their token order is the
//               MFMA K order), the staged Lc operand is read with the LDS
//               transpose load ds_read_b64_tr_b16, and 2^e normalises the largest Lc scale
//               of the block's token range below 1 so p * s / 2^e fits fp16.
//               fp16 rather than bf16 carries the probabilities: one bf16
//               rounding of p already costs ~1e-3 of the output, fp16 ~1e-4,
//               at the same MFMA rate, and every e4m3 value is exact in fp16.
//
// Both passes therefore run on fp16 MFMA: every e4m3 value and every
// (row-scaled) bf16 query element is exact in fp16, so the score products are
// the exact products of the dequantized cache and the queries.
//
// A block either writes the normalised output (one token range per
// sequence) or a partial (O, reference score m, sum l) that the log-sum-exp
// merge kernel combines.
#include <cfloat>
#include "kv8_device.hpp"
#include "kv8_internal.hpp"

namespace kv8 {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kTT = 32;                          // tokens per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;       // 128 query rows
constexpr int kNRaw = 3;                         // raw fp8 tile buffers
constexpr int kNDec = 2;                         // decoded fp16 tile buffers
constexpr int kChunks = kRowBytes / 16;          // 36 score k-steps of 16 columns
constexpr int kRawBytes = kTT * kRowBytes;       // 18432
constexpr int kDecStride = 2 * kRowBytes + 16;   // 1168: fp16 token row + padding
constexpr int kDecBytes = kTT * kDecStride;      // 37376
constexpr int kDmaPerTile = kRawBytes / 1024;    // 18 wave-wide 1 KiB copies
constexpr int kDmaSlots = (kDmaPerTile + kWaves - 1) / kWaves;  // 5 per wave at most
constexpr int kDecChunks = kRawBytes / 8 / kThreads;            // 9 x 8 codes per thread
constexpr int kScoreAhead = 4;                   // score operand loads in flight
constexpr float kLazyLog2 = 15.0f;

struct DecodeArgs {
    const uint16_t* q_lat;
    const uint16_t* q_rope;
    const uint8_t* codes;
    const float* scales;
    const int64_t* kv_start;
    const int32_t* kv_len;
    int B, Q, H, QH;
    int n_rb;          // row blocks per sequence
    int n_splits;      // token ranges per sequence (grid)
    int split_chunk;   // > 0: fixed tokens per range
    int n_sub;         // split_chunk == 0: sub-ranges per equal range
    float c;           // softmax_scale * log2(e)
    float* out;        // [B][QH][512] when no partials are written
    float* part_o;     // [n_splits][B][QH][512]
    float* part_ml;    // [n_splits][B][QH][2]: reference score m, sum l
};

// s_waitcnt with only the vector-memory counter limited (lgkm and exp free)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Direct global -> LDS copies, written as inline assembly.  The compiler then
// does not see them write LDS and inserts no wait for them before LDS reads
// (for a copy it knows of it would wait until every copy in flight has
// landed, serialising the tile pipeline); the kernel instead waits for each
// tile's copies itself with s_waitcnt vmcnt, which counts these copies.  M0
// holds the LDS byte address; the bytes of lane l land at M0 + size * l.  M0
// is written one wait state before the copy reads it.
__device__ __forceinline__ void copy_to_lds_b128(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void copy_to_lds_b32(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)p));
}

// 8 e4m3 codes (two dwords) -> 8 fp16 values, exact
__device__ __forceinline__ uint4 dec8_f16(uint32_t w0, uint32_t w1) {
    return make_uint4(dec2_f16<false>(w0), dec2_f16<true>(w0), dec2_f16<false>(w1),
                      dec2_f16<true>(w1));
}

// Combine a per-lane value with the one in lane l ^ 32 (the other half of the
// wave holds the other 16 tokens of the same query row).
__device__ __forceinline__ float other_half(float v) {
    return __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float pair_max(float v) { return fmaxf(v, other_half(v)); }
__device__ __forceinline__ float pair_min(float v) { return fminf(v, other_half(v)); }
__device__ __forceinline__ float pair_sum(float v) { return v + other_half(v); }

// Score MFMA with its accumulator pinned to VGPRs, leaving all 256 AGPRs to the
// context accumulator.  The leading s_nop 1 gives the two wait states a VALU
// write of an operand needs before an MFMA reads it (the compiler cannot see
// that the asm is an MFMA); back-to-back MFMAs on the same accumulator need
// none.
__device__ __forceinline__ void mfma_score(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Context MFMA with the accumulator pinned to AGPRs (same hazard note).
__device__ __forceinline__ void mfma_ctx(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last score MFMA and the first VALU read of its
// accumulator (conservatively more than the result latency).
__device__ __forceinline__ void mfma_score_drain(f32x16_t& a0, f32x16_t& a1) {
    asm("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}

// Zero a context accumulator in place (an MFMA of zeros with a zero C operand),
// keeping it in its AGPRs.
__device__ __forceinline__ void zero_acc(f32x16_t& acc) {
    const f16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %1, 0" : "+a"(acc) : "v"(z));
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 r = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, r);
}

// bf16 bits -> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t w) {
    return max((w << 16) & 0x7FFFFFFFu, w & 0x7FFF0000u);
}

// 8 bf16 values times 2^-k -> 8 fp16 values (exact for the scaled range)
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 q, int k) {
    uint4 r;
    r.x = pack_f16x2(__builtin_ldexpf(bf16_lo(q.x), -k), __builtin_ldexpf(bf16_hi(q.x), -k));
    r.y = pack_f16x2(__builtin_ldexpf(bf16_lo(q.y), -k), __builtin_ldexpf(bf16_hi(q.y), -k));
    r.z = pack_f16x2(__builtin_ldexpf(bf16_lo(q.z), -k), __builtin_ldexpf(bf16_hi(q.z), -k));
    r.w = pack_f16x2(__builtin_ldexpf(bf16_lo(q.w), -k), __builtin_ldexpf(bf16_hi(q.w), -k));
    return r;
}

// Lc operand of context MFMA n = 16 kc + dt: two transpose loads of the fp16
// staging tile, 4 tokens each (tokens 8 apart: second half of the k-group)
__device__ __forceinline__ f16x8_t ctx_operand(const uint8_t* dec_lane, int n) {
    const int off = (n >> 4) * 16 * kDecStride + 64 * (n & 15);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(dec_lane + off));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(dec_lane + off + 8 * kDecStride));
    const uint2 l2 = __builtin_bit_cast(uint2, lo);
    const uint2 h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(f16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

// O[dt] += P (32 rows x 16 tokens, two k-steps) . dec(Lc) (16 tokens x 32 dims)
// for the 16 dim tiles of 32 latent columns; the operand loads run kCtxAhead
// MFMAs ahead.
constexpr int kCtxAhead = 3;
__device__ __forceinline__ void context_pass(f32x16_t (&O)[16], const uint4 (&pa)[2],
                                             const uint8_t* dec_lane) {
    f16x8_t bq[kCtxAhead];
#pragma unroll
    for (int n = 0; n < kCtxAhead; ++n) bq[n] = ctx_operand(dec_lane, n);
#pragma unroll
    for (int n = 0; n < 32; ++n) {
        // (the scheduler may not sink the loads next to their MFMAs: the asm
        //  MFMAs carry no latency it could see)
        __builtin_amdgcn_sched_barrier(0);
        const f16x8_t bv = bq[n % kCtxAhead];
        if (n + kCtxAhead < 32) bq[n % kCtxAhead] = ctx_operand(dec_lane, n + kCtxAhead);
        mfma_ctx(O[n & 15], __builtin_bit_cast(f16x8_t, pa[n >> 4]), bv);
    }
    __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(kThreads, 1) void absorb_decode_kernel(DecodeArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_raw[kNRaw][kRawBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_dec[kNDec][kDecBytes];
    __shared__ __attribute__((aligned(16))) float s_sc[kNRaw][2 * kTT];
    __shared__ __attribute__((aligned(16))) float s_scd[kNDec][2 * kTT];
    __shared__ __attribute__((aligned(16))) float s_row[kWaves][32];
    __shared__ uint32_t s_red[kWaves];
    __shared__ int s_restart;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;        // lane half
    const int l32 = lane & 31;

    int bid = blockIdx.x;
    const int rb = bid % p.n_rb;
    bid /= p.n_rb;
    const int split = bid % p.n_splits;
    const int b = bid / p.n_splits;

    const int64_t L = p.kv_len[b];
    const int64_t row_base = p.kv_start[b];
    int64_t ts, te;
    if (p.split_chunk > 0) {
        ts = static_cast<int64_t>(split) * p.split_chunk;
        te = ts + p.split_chunk;
    } else {
        // equal ranges of ceil(L / n_outer) rows, each cut into n_sub sub-ranges
        const int n_outer = p.n_splits / p.n_sub;
        const int outer = split / p.n_sub, sub = split % p.n_sub;
        const int64_t chunk = (L + n_outer - 1) / n_outer;
        const int64_t sub_chunk = (chunk + p.n_sub - 1) / p.n_sub;
        const int64_t o0 = static_cast<int64_t>(outer) * chunk;
        const int64_t o1 = o0 + chunk;
        ts = o0 + static_cast<int64_t>(sub) * sub_chunk;
        te = ts + sub_chunk < o1 ? ts + sub_chunk : o1;
    }
    te = L < te ? L : te;

    const int row0 = rb * kRowsPerBlock;
    const int row_hi = (p.QH < row0 + kRowsPerBlock ? p.QH : row0 + kRowsPerBlock) - 1;
    const int64_t n_first = L - (p.Q - 1) + row0 / p.H;    // visible tokens, first row
    const int64_t n_last = L - (p.Q - 1) + row_hi / p.H;   // visible tokens, last row
    te = te < n_last ? te : n_last;
    const int64_t ntok = te > ts ? te - ts : 0;
    const int ntiles = static_cast<int>((ntok + kTT - 1) / kTT);
    const int64_t full_until = te < n_first ? te : n_first;  // no mask below this token

    const int row = row0 + 32 * w + l32;
    const bool row_ok = row < p.QH;
    const int64_t n_row = row_ok ? L - (p.Q - 1) + row / p.H : 0;
    const int64_t lim_row = n_row < te ? n_row : te;

    // ---- query row l32 of this wave: B operand of the score MFMA (columns
    //      16ks + 8g .. +8), fp16 after scaling the row by 2^-kq so that its
    //      largest magnitude lies in [2^12, 2^13): every bf16 element above
    //      2^-27 of the row maximum converts exactly.  Rows past
    //      Q*H (block padding) reuse row 0; their results are never stored.
    uint4 qv[kChunks];
    int kq = 0;
    {
        const int64_t qrow = static_cast<int64_t>(b) * p.QH + (row_ok ? row : 0);
        const uint4* ql = reinterpret_cast<const uint4*>(p.q_lat + qrow * kKvLora);
        const uint4* qr = reinterpret_cast<const uint4*>(p.q_rope + qrow * kRope);
#pragma unroll
        for (int ks = 0; ks < kChunks; ++ks) qv[ks] = ks < 32 ? ql[2 * ks + g] : qr[2 * (ks - 32) + g];
        uint32_t mbits = 0;
#pragma unroll
        for (int ks = 0; ks < kChunks; ++ks)
            mbits = max(max(mbits, max(absmax_bf16x2(qv[ks].x), absmax_bf16x2(qv[ks].y))),
                        max(absmax_bf16x2(qv[ks].z), absmax_bf16x2(qv[ks].w)));
        const float qmax = pair_max(__uint_as_float(mbits));
        if (qmax > 0.0f) {
            kq = static_cast<int>((__float_as_uint(qmax) >> 23) & 0xFF) - 127 - 12;
            kq = kq < -100 ? -100 : (kq > 120 ? 120 : kq);
        }
#pragma unroll
        for (int ks = 0; ks < kChunks; ++ks) qv[ks] = bf16x8_to_f16(qv[ks], kq);
    }

    // ---- 2^e above the largest Lc scale of the token range
    uint32_t rbits = 0;
    for (int64_t t = ts + tid; t < te; t += kThreads)
        rbits = max(rbits, __float_as_uint(p.scales[2 * (row_base + t)]));
    rbits = wave_max_u32(rbits);
    if (lane == 0) s_red[w] = rbits;
    __syncthreads();
    rbits = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
    int e = 0;
    if (rbits != 0) {
        e = static_cast<int>((rbits >> 23) & 0xFF) - 126;  // r < 2^e
        e = e < -126 ? -126 : e;
    }

    // ---- tile copies: wave w issues the 1 KiB copies i = w + 4k of a tile
    //      (lane's 16 bytes = tile byte 1024 i + 16 lane, token (64 i + lane)/36)
    auto issue_tile = [&](int tile) {
        const int buf = tile % kNRaw;
        const int64_t t0 = ts + static_cast<int64_t>(tile) * kTT;
        const int valid = static_cast<int>(te - t0 < kTT ? te - t0 : kTT);
        const uint8_t* src = p.codes + (row_base + t0) * kRowBytes;
#pragma unroll
        for (int k = 0; k < kDmaSlots; ++k) {
            const int i = w + kWaves * k;
            if (i < kDmaPerTile) {
                const int slot = 64 * i + lane;
                int tt = slot / kChunks;
                const int cc = slot - tt * kChunks;
                tt = tt < valid ? tt : valid - 1;  // past the range: repeat its last row
                copy_to_lds_b128(src + tt * kRowBytes + 16 * cc, lds_addr(&s_raw[buf][1024 * i]));
            }
        }
        if (w == kWaves - 1) {  // the tile's 32 (Lc, Rc) scale pairs, 4 bytes per lane
            int tt = lane >> 1;
            tt = tt < valid ? tt : valid - 1;
            copy_to_lds_b32(p.scales + 2 * (row_base + t0 + tt) + (lane & 1), lds_addr(&s_sc[buf][0]));
        }
    };
    // wait until the copies of an issued tile have landed, `later` tiles
    // having been issued after it (each wave issues at least 4 copies a tile)
    auto wait_tile = [&](int later) {
        if (later >= 2) wait_vmcnt<8>();
        else if (later == 1) wait_vmcnt<4>();
        else wait_vmcnt<0>();
    };

    // ---- decode stage: the 8 threads of token tid/8 convert its codes
    //      8 (tid % 8) + 64 j, j < 9, into the fp16 staging tile
    const int raw_off = (tid >> 3) * kRowBytes + 8 * (tid & 7);
    const int dec_off = (tid >> 3) * kDecStride + 16 * (tid & 7);
    auto decode_tile = [&](int tile) {
        const uint8_t* raw = &s_raw[tile % kNRaw][raw_off];
        uint8_t* dst = &s_dec[tile % kNDec][dec_off];
        uint2 r[kDecChunks];
#pragma unroll
        for (int j = 0; j < kDecChunks; ++j) r[j] = *reinterpret_cast<const uint2*>(raw + 64 * j);
#pragma unroll
        for (int j = 0; j < kDecChunks; ++j)
            *reinterpret_cast<uint4*>(dst + 128 * j) = dec8_f16(r[j].x, r[j].y);
        if (tid < 2 * kTT) s_scd[tile % kNDec][tid] = s_sc[tile % kNRaw][tid];
    };

    // ---- per-lane LDS offsets in a staging tile
    // score A operand: token l32, columns 16ks + 8g
    const int sc_off = l32 * kDecStride + 16 * g;
    // context B operand: in the 16-lane group G = lane/16 (k-group g = G/2,
    // dims 32dt + 16(G%2) + 0..15), transpose load h of k-step kc takes token
    // tau(g, 4h + gi/4) + 16kc at dims +4(gi%4), tau(g, s) = 4g + s + 4[s >= 4]
    const int G = lane >> 4;
    const int gi = lane & 15;
    const int ctx_off = (4 * g + (gi >> 2)) * kDecStride + 32 * (G & 1) + 8 * (gi & 3);

    f32x16_t O[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) O[dt][j] = 0.0f;
    // Scores x are kept in accumulator units (before the factor
    // c_row = softmax_scale * log2(e) * 2^kq); the row's reference m_x is its
    // largest x (smallest when c < 0), and the weights are
    // p = 2^(c_row (x - m_x)): the difference is taken first, so the
    // reference token gets exactly 1 at any score magnitude.
    // (clamped to the finite normal range so that c_row (x - m_x) is 0 at the
    // reference and -inf at masked tokens, never NaN)
    float c_row = __builtin_ldexpf(p.c, kq);
    if (!(fabsf(c_row) <= FLT_MAX)) c_row = copysignf(FLT_MAX, p.c);
    if (fabsf(c_row) < FLT_MIN) c_row = copysignf(FLT_MIN, p.c);
    const float mask_val = c_row >= 0.0f ? -INFINITY : INFINITY;  // masked x, "no reference"
    float m_x = mask_val;
    float l_run = 0.0f;        // this lane's half of the row sum
    const int64_t lim_rel0 = lim_row - ts;  // visible tokens of this row from the range start

    if (tid == 0) s_restart = 0;

    // At most two passes over the token range: a row whose later tile exceeds
    // its reference maximum by more than kLazyLog2 raises the reference and
    // flags the block; the pass still finishes (so every reference ends within
    // kLazyLog2 of every tile maximum) and the range is then run once more
    // from a zero accumulator.
    for (int attempt = 0; attempt < 2; ++attempt) {
        // prologue: three tiles in flight, the first one decoded
        if (ntiles > 0) issue_tile(0);
        if (ntiles > 1) issue_tile(1);
        if (ntiles > 2) issue_tile(2);
        if (ntiles > 0) {
            wait_tile(ntiles > 2 ? 2 : ntiles - 1);
            __syncthreads();
            decode_tile(0);
        }
        for (int it = 0; it < ntiles; ++it) {
            if (it + 1 < ntiles) wait_tile(it + 2 < ntiles ? 1 : 0);
            __syncthreads();
            if (it + 3 < ntiles) issue_tile(it + 3);
            if (it + 1 < ntiles) decode_tile(it + 1);
            const uint8_t* dec = &s_dec[it % kNDec][0];
            const float* scd = &s_scd[it % kNDec][0];

            // ---------------- score pass
            f32x16_t accL, accR;
#pragma unroll
            for (int j = 0; j < 16; ++j) { accL[j] = 0.0f; accR[j] = 0.0f; }
            // (operand loads run kScoreAhead MFMAs ahead)
            f16x8_t aq[kScoreAhead];
#pragma unroll
            for (int ks = 0; ks < kScoreAhead; ++ks)
                aq[ks] = *reinterpret_cast<const f16x8_t*>(dec + sc_off + 32 * ks);
#pragma unroll
            for (int ks = 0; ks < kChunks; ++ks) {
                __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead
                const f16x8_t a = aq[ks % kScoreAhead];
                if (ks + kScoreAhead < kChunks)
                    aq[ks % kScoreAhead] =
                        *reinterpret_cast<const f16x8_t*>(dec + sc_off + 32 * (ks + kScoreAhead));
                const f16x8_t qb = __builtin_bit_cast(f16x8_t, qv[ks]);
                if (ks < 32)
                    mfma_score(accL, a, qb);
                else
                    mfma_score(accR, a, qb);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_score_drain(accL, accR);

            // ---------------- scale, mask, softmax (row l32, tokens
            //                  8(j/4) + 4g + j%4 of the tile)
            float x[16], sL[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 s01 = *reinterpret_cast<const float4*>(&scd[2 * (8 * q4 + 4 * g)]);
                const float4 s23 =
                    *reinterpret_cast<const float4*>(&scd[2 * (8 * q4 + 4 * g) + 4]);
                const float lsc[4] = {s01.x, s01.z, s23.x, s23.z};
                const float rsc[4] = {s01.y, s01.w, s23.y, s23.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * q4 + r;
                    sL[j] = lsc[r];
                    x[j] = __builtin_fmaf(lsc[r], accL[j], rsc[r] * accR[j]);
                }
            }
            if (ts + static_cast<int64_t>(it) * kTT + kTT > full_until) {
                const int64_t rel = lim_rel0 - static_cast<int64_t>(it) * kTT;
                const int lim = rel < 0 ? 0 : (rel > kTT ? kTT : static_cast<int>(rel));
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int t = 8 * (j >> 2) + 4 * g + (j & 3);
                    x[j] = t < lim ? x[j] : mask_val;
                }
            }
            float mx = x[0];
            if (c_row >= 0.0f) {
#pragma unroll
                for (int j = 1; j < 16; ++j) mx = fmaxf(mx, x[j]);
                mx = pair_max(mx);
            } else {
#pragma unroll
                for (int j = 1; j < 16; ++j) mx = fminf(mx, x[j]);
                mx = pair_min(mx);
            }
            if (m_x == mask_val) {
                m_x = mx;  // nothing accumulated for this row yet
            } else if (c_row * (mx - m_x) > kLazyLog2) {
                m_x = mx;
                s_restart = 1;
            }
            const float ref = m_x == mask_val ? 0.0f : m_x;
            float pf[16];
            float lsum = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float pj = __builtin_amdgcn_exp2f(c_row * (x[j] - ref));
                lsum += pj;
                pf[j] = pj * __builtin_ldexpf(sL[j], -e);
            }
            l_run += lsum;

            // ---------------- context pass
            uint4 pa[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                pa[kc].x = pack_f16x2(pf[8 * kc + 0], pf[8 * kc + 1]);
                pa[kc].y = pack_f16x2(pf[8 * kc + 2], pf[8 * kc + 3]);
                pa[kc].z = pack_f16x2(pf[8 * kc + 4], pf[8 * kc + 5]);
                pa[kc].w = pack_f16x2(pf[8 * kc + 6], pf[8 * kc + 7]);
            }
            context_pass(O, pa, dec + ctx_off);
        }
        __syncthreads();
        if (!s_restart) break;
        __syncthreads();
        if (tid == 0) s_restart = 0;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) zero_acc(O[dt]);
        l_run = 0.0f;
    }
    wait_vmcnt<0>();  // no tile copy may land after the block has finished

    // ---------------- epilogue: rows of O register j are 8(j/4) + 4g + j%4
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]),
                   "+a"(O[6]), "+a"(O[7]), "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]),
                   "+a"(O[12]), "+a"(O[13]), "+a"(O[14]), "+a"(O[15]));
    const float l_tot = pair_sum(l_run);
    if (p.part_o == nullptr) {
        // the probabilities carried 2^-e: out = 2^e O / l
        if (g == 0) s_row[w][l32] = l_tot > 0.0f ? __builtin_ldexpf(1.0f / l_tot, e) : 0.0f;
    } else {
        if (g == 0 && row_ok) {
            float* ml = p.part_ml + ((static_cast<int64_t>(split) * p.B + b) * p.QH + row) * 2;
            ml[0] = __builtin_ldexpf(m_x, kq);  // reference score in true units
            ml[1] = l_tot;
        }
        if (g == 0) s_row[w][l32] = __builtin_ldexpf(1.0f, e);  // partial O in true units
    }
    __builtin_amdgcn_wave_barrier();
    float* dst = p.part_o == nullptr
                     ? p.out + static_cast<int64_t>(b) * p.QH * kKvLora
                     : p.part_o + (static_cast<int64_t>(split) * p.B + b) * p.QH * kKvLora;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float4 f4 = *reinterpret_cast<const float4*>(&s_row[w][8 * q4 + 4 * g]);
        const float fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int orow = row0 + 32 * w + 8 * q4 + 4 * g + r;
            if (orow < p.QH) {
                float* o = dst + static_cast<int64_t>(orow) * kKvLora + l32;
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) o[32 * dt] = O[dt][4 * q4 + r] * fv[r];
            }
        }
    }
}

// out[b, row, :] = sum_s w_s O_s / sum_s w_s l_s over the splits with
// l_s > 0, w_s = 2^(c (m_s - m*)) with m* the reference of largest c m_s;
// zero when no split saw a token.
__global__ __launch_bounds__(128) void lse_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        int B, int QH, int n_splits, float c,
                                                        float* __restrict__ out) {
    const int64_t br = blockIdx.x;  // b * QH + row
    const int64_t stride = static_cast<int64_t>(B) * QH;
    bool any = false;
    float mstar = 0.0f;
    for (int s = 0; s < n_splits; ++s) {
        const float* ml = part_ml + (s * stride + br) * 2;
        if (ml[1] > 0.0f && (!any || c * (ml[0] - mstar) > 0.0f)) {
            mstar = ml[0];
            any = true;
        }
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.0f;
    if (any) {
        for (int s = 0; s < n_splits; ++s) {
            const float* ml = part_ml + (s * stride + br) * 2;
            const float ls = ml[1];
            if (ls > 0.0f) {
                const float wgt = __builtin_amdgcn_exp2f(c * (ml[0] - mstar));
                lsum += wgt * ls;
                const float4 o = reinterpret_cast<const float4*>(
                    part_o + (s * stride + br) * kKvLora)[threadIdx.x];
                acc.x += wgt * o.x;
                acc.y += wgt * o.y;
                acc.z += wgt * o.z;
                acc.w += wgt * o.w;
            }
        }
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    reinterpret_cast<float4*>(out + br * kKvLora)[threadIdx.x] =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

}  // namespace

size_t splitT_workspace_bytes(int B, int Q, int H, int n_splits) {
    const size_t rows = static_cast<size_t>(n_splits) * B * Q * H;
    return rows * kKvLora * sizeof(float) + rows * 2 * sizeof(float);
}

int launch_absorb_decode(const DecodeLaunch& d, hipStream_t stream, bool merge) {
    DecodeArgs a;
    a.q_lat = d.q_lat;
    a.q_rope = d.q_rope;
    a.codes = d.codes;
    a.scales = d.scales;
    a.kv_start = d.kv_start;
    a.kv_len = d.kv_len;
    a.B = d.B;
    a.Q = d.Q;
    a.H = d.H;
    a.QH = d.Q * d.H;
    a.n_rb = (a.QH + kRowsPerBlock - 1) / kRowsPerBlock;
    a.n_splits = d.n_splits;
    a.split_chunk = d.split_chunk;
    a.n_sub = d.n_sub > 0 ? d.n_sub : 1;
    a.c = d.softmax_scale * 1.4426950408889634f;
    a.out = d.out;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    if (d.n_splits > 1 || !merge) {
        const size_t rows = static_cast<size_t>(d.n_splits) * d.B * a.QH;
        a.part_o = static_cast<float*>(d.workspace);
        a.part_ml = a.part_o + rows * kKvLora;
    }
    const int64_t blocks = static_cast<int64_t>(d.B) * a.n_splits * a.n_rb;
    hipLaunchKernelGGL(absorb_decode_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads),
                       0, stream, a);
    if (hipGetLastError() != hipSuccess) return -1;
    if (d.n_splits > 1 && merge) {
        hipLaunchKernelGGL(lse_merge_kernel, dim3(static_cast<uint32_t>(d.B * a.QH)), dim3(128), 0,
                           stream, a.part_o, a.part_ml, d.B, a.QH, d.n_splits, a.c, d.out);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

int launch_lse_merge(const float* partials, int B, int QH, int n_splits, float softmax_scale,
                     float* out, hipStream_t stream) {
    const size_t rows = static_cast<size_t>(n_splits) * B * QH;
    const float* ml = partials + rows * kKvLora;
    hipLaunchKernelGGL(lse_merge_kernel, dim3(static_cast<uint32_t>(B * QH)), dim3(128), 0, stream,
                       partials, ml, B, QH, n_splits, softmax_scale * 1.4426950408889634f, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
