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
//   (3 buffers, two tiles in flight), as raw fp8 rows whose 16-byte chunks
//   are rotated by token/4 so the score-pass reads spread over the banks;
//
//   score pass  S^T[token, row] = dec(KV)[token, 0:576] . q[row, 0:576]
//               36 MFMA 32x32x16 bf16 per tile, A = exactly decoded fp8 rows,
//               B = the wave's 32 query rows (resident in VGPRs), separate
//               accumulators for the Lc (512) and Rc (64) columns so the two
//               row scales are applied after the dot product;
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
//               MFMA K order), the Lc operand is read with the LDS transpose
//               load ds_read_b64_tr_b8, and 2^e normalises the largest Lc scale
//               of the block's token range below 1 so p * s / 2^e fits fp16.
//               fp16 rather than bf16 carries the probabilities: one bf16
//               rounding of p already costs ~1e-3 of the output, fp16 ~1e-4,
//               at the same MFMA rate, and every e4m3 value is exact in fp16.
//
// A block either writes the normalised output (one token range per
// sequence) or a partial (O, running max M, sum l) that the log-sum-exp merge
// kernel combines.
#include "kv8_device.hpp"
#include "kv8_internal.hpp"

namespace kv8 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kTT = 32;                          // tokens per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;       // 128 query rows
constexpr int kNBuf = 3;                         // LDS tile buffers
constexpr int kChunks = kRowBytes / 16;          // 36 chunks of 16 B per token row
constexpr int kTileBytes = kTT * kRowBytes;      // 18432
constexpr int kDmaPerTile = kTileBytes / 1024;   // 18 wave-wide 1 KiB copies
constexpr int kDmaSlots = (kDmaPerTile + kWaves - 1) / kWaves;  // 5 per wave at most
constexpr float kLazyLog2 = 15.0f;
constexpr int kQReg = 30;                        // score k-steps whose q lives in VGPRs
constexpr int kQLds = kChunks - kQReg;           // the rest is read from LDS per tile

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
    float* out;        // [B][QH][512] when n_splits == 1
    float* part_o;     // [n_splits][B][QH][512] when n_splits > 1
    float* part_ml;    // [n_splits][B][QH][2]: reference score m (before c), sum l
};

__device__ __forceinline__ void wait_vmcnt_4() { __builtin_amdgcn_s_waitcnt(0x0F74); }
__device__ __forceinline__ void wait_vmcnt_0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bf16x8_t dec8_bf16(uint32_t w0, uint32_t w1) {
    uint4 u = make_uint4(dec2_bf16<false>(w0), dec2_bf16<true>(w0), dec2_bf16<false>(w1),
                         dec2_bf16<true>(w1));
    return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ f16x8_t dec8_f16(uint32_t w0, uint32_t w1) {
    uint4 u = make_uint4(dec2_f16<false>(w0), dec2_f16<true>(w0), dec2_f16<false>(w1),
                         dec2_f16<true>(w1));
    return __builtin_bit_cast(f16x8_t, u);
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
__device__ __forceinline__ void mfma_score(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+v"(acc)
                 : "v"(a), "v"(b));
}

// Context MFMA with the accumulator pinned to AGPRs (same hazard note as
// above).
__device__ __forceinline__ void mfma_ctx(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last score MFMA and the first VALU read of its
// accumulator (conservatively more than the 16-pass result latency).
__device__ __forceinline__ void mfma_score_drain(f32x16_t& a0, f32x16_t& a1) {
    asm("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 r = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, r);
}

// LDS address of byte `col` (multiple of 8) of token row t in a tile: chunk
// c = col/16 sits at chunk slot (c + t/4) mod 36 of row t.
__device__ __forceinline__ int tile_addr(int t, int col) {
    int slot = (col >> 4) + (t >> 2);
    slot = slot >= kChunks ? slot - kChunks : slot;
    return t * kRowBytes + 16 * slot + (col & 15);
}

// O[dt] += P (32 rows x 16 tokens, two k-steps) . dec(Lc) (16 tokens x 32 dims)
// for the 16 dim tiles of 32 latent columns.
__device__ __forceinline__ void context_pass(f32x16_t (&O)[16], const uint4 (&pa)[2],
                                             const uint8_t* kvb, const int (&ctx_base)[2],
                                             const int (&ctx_slot)[2]) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const f16x8_t A = __builtin_bit_cast(f16x8_t, pa[kc]);
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            int off = ctx_base[kc] + 32 * dt;
            if (dt >= 14) off = ctx_slot[kc] + 2 * dt >= kChunks ? off - kRowBytes : off;
            const i32x2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2_t*)(kvb + off));
            const f16x8_t bv =
                dec8_f16(static_cast<uint32_t>(raw[0]), static_cast<uint32_t>(raw[1]));
            mfma_ctx(O[dt], A, bv);
        }
    }
}

// Zero a context accumulator in place (an MFMA of zeros with a zero C operand),
// keeping it in its AGPRs.
__device__ __forceinline__ void zero_acc(f32x16_t& acc) {
    const f16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %1, 0" : "+a"(acc) : "v"(z));
}

__global__ __launch_bounds__(kThreads, 1) void absorb_decode_kernel(DecodeArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_kv[kNBuf][kTileBytes];
    __shared__ __attribute__((aligned(16))) float s_sc[kNBuf][2 * kTT];
    __shared__ __attribute__((aligned(16))) uint4 s_q[kWaves][kQLds > 0 ? kQLds : 1][64];
    __shared__ int s_restart;
    __shared__ __attribute__((aligned(16))) float s_row[kWaves][32];
    __shared__ uint32_t s_red[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
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

    // ---- query rows of this wave: B operand of the score MFMA (row l32,
    //      columns 16ks + 8g .. +8): k-steps below kQReg stay in VGPRs, the
    //      others in this wave's LDS slice.  Rows past Q*H (block padding)
    //      reuse row 0; their results are never stored.
    uint4 qv[kQReg];
    {
        const int64_t qrow = static_cast<int64_t>(b) * p.QH + (row_ok ? row : 0);
        const uint4* ql = reinterpret_cast<const uint4*>(p.q_lat + qrow * kKvLora);
        const uint4* qr = reinterpret_cast<const uint4*>(p.q_rope + qrow * kRope);
#pragma unroll
        for (int ks = 0; ks < kQReg; ++ks) qv[ks] = ql[2 * ks + g];
#pragma unroll
        for (int ks = kQReg; ks < kChunks; ++ks)
            s_q[w][ks - kQReg][lane] = ks < 32 ? ql[2 * ks + g] : qr[2 * (ks - 32) + g];
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

    // ---- direct-to-LDS copy plan: wave w issues copies i = w + 4k; lane's
    //      16-byte chunk is tile slot 64 i + lane = token tt, rotated slot cs
    int dma_src[kDmaSlots];  // (tt << 16) | byte offset of the chunk in the token row
#pragma unroll
    for (int k = 0; k < kDmaSlots; ++k) {
        const int i = w + kWaves * k;
        const int slot = 64 * i + lane;
        const int tt = slot / kChunks;
        const int cs = slot - tt * kChunks;
        int c = cs - (tt >> 2);
        c = c < 0 ? c + kChunks : c;
        dma_src[k] = (tt << 16) | (16 * c);
    }

    auto issue_tile = [&](int tile) {
        const int buf = tile % kNBuf;
        const int64_t t0 = ts + static_cast<int64_t>(tile) * kTT;
        const int valid = static_cast<int>(te - t0 < kTT ? te - t0 : kTT);
        const uint8_t* src = p.codes + (row_base + t0) * kRowBytes;
#pragma unroll
        for (int k = 0; k < kDmaSlots; ++k) {
            const int i = w + kWaves * k;
            if (i < kDmaPerTile) {
                int tt = dma_src[k] >> 16;
                tt = tt < valid ? tt : valid - 1;
                const uint8_t* gp = src + tt * kRowBytes + (dma_src[k] & 0xFFFF);
                __builtin_amdgcn_global_load_lds(gp, (lds_u8*)&s_kv[buf][1024 * i], 16, 0, 0);
            }
        }
        if (w == kWaves - 1) {  // the tile's 32 (Lc, Rc) scale pairs, 4 bytes per lane
            int tt = lane >> 1;
            tt = tt < valid ? tt : valid - 1;
            const float* gp = p.scales + 2 * (row_base + t0 + tt) + (lane & 1);
            __builtin_amdgcn_global_load_lds(gp, (lds_u8*)&s_sc[buf][0], 4, 0, 0);
        }
    };

    // ---- per-lane LDS offsets
    // score A operand: token l32, columns 16ks + 8g
    const int sc_base = tile_addr(l32, 8 * g);
    // context B operand (transpose load): in the 16-lane group G = lane/16,
    // lane i supplies token tau(g, i/2) + 16 kc and column 16 (2dt + G%2) + 8 (i%2)
    const int G = lane >> 4;
    const int gi = lane & 15;
    const int kk = gi >> 1;
    const int tau = 4 * g + kk + (kk >= 4 ? 4 : 0);
    int ctx_base[2], ctx_slot[2];  // offset of dim tile 0 and its rotated chunk slot
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int tok = 16 * kc + tau;
        ctx_slot[kc] = (G & 1) + (tok >> 2);  // <= 8, no wrap for dim tile 0
        ctx_base[kc] = tok * kRowBytes + 16 * ctx_slot[kc] + 8 * (gi & 1);
    }

    f32x16_t O[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) O[dt][j] = 0.0f;
    // Scores x are kept before the factor c = softmax_scale * log2(e); the
    // row's reference m_x is its largest x (smallest when c < 0), and the
    // weights are p = 2^(c (x - m_x)): the difference is taken first, so the
    // reference token gets exactly 1 at any score magnitude.
    const float c = p.c;
    const float mask_val = c >= 0.0f ? -INFINITY : INFINITY;  // masked x, and "no reference"
    float m_x = mask_val;
    float l_run = 0.0f;        // this lane's half of the row sum
    // token offsets (relative to the range start) this lane's row may see
    const int64_t lim_rel0 = lim_row - ts;

    if (tid == 0) s_restart = 0;
    if (ntiles > 0) issue_tile(0);
    if (ntiles > 1) issue_tile(1);

    // At most two passes over the token range: a row whose later tile exceeds
    // its reference maximum by more than kLazyLog2 raises the reference and
    // flags the block; the pass still finishes (so every reference ends within
    // kLazyLog2 of every tile maximum) and the range is then run once more
    // from a zero accumulator.
    for (int attempt = 0; attempt < 2; ++attempt) {
        for (int it = 0; it < ntiles; ++it) {
            if (it + 1 < ntiles) wait_vmcnt_4(); else wait_vmcnt_0();
            __syncthreads();
            if (it + 2 < ntiles) issue_tile(it + 2);
            const int buf = it % kNBuf;
            const uint8_t* kvb = &s_kv[buf][0];

            // ---------------- score pass
            f32x16_t accL, accR;
#pragma unroll
            for (int j = 0; j < 16; ++j) { accL[j] = 0.0f; accR[j] = 0.0f; }
#pragma unroll
            for (int ks = 0; ks < kChunks; ++ks) {
                int off = sc_base + 16 * ks;
                if (ks >= kChunks - 8) {  // the rotated slot may wrap to the row start
                    const int slot = ks + (l32 >> 2);
                    off = slot >= kChunks ? off - kRowBytes : off;
                }
                const uint2 raw = *reinterpret_cast<const uint2*>(kvb + off);
                const bf16x8_t a = dec8_bf16(raw.x, raw.y);
                const bf16x8_t qb =
                    __builtin_bit_cast(bf16x8_t, ks < kQReg ? qv[ks] : s_q[w][ks - kQReg][lane]);
                if (ks < 32)
                    mfma_score(accL, a, qb);
                else
                    mfma_score(accR, a, qb);
            }
            mfma_score_drain(accL, accR);

            // ---------------- scale, mask, softmax (row l32, tokens
            //                  8(j/4) + 4g + j%4 of the tile)
            float x[16], sL[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 s01 =
                    *reinterpret_cast<const float4*>(&s_sc[buf][2 * (8 * q4 + 4 * g)]);
                const float4 s23 =
                    *reinterpret_cast<const float4*>(&s_sc[buf][2 * (8 * q4 + 4 * g) + 4]);
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
            if (c >= 0.0f) {
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
            } else if (c * (mx - m_x) > kLazyLog2) {
                m_x = mx;
                s_restart = 1;
            }
            const float ref = m_x == mask_val ? 0.0f : m_x;
            float pf[16];
            float lsum = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float pj = __builtin_amdgcn_exp2f(c * (x[j] - ref));
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
            context_pass(O, pa, kvb, ctx_base, ctx_slot);
        }
        __syncthreads();
        if (!s_restart) break;
        __syncthreads();
        if (tid == 0) s_restart = 0;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) zero_acc(O[dt]);
        l_run = 0.0f;
        if (ntiles > 0) issue_tile(0);
        if (ntiles > 1) issue_tile(1);
    }
    wait_vmcnt_0();  // no tile copy may land after the block has finished

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
            ml[0] = m_x;
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
