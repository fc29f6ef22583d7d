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
//   tiles of 32 tokens are copied global -> LDS by direct-to-LDS loads three
//   tiles ahead (four buffers of raw Lc codes, Rc codes and scale pairs);
//   both MFMA passes read the raw codes, and a tile's scale pairs become
//   (s_Lc, s_Rc, s_Lc / 2^e) in LDS before its scores are formed (rows of
//   block-scaled codes also decode their Lc codes one tile ahead into an
//   fp16 tile, two buffers, each block times its exponent relative to the
//   row's largest);
//
//   score pass  S^T[token, row] = dec(KV)[token, 0:576] . q[row, 0:576]
//               18 MFMA 32x32x64 fp8 per tile on the raw e4m3 codes (A,
//               ds_read_b128 from the raw tile) and the wave's 32 query rows
//               resident in VGPRs as two e4m3 terms q = hi + lo (B; each row
//               divided by a power of two so its largest element sits in
//               [2^7, 2^8), or by 2^-126 for rows below 2^-119: hi is the
//               nearest e4m3 value, lo the nearest to the exact remainder, and
//               hi + lo equals every bf16 element of at least 2^-9 of the row
//               maximum (every element of rows below 2^-119), the rest within
//               2^-17 of it; a NaN or infinite element makes the row NaN);
//               separate accumulators for the Lc (512) and Rc (64) columns so
//               the two row scales are applied after the dot product (rows of
//               block-scaled codes: the scaled MFMA applies each 32-value
//               block's exponent relative to the row's largest);
//
//   softmax     per row, with weights 2^(c (x - m)), c = |softmax_scale| log2(e)
//               (the sign of the softmax scale rides on the row scales); a lane
//               holds one row and 16 of the tile's tokens, so row maxima need
//               one cross-half exchange.  Each row's reference m is its largest
//               score in the first tile with a visible token and is only raised
//               when a later tile exceeds it by more than 15 (in log2 units;
//               p < 2^15 still fits fp16).  Raising it makes the block finish
//               the pass and run its token range once more with the final
//               references, so the context accumulator is never rescaled and
//               lives untouched in AGPRs; the result is the exact softmax either
//               way;
//
//   context     O[row, 0:512] += (p * s_Lc / 2^e)[row, token] . dec(Lc)[token, :]
//               32 MFMA 32x32x16 f16 per tile; the probabilities come straight
//               from the score accumulator registers (their token order is the
//               MFMA K order), the Lc operand is read from the raw codes with
//               the byte transpose load ds_read_b64_tr_b8 and converted
//               exactly to fp16 in registers (block-scaled rows: fp16 transpose
//               loads of the decoded tile), and 2^e normalises the largest Lc
//               scale of the block's token range below 1 so p * s / 2^e fits
//               fp16.  fp16 rather than bf16 carries the probabilities: one
//               bf16 rounding of p already costs ~1e-3 of the output, fp16
//               ~1e-4, at the same MFMA rate, and every e4m3 value is exact in
//               fp16.
//
// The score products are therefore the exact products of the dequantized
// cache and the (split) queries, and the context pass multiplies exact fp16
// values of the codes.
//
// A block either writes the normalised output (one token range per
// sequence) or a partial (O, reference score m, sum l) that the log-sum-exp
// merge kernel combines.
#include <cfloat>
#include <utility>
#include "kv8_device.hpp"
#include "kv8_internal.hpp"

namespace kv8 {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kTT = 32;                          // tokens per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;       // 128 query rows
constexpr int64_t kUnitRrBlocks = 1024;           // 4 blocks per compute unit of MI355X
constexpr int kRawBufs = 4;                      // raw Lc, raw Rc and copied scale buffers
constexpr int kDecBufs = 2;                      // fp16 Lc tile and decoded scale buffers
constexpr int kRawLcBytes = kTT * kKvLora;       // 16384: raw Lc codes of a tile
constexpr int kRawRcBytes = kTT * kRope;         // 2048: raw Rc codes of a tile
constexpr int kLcStride = 2 * kKvLora + 64;      // 1088: fp16 Lc row + padding
constexpr int kLcBytes = kTT * kLcStride;        // 34816

constexpr int kScoreAhead = 2;                   // score K-steps loaded ahead
constexpr int kCtxAhead = 3;                     // context operand loads in flight
constexpr float kLazyLog2 = 15.0f;

struct DecodeArgs {
    const uint16_t* q_lat;
    const uint16_t* q_rope;
    const uint8_t* codes;
    const float* scales;   // per-row scales [rows][2] (or the exponents below)
    const int64_t* kv_start;
    const int32_t* kv_len;
    int B, Q, H, QH;
    int n_rb;          // row blocks per sequence
    int n_splits;      // token ranges per sequence (grid)
    int split_chunk;   // > 0: fixed tokens per range
    int n_sub;         // split_chunk == 0: sub-ranges per equal range
    float c;           // softmax_scale * log2(e)
    float* out;        // [B][QH][512] when no partials are written
    int16_t* part_o;   // [n_splits][B][QH][512] codes, O = code * o_scale
    float* part_ml;    // [n_splits][B][QH] RangeStat records (16 bytes each)
    const uint8_t* exps;  // block exponents [rows][18] of block-scaled rows
    int unit_rr;          // block order: (sequence, range) units dealt to the XCDs in turn
};

// s_waitcnt with only the vector-memory counter limited (lgkm and exp free)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Wait for every copy and load of this wave in flight; also a compiler
// memory barrier, so that LDS reads of copied data stay after it.
__device__ __forceinline__ void wait_all_copies() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The lane id from an instruction that the compiler can neither hoist nor
// merge.  Copy offsets computed from it are rebuilt where they are used
// instead of being kept live (and possibly spilled: a scratch reload waits
// for every copy in flight).
__device__ __forceinline__ int fresh_lane_id() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// A load through the constant address space: with a uniform address it is a
// scalar load, counted by lgkmcnt, so waiting for it does not wait for the
// vector loads and copies in flight.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* ptr) {
    return *(const __attribute__((address_space(4))) T*)(ptr);
}

// Workgroup barrier after this wave's LDS operations and all of its tile
// copies except the last N (which stay in flight across the barrier).  The
// "memory" clobber keeps every LDS access on its side of the barrier; the
// compiler's own barrier would wait for every copy.
template <int N>
__device__ __forceinline__ void barrier_after_copies();
template <>
__device__ __forceinline__ void barrier_after_copies<4>() {
    asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <>
__device__ __forceinline__ void barrier_after_copies<5>() {
    asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct global -> LDS copies, written as inline assembly.  The compiler then
// does not see them write LDS and inserts no wait for them before LDS reads
// (for a copy it knows of it would wait until every copy in flight has
// landed, serialising the tile pipeline); the kernel instead waits for each
// tile's copies itself with s_waitcnt vmcnt, which counts these copies.  M0
// holds the LDS byte address; the bytes of lane l land at M0 + size * l.  M0
// is written one wait state before the copy reads it.  The source address
// is a wave-uniform base (SGPR pair) plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void copy_to_lds_b128(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
// The same copies through a raw buffer resource (base, no stride,
// num_records = nbytes): the buffer range check turns every dword of a lane
// at or past base + nbytes into a zero written to LDS, without a memory
// access.  Word 3 holds the raw-buffer format bits of this architecture.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t nbytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = static_cast<int>(static_cast<uint32_t>(a));
    r.y = static_cast<int>(static_cast<uint32_t>(a >> 32));  // (stride 0)
    r.z = static_cast<int>(nbytes);
    r.w = 0x00020000;
    return r;
}
__device__ __forceinline__ void copy_to_lds_b128_rc(const void* base, uint32_t nbytes, uint32_t off,
                                                    uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(buffer_rsrc(base, nbytes)), "s"(lds)
                 : "memory", "m0");
}
// the same through a given resource, the source moved by a uniform byte
// offset soff (not counted by the range check, which takes the lane offset
// alone; the LDS destination does not move)
__device__ __forceinline__ void copy_to_lds_b128_rsrc(i32x4_t rsrc, uint32_t off, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(off), "s"(rsrc), "s"(soff), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void copy_to_lds_b32_rc(const void* base, uint32_t nbytes, uint32_t off,
                                                   uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(buffer_rsrc(base, nbytes)), "s"(lds)
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
// the same times a power of two f <= 1 (block-scaled rows: 2^(E_block - E_max))
__device__ __forceinline__ uint32_t dec2_f16s(uint32_t four_codes, float f, bool hi) {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(four_codes, f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(four_codes, f, false));
}
__device__ __forceinline__ uint4 dec8_f16s(uint32_t w0, uint32_t w1, float f) {
    return make_uint4(dec2_f16s(w0, f, false), dec2_f16s(w0, f, true), dec2_f16s(w1, f, false),
                      dec2_f16s(w1, f, true));
}
// Block exponents of a block-scaled row: ue8m0 bytes, block b of the row at
// byte 18 t + b of its tile's exponent copy (16 Lc blocks, then 2 Rc blocks).
constexpr int kMxBlocksPerRow = (kKvLora + kRope) / 32;  // 18
constexpr int kMxTileExpBytes = kTT * kMxBlocksPerRow;   // 576
// largest of the 16 Lc exponent bytes of the row at byte a (even) of an LDS
// exponent copy whose base is 4-byte aligned
__device__ __forceinline__ int mx_lc_max(const uint8_t* base, int a) {
    const uint32_t* d = reinterpret_cast<const uint32_t*>(base + (a & ~3));
    const uint32_t sh = 8 * (a & 3);      // 0 or 16
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = __builtin_amdgcn_alignbit(d[i + 1], d[i], sh);  // bytes 4 i .. 4 i + 3
        m = max(m, max(max(v & 0xFFu, (v >> 8) & 0xFFu), max((v >> 16) & 0xFFu, v >> 24)));
    }
    return static_cast<int>(m);
}
// the 2 Rc exponent bytes of the row at byte a (even), low byte first
__device__ __forceinline__ uint32_t mx_rc_pair(const uint8_t* base, int a) {
    return *reinterpret_cast<const uint16_t*>(base + a + 16);
}
// 2^(E - 127) as a float (2^-127 for the byte 0 of an all-zero block)
__device__ __forceinline__ float mx_pow2(int E) { return __builtin_ldexpf(1.0f, E - 127); }

// Combine a per-lane value with the one in lane l ^ 32 (the other half of the
// wave holds the other 16 tokens of the same query row).
__device__ __forceinline__ float other_half(float v) {
    return __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float pair_sum(float v) { return v + other_half(v); }
// max(v, v of lane l ^ 32) with one lane swap between the wave halves (the
// swap of two copies of v leaves v of the lower half in one copy and v of
// the upper half in the other, in every lane); no NaN reaches it
__device__ __forceinline__ float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return m;
}

// Score MFMAs (fp8 e4m3 A and B, 32 x 32 x 64) with their accumulator pinned
// to VGPRs, leaving all 256 AGPRs to the context accumulator.  An MFMA needs
// two wait states after a VALU write of one of its operands, which the
// compiler does not insert for inline assembly; the score MFMAs take A from
// LDS loads (the load's s_waitcnt orders them) and B (the queries) and the
// block scales from registers written long before.  Back-to-back MFMAs on
// the same accumulator need no wait state.  The first MFMA of a chain starts
// from a zero C operand.
//
// Operand layout (32 x 32 x 64 fp8): lane l holds row l % 32 of A (column
// l % 32 of B); its bytes 0-15 are K = 16 (l / 32) + i and its bytes 16-31
// K = 32 + 16 (l / 32) + i, so each 32-value K block is bytes 0-15 (or
// 16-31) of both lane halves.  The scaled form multiplies row r's K block j
// by 2^(S - 127) for the byte S that lane 32 j + r selects in its scale
// register.
template <bool FIRST>
__device__ __forceinline__ void mfma_score8(f32x16_t& acc, const i32x8_t& a, const i32x8_t& b) {
    if constexpr (FIRST)
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// the same with A's blocks scaled by byte SEL of sa (B unscaled: sb holds
// 127; both scale operands must be VGPRs)
template <bool FIRST, int SEL>
__device__ __forceinline__ void mfma_score8s(f32x16_t& acc, const i32x8_t& a, const i32x8_t& b,
                                             uint32_t sa, uint32_t sb) {
#define KV8_MFMA8S(C, OPS) \
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, " C ", %3, %4 " OPS \
                 : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb))
    // (the first MFMA of a chain follows the VALU writes of the scale
    // registers: two wait states)
    if constexpr (FIRST) {
        asm volatile("s_nop 1" ::: "memory");
        if constexpr (SEL == 0) KV8_MFMA8S("0", "op_sel_hi:[0,0,0]");
        else if constexpr (SEL == 1) KV8_MFMA8S("0", "op_sel:[1,0,0] op_sel_hi:[0,0,0]");
        else if constexpr (SEL == 2) KV8_MFMA8S("0", "op_sel_hi:[1,0,0]");
        else KV8_MFMA8S("0", "op_sel:[1,0,0] op_sel_hi:[1,0,0]");
    } else {
        if constexpr (SEL == 0) KV8_MFMA8S("%0", "op_sel_hi:[0,0,0]");
        else if constexpr (SEL == 1) KV8_MFMA8S("%0", "op_sel:[1,0,0] op_sel_hi:[0,0,0]");
        else if constexpr (SEL == 2) KV8_MFMA8S("%0", "op_sel_hi:[1,0,0]");
        else KV8_MFMA8S("%0", "op_sel:[1,0,0] op_sel_hi:[1,0,0]");
    }
#undef KV8_MFMA8S
}

// Two e4m3 terms of 8 bf16 query elements q (one per code byte, in element
// order): hi = RNE_e4m3(q / qs) and lo = RNE_e4m3(q / qs - hi), where qs is
// a power of two (a normal float, inv = 1 / qs) and q / qs <= 256.  The
// remainder q inv - hi is formed exactly by one fused multiply-add in the
// scaled units (no f32 subnormal on the way, whatever the magnitude of q);
// hi + lo equals q / qs whenever the remainder is an e4m3 value (every
// element with q / qs >= 2^-2, and every bf16 value when qs = 2^-126), and is
// within 2^-10 of it otherwise.  A NaN or infinite q gives a NaN hi.
__device__ __forceinline__ f32x2_t fp8x2_lo_to_f32(uint32_t w, float s) {
    f32x2_t r;  // bytes 0, 1 times s
    asm("v_cvt_scalef32_pk_f32_fp8 %0, %1, %2" : "=v"(r) : "v"(w), "v"(s));
    return r;
}
__device__ __forceinline__ f32x2_t fp8x2_hi_to_f32(uint32_t w, float s) {
    f32x2_t r;  // bytes 2, 3 times s
    asm("v_cvt_scalef32_pk_f32_fp8 %0, %1, %2 op_sel:[1,0,0]" : "=v"(r) : "v"(w), "v"(s));
    return r;
}
__device__ __forceinline__ void split_q8(uint4 q, float qs, float inv, uint2& hi, uint2& lo) {
    const uint32_t x[4] = {q.x, q.y, q.z, q.w};
    i16x2_t h[2] = {{0, 0}, {0, 0}}, l[2] = {{0, 0}, {0, 0}};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2_t v = __builtin_bit_cast(bf16x2_t, x[i]);
        const float qa = __uint_as_float(x[i] << 16), qb = __uint_as_float(x[i] & 0xFFFF0000u);
        f32x2_t hb;
        if (i & 1) {
            h[i >> 1] = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h[i >> 1], v, qs, true);
            hb = fp8x2_hi_to_f32(__builtin_bit_cast(uint32_t, h[i >> 1]), 1.0f);
            l[i >> 1] = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
                l[i >> 1], __builtin_fmaf(qa, inv, -hb.x), __builtin_fmaf(qb, inv, -hb.y), 1.0f, true);
        } else {
            h[i >> 1] = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h[i >> 1], v, qs, false);
            hb = fp8x2_lo_to_f32(__builtin_bit_cast(uint32_t, h[i >> 1]), 1.0f);
            l[i >> 1] = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
                l[i >> 1], __builtin_fmaf(qa, inv, -hb.x), __builtin_fmaf(qb, inv, -hb.y), 1.0f, false);
        }
    }
    hi = make_uint2(__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]));
    lo = make_uint2(__builtin_bit_cast(uint32_t, l[0]), __builtin_bit_cast(uint32_t, l[1]));
}

// Context MFMA with the accumulator pinned to AGPRs; its operands are the
// packed probabilities (written before the phase starts) and LDS loads.
__device__ __forceinline__ void mfma_ctx(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// the same after two wait states (its B operand was just converted by VALU
// instructions)
__device__ __forceinline__ void mfma_ctx_nop(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last MFMA on an accumulator and the first VALU read
// of it (conservatively more than the result latency).
__device__ __forceinline__ void mfma_acc_drain(f32x16_t& a0, f32x16_t& a1) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}

// Zero a context accumulator in place (an MFMA of zeros with a zero C operand),
// keeping it in its AGPRs.
__device__ __forceinline__ void zero_acc(f32x16_t& acc) {
    const f16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %1, 0" : "+a"(acc) : "v"(z));
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded in the source:
// the pipelined phases select their work per step with `if constexpr`.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction order inside the software-pipelined phases is fixed in the
// source: the scheduler cannot see the latency of the asm MFMAs and would
// otherwise pull loads down next to their uses.  The MFMAs are volatile asm,
// so they keep their order relative to the LDS and memory instructions;
// pin(v) (an empty volatile asm reading and writing v) places plain
// arithmetic: work that depends on a pinned value cannot move above the pin,
// and a pinned result is computed before it.
__device__ __forceinline__ void order() { __builtin_amdgcn_sched_barrier(0); }
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;  // (no canonicalisation of the inputs: no NaN reaches the softmax)
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 r = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, r);
}

// Packed maximum of the magnitudes of two bf16 pairs: the bit patterns of
// non-negative bf16 values order as unsigned 16-bit integers.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax2_bf16x2(uint32_t m, uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, m),
                                                                  __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu)));
}


template <typename T>
__device__ __forceinline__ T lds_load(const uint8_t* base, int off) {
    return *reinterpret_cast<const T*>(base + off);
}

// Lc operand of context MFMA n = 16 kc + dt: two transpose loads of the fp16
// tile, 4 tokens each (the second half of the lane's k-group is 8 tokens on)
__device__ __forceinline__ f16x8_t ctx_operand(const uint8_t* lc, int tb0, int tb1, int n) {
    const int off = (n >> 4) * 16 * kLcStride + 64 * (n & 15);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(lc + tb0 + off));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(lc + tb1 + off));
    const uint2 l2 = __builtin_bit_cast(uint2, lo);
    const uint2 h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(f16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

// LDS layouts of a tile (32 tokens t; chunks are 16 bytes):
//   raw Lc  codes of t, chunk c (< 32), at chunk 32 c + (t ^ 4 (c & 1));
//   raw Rc  codes of t, chunk c (< 4), at chunk 32 c + t.  The tile copies
//           place the chunks there (each lane picks its source chunk).
//   fp16   Lc values of t, chunk c (< 64), at byte 1088 t + 16 (c ^ ((t >> 2) & 3)).
// With 64 LDS banks of 4 bytes every read and write below touches each bank
// once per 256 bytes: the score operand reads and the decode reads (16
// tokens, one chunk each), the byte transpose reads of the context operand
// (8 tokens x 16 bytes per 16 lanes, two chunk parities per 32 lanes), the
// fp16 transpose reads (4 tokens x 64 bytes per 32 lanes) and the decode
// writes (16 tokens, one fp16 chunk each).

// kMX: block-scaled rows (e4m3 codes with one ue8m0 exponent per 32 values).
// Each token's largest Lc and Rc block exponents E_L, E_R take the place of
// the per-row scales (s = 2^(E - 127)).  The score MFMAs scale each block by
// 2^(E_block - E_L) (or - E_R) exactly; the context pass decodes the Lc codes
// to fp16 times 2^(E_block - E_L): exact for blocks within 2^15 of the row's
// largest, smaller blocks round to fp16 subnormals.  The tile's exponent
// bytes (576) are copied where the per-row path copies its scale pairs (256).
template <bool kMX>
__global__ __launch_bounds__(kThreads, 1) void absorb_decode_kernel(DecodeArgs p) {
    // copied scales, or exponents (576 bytes from byte 0 or 2 of a 4-byte word)
    constexpr int kScBytes = kMX ? kMxTileExpBytes + 16 : 8 * kTT;
    // Raw buffers past kRawBufs - 1 only stage the queries (and keep the rope
    // query terms); the fp16 Lc tiles exist for block-scaled rows only (the
    // per-row path reads the context operand from the raw codes).
    constexpr int kRawArr = kMX ? kRawBufs + 1 : 2 * kRawBufs + 1;
    __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRawArr][kRawLcBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_rc[kRawBufs][kRawRcBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_lc[kMX ? kDecBufs : 1][kMX ? kLcBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_scb[kRawBufs][kScBytes];  // copied (Lc, Rc) scales or exponents
    __shared__ __attribute__((aligned(16))) float s_scd[kDecBufs][3 * kTT];  // s_Lc, s_Rc, s_Lc / 2^e
    __shared__ uint32_t s_red[3][kWaves];
    __shared__ int s_restart, s_shift;
    // per-row output factors of the epilogue, in the first raw Lc buffer (no
    // tile copy or decode is in flight by then)
    float (*const s_row)[32] = reinterpret_cast<float (*)[32]>(&s_raw[0][0]);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;        // lane half
    const int l32 = lane & 31;

    // Blocks are dealt round-robin to the 8 XCDs (block i to XCD i % 8).
    int rb, split, b;
    if (p.unit_rr) {
        // Launches of many blocks per compute unit (ragged lengths): the
        // (sequence, range) units go to the XCDs in turn, the row blocks of a
        // unit stay together on one XCD (they read the same KV tiles, through
        // its L2), and the range index skews the sequences, so that every XCD
        // gets a mix of long, short and empty ranges.  Needs B * n_splits to
        // be a multiple of 8 (unit k = 0 .. B * n_splits - 1 exactly once).
        const int x = static_cast<int>(blockIdx.x & 7), j = static_cast<int>(blockIdx.x >> 3);
        const int k = (j / p.n_rb) * 8 + x;
        split = k / p.B;
        b = (k % p.B + split) % p.B;
        rb = j % p.n_rb;
    } else {
        // Renumber the blocks so that each XCD runs a contiguous run of
        // logical blocks, i.e. all token ranges of the same sequences, which
        // then share their query rows in that XCD's L2.
        int bid = blockIdx.x;
        if ((gridDim.x & 7) == 0) bid = (bid & 7) * static_cast<int>(gridDim.x >> 3) + (bid >> 3);
        rb = bid % p.n_rb;
        bid /= p.n_rb;
        split = bid % p.n_splits;
        b = bid / p.n_splits;
    }

    const int row0 = rb * kRowsPerBlock;
    const int row = row0 + 32 * w + l32;
    const bool row_ok = row < p.QH;

    const int64_t L = load_uniform(p.kv_len + b);
    const int64_t row_base = load_uniform(p.kv_start + b);

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

    const int row_hi = (p.QH < row0 + kRowsPerBlock ? p.QH : row0 + kRowsPerBlock) - 1;
    const int64_t n_first = L - (p.Q - 1) + row0 / p.H;    // visible tokens, first row
    const int64_t n_last = L - (p.Q - 1) + row_hi / p.H;   // visible tokens, last row
    te = te < n_last ? te : n_last;
    const int64_t ntok = te > ts ? te - ts : 0;
    const int ntiles = static_cast<int>((ntok + kTT - 1) / kTT);
    const int64_t full_until = te < n_first ? te : n_first;  // no mask below this token
    // (block-scaled rows: a tile's exponent bytes start at byte 0 or 2 of a
    // 4-byte word, the same for every tile of the range)
    const int mx_shift = kMX ? 2 * static_cast<int>((row_base + ts) & 1) : 0;
    // rows of tile `tile` inside the range (the tiles past it re-copy the last)
    auto tile_valid = [&](int tile) {
        tile = tile < ntiles ? tile : ntiles - 1;
        const int64_t left = te - (ts + static_cast<int64_t>(tile) * kTT);
        return static_cast<int>(left < kTT ? left : kTT);
    };

    // visible tokens of this lane's row in the range, relative to ts (rebuilt
    // where a tile needs masking, so that it is not kept live across the loop)
    auto row_limit_rel = [&]() {
        const int r = row0 + 32 * w + (fresh_lane_id() & 31);
        const int64_t n_row = r < p.QH ? L - (p.Q - 1) + r / p.H : 0;
        const int64_t lim = n_row < te ? n_row : te;
        return static_cast<int>(lim - ts);
    };

    // A block whose token range holds no visible token (ranges past a short
    // sequence's end) writes its rows' (m, l) = (0, 0), which the merge skips,
    // and stops before any load: its partial codes are never read with a
    // nonzero weight.
    if (ntiles == 0 && p.part_o != nullptr) {
        if (g == 0 && row_ok) {  // (m = +0.0 as f64, l = 0, o_scale = 0)
            float* ml = p.part_ml + ((static_cast<int64_t>(split) * p.B + b) * p.QH + row) * 4;
            *reinterpret_cast<float4*>(ml) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        return;
    }

    // ---- query rows of this wave.  In the MFMA operand order every load
    //      would touch 32 rows (32 bytes of each), so the 32 latent rows
    //      (1 KiB each) are copied whole into LDS first, one row per copy, and
    //      read back in operand order once they have landed.  Lane l of the
    //      copy of row j takes the row's 16-byte chunk l ^ (j % 16), so that
    //      the 16 rows of a read fall on different banks.  The staging areas
    //      are raw buffers 2 w + 1 and 2 w + 2 (block-scaled rows: the fp16
    //      tile buffers for waves 0 and 1, raw buffers 1-2 and 3-4 for waves
    //      2 and 3), all free until tiles 1 to 3 are issued.  The rope parts
    //      (128 bytes a row) load directly.
    const uint8_t* const q_stage = !kMX ? &s_raw[2 * w + 1][0] : (w < kDecBufs ? &s_lc[w][0] : &s_raw[2 * w - 3][0]);
    {
        // (offsets from the sequence's first row: below 2^31, Q*H <= 2^21)
        const uint8_t* q_seq = reinterpret_cast<const uint8_t*>(p.q_lat + static_cast<int64_t>(b) * p.QH * kKvLora);
        const uint32_t lds0 = lds_addr(q_stage);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int r = row0 + 32 * w + j;
            const int rr = r < p.QH ? r : 0;  // (uniform)
            copy_to_lds_b128(q_seq, static_cast<uint32_t>(1024 * rr + 16 * (lane ^ (j & 15))),
                             lds0 + 1024 * j);
        }
    }
    // (qv[4 k + u]: chunk u of the query elements of score K-step k, below)
    uint4 qv[36];
    {
        const int64_t qrow = static_cast<int64_t>(b) * p.QH + (row_ok ? row : 0);
        const uint4* qr = reinterpret_cast<const uint4*>(p.q_rope + qrow * kRope);
#pragma unroll
        for (int u = 0; u < 4; ++u) qv[32 + u] = qr[2 * g + (u & 1) + 4 * (u >> 1)];
    }


    // ---- tile copies.  Wave w issues the 1 KiB copies i = w + 4k of a tile;
    //      the 16 bytes of lane l land at chunk 64 i + l of the raw Lc buffer
    //      (i < 16) or at chunk 64 (i - 16) + l of the raw Rc buffer, whose
    //      source chunk (token, offset in the token's row) follows the raw
    //      layouts: chunk 2 i + lane / 32 of token (lane % 32) ^ (4 (lane /
    //      32)) (Lc copy i < 16; the lane offset is the same for every copy,
    //      copy i's 32 i bytes go into the base) and Rc chunk 2 (i - 16) +
    //      lane / 32 of token lane % 32 (copy 4 of waves 0 and 1).
    auto dma_lc = [&](int ln) { return ((ln & 31) ^ (4 * (ln >> 5))) * kRowBytes + 16 * (ln >> 5); };
    auto dma_rc = [&](int ln) { return (ln & 31) * kRowBytes + kKvLora + 16 * (2 * (w & 1) + (ln >> 5)); };
    // The copies of a tile: tile i goes to the raw Lc, Rc and scale buffers
    // lbuf = i % 4.  Copy slot k < 4 of wave w is its Lc
    // copy w + 4 k; slot 4 is the Rc copy of wave w (waves 0 and 1) or the
    // tile's 32 (Lc, Rc) scale pairs, 4 bytes per lane (wave 3): waves 0, 1
    // and 3 issue five copies per tile, wave 2 four.  Tiles past the range
    // are replaced by the last tile (a harmless re-copy into free buffers).
    // The copies are range-checked at the range's end: rows past it arrive as
    // zero codes and zero scales (masked tokens, whose weight is 0).  The
    // per-lane byte offsets do not depend on the tile.
    // A tile's code rows: one buffer resource (its first row, valid rows x
    // 576 bytes) for all its code copies.
    // (token offsets inside a range fit 32 bits: kv_len is a 32-bit count)
    struct TileSrc {
        int rel;    // first token of the tile, relative to ts
        int valid;  // its tokens inside the range (uniform, >= 1)
        i32x4_t rsrc;
    };
    const uint8_t* const codes_rng = p.codes + (row_base + ts) * kRowBytes;
    const int ntok32 = static_cast<int>(ntok);
    auto tile_src = [&](int tile) {
        tile = tile < ntiles ? tile : ntiles - 1;
        TileSrc ts_;
        ts_.rel = tile * kTT;
        ts_.valid = ntok32 - ts_.rel < kTT ? ntok32 - ts_.rel : kTT;
        ts_.rsrc = buffer_rsrc(codes_rng + static_cast<int64_t>(ts_.rel) * kRowBytes,
                               static_cast<uint32_t>(ts_.valid * kRowBytes));
        return ts_;
    };
    const uint32_t lc_off = static_cast<uint32_t>(dma_lc(lane) + 32 * w);  // (Lc copy k: source + 128 k)
    auto issue_copy = [&](const TileSrc& src, int lbuf, auto kc, int ln) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < 4) {
            // Lc copy i = w + 4 k: lane offsets o = 576 t + 16 (lane / 32) +
            // 32 w from the tile's first row, moved by 128 k; the range check
            // o < 576 valid holds exactly for the tokens t < valid (whatever
            // the lane's token)
            copy_to_lds_b128_rsrc(src.rsrc, lc_off, 128 * k, lds_addr(&s_raw[lbuf][1024 * (w + kWaves * k)]));
        } else if (w < 2) {
            copy_to_lds_b128_rsrc(src.rsrc, static_cast<uint32_t>(dma_rc(ln)), 0, lds_addr(&s_rc[lbuf][1024 * w]));
        } else if (w == 3) {
            const int64_t t0 = ts + src.rel;
            const int valid = src.valid;
            if constexpr (kMX) {
                // the tile's 576 exponent bytes, 16 per lane on lanes 0-35; the
                // range check counts whole dwords, so the last one may carry
                // bytes of the row after the range (their tokens are masked
                // and get zero scales in decode_scales)
                if (ln < kScBytes / 16)
                    copy_to_lds_b128_rc(p.exps + (row_base + t0) * kMxBlocksPerRow - mx_shift,
                                        static_cast<uint32_t>((mx_shift + valid * kMxBlocksPerRow + 3) & ~3),
                                        static_cast<uint32_t>(16 * ln), lds_addr(&s_scb[lbuf][0]));
            } else {
                copy_to_lds_b32_rc(p.scales + 2 * (row_base + t0), static_cast<uint32_t>(8 * valid),
                                   static_cast<uint32_t>(4 * ln), lds_addr(&s_scb[lbuf][0]));
            }
        }
    };
    // (outside the tile loop, with offsets rebuilt from a fresh lane id)
    auto issue_tile = [&](int tile) {
        const int ln = fresh_lane_id();
        const TileSrc src = tile_src(tile);
        static_for<5>([&](auto kc) { issue_copy(src, tile % kRawBufs, kc, ln); });
    };

    // the first tile is in flight with the queries (tiles 1-3 go to buffers
    // that stage the queries)
    if (ntiles > 0) issue_tile(0);

    // ---- the range's largest Lc scale, largest Rc scale and smallest Lc
    //      scale (bit patterns of non-negative floats order as integers)
    uint32_t lbits = 0, rbits = 0, nbits = 0xFFFFFFFFu;
    if constexpr (kMX) {
        // a token's Lc and Rc scales are 2^(E - 127) for its largest block
        // exponents E (the bytes of one row: 9 two-byte loads, all inside it)
        const uint16_t* ex16 = reinterpret_cast<const uint16_t*>(p.exps);
        for (int64_t t0 = ts + tid; t0 < te; t0 += 2 * kThreads) {  // two rows in flight
            uint32_t v[2][9];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t t = t0 + u * kThreads;
#pragma unroll
                for (int i = 0; i < 9; ++i) v[u][i] = t < te ? ex16[(row_base + t) * 9 + i] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = max(m, max(v[u][i] & 0xFFu, v[u][i] >> 8));
                const uint32_t er = max(v[u][8] & 0xFFu, v[u][8] >> 8);
                const uint32_t lb = __float_as_uint(mx_pow2(static_cast<int>(m)));
                const uint32_t rb = __float_as_uint(mx_pow2(static_cast<int>(er)));
                const bool in = t0 + u * kThreads < te;
                lbits = in ? max(lbits, lb) : lbits;
                rbits = in ? max(rbits, rb) : rbits;
                nbits = in ? min(nbits, lb) : nbits;
            }
        }
    } else
    for (int64_t t0 = ts + tid; t0 < te; t0 += 4 * kThreads) {  // four loads in flight
        uint2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t t = t0 + u * kThreads;
            v[u] = t < te ? *reinterpret_cast<const uint2*>(p.scales + 2 * (row_base + t))
                          : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool in = t0 + u * kThreads < te;
            lbits = max(lbits, v[u].x);
            rbits = max(rbits, v[u].y);
            nbits = in ? min(nbits, v[u].x) : nbits;
        }
    }

    // ---- query row l32 of this wave: B operand of the score MFMA, two e4m3
    //      terms of the row divided by 2^kq so that its largest magnitude lies
    //      in [2^7, 2^8).  Score K-step k < 8 of lane half g holds the Lc
    //      columns 64 k + 16 g + [0, 16) (bytes 0-15) and 64 k + 32 + 16 g +
    //      [0, 16) (bytes 16-31), K-step 8 the rope columns 16 g + [0, 16) and
    //      32 + 16 g + [0, 16): the order of the cache codes in the A operand
    //      below, and each 32-column block of the row is one K block of the
    //      MFMA.  Rows past Q*H (block padding) reuse row 0; their results are
    //      never stored.
    wait_all_copies();  // (the queries, tile 0 and the scale loads)
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = 8 * k + 2 * g + (u & 1) + 4 * (u >> 1);  // bf16 chunk of 8 columns
            qv[4 * k + u] = lds_load<uint4>(q_stage, 1024 * l32 + 16 * (c ^ (l32 & 15)));
        }
    int kq = 0;
    {
        uint32_t m2 = 0;
#pragma unroll
        for (int ks = 0; ks < 36; ++ks)
            m2 = absmax2_bf16x2(absmax2_bf16x2(absmax2_bf16x2(absmax2_bf16x2(m2, qv[ks].x), qv[ks].y),
                                               qv[ks].z), qv[ks].w);
        const uint32_t mbits = max(m2 << 16, m2 & 0xFFFF0000u);  // (f32 bits)
        const float qmax = fmaxf(__uint_as_float(mbits), other_half(__uint_as_float(mbits)));
        if (qmax > 0.0f) {
            kq = static_cast<int>((__float_as_uint(qmax) >> 23) & 0xFF) - 127 - 7;
            kq = kq < -126 ? -126 : (kq > 120 ? 120 : kq);  // (2^kq and 2^-kq normal floats)
        }
    }

    lbits = wave_max_u32(lbits);
    rbits = wave_max_u32(rbits);
    nbits = ~wave_max_u32(~nbits);
    if (lane == 0) {
        s_red[0][w] = lbits;
        s_red[1][w] = rbits;
        s_red[2][w] = nbits;
    }
    __syncthreads();  // (also: every wave has read its staged queries)
    lbits = max(max(s_red[0][0], s_red[0][1]), max(s_red[0][2], s_red[0][3]));
    rbits = max(max(s_red[1][0], s_red[1][1]), max(s_red[1][2], s_red[1][3]));
    nbits = min(min(s_red[2][0], s_red[2][1]), min(s_red[2][2], s_red[2][3]));
    // 2^e just above the largest Lc scale (normalises the probabilities of
    // the context pass) and 2^ex just above the largest scale of either
    // segment (normalises the scores: s / 2^ex < 1 keeps every score below
    // 2^32 in accumulator units, whatever the magnitude of the rows)
    auto exp_above = [](uint32_t bits) {
        int k = 0;
        if (bits != 0) {
            k = static_cast<int>((bits >> 23) & 0xFF) - 126;  // value < 2^k
            k = k < -126 ? -126 : k;
        }
        return k;
    };
    const int e = __builtin_amdgcn_readfirstlane(exp_above(lbits));
    const int ex = __builtin_amdgcn_readfirstlane(exp_above(max(lbits, rbits)));
    // The probabilities of a row lose fp16 precision only when the tokens that
    // carry its weight have Lc scales far below the range's largest.  A range
    // whose smallest Lc scale (zero included) is more than 2^6 below its
    // largest is run "watched": the first pass records each row's largest
    // probability operand, and a row where it is small gets its operands
    // shifted up by a power of two in a second pass.
    const bool watched = nbits != 0xFFFFFFFFu && lbits != 0 &&
                         __uint_as_float(nbits) * 64.0f < __uint_as_float(lbits);

    // tiles 1 and 2 go to buffers that staged the queries; the conversion
    // below (pinned after them) runs while they are in flight
    if (ntiles > 0) {
        issue_tile(1);
        issue_tile(2);
    }
    {
        const float qs = __builtin_ldexpf(1.0f, kq), qinv = __builtin_ldexpf(1.0f, -kq);
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            uint2 hi[4], lo[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pin(qv[4 * k + u].x); pin(qv[4 * k + u].y); pin(qv[4 * k + u].z); pin(qv[4 * k + u].w);
                split_q8(qv[4 * k + u], qs, qinv, hi[u], lo[u]);
                order();  // (one chunk at a time: its f32 temporaries stay few)
            }
            qv[4 * k + 0] = make_uint4(hi[0].x, hi[0].y, hi[1].x, hi[1].y);
            qv[4 * k + 1] = make_uint4(hi[2].x, hi[2].y, hi[3].x, hi[3].y);
            qv[4 * k + 2] = make_uint4(lo[0].x, lo[0].y, lo[1].x, lo[1].y);
            qv[4 * k + 3] = make_uint4(lo[2].x, lo[2].y, lo[3].x, lo[3].y);
#pragma unroll
            for (int u = 0; u < 4; ++u) {  // (computed here, not next to their uses)
                pin(qv[4 * k + u].x); pin(qv[4 * k + u].y); pin(qv[4 * k + u].z); pin(qv[4 * k + u].w);
            }
        }
    }
    // The rope K-step's two terms (64 bytes a lane) wait in the staging-only
    // raw buffer (4 KiB a wave, lane l at 16 (l + 64 i) for 16-byte part i),
    // read back for each tile's first two score MFMAs: 16 fewer registers
    // for the rest of the tile.  (Every wave has read its staged queries: the
    // barrier after the staged reads.)
    uint8_t* const q_rope_lds = &s_raw[kRawBufs][4096 * w] + 16 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(q_rope_lds + 1024 * i) = qv[32 + i];
    auto q_term = [&](int k, int t) {  // term t (0: hi, 1: lo) of Lc K-step k
        const uint4 a = qv[4 * k + 2 * t], c = qv[4 * k + 2 * t + 1];
        i32x8_t r;
        r[0] = static_cast<int>(a.x); r[1] = static_cast<int>(a.y);
        r[2] = static_cast<int>(a.z); r[3] = static_cast<int>(a.w);
        r[4] = static_cast<int>(c.x); r[5] = static_cast<int>(c.y);
        r[6] = static_cast<int>(c.z); r[7] = static_cast<int>(c.w);
        return r;
    };

    // ---- per-lane LDS offsets
    // score A operand, K-step k: token l32, raw chunks 4 k + g (bytes 0-15)
    // and 4 k + 2 + g (bytes 16-31), at byte 512 c + 16 (l32 ^ 4 g) (the
    // rope K-step reads Rc chunks g and 2 + g at 512 c + 16 l32)
    const int sc_base = 16 * (l32 ^ (4 * g)) + 512 * g;
    const int sr_base = 16 * l32 + 512 * g;
    // Offsets of phase B (context and decode), rebuilt from a fresh lane id at
    // every phase B for block-scaled rows, whose phase A needs the registers.
    // context B operand: lane (G = lane / 16, gi = lane % 16) of k-group g
    // takes token 4 g + 8 h + gi / 4 (+ 16 kc) at dims 32 dt + 16 (G % 2) +
    // 4 (gi % 4) for its transpose load h (h = 1: 8 tokens on, the chunk
    // swizzle (g + 2) & 3 = g ^ 2 flips bit 5 of the byte offset)
    // decode: lane (token l32, half g) of wave w converts the raw chunks c =
    // 4 (2 w + g) + j (j < 4) of its token into fp16 chunks 2 c + e (e < 2):
    // reads at byte 512 c + 16 (l32 ^ 4 (c & 1)), writes at byte 1088 l32 +
    // 16 ((2 c + e) ^
    // ((l32 >> 2) & 3)) = (d_wA ^ (32 (j % 2) + 16 e)) + 64 (j / 2)
    // per-row context operand: lane L of group q addresses byte 512 c + 16
    // (t ^ 4 (c & 1)) + 8 (L % 2) of chunk c = 2 (n % 16) + q % 2 and token t
    // = 16 (n / 16) + 8 (L / 8) + 4 (q / 2) + (L / 2) % 4, which is c8_base +
    // 1024 (n % 16) + 256 (n / 16)
    int tb0 = 0, tb1 = 0, d_rA = 0, d_wA = 0, c8_base = 0;
    auto phase_b_offsets = [&](int ln) {
        const int lb = ln & 31, gb = ln >> 5;
        if constexpr (kMX) {
            const int G = ln >> 4, gi = ln & 15;
            const int cG = 2 * (G & 1) + ((gi & 3) >> 1);
            tb0 = (4 * gb + (gi >> 2)) * kLcStride + 16 * (cG ^ gb) + 8 * (gi & 1);
            tb1 = (tb0 + 8 * kLcStride) ^ 32;
            d_rA = 2048 * (2 * w + gb) + 16 * lb;  // + 512 j (odd j: ^ 64)
            d_wA = lb * kLcStride + 128 * (2 * w + gb) + 16 * ((lb >> 2) & 3);
        } else {
            const int q = ln >> 4, L = ln & 15;
            c8_base = 512 * (q & 1) + 128 * (L >> 3) + 64 * ((q >> 1) ^ (q & 1)) + 16 * ((L >> 1) & 3) + 8 * (L & 1);
        }
    };
    phase_b_offsets(lane);

    // Scores x are kept in accumulator units times sgn = sign(c) / 2^ex (the
    // row scales carry the sign and are divided by 2^ex, so |x| < 2^32 for
    // rows of any finite magnitude), so that with c_row = |softmax_scale
    // log2(e)| 2^(kq + ex) the weights are p = 2^(c_row (x - m_x) + dsh) with
    // m_x the row's largest x: the difference is taken first, so the reference
    // token gets exactly 2^dsh at any score magnitude.  dsh is 0 unless the
    // row's probability operands were found too small for fp16 (watched
    // ranges); the sum l carries the same 2^dsh, so O / l does not change.
    // (c_row is clamped to the finite normal range so that c_row (x - m_x) is
    // 0 at the reference and -inf at masked tokens, never NaN.)
    const float sgn = p.c >= 0.0f ? 1.0f : -1.0f;  // (uniform)
    float c_row = __builtin_ldexpf(fabsf(p.c), kq + ex);
    if (!(c_row <= FLT_MAX)) c_row = FLT_MAX;
    if (c_row < FLT_MIN) c_row = FLT_MIN;
    const float mask_val = -INFINITY;  // masked x, and "no reference yet"
    float m_x = mask_val;
    float l_run = 0.0f;        // this lane's half of the row sum
    float dsh = 0.0f;          // log2 of the row's operand shift (integer)
    float pmax = 0.0f;         // largest probability operand of the lane in this pass

    f32x16_t O[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) zero_acc(O[dt]);

    // ---- pipeline stages --------------------------------------------------
    // Tile i's raw Lc codes, raw Rc codes and copied scales (or block
    // exponents) live in s_raw / s_rc / s_scb [i % kRawBufs], its fp16 Lc tile
    // and decoded scales in s_lc / s_scd [i % kDecBufs].
    //
    // decode(tile): raw codes -> fp16 Lc tile, scales -> (s_Lc, s_Rc, s_Lc/2^e)
    uint4 draw[2];
    auto decode_load = [&](int rbuf, int j) {  // raw chunk 4 (2 w + g) + j of token l32
        draw[j & 1] = lds_load<uint4>(&s_raw[rbuf][0], ((j & 1) ? (d_rA ^ 64) : d_rA) + 512 * j);
    };
    // block-scaled rows: the exponents of the lane's two Lc blocks (raw chunks
    // j = 0, 1 and j = 2, 3) relative to the token's largest, E_block - E_L
    // >= -128 as signed bytes 2 and 3 of mx_sa[2] (below 2^-128 the fp16
    // value is 0 either way); set with the score's block scales (mx_scales)
    uint32_t mx_sa[3] = {0u, 0u, 0u};
    auto decode_store = [&](int dbuf, int j, int half) {
        uint8_t* lc = &s_lc[dbuf][0];
        const uint4 r = draw[j & 1];
        uint4 v;
        if constexpr (kMX) {
            const float f = __builtin_ldexpf(1.0f, static_cast<int>(mx_sa[2] << (8 - 8 * (j >> 1))) >> 24);
            v = half == 0 ? dec8_f16s(r.x, r.y, f) : dec8_f16s(r.z, r.w, f);
        } else {
            v = half == 0 ? dec8_f16(r.x, r.y) : dec8_f16(r.z, r.w);
        }
        *reinterpret_cast<uint4*>(lc + (d_wA ^ (32 * (j & 1) + 16 * half)) + 64 * (j >> 1)) = v;
    };
    // (every wave writes the same values: lane t < 32 the signed s_Lc / 2^ex,
    // s_Rc / 2^ex of token t, lane 32 + t the value s_Lc / 2^e of token t,
    // twice)
    auto decode_scales = [&](int rbuf, int dbuf, int tile) {
        float2 sc;
        if constexpr (kMX) {
            // 2^(E_L - 127), 2^(E_R - 127) of token l32; zero past the range
            const uint8_t* base = &s_scb[rbuf][0];
            const int tok = fresh_lane_id() & 31;
            const int a = mx_shift + kMxBlocksPerRow * tok;
            const uint32_t rp = mx_rc_pair(base, a);
            const bool in = tok < tile_valid(tile);
            sc.x = in ? mx_pow2(mx_lc_max(base, a)) : 0.0f;
            sc.y = in ? mx_pow2(static_cast<int>(max(rp & 0xFFu, rp >> 8))) : 0.0f;
        } else {
            (void)tile;
            sc = *reinterpret_cast<const float2*>(&s_scb[rbuf][8 * l32]);
        }
        float* d = &s_scd[dbuf][0];
        const float v0 = __builtin_ldexpf(g == 0 ? sgn * sc.x : sc.x, g == 0 ? -ex : -e);
        const float v1 = g == 0 ? __builtin_ldexpf(sgn * sc.y, -ex) : v0;
        d[g == 0 ? l32 : 2 * kTT + l32] = v0;
        d[g == 0 ? kTT + l32 : 2 * kTT + l32] = v1;
    };

    // x(tile) = s_Lc accL + s_Rc accR for row l32 and tokens 8 (j / 4) + 4 g +
    // j % 4 of the tile (the accumulator order), masked past the row's limit.
    // The token scales of the lane's 16 tokens are loaded into registers a
    // group ahead of their use (s_Lc, s_Rc when x is formed, s_Lc / 2^e for
    // P'), so that the arithmetic does not wait on LDS.
    float x[16];
    f32x16_t accL, accR;
    float4 sl4[4], sr4[4], se4[4];
    auto scales_load_l = [&](int buf, int q4) {
        sl4[q4] = *reinterpret_cast<const float4*>(&s_scd[buf][8 * q4 + 4 * g]);
    };
    auto scales_load_r = [&](int buf, int q4) {
        sr4[q4] = *reinterpret_cast<const float4*>(&s_scd[buf][kTT + 8 * q4 + 4 * g]);
    };
    auto scales_load_e = [&](int buf, int q4) {
        se4[q4] = *reinterpret_cast<const float4*>(&s_scd[buf][2 * kTT + 8 * q4 + 4 * g]);
    };
    auto form_x = [&](int q4) {
        const float4 sl = sl4[q4], sr = sr4[q4];
        x[4 * q4 + 0] = __builtin_fmaf(sl.x, accL[4 * q4 + 0], sr.x * accR[4 * q4 + 0]);
        x[4 * q4 + 1] = __builtin_fmaf(sl.y, accL[4 * q4 + 1], sr.y * accR[4 * q4 + 1]);
        x[4 * q4 + 2] = __builtin_fmaf(sl.z, accL[4 * q4 + 2], sr.z * accR[4 * q4 + 2]);
        x[4 * q4 + 3] = __builtin_fmaf(sl.w, accL[4 * q4 + 3], sr.w * accR[4 * q4 + 3]);
    };
    auto mask_x = [&](int tile) {
        if (ts + static_cast<int64_t>(tile) * kTT + kTT > full_until) {  // (uniform)
            const int rel = row_limit_rel() - tile * kTT - 4 * g;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int t = 8 * (j >> 2) + (j & 3);
                x[j] = t < rel ? x[j] : mask_val;
            }
        }
    };

    // score(tile): the rope K-step into accR first, then the Lc K-steps 0-7
    // into accL, two MFMAs (query terms hi, lo) per K-step; step s < 18
    // issues one MFMA so that other work can sit between the steps.  K-step q
    // of that order (0: rope, 1 + k: Lc k) is loaded kScoreAhead K-steps
    // ahead.
    i32x8_t aq[kScoreAhead];
    auto score_load = [&](int rbuf, int q) {
        const uint8_t* base = q == 0 ? &s_rc[rbuf][0] : &s_raw[rbuf][0] + 2048 * (q - 1);
        const int o = q == 0 ? sr_base : sc_base;
        const uint4 x = lds_load<uint4>(base, o), y = lds_load<uint4>(base, o + 1024);
        i32x8_t r;
        r[0] = static_cast<int>(x.x); r[1] = static_cast<int>(x.y);
        r[2] = static_cast<int>(x.z); r[3] = static_cast<int>(x.w);
        r[4] = static_cast<int>(y.x); r[5] = static_cast<int>(y.y);
        r[6] = static_cast<int>(y.z); r[7] = static_cast<int>(y.w);
        aq[q % kScoreAhead] = r;
    };
    // block-scaled rows: lane (token l32, half g) scales K block g of every
    // K-step: Lc block 2 k + g (byte k % 4 of mx_sa[k / 4]) and Rc block g
    // (byte 0 of mx_sa[2]), each by E_block - E_max + 127 (at least 0) for
    // the token's largest Lc (Rc) block exponent E_max
    const uint32_t mx_sb = 0x7F7F7F7Fu;  // (the queries unscaled)
    auto mx_scales = [&](int rbuf) {
        if constexpr (kMX) {
            const int ln = fresh_lane_id();
            const int a = mx_shift + kMxBlocksPerRow * (ln & 31);
            const uint32_t* d = reinterpret_cast<const uint32_t*>(&s_scb[rbuf][0] + (a & ~3));
            const uint32_t sh = 8 * (a & 3);  // (0 or 16)
            uint32_t v[4];
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = __builtin_amdgcn_alignbit(d[i + 1], d[i], sh);  // Lc bytes 4 i .. 4 i + 3
                m = max(m, max(max(v[i] & 0xFFu, (v[i] >> 8) & 0xFFu), max((v[i] >> 16) & 0xFFu, v[i] >> 24)));
            }
            const uint32_t rp = (d[4] >> sh) & 0xFFFFu;  // Rc bytes 16, 17
            const uint32_t mr = max(rp & 0xFFu, rp >> 8);
            const uint32_t gsh = 8 * static_cast<uint32_t>(ln >> 5);
            auto rel = [](uint32_t e, uint32_t mm) {
                const int r = static_cast<int>(e) - static_cast<int>(mm) + 127;
                return static_cast<uint32_t>(r < 0 ? 0 : r);
            };
            uint32_t s0 = 0, s1 = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                // block 2 k + g: byte 2 (k % 2) + g of v[k / 2]
                const uint32_t e = (v[k >> 1] >> (16 * (k & 1) + gsh)) & 0xFFu;
                if (k < 4) s0 |= rel(e, m) << (8 * k);
                else s1 |= rel(e, m) << (8 * (k - 4));
            }
            mx_sa[0] = s0;
            mx_sa[1] = s1;
            mx_sa[2] = rel((rp >> gsh) & 0xFFu, mr);
            // the decode's blocks 4 w + 2 g and 4 w + 2 g + 1: bytes 2 g and
            // 2 g + 1 of v[w] (w uniform)
            const uint32_t vw = w == 0 ? v[0] : (w == 1 ? v[1] : (w == 2 ? v[2] : v[3]));
            const int d0 = static_cast<int>((vw >> (2 * gsh)) & 0xFFu) - static_cast<int>(m);
            const int d1 = static_cast<int>((vw >> (2 * gsh + 8)) & 0xFFu) - static_cast<int>(m);
            mx_sa[2] |= ((static_cast<uint32_t>(d0 < -128 ? -128 : d0) & 0xFFu) << 16) |
                        ((static_cast<uint32_t>(d1 < -128 ? -128 : d1) & 0xFFu) << 24);
            // (all computed here: nothing of the exponent bytes stays live)
            pin(mx_sa[0]); pin(mx_sa[1]); pin(mx_sa[2]);
        }
    };
    i32x8_t qr[2];  // the rope K-step's query terms, for the first two MFMAs
    auto score_begin = [&](int rbuf) {
        mx_scales(rbuf);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint4 x = lds_load<uint4>(q_rope_lds, 2048 * t), y = lds_load<uint4>(q_rope_lds, 2048 * t + 1024);
            qr[t][0] = static_cast<int>(x.x); qr[t][1] = static_cast<int>(x.y);
            qr[t][2] = static_cast<int>(x.z); qr[t][3] = static_cast<int>(x.w);
            qr[t][4] = static_cast<int>(y.x); qr[t][5] = static_cast<int>(y.y);
            qr[t][6] = static_cast<int>(y.z); qr[t][7] = static_cast<int>(y.w);
        }
#pragma unroll
        for (int q = 0; q < kScoreAhead; ++q) score_load(rbuf, q);
    };
    auto score_step = [&](int rbuf, int st) {
        const int q = st >> 1, t = st & 1;  // K-step q, query term t
        const i32x8_t a = aq[q % kScoreAhead];
        const i32x8_t qb = q == 0 ? qr[t] : q_term(q - 1, t);
        if constexpr (kMX) {
            const uint32_t sa = mx_sa[q == 0 ? 2 : (q - 1) >> 2];
            const int sel = q == 0 ? 0 : (q - 1) & 3;
            f32x16_t& acc = q == 0 ? accR : accL;
            const bool first = t == 0 && q <= 1;
            if (first) mfma_score8s<true, 0>(acc, a, qb, sa, mx_sb);
            else if (sel == 0) mfma_score8s<false, 0>(acc, a, qb, sa, mx_sb);
            else if (sel == 1) mfma_score8s<false, 1>(acc, a, qb, sa, mx_sb);
            else if (sel == 2) mfma_score8s<false, 2>(acc, a, qb, sa, mx_sb);
            else mfma_score8s<false, 3>(acc, a, qb, sa, mx_sb);
        } else {
            if (q == 0) {
                if (t == 0) mfma_score8<true>(accR, a, qb);
                else mfma_score8<false>(accR, a, qb);
            } else {
                if (q == 1 && t == 0) mfma_score8<true>(accL, a, qb);
                else mfma_score8<false>(accL, a, qb);
            }
        }
        if (t == 1 && q + kScoreAhead < 9) score_load(rbuf, q + kScoreAhead);
    };

    // x(tile) in 9 steps (phase B, after the scales of the tile are decoded):
    // even step 2 q4 forms the scores of token group q4 - 1 (q4 > 0) and
    // loads the scales s_Lc, s_Rc of group q4 (q4 < 4); one group of scales
    // in flight at a time
    auto fx_step = [&](int k, int dbuf) {
        if (k % 2 == 1) return;
        const int q4 = k / 2;
        if (q4 > 0) {
            form_x(q4 - 1);
            pin(x[4 * q4 - 4]); pin(x[4 * q4 - 3]); pin(x[4 * q4 - 2]); pin(x[4 * q4 - 1]);
        }
        if (q4 < 4) {
            scales_load_l(dbuf, q4);
            scales_load_r(dbuf, q4);
        }
    };
    // softmax(tile) in 22 steps k of a few VALU instructions each
    // (phase A, between the score MFMAs of the next tile), from the scores x:
    //   0      mask (tiles past the first visible-token limit), maxima of
    //          three triples of the lane's 16 scores
    //   1      the lane's maximum
    //   2      the row maximum (with the other half of the wave)
    //   3      reference update
    //   4-11   p = 2^(c_row (x - ref) + dsh) for tokens 2 (k - 4) and
    //          2 (k - 4) + 1
    //   12-15  lsum = sum of the p (pairwise)
    //   16-19  P' = p s_Lc / 2^e for token group k - 16 (its scales loaded by
    //          se_load two steps before), and the lane's largest P'
    //   20-21  P' packed to fp16 as the A operand of context k-step k - 20
    uint4 pa[2];  // P' of the tile, the A operand of its context MFMAs
    float mx_part = 0.0f, mx_pair = 0.0f, ref = 0.0f, lsum = 0.0f;
    float mxa = 0.0f, mxb = 0.0f, mxc = 0.0f, sum_t[8];
    bool restart = false;  // this lane's row raised its reference in this pass
    auto soft_step = [&](int k, int tile) {
        if (k == 0) {
            mask_x(tile);
            mxa = max3(x[0], x[1], x[2]);
            mxb = max3(x[3], x[4], x[5]);
            mxc = max3(x[6], x[7], x[8]);
            pin(mxa); pin(mxb); pin(mxc);
        } else if (k == 1) {
            const float d = max3(x[9], x[10], x[11]);
            const float f = max3(x[12], x[13], x[14]);
            mx_part = fmaxf(max3(mxa, mxb, mxc), max3(d, f, x[15]));
            pin(mx_part);
        } else if (k == 2) {
            mx_pair = pair_max(mx_part);
            pin(mx_pair);
        } else if (k == 3) {
            const float mx = mx_pair;
            const bool first = m_x == mask_val;  // nothing accumulated for this row yet
            const bool raise = !first && c_row * (mx - m_x) > kLazyLog2;
            m_x = first || raise ? mx : m_x;
            restart = restart || raise;
            ref = m_x == mask_val ? 0.0f : m_x;
            pin(ref);
        } else if (k < 12) {
            const int j = 2 * (k - 4);
            pin(x[j]); pin(x[j + 1]);
            x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(c_row, x[j] - ref, dsh));
            x[j + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(c_row, x[j + 1] - ref, dsh));
            pin(x[j]); pin(x[j + 1]);
        } else if (k < 14) {
            const int j0 = 4 * (k - 12);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sum_t[j0 + i] = x[2 * (j0 + i)] + x[2 * (j0 + i) + 1];
                pin(sum_t[j0 + i]);
            }
        } else if (k == 14) {
            sum_t[0] = (sum_t[0] + sum_t[1]) + (sum_t[2] + sum_t[3]);
            sum_t[4] = (sum_t[4] + sum_t[5]) + (sum_t[6] + sum_t[7]);
            pin(sum_t[0]); pin(sum_t[4]);
        } else if (k == 15) {
            lsum = sum_t[0] + sum_t[4];
            pin(lsum);
        } else if (k < 20) {
            const int q4 = k - 16;
            pin(x[4 * q4]); pin(x[4 * q4 + 1]); pin(x[4 * q4 + 2]); pin(x[4 * q4 + 3]);
            x[4 * q4 + 0] *= se4[q4].x;
            x[4 * q4 + 1] *= se4[q4].y;
            x[4 * q4 + 2] *= se4[q4].z;
            x[4 * q4 + 3] *= se4[q4].w;
            pmax = max3(max3(pmax, x[4 * q4], x[4 * q4 + 1]), x[4 * q4 + 2], x[4 * q4 + 3]);
            pin(x[4 * q4]); pin(x[4 * q4 + 1]); pin(x[4 * q4 + 2]); pin(x[4 * q4 + 3]);
        } else {
            const int kc = k - 20;
            pa[kc].x = pack_f16x2(x[8 * kc + 0], x[8 * kc + 1]);
            pa[kc].y = pack_f16x2(x[8 * kc + 2], x[8 * kc + 3]);
            pa[kc].z = pack_f16x2(x[8 * kc + 4], x[8 * kc + 5]);
            pa[kc].w = pack_f16x2(x[8 * kc + 6], x[8 * kc + 7]);
            pin(pa[kc].x); pin(pa[kc].y); pin(pa[kc].z); pin(pa[kc].w);
        }
    };

    // context(tile): O[dt] += P (32 rows x 16 tokens) . dec(Lc) (16 tokens x
    // 32 dims), 32 MFMAs n (dims 32 (n % 16) .., tokens 16 (n / 16) ..).
    // Per-row path: the Lc operand comes straight from the raw codes: a byte
    // transpose load (ds_read_b64_tr_b8) gives lane t of each 16-lane group
    // byte t % 8 of the 8 bytes of lanes 2 j + t / 8 (j < 8), so lane 2 j + h
    // of group q addresses the codes of dims 16 (q % 2) + 8 h .. + 7 of the
    // token of MFMA K index j of lane half q / 2 (token 8 (j / 4) + 4 (q / 2)
    // + j % 4 of the 16, the order of the probabilities), and four exact
    // conversions make the fp16 operand.  Raw loads run kRawAhead MFMAs
    // ahead and conversions two (an MFMA does not wait on the conversions of
    // its own operand).  Block-scaled rows read the fp16 tile (two fp16
    // transpose loads per operand, kCtxAhead MFMAs ahead).
    constexpr int kRawAhead = 4;
    f16x8_t bq[kCtxAhead];
    uint2 craw[kRawAhead];
    auto ctx8_load = [&](int rbuf, int n) {
        const uint8_t* a = &s_raw[rbuf][0] + c8_base + 1024 * (n & 15) + 256 * (n >> 4);
        typedef int i32x2_t __attribute__((ext_vector_type(2)));
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(a));
        craw[n % kRawAhead] = make_uint2(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]));
    };
    auto ctx8_convert = [&](int n) {
        const uint2 r = craw[n % kRawAhead];
        uint4 c = dec8_f16(r.x, r.y);
        pin(c.x); pin(c.y); pin(c.z); pin(c.w);
        bq[n % 2] = __builtin_bit_cast(f16x8_t, c);
    };
    auto context_begin = [&](int buf) {
        if constexpr (kMX) {
            const uint8_t* lc = &s_lc[buf][0];
#pragma unroll
            for (int n = 0; n < kCtxAhead; ++n) bq[n] = ctx_operand(lc, tb0, tb1, n);
        } else {
#pragma unroll
            for (int n = 0; n < kRawAhead; ++n) ctx8_load(buf, n);
            ctx8_convert(0);
            ctx8_convert(1);
        }
    };
    auto context_step = [&](int buf, int n, uint4 pk) {
        if constexpr (kMX) {
            const uint8_t* lc = &s_lc[buf][0];
            const f16x8_t bv = bq[n % kCtxAhead];
            if (n + kCtxAhead < 32) bq[n % kCtxAhead] = ctx_operand(lc, tb0, tb1, n + kCtxAhead);
            mfma_ctx(O[n & 15], __builtin_bit_cast(f16x8_t, pk), bv);
        } else {
            if (n < 2) mfma_ctx_nop(O[n & 15], __builtin_bit_cast(f16x8_t, pk), bq[n % 2]);
            else mfma_ctx(O[n & 15], __builtin_bit_cast(f16x8_t, pk), bq[n % 2]);
            if (n + kRawAhead < 32) ctx8_load(buf, n + kRawAhead);
            if (n + 2 < 32) ctx8_convert(n + 2);
        }
    };

    if (tid == 0) {
        s_restart = 0;
        s_shift = 0;
    }

    // A row whose later tile exceeds its reference maximum by more than
    // kLazyLog2 raises the reference and flags the block; the pass still
    // finishes (so every reference ends within kLazyLog2 of every tile
    // maximum) and the range is then run once more from a zero accumulator.
    //
    // Software pipeline: the copies of tile i are issued three tiles ahead
    // into raw buffers i % 4 (free once tile i - 4 has passed its context
    // pass) and waited for at the end of iteration i - 2; iteration i runs
    //   phase A: score(i + 1) from its raw codes, with the softmax of tile i
    //            (its scores x were formed last iteration), three copies of
    //            tile i + 3 and the decoded scales of tile i + 1 (block-scaled
    //            rows: its scales in phase B, and the decode of tile i + 1
    //            into an fp16 Lc tile) between its MFMAs
    //   phase B: context(i) with the P' of that softmax (from tile i's raw
    //            codes, or its fp16 tile), with the scores x of tile i + 1
    //            and two copies of tile i + 3 between its MFMAs
    // and one barrier, after the copies of tile i + 2 have landed (those of
    // tile i + 3 stay in flight).  Stages past the last tile run on
    // re-copies of the last tile and their results are never used.
    auto end_barrier = [&]() {
        if (w == 2) barrier_after_copies<4>();
        else barrier_after_copies<5>();
    };
    // the decode of tile `tile` (raw buffers rb, fp16 buffers db), spread
    // over the steps n < 16 of a phase
    auto decode_step = [&](auto nc, int rb, int db) {
        constexpr int n = decltype(nc)::value;
        if constexpr (kMX && n % 4 == 0 && n < 16) decode_load(rb, n / 4);
        if constexpr (kMX && n % 4 == 2 && n < 16) decode_store(db, n / 4, 0);
        if constexpr (kMX && n % 4 == 3 && n < 16) decode_store(db, n / 4, 1);
    };
    // the scales of tile `tile` and its scores x, over steps n < 11
    auto scores_step = [&](auto nc, int rb, int db, int tile) {
        constexpr int n = decltype(nc)::value;
        if constexpr (n == 0) decode_scales(rb, db, tile);
        if constexpr (n >= 2 && n < 11) fx_step(n - 2, db);
    };
    // One pass over the token range (every pass also records each lane's
    // largest probability operand, which only a watched pass reads).
    auto run_pass = [&]() {
        if (ntiles > 0) {
            // tile 0 (landed; tiles 1 and 2 in flight): score, decode, scores x
            score_begin(0);
            static_for<18>([&](auto sc) {
                score_step(0, decltype(sc)::value);
                decode_step(sc, 0, 0);
            });
            mfma_acc_drain(accL, accR);
            static_for<11>([&](auto nc) { scores_step(nc, 0, 0, 0); });
            end_barrier();  // tile 1 landed; tile 2 may be in flight
        }
        // iteration `it` with R = it % kRawBufs known at compile time, so that
        // every LDS address is a lane offset plus an immediate
        auto iteration = [&](int it, auto rc) {
            constexpr int R = decltype(rc)::value;
            constexpr int RN = (R + 1) % kRawBufs;                        // tile it + 1
            constexpr int RC = (R + 3) % kRawBufs;                        // tile it + 3
            constexpr int CB = kMX ? R % kDecBufs : R;  // context operand buffer (fp16 or raw)
            constexpr int D0 = R % kDecBufs, D1 = (R + 1) % kDecBufs;
            // ---------------- phase A: score(it + 1) (and decode) of tile it + 1
            //                  from raw buffers RN, softmax of tile it (scales
            //                  in D0), copies of tile it + 3 into the raw
            //                  buffers of tile it - 1 (done with last
            //                  iteration)
            const TileSrc csrc = tile_src(it + 3);
            score_begin(RN);
            order();
            static_for<18>([&](auto sc) {
                constexpr int st = decltype(sc)::value;
                score_step(RN, st);
                // softmax steps: one per MFMA, two at steps 12, 13, 16 and
                // 17; the scales of P' loaded two MFMAs ahead of their use
                if constexpr (st < 12) soft_step(st, it);
                if constexpr (st == 12 || st == 13) {
                    soft_step(2 * st - 12, it);
                    soft_step(2 * st - 11, it);
                }
                if constexpr (st == 14 || st == 15) soft_step(st + 2, it);
                if constexpr (st == 16 || st == 17) {
                    soft_step(2 * st - 14, it);
                    soft_step(2 * st - 13, it);
                }
                if constexpr (st >= 12 && st < 16) scales_load_e(D0, st - 12);
                decode_step(sc, RN, D1);
                // per-row scales of tile it + 1 (landed at the last barrier):
                // decoded here, so that phase B only loads them
                if constexpr (!kMX && st == 2) decode_scales(RN, D1, it + 1);
                if constexpr (st == 5 || st == 9 || st == 13)
                    issue_copy(csrc, RC, std::integral_constant<int, (st - 5) / 4>{}, lane);
                order();
            });
            l_run += lsum;
            // ---------------- phase B: context(it) from buffer CB (written
            //                  before the last barrier), scores x of tile it + 1
            if constexpr (kMX) phase_b_offsets(fresh_lane_id());
            context_begin(CB);
            order();
            static_for<32>([&](auto nc) {
                constexpr int n = decltype(nc)::value;
                context_step(CB, n, n < 16 ? pa[0] : pa[1]);
                // (the scores x are formed from step 12 on: the score MFMAs of
                // phase A are more than 18 wait states back by then)
                if constexpr (kMX && n >= 12 && n < 23)
                    scores_step(std::integral_constant<int, n - 12>{}, RN, D1, it + 1);
                if constexpr (!kMX && n >= 12 && n < 20 && n % 2 == 0) {
                    // the scales of token group (n - 12) / 2, three MFMAs
                    // before its scores are formed
                    scales_load_l(D1, (n - 12) / 2);
                    scales_load_r(D1, (n - 12) / 2);
                }
                if constexpr (!kMX && n >= 15 && n < 23 && n % 2 == 1) {
                    constexpr int q4 = (n - 15) / 2;
                    form_x(q4);
                    pin(x[4 * q4]); pin(x[4 * q4 + 1]); pin(x[4 * q4 + 2]); pin(x[4 * q4 + 3]);
                }
                if constexpr (n == 5 || n == 25)
                    issue_copy(csrc, RC, std::integral_constant<int, 3 + n / 16>{}, lane);
                order();
            });
            end_barrier();  // tile it + 2 landed; tile it + 3 may be in flight
        };
        for (int it0 = 0; it0 < ntiles; it0 += kRawBufs) {
            iteration(it0, std::integral_constant<int, 0>{});
            if (it0 + 1 < ntiles) iteration(it0 + 1, std::integral_constant<int, 1>{});
            if (it0 + 2 < ntiles) iteration(it0 + 2, std::integral_constant<int, 2>{});
            if (it0 + 3 < ntiles) iteration(it0 + 3, std::integral_constant<int, 3>{});
        }
    };

    // At most three passes.  A pass in which some row raised its reference
    // is run again (the references are then final); a watched pass without a
    // raise then gives every row whose largest probability operand P' is
    // below 2^-6 the shift 2^dsh that brings it to [1, 2) (at most 2^100, and
    // with l 2^dsh below 2^120), and one more pass runs with those shifts.
    bool track = __builtin_amdgcn_readfirstlane(watched ? 1 : 0) != 0;
    for (int attempt = 0; attempt < 3; ++attempt) {
        if (attempt > 0 && ntiles > 0) {
            issue_tile(0);
            wait_all_copies();
            __syncthreads();
            issue_tile(1);
            issue_tile(2);
        }
        run_pass();
        if (restart) s_restart = 1;
        __syncthreads();
        const bool any_raise = s_restart != 0;
        if (track && !any_raise) {
            const float pr = fmaxf(pmax, other_half(pmax));  // the row's largest P'
            const float lt = pair_sum(l_run);
            if (lt > 0.0f && pr > 0.0f && pr < 0x1p-6f) {
                int pe, le;
                (void)frexpf(pr, &pe);  // pr in [2^(pe-1), 2^pe)
                (void)frexpf(lt, &le);
                int d = 1 - pe;
                d = d < 100 ? d : 100;
                d = d < 120 - le ? d : 120 - le;
                if (d > 0) {
                    dsh = static_cast<float>(d);
                    s_shift = 1;
                }
            }
        }
        __syncthreads();
        const bool any_shift = s_shift != 0;
        if (!any_raise && !any_shift) break;
        __syncthreads();  // (every wave has read the flags)
        if (tid == 0) {
            s_restart = 0;
            s_shift = 0;
        }
        track = any_raise && track;
        restart = false;
        wait_vmcnt<0>();  // the last re-copies land before the buffers are reused
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) zero_acc(O[dt]);
        l_run = 0.0f;
        pmax = 0.0f;
    }
    // No tile copy may land after this point: the epilogue reuses the first
    // raw buffer, which the last iteration's (clamped) re-copies of other
    // waves may still be writing, so every wave waits for its own copies and
    // then for the others at the barrier.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

    // ---------------- epilogue: rows of O register j are 8(j/4) + 4g + j%4
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]),
                   "+a"(O[6]), "+a"(O[7]), "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]),
                   "+a"(O[12]), "+a"(O[13]), "+a"(O[14]), "+a"(O[15]));
    const float l_tot = pair_sum(l_run);
    // (lane indices rebuilt here, so that no address of the stores below is
    // computed before the tile loop and kept live across it)
    const int el = fresh_lane_id();
    const int e32 = el & 31, eg = el >> 5;
    if (p.part_o == nullptr) {
        // the probabilities carried 2^-e: out = 2^e (O / l), with the shift
        // 2^dsh in both O and l (2^e / l alone could leave the float range)
        if (eg == 0) s_row[w][e32] = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        __builtin_amdgcn_wave_barrier();
        float* dst = p.out + static_cast<int64_t>(b) * p.QH * kKvLora;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 f4 = *reinterpret_cast<const float4*>(&s_row[w][8 * q4 + 4 * eg]);
            const float fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int orow = row0 + 32 * w + 8 * q4 + 4 * eg + r;
                if (orow < p.QH) {
                    float* o = dst + static_cast<int64_t>(orow) * kKvLora + e32;
#pragma unroll
                    for (int dt = 0; dt < 16; ++dt) {
                        float v;
                        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(O[dt][4 * q4 + r]));
                        o[32 * dt] = __builtin_ldexpf(v * fv[r], e);
                    }
                }
            }
        }
        return;
    }

    // Partial O / l as 16-bit codes, one scale per row: code = round(32767 O /
    // max_row |O|) (clamped to [-32767, 32767]), O / l = code * o_scale with
    // o_scale = 2^e max_row |O| / (32767 l) in true units (the normalised
    // context of the range, which stays within the range of its rows'
    // values, so it is finite for every finite cache).  |O| is compared as
    // the bit pattern of a non-negative float; the row maximum of register j
    // (row 8 (j / 4) + 4 g + j % 4, columns 32 dt + l32) combines the 16
    // registers of the lane and then the 32 lanes of its half.
    // Rows j, j + 1 at a time: their 32 values are read once, their maxima
    // reduced, and their codes stored.
    auto row_max = [&](uint32_t m) {
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0xB1, 0xF, 0xF, false)));
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x4E, 0xF, 0xF, false)));
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x141, 0xF, 0xF, false)));
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x140, 0xF, 0xF, false)));
        const auto sw = __builtin_amdgcn_permlane16_swap(m, m, false, false);
        return max(static_cast<uint32_t>(sw[0]), static_cast<uint32_t>(sw[1]));
    };
    int16_t* dst = p.part_o + (static_cast<int64_t>(split) * p.B + b) * p.QH * kKvLora;
    uint32_t mine = 0;  // lane t < 16 of each half: the maximum of register t's row
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
        // (each pair of rows reads its 32 values from the AGPRs here)
        float va[16], vb[16];
        uint32_t ma = 0, mb = 0;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(va[dt]) : "a"(O[dt][j]));
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(vb[dt]) : "a"(O[dt][j + 1]));
            ma = max(ma, __float_as_uint(va[dt]) & 0x7FFFFFFFu);
            mb = max(mb, __float_as_uint(vb[dt]) & 0x7FFFFFFFu);
        }
        ma = row_max(ma);
        mb = row_max(mb);
        mine = (e32 & 15) == j ? ma : mine;
        mine = (e32 & 15) == j + 1 ? mb : mine;
        const float r0 = __uint_as_float(ma), r1 = __uint_as_float(mb);
        // (an approximate reciprocal: only the code scale depends on it)
        const float i0 = r0 > 0.0f ? __builtin_amdgcn_rcpf(r0) : 0.0f;
        const float i1 = r1 > 0.0f ? __builtin_amdgcn_rcpf(r1) : 0.0f;
        const int orow0 = row0 + 32 * w + 8 * (j >> 2) + 4 * eg + (j & 3);
        int16_t* o0 = dst + static_cast<int64_t>(orow0) * kKvLora + e32;
        int16_t* o1 = o0 + kKvLora;  // (row of register j + 1)
        uint32_t c2[16];
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
            c2[dt] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(va[dt] * i0, vb[dt] * i1));
        if (orow0 < p.QH) {
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) o0[32 * dt] = static_cast<int16_t>(c2[dt] & 0xFFFFu);
        }
        if (orow0 + 1 < p.QH) {
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) o1[32 * dt] = static_cast<int16_t>(c2[dt] >> 16);
        }
        order();
    }
    if (e32 < 16) s_row[w][8 * (e32 >> 2) + 4 * eg + (e32 & 3)] = __uint_as_float(mine);
    __builtin_amdgcn_wave_barrier();
    if (eg == 0 && row_ok) {
        float* ml = p.part_ml + ((static_cast<int64_t>(split) * p.B + b) * p.QH + row) * 4;
        const float rmax = s_row[w][e32];
        const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        // reference score in true units (f64: scores of large rows and large
        // queries leave the f32 range), the unshifted sum, the code scale
        const double m_true = __builtin_ldexp(static_cast<double>(sgn * m_x), kq + ex);
        const uint64_t mb = __builtin_bit_cast(uint64_t, m_true);
        *reinterpret_cast<float4*>(ml) =
            make_float4(__uint_as_float(static_cast<uint32_t>(mb)), __uint_as_float(static_cast<uint32_t>(mb >> 32)),
                        __builtin_ldexpf(l_tot, -static_cast<int>(dsh)),
                        __builtin_ldexpf(rmax * inv_l * (1.0f / 32767.0f), e));
    }
}

// The per-range statistics of a partial row: the reference score m in true
// units (f64), the sum l = sum_t 2^(c (x_t - m)), and the scale of the 16-bit
// codes of the range's normalised context O / l.
struct RangeStat {
    double m;
    float l;
    float o_scale;
};
static_assert(sizeof(RangeStat) == 16, "partial statistics record");

// out[b, row, :] = sum_s (w_s l_s / L) (O_s / l_s) over the ranges with
// l_s > 0, w_s = 2^(c (m_s - m*)) with m* the reference of largest c m_s and
// L = sum_s w_s l_s; zero when no range saw a token, NaN when a range's sum
// l_s is NaN (its query row has a NaN or infinite element).  The weights are
// formed before they meet the codes, so no intermediate leaves the float
// range.
//
// four 16-bit codes (two dwords, low half first) as floats
__device__ __forceinline__ float4 codes4_to_f32(uint2 c) {
    return make_float4(static_cast<float>(static_cast<int16_t>(c.x & 0xFFFFu)),
                       static_cast<float>(static_cast<int16_t>(c.x >> 16)),
                       static_cast<float>(static_cast<int16_t>(c.y & 0xFFFFu)),
                       static_cast<float>(static_cast<int16_t>(c.y >> 16)));
}

// key = sign(c) m of a live range (-inf otherwise): c (m - m*) = |c| (key - max key)
__device__ __forceinline__ double range_key(const RangeStat& st, bool cpos) {
    return st.l > 0.0f ? (cpos ? st.m : -st.m) : -INFINITY;
}
__device__ __forceinline__ float range_weight(const RangeStat& st, bool cpos, double cabs, double kmax) {
    return st.l > 0.0f ? __builtin_amdgcn_exp2f(static_cast<float>(cabs * (range_key(st, cpos) - kmax)))
                       : 0.0f;
}
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Block = 256 threads = one (b, row) and one quarter (128 columns) of the
// output row: the largest key and L over all ranges first, then 8 groups of
// 32 lanes, group g summing the ranges s = g mod 8 (lane = 4 columns), and one
// reduction over the groups in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeGroups = 8;
constexpr int kMergeCols = kKvLora / 4;
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(const int16_t* __restrict__ part_o,
                                                                  const RangeStat* __restrict__ part_ml,
                                                                  int B, int QH, int n_splits, float c,
                                                                  float* __restrict__ out) {
    __shared__ double s_k[kMergeThreads / 64];
    __shared__ float s_l[kMergeThreads / 64];
    __shared__ float4 s_acc[kMergeGroups][32];
    const int tid = threadIdx.x;
    const int64_t br = blockIdx.x >> 2;  // b * QH + row
    const int col0 = (blockIdx.x & 3) * kMergeCols;
    const int64_t stride = static_cast<int64_t>(B) * QH;
    const bool cpos = c >= 0.0f;
    const double cabs = fabs(static_cast<double>(c));

    double kmax = -INFINITY;
    int bad = 0;  // a NaN sum
    for (int s = tid; s < n_splits; s += kMergeThreads) {
        const RangeStat st = part_ml[s * stride + br];
        kmax = fmax(kmax, range_key(st, cpos));
        bad |= !(st.l >= 0.0f);
    }
    kmax = wave_max_f64(kmax);
    if ((tid & 63) == 0) s_k[tid >> 6] = kmax;
    __syncthreads();
    bad = __syncthreads_or(bad);
    kmax = fmax(fmax(s_k[0], s_k[1]), fmax(s_k[2], s_k[3]));
    float lsum = 0.0f;
    if (kmax > -INFINITY) {
        for (int s = tid; s < n_splits; s += kMergeThreads) {
            const RangeStat st = part_ml[s * stride + br];
            lsum += range_weight(st, cpos, cabs, kmax) * st.l;
        }
    }
    lsum = wave_sum_f32(lsum);
    if ((tid & 63) == 0) s_l[tid >> 6] = lsum;
    __syncthreads();
    lsum = (s_l[0] + s_l[1]) + (s_l[2] + s_l[3]);
    const float inv_l = lsum > 0.0f ? 1.0f / lsum : 0.0f;

    const int grp = tid >> 5, q = tid & 31;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lsum > 0.0f) {
        // group grp sums the ranges grp, grp + 8, ... in that order, eight of
        // them loaded at once (indices past the last range repeat range grp
        // with weight 0: its codes are finite)
        const int16_t* po = part_o + br * kKvLora + col0 + 4 * q;
        for (int s0 = grp; s0 < n_splits; s0 += 8 * kMergeGroups) {
            RangeStat st8[8];
            uint2 o8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = s0 + u * kMergeGroups;
                const int sc = s < n_splits ? s : grp;
                st8[u] = part_ml[sc * stride + br];
                o8[u] = *reinterpret_cast<const uint2*>(po + static_cast<int64_t>(sc) * stride * kKvLora);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const RangeStat st = st8[u];
                const float ws = s0 + u * kMergeGroups < n_splits
                                     ? range_weight(st, cpos, cabs, kmax) * st.l * inv_l * st.o_scale
                                     : 0.0f;
                const float4 v = codes4_to_f32(o8[u]);
                acc.x += ws * v.x;
                acc.y += ws * v.y;
                acc.z += ws * v.z;
                acc.w += ws * v.w;
            }
        }
    }
    s_acc[grp][q] = acc;
    __syncthreads();
    if (grp == 0) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int g2 = 0; g2 < kMergeGroups; ++g2) {
            const float4 v = s_acc[g2][q];
            a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
        }
        if (bad) a = make_float4(NAN, NAN, NAN, NAN);
        *reinterpret_cast<float4*>(out + br * kKvLora + col0 + 4 * q) = a;
    }
}

// The same merge for at most 64 ranges: one wave per (b, row), lane s < n
// holding range s's statistics, every lane summing 8 columns over the ranges.
constexpr int kMergeRowsPerBlock = 4;
__global__ __launch_bounds__(64 * kMergeRowsPerBlock) void lse_merge_rows_kernel(
    const int16_t* __restrict__ part_o, const RangeStat* __restrict__ part_ml, int B, int QH,
    int n_splits, float c, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t br = static_cast<int64_t>(blockIdx.x) * kMergeRowsPerBlock + (threadIdx.x >> 6);
    const int64_t stride = static_cast<int64_t>(B) * QH;
    if (br >= stride) return;
    const bool cpos = c >= 0.0f;
    const double cabs = fabs(static_cast<double>(c));
    RangeStat st{0.0, 0.0f, 0.0f};
    if (lane < n_splits) st = part_ml[lane * stride + br];
    const bool bad = __any(!(st.l >= 0.0f));  // a NaN sum
    const double kmax = wave_max_f64(range_key(st, cpos));
    const float wgt = kmax > -INFINITY ? range_weight(st, cpos, cabs, kmax) : 0.0f;
    const float lsum = wave_sum_f32(wgt * st.l);
    // weight of range `lane`'s codes (0 for an empty range)
    const float wsc = lsum > 0.0f ? wgt * st.l * (1.0f / lsum) * st.o_scale : 0.0f;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    const int16_t* po = part_o + br * kKvLora + 8 * lane;
    // Only ranges up to the last one that saw a token are read (the ranges
    // past a sequence's end are empty).  Eight ranges' codes are loaded at
    // once, without branches: the codes of an empty range are not written,
    // but any int16 value is finite, so its zero weight adds exactly 0;
    // indices past the last live range repeat it with weight 0.
    const uint64_t live = __ballot(st.l != 0.0f);  // (NaN sums count as live)
    const int n_live = live != 0 ? 64 - __clzll(static_cast<long long>(live)) : 0;
    for (int s2 = 0; s2 < n_live; s2 += 8) {
        uint4 o8[8];
        float w8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int su = s2 + u < n_live ? s2 + u : n_live - 1;
            w8[u] = s2 + u < n_live ? __shfl(wsc, su, 64) : 0.0f;
            o8[u] = *reinterpret_cast<const uint4*>(po + static_cast<int64_t>(su) * stride * kKvLora);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w2 = w8[u];
            const float4 v0 = codes4_to_f32(make_uint2(o8[u].x, o8[u].y));
            const float4 v1 = codes4_to_f32(make_uint2(o8[u].z, o8[u].w));
            a0.x += w2 * v0.x; a0.y += w2 * v0.y; a0.z += w2 * v0.z; a0.w += w2 * v0.w;
            a1.x += w2 * v1.x; a1.y += w2 * v1.y; a1.z += w2 * v1.z; a1.w += w2 * v1.w;
        }
    }
    if (bad) a0 = a1 = make_float4(NAN, NAN, NAN, NAN);
    float* o = out + br * kKvLora + 8 * lane;
    *reinterpret_cast<float4*>(o) = a0;
    *reinterpret_cast<float4*>(o + 4) = a1;
}

void launch_merge(const int16_t* part_o, const RangeStat* part_ml, int B, int QH, int n_splits, float c,
                  float* out, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(B) * QH;
    if (n_splits <= 64) {
        hipLaunchKernelGGL(lse_merge_rows_kernel,
                           dim3(static_cast<uint32_t>((rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock)),
                           dim3(64 * kMergeRowsPerBlock), 0, stream, part_o, part_ml, B, QH, n_splits, c, out);
    } else {
        hipLaunchKernelGGL(lse_merge_kernel, dim3(static_cast<uint32_t>(4 * rows)), dim3(kMergeThreads),
                           0, stream, part_o, part_ml, B, QH, n_splits, c, out);
    }
}

}  // namespace

size_t splitT_workspace_bytes(int B, int Q, int H, int n_splits) {
    const size_t rows = static_cast<size_t>(n_splits) * B * Q * H;
    return rows * kKvLora * sizeof(int16_t) + rows * 4 * sizeof(float);
}

int launch_absorb_decode(const DecodeLaunch& d, hipStream_t stream, bool merge) {
    DecodeArgs a;
    a.q_lat = d.q_lat;
    a.q_rope = d.q_rope;
    a.codes = d.codes;
    a.scales = d.scales;
    a.exps = d.exps;
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
        a.part_o = static_cast<int16_t*>(d.workspace);
        a.part_ml = reinterpret_cast<float*>(a.part_o + rows * kKvLora);
    }
    const int64_t blocks = static_cast<int64_t>(d.B) * a.n_splits * a.n_rb;
    // from 4 blocks per compute unit on, the order that balances the XCDs
    // (the headline-sized launches, one block per unit, keep the order that
    // shares each sequence's queries within one XCD)
    a.unit_rr = blocks >= kUnitRrBlocks && (static_cast<int64_t>(d.B) * a.n_splits) % 8 == 0;
    if (d.exps != nullptr)
        hipLaunchKernelGGL(absorb_decode_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads),
                           0, stream, a);
    else
        hipLaunchKernelGGL(absorb_decode_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads),
                           0, stream, a);
    if (hipGetLastError() != hipSuccess) return -1;
    if (d.n_splits > 1 && merge) {
        launch_merge(a.part_o, reinterpret_cast<const RangeStat*>(a.part_ml), d.B, a.QH, d.n_splits, a.c,
                     d.out, stream);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

int launch_lse_merge(const void* partials, int B, int QH, int n_splits, float softmax_scale,
                     float* out, hipStream_t stream) {
    const size_t rows = static_cast<size_t>(n_splits) * B * QH;
    const int16_t* po = static_cast<const int16_t*>(partials);
    const RangeStat* ml = reinterpret_cast<const RangeStat*>(po + rows * kKvLora);
    launch_merge(po, ml, B, QH, n_splits, softmax_scale * 1.4426950408889634f, out, stream);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
