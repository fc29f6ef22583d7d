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
//   tiles ahead (three raw fp8 buffers); two tiles ahead, all 256 threads
//   decode a raw tile once, exactly, into an fp16 Lc tile (three buffers,
//   rows padded to 1088 bytes) and turn its scales into (s_Lc, s_Rc,
//   s_Lc / 2^e); the Rc codes stay in the raw tile;
//
//   score pass  S^T[token, row] = dec(KV)[token, 0:576] . q[row, 0:576]
//               36 MFMA 32x32x16 f16 per tile, A = fp16 Lc rows
//               (ds_read_b128) and the Rc codes converted in registers, B =
//               the wave's 32 query rows resident in VGPRs as fp16 (each row
//               scaled by a power of two so its largest element sits in
//               [2^12, 2^13): every bf16 element above 2^-27 of the row maximum
//               is then exact in fp16); separate accumulators for the Lc (512)
//               and Rc (64) columns so the two row scales are applied after the
//               dot product;
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
//               MFMA K order), the Lc operand is read with the LDS transpose
//               load ds_read_b64_tr_b16, and 2^e normalises the largest Lc
//               scale of the block's token range below 1 so p * s / 2^e fits
//               fp16.  fp16 rather than bf16 carries the probabilities: one
//               bf16 rounding of p already costs ~1e-3 of the output, fp16
//               ~1e-4, at the same MFMA rate, and every e4m3 value is exact in
//               fp16.
//
// Both passes therefore run on fp16 MFMA: every e4m3 value and every
// (row-scaled) bf16 query element is exact in fp16, so the score products are
// the exact products of the dequantized cache and the queries.
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
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kTT = 32;                          // tokens per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;       // 128 query rows
constexpr int64_t kUnitRrBlocks = 1024;           // 4 blocks per compute unit of MI355X
constexpr int kNBuf = 3;                         // raw Lc, decoded and scale buffers each
constexpr int kRcBufs = 4;                       // raw Rc buffers
constexpr int kRawLcBytes = kTT * kKvLora;       // 16384: raw Lc codes of a tile
constexpr int kRawRcBytes = kTT * kRope;         // 2048: raw Rc codes of a tile
constexpr int kLcStride = 2 * kKvLora + 64;      // 1088: fp16 Lc row + padding
constexpr int kLcBytes = kTT * kLcStride;        // 34816

constexpr int kScoreAhead = 3;                   // score operand loads in flight
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

// Score MFMAs with their accumulator pinned to VGPRs, leaving all 256 AGPRs to
// the context accumulator.  An MFMA needs two wait states after a VALU
// write of one of its operands, which the compiler does not insert for
// inline assembly: the variants taking an operand converted by VALU
// instructions (NOP = true) start with s_nop 1; the others take operands
// loaded from LDS (the load's s_waitcnt orders them) or registers written
// long before.  Back-to-back MFMAs on the same accumulator need no wait
// state.  The first MFMA of a chain starts from a zero C operand.
template <bool NOP>
__device__ __forceinline__ void mfma_score_first(f32x16_t& acc, const f16x8_t& a,
                                                 const f16x8_t& b) {
    if constexpr (NOP)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
template <bool NOP>
__device__ __forceinline__ void mfma_score(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
    if constexpr (NOP)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Context MFMA with the accumulator pinned to AGPRs; its operands are the
// packed probabilities (written before the phase starts) and LDS loads.
__device__ __forceinline__ void mfma_ctx(f32x16_t& acc, const f16x8_t& a, const f16x8_t& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
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

// bf16 bits -> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 bf16 values times 2^-k -> 8 fp16 values (exact for the scaled range)
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 q, int k) {
    uint4 r;
    r.x = pack_f16x2(__builtin_ldexpf(bf16_lo(q.x), -k), __builtin_ldexpf(bf16_hi(q.x), -k));
    r.y = pack_f16x2(__builtin_ldexpf(bf16_lo(q.y), -k), __builtin_ldexpf(bf16_hi(q.y), -k));
    r.z = pack_f16x2(__builtin_ldexpf(bf16_lo(q.z), -k), __builtin_ldexpf(bf16_hi(q.z), -k));
    r.w = pack_f16x2(__builtin_ldexpf(bf16_lo(q.w), -k), __builtin_ldexpf(bf16_hi(q.w), -k));
    return r;
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
//   raw Lc  codes of t, chunk q (< 32), at chunk 32 t + (q ^ 8 ((t >> 2) & 1));
//   raw Rc  codes of t, chunk c (< 4), at chunk 32 c + t.  The tile copies
//           place the chunks there (each lane picks its source chunk).
//   fp16   Lc values of t, chunk c (< 64), at byte 1088 t + 16 (c ^ ((t >> 2) & 3)).
// With 64 LDS banks of 4 bytes every read and write below touches each bank
// once per 256 bytes: the score operand reads (16 tokens, one chunk each),
// the transpose reads (4 tokens x 64 bytes per 32 lanes), the decode reads
// (tokens t and t + 4) and writes (tokens t and t + 4, both chunk parities).

// kMX: block-scaled rows (e4m3 codes with one ue8m0 exponent per 32 values).
// Each token's largest Lc and Rc block exponents E_L, E_R take the place of
// the per-row scales (s = 2^(E - 127)), and its codes are decoded to fp16
// times 2^(E_block - E_L) (or - E_R): exact for blocks within 2^15 of their
// segment's largest, smaller blocks round to fp16 subnormals.  The tile's
// exponent bytes (576) are copied where the per-row path copies its scale
// pairs (256), and the Rc codes cycle through three buffers instead of four
// to make room.
template <bool kMX>
__global__ __launch_bounds__(kThreads, 1) void absorb_decode_kernel(DecodeArgs p) {
    constexpr int kRcB = kMX ? 3 : kRcBufs;                  // raw Rc buffers
    // copied scales, or exponents (576 bytes from byte 0 or 2 of a 4-byte word)
    constexpr int kScBytes = kMX ? kMxTileExpBytes + 16 : 8 * kTT;
    __shared__ __attribute__((aligned(16))) uint8_t s_raw[kNBuf][kRawLcBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_rc[kRcB][kRawRcBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_lc[kNBuf][kLcBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_scb[kNBuf][kScBytes];  // copied (Lc, Rc) scales or exponents
    __shared__ __attribute__((aligned(16))) float s_scd[kNBuf][3 * kTT];  // s_Lc, s_Rc, s_Lc / 2^e
    auto rc_buf = [](int tile) { return kMX ? tile % kRcB : tile & (kRcBufs - 1); };
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
    //      are the fp16 tile buffers (waves 0-2) and raw buffers 1 and 2
    //      (wave 3), all free until the first tile is decoded.  The rope
    //      parts (128 bytes a row) load directly.
    const uint8_t* const q_stage = w < kNBuf ? &s_lc[w][0] : &s_raw[0][0] + kRawLcBytes;
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
    uint4 qv[36];
    {
        const int64_t qrow = static_cast<int64_t>(b) * p.QH + (row_ok ? row : 0);
        const uint4* qr = reinterpret_cast<const uint4*>(p.q_rope + qrow * kRope);
#pragma unroll
        for (int r = 0; r < 4; ++r) qv[32 + r] = qr[4 * g + r];
    }


    // ---- tile copies.  Wave w issues the 1 KiB copies i = w + 4k of a tile;
    //      the 16 bytes of lane l land at chunk 64 i + l of the raw Lc buffer
    //      (i < 16) or at chunk 64 (i - 16) + l of the raw Rc buffer, whose
    //      source chunk (token, offset in the token's row) follows the raw
    //      layouts.  Copy k < 4 (Lc) takes token 2 w + lane / 32 + 8 k, whose
    //      chunk swizzle does not depend on k; copy 4 (i = 16, 17) takes Rc
    //      chunk 2 (i - 16) + lane / 32 of token lane % 32.
    auto dma_tl = [&](int ln) { return 2 * w + (ln >> 5); };  // token of the wave's Lc copy 0
    auto dma_lc = [&](int ln) {
        return dma_tl(ln) * kRowBytes + 16 * ((ln & 31) ^ (8 * ((dma_tl(ln) >> 2) & 1)));
    };
    auto dma_rc = [&](int ln) { return (ln & 31) * kRowBytes + kKvLora + 16 * (2 * (w & 1) + (ln >> 5)); };
    // The copies of a tile: tile i goes to raw Lc and scale buffer lbuf
    // (= i % 3) and raw Rc buffer i % 4.  Copy slot k < 4 of wave w is its Lc
    // copy k; slot 4 is the Rc copy of wave w (waves 0 and 1) or the tile's 32
    // (Lc, Rc) scale pairs, 4 bytes per lane (wave 3): waves 0, 1 and 3 issue
    // five copies per tile, wave 2 four.  Tiles past the range are replaced
    // by the last tile (a harmless re-copy into free buffers).  The copies
    // are range-checked at the range's end: rows past it arrive as zero codes
    // and zero scales (masked tokens, whose weight is 0).  The per-lane byte
    // offsets do not depend on the tile; copy k's first row (8 k) goes into
    // the base.
    auto issue_copy = [&](int tile, int lbuf, int k, int ln) {
        const int rbuf = rc_buf(tile);  // (before the clamp)
        tile = tile < ntiles ? tile : ntiles - 1;
        const int64_t t0 = ts + static_cast<int64_t>(tile) * kTT;
        const uint8_t* base = p.codes + (row_base + t0) * kRowBytes;
        const int valid = static_cast<int>(te - t0 < kTT ? te - t0 : kTT);  // (uniform, >= 1)
        if (k < 4) {
            const int rows = valid - 8 * k > 0 ? valid - 8 * k : 0;
            copy_to_lds_b128_rc(base + 8 * k * kRowBytes, static_cast<uint32_t>(rows * kRowBytes),
                                static_cast<uint32_t>(dma_lc(ln)),
                                lds_addr(&s_raw[lbuf][1024 * (w + kWaves * k)]));
        } else if (w < 2) {
            copy_to_lds_b128_rc(base, static_cast<uint32_t>(valid * kRowBytes),
                                static_cast<uint32_t>(dma_rc(ln)), lds_addr(&s_rc[rbuf][1024 * w]));
        } else if (w == 3) {
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
#pragma unroll
        for (int k = 0; k < 5; ++k) issue_copy(tile, tile % kNBuf, k, ln);
    };

    // the first tile is in flight with the queries (tiles 1 and 2 go to
    // buffers that stage the queries)
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

    // ---- query row l32 of this wave: B operand of the score MFMA, fp16 after
    //      scaling the row by 2^-kq so that its largest magnitude lies in
    //      [2^12, 2^13): every bf16 element above 2^-27 of the row maximum
    //      converts exactly.  Lc k-step ks holds columns 16 ks + 8 g .. +8;
    //      Rc k-step r holds rope columns 32 g + 8 r .. +8 (the Rc operand
    //      below takes the same order).  Rows past Q*H (block padding) reuse
    //      row 0; their results are never stored.
    wait_all_copies();  // (the queries, tile 0 and the scale loads)
#pragma unroll
    for (int ks = 0; ks < 32; ++ks)
        qv[ks] = lds_load<uint4>(q_stage, 1024 * l32 + 16 * ((2 * ks + g) ^ (l32 & 15)));
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
            kq = static_cast<int>((__float_as_uint(qmax) >> 23) & 0xFF) - 127 - 12;
            kq = kq < -100 ? -100 : (kq > 120 ? 120 : kq);
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
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
        pin(qv[ks].x); pin(qv[ks].y); pin(qv[ks].z); pin(qv[ks].w);
        qv[ks] = bf16x8_to_f16(qv[ks], kq);
    }

    // ---- per-lane LDS offsets
    // score A operand, Lc k-step ks: token l32, chunk 2 ks + g
    const int hsw = (l32 >> 2) & 3;
    const int sc_base0 = l32 * kLcStride + 16 * (g ^ hsw);        // ks even (+64 (ks >> 1))
    const int sc_base1 = l32 * kLcStride + 16 * ((2 + g) ^ hsw);  // ks odd
    // score A operand, Rc: token l32, chunks 2 g and 2 g + 1
    // (token l32, chunks 2 g and 2 g + 1: byte 16 lane of the raw Rc layout)
    // context B operand: lane (G = lane / 16, gi = lane % 16) of k-group g
    // takes token 4 g + 8 h + gi / 4 (+ 16 kc) at dims 32 dt + 16 (G % 2) +
    // 4 (gi % 4) for its transpose load h
    const int G = lane >> 4, gi = lane & 15;
    const int cG = 2 * (G & 1) + ((gi & 3) >> 1);
    const int tb0 = (4 * g + (gi >> 2)) * kLcStride + 16 * (cG ^ (g & 3)) + 8 * (gi & 1);
    const int tb1 = (4 * g + 8 + (gi >> 2)) * kLcStride + 16 * (cG ^ ((g + 2) & 3)) + 8 * (gi & 1);
    // decode: lane 16 a + 8 bb + s of wave w converts token 8 w + a + 4 bb,
    // raw chunks 8 j + s (j < 4) into fp16 chunks 16 j + 2 s, 16 j + 2 s + 1
    const int d_bb = (lane >> 3) & 1, d_s = lane & 7;
    const int d_t = 8 * w + (lane >> 4) + 4 * d_bb;
    // (raw chunk 8 j + s sits at 8 (j ^ bb) + s; fp16 chunk 2 s + 1 is
    //  chunk 2 s with bit 4 of the byte offset flipped)
    const int d_rA = 512 * d_t + 16 * d_s + 128 * d_bb;         // j = 0, 2 (+256); j odd: ^ 128
    const int d_hs = (d_t >> 2) & 3;
    const int d_wA = d_t * kLcStride + 16 * ((2 * d_s) ^ d_hs);  // + 256 j; odd chunk: ^ 16

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
    // decode(tile): raw codes -> fp16 Lc tile, scales -> (s_Lc, s_Rc, s_Lc/2^e)
    uint4 draw[2];
    auto decode_load = [&](int buf, int j) {  // raw chunk 8 j + s
        const uint8_t* raw = &s_raw[buf][0];
        draw[j & 1] = lds_load<uint4>(raw, ((j & 1) ? (d_rA ^ 128) : d_rA) + 256 * (j >> 1));
    };
    // block-scaled rows: for the lane's four Lc blocks 4 j + s / 2 (s = lane
    // % 8; the token's 8 lanes cover its 16 blocks) the exponent relative to
    // the token's largest, E_block - E_L >= -128 as a signed byte j of
    // mx_pack (below 2^-128 the fp16 value is 0 either way)
    uint32_t mx_pack = 0;
    auto mx_prep = [&](int buf) {
        if constexpr (kMX) {
            // (the lane's token and block rebuilt from a fresh lane id, so that
            // no offset stays live across the tile loop)
            const int ln = fresh_lane_id();
            const int tok = 8 * w + (ln >> 4) + 4 * ((ln >> 3) & 1);
            const uint8_t* ex = &s_scb[buf][mx_shift + kMxBlocksPerRow * tok + ((ln & 7) >> 1)];
            int b[4];
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = ex[4 * j];
                m = max(m, static_cast<uint32_t>(b[j]));
            }
            m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x4E, 0xF, 0xF, false)));
            m = max(m, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(m), 0x141, 0xF, 0xF, false)));
            mx_pack = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = b[j] - static_cast<int>(m);
                mx_pack |= (static_cast<uint32_t>(d < -128 ? -128 : d) & 0xFFu) << (8 * j);
            }
        }
    };
    auto decode_store = [&](int buf, int j, int half) {
        uint8_t* lc = &s_lc[buf][0];
        const uint4 r = draw[j & 1];
        uint4 v;
        if constexpr (kMX) {
            const float f = __builtin_ldexpf(1.0f, static_cast<int>(mx_pack << (24 - 8 * j)) >> 24);
            v = half == 0 ? dec8_f16s(r.x, r.y, f) : dec8_f16s(r.z, r.w, f);
        } else {
            v = half == 0 ? dec8_f16(r.x, r.y) : dec8_f16(r.z, r.w);
        }
        *reinterpret_cast<uint4*>(lc + (half == 0 ? d_wA : (d_wA ^ 16)) + 256 * j) = v;
    };
    // (every wave writes the same values: lane t < 32 the signed s_Lc / 2^ex,
    // s_Rc / 2^ex of token t, lane 32 + t the value s_Lc / 2^e of token t,
    // twice)
    auto decode_scales = [&](int buf, int tile) {
        float2 sc;
        if constexpr (kMX) {
            // 2^(E_L - 127), 2^(E_R - 127) of token l32; zero past the range
            const uint8_t* base = &s_scb[buf][0];
            const int tok = fresh_lane_id() & 31;
            const int a = mx_shift + kMxBlocksPerRow * tok;
            const uint32_t rp = mx_rc_pair(base, a);
            const bool in = tok < tile_valid(tile);
            sc.x = in ? mx_pow2(mx_lc_max(base, a)) : 0.0f;
            sc.y = in ? mx_pow2(static_cast<int>(max(rp & 0xFFu, rp >> 8))) : 0.0f;
        } else {
            (void)tile;
            sc = *reinterpret_cast<const float2*>(&s_scb[buf][8 * l32]);
        }
        float* d = &s_scd[buf][0];
        const float v0 = __builtin_ldexpf(g == 0 ? sgn * sc.x : sc.x, g == 0 ? -ex : -e);
        const float v1 = g == 0 ? __builtin_ldexpf(sgn * sc.y, -ex) : v0;
        d[g == 0 ? l32 : 2 * kTT + l32] = v0;
        d[g == 0 ? kTT + l32 : 2 * kTT + l32] = v1;
    };

    // x(tile) = s_Lc accL + s_Rc accR for row l32 and tokens 8 (j / 4) + 4 g +
    // j % 4 of the tile (the accumulator order), masked past the row's limit.
    // The token scales of the lane's 16 tokens are loaded into registers
    // during the score MFMAs (s_Rc, s_Lc) and before the accumulator drain
    // (s_Lc / 2^e), so that the softmax does not wait on LDS.
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

    // score(tile): accR = dec(Rc) . q_rope (4 MFMAs, first), then accL =
    // dec(Lc) . q_lat (32 MFMAs); step ks < 36 issues one MFMA so that other
    // work can sit between the steps.  The Rc codes of the lane's token are
    // loaded before the phase (rope_load) and converted one MFMA ahead.
    f16x8_t aq[kScoreAhead];
    uint4 rope[2];
    f16x8_t ropeop;
    float mx_rf = 1.0f;  // block-scaled rows: 2^(E of Rc block g - E_R) of the lane's token
    auto rope_load = [&](int tile) {
        const uint8_t* rc = &s_rc[rc_buf(tile)][0];
        const int ln = fresh_lane_id();
        const int rope_off = 16 * (ln + (ln & 32));  // (= 16 (64 g + l32))
        rope[0] = lds_load<uint4>(rc, rope_off);
        rope[1] = lds_load<uint4>(rc, rope_off + 16 * 32);
        if constexpr (kMX) {
            const uint32_t rp = mx_rc_pair(&s_scb[tile % kNBuf][0], mx_shift + kMxBlocksPerRow * (ln & 31));
            const int eg = static_cast<int>((ln & 32) ? rp >> 8 : rp & 0xFFu);
            mx_rf = __builtin_ldexpf(1.0f, eg - static_cast<int>(max(rp & 0xFFu, rp >> 8)));
        }
    };
    auto rope_operand = [&](int r) {
        const uint4 c4 = rope[r >> 1];
        if constexpr (kMX)
            ropeop = __builtin_bit_cast(f16x8_t, (r & 1) ? dec8_f16s(c4.z, c4.w, mx_rf) : dec8_f16s(c4.x, c4.y, mx_rf));
        else
            ropeop = __builtin_bit_cast(f16x8_t, (r & 1) ? dec8_f16(c4.z, c4.w) : dec8_f16(c4.x, c4.y));
    };
    auto score_begin = [&](int buf) {
        const uint8_t* lc = &s_lc[buf][0];
#pragma unroll
        for (int k = 0; k < kScoreAhead; ++k)
            aq[k] = lds_load<f16x8_t>(lc, (k & 1 ? sc_base1 : sc_base0) + 64 * (k >> 1));
        rope_operand(0);
    };
    auto score_step = [&](int buf, int ks) {
        const uint8_t* lc = &s_lc[buf][0];
        if (ks < 4) {
            const f16x8_t qb = __builtin_bit_cast(f16x8_t, qv[32 + ks]);
            if (ks == 0) mfma_score_first<true>(accR, ropeop, qb);
            else mfma_score<true>(accR, ropeop, qb);
            if (ks < 3) rope_operand(ks + 1);
        } else {
            const int kl = ks - 4;
            const f16x8_t a = aq[kl % kScoreAhead];
            const int kn = kl + kScoreAhead;
            if (kn < 32) aq[kl % kScoreAhead] = lds_load<f16x8_t>(lc, (kn & 1 ? sc_base1 : sc_base0) + 64 * (kn >> 1));
            const f16x8_t qb = __builtin_bit_cast(f16x8_t, qv[kl]);
            if (kl == 0) mfma_score_first<false>(accL, a, qb);
            else mfma_score<false>(accL, a, qb);
        }
    };

    // softmax(tile) in steps k < kSoftSteps of a few VALU instructions each,
    // so that they can sit between the context MFMAs of the previous tile:
    //   0-8    even k: x of token group k / 2 - 1 (k > 0), then the loads of
    //          s_Lc and s_Rc for group k / 2 (k < 8); one group of scales in
    //          flight at a time
    //   9-10   mask (tiles past the first visible-token limit) and the maximum
    //          of the lane's 16 scores
    //   11     the row maximum (with the other half of the wave)
    //   12     reference update
    //   13-20  p = 2^(c_row (x - ref) + dsh) for tokens 2 (k - 13) and
    //          2 (k - 13) + 1
    //   21-24  lsum = sum of the p (pairwise), loads of s_Lc / 2^e for token
    //          group k - 21
    //   25-28  P' = p s_Lc / 2^e for token group k - 25, and the lane's largest
    //          P' of the real tiles
    //   29-30  P' packed to fp16 as the A operand of context k-step k - 29
    constexpr int kSoftSteps = 31;
    uint4 pa[2], pn[2];  // P' of the tile in the context MFMAs, and of the next
    float mx_part = 0.0f, mx_pair = 0.0f, ref = 0.0f, lsum = 0.0f;
    float mxa = 0.0f, mxb = 0.0f, mxc = 0.0f, sum_t[8];
    bool restart = false;  // this lane's row raised its reference in this pass
    auto soft_step = [&](int k, int buf, int tile, bool real) {
        if (k < 9) {
            if (k % 2 == 1) return;
            const int q4 = k / 2;
            if (q4 > 0) {
                form_x(q4 - 1);
                pin(x[4 * q4 - 4]); pin(x[4 * q4 - 3]); pin(x[4 * q4 - 2]); pin(x[4 * q4 - 1]);
            }
            if (q4 < 4) {
                scales_load_l(buf, q4);
                scales_load_r(buf, q4);
            }
            return;
        }
        k -= 5;
        if (k == 4) {
            mask_x(tile);
            mxa = max3(x[0], x[1], x[2]);
            mxb = max3(x[3], x[4], x[5]);
            mxc = max3(x[6], x[7], x[8]);
            pin(mxa); pin(mxb); pin(mxc);
        } else if (k == 5) {
            const float d = max3(x[9], x[10], x[11]);
            const float f = max3(x[12], x[13], x[14]);
            mx_part = fmaxf(max3(mxa, mxb, mxc), max3(d, f, x[15]));
            pin(mx_part);
        } else if (k == 6) {
            mx_pair = pair_max(mx_part);
            pin(mx_pair);
        } else if (k == 7) {
            const float mx = mx_pair;
            const bool first = m_x == mask_val;  // nothing accumulated for this row yet
            const bool raise = !first && c_row * (mx - m_x) > kLazyLog2;
            m_x = real && (first || raise) ? mx : m_x;
            restart = restart || (real && raise);
            ref = m_x == mask_val ? 0.0f : m_x;
            pin(ref);
        } else if (k < 16) {
            const int j = 2 * (k - 8);
            pin(x[j]); pin(x[j + 1]);
            x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(c_row, x[j] - ref, dsh));
            x[j + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(c_row, x[j + 1] - ref, dsh));
            pin(x[j]); pin(x[j + 1]);
        } else if (k < 18) {
            scales_load_e(buf, k - 16);
            const int j0 = 4 * (k - 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sum_t[j0 + i] = x[2 * (j0 + i)] + x[2 * (j0 + i) + 1];
                pin(sum_t[j0 + i]);
            }
        } else if (k == 18) {
            scales_load_e(buf, 2);
            sum_t[0] = (sum_t[0] + sum_t[1]) + (sum_t[2] + sum_t[3]);
            sum_t[4] = (sum_t[4] + sum_t[5]) + (sum_t[6] + sum_t[7]);
            pin(sum_t[0]); pin(sum_t[4]);
        } else if (k == 19) {
            scales_load_e(buf, 3);
            lsum = sum_t[0] + sum_t[4];
            pin(lsum);
        } else if (k < 24) {
            const int q4 = k - 20;
            pin(x[4 * q4]); pin(x[4 * q4 + 1]); pin(x[4 * q4 + 2]); pin(x[4 * q4 + 3]);
            x[4 * q4 + 0] *= se4[q4].x;
            x[4 * q4 + 1] *= se4[q4].y;
            x[4 * q4 + 2] *= se4[q4].z;
            x[4 * q4 + 3] *= se4[q4].w;
            {
                const float t = max3(max3(pmax, x[4 * q4], x[4 * q4 + 1]), x[4 * q4 + 2], x[4 * q4 + 3]);
                pmax = real ? t : pmax;
            }
            pin(x[4 * q4]); pin(x[4 * q4 + 1]); pin(x[4 * q4 + 2]); pin(x[4 * q4 + 3]);
        } else {
            const int kc = k - 24;
            pn[kc].x = pack_f16x2(x[8 * kc + 0], x[8 * kc + 1]);
            pn[kc].y = pack_f16x2(x[8 * kc + 2], x[8 * kc + 3]);
            pn[kc].z = pack_f16x2(x[8 * kc + 4], x[8 * kc + 5]);
            pn[kc].w = pack_f16x2(x[8 * kc + 6], x[8 * kc + 7]);
            pin(pn[kc].x); pin(pn[kc].y); pin(pn[kc].z); pin(pn[kc].w);
        }
    };

    // context(tile): O[dt] += P (32 rows x 16 tokens) . dec(Lc) (16 tokens x
    // 32 dims), 32 MFMAs, operand loads kCtxAhead MFMAs ahead
    f16x8_t bq[kCtxAhead];
    auto context_begin = [&](int buf) {
        const uint8_t* lc = &s_lc[buf][0];
#pragma unroll
        for (int n = 0; n < kCtxAhead; ++n) bq[n] = ctx_operand(lc, tb0, tb1, n);
    };
    auto context_step = [&](int buf, int n, uint4 pk) {
        const uint8_t* lc = &s_lc[buf][0];
        const f16x8_t bv = bq[n % kCtxAhead];
        if (n + kCtxAhead < 32) bq[n % kCtxAhead] = ctx_operand(lc, tb0, tb1, n + kCtxAhead);
        mfma_ctx(O[n & 15], __builtin_bit_cast(f16x8_t, pk), bv);
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
    // Software pipeline (tile i): copy(i) is issued four tiles ahead and
    // waited for at the end of the next iteration, decode(i) runs two tiles
    // ahead; iteration i runs
    //   phase A: score(i + 1), with the decode of tile i + 2 between its
    //            MFMAs
    //   phase B: context(i), with the softmax steps of tile i + 1 between its
    //            MFMAs (the P' they pack feeds context(i + 1))
    // and the five copy slots of tile i + 4 spread over both phases (a burst
    // of copies stalls their issue while earlier misses are outstanding)
    // and one barrier, after the copies of tile i + 3 have landed.  Stages
    // past the last tile run on stale buffers and their results are never
    // used.
    auto end_barrier = [&]() {
        if (w == 2) barrier_after_copies<4>();
        else barrier_after_copies<5>();
    };
    // One pass over the token range (every pass also records each lane's
    // largest probability operand, which only a watched pass reads).
    auto run_pass = [&]() {
        if (ntiles > 0) {
            mx_prep(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                decode_load(0, j);
                decode_store(0, j, 0);
                decode_store(0, j, 1);
            }
            decode_scales(0, 0);
            end_barrier();  // tile 0 decoded; tile 1 landed, tile 2 may be in flight
            if constexpr (kMX) {
                // (tile 3's Rc codes and exponents reuse tile 0's buffers)
                rope_load(0);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue_tile(3);
            } else {
                issue_tile(3);  // (raw buffers of tile 0, decoded)
                rope_load(0);
            }
            score_begin(0);
            static_for<36>([&](auto kc) {
                constexpr int ks = decltype(kc)::value;
                score_step(0, ks);
                // decode of tile 1 between the score MFMAs (as in phase A)
                if constexpr (ks >= 6 && ks <= 30 && (ks - 6) % 8 == 0) decode_load(1, (ks - 6) / 8);
                if constexpr (ks == 7) mx_prep(1);
                if constexpr (ks >= 9 && ks <= 33 && (ks - 9) % 8 == 0) decode_store(1, (ks - 9) / 8, 0);
                if constexpr (ks >= 11 && ks <= 35 && (ks - 11) % 8 == 0) decode_store(1, (ks - 11) / 8, 1);
                if constexpr (ks == 35) decode_scales(1, 1);
            });
            mfma_acc_drain(accL, accR);
            static_for<kSoftSteps>([&](auto k) { soft_step(decltype(k)::value, 0, 0, true); });
            l_run += lsum;
            pa[0] = pn[0];
            pa[1] = pn[1];
            // tile 1 decoded, tile 2 landed; tile 0's Rc codes are read before
            // copy(4) reuses them
            end_barrier();
        }
        // iteration `it` with R = it % kNBuf known at compile time, so that
        // every LDS address is a lane offset plus an immediate
        auto iteration = [&](int it, auto rc) {
            constexpr int R = decltype(rc)::value;
            constexpr int B0 = R, B1 = (R + 1) % kNBuf, B2 = (R + 2) % kNBuf;
            const bool real_next = it + 1 < ntiles;
            // ---------------- phase A: score(it + 1), decode of tile it + 2,
            //                  copies of tile it + 4 into the buffers of tile
            //                  it + 1 (raw Lc, scales: decoded last iteration)
            //                  and tile it (raw Rc: scored last iteration)
            rope_load(it + 1);
            score_begin(B1);
            order();
            static_for<36>([&](auto kc) {
                constexpr int ks = decltype(kc)::value;
                score_step(B1, ks);
                // decode of tile it + 2 between the score MFMAs (loads well
                // ahead of their conversions and stores)
                if constexpr (ks >= 6 && ks <= 30 && (ks - 6) % 8 == 0) decode_load(B2, (ks - 6) / 8);
                if constexpr (ks == 7) mx_prep(B2);
                if constexpr (ks >= 9 && ks <= 33 && (ks - 9) % 8 == 0) decode_store(B2, (ks - 9) / 8, 0);
                if constexpr (ks >= 11 && ks <= 35 && (ks - 11) % 8 == 0) decode_store(B2, (ks - 11) / 8, 1);
                if constexpr (ks == 35) decode_scales(B2, it + 2);
                if constexpr (ks % 11 == 3) issue_copy(it + 4, B1, ks / 11, lane);
                order();
            });
            // ---------------- phase B: context(it) (it reads only buffers
            //                  written before the last barrier), softmax of
            //                  tile it + 1 (its result is only used when real)
            context_begin(B0);
            order();
            static_for<32>([&](auto nc) {
                constexpr int n = decltype(nc)::value;
                context_step(B0, n, n < 16 ? pa[0] : pa[1]);
                if constexpr (n == 0) mfma_acc_drain(accL, accR);
                if constexpr (n < kSoftSteps) soft_step(n, B1, it + 1, real_next);
                if constexpr (n % 11 == 5 && n / 11 < 2) issue_copy(it + 4, B1, 3 + n / 11, lane);
                order();
            });
            l_run += real_next ? lsum : 0.0f;
            pa[0] = pn[0];
            pa[1] = pn[1];
            end_barrier();  // tile it + 3 landed; tile it + 4 may be in flight
        };
        for (int it0 = 0; it0 < ntiles; it0 += kNBuf) {
            iteration(it0, std::integral_constant<int, 0>{});
            if (it0 + 1 < ntiles) iteration(it0 + 1, std::integral_constant<int, 1>{});
            if (it0 + 2 < ntiles) iteration(it0 + 2, std::integral_constant<int, 2>{});
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
// L = sum_s w_s l_s; zero when no range saw a token.  The weights are formed
// before they meet the codes, so no intermediate leaves the float range.
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
    for (int s = tid; s < n_splits; s += kMergeThreads) kmax = fmax(kmax, range_key(part_ml[s * stride + br], cpos));
    kmax = wave_max_f64(kmax);
    if ((tid & 63) == 0) s_k[tid >> 6] = kmax;
    __syncthreads();
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
        const int16_t* po = part_o + br * kKvLora + col0 + 4 * q;
        for (int s = grp; s < n_splits; s += kMergeGroups) {
            const RangeStat st = part_ml[s * stride + br];
            const uint2 o = *reinterpret_cast<const uint2*>(po + static_cast<int64_t>(s) * stride * kKvLora);
            const float ws = range_weight(st, cpos, cabs, kmax) * st.l * inv_l * st.o_scale;
            const float4 v = codes4_to_f32(o);
            acc.x += ws * v.x;
            acc.y += ws * v.y;
            acc.z += ws * v.z;
            acc.w += ws * v.w;
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
    const double kmax = wave_max_f64(range_key(st, cpos));
    const float wgt = kmax > -INFINITY ? range_weight(st, cpos, cabs, kmax) : 0.0f;
    const float lsum = wave_sum_f32(wgt * st.l);
    // weight of range `lane`'s codes (0 for an empty range)
    const float wsc = lsum > 0.0f ? wgt * st.l * (1.0f / lsum) * st.o_scale : 0.0f;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    const int16_t* po = part_o + br * kKvLora + 8 * lane;
    // eight ranges' codes loaded at once, without branches: the codes of an
    // empty range are not written, but any int16 value is finite, so its zero
    // weight adds exactly 0; indices past the last range repeat it with
    // weight 0
    for (int s2 = 0; s2 < n_splits; s2 += 8) {
        uint4 o8[8];
        float w8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int su = s2 + u < n_splits ? s2 + u : n_splits - 1;
            w8[u] = s2 + u < n_splits ? __shfl(wsc, su, 64) : 0.0f;
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
