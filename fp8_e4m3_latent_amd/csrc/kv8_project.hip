// Non-absorbed projection of fp8 cache rows.  gfx950.
//
// Page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
// (colibri PR #299), commit message, attention_rows item: the non-absorbed
// prefill dequantizes Lc into a staging row for the kv_b matmul and reads Rc
// through the decode table.
//
//   out[m][n]  = bf16( s_Lc[m] * sum_k dec(code[m][k]) * W[n][k] ),  k < 512
//   rope[m][j] = s_Rc[m] * dec(code[m][512 + j]),                    j < 64
//
// W is bf16 [N][512] (row n holds output column n's weights, the layout of a
// linear layer's weight), so both MFMA operands are contiguous in k.
//
// One block = 4 waves computes a 128 x 128 tile of out.  k runs in 8 chunks
// of 64: each thread loads 32 codes of one row and 32 weights of one column
// of the chunk three ahead into registers while the current chunk is multiplied;
// the codes are decoded exactly to bf16 (every e4m3 value is a bf16 value)
// on their way into LDS.  Operand rows in LDS are 144 bytes (64 bf16 plus 16
// bytes of padding), so the 16 rows one ds_read_b128 pass serves fall on 16
// different 4-bank groups.  Wave w multiplies rows 64 (w / 2) .. +64 by
// columns 64 (w % 2) .. +64 with four 32x32 accumulators (bf16 MFMA 32x32x16,
// f32 accumulation); the row's Lc scale multiplies the f32 sum before the
// bf16 rounding (round to nearest even).
#include "kv8_device.hpp"
#include "kv8_internal.hpp"

namespace kv8 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPM = 128;                 // rows per block
constexpr int kPN = 128;                 // output columns per block
constexpr int kPK = 64;                  // k per chunk
constexpr int kPRow = 2 * kPK + 16;      // 144: bytes per operand row in LDS
constexpr int kPTile = kPM * kPRow;      // 18432

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 8 codes (two dwords) -> 8 bf16 values, exact
__device__ __forceinline__ u32x4_t dec8_bf16(uint32_t w0, uint32_t w1) {
    const u32x4_t r = {dec2_bf16<false>(w0), dec2_bf16<true>(w0), dec2_bf16<false>(w1),
                       dec2_bf16<true>(w1)};
    return r;
}

__global__ __launch_bounds__(256) void project_rows_kernel(const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales,
                                                           int64_t n_rows,
                                                           const uint16_t* __restrict__ wkv, int N,
                                                           int64_t n_mtiles,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ rope_out) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][kPTile];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][kPTile];
    __shared__ float s_rs[kPM];  // Lc scales of the block's rows

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    // consecutive blocks share a column tile (its weights stay in L2)
    const int64_t mt = static_cast<int64_t>(blockIdx.x) % n_mtiles;
    const int nt = static_cast<int>(static_cast<int64_t>(blockIdx.x) / n_mtiles);
    const int64_t m0 = mt * kPM;
    const int n0 = nt * kPN;

    // loader: thread t takes half h = t % 2 (32 k values) of operand row t / 2
    const int lr = tid >> 1, lh = tid & 1;
    const int64_t am = m0 + lr < n_rows ? m0 + lr : n_rows - 1;  // (rows past the end: not stored)
    const uint8_t* arow = codes + am * kRowBytes + 32 * lh;
    const uint16_t* wrow = wkv + static_cast<int64_t>(n0 + lr) * kKvLora + 32 * lh;

    // three register sets: set kc % 3 holds chunk kc
    u32x4_t ra[3][2], rw[3][4];
    auto gload = [&](int kc, int p) {
        ra[p][0] = *reinterpret_cast<const u32x4_t*>(arow + kPK * kc);
        ra[p][1] = *reinterpret_cast<const u32x4_t*>(arow + kPK * kc + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) rw[p][i] = *reinterpret_cast<const u32x4_t*>(wrow + kPK * kc + 8 * i);
    };
    auto lstore = [&](int p, int buf) {
        uint8_t* a = &sA[buf][lr * kPRow + 64 * lh];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<u32x4_t*>(a + 32 * i) = dec8_bf16(ra[p][i][0], ra[p][i][1]);
            *reinterpret_cast<u32x4_t*>(a + 32 * i + 16) = dec8_bf16(ra[p][i][2], ra[p][i][3]);
        }
        uint8_t* b = &sW[buf][lr * kPRow + 64 * lh];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(b + 16 * i) = rw[p][i];
    };

    const int wm = 64 * (w >> 1), wn = 64 * (w & 1);
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // k-step ks of a chunk: lane (l32, g) supplies row l32 of each operand tile
    // at k = 16 ks + 8 g .. +8
    auto compute = [&](int buf) {
        const uint8_t* a = &sA[buf][0];
        const uint8_t* b = &sW[buf][0];
#pragma unroll
        for (int ks = 0; ks < kPK / 16; ++ks) {
            bf16x8_t av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *reinterpret_cast<const bf16x8_t*>(a + (wm + 32 * i + l32) * kPRow + 2 * (16 * ks + 8 * g));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *reinterpret_cast<const bf16x8_t*>(b + (wn + 32 * j + l32) * kPRow + 2 * (16 * ks + 8 * g));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };

    // chunk kc + 3 is loaded while chunk kc is multiplied and goes into LDS
    // after chunk kc + 2's products: three product phases for its loads to land
    constexpr int kChunks = kKvLora / kPK;
    // the row scales go to LDS at the start, so that the epilogue does not
    // wait for their loads
    if (tid < kPM) s_rs[tid] = m0 + tid < n_rows ? scales[2 * (m0 + tid)] : 0.0f;
    gload(0, 0);
    gload(1, 1);
    gload(2, 2);
    lstore(0, 0);
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < kChunks; ++kc) {
        if (kc + 3 < kChunks) gload(kc + 3, kc % 3);  // (set kc % 3 is in LDS already)
        compute(kc & 1);
        // the other buffer was last read before the previous barrier
        if (kc + 1 < kChunks) lstore((kc + 1) % 3, (kc + 1) & 1);
        __syncthreads();
    }

    // epilogue: register r of accumulator (i, j) is row wm + 32 i + 8 (r / 4) +
    // 4 g + r % 4 and column wn + 32 j + l32.  Each wave's 64 x 64 bf16 tile
    // goes through LDS (rows of 144 bytes, in the first operand buffers, free
    // after the last barrier) so that it leaves as 16-byte stores, 8 rows of
    // 128 bytes per instruction, instead of 2 bytes a lane.
    uint8_t* const st = &sA[0][0] + w * 64 * kPRow;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lrow = 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
            const float s = s_rs[wm + lrow];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                *reinterpret_cast<uint16_t*>(st + lrow * kPRow + 2 * (32 * j + l32)) =
                    __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][r] * s));
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int lrow = 8 * q + (lane >> 3);
        const int64_t m = m0 + wm + lrow;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + lrow * kPRow + 16 * (lane & 7));
        if (m < n_rows) *reinterpret_cast<u32x4_t*>(out + m * N + n0 + wn + 8 * (lane & 7)) = v;
    }

    // Rc of the block's rows, written by the blocks of the first column tile:
    // thread t converts 32 codes of row t / 2
    if (nt == 0 && rope_out != nullptr && m0 + lr < n_rows) {
        const float s = scales[2 * am + 1];
        const uint8_t* rc = codes + am * kRowBytes + kKvLora + 32 * lh;
        float* ro = rope_out + am * kRope + 32 * lh;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(rc + 16 * i);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = dec2_bf16<false>(cw[q]), hi = dec2_bf16<true>(cw[q]);
                *reinterpret_cast<float4*>(ro + 16 * i + 4 * q) =
                    make_float4(__uint_as_float(lo << 16) * s, __uint_as_float(lo & 0xFFFF0000u) * s,
                                __uint_as_float(hi << 16) * s, __uint_as_float(hi & 0xFFFF0000u) * s);
            }
        }
    }
}

}  // namespace

int launch_project_rows(const uint8_t* codes, const float* scales, int64_t n_rows,
                        const uint16_t* w_kv_b, int N, uint16_t* out, float* rope_out,
                        hipStream_t stream) {
    const int64_t n_mtiles = (n_rows + kPM - 1) / kPM;
    const int64_t blocks = n_mtiles * (N / kPN);
    hipLaunchKernelGGL(project_rows_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       codes, scales, n_rows, w_kv_b, N, n_mtiles, out, rope_out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
