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
// One block = 8 waves computes a 256 x 256 tile of out.  k runs in 8 chunks
// of 64: each thread loads 32 codes and 32 weights of the chunk two ahead
// into registers (loads that cover whole runs of a row) while the current
// chunk is multiplied; the codes are decoded exactly to bf16 (every e4m3 value is a
// bf16 value) on their way into LDS.  Operand rows in LDS are 144 bytes (64
// bf16 plus 16 bytes of padding), so the 16 rows one ds_read_b128 pass serves
// fall on 16 different 4-bank groups.  Wave w multiplies rows 128 (w / 4) ..
// +128 by columns 64 (w % 4) .. +64 with eight 32x32 accumulators (bf16 MFMA
// 32x32x16, f32 accumulation): 768 LDS bytes per MFMA.  Two waves share each
// SIMD.  The row's Lc scale multiplies the f32 sum, which is stored as f32 or
// rounded to bf16 (round to nearest even), with non-temporal stores.
//
// Blocks are ordered so that each XCD (every 8th block goes to the same one)
// works through a contiguous run of tiles: a column tile's 256 KiB of weights
// is read into that XCD's L2 once for all of its row tiles.
#include "kv8_device.hpp"
#include "kv8_internal.hpp"

namespace kv8 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPM = 256;                 // rows per block
constexpr int kPN = 256;                 // output columns per block
constexpr int kPK = 64;                  // k per chunk
constexpr int kPThreads = 512;
constexpr int kPRow = 2 * kPK + 16;      // 144: bytes per operand row in LDS
constexpr int kPTile = kPM * kPRow;      // 36864

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 8 codes (two dwords) -> 8 bf16 values, exact
__device__ __forceinline__ u32x4_t dec8_bf16(uint32_t w0, uint32_t w1) {
    const u32x4_t r = {dec2_bf16<false>(w0), dec2_bf16<true>(w0), dec2_bf16<false>(w1),
                       dec2_bf16<true>(w1)};
    return r;
}

template <bool kF32>
__global__ __launch_bounds__(kPThreads) void project_rows_kernel(const uint8_t* __restrict__ codes,
                                                                 const float* __restrict__ scales,
                                                                 int64_t n_rows,
                                                                 const uint16_t* __restrict__ wkv, int N,
                                                                 int64_t n_mtiles, void* __restrict__ out_v,
                                                                 float* __restrict__ rope_out) {
    // two operand buffers of A (decoded codes) then two of W; after the last
    // chunk the whole array stages the bf16 output tiles
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kPTile];
    __shared__ float s_rs[kPM];  // Lc scales of the block's rows
    uint8_t* const sA = smem;
    uint8_t* const sW = smem + 2 * kPTile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    int64_t bid = blockIdx.x;
    const int64_t nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    // consecutive tiles share a column tile
    const int64_t mt = bid % n_mtiles;
    const int nt = static_cast<int>(bid / n_mtiles);
    const int64_t m0 = mt * kPM;
    const int n0 = nt * kPN;

    // loader, per chunk: wave w brings operand rows 32 w .. +32.  Codes: lane
    // l reads 16 codes (chunk bytes 16 (l % 4) ..) of row 16 i + l / 4 for
    // i < 2, so one load covers 64 contiguous bytes of 16 rows.  Weights:
    // lane l reads 8 weights (16 bytes) of row 8 i + l / 8 for i < 4, so one
    // load covers the chunk's whole 128 bytes of 8 rows.  Rows past the end
    // re-read the last row and columns past N the last column (their results
    // are not stored).
    const uint8_t* arow[2];
    const uint16_t* wrow[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 32 * w + 16 * i + (lane >> 2);
        const int64_t m = m0 + r < n_rows ? m0 + r : n_rows - 1;
        arow[i] = codes + m * kRowBytes + 16 * (lane & 3);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * w + 8 * i + (lane >> 3);
        const int n = n0 + r < N ? n0 + r : N - 1;
        wrow[i] = wkv + static_cast<int64_t>(n) * kKvLora + 8 * (lane & 7);
    }

    // two register sets: set kc % 2 holds chunk kc
    u32x4_t ra[2][2], rw[2][4];
    auto gload = [&](int kc, int p) {
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[p][i] = *reinterpret_cast<const u32x4_t*>(arow[i] + kPK * kc);
#pragma unroll
        for (int i = 0; i < 4; ++i) rw[p][i] = *reinterpret_cast<const u32x4_t*>(wrow[i] + kPK * kc);
    };
    auto lstore = [&](int p, int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint8_t* a = sA + buf * kPTile + (32 * w + 16 * i + (lane >> 2)) * kPRow + 32 * (lane & 3);
            *reinterpret_cast<u32x4_t*>(a) = dec8_bf16(ra[p][i][0], ra[p][i][1]);
            *reinterpret_cast<u32x4_t*>(a + 16) = dec8_bf16(ra[p][i][2], ra[p][i][3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4_t*>(sW + buf * kPTile + (32 * w + 8 * i + (lane >> 3)) * kPRow +
                                        16 * (lane & 7)) = rw[p][i];
    };

    const int wm = 128 * (w >> 2), wn = 64 * (w & 3);
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // k-step ks of a chunk: lane (l32, g) supplies row l32 of each operand tile
    // at k = 16 ks + 8 g .. +8
    auto compute = [&](int buf) {
        const uint8_t* a = sA + buf * kPTile;
        const uint8_t* b = sW + buf * kPTile;
#pragma unroll
        for (int ks = 0; ks < kPK / 16; ++ks) {
            bf16x8_t av[4], bv[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *reinterpret_cast<const bf16x8_t*>(b + (wn + 32 * j + l32) * kPRow + 2 * (16 * ks + 8 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *reinterpret_cast<const bf16x8_t*>(a + (wm + 32 * i + l32) * kPRow + 2 * (16 * ks + 8 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };

    // chunk kc + 2 is loaded while chunk kc is multiplied; chunk kc + 1 goes
    // into LDS after chunk kc's products (its loads had one product phase)
    constexpr int kChunks = kKvLora / kPK;
    if (tid < kPM) s_rs[tid] = m0 + tid < n_rows ? scales[2 * (m0 + tid)] : 0.0f;
    gload(0, 0);
    gload(1, 1);
    lstore(0, 0);
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < kChunks; ++kc) {
        if (kc + 2 < kChunks) gload(kc + 2, kc % 2);  // (set kc % 2 is in LDS already)
        compute(kc & 1);
        // the other buffer was last read before the previous barrier
        if (kc + 1 < kChunks) lstore((kc + 1) % 2, (kc + 1) & 1);
        __syncthreads();
    }

    // epilogue: register r of accumulator (i, j) is row wm + 32 i + 8 (r / 4) +
    // 4 g + r % 4 and column wn + 32 j + l32
    const bool cols_ok = n0 + wn < N;  // (N - n0 is a multiple of 128)
    // The output is written once and not read back here: non-temporal stores
    // (8% faster on 8,192 x 32,768 than plain ones).
    if constexpr (kF32) {
        // 32 consecutive f32 (128 bytes) of one row per half-wave store.  The
        // lane's 64 row scales (rows wm + 32 i + 8 q + 4 g + 0..3) are read
        // at once; row lrow starts at out + (m0 + wm + lrow) * N + n0 + wn.
        float4 sc4[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) sc4[i][q] = *reinterpret_cast<const float4*>(&s_rs[wm + 32 * i + 8 * q + 4 * g]);
        auto scale_of = [&](int i, int r) {
            const float4 v = sc4[i][r >> 2];
            return (r & 3) == 0 ? v.x : (r & 3) == 1 ? v.y : (r & 3) == 2 ? v.z : v.w;
        };
        float* const ob = static_cast<float*>(out_v) + (m0 + wm + 4 * g) * static_cast<int64_t>(N) + n0 + wn + l32;
        auto store_all = [&](auto row_ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int urow = 32 * i + 8 * (r >> 2) + (r & 3);  // lrow - 4 g
                    const float sc = scale_of(i, r);
                    float* const p = ob + static_cast<int64_t>(urow) * N;
                    if (row_ok(urow)) {
                        __builtin_nontemporal_store(acc[i][0][r] * sc, p);
                        __builtin_nontemporal_store(acc[i][1][r] * sc, p + 32);
                    }
                }
        };
        // no row or column of the wave's tile past the end (wave-uniform, so
        // the stores of a whole tile run without per-row branches)
        const bool full = m0 + kPM <= n_rows && n0 + 64 * (__builtin_amdgcn_readfirstlane(w) & 3) < N;
        if (full)
            store_all([](int) { return true; });
        else
            store_all([&](int urow) { return m0 + wm + urow + 4 * g < n_rows && cols_ok; });
    } else {
        // each wave's 128 x 64 bf16 tile goes through LDS (rows of 144 bytes)
        // so that it leaves as 16-byte stores, 8 rows of 128 bytes per
        // instruction, instead of 2 bytes a lane
        uint16_t* out = static_cast<uint16_t*>(out_v);
        uint8_t* const st = smem + w * 128 * kPRow;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lrow = 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
                const float sc = s_rs[wm + lrow];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    *reinterpret_cast<uint16_t*>(st + lrow * kPRow + 2 * (32 * j + l32)) =
                        __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][r] * sc));
            }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int lrow = 8 * q + (lane >> 3);
            const int64_t m = m0 + wm + lrow;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + lrow * kPRow + 16 * (lane & 7));
            if (m < n_rows && cols_ok)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + m * N + n0 + wn + 8 * (lane & 7)));
        }
    }

    // Rc of the block's rows, written by the blocks of the first column tile:
    // thread t converts 32 codes of row t / 2
    const int lr = tid >> 1, lh = tid & 1;
    const int64_t am = m0 + lr < n_rows ? m0 + lr : n_rows - 1;
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
                        const uint16_t* w_kv_b, int N, void* out, bool out_f32, float* rope_out,
                        hipStream_t stream) {
    const int64_t n_mtiles = (n_rows + kPM - 1) / kPM;
    const int64_t blocks = n_mtiles * ((N + kPN - 1) / kPN);
    if (out_f32)
        hipLaunchKernelGGL(project_rows_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(kPThreads), 0,
                           stream, codes, scales, n_rows, w_kv_b, N, n_mtiles, out, rope_out);
    else
        hipLaunchKernelGGL(project_rows_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(kPThreads), 0,
                           stream, codes, scales, n_rows, w_kv_b, N, n_mtiles, out, rope_out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
