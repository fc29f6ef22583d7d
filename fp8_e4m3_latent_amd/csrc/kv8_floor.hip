// HBM floor for a kernel's byte traffic: one launch that reads the given
// byte ranges and writes the given number of bytes with plain 16-byte
// grid-stride loads and stores, and does nothing else.  A kernel that moves
// the same bytes cannot beat this by much; the ratio of its time to the
// floor's separates traffic cost from everything else the kernel does.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv8.h"

namespace {

constexpr int kFloorThreads = 256;
constexpr int kFloorBlocks = 8192;  // 32 per CU on 256 CUs

// one word per block keeps the loads alive; never read
__device__ uint32_t g_floor_sink[kFloorBlocks];

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Reads and writes interleave as in a kernel that produces while it reads:
// wave tile w writes dst words [64 w, 64 w + 64) after reading read words
// [64 r w, 64 r (w + 1)) of the range a then b (nr words, r = ceil(nr / nw)),
// each load a whole wave's 1 KiB of consecutive words.  Read words past the
// last tile (all of them when nw = 0) are read by a grid-stride tail.
__global__ __launch_bounds__(kFloorThreads) void stream_floor_kernel(const u32x4_t* __restrict__ a, int64_t na,
                                                                     const u32x4_t* __restrict__ b, int64_t nb,
                                                                     u32x4_t* __restrict__ dst, int64_t nw,
                                                                     int64_t r) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (kFloorThreads / 64);
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * (kFloorThreads / 64) + (threadIdx.x >> 6);
    const int64_t nr = na + nb;
    auto word = [&](int64_t k) {
        return k < na ? __builtin_nontemporal_load(a + k) : __builtin_nontemporal_load(b + (k - na));
    };
    u32x4_t acc = {0, 0, 0, 0};
    const int64_t tiles = (nw + 63) / 64;
    for (int64_t w = gw; w < tiles; w += waves) {
        const int64_t k0 = 64 * r * w + lane, k1 = 64 * r * (w + 1) < nr ? 64 * r * (w + 1) : nr;
        int64_t k = k0;
        for (; k + 64 * 7 < k1; k += 64 * 8) {
            u32x4_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = k + 64 * u < k1 ? word(k + 64 * u) : u32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < 8; ++u) acc ^= v[u];
        }
        for (; k < k1; k += 64) acc ^= word(k);
        const int64_t j = 64 * w + lane;
        const unsigned h = acc.x ^ acc.y ^ acc.z ^ acc.w;
        if (j < nw) __builtin_nontemporal_store(u32x4_t{h, h, h, h}, dst + j);
    }
    const int64_t stride = waves * 64;
    for (int64_t k = 64 * r * tiles + gw * 64 + lane; k < nr; k += stride) acc ^= word(k);
    if (threadIdx.x == 0) g_floor_sink[blockIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" int kv8_stream_floor(const void* src0, uint64_t bytes0, const void* src1, uint64_t bytes1, void* dst,
                                uint64_t dst_bytes, void* stream) {
    if ((bytes0 | bytes1 | dst_bytes) % 16 != 0) return KV8_EINVAL;
    if ((bytes0 && (!src0 || reinterpret_cast<uintptr_t>(src0) % 16)) ||
        (bytes1 && (!src1 || reinterpret_cast<uintptr_t>(src1) % 16)) ||
        (dst_bytes && (!dst || reinterpret_cast<uintptr_t>(dst) % 16)))
        return KV8_EINVAL;
    if (bytes0 + bytes1 + dst_bytes == 0) return KV8_OK;
    const int64_t nr = static_cast<int64_t>((bytes0 + bytes1) / 16), nw = static_cast<int64_t>(dst_bytes / 16);
    const int64_t r = nw > 0 ? (nr + nw - 1) / nw : 0;
    hipLaunchKernelGGL(stream_floor_kernel, dim3(kFloorBlocks), dim3(kFloorThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src0),
                       static_cast<int64_t>(bytes0 / 16), static_cast<const u32x4_t*>(src1),
                       static_cast<int64_t>(bytes1 / 16), static_cast<u32x4_t*>(dst), nw, r);
    return hipGetLastError() == hipSuccess ? KV8_OK : KV8_ELAUNCH;
}
