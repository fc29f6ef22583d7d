// Shader clock under matrix-core load, for reading measured kernel times
// against the MFMA peak: MI355X's dense fp16/bf16 peak is quoted at the
// 2.4 GHz peak engine clock, and MFMA-heavy kernels run below it.
//
// Every wave of a full grid runs a chain of 32x32x16 f16 MFMAs; wave 0 of each
// block reads the shader-clock counter (s_memtime) and the constant-rate
// wall-clock counter (s_memrealtime) before and after.  The host divides the
// two deltas and scales by the wall clock's rate (hipDeviceAttributeWallClockRate).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "kv8.h"

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void clock_probe_kernel(int iters, unsigned long long* stamps,
                                                          float* sink) {
    const int tid = threadIdx.x;
    f16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<_Float16>(1e-3f * static_cast<float>((tid + i) & 15));
        b[i] = static_cast<_Float16>(1e-3f * static_cast<float>(i));
    }
    f32x16_t c0 = {}, c1 = {};
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c1, 0, 0, 0);
    }
    float s = 0.0f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
    __syncthreads();
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
        stamps[2 * blockIdx.x] = t1 - t0;
        stamps[2 * blockIdx.x + 1] = r1 - r0;
    }
    sink[blockIdx.x * 256 + tid] = s;
}

}  // namespace

extern "C" int kv8_shader_clock_mhz(int32_t busy_us, double* mhz, void* stream) {
    if (mhz == nullptr || busy_us < 1 || busy_us > 100000) return KV8_EINVAL;
    int dev = 0, cus = 0, wall_khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KV8_ELAUNCH;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        cus <= 0 || wall_khz <= 0)
        return KV8_ELAUNCH;
    const int blocks = 4 * cus;  // four blocks of four waves per CU: every SIMD busy
    // four 32-cycle MFMAs per iteration per wave, four waves per SIMD: ~512
    // cycles per iteration, sized for ~2 GHz
    const int iters = static_cast<int>(std::min<int64_t>(int64_t{busy_us} * 4, 400000));
    unsigned long long* d_stamps = nullptr;
    float* d_sink = nullptr;
    if (hipMalloc(&d_stamps, sizeof(unsigned long long) * 2 * blocks) != hipSuccess) return KV8_ENOMEM;
    if (hipMalloc(&d_sink, sizeof(float) * 256 * blocks) != hipSuccess) {
        (void)hipFree(d_stamps);
        return KV8_ENOMEM;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(256), 0, st, iters, d_stamps, d_sink);
    std::vector<unsigned long long> h(2 * static_cast<size_t>(blocks));
    int rc = KV8_OK;
    if (hipGetLastError() != hipSuccess ||
        hipMemcpyAsync(h.data(), d_stamps, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        rc = KV8_ELAUNCH;
    (void)hipFree(d_stamps);
    (void)hipFree(d_sink);
    if (rc != KV8_OK) return rc;
    std::vector<double> r;
    r.reserve(blocks);
    for (int i = 0; i < blocks; ++i)
        if (h[2 * i + 1] > 0) r.push_back(static_cast<double>(h[2 * i]) / static_cast<double>(h[2 * i + 1]));
    if (r.empty()) return KV8_ELAUNCH;
    std::nth_element(r.begin(), r.begin() + r.size() / 2, r.end());
    *mhz = r[r.size() / 2] * (wall_khz / 1000.0);
    return KV8_OK;
}
