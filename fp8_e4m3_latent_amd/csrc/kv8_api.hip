// C ABI of libkv8 (declared in include/kv8.h): argument checks and launches.
// No call allocates except kv8_absorb_decode's stream-ordered split partials
// (from a pool of the library's own), none synchronizes the host, none prints
// or aborts.
#include "kv8.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "kv8_internal.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kPoolDevices = 64;

// The stream-ordered memory pool of the current device from which
// kv8_absorb_decode takes its split partials (created on the first call on
// the device), or nullptr on failure.  Its release threshold keeps the memory
// a call frees in the pool, so the next call reuses it instead of asking the
// driver again; the pool holds the largest partials in use at once until the
// process ends.
hipMemPool_t partials_pool() {
    static std::mutex mu;
    static hipMemPool_t pools[kPoolDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kPoolDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (pools[dev] == nullptr) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess || pool == nullptr) return nullptr;
        uint64_t keep = UINT64_MAX;
        if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return nullptr;
        }
        pools[dev] = pool;
    }
    return pools[dev];
}

int launched(int rc) { return rc == 0 ? KV8_OK : KV8_ELAUNCH; }

}  // namespace

extern "C" {

const char* kv8_status_string(int status) {
    switch (status) {
        case KV8_OK: return "ok";
        case KV8_EINVAL: return "invalid argument";
        case KV8_EUNSUPPORTED: return "unsupported shape (kv_lora must be 512, rope 64)";
        case KV8_ELAUNCH: return "HIP launch failed";
        case KV8_EWORKSPACE: return "split-T workspace missing or too small";
        case KV8_ENOMEM: return "device allocation failed";
        case KV8_EIO: return "file system call failed";
        case KV8_EFORMAT: return "not a kv8 store, torn header, or other dimensions";
        default: return "unknown kv8 status";
    }
}

int kv8_quantize_rows(const float* src, int64_t src_row_stride, int64_t n_rows, int32_t kv_lora,
                      int32_t rope, uint8_t* codes, float* scales, const int64_t* dst_rows,
                      void* stream) {
    if (n_rows < 0) return KV8_EINVAL;
    if (kv_lora != kv8::kKvLora || rope != kv8::kRope) return KV8_EUNSUPPORTED;
    if (n_rows == 0) return KV8_OK;
    if (!src || !codes || !scales) return KV8_EINVAL;
    if (src_row_stride < kv_lora + rope || src_row_stride % 4 != 0) return KV8_EINVAL;
    if (!aligned(src, 16) || !aligned(codes, 4) || !aligned(scales, 8)) return KV8_EINVAL;
    if (dst_rows && !aligned(dst_rows, 8)) return KV8_EINVAL;
    return launched(kv8::launch_quantize_rows(src, src_row_stride, n_rows, codes, scales, dst_rows,
                                              static_cast<hipStream_t>(stream)));
}

int kv8_quantize_rows_mx(const float* src, int64_t src_row_stride, int64_t n_rows, int32_t kv_lora,
                         int32_t rope, uint8_t* codes, uint8_t* exps, const int64_t* dst_rows,
                         void* stream) {
    if (n_rows < 0) return KV8_EINVAL;
    if (kv_lora != kv8::kKvLora || rope != kv8::kRope) return KV8_EUNSUPPORTED;
    if (n_rows == 0) return KV8_OK;
    if (!src || !codes || !exps) return KV8_EINVAL;
    if (src_row_stride < kv_lora + rope || src_row_stride % 4 != 0) return KV8_EINVAL;
    if (!aligned(src, 16) || !aligned(codes, 4)) return KV8_EINVAL;
    if (dst_rows && !aligned(dst_rows, 8)) return KV8_EINVAL;
    return launched(kv8::launch_quantize_rows_mx(src, src_row_stride, n_rows, codes, exps, dst_rows,
                                                 static_cast<hipStream_t>(stream)));
}

int kv8_norm_rope_quantize_rows(const float* src, int64_t src_row_stride, int64_t n_rows,
                                int32_t kv_lora, int32_t rope, const float* norm_weight, float eps,
                                const int64_t* positions, float rope_theta, uint8_t* codes,
                                float* scales, const int64_t* dst_rows, void* stream) {
    if (n_rows < 0) return KV8_EINVAL;
    if (kv_lora != kv8::kKvLora || rope != kv8::kRope) return KV8_EUNSUPPORTED;
    if (!(eps >= 0.0f && eps <= 3.0e38f) || !(rope_theta > 0.0f && rope_theta <= 3.0e38f))
        return KV8_EINVAL;
    if (n_rows == 0) return KV8_OK;
    if (!src || !codes || !scales || !norm_weight || !positions) return KV8_EINVAL;
    if (src_row_stride < kv_lora + rope || src_row_stride % 4 != 0) return KV8_EINVAL;
    if (!aligned(src, 16) || !aligned(codes, 4) || !aligned(scales, 8) || !aligned(norm_weight, 16) ||
        !aligned(positions, 8))
        return KV8_EINVAL;
    if (dst_rows && !aligned(dst_rows, 8)) return KV8_EINVAL;
    return launched(kv8::launch_norm_rope_quantize_rows(src, src_row_stride, n_rows, norm_weight, eps,
                                                        positions, rope_theta, codes, scales, dst_rows,
                                                        static_cast<hipStream_t>(stream)));
}

static int project_rows(const uint8_t* codes, const float* scales, int64_t n_rows, int32_t kv_lora,
                        int32_t rope, const uint16_t* w_kv_b, int32_t N, void* out, bool out_f32,
                        float* rope_out, void* stream) {
    if (n_rows < 0 || N < 0) return KV8_EINVAL;
    if (kv_lora != kv8::kKvLora || rope != kv8::kRope) return KV8_EUNSUPPORTED;
    if (N % 128 != 0) return KV8_EUNSUPPORTED;
    if (n_rows == 0 || N == 0) return KV8_OK;
    if (!codes || !scales || !w_kv_b || !out) return KV8_EINVAL;
    if (!aligned(codes, 16) || !aligned(scales, 8) || !aligned(w_kv_b, 16) || !aligned(out, 16) ||
        (rope_out && !aligned(rope_out, 16)))
        return KV8_EINVAL;
    if ((n_rows + 255) / 256 * ((N + 255) / 256) > (int64_t(1) << 31) - 1) return KV8_EUNSUPPORTED;
    return launched(kv8::launch_project_rows(codes, scales, n_rows, w_kv_b, N, out, out_f32, rope_out,
                                             static_cast<hipStream_t>(stream)));
}

int kv8_project_rows(const uint8_t* codes, const float* scales, int64_t n_rows, int32_t kv_lora,
                     int32_t rope, const uint16_t* w_kv_b, int32_t N, uint16_t* out,
                     float* rope_out, void* stream) {
    return project_rows(codes, scales, n_rows, kv_lora, rope, w_kv_b, N, out, false, rope_out, stream);
}

int kv8_project_rows_f32(const uint8_t* codes, const float* scales, int64_t n_rows, int32_t kv_lora,
                         int32_t rope, const uint16_t* w_kv_b, int32_t N, float* out,
                         float* rope_out, void* stream) {
    return project_rows(codes, scales, n_rows, kv_lora, rope, w_kv_b, N, out, true, rope_out, stream);
}

int kv8_encode_bits(uint32_t first, uint64_t count, int32_t encoder, uint8_t* out, void* stream) {
    if (encoder != 0 && encoder != 1) return KV8_EINVAL;
    if (count == 0) return KV8_OK;
    if (!out || !aligned(out, 4)) return KV8_EINVAL;
    if (count > (uint64_t(1) << 32) - first) return KV8_EINVAL;
    return launched(kv8::launch_encode_bits(first, count, encoder, out, static_cast<hipStream_t>(stream)));
}

int kv8_decode_codes(const uint8_t* codes, int64_t n, uint16_t* out_bf16, uint16_t* out_f16,
                     void* stream) {
    if (n < 0) return KV8_EINVAL;
    if (n == 0) return KV8_OK;
    if (!codes || !out_bf16 || !out_f16) return KV8_EINVAL;
    return launched(kv8::launch_decode_codes(codes, n, out_bf16, out_f16,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Absorbed decode
// ---------------------------------------------------------------------------
namespace {

constexpr int kRowsPerBlock = 128;   // query rows per decode block
constexpr int kTargetBlocks = 256;   // one block per compute unit
constexpr int kMaxRange = 4096;      // longest token range of the internal plan

int64_t row_blocks(int32_t Q, int32_t H) {
    return (static_cast<int64_t>(Q) * H + kRowsPerBlock - 1) / kRowsPerBlock;
}

int check_decode(const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* codes,
                 const void* scales, const int64_t* kv_start, const int32_t* kv_len,
                 int32_t max_len, int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                 float softmax_scale, const float* out, uintptr_t scales_align = 8) {
    if (B < 1 || Q < 1 || H < 1 || max_len < 0) return KV8_EINVAL;
    if (kv_lora != kv8::kKvLora || rope != kv8::kRope) return KV8_EUNSUPPORTED;
    if (!q_lat || !q_rope || !codes || !scales || !kv_start || !kv_len || !out) return KV8_EINVAL;
    if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY ||
        softmax_scale == -INFINITY)
        return KV8_EINVAL;
    if (!aligned(q_lat, 16) || !aligned(q_rope, 16) || !aligned(codes, 16) ||
        !aligned(scales, scales_align) || !aligned(kv_start, 8) || !aligned(kv_len, 4) || !aligned(out, 16))
        return KV8_EINVAL;
    const int64_t blocks = static_cast<int64_t>(B) * row_blocks(Q, H);
    // (a sequence's latent query rows must span less than 2^31 bytes: the
    // decode addresses them with 32-bit offsets)
    if (blocks > (int64_t(1) << 30) || static_cast<int64_t>(Q) * H > (int64_t(1) << 21))
        return KV8_EUNSUPPORTED;
    return KV8_OK;
}

// sub-ranges per requested split so that the grid reaches one block per CU
int sub_splits(int32_t B, int32_t Q, int32_t H, int32_t num_splits) {
    const int64_t units = static_cast<int64_t>(B) * row_blocks(Q, H) * num_splits;
    const int64_t sub = units >= kTargetBlocks ? 1 : kTargetBlocks / units;
    return static_cast<int>(sub < 1 ? 1 : sub);
}

kv8::DecodeLaunch make_launch(const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* codes,
                              const float* scales, const int64_t* kv_start,
                              const int32_t* kv_len, int32_t B, int32_t Q, int32_t H,
                              float softmax_scale, float* out) {
    kv8::DecodeLaunch d{};
    d.q_lat = q_lat;
    d.q_rope = q_rope;
    d.codes = codes;
    d.scales = scales;
    d.kv_start = kv_start;
    d.kv_len = kv_len;
    d.B = B;
    d.Q = Q;
    d.H = H;
    // a zero scale would turn masked scores into 0 * inf; the smallest normal
    // scale gives the same (uniform) softmax
    d.softmax_scale = softmax_scale == 0.0f ? 1.17549435e-38f : softmax_scale;
    d.out = out;
    d.n_splits = 1;
    d.split_chunk = 0;
    d.n_sub = 1;
    d.workspace = nullptr;
    return d;
}

}  // namespace

extern "C" {

size_t kv8_splitT_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t kv_lora,
                                  int32_t num_splits) {
    if (B < 1 || Q < 1 || H < 1 || num_splits < 1 || kv_lora != kv8::kKvLora) return 0;
    const int total = num_splits * sub_splits(B, Q, H, num_splits);
    return total > 1 ? kv8::splitT_workspace_bytes(B, Q, H, total) : 0;
}

int kv8_decode_plan(int32_t B, int32_t Q, int32_t H, int32_t max_len, int32_t* split_tokens,
                    int32_t* num_splits) {
    if (B < 1 || Q < 1 || H < 1 || max_len < 0 || !split_tokens || !num_splits) return KV8_EINVAL;
    // token ranges of a fixed size (a multiple of the 32-token tile) so that
    // B x row blocks x ranges fills the compute units, and no range is longer
    // than kMaxRange tokens (with ragged lengths the longest sequences would
    // otherwise set the time while most blocks have finished)
    const int64_t units = static_cast<int64_t>(B) * row_blocks(Q, H);
    int64_t splits = (kTargetBlocks + units - 1) / units;
    const int64_t by_cap = (static_cast<int64_t>(max_len) + kMaxRange - 1) / kMaxRange;
    splits = splits > by_cap ? splits : by_cap;
    const int64_t by_len = (static_cast<int64_t>(max_len) + 1023) / 1024;
    splits = splits < by_len ? splits : by_len;
    if (splits <= 1) {
        *split_tokens = max_len;
        *num_splits = 1;
        return KV8_OK;
    }
    int64_t chunk = (max_len + splits - 1) / splits;
    chunk = (chunk + 31) / 32 * 32;
    *split_tokens = static_cast<int32_t>(chunk);
    *num_splits = static_cast<int32_t>((max_len + chunk - 1) / chunk);
    return KV8_OK;
}

size_t kv8_partials_bytes(int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t num_splits) {
    if (B < 1 || Q < 1 || H < 1 || num_splits < 1 || kv_lora != kv8::kKvLora) return 0;
    return kv8::splitT_workspace_bytes(B, Q, H, num_splits);
}

int kv8_absorb_decode_partials(const uint16_t* q_lat, const uint16_t* q_rope,
                               const uint8_t* codes, const float* scales,
                               const int64_t* kv_start, const int32_t* kv_len, int32_t max_len,
                               int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                               float softmax_scale, int32_t split_tokens, int32_t num_splits,
                               void* partials, size_t partials_bytes, void* stream) {
    int rc = check_decode(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, B, Q, H,
                          kv_lora, rope, softmax_scale, static_cast<float*>(partials) /* no out */);
    if (rc != KV8_OK) return rc;
    if (num_splits < 1 || num_splits > (1 << 20) || split_tokens < 0) return KV8_EINVAL;
    // fixed-size ranges must cover every row a sequence may hold
    if (split_tokens > 0 && static_cast<int64_t>(split_tokens) * num_splits < max_len)
        return KV8_EINVAL;
    if (!partials || !aligned(partials, 256) ||
        partials_bytes < kv8::splitT_workspace_bytes(B, Q, H, num_splits))
        return KV8_EWORKSPACE;
    kv8::DecodeLaunch d = make_launch(q_lat, q_rope, codes, scales, kv_start, kv_len, B, Q, H,
                                      softmax_scale, nullptr);
    d.n_splits = num_splits;
    d.split_chunk = split_tokens;
    d.n_sub = 1;
    d.workspace = partials;
    return launched(kv8::launch_absorb_decode(d, static_cast<hipStream_t>(stream), false));
}

int kv8_lse_merge(const void* partials, size_t partials_bytes, int32_t B, int32_t Q, int32_t H,
                  int32_t kv_lora, int32_t num_splits, float softmax_scale, float* out,
                  void* stream) {
    if (B < 1 || Q < 1 || H < 1 || num_splits < 1 || num_splits > (1 << 20)) return KV8_EINVAL;
    if (kv_lora != kv8::kKvLora) return KV8_EUNSUPPORTED;
    if (!partials || !out || !aligned(partials, 16) || !aligned(out, 16)) return KV8_EINVAL;
    if (static_cast<int64_t>(Q) * H > (int64_t(1) << 21)) return KV8_EUNSUPPORTED;
    if (partials_bytes < kv8::splitT_workspace_bytes(B, Q, H, num_splits)) return KV8_EWORKSPACE;
    if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY ||
        softmax_scale == -INFINITY)
        return KV8_EINVAL;
    const float sc = softmax_scale == 0.0f ? 1.17549435e-38f : softmax_scale;
    return launched(kv8::launch_lse_merge(partials, B, Q * H, num_splits, sc, out,
                                          static_cast<hipStream_t>(stream)));
}

int kv8_absorb_decode(const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* codes,
                      const float* scales, const int64_t* kv_start, const int32_t* kv_len,
                      int32_t max_len, int32_t B, int32_t Q, int32_t H, int32_t kv_lora,
                      int32_t rope, float softmax_scale, float* out, void* stream) {
    int rc = check_decode(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, B, Q, H,
                          kv_lora, rope, softmax_scale, out);
    if (rc != KV8_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    kv8::DecodeLaunch d =
        make_launch(q_lat, q_rope, codes, scales, kv_start, kv_len, B, Q, H, softmax_scale, out);
    int32_t chunk = 0, splits = 1;
    kv8_decode_plan(B, Q, H, max_len, &chunk, &splits);
    if (splits <= 1) return launched(kv8::launch_absorb_decode(d, st));
    d.n_splits = splits;
    d.split_chunk = chunk;
    const size_t bytes = kv8::splitT_workspace_bytes(B, Q, H, d.n_splits);
    hipMemPool_t pool = partials_pool();
    if (pool == nullptr || hipMallocFromPoolAsync(&d.workspace, bytes, pool, st) != hipSuccess)
        return KV8_ENOMEM;
    rc = launched(kv8::launch_absorb_decode(d, st));
    if (hipFreeAsync(d.workspace, st) != hipSuccess && rc == KV8_OK) rc = KV8_ELAUNCH;
    return rc;
}

int kv8_absorb_decode_mx(const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* codes,
                         const uint8_t* exps, const int64_t* kv_start, const int32_t* kv_len,
                         int32_t max_len, int32_t B, int32_t Q, int32_t H, int32_t kv_lora,
                         int32_t rope, float softmax_scale, float* out, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, void* stream) {
    // (the exponents take the place of the scales, 4-byte aligned)
    int rc = check_decode(q_lat, q_rope, codes, exps, kv_start, kv_len, max_len, B, Q, H, kv_lora,
                          rope, softmax_scale, out, 4);
    if (rc != KV8_OK) return rc;
    if (num_splits < 1 || num_splits > (1 << 20)) return KV8_EINVAL;
    kv8::DecodeLaunch d =
        make_launch(q_lat, q_rope, codes, nullptr, kv_start, kv_len, B, Q, H, softmax_scale, out);
    d.exps = exps;
    d.n_sub = sub_splits(B, Q, H, num_splits);
    d.n_splits = num_splits * d.n_sub;
    if (d.n_splits > 1) {
        const size_t need = kv8::splitT_workspace_bytes(B, Q, H, d.n_splits);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return KV8_EWORKSPACE;
        d.workspace = workspace;
    }
    return launched(kv8::launch_absorb_decode(d, static_cast<hipStream_t>(stream)));
}

size_t kv8_mx_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t num_splits) {
    if (B < 1 || Q < 1 || H < 1 || num_splits < 1 || kv_lora != kv8::kKvLora) return 0;
    const int total = num_splits * sub_splits(B, Q, H, num_splits);
    return total > 1 ? kv8::splitT_workspace_bytes(B, Q, H, total) : 0;
}

int kv8_absorb_decode_splitT(const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* codes,
                             const float* scales, const int64_t* kv_start, const int32_t* kv_len,
                             int32_t max_len, int32_t B, int32_t Q, int32_t H, int32_t kv_lora,
                             int32_t rope, float softmax_scale, float* out, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_decode(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, B, Q, H,
                          kv_lora, rope, softmax_scale, out);
    if (rc != KV8_OK) return rc;
    if (num_splits < 1 || num_splits > (1 << 20)) return KV8_EINVAL;
    kv8::DecodeLaunch d =
        make_launch(q_lat, q_rope, codes, scales, kv_start, kv_len, B, Q, H, softmax_scale, out);
    d.n_sub = sub_splits(B, Q, H, num_splits);
    d.n_splits = num_splits * d.n_sub;
    if (d.n_splits > 1) {
        const size_t need = kv8::splitT_workspace_bytes(B, Q, H, d.n_splits);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return KV8_EWORKSPACE;
        d.workspace = workspace;
    }
    return launched(kv8::launch_absorb_decode(d, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free decode: the split partials live in a static device array.
// ---------------------------------------------------------------------------
namespace {

// The array's name is a host-side stand-in in host code; kernels get its
// device address, looked up once per device.
static __device__ __align__(256) uint8_t scratch[KV8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (first call on a device:
// hipGetSymbolAddress with that device current), or nullptr on failure.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" int kv8_absorb_decode_noalloc(const uint16_t* q_lat, const uint16_t* q_rope,
                                         const uint8_t* codes, const float* scales,
                                         const int64_t* kv_start, const int32_t* kv_len,
                                         int32_t max_len, int32_t B, int32_t Q, int32_t H,
                                         int32_t kv_lora, int32_t rope, float softmax_scale,
                                         float* out, void* stream) {
    int rc = check_decode(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, B, Q, H,
                          kv_lora, rope, softmax_scale, out);
    if (rc != KV8_OK) return rc;
    kv8::DecodeLaunch d =
        make_launch(q_lat, q_rope, codes, scales, kv_start, kv_len, B, Q, H, softmax_scale, out);
    int32_t chunk = 0, splits = 1;
    kv8_decode_plan(B, Q, H, max_len, &chunk, &splits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (splits <= 1) return launched(kv8::launch_absorb_decode(d, st));
    // the same split as kv8_absorb_decode, so the results are the same
    if (kv8::splitT_workspace_bytes(B, Q, H, splits) > KV8_NOALLOC_SCRATCH_BYTES) return KV8_EWORKSPACE;
    void* ws = scratch_on_current_device();
    if (ws == nullptr) return KV8_ELAUNCH;
    d.n_splits = splits;
    d.split_chunk = chunk;
    d.workspace = ws;
    return launched(kv8::launch_absorb_decode(d, st));
}
