// Slot pool, byte accounting and persistence of the fp8 latent cache
// (declared in include/kv8_pool.h).  Host code: POSIX file calls for the
// store, HIP runtime calls and the row quantizer for the pool.
//
// Page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
// (colibri PR #299): commit message, first paragraph (the pool reports its
// bytes with fp8 rows) and .coli_kv v2 item (magic and dtype in the header,
// appends through a persistent handle, f32 files quantized on resume and kept
// intact until the first append rewrites them, repair on open).
#include "kv8_pool.h"

#include <errno.h>
#include <fcntl.h>
#include <hip/hip_runtime.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <string>
#include <vector>

#include "kv8.h"
#include "kv8_internal.hpp"

namespace {

constexpr char kMagic[8] = {'K', 'V', '8', 'S', 'T', 'O', 'R', 'E'};
constexpr uint32_t kVersion = 1;
constexpr int64_t kHeaderBytes = 64;
constexpr int64_t kChunkTokens = 4096;  // tokens per host staging chunk

uint64_t fnv1a64(const uint8_t* p, size_t n) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 0x100000001b3ull;
    }
    return h;
}

int64_t token_bytes(int32_t dtype, int32_t n_layers, int32_t width) {
    return dtype == KV8_DTYPE_E4M3 ? static_cast<int64_t>(n_layers) * (width + 8)
                                   : static_cast<int64_t>(n_layers) * width * 4;
}

struct Header {
    uint32_t dtype, n_layers, kv_lora, rope;
    uint64_t n_tokens;
};

void encode_header(const Header& h, uint8_t out[kHeaderBytes]) {
    memset(out, 0, kHeaderBytes);
    memcpy(out, kMagic, 8);
    const uint32_t w[6] = {kVersion, h.dtype, h.n_layers, h.kv_lora, h.rope,
                           static_cast<uint32_t>(kHeaderBytes)};
    memcpy(out + 8, w, sizeof(w));
    memcpy(out + 32, &h.n_tokens, 8);
    const uint64_t check = fnv1a64(out, 40);
    memcpy(out + 40, &check, 8);
}

// KV8_OK, or KV8_EFORMAT for anything but a version-1 header with a good check
int decode_header(const uint8_t in[kHeaderBytes], Header* h) {
    if (memcmp(in, kMagic, 8) != 0) return KV8_EFORMAT;
    uint64_t check;
    memcpy(&check, in + 40, 8);
    if (check != fnv1a64(in, 40)) return KV8_EFORMAT;
    uint32_t w[6];
    memcpy(w, in + 8, sizeof(w));
    if (w[0] != kVersion || w[5] != kHeaderBytes) return KV8_EFORMAT;
    if (w[1] != KV8_DTYPE_F32 && w[1] != KV8_DTYPE_E4M3) return KV8_EFORMAT;
    h->dtype = w[1];
    h->n_layers = w[2];
    h->kv_lora = w[3];
    h->rope = w[4];
    memcpy(&h->n_tokens, in + 32, 8);
    return KV8_OK;
}

bool write_all(int fd, const void* p, size_t n, int64_t off) {
    const uint8_t* b = static_cast<const uint8_t*>(p);
    while (n > 0) {
        const ssize_t k = pwrite(fd, b, n, off);
        if (k < 0) {
            if (errno == EINTR) continue;
            return false;
        }
        b += k;
        n -= static_cast<size_t>(k);
        off += k;
    }
    return true;
}

bool read_all(int fd, void* p, size_t n, int64_t off) {
    uint8_t* b = static_cast<uint8_t*>(p);
    while (n > 0) {
        const ssize_t k = pread(fd, b, n, off);
        if (k < 0) {
            if (errno == EINTR) continue;
            return false;
        }
        if (k == 0) return false;
        b += k;
        n -= static_cast<size_t>(k);
        off += k;
    }
    return true;
}

// Make a rename or creation in the file's directory durable.
void sync_dir(const std::string& path) {
    const size_t slash = path.find_last_of('/');
    const std::string dir = slash == std::string::npos ? "." : path.substr(0, slash + 1);
    const int fd = open(dir.c_str(), O_RDONLY | O_DIRECTORY);
    if (fd >= 0) {
        (void)fsync(fd);
        close(fd);
    }
}

}  // namespace

struct kv8_store {
    std::string path;
    int fd = -1;
    Header h{};
    int32_t width = 0;  // kv_lora + rope
};

struct kv8_pool {
    void* arena = nullptr;
    int32_t n_layers = 0, n_slots = 0;
    int64_t slot_tokens = 0;
    std::vector<uint8_t*> codes;
    std::vector<float*> scales;
    std::vector<int64_t> len;
};

extern "C" {

uint64_t kv8_pool_bytes(int32_t n_layers, int32_t n_slots, int64_t slot_tokens, int32_t kv_lora,
                        int32_t rope, int32_t dtype) {
    if (n_layers < 0 || n_slots < 0 || slot_tokens < 0 || kv_lora < 0 || rope < 0) return 0;
    if (dtype != KV8_DTYPE_F32 && dtype != KV8_DTYPE_E4M3) return 0;
    return static_cast<uint64_t>(n_slots) * static_cast<uint64_t>(slot_tokens) *
           static_cast<uint64_t>(token_bytes(dtype, n_layers, kv_lora + rope));
}

int64_t kv8_pool_slot_tokens_for(uint64_t budget_bytes, int32_t n_layers, int32_t n_slots,
                                 int32_t kv_lora, int32_t rope, int32_t dtype) {
    if (n_layers < 1 || n_slots < 1 || kv_lora < 0 || rope < 0 || kv_lora + rope < 1) return -1;
    if (dtype != KV8_DTYPE_F32 && dtype != KV8_DTYPE_E4M3) return -1;
    const uint64_t per_token = static_cast<uint64_t>(n_slots) *
                               static_cast<uint64_t>(token_bytes(dtype, n_layers, kv_lora + rope));
    const uint64_t t = budget_bytes / per_token;
    return static_cast<int64_t>(t / 32 * 32);
}

int kv8_store_open(const char* path, int32_t n_layers, int32_t kv_lora, int32_t rope,
                   kv8_store** out) {
    if (!path || !out || n_layers < 1 || kv_lora < 1 || rope < 0) return KV8_EINVAL;
    *out = nullptr;
    const std::string p(path);
    // a rewrite that never reached its rename: the original is intact
    const std::string tmp = p + ".kv8tmp";
    if (unlink(tmp.c_str()) == 0) sync_dir(p);

    int fd = open(path, O_RDWR);
    if (fd < 0 && errno == ENOENT) {
        fd = open(path, O_RDWR | O_CREAT | O_EXCL, 0644);
        if (fd < 0) return KV8_EIO;
        uint8_t hb[kHeaderBytes];
        encode_header(Header{KV8_DTYPE_E4M3, static_cast<uint32_t>(n_layers),
                             static_cast<uint32_t>(kv_lora), static_cast<uint32_t>(rope), 0},
                      hb);
        if (!write_all(fd, hb, kHeaderBytes, 0) || fsync(fd) != 0) {
            close(fd);
            return KV8_EIO;
        }
        sync_dir(p);
    }
    if (fd < 0) return KV8_EIO;
    struct stat sb;
    if (fstat(fd, &sb) != 0) {
        close(fd);
        return KV8_EIO;
    }
    uint8_t hb[kHeaderBytes];
    Header h{};
    if (sb.st_size < kHeaderBytes || !read_all(fd, hb, kHeaderBytes, 0) ||
        decode_header(hb, &h) != KV8_OK || h.n_layers != static_cast<uint32_t>(n_layers) ||
        h.kv_lora != static_cast<uint32_t>(kv_lora) || h.rope != static_cast<uint32_t>(rope)) {
        close(fd);
        return KV8_EFORMAT;
    }
    const int64_t rec = token_bytes(static_cast<int32_t>(h.dtype), n_layers, kv_lora + rope);
    const int64_t held = (static_cast<int64_t>(sb.st_size) - kHeaderBytes) / rec;  // complete records
    bool repaired = false;
    if (static_cast<int64_t>(h.n_tokens) > held) {  // counted records missing: count the complete ones
        h.n_tokens = static_cast<uint64_t>(held);
        encode_header(h, hb);
        if (!write_all(fd, hb, kHeaderBytes, 0)) {
            close(fd);
            return KV8_EIO;
        }
        repaired = true;
    }
    const int64_t want = kHeaderBytes + static_cast<int64_t>(h.n_tokens) * rec;
    if (static_cast<int64_t>(sb.st_size) > want) {  // an append that never raised the count
        if (ftruncate(fd, want) != 0) {
            close(fd);
            return KV8_EIO;
        }
        repaired = true;
    }
    if (repaired && fsync(fd) != 0) {
        close(fd);
        return KV8_EIO;
    }
    kv8_store* st = new kv8_store;
    st->path = p;
    st->fd = fd;
    st->h = h;
    st->width = kv_lora + rope;
    *out = st;
    return KV8_OK;
}

int kv8_store_info(const kv8_store* st, int32_t* dtype, int64_t* n_tokens) {
    if (!st) return KV8_EINVAL;
    if (dtype) *dtype = static_cast<int32_t>(st->h.dtype);
    if (n_tokens) *n_tokens = static_cast<int64_t>(st->h.n_tokens);
    return KV8_OK;
}

int kv8_store_read(kv8_store* st, int64_t t0, int64_t n, uint8_t* codes, float* scales,
                   float* rows_f32) {
    if (!st || t0 < 0 || n < 0 || t0 + n > static_cast<int64_t>(st->h.n_tokens)) return KV8_EINVAL;
    if (n == 0) return KV8_OK;
    const int32_t L = static_cast<int32_t>(st->h.n_layers), W = st->width;
    const bool fp8 = st->h.dtype == KV8_DTYPE_E4M3;
    if (fp8 ? (!codes || !scales) : !rows_f32) return KV8_EINVAL;
    const int64_t rec = token_bytes(static_cast<int32_t>(st->h.dtype), L, W);
    if (!fp8) {  // the record layout is the caller's layout
        return read_all(st->fd, rows_f32, static_cast<size_t>(n * rec), kHeaderBytes + t0 * rec)
                   ? KV8_OK
                   : KV8_EIO;
    }
    std::vector<uint8_t> buf(static_cast<size_t>(std::min<int64_t>(n, kChunkTokens) * rec));
    for (int64_t c0 = 0; c0 < n; c0 += kChunkTokens) {
        const int64_t cn = std::min<int64_t>(kChunkTokens, n - c0);
        if (!read_all(st->fd, buf.data(), static_cast<size_t>(cn * rec), kHeaderBytes + (t0 + c0) * rec))
            return KV8_EIO;
        for (int64_t t = 0; t < cn; ++t)
            for (int32_t l = 0; l < L; ++l) {
                const uint8_t* r = buf.data() + t * rec + static_cast<int64_t>(l) * (W + 8);
                const int64_t k = (c0 + t) * L + l;
                memcpy(codes + k * W, r, static_cast<size_t>(W));
                memcpy(scales + 2 * k, r + W, 8);
            }
    }
    return KV8_OK;
}

namespace {

// n E4M3 records packed token-major into buf (staging of an append)
void pack_e4m3(int32_t L, int32_t W, int64_t n, const uint8_t* codes, const float* scales,
               uint8_t* buf) {
    for (int64_t t = 0; t < n; ++t)
        for (int32_t l = 0; l < L; ++l) {
            uint8_t* r = buf + (t * L + l) * (W + 8);
            const int64_t k = t * L + l;
            memcpy(r, codes + k * W, static_cast<size_t>(W));
            memcpy(r + W, scales + 2 * k, 8);
        }
}

// write n records at record index t0 of fd, through a bounded staging buffer
bool write_records(int fd, int32_t L, int32_t W, int64_t t0, int64_t n, const uint8_t* codes,
                   const float* scales) {
    const int64_t rec = token_bytes(KV8_DTYPE_E4M3, L, W);
    std::vector<uint8_t> buf(static_cast<size_t>(std::min<int64_t>(std::max<int64_t>(n, 1), kChunkTokens) * rec));
    for (int64_t c0 = 0; c0 < n; c0 += kChunkTokens) {
        const int64_t cn = std::min<int64_t>(kChunkTokens, n - c0);
        pack_e4m3(L, W, cn, codes + c0 * L * W, scales + 2 * c0 * L, buf.data());
        if (!write_all(fd, buf.data(), static_cast<size_t>(cn * rec), kHeaderBytes + (t0 + c0) * rec))
            return false;
    }
    return true;
}

}  // namespace

int kv8_store_append(kv8_store* st, int64_t n, const uint8_t* codes, const float* scales,
                     const uint8_t* prior_codes, const float* prior_scales) {
    if (!st || n < 0 || (n > 0 && (!codes || !scales))) return KV8_EINVAL;
    const int32_t L = static_cast<int32_t>(st->h.n_layers), W = st->width;
    const int64_t old = static_cast<int64_t>(st->h.n_tokens);
    uint8_t hb[kHeaderBytes];
    if (st->h.dtype == KV8_DTYPE_E4M3) {
        if (n == 0) return KV8_OK;
        // records first, made durable; then the count
        if (!write_records(st->fd, L, W, old, n, codes, scales) || fsync(st->fd) != 0) return KV8_EIO;
        Header h = st->h;
        h.n_tokens = static_cast<uint64_t>(old + n);
        encode_header(h, hb);
        if (!write_all(st->fd, hb, kHeaderBytes, 0) || fsync(st->fd) != 0) return KV8_EIO;
        st->h = h;
        return KV8_OK;
    }
    // F32 on disk: rewrite the whole store in E4M3 beside it, then rename
    if (old > 0 && (!prior_codes || !prior_scales)) return KV8_EINVAL;
    const std::string tmp = st->path + ".kv8tmp";
    const int fd = open(tmp.c_str(), O_RDWR | O_CREAT | O_TRUNC, 0644);
    if (fd < 0) return KV8_EIO;
    Header h = st->h;
    h.dtype = KV8_DTYPE_E4M3;
    h.n_tokens = static_cast<uint64_t>(old + n);
    encode_header(h, hb);
    const bool ok = write_all(fd, hb, kHeaderBytes, 0) &&
                    write_records(fd, L, W, 0, old, prior_codes, prior_scales) &&
                    write_records(fd, L, W, old, n, codes, scales) && fsync(fd) == 0;
    if (!ok || rename(tmp.c_str(), st->path.c_str()) != 0) {
        close(fd);
        unlink(tmp.c_str());
        return KV8_EIO;
    }
    sync_dir(st->path);
    close(st->fd);
    st->fd = fd;
    st->h = h;
    return KV8_OK;
}

int kv8_store_close(kv8_store* st) {
    if (!st) return KV8_EINVAL;
    const int rc = close(st->fd) == 0 ? KV8_OK : KV8_EIO;
    delete st;
    return rc;
}

int kv8_store_write_f32(const char* path, int32_t n_layers, int32_t kv_lora, int32_t rope,
                        int64_t n_tokens, const float* rows_f32) {
    if (!path || n_layers < 1 || kv_lora < 1 || rope < 0 || n_tokens < 0 || (n_tokens > 0 && !rows_f32))
        return KV8_EINVAL;
    const std::string tmp = std::string(path) + ".kv8tmp";
    const int fd = open(tmp.c_str(), O_RDWR | O_CREAT | O_TRUNC, 0644);
    if (fd < 0) return KV8_EIO;
    uint8_t hb[kHeaderBytes];
    encode_header(Header{KV8_DTYPE_F32, static_cast<uint32_t>(n_layers), static_cast<uint32_t>(kv_lora),
                         static_cast<uint32_t>(rope), static_cast<uint64_t>(n_tokens)},
                  hb);
    const int64_t bytes = n_tokens * token_bytes(KV8_DTYPE_F32, n_layers, kv_lora + rope);
    const bool ok = write_all(fd, hb, kHeaderBytes, 0) &&
                    write_all(fd, rows_f32, static_cast<size_t>(bytes), kHeaderBytes) && fsync(fd) == 0;
    close(fd);
    if (!ok || rename(tmp.c_str(), path) != 0) {
        unlink(tmp.c_str());
        return KV8_EIO;
    }
    sync_dir(path);
    return KV8_OK;
}

// ---------------------------------------------------------------------------
// Device pool
// ---------------------------------------------------------------------------

int kv8_pool_create(int32_t n_layers, int32_t n_slots, int64_t slot_tokens, kv8_pool** out) {
    if (!out || n_layers < 1 || n_slots < 1 || slot_tokens < 32 || slot_tokens % 32 != 0)
        return KV8_EINVAL;
    *out = nullptr;
    const int64_t rows = static_cast<int64_t>(n_slots) * slot_tokens;
    const int64_t codes_bytes = (rows * (kv8::kKvLora + kv8::kRope) + 255) / 256 * 256;
    const int64_t scales_bytes = (rows * 8 + 255) / 256 * 256;
    void* arena = nullptr;
    if (hipMalloc(&arena, static_cast<size_t>(n_layers * (codes_bytes + scales_bytes))) != hipSuccess)
        return KV8_ENOMEM;
    kv8_pool* p = new kv8_pool;
    p->arena = arena;
    p->n_layers = n_layers;
    p->n_slots = n_slots;
    p->slot_tokens = slot_tokens;
    p->len.assign(static_cast<size_t>(n_slots), 0);
    uint8_t* a = static_cast<uint8_t*>(arena);
    for (int32_t l = 0; l < n_layers; ++l) {
        p->codes.push_back(a);
        p->scales.push_back(reinterpret_cast<float*>(a + codes_bytes));
        a += codes_bytes + scales_bytes;
    }
    *out = p;
    return KV8_OK;
}

int kv8_pool_destroy(kv8_pool* pool) {
    if (!pool) return KV8_EINVAL;
    const int rc = hipFree(pool->arena) == hipSuccess ? KV8_OK : KV8_ELAUNCH;
    delete pool;
    return rc;
}

uint64_t kv8_pool_used_bytes(const kv8_pool* pool) {
    return pool ? kv8_pool_bytes(pool->n_layers, pool->n_slots, pool->slot_tokens, kv8::kKvLora,
                                 kv8::kRope, KV8_DTYPE_E4M3)
                : 0;
}

int kv8_pool_layer(const kv8_pool* pool, int32_t layer, uint8_t** codes, float** scales) {
    if (!pool || layer < 0 || layer >= pool->n_layers || !codes || !scales) return KV8_EINVAL;
    *codes = pool->codes[static_cast<size_t>(layer)];
    *scales = pool->scales[static_cast<size_t>(layer)];
    return KV8_OK;
}

int64_t kv8_pool_slot_row(const kv8_pool* pool, int32_t slot) {
    if (!pool || slot < 0 || slot >= pool->n_slots) return -1;
    return static_cast<int64_t>(slot) * pool->slot_tokens;
}

int64_t kv8_pool_len(const kv8_pool* pool, int32_t slot) {
    if (!pool || slot < 0 || slot >= pool->n_slots) return -1;
    return pool->len[static_cast<size_t>(slot)];
}

int kv8_pool_set_len(kv8_pool* pool, int32_t slot, int64_t len) {
    if (!pool || slot < 0 || slot >= pool->n_slots || len < 0 || len > pool->slot_tokens) return KV8_EINVAL;
    pool->len[static_cast<size_t>(slot)] = len;
    return KV8_OK;
}

int kv8_pool_load(kv8_pool* pool, int32_t slot, kv8_store* st, void* stream) {
    if (!pool || !st || slot < 0 || slot >= pool->n_slots) return KV8_EINVAL;
    const int32_t L = static_cast<int32_t>(st->h.n_layers), W = st->width;
    if (L != pool->n_layers || W != kv8::kKvLora + kv8::kRope || static_cast<int32_t>(st->h.rope) != kv8::kRope)
        return KV8_EINVAL;
    const int64_t n = static_cast<int64_t>(st->h.n_tokens);
    if (n > pool->slot_tokens) return KV8_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t base = kv8_pool_slot_row(pool, slot);
    const int64_t cmax = std::min<int64_t>(std::max<int64_t>(n, 1), kChunkTokens);
    const bool fp8 = st->h.dtype == KV8_DTYPE_E4M3;
    std::vector<uint8_t> hc(fp8 ? static_cast<size_t>(cmax * L * W) : 0);
    std::vector<float> hs(fp8 ? static_cast<size_t>(cmax * L * 2) : 0);
    std::vector<float> hf(fp8 ? 0 : static_cast<size_t>(cmax * L * W));
    std::vector<uint8_t> lc(static_cast<size_t>(cmax * W));
    std::vector<float> ls(static_cast<size_t>(cmax * 2)), lf(fp8 ? 0 : static_cast<size_t>(cmax * W));
    float* dev_rows = nullptr;  // f32 rows of one layer chunk, quantized on the device
    if (!fp8 && hipMalloc(&dev_rows, static_cast<size_t>(cmax * W) * sizeof(float)) != hipSuccess)
        return KV8_ENOMEM;
    int rc = KV8_OK;
    for (int64_t c0 = 0; c0 < n && rc == KV8_OK; c0 += kChunkTokens) {
        const int64_t cn = std::min<int64_t>(kChunkTokens, n - c0);
        rc = kv8_store_read(st, c0, cn, hc.data(), hs.data(), hf.data());
        for (int32_t l = 0; l < L && rc == KV8_OK; ++l) {
            uint8_t* dc = pool->codes[static_cast<size_t>(l)] + (base + c0) * W;
            float* ds = pool->scales[static_cast<size_t>(l)] + 2 * (base + c0);
            if (fp8) {
                for (int64_t t = 0; t < cn; ++t) {
                    memcpy(lc.data() + t * W, hc.data() + (t * L + l) * W, static_cast<size_t>(W));
                    memcpy(ls.data() + 2 * t, hs.data() + 2 * (t * L + l), 8);
                }
                if (hipMemcpyAsync(dc, lc.data(), static_cast<size_t>(cn * W), hipMemcpyHostToDevice, s) != hipSuccess ||
                    hipMemcpyAsync(ds, ls.data(), static_cast<size_t>(cn * 8), hipMemcpyHostToDevice, s) != hipSuccess)
                    rc = KV8_ELAUNCH;
            } else {
                for (int64_t t = 0; t < cn; ++t)
                    memcpy(lf.data() + t * W, hf.data() + (t * L + l) * W, static_cast<size_t>(W) * sizeof(float));
                if (hipMemcpyAsync(dev_rows, lf.data(), static_cast<size_t>(cn * W) * sizeof(float),
                                   hipMemcpyHostToDevice, s) != hipSuccess)
                    rc = KV8_ELAUNCH;
                else
                    rc = kv8_quantize_rows(dev_rows, W, cn, kv8::kKvLora, kv8::kRope, dc, ds, nullptr, stream);
            }
            // (the host staging of this layer is reused by the next one)
            if (rc == KV8_OK && hipStreamSynchronize(s) != hipSuccess) rc = KV8_ELAUNCH;
        }
    }
    if (dev_rows) (void)hipFree(dev_rows);
    if (rc == KV8_OK) pool->len[static_cast<size_t>(slot)] = n;
    return rc;
}

int kv8_pool_save(kv8_pool* pool, int32_t slot, kv8_store* st, void* stream) {
    if (!pool || !st || slot < 0 || slot >= pool->n_slots) return KV8_EINVAL;
    const int32_t L = static_cast<int32_t>(st->h.n_layers), W = st->width;
    if (L != pool->n_layers || W != kv8::kKvLora + kv8::kRope) return KV8_EINVAL;
    const int64_t len = pool->len[static_cast<size_t>(slot)];
    const int64_t have = static_cast<int64_t>(st->h.n_tokens);
    if (have > len) return KV8_EINVAL;
    const bool rewrite = st->h.dtype != KV8_DTYPE_E4M3;
    const int64_t t0 = rewrite ? 0 : have;  // an f32 store needs every token in fp8
    const int64_t n = len - t0;
    if (n == 0 && !rewrite) return KV8_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t base = kv8_pool_slot_row(pool, slot);
    std::vector<uint8_t> hc(static_cast<size_t>(n * L * W));
    std::vector<float> hs(static_cast<size_t>(n * L * 2));
    std::vector<uint8_t> lc(static_cast<size_t>(std::max<int64_t>(n, 1) * W));
    std::vector<float> ls(static_cast<size_t>(std::max<int64_t>(n, 1) * 2));
    for (int32_t l = 0; l < L && n > 0; ++l) {
        const uint8_t* dc = pool->codes[static_cast<size_t>(l)] + (base + t0) * W;
        const float* ds = pool->scales[static_cast<size_t>(l)] + 2 * (base + t0);
        if (hipMemcpyAsync(lc.data(), dc, static_cast<size_t>(n * W), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipMemcpyAsync(ls.data(), ds, static_cast<size_t>(n * 8), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return KV8_ELAUNCH;
        for (int64_t t = 0; t < n; ++t) {
            memcpy(hc.data() + (t * L + l) * W, lc.data() + t * W, static_cast<size_t>(W));
            memcpy(hs.data() + 2 * (t * L + l), ls.data() + 2 * t, 8);
        }
    }
    if (!rewrite) return kv8_store_append(st, n, hc.data(), hs.data(), nullptr, nullptr);
    // tokens [0, have) are the prior records of the rewrite, the rest are new
    return kv8_store_append(st, len - have, hc.data() + have * L * W, hs.data() + 2 * have * L,
                            hc.data(), hs.data());
}

}  // extern "C"
