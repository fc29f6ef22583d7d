/* kv8 slot pool, byte accounting and persistence of the fp8 latent cache.
 *
 * Part of libkv8.so (include/kv8.h holds the status codes and the kernels).
 * The behaviours follow the page "KV8=1: fp8 e4m3 latent KV cache (CPU +
 * CUDA) with .coli_kv v2" (colibri pull request #299), cited as
 * [colibri#299]:
 *
 *   commit message, first paragraph: the pool of KV slots reports its bytes
 *     with fp8 rows (kv_pool_bytes), so that sizing against the memory
 *     budget (cap_for_ram) sees the smaller pool;
 *   commit message, .coli_kv v2 item (and the PR description): an on-disk
 *     format with a magic and the dtype in its header, fp8 rows plus scales
 *     appended through a persistent handle; files of f32 rows are quantized
 *     on resume and stay intact on disk until the first append rewrites them
 *     in fp8, so a crash before that loses nothing; opening repairs what an
 *     interrupted write left behind;
 *   commit message, Tests item: disk round trip, upgrade, rejection and
 *     self-heal.
 *
 * The byte layout of the page's own file is not given; this is a format of
 * its own (described below) with the same behaviours.
 *
 * Memory (one GPU's share; every slot is one sequence's rows in every layer):
 *   layer l of the pool is a cache in the layout of include/kv8.h:
 *   codes uint8 [n_slots * slot_tokens][kv_lora + rope] and scales f32
 *   [n_slots * slot_tokens][2]; slot s occupies rows
 *   [s * slot_tokens, s * slot_tokens + len(s)) of every layer, so a decode
 *   over slots passes kv_start = kv8_pool_slot_row(pool, s), kv_len = len(s).
 *
 * Store file ("kv8 latent store"), little-endian:
 *   bytes 0-7    magic "KV8STORE"
 *   8            uint32 version (1)
 *   12           uint32 dtype (KV8_DTYPE_F32 or KV8_DTYPE_E4M3)
 *   16, 20, 24   uint32 n_layers, kv_lora, rope
 *   28           uint32 header bytes (64)
 *   32           uint64 n_tokens: complete token records in the file
 *   40           uint64 FNV-1a 64 of bytes 0-39 (a torn header is rejected)
 *   48-63        zero
 *   64...        n_tokens records, token-major; per token, for each layer:
 *                E4M3: kv_lora + rope codes, then the f32 Lc and Rc scales
 *                      (kv_lora + rope + 8 bytes);
 *                F32:  kv_lora + rope f32 values.
 *
 * All calls are host calls; they return KV8_OK or a negative kv8_status.
 * Store calls never touch the GPU.  Pool calls that move data are
 * synchronous: they return after their copies and kernels have finished. */
#ifndef KV8_POOL_H
#define KV8_POOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { KV8_DTYPE_F32 = 0, KV8_DTYPE_E4M3 = 1 };

/* Bytes of a pool of n_slots slots of slot_tokens tokens in n_layers layers
 * ([colibri#299] commit message, first paragraph: kv_pool_bytes):
 * E4M3: kv_lora + rope code bytes + 8 scale bytes per token and layer (584
 * for 512 + 64); F32: 4 (kv_lora + rope).  0 for a negative size or an
 * unknown dtype. */
uint64_t kv8_pool_bytes(int32_t n_layers, int32_t n_slots, int64_t slot_tokens, int32_t kv_lora,
                        int32_t rope, int32_t dtype);

/* The largest slot capacity, a multiple of 32 tokens, whose pool fits in
 * budget_bytes ([colibri#299]: cap_for_ram sizing against the smaller pool);
 * 0 when not even 32 tokens fit, -1 for a bad argument. */
int64_t kv8_pool_slot_tokens_for(uint64_t budget_bytes, int32_t n_layers, int32_t n_slots,
                                 int32_t kv_lora, int32_t rope, int32_t dtype);

/* ---- Store (file) ---- */
typedef struct kv8_store kv8_store;

/* Open (or create, as an empty E4M3 store) the store at path for caches of
 * n_layers layers of kv_lora + rope rows.  Opening repairs what an
 * interrupted write can leave: a leftover "<path>.kv8tmp" from a rewrite
 * that never reached its rename is removed (the original is intact), bytes
 * past the last complete record are cut off (an append whose header update
 * never happened), and a header that counts records the file does not hold
 * is lowered to the complete ones.  Returns KV8_EFORMAT for a file that is
 * not a store, has a torn header, or holds other dimensions, and KV8_EIO
 * for a failed system call. */
int kv8_store_open(const char* path, int32_t n_layers, int32_t kv_lora, int32_t rope,
                   kv8_store** out);

/* dtype of the records on disk and their number. */
int kv8_store_info(const kv8_store* st, int32_t* dtype, int64_t* n_tokens);

/* Read records [t0, t0 + n) into host buffers, token-major:
 * E4M3 store: codes [n][n_layers][kv_lora + rope], scales [n][n_layers][2];
 * F32 store:  rows_f32 [n][n_layers][kv_lora + rope].
 * The buffers of the other dtype may be NULL. */
int kv8_store_read(kv8_store* st, int64_t t0, int64_t n, uint8_t* codes, float* scales,
                   float* rows_f32);

/* Append n E4M3 records (host buffers, token-major as above).  On an E4M3
 * store the records are written after the last one and made durable, and
 * only then the header's count is raised.  On an F32 store (one opened for
 * resume) the whole file is rewritten in E4M3: prior_codes / prior_scales
 * must hold the quantized form of its n_tokens records (what the resume
 * produced); the new file is written beside it as "<path>.kv8tmp", made
 * durable, and renamed over the original, so the f32 file stays intact
 * until the complete E4M3 file replaces it.  KV8_EINVAL if the prior
 * records are missing for an F32 store. */
int kv8_store_append(kv8_store* st, int64_t n, const uint8_t* codes, const float* scales,
                     const uint8_t* prior_codes, const float* prior_scales);

int kv8_store_close(kv8_store* st);

/* Write a store of F32 records (the unquantized form, KV8=0), replacing any
 * file at path: rows_f32 [n_tokens][n_layers][kv_lora + rope]. */
int kv8_store_write_f32(const char* path, int32_t n_layers, int32_t kv_lora, int32_t rope,
                        int64_t n_tokens, const float* rows_f32);

/* ---- Pool (device memory of the current device) ---- */
typedef struct kv8_pool kv8_pool;

/* One device allocation holding n_layers caches of n_slots * slot_tokens
 * rows (kv_lora = 512, rope = 64); every slot starts empty.  slot_tokens a
 * multiple of 32.  KV8_ENOMEM when the allocation fails. */
int kv8_pool_create(int32_t n_layers, int32_t n_slots, int64_t slot_tokens, kv8_pool** out);
int kv8_pool_destroy(kv8_pool* pool);

/* Bytes the pool's caches occupy (kv8_pool_bytes of its shape, E4M3). */
uint64_t kv8_pool_used_bytes(const kv8_pool* pool);

/* Device pointers of layer l's cache (layout of include/kv8.h). */
int kv8_pool_layer(const kv8_pool* pool, int32_t layer, uint8_t** codes, float** scales);

/* First row of slot s in every layer (-1 for a bad slot). */
int64_t kv8_pool_slot_row(const kv8_pool* pool, int32_t slot);

/* Tokens held by slot s (host-side bookkeeping: kernels that append rows
 * do not update it; the caller sets it after its appends). */
int64_t kv8_pool_len(const kv8_pool* pool, int32_t slot);
int kv8_pool_set_len(kv8_pool* pool, int32_t slot, int64_t len);

/* Resume slot s from a store: E4M3 records are copied in; F32 records are
 * quantized into the slot by the device quantizer (kv8_quantize_rows), and
 * the file is left as it is.  Sets the slot's length to the store's count.
 * KV8_EINVAL if the store holds more tokens than a slot. */
int kv8_pool_load(kv8_pool* pool, int32_t slot, kv8_store* st, void* stream);

/* Persist slot s: appends its tokens [n_store, len) to the store, where
 * n_store is the store's count; an F32 store is first rewritten in E4M3
 * from the slot's quantized rows (kv8_store_append).  KV8_EINVAL if the
 * store holds more tokens than the slot. */
int kv8_pool_save(kv8_pool* pool, int32_t slot, kv8_store* st, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KV8_POOL_H */
