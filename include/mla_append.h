/*
 * mla_append.h — C ABI of the paged latent append (gfx950).
 *
 * The operation.  Each layer's latent cache is a paged array [NB, BS, 576]
 * bf16 whose elements 0..511 are the compressed kv_c and 512..575 the k_rope
 * shared by all heads (page "MLA 的 TP 切分：为什么 8 张 GPU 存了同一份 KV
 * cache", section 3.1).  Decode reads token t of request b from row
 * (block_table[b*M + t/BS], t%BS).  The append stores, for every request b
 * with positions[b] = p >= 0,
 *
 *   latent_cache[block_table[b*M + p/BS], p%BS, 0:512]   = kv_c[b, 0:512]
 *   latent_cache[block_table[b*M + p/BS], p%BS, 512:576] = k_rope[b, 0:64]
 *
 * bit for bit, so that a decode over p + 1 tokens attends to the new token
 * last.  k_rope is stored as given: the caller has already applied the
 * rotary embedding.  Nothing else in the cache changes.
 *
 * Conventions: as in mla_decode.h (device pointers owned by the caller,
 * asynchronous on `stream`, host-side argument checks before any HIP call,
 * no allocation).
 *
 * Arguments:
 *   kv_c          bf16, row b at kv_c + b*kv_c_stride (elements); the first 512
 *                 elements of the row are used.  16-byte aligned, stride a
 *                 multiple of 8 and >= 512.
 *   k_rope        bf16, row b at k_rope + b*k_rope_stride; first 64 elements.
 *                 16-byte aligned, stride a multiple of 8 and >= 64.  (Both
 *                 may point into one [B, 576] row-major buffer: kv_c = base,
 *                 k_rope = base + 512, both strides 576.)
 *   positions     int32 [B]: index of the new token in its request (the
 *                 request's length before the append).  A negative value
 *                 means no token for that request (padding) and is skipped.
 *   block_table   int32 [B, M], the decode's table.
 *   latent_cache  bf16 [NB, BS, 576], 16-byte aligned (written).
 *   skipped       int32 device counter or NULL.  Requests whose position is
 *                 >= M*BS or whose block id is outside [0, NB) are not
 *                 written; each adds 1 here (the caller zeroes it).
 *   B >= 0 (0 is a no-op), NB >= 1, M >= 1, BS a power of two in [16, 1024],
 *   M*BS <= 2^28.
 *
 * Two requests that map to the same row race: which one lands is unspecified.
 */
#ifndef MLA_APPEND_H
#define MLA_APPEND_H

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

mla_status mla_append_latent(const void* kv_c, int32_t kv_c_stride,
                             const void* k_rope, int32_t k_rope_stride,
                             const int32_t* positions, const int32_t* block_table,
                             void* latent_cache, int32_t* skipped,
                             int32_t B, int32_t NB, int32_t BS, int32_t M, void* stream);

/* The same append into an FP8 latent cache [NB, BS, 576] of OCP e4m3 bytes
 * holding the values kv_scale * e4m3(byte), as mla_decode_fp8 reads it (page
 * "MLA 的 TP 切分：为什么 8 张 GPU 存了同一份 KV cache", sections 2.3 and 5.1
 * price the FP8 cache; they give no scale convention).  Each bf16 input
 * value v is stored as the e4m3 code nearest to fp32(v) / kv_scale (the
 * quotient correctly rounded to fp32, then rounded to the nearest code with
 * ties to the even mantissa), magnitudes past 448 saturated to +-448 and NaN
 * stored as 0x7F.  kv_scale must be finite and non-zero (else
 * MLA_ERR_BAD_SCALE); every other argument, check and error is as for
 * mla_append_latent, with latent_cache_fp8 16-byte aligned. */
mla_status mla_append_latent_fp8(const void* kv_c, int32_t kv_c_stride,
                                 const void* k_rope, int32_t k_rope_stride,
                                 const int32_t* positions, const int32_t* block_table,
                                 void* latent_cache_fp8, float kv_scale, int32_t* skipped,
                                 int32_t B, int32_t NB, int32_t BS, int32_t M, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_APPEND_H */
