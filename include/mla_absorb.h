/*
 * mla_absorb.h — C ABI of the products on either side of the absorbed
 * decode (gfx950): query absorption before it, value up-projection after it.
 *
 * The operation.  In decode the engine runs MLA in its absorbed form: each
 * head's query is projected into the latent space and attends over the
 * shared latent directly (page "DP attention + expert parallel: MLA KV
 * replication", section "A strong answer"), and the head's attention output,
 * a latent-space vector, is projected to the value head afterwards.  The
 * latent is kv_lora_rank = 512 wide with a 64-wide RoPE part (page "MLA 的
 * TP 切分：为什么 8 张 GPU 存了同一份 KV cache", section 一); each query
 * head has a 128-wide nope part and each value head is 128 wide (that page's
 * MHA baseline head_dim).  With W_UK[h], W_UV[h] the [128, 512] key and
 * value up-projections of head h (rows of the usual kv_b_proj weight):
 *
 *   q[b,h,0:512]   = sum_d W_UK[h,d,:] q_in[b,h,d]       (d < 128)
 *   q[b,h,512:576] = q_in[b,h,128:192]                    (copied bits)
 *   o[b,h,i]       = sum_j W_UV[h,i,j] out[b,h,j]         (i < 128, j < 512)
 *
 * q is the decode's query input and out its output (mla_decode.h).  Products
 * are exact bf16 x bf16 with fp32 accumulation; results are rounded to bf16
 * to nearest-even.
 *
 * Conventions: as in mla_decode.h (device pointers owned by the caller,
 * asynchronous on `stream`, host checks before any HIP call, no allocation;
 * every pointer 16-byte aligned).  Supported: 1 <= H <= 128, 0 <= B <= 2^24
 * (B = 0 is a no-op).
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Once, when the weights are loaded: w_uk bf16 [H, 128, 512] (W_UK) ->
 * w_uk_t bf16 [H, 512, 128] (each head's W_UK transposed), the layout
 * mla_absorb_query reads.  Exact copy of the bits. */
mla_status mla_absorb_prepare(const void* w_uk, void* w_uk_t, int32_t H, void* stream);

/* q_in bf16 [B, H, 192] (per head: 128 nope values, then 64 RoPE values,
 * already rotated); w_uk_t bf16 [H, 512, 128] from mla_absorb_prepare;
 * q bf16 [B, H, 576] (written).  q_in and q must not overlap. */
mla_status mla_absorb_query(const void* q_in, const void* w_uk_t, void* q,
                            int32_t B, int32_t H, void* stream);

/* out bf16 [B, H, 512] (the decode's output); w_uv bf16 [H, 128, 512]
 * (W_UV); o bf16 [B, H, 128] (written; as [B, H*128] it is the input of
 * the output projection).  out and o must not overlap. */
mla_status mla_up_project(const void* out, const void* w_uv, void* o,
                          int32_t B, int32_t H, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
