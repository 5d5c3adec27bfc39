/*
 * mla_decode.h — C ABI of the absorbed-MLA decode library for MI355X (gfx950).
 *
 * The operation.  In decode, absorbed Multi-head Latent Attention lets every
 * query head, already projected into the latent space, attend directly over
 * one shared latent per cached token (page "DP attention + expert parallel:
 * MLA KV replication", section "A strong answer").  Per layer the cache is a
 * paged array [NB, BS, 576] whose elements 0..511 are kv_c and 512..575 are
 * k_rope; the 64 RoPE dimensions are shared by all heads MQA-style (page
 * "MLA 的 TP 切分：为什么 8 张 GPU 存了同一份 KV cache", sections 一 and
 * 3.1).  The value vector is the kv_c part, since the value head size equals
 * kv_lora_rank (page "DP 与 DPA 的区别：SGLang 并行部署与路由", section
 * "MLA：KV 是一份共享 latent，没有多个 head 可切").  For request b with
 * L = seq_lens[b] cached tokens, token t lives in row
 * latent_cache[block_table[b*M + t/BS], t%BS, :] and, for each head h,
 *
 *   s_t      = scale * sum_{d<576} q[b,h,d] * c_t[d]
 *   out[b,h] = sum_t softmax_t(s)_t * c_t[0:512]            (bf16, RNE)
 *   lse[b,h] = ln sum_t exp(s_t)                            (fp32)
 *
 * L = 0 gives out = 0 and lse = -inf.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library only borrows them for the work it enqueues on `stream`.
 *   - Calls are asynchronous: they enqueue kernels on `stream` and return
 *     without synchronising.  seq_lens is never read on the host.
 *   - The library allocates no device memory.  Scratch (the work plan and
 *     split-KV partial results) lives in a caller-provided workspace of at
 *     least mla_decode_workspace_bytes(...) bytes, 256-byte aligned.
 *   - Argument checks run on the host before any HIP call; a failed check
 *     returns its status and enqueues nothing.  MLA_ERR_HIP reports a
 *     launch failure (hipGetLastError after the launch).
 *   - Data-dependent contract violations (seq_lens[b] < 0 or > M*BS, a used
 *     block-table entry outside [0, NB)) never cause out-of-bounds accesses:
 *     lengths are clamped to [0, M*BS] and bad block ids are replaced by 0.
 *     The affected outputs are unspecified and a flag is raised in the
 *     workspace (read it with mla_decode_read_error).
 *   - Calls that share a workspace must be ordered (same stream, or
 *     synchronised); concurrent calls need separate workspaces.
 *   - Supported shapes: 1 <= H <= 128; BS a power of two in [16, 1024];
 *     B >= 0 (B = 0 is a no-op); M >= 1; NB >= 1; M*BS <= 2^28.
 *
 * Layouts (all row-major, contiguous):
 *   q            bf16  [B, H, 576]    16-byte aligned
 *   latent_cache bf16  [NB, BS, 576]  16-byte aligned
 *   block_table  int32 [B, M]
 *   seq_lens     int32 [B]
 *   out          bf16  [B, H, 512]    16-byte aligned  (written)
 *   lse          fp32  [B, H]         4-byte aligned   (written, natural log)
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                        */
  MLA_ERR_BAD_SHAPE = 2,    /* negative or overflowing sizes                      */
  MLA_ERR_UNSUPPORTED = 3,  /* H, BS or chunk_tokens outside the supported set    */
  MLA_ERR_BAD_SCALE = 4,    /* scale (or kv_scale) is not finite, or the factor the
                               kernels apply to raw scores, scale * kv_scale * log2(e)
                               rounded to fp32, overflows                         */
  MLA_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required         */
  MLA_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed         */
  MLA_ERR_ALIGNMENT = 7,    /* a pointer violates the alignment stated above      */
  /* Not statuses: they widen the type's range to every int32 value, so that
   * any value a caller passes to mla_status_string is a valid mla_status. */
  MLA_STATUS_RANGE_MIN_ = -2147483647 - 1,
  MLA_STATUS_RANGE_MAX_ = 2147483647
} mla_status;

/* Bits of the data-check word raised in the workspace (see mla_decode_read_error). */
#define MLA_CHECK_SEQ_LEN_RANGE 1  /* some seq_lens[b] < 0 or > M*BS (clamped)       */
#define MLA_CHECK_BLOCK_ID_RANGE 2 /* some used block id outside [0, NB) (set to 0)  */
#define MLA_CHECK_SCORE_RANGE 8    /* some request's scaled scores lie beyond what the
                                      fp32 softmax resolves (about 2^30 in log2 units,
                                      where one ulp exceeds the kernel's exponent
                                      headroom of 64); that request's outputs are
                                      unspecified                                     */
#define MLA_CHECK_MERGE_WAIT 4     /* a split merge stopped waiting for its partners
                                      (never expected; outputs of that request are
                                      unspecified)                                    */

/* Bytes of workspace needed for a batch of B requests with H heads, a block
 * table of M entries per request and block size BS.  Returns 0 when the sizes
 * are outside the supported set.  The figure covers the work plan, two
 * counters per request and split-KV partials for at most B + 1024 work
 * items (normalised outputs in bf16 with 33 or more heads, in fp32 with 32
 * or fewer; log-sum-exps in fp32). */
size_t mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t M, int32_t BS);

/* Whole decode: the plan call followed by the attend call below.  The chunk
 * size of the split-KV plan is chosen on the device from seq_lens. */
mla_status mla_decode(const void* q, const void* latent_cache,
                      const int32_t* block_table, const int32_t* seq_lens,
                      float scale, void* out, float* lse,
                      int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Step 1 — split-KV work plan.  One small kernel reads seq_lens and writes
 * into the workspace a list of work items (request, token range), each at
 * most chunk_tokens long: first the items of requests split into exactly two
 * (pairs; the two items of pair j sit nx positions apart for the first
 * nx * floor(pairs / nx) pairs, nx being the GPU's XCD count for 33 or more
 * heads and 1 otherwise, so that workgroups on one XCD take both, and side
 * by side after them), then the full chunks of every other request, then
 * their shorter last chunks, then one item per empty request.
 * chunk_tokens = 0 lets the device
 * pick the chunk (a multiple of 32 tokens) that minimises an estimate of the
 * makespan on this GPU's compute units; a positive value forces that chunk
 * size (it must be a multiple of 32, and B * ceil(M*BS / chunk_tokens) must
 * not exceed B + 1024).  The plan depends only on seq_lens, so one plan
 * serves every layer of a decode step.
 *
 * Workspace layout written by the plan (int32 words unless noted):
 *   [0] number of work items   [1] chunk tokens   [2] data-check bits
 *   [3] work-queue counter (0 after the plan and after every attend call)
 *   [4] number of items placed as XCD-sharing pairs (2 nx floor(pairs/nx))
 *   [5] number of merge units (16 per request split into 3 or more items
 *   with 65 or more heads, 8 with 33 to 64, 4 with 32 or fewer)
 *   [6] merge-unit queue counter (0 between calls)
 *   at byte 256: per request 4 words: for a pair (position of its first
 *   item, 1, position of its second item, 2), otherwise (first full item,
 *   full-item count, remainder item or -1, total item count); then,
 *   256-byte aligned, two counters per request (a pair with 33 or more
 *   heads: each item's publish word; otherwise tickets taken, partials
 *   published; 0 between calls); then the list of requests split into 3 or more items; then per
 *   item 4 words (request, first token, end token, the request's item
 *   count). */
mla_status mla_decode_plan(const int32_t* seq_lens, int32_t B, int32_t H,
                           int32_t M, int32_t BS, int32_t chunk_tokens,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Step 2 — attention over every work item of the plan (the hot kernel), and
 * the split-KV merge.  An item that covers a whole request writes out/lse
 * directly; an empty request gets out = 0, lse = -inf.  When a request is
 * split, its items' normalised outputs and log-sum-exps are merged, summing
 * in item order: lse = ln sum_s exp(lse_s), out = sum_s exp(lse_s - lse) *
 * o_s (bf16, RNE).  With 33 or more heads the two items of a request split
 * in two each merge half of its heads: each publishes, in the workspace,
 * its bf16 partial of the heads the other item merges (with its
 * log-sum-exps), sets its publish word, waits for the other's, and
 * combines; with 32 or fewer heads the item that finishes second merges
 * the other's fp32 partial.  Wider splits write partials (bf16 with 33 or
 * more heads, fp32 with fewer) and are merged in column blocks by
 * whichever workgroups are free once every item has been taken.  A bf16
 * partial adds at most one bf16 rounding of the partial (2^-8 of its
 * magnitude, which is at most max |V| over the request's tokens) to the
 * merged output.  The result does not depend on which
 * workgroup merges or when.
 * Needs a plan made with the same B, H, M, BS. */
mla_status mla_decode_attend(const void* q, const void* latent_cache,
                             const int32_t* block_table, float scale,
                             void* out, float* lse,
                             int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The whole decode (plan + attend) without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, layouts,
 * results and errors as mla_decode, except:
 *   - the plan and split partials live in a library-owned device array of
 *     64 MiB, one per GPU the library runs on, held until the process ends;
 *     its device address is taken on the first call on each device;
 *   - batches whose plan and partials do not fit it return MLA_ERR_WORKSPACE
 *     before anything is enqueued (at 128 heads that is B above 255; the
 *     plan is limited to the work items that fit, which for large splits can
 *     give a coarser split than mla_decode chooses, never a different result
 *     beyond rounding);
 *   - every call on one GPU shares that array, so calls on one GPU must not
 *     overlap: two such calls in flight at once (on different streams, or
 *     from different host threads without ordering) race and their results
 *     are unspecified.  Each call's plan rewrites every word the attend step
 *     reads and leaves its counters at zero.
 * It calls no hipMalloc, hipFree or other allocating routine. */
mla_status mla_decode_noalloc(const void* q, const void* latent_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              float scale, void* out, float* lse,
                              int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                              void* stream);

/* FP8 latent cache.  The cache holds one byte per element, OCP e4m3 (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7F and
 * 0xFF are NaN), 576 bytes per token: [NB, BS, 576], elements 0..511 kv_c
 * and 512..575 k_rope as for bf16.  The pages price the cache at 576 bytes
 * per token and layer in FP8 (page "MLA 的 TP 切分：为什么 8 张 GPU 存了同一份
 * KV cache", sections 2.3 and 5.1) but give no scale convention; here one
 * fp32 scale per cache dequantises every element: c_t[d] = kv_scale *
 * e4m3(latent_cache[...][d]).  The result is the bf16 decode above over that
 * dequantised cache:
 *
 *   s_t = scale * kv_scale * sum_d q[b,h,d] * e4m3(c8_t[d])
 *   out = kv_scale * sum_t softmax_t(s) * e4m3(c8_t[0:512])
 *
 * (e4m3 values are exact in bf16, so products are exact and accumulate in
 * fp32 as for a bf16 cache.)  Supported: the head counts and block sizes of
 * mla_decode (otherwise MLA_ERR_UNSUPPORTED); kv_scale finite and
 * scale * kv_scale * log2(e) finite in fp32 (else MLA_ERR_BAD_SCALE).
 * Everything else (plan, workspace, layouts of q, block_table, seq_lens,
 * out, lse, errors) is as for mla_decode / mla_decode_attend; the plan call
 * is shared. */
mla_status mla_decode_fp8(const void* q, const void* latent_cache_fp8,
                          const int32_t* block_table, const int32_t* seq_lens,
                          float scale, float kv_scale, void* out, float* lse,
                          int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                          void* workspace, size_t workspace_bytes, void* stream);

mla_status mla_decode_attend_fp8(const void* q, const void* latent_cache_fp8,
                                 const int32_t* block_table, float scale, float kv_scale,
                                 void* out, float* lse,
                                 int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Synchronises `stream`, then copies the data-check word of the workspace
 * into *flags (0 = no violation seen since the last plan). */
mla_status mla_decode_read_error(const void* workspace, int32_t* flags, void* stream);

/* Human-readable name of a status code (static storage). */
const char* mla_status_string(mla_status s);

/* Library ABI version (increments on any signature change). */
int32_t mla_decode_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
