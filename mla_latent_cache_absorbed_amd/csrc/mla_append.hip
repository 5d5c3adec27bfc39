// Paged latent append for gfx950: the step before decode, which stores each
// request's newest token into the paged latent cache.
//
// The cache of one layer is [NB, BS, 576] bf16 with elements 0..511 the
// compressed kv_c and 512..575 the MQA-shared k_rope (page "MLA 的 TP
// 切分…", section 3.1).  Token t of request b lives at row
// (block_table[b*M + t/BS], t%BS), the mapping the decode reads with, so the
// token at position p is written there; a decode over p+1 tokens then sees it
// as its last token.
//
// One wave per request: 64 lanes store the 1,024 bytes of kv_c as 16-byte
// vectors, 8 of them also the 128 bytes of k_rope.  The kernel is bound by
// launch and memory latency (one 1,152-byte row per request).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_append.h"

namespace {

constexpr int kD = 576;
constexpr int kDV = 512;
constexpr int kRowsPerBlock = 4;  // one wave per request, four waves per workgroup

__global__ __launch_bounds__(64 * kRowsPerBlock) void mla_append_kernel(
    const uint16_t* __restrict__ kv_c, int kv_c_stride, const uint16_t* __restrict__ k_rope,
    int k_rope_stride, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ block_table, uint16_t* __restrict__ cache,
    int32_t* __restrict__ skipped, int B, int NB, int lgBS, int M) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (b >= B) return;
  const int p = positions[b];
  if (p < 0) return;  // no token for this request
  const int BS = 1 << lgBS;
  int blk = -1;
  if (p < M * BS) blk = block_table[(long long)b * M + (p >> lgBS)];
  if (blk < 0 || blk >= NB) {
    if (lane == 0 && skipped != nullptr) atomicAdd(skipped, 1);
    return;
  }
  uint16_t* row = cache + ((long long)blk * BS + (p & (BS - 1))) * kD;
  const uint4 v = *reinterpret_cast<const uint4*>(kv_c + (long long)b * kv_c_stride + 8 * lane);
  *reinterpret_cast<uint4*>(row + 8 * lane) = v;
  if (lane < 8) {
    const uint4 r = *reinterpret_cast<const uint4*>(k_rope + (long long)b * k_rope_stride + 8 * lane);
    *reinterpret_cast<uint4*>(row + kDV + 8 * lane) = r;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int ilog2_pow2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

}  // namespace

extern "C" {

mla_status mla_append_latent(const void* kv_c, int32_t kv_c_stride, const void* k_rope,
                             int32_t k_rope_stride, const int32_t* positions,
                             const int32_t* block_table, void* latent_cache, int32_t* skipped,
                             int32_t B, int32_t NB, int32_t BS, int32_t M, void* stream) {
  if (B < 0 || NB < 1 || M < 1) return MLA_ERR_BAD_SHAPE;
  const int lg = ilog2_pow2(BS);
  if (lg < 4 || lg > 10) return MLA_ERR_UNSUPPORTED;
  if ((long long)M * BS > (1ll << 28)) return MLA_ERR_UNSUPPORTED;
  if (kv_c_stride < kDV || k_rope_stride < kD - kDV) return MLA_ERR_BAD_SHAPE;
  if (B == 0) return MLA_OK;
  if (!kv_c || !k_rope || !positions || !block_table || !latent_cache)
    return MLA_ERR_NULL_POINTER;
  if (!aligned16(kv_c) || !aligned16(k_rope) || !aligned16(latent_cache) ||
      (kv_c_stride % 8) || (k_rope_stride % 8) ||
      (reinterpret_cast<uintptr_t>(positions) & 3) || (reinterpret_cast<uintptr_t>(block_table) & 3) ||
      (reinterpret_cast<uintptr_t>(skipped) & 3))
    return MLA_ERR_ALIGNMENT;
  const int grid = (B + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(mla_append_kernel, dim3(grid), dim3(64 * kRowsPerBlock), 0,
                     (hipStream_t)stream, static_cast<const uint16_t*>(kv_c), (int)kv_c_stride,
                     static_cast<const uint16_t*>(k_rope), (int)k_rope_stride, positions,
                     block_table, static_cast<uint16_t*>(latent_cache), skipped, (int)B, (int)NB,
                     lg, (int)M);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
