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

// FP8 (e4m3) cache of values kv_scale * e4m3(byte): each bf16 value v is
// stored as the e4m3 code nearest to fp32(v) / kv_scale (the quotient
// correctly rounded to fp32, then to the nearest code with ties to even by
// the hardware conversion), magnitudes past 448 saturated to +-448 (the
// conversion alone would give NaN there) and NaN stored as 0x7F.
__device__ __forceinline__ uint32_t e4m3_byte(float q) {
  if (q != q) return 0x7Fu;
  const float c = fminf(fmaxf(q, -448.0f), 448.0f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false)) & 0xFFu;
}
// 8 bf16 values (16 bytes) to 8 e4m3 bytes (low byte first)
__device__ __forceinline__ uint2 e4m3x8(uint4 v, float kv_scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t bits = (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
    const float q = __uint_as_float(bits) / kv_scale;
    out[i >> 2] |= e4m3_byte(q) << (8 * (i & 3));
  }
  return make_uint2(out[0], out[1]);
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void mla_append_fp8_kernel(
    const uint16_t* __restrict__ kv_c, int kv_c_stride, const uint16_t* __restrict__ k_rope,
    int k_rope_stride, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ block_table, uint8_t* __restrict__ cache, float kv_scale,
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
  // one 576-byte row: lane l stores kv_c bytes 8l .. 8l+7, lanes 0..7 also
  // the k_rope bytes 512 + 8l .. +7
  uint8_t* row = cache + ((long long)blk * BS + (p & (BS - 1))) * kD;
  const uint4 v = *reinterpret_cast<const uint4*>(kv_c + (long long)b * kv_c_stride + 8 * lane);
  *reinterpret_cast<uint2*>(row + 8 * lane) = e4m3x8(v, kv_scale);
  if (lane < 8) {
    const uint4 r = *reinterpret_cast<const uint4*>(k_rope + (long long)b * k_rope_stride + 8 * lane);
    *reinterpret_cast<uint2*>(row + kDV + 8 * lane) = e4m3x8(r, kv_scale);
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

mla_status mla_append_latent_fp8(const void* kv_c, int32_t kv_c_stride, const void* k_rope,
                                 int32_t k_rope_stride, const int32_t* positions,
                                 const int32_t* block_table, void* latent_cache_fp8, float kv_scale,
                                 int32_t* skipped, int32_t B, int32_t NB, int32_t BS, int32_t M,
                                 void* stream) {
  if (B < 0 || NB < 1 || M < 1) return MLA_ERR_BAD_SHAPE;
  const int lg = ilog2_pow2(BS);
  if (lg < 4 || lg > 10) return MLA_ERR_UNSUPPORTED;
  if ((long long)M * BS > (1ll << 28)) return MLA_ERR_UNSUPPORTED;
  if (kv_c_stride < kDV || k_rope_stride < kD - kDV) return MLA_ERR_BAD_SHAPE;
  if (!(kv_scale == kv_scale) || kv_scale == 0.0f || kv_scale > 3.4e38f || kv_scale < -3.4e38f)
    return MLA_ERR_BAD_SCALE;
  if (B == 0) return MLA_OK;
  if (!kv_c || !k_rope || !positions || !block_table || !latent_cache_fp8)
    return MLA_ERR_NULL_POINTER;
  if (!aligned16(kv_c) || !aligned16(k_rope) || !aligned16(latent_cache_fp8) ||
      (kv_c_stride % 8) || (k_rope_stride % 8) ||
      (reinterpret_cast<uintptr_t>(positions) & 3) || (reinterpret_cast<uintptr_t>(block_table) & 3) ||
      (reinterpret_cast<uintptr_t>(skipped) & 3))
    return MLA_ERR_ALIGNMENT;
  const int grid = (B + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(mla_append_fp8_kernel, dim3(grid), dim3(64 * kRowsPerBlock), 0,
                     (hipStream_t)stream, static_cast<const uint16_t*>(kv_c), (int)kv_c_stride,
                     static_cast<const uint16_t*>(k_rope), (int)k_rope_stride, positions,
                     block_table, static_cast<uint8_t*>(latent_cache_fp8), kv_scale, skipped,
                     (int)B, (int)NB, lg, (int)M);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
