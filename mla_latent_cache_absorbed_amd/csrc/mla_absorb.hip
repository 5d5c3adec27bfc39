// Query absorption and value up-projection around the absorbed decode, for
// gfx950.
//
// In the absorbed form each head's query is projected into the latent space
// before attention and its latent-space output is projected back to the
// value head after it (page "DP attention + expert parallel: MLA KV
// replication", section "A strong answer"; the latent is kv_lora_rank = 512
// wide and the RoPE part 64 wide, page "MLA 的 TP 切分…", section 一; the
// per-head nope and value widths are 128, the head_dim of that page's MHA
// baseline).  With W_UK[h] and W_UV[h] the [128, 512] up-projections of
// head h:
//
//   q[b,h,0:512]   = W_UK[h]^T q_nope[b,h]      q[b,h,512:576] = q_rope[b,h]
//   o[b,h,0:128]   = W_UV[h] out[b,h]
//
// Both are per-head products with a small batch, Y[b,h,n] = sum_k
// W[h,n,k] X[b,h,k], and one kernel serves both: each wave computes 32x32
// tiles of Y^T (32 rows n of W against 32 requests b) over the whole K on
// 32x32x16 bf16 MFMA, loading both operands straight from global memory as
// 16-byte K-contiguous fragments.  W_UK is used transposed ([H, 512, 128], K
// contiguous); mla_absorb_prepare makes that copy once, when the weights are
// loaded.  The four waves of a workgroup share the W rows (their four request
// tiles); all workgroups of one head land on one XCD, so the head's X rows are
// read from HBM once and then from that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_absorb.h"

namespace {

constexpr int kD = 576;
constexpr int kDV = 512;
constexpr int kDN = 128;    // nope part of a query head
constexpr int kDR = 64;     // RoPE part
constexpr int kDQ = kDN + kDR;
constexpr int kDVH = 128;   // value head

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const __bf16* W;  // [H, N, K]
  const __bf16* X;  // row b, head h at X + b*x_row + h*x_head, K contiguous
  __bf16* Y;        // row b, head h at Y + b*y_row + h*y_head, N contiguous
  long long x_row, y_row;
  int x_head, y_head;
  int B, H, N;
  // optional copy of a 64-wide part: R[b,h,0:64] -> Y[b,h,N:N+64]
  const __bf16* R;
  long long r_row;
  int r_head;
};

// Workgroup i -> (head, group of NT n-tiles), with all groups of a head on
// XCD i % 8.  Each wave computes NT 32x32 tiles of Y^T for one tile of 32
// requests, so its X fragments serve NT products.  Loads are issued a batch
// of kBatch k-steps ahead of the MFMAs that use them (scheduling barriers
// keep the compiler from interleaving them one step at a time, which leaves
// a wave waiting on each load in turn).  Measured at 124 requests x 128
// heads: NT = 4, kBatch = 4 for the absorption (K = 128) and NT = 2,
// kBatch = 4 for the up-projection (K = 512) were the fastest of the
// shapes tried.
template <int K, int NT, int kBatch>
__global__ __launch_bounds__(256) void mla_head_gemm_kernel(GemmArgs a) {
  constexpr int kSteps = K / 16;
  constexpr int kBatches = kSteps / kBatch;
  static_assert(kSteps % kBatch == 0, "K / 16 must be a multiple of the batch");
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int T = a.N / (32 * NT);
  const int i = blockIdx.x;
  const int r = i >> 3;
  const int h = (i & 7) + 8 * (r / T);
  const int ng = r % T;
  const int b0 = 128 * blockIdx.y + 32 * w;
  if (h >= a.H || b0 >= a.B) return;

  const int kh = 8 * (lane >> 5);
  const int bl = min(b0 + (lane & 31), a.B - 1);  // rows past B load row B-1, never stored
  const __bf16* wp = a.W + ((long long)h * a.N + 32 * NT * ng + (lane & 31)) * K + kh;
  const __bf16* xp = a.X + (long long)bl * a.x_row + (long long)h * a.x_head + kh;

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  bf16x8 fx[2][kBatch], fw[2][kBatch][NT];
  auto load = [&](int buf, int j) {
#pragma unroll
    for (int s = 0; s < kBatch; ++s) {
      const int k = 16 * (kBatch * j + s);
      fx[buf][s] = *reinterpret_cast<const bf16x8*>(xp + k);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        fw[buf][s][t] = *reinterpret_cast<const bf16x8*>(wp + (long long)32 * t * K + k);
    }
  };
  load(0, 0);
#pragma unroll
  for (int j = 0; j < kBatches; ++j) {
    if (j + 1 < kBatches) load((j + 1) & 1, j + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kBatch; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j & 1][s][t], fx[j & 1][s], acc[t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the RoPE part rides along with group 0: 32 rows x 128 B per wave, all
  // loads issued before the stores
  bf16x8 rv[4];
  const bool rope = a.R != nullptr && ng == 0;
  if (rope) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = lane + 64 * j;
      const int row = min(b0 + (c >> 3), a.B - 1);
      rv[j] = *reinterpret_cast<const bf16x8*>(a.R + (long long)row * a.r_row +
                                               (long long)h * a.r_head + 8 * (c & 7));
    }
  }

  // acc[t][e] is Y^T[row 8(e/4) + 4(lane/32) + e%4, column lane%32] of tile t:
  // four consecutive n of one request per group of four registers
  const int b = b0 + (lane & 31);
  if (b < a.B) {
    __bf16* yp = a.Y + (long long)b * a.y_row + (long long)h * a.y_head + 32 * NT * ng + 4 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[t][4 * g + e]);
        *reinterpret_cast<bf16x4*>(yp + 32 * t + 8 * g) = v;
      }
  }
  if (rope) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = lane + 64 * j;
      const int row = b0 + (c >> 3);
      if (row < a.B)
        *reinterpret_cast<bf16x8*>(a.Y + (long long)row * a.y_row + (long long)h * a.y_head + a.N +
                                   8 * (c & 7)) = rv[j];
    }
  }
}

// W_UK [H, 128, 512] -> [H, 512, 128], one 64x64 tile per workgroup through LDS.
__global__ __launch_bounds__(256) void mla_transpose_wuk_kernel(const uint16_t* __restrict__ src,
                                                                uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][65];
  const int j0 = 64 * blockIdx.x, d0 = 64 * blockIdx.y, h = blockIdx.z;
  const int t = threadIdx.x;
  for (int e = t; e < 64 * 64; e += 256) {
    const int rr = e >> 6, cc = e & 63;
    tile[rr][cc] = src[((long long)h * kDN + d0 + rr) * kDV + j0 + cc];
  }
  __syncthreads();
  for (int e = t; e < 64 * 64; e += 256) {
    const int rr = e >> 6, cc = e & 63;
    dst[((long long)h * kDV + j0 + rr) * kDN + d0 + cc] = tile[cc][rr];
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

mla_status check_bh(int32_t B, int32_t H) {
  if (B < 0 || H < 1) return MLA_ERR_BAD_SHAPE;
  if (H > 128 || B > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

template <int K, int NT, int KB>
mla_status launch_gemm(const GemmArgs& a, void* stream) {
  const int T = a.N / (32 * NT);
  const int groups = (a.H + 7) / 8;
  dim3 grid(8 * T * groups, (a.B + 127) / 128);
  hipLaunchKernelGGL((mla_head_gemm_kernel<K, NT, KB>), grid, dim3(256), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

mla_status mla_absorb_prepare(const void* w_uk, void* w_uk_t, int32_t H, void* stream) {
  if (H < 1) return MLA_ERR_BAD_SHAPE;
  if (H > 128) return MLA_ERR_UNSUPPORTED;
  if (!w_uk || !w_uk_t) return MLA_ERR_NULL_POINTER;
  if (!aligned16(w_uk) || !aligned16(w_uk_t)) return MLA_ERR_ALIGNMENT;
  hipLaunchKernelGGL(mla_transpose_wuk_kernel, dim3(kDV / 64, kDN / 64, H), dim3(256), 0,
                     (hipStream_t)stream, static_cast<const uint16_t*>(w_uk),
                     static_cast<uint16_t*>(w_uk_t));
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_absorb_query(const void* q_in, const void* w_uk_t, void* q, int32_t B, int32_t H,
                            void* stream) {
  mla_status s = check_bh(B, H);
  if (s != MLA_OK || B == 0) return s;
  if (!q_in || !w_uk_t || !q) return MLA_ERR_NULL_POINTER;
  if (!aligned16(q_in) || !aligned16(w_uk_t) || !aligned16(q)) return MLA_ERR_ALIGNMENT;
  GemmArgs a;
  a.W = static_cast<const __bf16*>(w_uk_t);
  a.X = static_cast<const __bf16*>(q_in);
  a.Y = static_cast<__bf16*>(q);
  a.x_row = (long long)H * kDQ;
  a.x_head = kDQ;
  a.y_row = (long long)H * kD;
  a.y_head = kD;
  a.B = B;
  a.H = H;
  a.N = kDV;
  a.R = static_cast<const __bf16*>(q_in) + kDN;
  a.r_row = (long long)H * kDQ;
  a.r_head = kDQ;
  return launch_gemm<kDN, 4, 4>(a, stream);
}

mla_status mla_up_project(const void* out, const void* w_uv, void* o, int32_t B, int32_t H,
                          void* stream) {
  mla_status s = check_bh(B, H);
  if (s != MLA_OK || B == 0) return s;
  if (!out || !w_uv || !o) return MLA_ERR_NULL_POINTER;
  if (!aligned16(out) || !aligned16(w_uv) || !aligned16(o)) return MLA_ERR_ALIGNMENT;
  GemmArgs a;
  a.W = static_cast<const __bf16*>(w_uv);
  a.X = static_cast<const __bf16*>(out);
  a.Y = static_cast<__bf16*>(o);
  a.x_row = (long long)H * kDV;
  a.x_head = kDV;
  a.y_row = (long long)H * kDVH;
  a.y_head = kDVH;
  a.B = B;
  a.H = H;
  a.N = kDVH;
  a.R = nullptr;
  a.r_row = 0;
  a.r_head = 0;
  return launch_gemm<kDV, 2, 4>(a, stream);
}

}  // extern "C"
