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
// 32x32x16 bf16 MFMA.  The K dimension goes in chunks of 128: each chunk's W
// rows and X rows are staged in LDS with coalesced 16-byte loads (16-byte
// chunk c of row r at slot c ^ (r % 16)), the MFMA fragments are read from
// there, and the output tile goes back through LDS so that each request's
// contiguous output bytes are stored by consecutive lanes.  W_UK is used
// transposed ([H, 512, 128], K contiguous); mla_absorb_prepare makes that
// copy once, when the weights are loaded.  The four waves of a workgroup
// share the W rows (their four request tiles); all workgroups of one head
// land on one XCD, so the head's X rows are read from HBM once and then from
// that XCD's L2.

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
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

// Workgroup (i, y) -> head h and group ng of NT n-tiles (all groups of a
// head on XCD i % 8, so its X rows come from HBM once and then from that
// XCD's L2), requests 128 y .. 128 y + 127.  K goes in chunks of 128: the
// workgroup stages the chunk of its 32 NT rows of W and of its 128 X rows in
// LDS with coalesced 16-byte loads (each row's 256 bytes are contiguous),
// then each wave multiplies its 32 requests by the NT n-tiles from LDS.  The
// 16-byte chunk c of LDS row r sits at slot c ^ (r % 16), so the fragment
// reads of 32 rows at one chunk hit distinct banks.
constexpr int kKC = 128;                 // K per LDS chunk
constexpr int kRowB = kKC * 2;           // bytes per LDS row

__device__ __forceinline__ int lds_slot(int row, int c16) { return row * kRowB + 16 * (c16 ^ (row & 15)); }

// kWStream: W is read with non-temporal loads (it streams through the
// caches; a gain for the absorption, a loss for the up-projection, measured)
template <int K, int NT, bool kWStream>
__global__ __launch_bounds__(256, 2) void mla_head_gemm_kernel(GemmArgs a) {
  static_assert(K % kKC == 0, "K is a multiple of the chunk");
  constexpr int kWRows = 32 * NT;
  constexpr int kXRows = 128;
  constexpr int kLoads = (kWRows + kXRows) * (kRowB / 16) / 256;  // 16-byte loads per thread
  __shared__ __attribute__((aligned(16))) char lds[(kWRows + kXRows) * kRowB];
  char* const lw = lds;
  char* const lx = lds + kWRows * kRowB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int T = a.N / kWRows;
  const int i = blockIdx.x;
  const int r = i >> 3;
  const int h = (i & 7) + 8 * (r / T);
  const int ng = r % T;
  const int bbase = 128 * blockIdx.y;
  if (h >= a.H) return;  // uniform over the workgroup
  const int n0 = kWRows * ng;

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  for (int kc = 0; kc < K; kc += kKC) {
    // stage: row q < kWRows is W row n0 + q, else X row bbase + q - kWRows
    // (rows past B load row B - 1; their results are never stored).  Load j
    // covers rows 16 j .. 16 j + 15, so whether it reads W or X is known at
    // compile time.
    static_assert(kWRows % 16 == 0, "W rows fill whole loads");
    constexpr int kWLoads = kWRows / 16;
    const int c16 = tid & 15;
    i32x4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
      const int row = (tid >> 4) + 16 * j;
      const i32x4* src = reinterpret_cast<const i32x4*>(a.W + ((long long)h * a.N + n0 + row) * K + kc + 8 * c16);
      if constexpr (kWStream) v[j] = __builtin_nontemporal_load(src);
      else v[j] = *src;
    }
#pragma unroll
    for (int j = kWLoads; j < kLoads; ++j) {
      const int b = min(bbase + (tid >> 4) + 16 * j - kWRows, a.B - 1);
      v[j] = *reinterpret_cast<const i32x4*>(a.X + (long long)b * a.x_row + (long long)h * a.x_head + kc + 8 * c16);
    }
    if (kc > 0) __syncthreads();  // the previous chunk's fragment reads are done
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int c = tid + 256 * j;
      *reinterpret_cast<i32x4*>(lds + lds_slot(c >> 4, c & 15)) = v[j];
    }
    __syncthreads();
    // wave w: requests bbase + 32 w .. +31 (B operand), NT n-tiles (A)
    const int xr = 32 * w + (lane & 31);
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s) {
      const int c16 = 2 * s + (lane >> 5);
      const bf16x8 fb = *reinterpret_cast<const bf16x8*>(lx + lds_slot(xr, c16));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 fa = *reinterpret_cast<const bf16x8*>(lw + lds_slot(32 * t + (lane & 31), c16));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[t], 0, 0, 0);
      }
    }
  }

  // acc[t][e] is Y^T[row 8(e/4) + 4(lane/32) + e%4, column lane%32] of tile t:
  // four consecutive n of one request per group of four registers.  The
  // workgroup's output block (128 requests x 32 NT values of n) goes through
  // LDS, 16-byte chunk c of request row q at slot c ^ (q % (4 NT)), so that
  // each request's 64 NT contiguous bytes are stored by consecutive lanes.
  constexpr int kOutRow = 64 * NT;  // bytes per request row of the block
  constexpr int kChunks = 4 * NT;   // 16-byte chunks per row
  static_assert(128 * kOutRow <= (kWRows + kXRows) * kRowB, "output block fits the LDS");
  auto out_slot = [&](int q, int c) { return q * kOutRow + 16 * (c ^ (q & (kChunks - 1))); };
  __syncthreads();  // every fragment read is done
  {
    const int q = 32 * w + (lane & 31);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = static_cast<__bf16>(acc[t][4 * g + e]);
        *reinterpret_cast<bf16x4*>(lds + out_slot(q, 4 * t + g) + 8 * (lane >> 5)) = o;
      }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 128 * kChunks / 256; ++j) {
    const int idx = tid + 256 * j;
    const int q = idx / kChunks, c = idx % kChunks;
    const int b = bbase + q;
    // the output is written once and read by the next kernel: it streams
    // out (non-temporal stores)
    if (b < a.B)
      __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(lds + out_slot(q, c)),
                                  reinterpret_cast<i32x4*>(a.Y + (long long)b * a.y_row +
                                                           (long long)h * a.y_head + n0 + 8 * c));
  }
  // the RoPE part rides along with group 0: 32 rows x 128 B per wave
  if (a.R != nullptr && ng == 0) {
    const int b0 = bbase + 32 * w;
    bf16x8 rv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = lane + 64 * j;
      const int row = min(b0 + (c >> 3), a.B - 1);
      rv[j] = *reinterpret_cast<const bf16x8*>(a.R + (long long)row * a.r_row +
                                               (long long)h * a.r_head + 8 * (c & 7));
    }
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

template <int K, int NT, bool kWStream>
mla_status launch_gemm(const GemmArgs& a, void* stream) {
  const int T = a.N / (32 * NT);
  const int groups = (a.H + 7) / 8;
  dim3 grid(8 * T * groups, (a.B + 127) / 128);
  hipLaunchKernelGGL((mla_head_gemm_kernel<K, NT, kWStream>), grid, dim3(256), 0, (hipStream_t)stream, a);
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
  return launch_gemm<kDN, 4, true>(a, stream);
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
  return launch_gemm<kDV, 1, false>(a, stream);
}

}  // extern "C"
