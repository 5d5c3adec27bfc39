// Read-only streaming probes of HBM bandwidth on gfx950, used by the
// benchmark to state the read bandwidth this GPU attains next to its 8 TB/s
// peak, and MFMA loops that state the bf16 matrix rate it attains next to
// its 2.5 PFLOP/s peak, for the 32x32x16 and 16x16x32 shapes.  Not part of the decode path: built as its own small
// library.
//
//   mode 0  plain 16-byte global loads into registers, eight in flight per
//           lane, folded with xor into one word per lane (written once);
//   mode 1  16-byte direct-to-LDS loads, the path the decode kernel stages
//           latent rows with: each wave keeps eight 1 KB loads in flight into
//           its own 8 KB of LDS.
//   modes 2 and 3  as 0 and 1, but each workgroup streams its own contiguous
//           region of the buffer (bytes / grid) from start to end, the access
//           pattern of a decode whose work items each walk their own run of
//           cache blocks; in modes 0 and 1 every workgroup walks the buffer
//           with a grid stride, so the whole GPU sweeps it front to back
//           (consecutive workgroups read consecutive 32 KB pieces).
//
// bytes must be a multiple of (grid * 32 KB); the host entry point rounds it
// down.
//
// Every probe kernel holds 160 KB / (workgroups per CU) of LDS, so that the
// dispatcher places exactly that many workgroups on each compute unit (with
// less, it may double some up and leave others idle, and the launch then
// ends with the busiest unit), as the decode kernel's 160 KB does.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr size_t kStep = size_t(kThreads) * 16 * kUnroll;  // bytes per workgroup iteration
constexpr int kLdsPerCu = 160 * 1024;                       // gfx950

// LDS words of a workgroup when kWpc of them are to share a compute unit
template <int kWpc>
constexpr int occ_words() {
  return kLdsPerCu / kWpc / 4;
}

// Keeps a workgroup's occupancy array allocated: every thread passes its
// value through it (one barrier), and the result goes to the sink.
template <int kWords>
__device__ __forceinline__ uint32_t through_lds(uint32_t (&occ)[kWords], uint32_t v) {
  static_assert(kWords >= kThreads, "occupancy array");
  occ[kWords - kThreads + threadIdx.x] = v;
  __syncthreads();
  return occ[kWords - kThreads + ((threadIdx.x + 1) % kThreads)];
}

// index of the 32 KB piece a workgroup reads in iteration it
template <bool kOwnRegion>
__device__ __forceinline__ size_t piece(size_t it, size_t n_iter) {
  return kOwnRegion ? size_t(blockIdx.x) * n_iter + it : it * gridDim.x + blockIdx.x;
}

template <bool kOwnRegion, int kWpc>
__global__ __launch_bounds__(kThreads) void read_regs(const uint4* __restrict__ p, size_t n_iter,
                                                      uint32_t* __restrict__ sink) {
  __shared__ uint32_t occ[occ_words<kWpc>()];
  uint32_t acc = 0;
  for (size_t it = 0; it < n_iter; ++it) {
    const uint4* base = p + piece<kOwnRegion>(it, n_iter) * (kStep / 16) + threadIdx.x;
    uint4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) v[j] = base[j * kThreads];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  sink[size_t(blockIdx.x) * kThreads + threadIdx.x] = through_lds(occ, acc);
}

template <bool kOwnRegion, int kWpc>
__global__ __launch_bounds__(kThreads) void read_lds(const char* __restrict__ p, size_t n_iter,
                                                     uint32_t* __restrict__ sink) {
  // 4 waves x 8 KB at the start of the workgroup's occupancy array
  static_assert(occ_words<kWpc>() >= kThreads / 64 * 8 * 256, "ring fits");
  __shared__ __attribute__((aligned(1024))) uint32_t ring[occ_words<kWpc>()];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* mine = ring + w * 8 * 256;
  for (size_t it = 0; it < n_iter; ++it) {
    // the workgroup's 32 KB: wave w takes 1 KB pieces w, w + 4, ...
    const char* base = p + piece<kOwnRegion>(it, n_iter) * kStep + size_t(w) * 1024 + lane * 16;
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      __builtin_amdgcn_global_load_lds(base + j * 4096, mine + j * 256, 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's eight loads have landed
  }
  __syncthreads();
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) acc ^= mine[j * 256 + lane * 4];
  sink[size_t(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// MFMA loop: every wave runs `iters` rounds of 262,144 flop of bf16 MFMAs
// on operands loaded once from `ab` (random bf16, so the products toggle
// like real data): two A fragments, and the two B fragments in turn.
// kShape 32: 2 x 4 v_mfma_f32_32x32x16_bf16 (32,768 flop each) into four
// independent accumulators; kShape 16: 2 x 8 v_mfma_f32_16x16x32_bf16
// (16,384 flop each) into eight.  One word per lane goes to the sink so that
// nothing is optimised away.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr double kRoundFlop = 8 * 32768.0;  // flop per wave and round, both shapes

template <int kShape>
__device__ __forceinline__ float mfma_rounds(bf16x8 a0, bf16x8 a1, bf16x8 b0, bf16x8 b1, int iters) {
  float s = 0.0f;
  if constexpr (kShape == 32) {
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((c & 1) ? a1 : a0, b0, acc[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((c & 1) ? a1 : a0, b1, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[c][r];
  } else {
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((c & 1) ? a1 : a0, b0, acc[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((c & 1) ? a1 : a0, b1, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += acc[c][r];
  }
  return s;
}

template <int kWpc, int kShape>
__global__ __launch_bounds__(kThreads) void mfma_loop(const bf16x8* __restrict__ ab, int iters,
                                                     float* __restrict__ sink, uint64_t* __restrict__ clk) {
  __shared__ uint32_t occ[occ_words<kWpc>()];
  const int lane = threadIdx.x & 63;
  const bf16x8 a0 = ab[lane], a1 = ab[64 + lane], b0 = ab[128 + lane], b1 = ab[192 + lane];
  // operands in registers before the clocks start
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const float s = mfma_rounds<kShape>(a0, a1, b0, b1, iters);
  // the sum depends on every accumulator, so the clocks below follow the loop
  sink[size_t(blockIdx.x) * kThreads + threadIdx.x] = __uint_as_float(through_lds(occ, __float_as_uint(s)));
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  // first workgroup, first wave: core cycles and 100 MHz ticks of its loop
  if (clk && blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Streams `bytes` (rounded down to a whole number of workgroup iterations)
// of the device buffer `buf` once, with `wg_per_cu` (1, 2 or 4) workgroups of 256
// threads per compute unit, on `stream`.  `sink` is a device buffer of at
// least mla_probe_sink_bytes(wg_per_cu) bytes.  Returns the bytes streamed,
// or 0 on a bad argument or launch failure.
size_t mla_probe_sink_bytes(int32_t wg_per_cu) {
  int dev = 0, ncu = 0;
  if (wg_per_cu < 1 || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return size_t(ncu) * wg_per_cu * kThreads * 4;
}

size_t mla_probe_stream_read(const void* buf, size_t bytes, int32_t mode, int32_t wg_per_cu,
                             void* sink, void* stream) {
  if (!buf || !sink || !(wg_per_cu == 1 || wg_per_cu == 2 || wg_per_cu == 4) || mode < 0 || mode > 3) return 0;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const size_t grid = size_t(ncu) * wg_per_cu;
  const size_t n_iter = bytes / (grid * kStep);
  if (n_iter == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const uint4* p4 = static_cast<const uint4*>(buf);
  const char* pc = static_cast<const char*>(buf);
  uint32_t* sk = static_cast<uint32_t*>(sink);
  auto launch = [&](auto wpc_c) {
    constexpr int W = decltype(wpc_c)::value;
    switch (mode) {
      case 0: hipLaunchKernelGGL((read_regs<false, W>), dim3(grid), dim3(kThreads), 0, st, p4, n_iter, sk); break;
      case 1: hipLaunchKernelGGL((read_lds<false, W>), dim3(grid), dim3(kThreads), 0, st, pc, n_iter, sk); break;
      case 2: hipLaunchKernelGGL((read_regs<true, W>), dim3(grid), dim3(kThreads), 0, st, p4, n_iter, sk); break;
      default: hipLaunchKernelGGL((read_lds<true, W>), dim3(grid), dim3(kThreads), 0, st, pc, n_iter, sk); break;
    }
  };
  switch (wg_per_cu) {
    case 1: launch(std::integral_constant<int, 1>{}); break;
    case 2: launch(std::integral_constant<int, 2>{}); break;
    default: launch(std::integral_constant<int, 4>{}); break;
  }
  if (hipGetLastError() != hipSuccess) return 0;
  return n_iter * grid * kStep;
}

// Runs the MFMA loop of `shape` (32: 32x32x16, 16: 16x16x32) with
// `wg_per_cu` (1, 2 or 4) workgroups of 256 threads (4 waves)
// per compute unit, `iters` rounds each, on `stream`.  `ab` is a device
// buffer of at least 256 x 16 bytes of bf16 operands; `sink` as for the
// stream probe; `clk`, if not null, a device buffer of two uint64 that gets
// the core-clock cycles and the 100 MHz real-time ticks of the first wave's
// loop.  Returns the flops of the launch, or 0 on a bad argument or launch
// failure.
double mla_probe_mfma(const void* ab, int32_t iters, int32_t wg_per_cu, int32_t shape, void* sink, void* clk,
                      void* stream) {
  if (!ab || !sink || iters < 1 || !(wg_per_cu == 1 || wg_per_cu == 2 || wg_per_cu == 4) ||
      !(shape == 32 || shape == 16))
    return 0.0;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0.0;
  const size_t grid = size_t(ncu) * wg_per_cu;
  auto launch = [&](auto wpc_c, auto shape_c) {
    constexpr int W = decltype(wpc_c)::value, SH = decltype(shape_c)::value;
    hipLaunchKernelGGL((mfma_loop<W, SH>), dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const bf16x8*>(ab), iters, static_cast<float*>(sink),
                       static_cast<uint64_t*>(clk));
  };
  auto by_shape = [&](auto wpc_c) {
    if (shape == 32) launch(wpc_c, std::integral_constant<int, 32>{});
    else launch(wpc_c, std::integral_constant<int, 16>{});
  };
  switch (wg_per_cu) {
    case 1: by_shape(std::integral_constant<int, 1>{}); break;
    case 2: by_shape(std::integral_constant<int, 2>{}); break;
    default: by_shape(std::integral_constant<int, 4>{}); break;
  }
  if (hipGetLastError() != hipSuccess) return 0.0;
  return double(grid) * (kThreads / 64) * double(iters) * kRoundFlop;
}

}  // extern "C"
