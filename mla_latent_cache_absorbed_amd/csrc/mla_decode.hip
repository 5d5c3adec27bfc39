// Absorbed-MLA decode over a paged 576-wide bf16 latent cache, for gfx950.
//
// Two kernels behind the C ABI declared in include/mla_decode.h:
//
//   mla_plan_kernel    one workgroup: reads seq_lens, picks a split-KV chunk
//                      size, writes the list of (request, token range) work
//                      items into the workspace.
//   mla_attend_kernel  the hot loop.  One workgroup per compute unit pulls
//                      work items from a queue.  Each wave owns 32 heads.
//                      Latent rows are streamed HBM -> LDS with direct-to-LDS
//                      loads into a ring of 32-token stages; every staged row
//                      is reused by all heads of the request.  Scores
//                      S^T[token, head] = K * Q^T over all 576 dims and the
//                      weighted sum O^T[col, head] += V^T * P^T over the 512
//                      kv_c dims run on 32x32x16 bf16 MFMA with fp32
//                      accumulation, software-pipelined: the score MFMAs of
//                      stage k+1 are interleaved with the weighted-sum MFMAs
//                      of stage k.  When a request is split over several
//                      items, each writes a normalised fp32 partial and its
//                      log-sum-exp, and the last item of the request to
//                      finish merges them (split-KV log-sum-exp merge).
//
// The operation: each head's absorbed query attends over the shared latent
// directly (page "DP attention + expert parallel: MLA KV replication",
// section "A strong answer"); scores use all 576 dims including the MQA-shared
// k_rope (page "MLA 的 TP 切分…", section 一, and the first of page 1's
// "Common mistakes"); the value is the kv_c half of the same row (page
// "DP 与 DPA 的区别…", section "MLA：KV 是一份共享 latent…").

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <mutex>

#include "../../include/mla_decode.h"

namespace {

// ---------------------------------------------------------------------------
// constants of the layout
// ---------------------------------------------------------------------------
constexpr int kD = 576;                   // latent width (kv_c 512 + k_rope 64)
constexpr int kDV = 512;                  // value width (kv_c)
constexpr int kSub = 32;                  // tokens per LDS stage
constexpr int kRegionB = kSub * 64 * 16;  // byte offset of the k_rope region in a stage
constexpr int kStageBytes = kSub * kD * 2;  // 36,864 B
constexpr int kLoadsPerStage = kSub + 4;  // 1 KB direct-to-LDS loads per stage
constexpr int kMaxExtraItems = 1024;      // work items beyond B the workspace holds
constexpr int kHdrBytes = 256;
constexpr float kRefHeadroom = 64.0f;     // log2 units: P <= 2^64 before an item is redone
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kSc1 = 16;                  // cache-policy bit sc1: agent-scope coherent access
constexpr int kSc0 = 1;                   // cache-policy bit sc0: misses L1
constexpr int kMergeMinItems = 3;         // splits this wide are merged by merge units
// Per-request counters: tickets taken (or merge units done) and partials
// published.  Both are 0 between calls.
constexpr int kCtr = 2;
enum { kTicket = 0, kPublished = 1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

// Heads covered by one workgroup: 32 per wave, waves chosen from H.
__host__ __device__ inline int heads_padded(int H) { return H > 64 ? 128 : H > 32 ? 64 : 32; }

// Workspace sections (byte offsets).
struct WsLayout {
  size_t req_off, ctr_off, big_off, item_off, plse_off, po_off, total;
  int cap;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// cap: work items the layout holds (default B + kMaxExtraItems)
__host__ __device__ inline WsLayout ws_layout(int B, int H, int cap = -1) {
  WsLayout w;
  const int hp = heads_padded(H);
  w.cap = cap < 0 ? B + kMaxExtraItems : cap;
  w.req_off = kHdrBytes;
  w.ctr_off = align256(w.req_off + size_t(B) * 16);
  w.big_off = align256(w.ctr_off + size_t(B) * kCtr * 4);
  w.item_off = align256(w.big_off + size_t(B) * 4);
  w.plse_off = align256(w.item_off + size_t(w.cap) * 16);
  w.po_off = align256(w.plse_off + size_t(w.cap) * hp * 4);
  w.total = align256(w.po_off + size_t(w.cap) * hp * kDV * 4);
  return w;
}

// ---------------------------------------------------------------------------
// LDS stage layout and swizzles
//
// A stage holds 32 latent rows (36,864 B):
//   region A, bytes [0, 32768): kv_c, row-major [token][64 chunks of 16 B];
//             chunk c of token t sits at slot c ^ swzA(t) of row t.
//   region B, bytes [32768, 36864): k_rope, chunk-major [8 chunks][32 tokens];
//             chunk c' of token t at 32768 + 512 c' + 16 t.
// Region A is filled one token row (1 KB, fully coalesced) per load.  Its
// swizzle makes the MFMA operand reads bank-conflict free under both a
// 128-byte and a 256-byte LDS line:
//   QK reads : lanes 0..31 read tokens 0..31 at one chunk (16 B each);
//   PV reads : ds_read_b64_tr_b16, each 16-lane group reads 4 consecutive
//              tokens x 2 consecutive chunks x 2 halves (8 B each).
// Region B is read only by QK: 32 consecutive tokens of one chunk are 512
// contiguous bytes, so it needs no swizzle.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swzA(int t) {
  const int t0 = t & 1, t1 = (t >> 1) & 1, t2 = (t >> 2) & 1, t3 = (t >> 3) & 1;
  return ((t1 ^ t3) << 3) | (t0 << 2) | (t1 << 1) | t2;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  // s_waitcnt vmcnt(N) expcnt(7) lgkmcnt(0), gfx9 encoding.
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// No divergent regions while accumulators are live.  The compiler has been
// seen to place copies of live registers inside a region entered with part
// of the wave masked off, which copies only the active lanes.  So the attend
// kernels never branch on a lane index: a single-lane atomic sets and
// restores the exec mask inside one asm statement (callers run with the whole
// wave active), polls are made by every lane with a uniform exit, and a store
// that only some lanes need is made by all lanes with identical values or
// falls outside its buffer resource.

// Lane 0 adds v to *p (relaxed, agent scope); returns the old value.
__device__ __forceinline__ int lane0_fetch_add(int32_t* p, int v) {
  int old, res;
  uint64_t keep;
  asm volatile(
      "s_mov_b64 %2, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %0, %3, %4, off sc0\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "s_mov_b64 exec, %2\n\t"
      "v_readlane_b32 %1, %0, 0\n\t"
      "s_nop 4"
      : "=&v"(old), "=s"(res), "=&s"(keep)
      : "v"(p), "v"(v)
      : "memory");
  return res;
}
// Lane 0 adds v to *p (relaxed, agent scope), without waiting for it.
__device__ __forceinline__ void lane0_atomic_add(int32_t* p, int v) {
  uint64_t keep;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %1, %2, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(keep)
      : "v"(p), "v"(v)
      : "memory");
}
// Lane 0 ors v into *p (relaxed, agent scope).
__device__ __forceinline__ void lane0_atomic_or(int32_t* p, int v) {
  uint64_t keep;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_or %1, %2, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(keep)
      : "v"(p), "v"(v)
      : "memory");
}
// Every lane of the wave polls *p until it reaches target; the exit is
// uniform.  Bounded: past the bound `flag` is raised in *flags.
__device__ __forceinline__ void wave_poll(int32_t* p, int target, int32_t* flags, int flag) {
  for (int spin = 0;; ++spin) {
    const int v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v >= target) break;
    if (spin >= (1 << 22)) {
      lane0_atomic_or(flags, flag);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// As wave_poll, for a word that a partner sets to a non-zero value; returns
// the value seen (0 if the bound was hit).
__device__ __forceinline__ int wave_poll_value(int32_t* p, int32_t* flags, int flag) {
  for (int spin = 0;; ++spin) {
    const int v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v != 0) return v;
    if (spin >= (1 << 22)) {
      lane0_atomic_or(flags, flag);
      return 0;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The XCD (accelerator complex die) this wave runs on.  Each XCD has its own
// L2; a buffer written through to memory by one wave is read back coherently
// by a wave of the same XCD with a load that only misses L1.
__device__ __forceinline__ int xcd_id() {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
  return x;
}

// MFMAs of the hot loop are written out so that register classes are pinned:
// the 16 output accumulators of a wave (512 values per lane, fp32) fill all
// 256 AGPRs and the score accumulator lives in VGPRs.  Left to itself the
// compiler gives every MFMA builtin of a kernel this size the AGPR form and
// then spills.  The compiler cannot see the hazards of asm it does not parse:
//   * an MFMA reading a register that a VALU instruction wrote needs two wait
//     states.  Operands that come from LDS or global loads never do, so the
//     plain forms carry no nop; pv_mfma_v, for weights just converted by the
//     VALU, does.  isa_check.py scans the compiled code for any VALU write of
//     an MFMA operand closer than that and fails the build;
//   * back-to-back accumulation into the same registers needs none;
//   * the drains provide >= 19 wait states between the last XDL write of an
//     accumulator and any non-MFMA access to it.
__device__ __forceinline__ void qk_mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// the same with two wait states first, for operands just converted by the VALU
__device__ __forceinline__ void qk_mfma_first_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}
__device__ __forceinline__ void pv_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void pv_mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void pv_drain(f32x16 (&o)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
}

struct AttendArgs {
  const __bf16* q;
  const __bf16* cache;
  const int32_t* table;
  __bf16* out;
  float* lse;
  int32_t* hdr;          // workspace header (n_items, chunk, check bits, queue)
  const int4* req;       // per request: first full item, full count, remainder item, count
  int32_t* ctr;          // per request: kCtr counters (0 between calls)
  const int32_t* big;    // requests whose split is merged by merge units
  const int4* items;     // per item: request, first token, end token, request's item count
  float* part_lse;       // [cap, Hp]  log2-domain log-sum-exp of each split item
  float* part_o;         // [cap, Hp * 512] normalised output of each split item, in the
                         // accumulator layout of the waves (see the epilogue)
  float scale_log2;      // scale * log2(e) (times the fp8 cache scale for an fp8 cache)
  float v_scale;         // fp8 cache scale applied to the output (1 for a bf16 cache)
  int32_t B, H, NB, M, lgBS;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const char* cache, int blk,
                                                             uint32_t blk_bytes) {
  // raw buffer over one physical block; accesses past its end read zero
  return __builtin_amdgcn_make_buffer_rsrc((void*)(cache + size_t(blk) * blk_bytes), (short)0,
                                           (int)blk_bytes, 0x00020000);
}

// Direct-to-LDS loads, written out: the LDS address goes in M0 and each lane's
// 16 bytes land at M0 + 16 * lane.  The compiler does not model these as LDS
// writes, so it adds no waits of its own before later LDS reads; the stage
// pipeline waits for them explicitly (vmcnt counts them in issue order), and
// the waits and barriers that order them against LDS reads carry memory
// clobbers.  Nor does the compiler see the asm's scalar operands, so the
// hazards before a vector memory instruction are covered here: five wait
// states, for a buffer resource or M0 just written by a VALU instruction
// (the compiler reloads spilled SGPRs with v_readlane), which also covers the
// one needed after an SALU write of M0.
// Loads of latent stages carry sc1 nt: every cached row is read once per
// launch, so it streams through the caches as non-temporal data at device
// scope (about 1% faster than the default policy on 124 x 4,096 tokens).
__device__ __forceinline__ void dma16_buffer_sc0(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 const char LDS_AS* dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  // sc0: misses L1, may hit the L2 of this XCD
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc0 lds"
               :: "v"(voff), "s"(r), "{m0}"(m0));
}
__device__ __forceinline__ void dma16_buffer(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                             const char LDS_AS* dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  // sc1: agent-scope coherent, for partials another compute unit published
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc1 lds"
               :: "v"(voff), "s"(r), "{m0}"(m0));
}
// The same load for a staged latent row: byte offset soff (uniform) within the
// block, and this lane's 16 bytes at lane16 ^ sw (sw uniform, the row's
// swizzle); the per-lane offset is formed inside the asm so that no per-row
// VGPR is live (and spilled) across the issue sequence.
__device__ __forceinline__ void dma16_row(__amdgpu_buffer_rsrc_t r, uint32_t soff, uint32_t lane16,
                                          uint32_t sw, const char LDS_AS* dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  uint32_t tmp;
  asm volatile("v_xor_b32 %0, %1, %2\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %3, %4 offen sc1 nt lds"
               : "=&v"(tmp)
               : "s"(sw), "v"(lane16), "s"(r), "s"(soff), "{m0}"(m0));
}
__device__ __forceinline__ void dma16_global(const char* src, const char LDS_AS* dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off sc1 nt"
               :: "v"(src), "{m0}"(m0));
}

// Physical blocks of one 32-token stage (wave-uniform).  base is a multiple
// of 32 and BS >= 16, so a stage spans at most two blocks.
struct StageIds {
  int base;        // first token of the stage
  int lb0;         // logical block of the first token
  int blk0, blk1;  // physical blocks of the first and the last token
};

// Reads the block ids of the stage starting at `base` (scalar loads of a
// table that is constant during the kernel).  Ids outside [0, NB) are
// replaced by 0 and flagged.
__device__ __forceinline__ StageIds stage_ids(const AttendArgs& a, int b, int base, int t1,
                                              int& bad) {
  const CONST_AS int32_t* trow = (const CONST_AS int32_t*)(a.table) + size_t(b) * a.M;
  StageIds s;
  s.base = base;
  s.lb0 = base >> a.lgBS;
  const int lb1 = min(base + kSub - 1, t1 - 1) >> a.lgBS;
  s.blk0 = trow[s.lb0];
  s.blk1 = trow[lb1];
  if ((unsigned)s.blk0 >= (unsigned)a.NB) { s.blk0 = 0; bad = 1; }
  if ((unsigned)s.blk1 >= (unsigned)a.NB) { s.blk1 = 0; bad = 1; }
  return s;
}

// Issues load j (of 36/NW) of this wave's share of a stage: rows w, w+NW, ...
// of region A (one 1 KB kv_c row each), then region-B loads (k_rope chunks
// 2jb, 2jb+1 of all 32 tokens).  Tokens past t1 are clamped to t1-1, a row
// of the request that is always valid; the softmax masks them.
template <int NW>
__device__ __forceinline__ void issue_load(const AttendArgs& a, const StageIds& id,
                                           char LDS_AS* sbuf, int t1, int w, uint32_t lane16,
                                           int j) {
  const int lg = a.lgBS;
  const int bs_mask = (1 << lg) - 1;
  const int last = t1 - 1;
  const char* cbase = reinterpret_cast<const char*>(a.cache);
  if (j < kSub / NW) {
    const int i = w + NW * j;  // region-A row, wave-uniform
    const int tok = min(id.base + i, last);
    const uint32_t blk_bytes = uint32_t(kD * 2) << lg;
    const __amdgpu_buffer_rsrc_t r =
        block_rsrc(cbase, ((tok >> lg) == id.lb0) ? id.blk0 : id.blk1, blk_bytes);
    dma16_row(r, uint32_t(tok & bs_mask) * (kD * 2), lane16, uint32_t(swzA(i) * 16), sbuf + i * 1024);
  } else {
    const int jb = w + NW * (j - kSub / NW);  // region-B load: chunks 2jb, 2jb+1
    const int t = (lane16 >> 4) & 31;
    const int cp = 2 * jb + (lane16 >> 9);
    const int tok = min(id.base + t, last);
    const int blk = ((tok >> lg) == id.lb0) ? id.blk0 : id.blk1;
    const size_t row = (size_t(blk) << lg) | size_t(tok & bs_mask);
    dma16_global(cbase + row * (kD * 2) + 1024 + cp * 16, sbuf + kRegionB + jb * 1024);
  }
}

// With blocks of 32 tokens or more a stage (32 tokens from a multiple of 32)
// lies inside one physical block, so one buffer resource and two row offsets
// serve every load of it and each load takes a few instructions.
struct StageOne {
  __amdgpu_buffer_rsrc_t r;  // the stage's physical block
  uint32_t row0;             // byte offset of the stage's first row in the block
  uint32_t rowlast;          // byte offset of its last row before t1: later rows load that one
};
template <int kRowBytes = kD * 2>
__device__ __forceinline__ StageOne stage_one(const AttendArgs& a, int b, int base, int t1, int& bad) {
  const CONST_AS int32_t* trow = (const CONST_AS int32_t*)(a.table) + size_t(b) * a.M;
  int blk = trow[base >> a.lgBS];
  if ((unsigned)blk >= (unsigned)a.NB) { blk = 0; bad = 1; }
  StageOne s;
  s.r = block_rsrc(reinterpret_cast<const char*>(a.cache), blk, uint32_t(kRowBytes) << a.lgBS);
  s.row0 = uint32_t(base & ((1 << a.lgBS) - 1)) * kRowBytes;
  s.rowlast = s.row0 + uint32_t(min(t1 - 1 - base, kSub - 1)) * kRowBytes;
  return s;
}
// Row load with the swizzle given as a constant: lane_sw is this lane's 16
// bytes xor the swizzle of the wave's first row (swzA is linear over bit
// xor, and row w + NW j = w ^ NW j), sw the swizzle of NW j.
__device__ __forceinline__ void dma16_row_c(__amdgpu_buffer_rsrc_t r, uint32_t soff, uint32_t lane_sw,
                                            int sw, const char LDS_AS* dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  uint32_t tmp;
  asm volatile("v_xor_b32 %0, %1, %2\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %3, %4 offen sc1 nt lds"
               : "=&v"(tmp)
               : "i"(sw), "v"(lane_sw), "s"(r), "s"(soff), "{m0}"(m0));
}
__device__ __forceinline__ void dma16_plain(__amdgpu_buffer_rsrc_t r, uint32_t voff, const char LDS_AS* dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc1 nt lds" :: "v"(voff), "s"(r), "{m0}"(m0));
}
// Load j of this wave's share of a one-block stage (as issue_load).
// rb_tok: this lane's region-B token times the row size; rb_cp: 1024 plus
// its 16-byte chunk within a pair.
template <int NW>
__device__ __forceinline__ void issue_one(const StageOne& s, char LDS_AS* sbuf, int w, uint32_t lane_sw,
                                          uint32_t rb_tok, uint32_t rb_cp, int j) {
  if (j < kSub / NW) {
    const int i = w + NW * j;
    dma16_row_c(s.r, min(s.row0 + uint32_t(i) * (kD * 2), s.rowlast), lane_sw, swzA(NW * j) * 16,
                sbuf + i * 1024);
  } else {
    const int jb = w + NW * (j - kSub / NW);  // k_rope chunks 2jb, 2jb+1 of all 32 tokens
    dma16_plain(s.r, min(s.row0 + rb_tok, s.rowlast) + rb_cp + 32 * jb, sbuf + kRegionB + jb * 1024);
  }
}

// ---------------------------------------------------------------------------
// FP8 latent (OCP e4m3, one scale per cache).  A stage holds 32 rows of 576
// bytes, row-major as in memory (with blocks of 32 tokens or more a stage is
// one contiguous 18,432-byte run of its block, with 16-token blocks two runs
// of 9,216 bytes, so its 18 loads of 1 KB are fully coalesced), except that the 16-byte chunk c of token t sits at slot
// c ^ x8(t) of its row.  x8(t) (two bits: bit 2 of t, and bit 3 xor bit 1)
// keeps c within its aligned group of four and spreads both operand reads
// over distinct banks (the row stride is 576 = 9 * 64 bytes):
//   scores : lanes 0..31 read one 16-byte chunk of tokens 0..31 (lanes
//            32..63 the next chunk), each read serving two k-steps;
//   V^T    : ds_read_b64_tr_b8, each 16-lane group reads 8 tokens x 16
//            bytes of one chunk, and each lane gets one column of 8 tokens.
// Both operands are converted to bf16 in registers just before their MFMAs.
// e4m3 values are exact in bf16, so the products are the same as for a bf16
// cache holding the dequantised values divided by the scale; the scale
// multiplies the scores and the output.
// ---------------------------------------------------------------------------
constexpr int kRow8 = kD;               // bytes per fp8 row
constexpr int kStage8 = kSub * kRow8;   // 18,432 B
constexpr int kLoads8 = kStage8 / 1024; // 18 loads of 1 KB per stage

__device__ __forceinline__ int x8(int t) { return ((t >> 2) & 1) | ((((t >> 3) ^ (t >> 1)) & 1) << 1); }

// Load L (< 18) of a one-block fp8 stage: LDS bytes [1024 L, 1024 L + 1024).
// Lane i's 16 bytes land at 1024 L + 16 i = row t, slot; they come from
// chunk slot ^ x8(t) of row t (rows past t1 load the last valid row).
__device__ __forceinline__ void issue_one8(const StageOne& s, char LDS_AS* sbuf, uint32_t lane16,
                                           int L) {
  const uint32_t o = uint32_t(L) * 1024 + lane16;
  const uint32_t t = (o * 29128u) >> 24;  // o / 576, exact for o < 18,432
  const uint32_t slot = (o - t * kRow8) >> 4;
  const uint32_t chunk = slot ^ uint32_t(x8(int(t)));
  dma16_plain(s.r, min(s.row0 + t * kRow8, s.rowlast) + chunk * 16, sbuf + L * 1024);
}

// Load L (< 18) of an fp8 stage over two blocks of 16 tokens (BS = 16).  A
// block holds 16 rows = 9,216 bytes = 9 loads, so loads 0..8 read the first
// block and loads 9..17 the second; rows past t1 read the last valid row,
// which lies in the first block when the request ends there (then loads
// 9..17 read it too).  The block of a load is therefore wave-uniform.
__device__ __forceinline__ void issue_ids8(const AttendArgs& a, const StageIds& id, char LDS_AS* sbuf,
                                           int t1, uint32_t lane16, int L) {
  const int last = t1 - 1;
  const uint32_t o = uint32_t(L) * 1024 + lane16;
  const uint32_t t = (o * 29128u) >> 24;  // o / 576, exact for o < 18,432
  const uint32_t slot = (o - t * kRow8) >> 4;
  const uint32_t chunk = slot ^ uint32_t(x8(int(t)));
  const bool second = L >= 9 && last >= id.base + 16;
  const int tok0 = second ? id.base + 16 : id.base;  // first token of the block read
  const int tok = min(id.base + int(t), last);
  const __amdgpu_buffer_rsrc_t r =
      block_rsrc(reinterpret_cast<const char*>(a.cache), second ? id.blk1 : id.blk0, 16 * kRow8);
  dma16_plain(r, uint32_t(tok - tok0) * kRow8 + chunk * 16, sbuf + L * 1024);
}

// 8 e4m3 values (low byte first) to bf16, exactly: one packed conversion per
// pair of bytes (op_sel picks the high 16 bits of the source), with a unit
// scale.  Written out: the compiler's lowering of the builtin for this
// instruction was seen to return the first value of a pair for both.
__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t v) {
  uint32_t r;
  asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(v));
  return r;
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t v) {
  uint32_t r;
  asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(v));
  return r;
}
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 v) {
  return __builtin_bit_cast(bf16x8, i32x4{(int)fp8x2_lo(v[0]), (int)fp8x2_hi(v[0]),
                                          (int)fp8x2_lo(v[1]), (int)fp8x2_hi(v[1])});
}

template <bool V>
struct BoolC {
  static constexpr bool value = V;
};
template <bool C, class A, class B>
struct Pick {
  using T = A;
};
template <class A, class B>
struct Pick<false, A, B> {
  using T = B;
};

constexpr int kWaveBytesM = 32 * kDV * 2;  // one wave's share of an item's bf16 partial (32 heads)

// kOne: the block size is 32 tokens or more, so every stage lies in one block.
// kF8: the cache is fp8 (e4m3); stages hold fp8 rows, whose operands are
// converted in registers.
template <int NW, int NS, bool kOne, bool kF8 = false>
__global__ __launch_bounds__(NW * 64, 1) void mla_attend_kernel(AttendArgs a) {
  static_assert(NW == 2 || NW == 4, "waves per workgroup");
  static_assert(NS >= 3, "the pipeline reads two stages while one more loads");
  constexpr int kSB = kF8 ? kStage8 : kStageBytes;       // bytes of a ring stage
  constexpr int kRing = NS * kSB;                        // the stage ring
  // loads per wave per stage (fp8: 18 loads over NW waves, the last repeated)
  constexpr int LPW = kF8 ? (kLoads8 + NW - 1) / NW : kLoadsPerStage / NW;
  // score operand reads in flight: bf16 k-steps, or fp8 16-byte reads of
  // two k-steps each (converted just before their MFMAs)
  constexpr int PFK = kF8 ? 2 : 4;
  constexpr int PFV = 2;                    // weighted-sum operand reads in flight
  constexpr int HP = NW * 32;               // heads covered by the workgroup
  constexpr int CPW = 16 / NW;              // 32-column blocks of O per wave
  constexpr int PBUF = NW * 2 * 1024;       // one stage's weights P (bf16)
  // LDS: the stage ring, then two buffers of weights.  Outside the stage loop
  // the first weight buffer holds instead the per-head row sums and
  // log-sum-exps being exchanged, the waves' redo votes and two scalars.
  __shared__ __attribute__((aligned(1024))) char lds_raw[kRing + 2 * PBUF];
  char LDS_AS* lds = (char LDS_AS*)(lds_raw);
  char LDS_AS* const pw = lds + kRing;
  float LDS_AS* const x_l = (float LDS_AS*)pw;          // [HP] row sums
  float LDS_AS* const x_lse = x_l + HP;                 // [HP] log2-domain log-sum-exps
  int LDS_AS* const s_vote = (int LDS_AS*)(x_lse + HP);  // [NW] redo votes
  int LDS_AS* const s_item = s_vote + NW;               // fetched item or merge unit
  int LDS_AS* const s_ticket = s_item + 1;              // ticket of a two-item split
  static_assert((2 * HP + NW + 2) * 4 <= PBUF, "exchange area");

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int hl = lane & 31;
  const int hi = lane >> 5;
  const int head = w * 32 + hl;
  const bool head_ok = head < a.H;
  const float c2 = a.scale_log2;
  const int n_items = __builtin_amdgcn_readfirstlane(((const CONST_AS int32_t*)a.hdr)[0]);
  // lanes l and l^32 hold the same head: exchange through ds_bpermute
  const int xlane = (lane ^ 32) << 2;
  auto pair_max = [&](float x) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_ds_bpermute(xlane, __float_as_int(x))));
  };
  auto pair_sum = [&](float x) {
    return x + __int_as_float(__builtin_amdgcn_ds_bpermute(xlane, __float_as_int(x)));
  };

  // Per-lane LDS offsets of the MFMA operand reads (relative to a stage).
  // QK region A: k-step s = 8q + j reads chunk 2s + hi of token hl at
  // qk_off[j] + 256 q.  QK region B: k-step 32 + jj at qkb + 1024 jj.
  int qk_off[8];
  {
    const int xa = swzA(hl);
#pragma unroll
    for (int j = 0; j < 8; ++j) qk_off[j] = hl * 1024 + ((((2 * j) | hi)) ^ xa) * 16;
  }
  const int qkb = kRegionB + hi * 512 + hl * 16;
  // fp8: read m (k-steps 2m, 2m + 1) takes chunk 2m + hi of token hl, at
  // qk16_off[m & 1] + 64 (m >> 1); k-step 2m + e uses its bytes 8e .. 8e + 7.
  int qk16_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) qk16_off[j] = hl * kRow8 + 16 * (((2 * j) | hi) ^ x8(hl));
  // Weighted sum.  Wave w owns columns 32 CPW w .. 32 CPW (w + 1) - 1 of O
  // for all HP heads: accumulator o[hb CPW + c] is O^T of the 32 columns of
  // block cb = CPW w + c for heads 32 hb .. 32 hb + 31.  So each wave reads
  // only its slab of V, and the weights P of all heads go through LDS.
  // V fragment f (kk = f / CPW, c = f % CPW) is V^T of block cb over the 16
  // tokens of half kk, read transposed: the lane reads token 16 kk + 8 e +
  // 4 hi + r, chunk 4 cb + cc, half u0 (r = lane bits 3:2, cc = 2 bit4 +
  // bit1, u0 = bit0) at pv_off[e][c & 3] + 16384 kk + 256 (c >> 2).
  int pv_off[2][4];
  {
    const int r = (lane >> 2) & 3;
    const int cc = (((lane >> 4) & 1) << 1) | ((lane >> 1) & 1);
    const int u0 = lane & 1;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int T = 8 * e + 4 * hi + r;
      const int sa = swzA(T);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pv_off[e][j] = T * 1024 + (((4 * j) | cc) ^ sa) * 16 + 8 * u0 + 256 * (CPW / 4) * w;
    }
  }
  // fp8 V fragment f (kk, c as above): lane 16 g + i of the transposing
  // read supplies token 16 kk + 4 (g >> 1) + tok(i >> 1) (tok(j) = j % 4 +
  // 8 (j / 4)), bytes 8 (i & 1) .. +7 of chunk 2 cb + (g & 1); the read hands
  // lane l column 32 cb + l % 32 of tokens 16 kk + 4 hi + tok(0..7), the
  // tokens of the P fragment's lane.  Offset pv8_off[c & 1] + 64 (c >> 1) +
  // 16 kk rows.
  int pv8_off[2];
  {
    const int g = lane >> 4, i = lane & 15, j = i >> 1;
    const int T = 4 * (g >> 1) + (j & 3) + 8 * (j >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      pv8_off[e] = T * kRow8 + 16 * (2 * CPW * w + (((2 * e) | (g & 1)) ^ x8(T))) + 8 * (i & 1);
  }
  // P fragment (hb, kk): the B operand of the weighted sum for heads of
  // block hb over token half kk, as wave hb's lanes hold it (head 32 hb +
  // lane % 32, the same 8 tokens per lane as the V fragments); 1 KB
  // contiguous at (2 hb + kk) KB of a weight buffer.
  const int p_lane = lane * 16;

  // Workgroup g takes item g directly; items grid, grid+1, ... come from the
  // queue.  With no more items than workgroups no atomic is needed at all.
  // Otherwise every workgroup makes exactly one failing fetch, and the last
  // fetch of all (it returns n_items - 1) leaves the queue at 0 so that the
  // same plan serves the next call.
  const int grid = int(gridDim.x);
  const int xcd = xcd_id();
  bool first = true;
  for (;;) {
    int it = int(blockIdx.x);
    if (!first) {
      if (n_items <= grid) break;
      if (w == 0) {
        const int f = lane0_fetch_add(&a.hdr[3], 1);
        *s_item = f;
      }
      __syncthreads();
      const int v = __builtin_amdgcn_readfirstlane(*s_item);
      __syncthreads();
      if (v + grid >= n_items) {
        if (w == 0 && v == n_items - 1) __hip_atomic_store(&a.hdr[3], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      it = v + grid;
    }
    first = false;
    if (it >= n_items) continue;

    const i32x4 item = ((const CONST_AS i32x4*)a.items)[it];
    const int b = __builtin_amdgcn_readfirstlane(item[0]);
    const int t0 = __builtin_amdgcn_readfirstlane(item[1]);
    const int t1 = __builtin_amdgcn_readfirstlane(item[2]);
    const int cnt = __builtin_amdgcn_readfirstlane(item[3]);

    if (t1 <= t0) {
      // a request with no cached tokens: out = 0, lse = -inf
      int lane_z = lane;
      asm volatile("" : "+v"(lane_z));
      const int head_z = w * 32 + (lane_z & 31);
      // lanes of heads >= H fall outside both resources
      const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.out + size_t(b) * a.H * kDV), (short)0, a.H * kDV * 2, 0x00020000);
      const __amdgpu_buffer_rsrc_t zl = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.lse + size_t(b) * a.H), (short)0, a.H * 4, 0x00020000);
      const uint32_t zoff = uint32_t(head_z * kDV + 4 * (lane_z >> 5)) * 2;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, zr, zoff + (32 * cb + 8 * g) * 2, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-INFINITY), zl, uint32_t(head_z) * 4, 0, 0);
      continue;
    }
    const int nst = (t1 - t0 + kSub - 1) / kSub;
    int bad = 0;

    f32x16 o[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16{};
    float m_run = -INFINITY;  // exponent reference of this head (log2 units)
    float amax = -INFINITY;   // largest exponent argument (score * c2 - m_run) of this lane
    float la = 0.0f, lb = 0.0f;  // this lane's share of the row sum, in two chains
    bool first_pass = true;   // uniform: false on a redo

    // score operand read ahead: a bf16 k-step, or (fp8) 16 bytes of two
    using KRaw = typename Pick<kF8, i32x4, bf16x8>::T;
    auto kread = [&](const char LDS_AS* sb, int s) -> KRaw {
      if constexpr (kF8) return *(const i32x4 LDS_AS*)(sb + qk16_off[s & 1] + 64 * (s >> 1));
      else
        return s < 32 ? *(const bf16x8 LDS_AS*)(sb + qk_off[s & 7] + 256 * (s >> 3))
                      : *(const bf16x8 LDS_AS*)(sb + qkb + 1024 * (s - 32));
    };
    // fp8 k-step s of the read held in x
    auto kcvt = [&](const i32x4& x, int s) -> bf16x8 {
      return fp8x8_to_bf16(u32x2{(uint32_t)x[2 * (s & 1)], (uint32_t)x[2 * (s & 1) + 1]});
    };
    // weighted-sum operand read ahead: bf16, or (fp8) 8 raw bytes
    using VRaw = typename Pick<kF8, u32x2, bf16x8>::T;
#define MLA_VREAD(sb, f, dst)                                                               \
  do {                                                                                      \
    const int c_ = (f) % CPW, kk_ = (f) / CPW;                                              \
    if constexpr (kF8) {                                                                    \
      dst = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(               \
          (i32x2 LDS_AS*)((sb) + pv8_off[c_ & 1] + 64 * (c_ >> 1) + kk_ * (16 * kRow8))));   \
    } else {                                                                                \
      const int imm_ = kk_ * 16384 + 256 * (c_ >> 2);                                       \
      const bf16x4 lo_ = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(                          \
          (bf16x4 LDS_AS*)((sb) + pv_off[0][c_ & 3] + imm_));                               \
      const bf16x4 hi_ = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(                          \
          (bf16x4 LDS_AS*)((sb) + pv_off[1][c_ & 3] + imm_));                               \
      dst = bf16x8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};         \
    }                                                                                       \
  } while (0)
#define MLA_PREAD(pb, hb, kk) (*(const bf16x8 LDS_AS*)((pb) + ((hb) * 2 + (kk)) * 1024 + p_lane))
#define MLA_PWRITE(pb, kk, val) (*(bf16x8 LDS_AS*)((pb) + (w * 2 + (kk)) * 1024 + p_lane) = (val))

    // ---- stage pipeline ----
    // Each head's exponent reference m_run is fixed from the item's first
    // stage (where O is still zero), so O is never rescaled: P = 2^(s - m_run)
    // may grow up to 2^kRefHeadroom on later stages, which fp32 sums and bf16
    // weights carry exactly in relative terms.  Each lane tracks the largest
    // exponent argument it produced; if one exceeds the headroom (not seen
    // with attention-like data), the whole item is redone with the larger
    // reference.  With the reference fixed, a stage's weights need no
    // cross-lane step, so its softmax runs in the shadow of MFMAs.
    //
    // Iteration k finds P(k) of all heads in weight buffer k % 2.  Phase 1
    // runs the 36 score MFMAs of stage k+1 interleaved with the 16
    // weighted-sum MFMAs of stage k's first token half, and issues this
    // wave's loads of stage k+NS-1 spread between them; phase 2 runs the 16
    // of the second half with the softmax of stage k+1 between them, whose
    // weights go to the other buffer.  Stages k+2 .. k+NS-2 stay in flight.
    // Every iteration issues a full stage (past the item's end, a copy of its
    // last stage into a free slot) so that one wait count serves all
    // iterations.  Only a request's last stage can be partial, so only the
    // last iteration applies the mask.
    //
    // Weighted-sum MFMA n (0..31) of a stage uses V fragment f = n / NW with
    // the P fragment of head block hb = n % NW, into o[hb CPW + f % CPW].
    uint32_t lane16 = uint32_t(lane) * 16;
    uint32_t lane_sw = lane16 ^ uint32_t(swzA(w) * 16);
    uint32_t rb_tok = ((lane16 >> 4) & 31) * (kD * 2);
    uint32_t rb_cp = 1024 + (lane16 >> 9) * 16;
    // keep the per-lane load offsets from being hoisted out of the item loop
    asm volatile("" : "+v"(lane16), "+v"(lane_sw), "+v"(rb_tok), "+v"(rb_cp));
    auto stage_base = [&](int p) { return t0 + min(p, nst - 1) * kSub; };
    using Src = typename Pick<kOne, StageOne, StageIds>::T;
    auto src_of = [&](int base) -> Src {
      if constexpr (kF8 && kOne) return stage_one<kRow8>(a, b, base, t1, bad);
      else if constexpr (kOne) return stage_one(a, b, base, t1, bad);
      else return stage_ids(a, b, base, t1, bad);
    };
    auto issue = [&](const Src& sr, char LDS_AS* sbuf, int j) {
      if constexpr (kF8 && kOne) issue_one8(sr, sbuf, lane16, min(w + NW * j, kLoads8 - 1));
      else if constexpr (kF8) issue_ids8(a, sr, sbuf, t1, lane16, min(w + NW * j, kLoads8 - 1));
      else if constexpr (kOne) issue_one<NW>(sr, sbuf, w, lane_sw, rb_tok, rb_cp, j);
      else issue_load<NW>(a, sr, sbuf, t1, w, lane16, j);
    };
    auto qk_first = [&](f32x16& acc, const bf16x8& x, const bf16x8& y) {
      if constexpr (kF8) qk_mfma_first_v(acc, x, y);
      else qk_mfma_first(acc, x, y);
    };
    auto qk_next = [&](f32x16& acc, const bf16x8& x, const bf16x8& y) {
      if constexpr (kF8) qk_mfma_v(acc, x, y);
      else qk_mfma(acc, x, y);
    };
    for (;;) {
      // Queries of this wave's 32 heads, as the B operand of the QK MFMA:
      // lane holds head hl, dims 16s + 8hi .. +7 for k-step s (fp8: dims
      // 16 (2 (s >> 1) + hi) + 8 (s & 1) .. +7, the order of the 16-byte
      // score reads), reloaded on a redo so that they are not live past the
      // last score MFMA of a pass.
      // Lanes of padding heads load head 0's query (their results are never
      // written); no select follows the loads, so they all go out at once.
      bf16x8 qreg[36];
      {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            a.q + (size_t(b) * a.H + (head_ok ? head : 0)) * kD + (kF8 ? 16 : 8) * hi);
#pragma unroll
        for (int s = 0; s < 36; ++s) qreg[s] = kF8 ? qp[4 * (s >> 1) + (s & 1)] : qp[2 * s];
      }
      // Stage 0 goes out behind the queries, and both are waited for before
      // the next stages go out: the compiler counts only its own (query)
      // loads, so its waits before the score MFMAs would otherwise also wait
      // for later stages.
      {
        const Src id = src_of(stage_base(0));
#pragma unroll
        for (int j = 0; j < LPW; ++j) issue(id, lds, j);
      }
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
#pragma unroll
      for (int p = 1; p < NS - 1; ++p) {
        const Src id = src_of(stage_base(p));
#pragma unroll
        for (int j = 0; j < LPW; ++j) issue(id, lds + p * kSB, j);
      }
      Src nxt = src_of(stage_base(NS - 1));
      // stage 0 scores (a lone chain, once per item)
      block_barrier();
      f32x16 sacc;
      {
        const char LDS_AS* sb = lds;
        KRaw kf[PFK];
#pragma unroll
        for (int s = 0; s < PFK; ++s) kf[s] = kread(sb, s);
#pragma unroll
        for (int s = 0; s < 36; ++s) {
          if constexpr (kF8) {
            const int m = s >> 1;
            const bf16x8 kb = kcvt(kf[m % PFK], s);
            if ((s & 1) && m + PFK < 18) kf[m % PFK] = kread(sb, m + PFK);
            if (s == 0) qk_first(sacc, kb, qreg[0]);
            else qk_next(sacc, kb, qreg[s]);
          } else {
            if (s == 0) qk_first(sacc, kf[0], qreg[0]);
            else qk_next(sacc, kf[s % PFK], qreg[s]);
            if (s + PFK < 36) kf[s % PFK] = kread(sb, s + PFK);
          }
        }
        qk_drain(sacc);
      }
      // register v holds token 4hi + 8(v/4) + (v%4) of its stage: valid
      // while 8(v/4) + (v%4) < (stage end) - 4hi
      VRaw vf[PFV];  // weighted-sum operands, read ahead
      {
        const int lim = t1 - t0 - 4 * hi;
        if (first_pass) {
          // the reference is the head's largest stage-0 score
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mx = fmaxf(mx, (8 * (v >> 2) + (v & 3) < lim) ? sacc[v] * c2 : -INFINITY);
          m_run = pair_max(mx);
        }
        bf16x8 p0, p1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float arg = (8 * (v >> 2) + (v & 3) < lim) ? fmaf(sacc[v], c2, -m_run) : -INFINITY;
          amax = fmaxf(amax, arg);
          const float pv = __builtin_amdgcn_exp2f(arg);
          if (v & 1) lb += pv;
          else la += pv;
          if (v < 8) p0[v] = (__bf16)pv;
          else p1[v - 8] = (__bf16)pv;
        }
        MLA_PWRITE(pw, 0, p0);
        MLA_PWRITE(pw, 1, p1);
#pragma unroll
        for (int s = 0; s < PFV; ++s) MLA_VREAD(lds, s, vf[s]);
      }

      auto iteration = [&](int k, auto mask_tag) {
        constexpr bool kMask = decltype(mask_tag)::value;
        constexpr int kDmaEvery = 36 / LPW;  // score MFMAs per load issued
        // bf16: the first load goes out after the second score MFMA, not
        // beside the first one, whose operand reads just left the barrier
        // (1-2 % faster); with fp8 operands the offset measured slower.
        constexpr int kDmaAt = kF8 ? 0 : 1;
        static_assert(kDmaAt + (LPW - 1) * kDmaEvery < 36, "all loads issued in phase 1");
        const char LDS_AS* sbv = lds + (k % NS) * kSB;
        const char LDS_AS* pcur = pw + (k & 1) * PBUF;
        char LDS_AS* pnxt = pw + ((k + 1) & 1) * PBUF;
        // stage k+1 and every wave's P(k) must be in LDS; stage k+2 may
        // still be loading
        wait_vmcnt_lgkm0<LPW * (NS - 3)>();
        block_barrier();
        const Src cur = nxt;
        char LDS_AS* sdst = lds + ((k + NS - 1) % NS) * kSB;
        nxt = src_of(stage_base(k + NS));
        const char LDS_AS* sbk = lds + ((k + 1) % NS) * kSB;
        // With four waves each issues 9 loads per stage, spread between the
        // score MFMAs; a pair of waves issues its 18 in a burst (spread that
        // thin, every stall of the memory pipeline would land on an MFMA).
        constexpr bool kSpread = NW == 4;
        if (!kSpread)
#pragma unroll
          for (int j = 0; j < LPW; ++j) issue(cur, sdst, j);
        KRaw kf[PFK];
#pragma unroll
        for (int s = 0; s < PFK; ++s) kf[s] = kread(sbk, s);
        bf16x8 pa[NW], pb[NW];  // P(k) fragments of the two token halves
#pragma unroll
        for (int h = 0; h < NW; ++h) pa[h] = MLA_PREAD(pcur, h, 0);
        bf16x8 vcur;  // fp8: the V fragment in use, converted
        auto pv_step = [&](int n) {
          const int f = n / NW, h = n % NW;
          if constexpr (kF8) {
            if (h == 0) {
              vcur = fp8x8_to_bf16(vf[f % PFV]);
              pv_mfma_v(o[h * CPW + f % CPW], vcur, n < 16 ? pa[h] : pb[h]);
            } else {
              pv_mfma(o[h * CPW + f % CPW], vcur, n < 16 ? pa[h] : pb[h]);
            }
          } else {
            pv_mfma(o[h * CPW + f % CPW], vf[f % PFV], n < 16 ? pa[h] : pb[h]);
          }
          if (h == NW - 1 && f + PFV < 2 * CPW) MLA_VREAD(sbv, f + PFV, vf[f % PFV]);
          if (n >= 16 - NW && n < 16) pb[h] = MLA_PREAD(pcur, h, 1);
        };
        // phase 1
#pragma unroll
        for (int s = 0; s < 36; ++s) {
          if constexpr (kF8) {
            const int m = s >> 1;
            const bf16x8 kb = kcvt(kf[m % PFK], s);
            if ((s & 1) && m + PFK < 18) kf[m % PFK] = kread(sbk, m + PFK);
            if (s == 0) qk_first(sacc, kb, qreg[0]);
            else qk_next(sacc, kb, qreg[s]);
          } else {
            if (s == 0) qk_first(sacc, kf[0], qreg[0]);
            else qk_next(sacc, kf[s % PFK], qreg[s]);
            if (s + PFK < 36) kf[s % PFK] = kread(sbk, s + PFK);
          }
          if (kSpread && s >= kDmaAt && (s - kDmaAt) % kDmaEvery == 0 && (s - kDmaAt) / kDmaEvery < LPW)
            issue(cur, sdst, (s - kDmaAt) / kDmaEvery);
          if ((s & 1) && (s >> 1) < 16) pv_step(s >> 1);
        }
        qk_drain(sacc);
        // phase 2
        const int lim = t1 - (t0 + (k + 1) * kSub) - 4 * hi;
        bf16x8 n0, n1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          pv_step(16 + v);
          float arg = fmaf(sacc[v], c2, -m_run);
          if (kMask) arg = (8 * (v >> 2) + (v & 3) < lim) ? arg : -INFINITY;
          amax = fmaxf(amax, arg);
          const float pv = __builtin_amdgcn_exp2f(arg);
          if (v & 1) lb += pv;
          else la += pv;
          if (v < 8) n0[v] = (__bf16)pv;
          else n1[v - 8] = (__bf16)pv;
          if (v == 7) MLA_PWRITE(pnxt, 0, n0);
          if (v == 15) MLA_PWRITE(pnxt, 1, n1);
          __builtin_amdgcn_sched_barrier(0);
        }
        // operands of the next weighted sum (stage k+1, already in LDS)
#pragma unroll
        for (int s = 0; s < PFV; ++s) MLA_VREAD(sbk, s, vf[s]);
      };
      for (int k = 0; k + 2 < nst; ++k) iteration(k, BoolC<false>{});
      if (nst >= 2) iteration(nst - 2, BoolC<true>{});
      {
        // weighted sum of the last stage, once every wave's weights are in
        const char LDS_AS* sbv = lds + ((nst - 1) % NS) * kSB;
        const char LDS_AS* pcur = pw + ((nst - 1) & 1) * PBUF;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        block_barrier();
        bf16x8 pa[NW], pb[NW];
#pragma unroll
        for (int h = 0; h < NW; ++h) pa[h] = MLA_PREAD(pcur, h, 0);
        bf16x8 vcur;  // fp8: the V fragment in use, converted
#pragma unroll
        for (int n = 0; n < 32; ++n) {
          const int f = n / NW, h = n % NW;
          if constexpr (kF8) {
            if (h == 0) {
              vcur = fp8x8_to_bf16(vf[f % PFV]);
              pv_mfma_v(o[h * CPW + f % CPW], vcur, n < 16 ? pa[h] : pb[h]);
            } else {
              pv_mfma(o[h * CPW + f % CPW], vcur, n < 16 ? pa[h] : pb[h]);
            }
          } else {
            pv_mfma(o[h * CPW + f % CPW], vf[f % PFV], n < 16 ? pa[h] : pb[h]);
          }
          if (h == NW - 1 && f + PFV < 2 * CPW) MLA_VREAD(sbv, f + PFV, vf[f % PFV]);
          if (n >= 16 - NW && n < 16) pb[h] = MLA_PREAD(pcur, h, 1);
        }
      }
      // Copies issued past the item's end are drained and all waves are done
      // reading the ring and the weights before either is reused.
      wait_vmcnt_lgkm0<0>();
      block_barrier();
      {
        const bool vote = __ballot(amax > kRefHeadroom) != 0;
        s_vote[w] = vote ? 1 : 0;
      }
      __syncthreads();
      int redo = 0;
#pragma unroll
      for (int h = 0; h < NW; ++h) redo |= s_vote[h];
      if (!__builtin_amdgcn_readfirstlane(redo)) break;
      // One redo at most.  Its reference is each head's largest score of the
      // item, so an excess left after it is fp32 rounding of scores beyond
      // what the softmax resolves (scaled scores past about 2^30 in log2
      // units, where one ulp exceeds the headroom).  Redoing again would
      // not change the reference, so the request is flagged instead (its
      // outputs are unspecified) and the item ends.
      if (!first_pass) {
        if (w == 0) lane0_atomic_or(&a.hdr[2], MLA_CHECK_SCORE_RANGE);
        break;
      }
      // Redo the item from its first stage with the head's largest score as
      // the reference.
      m_run += pair_max(amax);
      first_pass = false;
      amax = -INFINITY;
      la = 0.0f;
      lb = 0.0f;
      pv_drain(o);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16{};
    }
#undef MLA_VREAD
#undef MLA_PREAD
#undef MLA_PWRITE
    pv_drain(o);
    if (__builtin_amdgcn_readfirstlane(bad)) lane0_atomic_or(&a.hdr[2], MLA_CHECK_BLOCK_ID_RANGE);

    // ---- finalize ----
    // Per-lane offsets of the epilogue derive from an opaque copy of the
    // lane index, so that none of them is hoisted out of the item loop and
    // kept live (or spilled) across the stage pipeline.
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int hl_e = lane_e & 31;
    const int hi_e = lane_e >> 5;
    const int head_e = w * 32 + hl_e;
    const float l_tot = pair_sum(la + lb);
    const float lse2 = m_run + log2f(l_tot);  // log2 of sum_t 2^(scaled score)
    // every wave needs the row sums (and a merger the log-sum-exps) of all
    // heads of its slab; lanes l and l + 32 hold the same values
    x_l[head_e] = l_tot;
    x_lse[head_e] = lse2;
    __syncthreads();
    float inv[NW];
#pragma unroll
    for (int h = 0; h < NW; ++h) {
      if constexpr (kF8) inv[h] = a.v_scale / x_l[h * 32 + hl_e];
      else inv[h] = 1.0f / x_l[h * 32 + hl_e];
    }
    // out and lse of request b through buffer resources (32-bit lane
    // offsets); stores past the request's H heads fall outside the resource
    // and are dropped
    const __amdgpu_buffer_rsrc_t out_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.out + size_t(b) * a.H * kDV), (short)0, a.H * kDV * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t lse_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.lse + size_t(b) * a.H), (short)0, a.H * 4, 0x00020000);
    const uint32_t out_off = uint32_t(hl_e * kDV + 4 * hi_e + 32 * CPW * w) * 2;
    // bf16 of columns 32 (CPW w + c) + 8 g + 4 hi .. +3 of head 32 h + hl
    auto store_out4 = [&](int h, int c, int g, const float (&v)[4]) {
      bf16x4 h4;
#pragma unroll
      for (int r = 0; r < 4; ++r) h4[r] = (__bf16)v[r];
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h4), out_r,
                                            out_off + (h * 32 * kDV + 32 * c + 8 * g) * 2, 0, 0);
    };
    if (cnt == 1) {
#pragma unroll
      for (int h = 0; h < NW; ++h)
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = o[h * CPW + c][4 * g + r] * inv[h];
            store_out4(h, c, g, v);
          }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2 * kLn2), lse_r, head_e * 4, 0, 0);
      continue;
    }

    // Split request.  An item's partial is HP x 512 normalised values in
    // bf16, in 1 KB block pairs, inside a slot of HP x 512 fp32: block
    // (h, cb, g) stands for columns 32 cb + 8 g + 4 (l / 32) .. +3 of head
    // 32 h + l % 32 in lane l (the accumulator layout), and block pair
    // (h, cb, p) at byte (32 h + 2 cb + p) KB holds, in lane l's 16 bytes,
    // that lane's values of blocks (h, cb, 2p) and (h, cb, 2p + 1), so that
    // each store instruction writes 1 KB contiguous and a merging wave reads
    // back the same lanes' values.  (bf16 rounding of a normalised partial,
    // 2^-9 relative, is below the output's own bf16 rounding.)
    // Partials are written and read with sc1 accesses, which are coherent at
    // agent scope (the form that relaxed agent-scope atomics take), so items
    // on different XCDs exchange them without writing back or invalidating
    // whole L2 caches; an item counts itself published only after its
    // stores have completed.  A request split in two is merged by its last
    // item; wider splits by merge units once the item queue is empty.
    auto part_rsrc = [&](int slot) {
      return __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.part_o + size_t(slot) * HP * kDV), (short)0, HP * kDV * 2, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t plse_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.part_lse, (short)0, 0x7ffffff0, 0x00020000);
    // this lane's 16 bytes of block pair (h, CPW w + c, pp): slabp + (32 h +
    // 2 c + pp) KB; pad[h] moves the lanes of padding heads past the
    // resource, so their stores and loads are dropped without a branch
    const uint32_t slabp = uint32_t(2 * CPW * w) * 1024 + uint32_t(lane_e) * 16;
    uint32_t pad[NW];
#pragma unroll
    for (int h = 0; h < NW; ++h) pad[h] = (h * 32 + hl_e < a.H) ? 0u : 0x40000000u;
    auto publish = [&]() {
      const __amdgpu_buffer_rsrc_t pr = part_rsrc(it);
#pragma unroll
      for (int h = 0; h < NW; ++h)
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            bf16x8 v8;
#pragma unroll
            for (int r = 0; r < 8; ++r) v8[r] = (__bf16)(o[h * CPW + c][8 * pp + r] * inv[h]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v8), pr,
                                                   slabp + pad[h] + (32 * h + 2 * c + pp) * 1024, 0, kSc1);
          }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2), plse_r, uint32_t(it * HP + head_e) * 4, 0, kSc1);
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): this lane's partial is out
      __syncthreads();
      if (w == 0) lane0_fetch_add(&a.ctr[kCtr * b + kPublished], 1);
    };
    if (cnt >= kMergeMinItems) {
      publish();
      continue;
    }
    // Two items: a symmetric half merge.  Item s of the request (s = 0 for
    // the item over the first tokens) merges head blocks [s NW/2, (s+1)
    // NW/2) and publishes the other half for its partner, so each item
    // stores and loads half a partial and both halves of the output are
    // written at once; no item waits for a ticket.  The half goes out in
    // bf16 (its own term stays fp32).  The request's two
    // counters become one publish word per item: 0 until the item's half is
    // out, then 1 + the XCD it ran on.  Halves are written through to memory
    // (sc1), so every reader sees them; a reader on the publisher's XCD
    // loads them with L1-missing loads that the shared L2 can serve, any
    // other reader with agent-scope loads.  Each item clears its partner's
    // word once it has read the half, which leaves both at zero for the next
    // call.
    auto half_merge = [&](auto me_c) {
      constexpr int me = decltype(me_c)::value;
      constexpr int kHalf = NW / 2;              // head blocks per half
      constexpr int mine0 = me * kHalf;          // first head block this item merges
      constexpr int theirs0 = (1 - me) * kHalf;  // first head block it publishes
      const i32x4 rq = ((const CONST_AS i32x4*)a.req)[b];
      const int other = me ? ((0 < rq[1]) ? rq[0] : rq[2]) : ((1 < rq[1]) ? rq[0] + 1 : rq[2]);
      {
        // the half goes out in bf16: 1 KB block pair (h, cb, p) holds, in
        // lane l's 16 bytes, the values of blocks (h, cb, 2p) and (h, cb,
        // 2p + 1) of that lane (the fp32 layout above, two blocks a lane)
        const __amdgpu_buffer_rsrc_t pr = part_rsrc(it);
#pragma unroll
        for (int hh = 0; hh < kHalf; ++hh)
#pragma unroll
          for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int h = theirs0 + hh;
              bf16x8 v8;
#pragma unroll
              for (int r = 0; r < 8; ++r) v8[r] = (__bf16)(o[h * CPW + c][8 * pp + r] * inv[h]);
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v8), pr,
                                                     slabp + pad[h] + (32 * h + 2 * c + pp) * 1024, 0, kSc1);
            }
        // every lane stores its head's log-sum-exp (the partner reads those of its half)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2), plse_r, uint32_t(it * HP + head_e) * 4, 0, kSc1);
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): this lane's half is out
        __syncthreads();
        if (w == 0)
          __hip_atomic_store(&a.ctr[kCtr * b + me], 1 + xcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // The partner is running (both items of a request are taken before
      // either can finish), so the wait ends; it is bounded all the same.
      if (w == 0) *s_item = wave_poll_value(&a.ctr[kCtr * b + (1 - me)], &a.hdr[2], MLA_CHECK_MERGE_WAIT);
      __syncthreads();
      const bool near = __builtin_amdgcn_readfirstlane(*s_item) == 1 + xcd;
      // log-sum-exp merge (log2 domain): lse = log2 sum_s 2^lse_s,
      // out = sum_s 2^(lse_s - lse) o_s, with o_s the normalised partials,
      // summed in item order; this item's own term is the value it would
      // have published, so the result does not depend on which item merges
      // which half.  The partner's blocks of this wave's slab for this
      // item's half come in through the wave's part of the (free) LDS ring.
      constexpr int kWB8 = kRing / NW / 1024 * 1024;
      constexpr int kWaveBuf = (kF8 && kWB8 < kStageBytes) ? kWB8 : kStageBytes;
      static_assert(NW * kWaveBuf <= kRing, "merge staging fits the ring");
      constexpr int kBlocks = kHalf * CPW * 2;   // 1 KB block pairs per wave
      static_assert(kBlocks * 1024 <= kWaveBuf, "one round of loads");
      char LDS_AS* mb = lds + w * kWaveBuf;
      const __amdgpu_buffer_rsrc_t pr = part_rsrc(other);
      asm volatile("" ::: "memory");
      float lo[kHalf];
      if (near) {
#pragma unroll
        for (int j = 0; j < kBlocks; ++j) {
          const int hh = j / (2 * CPW), c = (j / 2) % CPW, pp = j % 2;
          const int h = mine0 + hh;
          dma16_buffer_sc0(pr, slabp + pad[h] + uint32_t(32 * h + 2 * c + pp) * 1024, mb + j * 1024);
        }
#pragma unroll
        for (int hh = 0; hh < kHalf; ++hh)
          lo[hh] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              plse_r, uint32_t(other * HP + (mine0 + hh) * 32 + hl_e) * 4, 0, kSc0));
      } else {
#pragma unroll
        for (int j = 0; j < kBlocks; ++j) {
          const int hh = j / (2 * CPW), c = (j / 2) % CPW, pp = j % 2;
          const int h = mine0 + hh;
          dma16_buffer(pr, slabp + pad[h] + uint32_t(32 * h + 2 * c + pp) * 1024, mb + j * 1024);
        }
#pragma unroll
        for (int hh = 0; hh < kHalf; ++hh)
          lo[hh] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              plse_r, uint32_t(other * HP + (mine0 + hh) * 32 + hl_e) * 4, 0, kSc1));
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // every wave has read its part of the partner's half: clear the
      // partner's word for the next call
      __syncthreads();
      if (w == 0)
        __hip_atomic_store(&a.ctr[kCtr * b + (1 - me)], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float wa[kHalf], wb[kHalf];  // weights of the first and the second item
      float lse_out = 0.0f;
      bool lse_mine = false;       // this wave's head block lies in this item's half
#pragma unroll
      for (int hh = 0; hh < kHalf; ++hh) {
        const int h = mine0 + hh;
        const float lown = x_lse[h * 32 + hl_e];
        const float l0 = me ? lo[hh] : lown, l1 = me ? lown : lo[hh];
        const float mlse = fmaxf(l0, l1);
        const float e0 = __builtin_amdgcn_exp2f(l0 - mlse), e1 = __builtin_amdgcn_exp2f(l1 - mlse);
        const float lam = e0 + e1;
        const float rl = 1.0f / lam;
        wa[hh] = e0 * rl;
        wb[hh] = e1 * rl;
        if (h == w) {
          lse_out = (mlse + log2f(lam)) * kLn2;
          lse_mine = true;
        }
      }
      constexpr int kGroup = 8;
      static_assert(kBlocks % kGroup == 0, "groups of block pairs");
#pragma unroll
      for (int jg = 0; jg < kBlocks; jg += kGroup) {
        bf16x8 xs[kGroup];
#pragma unroll
        for (int jj = 0; jj < kGroup; ++jj) xs[jj] = *(const bf16x8 LDS_AS*)(mb + (jg + jj) * 1024 + lane_e * 16);
#pragma unroll
        for (int jj = 0; jj < kGroup; ++jj) {
          const int j = jg + jj;
          const int hh = j / (2 * CPW), c = (j / 2) % CPW, pp = j % 2;
          const int h = mine0 + hh;
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            const int g = 2 * pp + gi;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float own = o[h * CPW + c][4 * g + r] * inv[h];
              const float oth = (float)xs[jj][4 * gi + r];
              v[r] = me ? fmaf(wb[hh], own, wa[hh] * oth) : fmaf(wb[hh], oth, wa[hh] * own);
            }
            store_out4(h, c, g, v);
          }
        }
      }
      // the lse of this wave's head block, if that block is in this item's
      // half (stores of the other waves fall outside the resource)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse_out), lse_r,
                                            lse_mine ? uint32_t(head_e) * 4 : 0x40000000u, 0, 0);
    };
    {
      const i32x4 rq = ((const CONST_AS i32x4*)a.req)[b];
      const int s0 = (0 < rq[1]) ? rq[0] : rq[2];
      if (s0 == it) half_merge(BoolC<false>{});
      else half_merge(BoolC<true>{});
    }
    __syncthreads();
  }

  // ---- merge units ----
  // Requests split into kMergeMinItems or more items are merged after the
  // item queue is empty, by every workgroup: a request has 4 NW units, unit
  // u covering the 512 / (4 NW) columns starting at kCb * 32 * (u % (4 NW))
  // of request big[u / (4 NW)], for all heads (one 32-head block per wave).
  // Every item of those requests has been taken from the queue, so each is
  // running or done and the wait for their partials ends; it is bounded all
  // the same.  Terms are summed in item order from the published values, so
  // the result does not depend on which workgroup merges or when.
  constexpr int kUnits = 4 * NW;      // units per request
  constexpr int kCb = 16 / kUnits;    // 32-column blocks per unit
  const int n_units = __builtin_amdgcn_readfirstlane(((const CONST_AS int32_t*)a.hdr)[5]);
  for (;;) {
    if (n_units == 0) break;
    if (w == 0) {
      const int f = lane0_fetch_add(&a.hdr[6], 1);
      *s_item = f;
    }
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(*s_item);
    __syncthreads();
    if (u >= n_units) {
      if (w == 0 && u == n_units + int(gridDim.x) - 1)
        __hip_atomic_store(&a.hdr[6], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    const int b = __builtin_amdgcn_readfirstlane(((const CONST_AS int32_t*)a.big)[u / kUnits]);
    const int cb0 = (u % kUnits) * kCb;
    const i32x4 rq = ((const CONST_AS i32x4*)a.req)[b];
    const int cnt = __builtin_amdgcn_readfirstlane(rq[3]);
    if (w == 0) {
      wave_poll(&a.ctr[kCtr * b + kPublished], cnt, &a.hdr[2], MLA_CHECK_MERGE_WAIT);
    }
    __syncthreads();
    int lane_m = lane;
    asm volatile("" : "+v"(lane_m));
    const int head_m = w * 32 + (lane_m & 31);
    const int hi_m = lane_m >> 5;
    // lanes of padding heads read past the resource (zeros, no traffic)
    const uint32_t moff = (head_m < a.H ? uint32_t(lane_m) * 16 : 0x40000000u) + uint32_t(cb0) * 2048;
    auto slot_of = [&](int s) { return (s < rq[1]) ? rq[0] + s : rq[2]; };
    const __amdgpu_buffer_rsrc_t plse_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.part_lse, (short)0, 0x7ffffff0, 0x00020000);
    auto lse_of = [&](int slot) {
      return __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(plse_r, uint32_t(slot * HP + head_m) * 4, 0, kSc1));
    };
    // per-item log-sum-exps of this lane's head, then the weights, staged in
    // the LDS ring (free now) for up to kSlots items
    constexpr int kSlots = kRing / (NW * 32 * 4);
    float LDS_AS* wsl = (float LDS_AS*)(lds) + w * 32 * kSlots + (lane_m & 31);
    const bool in_lds = cnt <= kSlots;
    // items' log-sum-exps in batches of 16, every load of a batch in flight
    float mlse = -INFINITY;
    for (int s0 = 0; s0 < cnt; s0 += 16) {
      float lv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) lv[j] = (s0 + j < cnt) ? lse_of(slot_of(s0 + j)) : -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        mlse = fmaxf(mlse, lv[j]);
        if (in_lds && s0 + j < cnt) wsl[32 * (s0 + j)] = lv[j];
      }
    }
    float lam = 0.0f;
    for (int s = 0; s < cnt; ++s) {
      const float e = __builtin_amdgcn_exp2f((in_lds ? wsl[32 * s] : lse_of(slot_of(s))) - mlse);
      lam += e;
      if (in_lds) wsl[32 * s] = e;
    }
    const float inv = 1.0f / lam;
    auto weight = [&](int s) {
      return (in_lds ? wsl[32 * s] : __builtin_amdgcn_exp2f(lse_of(slot_of(s)) - mlse)) * inv;
    };
    // 2 kCb KB of each item per wave (block pairs 2 c + pp of head block w,
    // at 32 w KB of the item's slot), 32 loads in flight at a time
    constexpr int kNB = 4 * kCb;           // fp32 accumulator blocks
    constexpr int kNP = 2 * kCb;           // 1 KB block pairs per item
    constexpr int kBatch = 32 / kNP;       // items per batch of loads
    f32x4 acc[kNB] = {};
    for (int s0 = 0; s0 < cnt; s0 += kBatch) {
      i32x4 x[kBatch][kNP];
      float wt[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (s0 + j < cnt) {
          const int slot = slot_of(s0 + j);
          const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(reinterpret_cast<char*>(a.part_o + size_t(slot) * HP * kDV) + w * kWaveBytesM), (short)0,
              kWaveBytesM, 0x00020000);
#pragma unroll
          for (int pq = 0; pq < kNP; ++pq)
            x[j][pq] = __builtin_amdgcn_raw_buffer_load_b128(pr, moff + pq * 1024, 0, kSc1);
          wt[j] = weight(s0 + j);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (s0 + j < cnt)
#pragma unroll
          for (int pq = 0; pq < kNP; ++pq) {
            const bf16x8 v8 = __builtin_bit_cast(bf16x8, x[j][pq]);
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[2 * pq + k][r] = fmaf(wt[j], (float)v8[4 * k + r], acc[2 * pq + k][r]);
          }
    }
    {
      // stores of heads >= H fall outside the resources
      const __amdgpu_buffer_rsrc_t out_r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.out + size_t(b) * a.H * kDV), (short)0, a.H * kDV * 2, 0x00020000);
      // block g = 4 c + gg holds columns 32 (cb0 + c) + 8 gg + 4 hi .. +3
      const uint32_t ooff = uint32_t(head_m * kDV + 4 * hi_m + 32 * cb0) * 2;
#pragma unroll
      for (int g = 0; g < kNB; ++g) {
        bf16x4 h4;
#pragma unroll
        for (int r = 0; r < 4; ++r) h4[r] = (__bf16)acc[g][r];
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h4), out_r,
                                              ooff + (32 * (g >> 2) + 8 * (g & 3)) * 2, 0, 0);
      }
      if (cb0 == 0) {
        const __amdgpu_buffer_rsrc_t lse_r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.lse + size_t(b) * a.H), (short)0, a.H * 4, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((mlse + log2f(lam)) * kLn2), lse_r,
                                              head_m * 4, 0, 0);
      }
    }
    // the request's last unit leaves its counters ready for the next call
    __syncthreads();
    if (w == 0) {
      const int t = lane0_fetch_add(&a.ctr[kCtr * b + kTicket], 1);
      if (t == kUnits - 1) {
        __hip_atomic_store(&a.ctr[kCtr * b + kTicket], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.ctr[kCtr * b + kPublished], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// attend, narrow variant (H <= 32): independent wave workers
//
// With at most 32 heads each cached token carries at most 32 heads' worth of
// MFMA work for its 1,152 bytes, far below the MFMA ridge: this shape is
// bound by HBM.  So every wave of a workgroup is an independent worker with
// its own 36 KB LDS slot: it takes items from the queue itself, loads a
// stage, runs the 36 score MFMAs, the softmax and the 32 weighted-sum MFMAs,
// and only then loads its next stage into the same slot.  The four waves of
// a compute unit overlap one another's load latency (up to four stages in
// flight per compute unit) and none ever waits for another.  Splits are
// merged as in the wide kernel, by wave: a request split in two by its last
// item, wider splits by merge units of 128 columns.
//
// kF8: the cache is fp8 (e4m3).  A stage is
// then 18 KB, so a wave's slot holds two: while the wave computes stage st
// from one half, stage st + 1 loads into the other, and the wave waits only
// for loads issued a whole stage earlier.  Operands are read and converted
// as in the wide kernel's fp8 path.
// ---------------------------------------------------------------------------
constexpr int kNarrowWaves = 4;
constexpr int kNarrowUnits = 4;  // merge units per widely split request

template <bool kOne, bool kF8 = false>  // kOne as for the wide kernel: every stage lies in one block
__global__ __launch_bounds__(kNarrowWaves * 64, 1) void mla_attend_narrow_kernel(AttendArgs a) {
  static_assert(2 * kStage8 <= kStageBytes, "two fp8 stages fit a slot");
  __shared__ __attribute__((aligned(1024))) char lds_raw[kNarrowWaves * kStageBytes];
  constexpr int PFK = 4;  // score operand reads in flight
  constexpr int PFV = 2;  // weighted-sum operand reads in flight
  constexpr int HP = 32;  // heads of a partial
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char LDS_AS* slot = (char LDS_AS*)(lds_raw) + w * kStageBytes;
  const int hl = lane & 31;
  const int hi = lane >> 5;
  const bool head_ok = hl < a.H;
  const float c2 = a.scale_log2;
  const int n_items = __builtin_amdgcn_readfirstlane(((const CONST_AS int32_t*)a.hdr)[0]);
  const int n_units = __builtin_amdgcn_readfirstlane(((const CONST_AS int32_t*)a.hdr)[5]);
  const int n_workers = int(gridDim.x) * kNarrowWaves;
  const int xlane = (lane ^ 32) << 2;
  auto pair_max = [&](float x) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_ds_bpermute(xlane, __float_as_int(x))));
  };
  auto pair_sum = [&](float x) {
    return x + __int_as_float(__builtin_amdgcn_ds_bpermute(xlane, __float_as_int(x)));
  };
  // one atomic per wave (lane 0), the old value in every lane
  auto wave_fetch_add = [&](int32_t* p) { return lane0_fetch_add(p, 1); };
  // the wave polls a counter until it reaches `target` (bounded)
  auto wave_wait = [&](int32_t* p, int target) { wave_poll(p, target, &a.hdr[2], MLA_CHECK_MERGE_WAIT); };

  // operand read offsets, as in the wide kernel
  int qk_off[8];
  {
    const int xa = swzA(hl);
#pragma unroll
    for (int j = 0; j < 8; ++j) qk_off[j] = hl * 1024 + ((((2 * j) | hi)) ^ xa) * 16;
  }
  const int qkb = kRegionB + hi * 512 + hl * 16;
  int pv_off[2][4];
  {
    const int r = (lane >> 2) & 3;
    const int cc = (((lane >> 4) & 1) << 1) | ((lane >> 1) & 1);
    const int u0 = lane & 1;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int T = 8 * e + 4 * hi + r;
      const int sa = swzA(T);
#pragma unroll
      for (int j = 0; j < 4; ++j) pv_off[e][j] = T * 1024 + (((4 * j) | cc) ^ sa) * 16 + 8 * u0;
    }
  }
  // fp8 offsets, as in the wide kernel's fp8 path with one wave owning all
  // 16 column blocks: score read m at qk16_off[m & 1] + 64 (m >> 1); V
  // fragment (cb, kk) at pv8_off[cb & 1] + 64 (cb >> 1) + 16 kk rows
  int qk16_off[2], pv8_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) qk16_off[j] = hl * kRow8 + 16 * (((2 * j) | hi) ^ x8(hl));
  {
    const int g = lane >> 4, i = lane & 15, j = i >> 1;
    const int T = 4 * (g >> 1) + (j & 3) + 8 * (j >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e) pv8_off[e] = T * kRow8 + 16 * (((2 * e) | (g & 1)) ^ x8(T)) + 8 * (i & 1);
  }
#define MLA_KREAD(sb, s)                                                               \
  ((s) < 32 ? *(const bf16x8 LDS_AS*)((sb) + qk_off[(s) & 7] + 256 * ((s) >> 3))      \
            : *(const bf16x8 LDS_AS*)((sb) + qkb + 1024 * ((s) - 32)))
#define MLA_KREAD16(sb, m) (*(const i32x4 LDS_AS*)((sb) + qk16_off[(m) & 1] + 64 * ((m) >> 1)))
#define MLA_VREAD(sb, n, dst)                                                               \
  do {                                                                                      \
    const int cb_ = (n) & 15, kk_ = (n) >> 4;                                               \
    if constexpr (kF8) {                                                                    \
      dst = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(               \
          (i32x2 LDS_AS*)((sb) + pv8_off[cb_ & 1] + 64 * (cb_ >> 1) + kk_ * (16 * kRow8)))); \
    } else {                                                                                \
      const int imm_ = kk_ * 16384 + 256 * (cb_ >> 2);                                      \
      const bf16x4 lo_ = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(                          \
          (bf16x4 LDS_AS*)((sb) + pv_off[0][cb_ & 3] + imm_));                              \
      const bf16x4 hi_ = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(                          \
          (bf16x4 LDS_AS*)((sb) + pv_off[1][cb_ & 3] + imm_));                              \
      dst = bf16x8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};         \
    }                                                                                       \
  } while (0)

  // worker k takes item k directly, later items from the queue (as in the
  // wide kernel, by wave)
  const int worker = int(blockIdx.x) * kNarrowWaves + w;
  bool first = true;
  for (;;) {
    int it = worker;
    if (!first) {
      if (n_items <= n_workers) break;
      const int v = wave_fetch_add(&a.hdr[3]);
      if (v + n_workers >= n_items) {
        if (v == n_items - 1) __hip_atomic_store(&a.hdr[3], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      it = v + n_workers;
    }
    first = false;
    if (it >= n_items) continue;
    const i32x4 item = ((const CONST_AS i32x4*)a.items)[it];
    const int b = __builtin_amdgcn_readfirstlane(item[0]);
    const int t0 = __builtin_amdgcn_readfirstlane(item[1]);
    const int t1 = __builtin_amdgcn_readfirstlane(item[2]);
    const int cnt = __builtin_amdgcn_readfirstlane(item[3]);
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int hl_e = lane_e & 31;
    const int hi_e = lane_e >> 5;
    const __amdgpu_buffer_rsrc_t out_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.out + size_t(b) * a.H * kDV), (short)0, a.H * kDV * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t lse_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.lse + size_t(b) * a.H), (short)0, a.H * 4, 0x00020000);
    const uint32_t out_off = uint32_t(hl_e * kDV + 4 * hi_e) * 2;
    auto store_out4 = [&](int cb, int g, const float (&v)[4]) {
      bf16x4 h4;
#pragma unroll
      for (int r = 0; r < 4; ++r) h4[r] = (__bf16)v[r];
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h4), out_r,
                                            out_off + (32 * cb + 8 * g) * 2, 0, 0);
    };
    if (t1 <= t0) {
      // a request with no cached tokens: out = 0, lse = -inf (stores of
      // heads >= H fall outside the resources)
      const float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) store_out4(cb, g, z);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-INFINITY), lse_r, hl_e * 4, 0, 0);
      continue;
    }
    const int nst = (t1 - t0 + kSub - 1) / kSub;
    int bad = 0;
    f32x16 o[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16{};
    float m_run = -INFINITY, amax = -INFINITY, la = 0.0f, lb = 0.0f;
    bool first_pass = true;  // uniform: false on a redo
    uint32_t lane16 = uint32_t(lane) * 16;
    uint32_t rb_tok = ((lane16 >> 4) & 31) * (kD * 2);
    uint32_t rb_cp = 1024 + (lane16 >> 9) * 16;
    asm volatile("" : "+v"(lane16), "+v"(rb_tok), "+v"(rb_cp));
    for (;;) {
      // fixed exponent reference from the item's first stage, with a redo if
      // a later score exceeds it by more than the headroom (as in the wide
      // kernel)
      bf16x8 qreg[36];
      {
        // padding heads load head 0's query (never written out); no select
        // follows the loads, so they all go out at once
        // (fp8: in the order of the 16-byte score reads, as in the wide kernel)
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            a.q + (size_t(b) * a.H + (head_ok ? hl : 0)) * kD + (kF8 ? 16 : 8) * hi);
#pragma unroll
        for (int s = 0; s < 36; ++s) qreg[s] = kF8 ? qp[4 * (s >> 1) + (s & 1)] : qp[2 * s];
      }
      // an fp8 stage into the slot half at dst (this wave's 18 loads)
      auto issue8 = [&](int base, char LDS_AS* dst) {
        if constexpr (kOne) {
          const StageOne id = stage_one<kRow8>(a, b, base, t1, bad);
#pragma unroll
          for (int L = 0; L < kLoads8; ++L) issue_one8(id, dst, lane16, L);
        } else {
          const StageIds id = stage_ids(a, b, base, t1, bad);
#pragma unroll
          for (int L = 0; L < kLoads8; ++L) issue_ids8(a, id, dst, t1, lane16, L);
        }
      };
      // stage 0 into the first half (the query loads are older, so the
      // first stage wait covers them too)
      if constexpr (kF8) issue8(t0, slot);
      for (int st = 0; st < nst; ++st) {
        const char LDS_AS* cur = kF8 ? slot + (st & 1) * kStage8 : slot;
        // this wave's reads of the slot are done before it is refilled
        if constexpr (kF8) {
          if (st + 1 < nst) {
            // the other half held stage st - 1, whose reads are done
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue8(t0 + (st + 1) * kSub, slot + ((st + 1) & 1) * kStage8);
            asm volatile("s_waitcnt vmcnt(18)" ::: "memory");  // stage st is in
          } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          }
        } else if constexpr (kOne) {
          const StageOne id = stage_one(a, b, t0 + st * kSub, t1, bad);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int j = 0; j < 36; ++j) issue_one<1>(id, slot, 0, lane16, rb_tok, rb_cp, j);
        } else {
          const StageIds id = stage_ids(a, b, t0 + st * kSub, t1, bad);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int j = 0; j < 36; ++j) issue_load<1>(a, id, slot, t1, 0, lane16, j);
        }
        if constexpr (!kF8) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        f32x16 sacc;
        if constexpr (kF8) {
          // 16-byte reads of two k-steps each, two reads ahead
          i32x4 kq[2];
          kq[0] = MLA_KREAD16(cur, 0);
          kq[1] = MLA_KREAD16(cur, 1);
#pragma unroll
          for (int s = 0; s < 36; ++s) {
            const int m = s >> 1;
            const bf16x8 kb = fp8x8_to_bf16(u32x2{(uint32_t)kq[m & 1][2 * (s & 1)], (uint32_t)kq[m & 1][2 * (s & 1) + 1]});
            if ((s & 1) && m + 2 < 18) kq[m & 1] = MLA_KREAD16(cur, m + 2);
            if (s == 0) qk_mfma_first_v(sacc, kb, qreg[0]);
            else qk_mfma_v(sacc, kb, qreg[s]);
          }
          qk_drain(sacc);
        } else {
          bf16x8 kf[PFK];
#pragma unroll
          for (int s = 0; s < PFK; ++s) kf[s] = MLA_KREAD(slot, s);
#pragma unroll
          for (int s = 0; s < 36; ++s) {
            if (s == 0) qk_mfma_first(sacc, kf[0], qreg[0]);
            else qk_mfma(sacc, kf[s % PFK], qreg[s]);
            if (s + PFK < 36) kf[s % PFK] = MLA_KREAD(slot, s + PFK);
          }
          qk_drain(sacc);
        }
        bf16x8 p0, p1;
        {
          // register v holds token 4hi + 8(v/4) + (v%4) of the stage
          const int lim = t1 - (t0 + st * kSub) - 4 * hi;
          if (first_pass && st == 0) {
            float mx = -INFINITY;
#pragma unroll
            for (int v = 0; v < 16; ++v)
              mx = fmaxf(mx, (8 * (v >> 2) + (v & 3) < lim) ? sacc[v] * c2 : -INFINITY);
            m_run = pair_max(mx);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float arg = (8 * (v >> 2) + (v & 3) < lim) ? fmaf(sacc[v], c2, -m_run) : -INFINITY;
            amax = fmaxf(amax, arg);
            const float pv = __builtin_amdgcn_exp2f(arg);
            if (v & 1) lb += pv;
            else la += pv;
            if (v < 8) p0[v] = (__bf16)pv;
            else p1[v - 8] = (__bf16)pv;
          }
        }
        {
          typename Pick<kF8, u32x2, bf16x8>::T vf[PFV];
#pragma unroll
          for (int s = 0; s < PFV; ++s) MLA_VREAD(cur, s, vf[s]);
#pragma unroll
          for (int s = 0; s < 32; ++s) {
            if constexpr (kF8) pv_mfma_v(o[s & 15], fp8x8_to_bf16(vf[s % PFV]), (s >> 4) ? p1 : p0);
            else pv_mfma_v(o[s & 15], vf[s % PFV], (s >> 4) ? p1 : p0);
            if (s + PFV < 32) MLA_VREAD(cur, s + PFV, vf[s % PFV]);
          }
        }
      }
      if (__ballot(amax > kRefHeadroom) == 0) break;
      // one redo at most, as in the wide kernel
      if (!first_pass) {
        lane0_atomic_or(&a.hdr[2], MLA_CHECK_SCORE_RANGE);
        break;
      }
      m_run += pair_max(amax);
      first_pass = false;
      amax = -INFINITY;
      la = 0.0f;
      lb = 0.0f;
      pv_drain(o);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16{};
    }
    pv_drain(o);
    if (__builtin_amdgcn_readfirstlane(bad)) lane0_atomic_or(&a.hdr[2], MLA_CHECK_BLOCK_ID_RANGE);

    const float l_tot = pair_sum(la + lb);
    const float lse2 = m_run + log2f(l_tot);
    const float own_inv = (kF8 ? a.v_scale : 1.0f) / l_tot;
    if (cnt == 1) {
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = o[cb][4 * g + r] * own_inv;
          store_out4(cb, g, v);
        }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2 * kLn2), lse_r, hl_e * 4, 0, 0);
      continue;
    }
    // split request: partial in the accumulator layout (lanes of padding
    // heads store values that no merge uses)
    auto part_rsrc = [&](int sl) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(a.part_o + size_t(sl) * HP * kDV), (short)0,
                                               HP * kDV * 4, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t plse_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.part_lse, (short)0, 0x7ffffff0, 0x00020000);
    const uint32_t lane_off = uint32_t(lane_e) * 16;
    // partial offset of this lane: lanes of padding heads point past the
    // resource, so their stores and loads are dropped without a branch
    const uint32_t part_off = hl_e < a.H ? lane_off : 0x40000000u;
    auto publish = [&]() {
      const __amdgpu_buffer_rsrc_t pr = part_rsrc(it);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4;
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = o[cb][4 * g + r] * own_inv;
          __builtin_amdgcn_raw_buffer_store_b128(v4, pr, (cb * 4 + g) * 1024 + part_off, 0, kSc1);
        }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2), plse_r, uint32_t(it * HP + hl_e) * 4, 0, kSc1);
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the partial is out
      lane0_fetch_add(&a.ctr[kCtr * b + kPublished], 1);
    };
    if (cnt >= kMergeMinItems) {
      publish();
      continue;
    }
    const int ticket = wave_fetch_add(&a.ctr[kCtr * b + kTicket]);
    if (ticket == 0) {
      publish();
      continue;
    }
    // the last of two: its partner took its ticket earlier and only has
    // stores left
    wave_wait(&a.ctr[kCtr * b + kPublished], 1);
    __hip_atomic_store(&a.ctr[kCtr * b + kTicket], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.ctr[kCtr * b + kPublished], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    {
      const i32x4 rq = ((const CONST_AS i32x4*)a.req)[b];
      auto slot_of = [&](int s) { return (s < rq[1]) ? rq[0] + s : rq[2]; };
      auto lse_of = [&](int sl) {
        return sl == it ? lse2
                        : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                              plse_r, uint32_t(sl * HP + hl_e) * 4, 0, kSc1));
      };
      const int s0 = slot_of(0), s1 = slot_of(1);
      const float l0 = lse_of(s0), l1 = lse_of(s1);
      const float mlse = fmaxf(l0, l1);
      const float e0 = __builtin_amdgcn_exp2f(l0 - mlse), e1 = __builtin_amdgcn_exp2f(l1 - mlse);
      const float lam = e0 + e1;
      const float inv = 1.0f / lam;
      const float w0 = e0 * inv, w1 = e1 * inv;
      const bool own_first = s0 == it;
      const __amdgpu_buffer_rsrc_t pr = part_rsrc(own_first ? s1 : s0);
      // the partner's partial through this wave's slot, in two rounds
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      constexpr int kRound = kStageBytes / 1024;  // 36 blocks
#pragma unroll
      for (int r0 = 0; r0 < 64; r0 += kRound) {
        const int n = (64 - r0) < kRound ? (64 - r0) : kRound;
#pragma unroll
        for (int j = 0; j < kRound; ++j)
          if (j < n) dma16_buffer(pr, uint32_t(r0 + j) * 1024 + part_off, slot + j * 1024);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        constexpr int kGroup = 6;
#pragma unroll
        for (int j0 = 0; j0 < kRound; j0 += kGroup) {
          f32x4 xs[kGroup];
#pragma unroll
          for (int jj = 0; jj < kGroup; ++jj)
            if (j0 + jj < n) xs[jj] = *(const f32x4 LDS_AS*)(slot + (j0 + jj) * 1024 + lane_off);
#pragma unroll
          for (int jj = 0; jj < kGroup; ++jj) {
            if (j0 + jj < n) {
              const int blk = r0 + j0 + jj, cb = blk >> 2, g = blk & 3;
              float v[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float own = o[cb][4 * g + r] * own_inv;
                v[r] = own_first ? fmaf(w1, xs[jj][r], w0 * own) : fmaf(w1, own, w0 * xs[jj][r]);
              }
              store_out4(cb, g, v);
            }
          }
        }
        // this round's reads are done before the next round refills the slot
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((mlse + log2f(lam)) * kLn2), lse_r, hl_e * 4, 0, 0);
    }
  }
#undef MLA_KREAD
#undef MLA_KREAD16
#undef MLA_VREAD

  // ---- merge units: 128 columns (16 blocks of 1 KB per item) each ----
  for (;;) {
    if (n_units == 0) break;
    const int u = wave_fetch_add(&a.hdr[6]);
    if (u >= n_units) {
      if (u == n_units + n_workers - 1) __hip_atomic_store(&a.hdr[6], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    const int b = __builtin_amdgcn_readfirstlane(((const CONST_AS int32_t*)a.big)[u / kNarrowUnits]);
    const int cb0 = (u % kNarrowUnits) * (16 / kNarrowUnits);
    const i32x4 rq = ((const CONST_AS i32x4*)a.req)[b];
    const int cnt = __builtin_amdgcn_readfirstlane(rq[3]);
    wave_wait(&a.ctr[kCtr * b + kPublished], cnt);
    int lane_m = lane;
    asm volatile("" : "+v"(lane_m));
    const int hl_m = lane_m & 31;
    const int hi_m = lane_m >> 5;
    // lanes of padding heads read past the resource (zeros, no traffic)
    const uint32_t moff = (hl_m < a.H ? uint32_t(lane_m) * 16 : 0x40000000u) + uint32_t(cb0) * 4096;
    auto slot_of = [&](int s) { return (s < rq[1]) ? rq[0] + s : rq[2]; };
    const __amdgpu_buffer_rsrc_t plse_r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.part_lse, (short)0, 0x7ffffff0, 0x00020000);
    auto lse_of = [&](int sl) {
      return __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(plse_r, uint32_t(sl * HP + hl_m) * 4, 0, kSc1));
    };
    // weights of this lane's head in this wave's slot (the slot's previous
    // reads are done), up to kSlots items
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr int kSlots = kStageBytes / (32 * 4);
    float LDS_AS* wsl = (float LDS_AS*)(slot) + hl_m;
    const bool in_lds = cnt <= kSlots;
    // items' log-sum-exps in batches of 16, every load of a batch in flight
    float mlse = -INFINITY;
    for (int s0 = 0; s0 < cnt; s0 += 16) {
      float lv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) lv[j] = (s0 + j < cnt) ? lse_of(slot_of(s0 + j)) : -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        mlse = fmaxf(mlse, lv[j]);
        if (in_lds && s0 + j < cnt) wsl[32 * (s0 + j)] = lv[j];
      }
    }
    float lam = 0.0f;
    for (int s = 0; s < cnt; ++s) {
      const float e = __builtin_amdgcn_exp2f((in_lds ? wsl[32 * s] : lse_of(slot_of(s))) - mlse);
      lam += e;
      if (in_lds) wsl[32 * s] = e;
    }
    const float inv = 1.0f / lam;
    auto weight = [&](int s) {
      return (in_lds ? wsl[32 * s] : __builtin_amdgcn_exp2f(lse_of(slot_of(s)) - mlse)) * inv;
    };
    constexpr int kNB = 4 * (16 / kNarrowUnits);  // 1 KB blocks per item
    constexpr int kBatch = 32 / kNB;
    f32x4 acc[kNB] = {};
    for (int s0 = 0; s0 < cnt; s0 += kBatch) {
      f32x4 x[kBatch][kNB];
      float wt[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (s0 + j < cnt) {
          const int sl = slot_of(s0 + j);
          const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(a.part_o + size_t(sl) * HP * kDV), (short)0, HP * kDV * 4, 0x00020000);
#pragma unroll
          for (int g = 0; g < kNB; ++g)
            x[j][g] = __builtin_amdgcn_raw_buffer_load_b128(pr, moff + g * 1024, 0, kSc1);
          wt[j] = weight(s0 + j);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (s0 + j < cnt)
#pragma unroll
          for (int g = 0; g < kNB; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[g][r] = fmaf(wt[j], x[j][g][r], acc[g][r]);
    }
    {
      // stores of heads >= H fall outside the resources
      const __amdgpu_buffer_rsrc_t out_r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.out + size_t(b) * a.H * kDV), (short)0, a.H * kDV * 2, 0x00020000);
      const uint32_t ooff = uint32_t(hl_m * kDV + 4 * hi_m + 32 * cb0) * 2;
#pragma unroll
      for (int g = 0; g < kNB; ++g) {
        bf16x4 h4;
#pragma unroll
        for (int r = 0; r < 4; ++r) h4[r] = (__bf16)acc[g][r];
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h4), out_r,
                                              ooff + (32 * (g >> 2) + 8 * (g & 3)) * 2, 0, 0);
      }
      if (cb0 == 0) {
        const __amdgpu_buffer_rsrc_t lse_r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.lse + size_t(b) * a.H), (short)0, a.H * 4, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((mlse + log2f(lam)) * kLn2), lse_r,
                                              hl_m * 4, 0, 0);
      }
    }
    // the request's last unit leaves its counters ready for the next call
    const int t = wave_fetch_add(&a.ctr[kCtr * b + kTicket]);
    if (t == kNarrowUnits - 1) {
      __hip_atomic_store(&a.ctr[kCtr * b + kTicket], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctr[kCtr * b + kPublished], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanCands = 256;  // candidate chunk sizes
constexpr int kPlanParts = kPlanThreads / kPlanCands;  // threads per candidate
constexpr int kPlanLens = 4096;  // seq_lens staged in LDS per pass

__device__ __forceinline__ int plan_candidate(int i) {
  // chunk = 32 * k: k = 1..128, then geometric up to 32 * 32768 tokens
  if (i < 128) return 32 * (i + 1);
  const int e = i - 128;  // 0..127
  const float k = 128.0f * exp2f((e + 1) * (8.0f / 128.0f));
  return 32 * int(k);
}

// Wave-wide inclusive scans on DPP: row shifts by 1, 2, 4 and 8 scan each
// row of 16 lanes, then the last lane of row 0 (row 2) is broadcast into
// row 1 (row 3), and the last lane of row 1 into rows 2 and 3.  A lane whose
// source is outside its row, or whose row the mask leaves out, keeps `old`,
// the operation's identity.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_i32(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, kCtrl, kRowMask, 0xf, false);
}
__device__ __forceinline__ int wave_incl_add(int x) {
  x += dpp_i32<0x111, 0xf>(0, x);  // row_shr:1
  x += dpp_i32<0x112, 0xf>(0, x);  // row_shr:2
  x += dpp_i32<0x114, 0xf>(0, x);  // row_shr:4
  x += dpp_i32<0x118, 0xf>(0, x);  // row_shr:8
  x += dpp_i32<0x142, 0xa>(0, x);  // row_bcast:15 into rows 1 and 3
  x += dpp_i32<0x143, 0xc>(0, x);  // row_bcast:31 into rows 2 and 3
  return x;
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ unsigned long long dpp_min_u64(unsigned long long x) {
  const int lo = dpp_i32<kCtrl, kRowMask>(-1, int(uint32_t(x)));
  const int hi = dpp_i32<kCtrl, kRowMask>(-1, int(uint32_t(x >> 32)));
  const unsigned long long y = (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
  return y < x ? y : x;
}
// the least of the wave's 64 values, in every lane
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long x) {
  x = dpp_min_u64<0x111, 0xf>(x);
  x = dpp_min_u64<0x112, 0xf>(x);
  x = dpp_min_u64<0x114, 0xf>(x);
  x = dpp_min_u64<0x118, 0xf>(x);
  x = dpp_min_u64<0x142, 0xa>(x);
  x = dpp_min_u64<0x143, 0xc>(x);
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(x)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(x >> 32)), 63);
  return (uint64_t(hi) << 32) | lo;
}

// Inclusive block-wide scan of four ints per thread; returns the inclusive
// scan and the block totals.  A DPP scan in each wave, then the wave totals
// through LDS.
struct Scan4 {
  int4 incl, total;
};
// kReuse: s_scan is written again after this scan, so every wave must have
// read it first (a second barrier).
template <bool kReuse = true>
__device__ __forceinline__ Scan4 block_scan4(int4 v, int4* s_scan) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int4 x = make_int4(wave_incl_add(v.x), wave_incl_add(v.y), wave_incl_add(v.z), wave_incl_add(v.w));
  if (lane == 63) s_scan[wv] = x;
  __syncthreads();
  int4 pre = make_int4(0, 0, 0, 0), tot = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < kPlanThreads / 64; ++i) {
    const int4 t = s_scan[i];
    if (i < wv) {
      pre.x += t.x;
      pre.y += t.y;
      pre.z += t.z;
      pre.w += t.w;
    }
    tot.x += t.x;
    tot.y += t.y;
    tot.z += t.z;
    tot.w += t.w;
  }
  Scan4 r;
  r.incl = make_int4(x.x + pre.x, x.y + pre.y, x.z + pre.z, x.w + pre.w);
  r.total = tot;
  if (kReuse) __syncthreads();  // every wave has read s_scan before the next scan writes it
  return r;
}

// Items are laid out as the pairs (requests split into exactly two items)
// first, then the full chunks of every other request, then their last
// (shorter) chunks, then one item per empty request.  With at most kPlanLens
// requests the (clamped) lengths are read from memory once and kept in LDS.
// kSingle: B <= kPlanThreads, placed in one pass (the instantiation holds
// only that path, so none of the multi-pass code's registers are live).
template <bool kSingle>
__global__ __launch_bounds__(kPlanThreads) void mla_plan_kernel(
    const int32_t* __restrict__ seq_lens, int B, int M, int lgBS, int n_slots, int forced,
    int ovh, int cap, int units_per_req, int nx, int32_t* __restrict__ hdr, int4* __restrict__ req,
    int32_t* __restrict__ ctr, int32_t* __restrict__ big, int4* __restrict__ items) {
  __shared__ unsigned long long s_key[kPlanCands / 64];
  __shared__ long long s_part[kPlanParts][kPlanCands];
  __shared__ int4 s_scan[kPlanThreads / 64];
  __shared__ __attribute__((aligned(16))) int s_len[kPlanLens];
  __shared__ __attribute__((aligned(16))) float s_m[kPlanLens];
  const int tid = threadIdx.x;
  const int Lmax = M << lgBS;
  const bool resident = kSingle || B <= kPlanLens;
  auto clamp_len = [&](int L0) { return min(max(L0, 0), Lmax); };
  // lengths of requests b0 .. b0 + nb - 1 into LDS, padded with -1 to a
  // multiple of 4, and ceil(L / 32) as floats, padded with 0; returns this
  // thread's range-check bit
  auto stage = [&](int b0, int nb) {
    int bad = 0;
    const int nb4 = (nb + 3) & ~3;
    for (int i = tid; i < nb4; i += kPlanThreads) {
      int L = -1;
      if (i < nb) {
        const int L0 = seq_lens[b0 + i];
        bad |= (L0 < 0 || L0 > Lmax) ? 1 : 0;
        L = clamp_len(L0);
      }
      s_len[i] = L;
      s_m[i] = float((max(L, 0) + 31) >> 5);
    }
    __syncthreads();
    return bad;
  };
  int bad = 0;
  if (resident) bad = stage(0, B);
  auto len_of = [&](int b) { return resident ? s_len[b] : clamp_len(seq_lens[b]); };

  // 1) chunk size: four threads price each of the kPlanCands candidates,
  //    cost = ceil(items / slots) * (chunk + per-item overhead), each over a
  //    quarter of the requests (every fourth group of four lengths).
  int chunk = forced;
  if (forced <= 0) {
    const int cand = tid % kPlanCands, part = tid / kPlanCands;
    const int T = plan_candidate(cand);
    // ceil(L / T) for T = 32 d: ceil(ceil(L / 32) / d), with the quotient from
    // a float reciprocal (off by at most one for these sizes) and one exact
    // correction; this keeps integer division out of the B x 256 loop.
    const int d = T >> 5;
    const float inv_d = 1.0f / float(d);
    auto items_of = [&](int L) {
      const int m = (L + 31) >> 5;
      int q = int(float(m) * inv_d);
      const int r = m - q * d;
      q += (r >= d) - (r < 0);
      const int rr = m - q * d;
      return (L < 0) ? 0 : max(1, q + (rr > 0));  // L < 0: padding
    };
    // Float form of the same count, four VALU ops per request: with m < 2^22
    // and 1/d within one ulp, fma(m, 1/d, -1/(2d)) lies within 1/(2d) of
    // (m - 1/2) / d, so its ceiling is ceil(m / d) exactly.  Each thread's
    // float sum is exact below 2^24 and stays at or above 2^24 (past any
    // workspace cap) once its count gets there.  Padding entries (m = 0)
    // count one each.
    const bool fast = Lmax <= (1 << 26);
    const float inv_df = 1.0f / float(d);
    const float half_df = 0.5f * inv_df;
    auto items_f = [&](float m) { return fmaxf(1.0f, ceilf(__builtin_fmaf(m, inv_df, -half_df))); };
    long long n = 0;
    for (int b0 = 0; b0 < B; b0 += kPlanLens) {
      const int nb = min(kPlanLens, B - b0);
      if (!resident) bad |= stage(b0, nb);
      const int nb4 = (nb + 3) & ~3;
      if (fast) {
        float acc = 0.0f;
#pragma unroll 2
        for (int i = 4 * part; i < nb4; i += 4 * kPlanParts) {
          const float4 m4 = *reinterpret_cast<const float4*>(&s_m[i]);
          acc += (items_f(m4.x) + items_f(m4.y)) + (items_f(m4.z) + items_f(m4.w));
        }
        n += (long long)acc - (part == 0 ? nb4 - nb : 0);
      } else {
#pragma unroll 2
        for (int i = 4 * part; i < nb4; i += 4 * kPlanParts) {
          const int4 m4 = *reinterpret_cast<const int4*>(&s_len[i]);
          n += items_of(m4.x) + items_of(m4.y) + items_of(m4.z) + items_of(m4.w);
        }
      }
      if (!resident) __syncthreads();
    }
    s_part[part][cand] = n;
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int p = 1; p < kPlanParts; ++p) n += s_part[p][cand];
      // A count within the cap fits 32 bits, and so does its division.  The
      // key orders candidates by cost, then by larger chunk (candidates
      // grow with their index): cost * 256 + (255 - index), below 2^60;
      // 2^62 marks a candidate whose items exceed the cap.
      const unsigned long long cost =
          (unsigned long long)((uint32_t(n) + uint32_t(n_slots) - 1u) / uint32_t(n_slots)) *
          (unsigned long long)(T + ovh);
      const unsigned long long key = (n <= cap) ? (cost << 8) | uint32_t(kPlanCands - 1 - cand) : (1ull << 62);
      const unsigned long long wmin = wave_min_u64(key);
      if ((tid & 63) == 0) s_key[tid >> 6] = wmin;
    }
    __syncthreads();
    unsigned long long kmin = s_key[0];
#pragma unroll
    for (int i = 1; i < kPlanCands / 64; ++i) kmin = s_key[i] < kmin ? s_key[i] : kmin;
    const int kb = plan_candidate(kPlanCands - 1 - int(kmin & 0xff));
    chunk = kb;
    // no candidate fits the workspace: one item per request
    if (kmin >= (1ull << 62)) chunk = ((Lmax + 31) / 32) * 32;
  } else if (!resident) {
    for (int b0 = 0; b0 < B; b0 += kPlanLens) {
      bad |= stage(b0, min(kPlanLens, B - b0));
      __syncthreads();
    }
  }

  // Pairs (requests split into exactly two items) come first.  The two
  // items of pair j of the first nx * G pairs (G = NP / nx) sit nx
  // positions apart, so that workgroups w and w + nx, which the dispatcher
  // places on the same XCD, take them; the last NP % nx pairs follow side
  // by side, then the other items in the order full chunks, remainders,
  // empty requests.
  int NF, NR, NE, NP, NBIG, any_bad;
  auto pair_pos = [&](int j, int half, int G) {
    if (j < G * nx) return 2 * nx * (j / nx) + (j % nx) + half * nx;
    return 2 * j + half;
  };
  // Writes request b's record, its items and its merge-unit entry, given
  // the exclusive prefix counts of the requests before it (full chunks,
  // remainders, empties, pairs and widely split requests of the others).
  auto place = [&](int b, int L, int nf0, int nr0, int4 pre, int pre_big) {
    const int cnt = nf0 + nr0;
    const int Q0 = 2 * NP;  // first position of the other items
    if (cnt == 2) {
      const int G = NP / nx;
      const int p0 = pair_pos(pre.w, 0, G), p1 = pair_pos(pre.w, 1, G);
      req[b] = make_int4(p0, 1, p1, 2);
      items[p0] = make_int4(b, 0, chunk, 2);
      items[p1] = make_int4(b, chunk, L, 2);
    } else {
      const int fbeg = Q0 + pre.x;
      const int ritem = nr0 ? (Q0 + NF + pre.y) : -1;
      req[b] = make_int4(fbeg, nf0, ritem, cnt);
      for (int s = 0; s < nf0; ++s) items[fbeg + s] = make_int4(b, s * chunk, (s + 1) * chunk, cnt);
      if (nr0) items[ritem] = make_int4(b, nf0 * chunk, L, cnt);
      if (L == 0) items[Q0 + NF + NR + pre.z] = make_int4(b, 0, 0, 0);
      if (cnt >= kMergeMinItems) big[pre_big] = b;
    }
#pragma unroll
    for (int k = 0; k < kCtr; ++k) ctr[kCtr * b + k] = 0;
  };
  // this request's counts (full chunks, remainders, empty, pair) and
  // whether it is split widely enough for the merge units
  auto counts = [&](int b, int L, int& nbg, int& nf0, int& nr0) {
    nf0 = L / chunk;
    nr0 = (L - nf0 * chunk) ? 1 : 0;
    const bool pair = b < B && nf0 + nr0 == 2;
    nbg = (b < B && nf0 + nr0 >= kMergeMinItems) ? 1 : 0;
    return make_int4(pair ? 0 : nf0, pair ? 0 : nr0, (b < B && L == 0) ? 1 : 0, pair ? 1 : 0);
  };

  if (kSingle || (resident && B <= kPlanThreads)) {
    // 2) one pass: a single scan gives every request's prefix and the
    //    totals.  With B <= 1024 every count and prefix fits 16 bits, so
    //    the empty and widely-split counts share a word, as do the pair
    //    count and the range-check bits.
    const int b = tid;
    const int L = (b < B) ? s_len[b] : 0;
    int nbg, nf0, nr0;
    const int4 c = counts(b, L, nbg, nf0, nr0);
    const int4 packed = make_int4(c.x, c.y, c.z | (nbg << 16), c.w | ((b < B && bad) ? 1 << 16 : 0));
    const Scan4 sc = block_scan4<false>(packed, s_scan);
    NF = sc.total.x;
    NR = sc.total.y;
    NE = sc.total.z & 0xffff;
    NBIG = sc.total.z >> 16;
    NP = sc.total.w & 0xffff;
    any_bad = (sc.total.w >> 16) != 0;
    if (b < B) {
      const int4 pre = make_int4(sc.incl.x - c.x, sc.incl.y - c.y, (sc.incl.z & 0xffff) - c.z,
                                 (sc.incl.w & 0xffff) - c.w);
      place(b, L, nf0, nr0, pre, (sc.incl.z >> 16) - nbg);
    }
  } else if constexpr (!kSingle) {
    // 2) totals: the items of pairs and of all other requests, empty
    //    requests, widely split requests and the range-check bits
    int4 loc = make_int4(0, 0, 0, 0);
    int locbig = 0;
    for (int b = tid; b < B; b += kPlanThreads) {
      int nbg, nf0, nr0;
      const int4 c = counts(b, len_of(b), nbg, nf0, nr0);
      loc.x += c.x;
      loc.y += c.y;
      loc.z += c.z;
      loc.w += c.w;
      locbig += nbg;
    }
    const int4 tot = block_scan4(loc, s_scan).total;
    NF = tot.x;
    NR = tot.y;
    NE = tot.z;
    NP = tot.w;
    NBIG = block_scan4(make_int4(locbig, 0, 0, 0), s_scan).total.x;
    any_bad = __syncthreads_or(bad);
    // 3) per-request placement from exclusive scans, kPlanThreads requests
    //    at a time
    int4 carry = make_int4(0, 0, 0, 0);
    int carry_big = 0;
    for (int b0 = 0; b0 < B; b0 += kPlanThreads) {
      const int b = b0 + tid;
      const int L = (b < B) ? len_of(b) : 0;
      int nbg, nf0, nr0;
      const int4 c = counts(b, L, nbg, nf0, nr0);
      const Scan4 sc = block_scan4(c, s_scan);
      const Scan4 sb = block_scan4(make_int4(nbg, 0, 0, 0), s_scan);
      if (b < B) {
        const int4 pre = make_int4(carry.x + sc.incl.x - c.x, carry.y + sc.incl.y - c.y,
                                   carry.z + sc.incl.z - c.z, carry.w + sc.incl.w - c.w);
        place(b, L, nf0, nr0, pre, carry_big + sb.incl.x - nbg);
      }
      carry.x += sc.total.x;
      carry.y += sc.total.y;
      carry.z += sc.total.z;
      carry.w += sc.total.w;
      carry_big += sb.total.x;
    }
  }

  // 4) header
  if (tid == 0) {
    hdr[0] = 2 * NP + NF + NR + NE;
    hdr[1] = chunk;
    hdr[2] = any_bad ? MLA_CHECK_SEQ_LEN_RANGE : 0;
    hdr[3] = 0;
    hdr[4] = 2 * nx * (NP / nx);  // items placed as XCD-sharing pairs
    hdr[5] = NBIG * units_per_req;
    hdr[6] = 0;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];  // 0 = not queried yet

mla_status device_cu_count(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  int c = g_cu_count[dev];
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MLA_ERR_HIP;
    g_cu_count[dev] = c;
  }
  *n = c;
  return MLA_OK;
}

int g_xcd_count[kMaxDevices];  // 0 = not queried yet

// XCDs of the current device (1 where the runtime does not report them).
mla_status device_xcd_count(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  int c = g_xcd_count[dev];
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || c < 1) c = 1;
    g_xcd_count[dev] = c;
  }
  *n = c;
  return MLA_OK;
}

int ilog2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

mla_status check_sizes(int32_t B, int32_t H, int32_t M, int32_t BS) {
  if (B < 0 || H < 0 || M < 0 || BS < 0) return MLA_ERR_BAD_SHAPE;
  if (H < 1 || H > 128) return MLA_ERR_UNSUPPORTED;
  const int lg = ilog2_exact(BS);
  if (lg < 4 || lg > 10) return MLA_ERR_UNSUPPORTED;
  if (M < 1) return MLA_ERR_BAD_SHAPE;
  if ((long long)M * BS > (1ll << 28)) return MLA_ERR_BAD_SHAPE;
  if (B > (1 << 24)) return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mla_status check_workspace(const void* ws, size_t ws_bytes, int B, int H) {
  if (!ws) return MLA_ERR_NULL_POINTER;
  if (!aligned(ws, 256)) return MLA_ERR_ALIGNMENT;
  if (ws_bytes < ws_layout(B, H).total) return MLA_ERR_WORKSPACE;
  return MLA_OK;
}

// Kernel variant for H heads: waves per workgroup, LDS stages, workgroups per CU.
// Kernel variant for H heads: waves per workgroup (0: the narrow kernel of
// independent wave workers), queue workers per compute unit, merge units per
// widely split request.
struct Variant {
  int nw, workers_per_cu, units_per_req;
};
Variant pick_variant(int H) {
  if (H > 64) return {4, 1, 16};
  if (H > 32) return {2, 1, 8};
  return {0, kNarrowWaves, kNarrowUnits};
}

int item_overhead_tokens(int H) { return 32 + 2 * H; }

template <int NW, int NS>
hipError_t launch_attend(const AttendArgs& a, int grid, hipStream_t st) {
  // block sizes of 32 tokens or more keep every stage in one block
  if (a.lgBS >= 5)
    hipLaunchKernelGGL((mla_attend_kernel<NW, NS, true>), dim3(grid), dim3(NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((mla_attend_kernel<NW, NS, false>), dim3(grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

// The factor the kernels apply to raw scores: scale * kv_scale * log2(e), in
// fp32 as they receive it.  Finite inputs can still overflow it (scale near
// the fp32 maximum, or a large product), which would turn every score into
// +-inf and the outputs into NaN, so it is checked on its own.
float scale_log2(float scale, float kv_scale) { return scale * kv_scale * 1.4426950408889634f; }

mla_status validate_attend(const void* q, const void* latent_cache, const int32_t* block_table,
                           float scale, const void* out, const float* lse, int32_t B, int32_t H,
                           int32_t NB, int32_t BS, int32_t M, const void* workspace,
                           size_t workspace_bytes) {
  mla_status s = check_sizes(B, H, M, BS);
  if (s != MLA_OK) return s;
  if (NB < 1) return MLA_ERR_BAD_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !latent_cache || !block_table || !out || !lse) return MLA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(latent_cache, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      !aligned(block_table, 4))
    return MLA_ERR_ALIGNMENT;
  if (!isfinite(scale) || !isfinite(scale_log2(scale, 1.0f))) return MLA_ERR_BAD_SCALE;
  return check_workspace(workspace, workspace_bytes, B, H);
}

// The fp8 cache runs on every kernel and block size the bf16 cache does.
mla_status validate_attend_fp8(const void* q, const void* latent_cache, const int32_t* block_table,
                               float scale, float kv_scale, const void* out, const float* lse,
                               int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                               const void* workspace, size_t workspace_bytes) {
  mla_status s = validate_attend(q, latent_cache, block_table, scale, out, lse, B, H, NB, BS, M,
                                 workspace, workspace_bytes);
  if (s != MLA_OK) return s;
  if (!isfinite(kv_scale) || !isfinite(scale_log2(scale, kv_scale))) return MLA_ERR_BAD_SCALE;
  return MLA_OK;
}

AttendArgs attend_args(const void* q, const void* latent_cache, const int32_t* block_table,
                       float scale, float kv_scale, void* out, float* lse, int32_t B, int32_t H,
                       int32_t NB, int32_t BS, int32_t M, const WsLayout& L, char* ws) {
  AttendArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.cache = static_cast<const __bf16*>(latent_cache);
  a.table = block_table;
  a.out = static_cast<__bf16*>(out);
  a.lse = lse;
  a.hdr = reinterpret_cast<int32_t*>(ws);
  a.req = reinterpret_cast<const int4*>(ws + L.req_off);
  a.ctr = reinterpret_cast<int32_t*>(ws + L.ctr_off);
  a.items = reinterpret_cast<const int4*>(ws + L.item_off);
  a.big = reinterpret_cast<const int32_t*>(ws + L.big_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.plse_off);
  a.part_o = reinterpret_cast<float*>(ws + L.po_off);
  a.scale_log2 = scale_log2(scale, kv_scale);
  a.v_scale = kv_scale;
  a.B = B;
  a.H = H;
  a.NB = NB;
  a.M = M;
  a.lgBS = ilog2_exact(BS);
  return a;
}

mla_status validate_plan(const int32_t* seq_lens, int32_t B, int32_t H, int32_t M, int32_t BS,
                         int32_t chunk_tokens, const void* workspace, size_t workspace_bytes) {
  mla_status s = check_sizes(B, H, M, BS);
  if (s != MLA_OK) return s;
  if (B == 0) return MLA_OK;
  if (!seq_lens) return MLA_ERR_NULL_POINTER;
  if (!aligned(seq_lens, 4)) return MLA_ERR_ALIGNMENT;
  if ((s = check_workspace(workspace, workspace_bytes, B, H)) != MLA_OK) return s;
  if (chunk_tokens < 0) return MLA_ERR_UNSUPPORTED;
  if (chunk_tokens > 0) {
    if (chunk_tokens % kSub) return MLA_ERR_UNSUPPORTED;
    const long long per = ((long long)M * BS + chunk_tokens - 1) / chunk_tokens;
    if ((long long)B * per > ws_layout(B, H).cap) return MLA_ERR_UNSUPPORTED;
  }
  return MLA_OK;
}

// The plan kernel over a workspace of layout L at ws.
mla_status launch_plan(const int32_t* seq_lens, int32_t B, int32_t H, int32_t M, int32_t BS,
                       int32_t chunk_tokens, const WsLayout& L, char* ws, hipStream_t st) {
  int ncu = 0, nxcd = 1;
  mla_status s;
  if ((s = device_cu_count(&ncu)) != MLA_OK) return s;
  if ((s = device_xcd_count(&nxcd)) != MLA_OK) return s;
  const Variant v = pick_variant(H);
  // the wide kernels take their first items in workgroup order, so pairs
  // placed nx apart land on one XCD; the narrow kernel's workers do not
  const int nx = v.nw ? nxcd : 1;
  auto launch_plan = [&](auto single_c) {
    hipLaunchKernelGGL((mla_plan_kernel<decltype(single_c)::value>), dim3(1), dim3(kPlanThreads), 0, st,
                       seq_lens, (int)B, (int)M, ilog2_exact(BS), ncu * v.workers_per_cu,
                       (int)chunk_tokens, item_overhead_tokens(H), L.cap, v.units_per_req, nx,
                       reinterpret_cast<int32_t*>(ws), reinterpret_cast<int4*>(ws + L.req_off),
                       reinterpret_cast<int32_t*>(ws + L.ctr_off),
                       reinterpret_cast<int32_t*>(ws + L.big_off),
                       reinterpret_cast<int4*>(ws + L.item_off));
  };
  if (B <= kPlanThreads) launch_plan(BoolC<true>{});
  else launch_plan(BoolC<false>{});
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// The attend kernel (bf16 cache) over a workspace of layout L at ws.
mla_status launch_attend_bf16(const void* q, const void* latent_cache, const int32_t* block_table,
                              float scale, void* out, float* lse, int32_t B, int32_t H, int32_t NB,
                              int32_t BS, int32_t M, const WsLayout& L, char* ws, hipStream_t st) {
  int ncu = 0;
  mla_status s;
  if ((s = device_cu_count(&ncu)) != MLA_OK) return s;
  const AttendArgs a = attend_args(q, latent_cache, block_table, scale, 1.0f, out, lse, B, H, NB,
                                   BS, M, L, ws);
  const Variant v = pick_variant(H);
  const int grid = ncu;  // one workgroup per compute unit
  hipError_t e;
  switch (v.nw) {
    case 4: e = launch_attend<4, 4>(a, grid, st); break;
    case 2: e = launch_attend<2, 4>(a, grid, st); break;
    default:
      if (a.lgBS >= 5)
        hipLaunchKernelGGL(mla_attend_narrow_kernel<true>, dim3(grid), dim3(kNarrowWaves * 64), 0, st, a);
      else
        hipLaunchKernelGGL(mla_attend_narrow_kernel<false>, dim3(grid), dim3(kNarrowWaves * 64), 0, st, a);
      e = hipGetLastError();
      break;
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The decode without a workspace argument: its plan and split partials live
// in this file-scope array, one per GPU the library runs on, held until the
// process ends.  Host code reaches it only through the device address that
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB
static __device__ __align__(256) char scratch[kScratchBytes];
void* g_scratch[kMaxDevices];  // device address of scratch on each device (null: not taken yet)
std::mutex g_scratch_mu;

mla_status scratch_address(void** p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return MLA_ERR_HIP;
    g_scratch[dev] = a;
  }
  *p = g_scratch[dev];
  return MLA_OK;
}

// The largest work-item capacity (at most B + kMaxExtraItems) whose layout
// fits the scratch array; below B the batch does not fit at all.
int scratch_cap(int B, int H) {
  int hi = B + kMaxExtraItems;
  if (ws_layout(B, H, hi).total <= kScratchBytes) return hi;
  int lo = -1;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (ws_layout(B, H, mid).total <= kScratchBytes) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace

extern "C" {

size_t mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t M, int32_t BS) {
  if (check_sizes(B, H, M, BS) != MLA_OK) return 0;
  return ws_layout(B, H).total;
}

mla_status mla_decode_plan(const int32_t* seq_lens, int32_t B, int32_t H, int32_t M,
                           int32_t BS, int32_t chunk_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  mla_status s = validate_plan(seq_lens, B, H, M, BS, chunk_tokens, workspace, workspace_bytes);
  if (s != MLA_OK || B == 0) return s;
  return launch_plan(seq_lens, B, H, M, BS, chunk_tokens, ws_layout(B, H),
                     static_cast<char*>(workspace), (hipStream_t)stream);
}

mla_status mla_decode_attend(const void* q, const void* latent_cache,
                             const int32_t* block_table, float scale, void* out, float* lse,
                             int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                             void* workspace, size_t workspace_bytes, void* stream) {
  mla_status s = validate_attend(q, latent_cache, block_table, scale, out, lse, B, H, NB, BS, M,
                                 workspace, workspace_bytes);
  if (s != MLA_OK || B == 0) return s;
  return launch_attend_bf16(q, latent_cache, block_table, scale, out, lse, B, H, NB, BS, M,
                            ws_layout(B, H), static_cast<char*>(workspace), (hipStream_t)stream);
}

mla_status mla_decode(const void* q, const void* latent_cache, const int32_t* block_table,
                      const int32_t* seq_lens, float scale, void* out, float* lse, int32_t B,
                      int32_t H, int32_t NB, int32_t BS, int32_t M, void* workspace,
                      size_t workspace_bytes, void* stream) {
  // Validate everything up front so that nothing is enqueued on failure.
  mla_status s = validate_attend(q, latent_cache, block_table, scale, out, lse, B, H, NB, BS, M,
                                 workspace, workspace_bytes);
  if (s != MLA_OK || B == 0) return s;
  if ((s = validate_plan(seq_lens, B, H, M, BS, 0, workspace, workspace_bytes)) != MLA_OK) return s;
  if ((s = mla_decode_plan(seq_lens, B, H, M, BS, 0, workspace, workspace_bytes, stream)) != MLA_OK)
    return s;
  return mla_decode_attend(q, latent_cache, block_table, scale, out, lse, B, H, NB, BS, M,
                           workspace, workspace_bytes, stream);
}

mla_status mla_decode_noalloc(const void* q, const void* latent_cache, const int32_t* block_table,
                              const int32_t* seq_lens, float scale, void* out, float* lse,
                              int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M, void* stream) {
  // the argument checks of mla_decode, with the scratch array's layout in
  // place of a caller's workspace; nothing is enqueued on failure
  mla_status s = check_sizes(B, H, M, BS);
  if (s != MLA_OK) return s;
  if (NB < 1) return MLA_ERR_BAD_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !latent_cache || !block_table || !seq_lens || !out || !lse) return MLA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(latent_cache, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return MLA_ERR_ALIGNMENT;
  if (!isfinite(scale) || !isfinite(scale_log2(scale, 1.0f))) return MLA_ERR_BAD_SCALE;
  const int cap = scratch_cap(B, H);
  if (cap < B) return MLA_ERR_WORKSPACE;  // the batch needs more than the scratch array holds
  void* base = nullptr;
  if ((s = scratch_address(&base)) != MLA_OK) return s;
  const WsLayout L = ws_layout(B, H, cap);
  char* ws = static_cast<char*>(base);
  hipStream_t st = (hipStream_t)stream;
  if ((s = launch_plan(seq_lens, B, H, M, BS, 0, L, ws, st)) != MLA_OK) return s;
  return launch_attend_bf16(q, latent_cache, block_table, scale, out, lse, B, H, NB, BS, M, L, ws, st);
}

mla_status mla_decode_attend_fp8(const void* q, const void* latent_cache,
                                 const int32_t* block_table, float scale, float kv_scale,
                                 void* out, float* lse, int32_t B, int32_t H, int32_t NB,
                                 int32_t BS, int32_t M, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  mla_status s = validate_attend_fp8(q, latent_cache, block_table, scale, kv_scale, out, lse, B, H,
                                     NB, BS, M, workspace, workspace_bytes);
  if (s != MLA_OK || B == 0) return s;
  int ncu = 0;
  if ((s = device_cu_count(&ncu)) != MLA_OK) return s;
  const AttendArgs a = attend_args(q, latent_cache, block_table, scale, kv_scale, out, lse, B, H,
                                   NB, BS, M, ws_layout(B, H), static_cast<char*>(workspace));
  hipStream_t st = (hipStream_t)stream;
  // wide kernels: eight fp8 stages and the two weight buffers fill the 160
  // KiB of LDS; narrow kernel (H <= 32): two fp8 stages per wave slot
  // (blocks of 16 tokens: each stage spans two blocks)
  const bool one = a.lgBS >= 5;
  switch (pick_variant(H).nw) {
    case 4:
      if (one) hipLaunchKernelGGL((mla_attend_kernel<4, 8, true, true>), dim3(ncu), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((mla_attend_kernel<4, 8, false, true>), dim3(ncu), dim3(256), 0, st, a);
      break;
    case 2:
      if (one) hipLaunchKernelGGL((mla_attend_kernel<2, 8, true, true>), dim3(ncu), dim3(128), 0, st, a);
      else hipLaunchKernelGGL((mla_attend_kernel<2, 8, false, true>), dim3(ncu), dim3(128), 0, st, a);
      break;
    default:
      if (one) hipLaunchKernelGGL((mla_attend_narrow_kernel<true, true>), dim3(ncu), dim3(kNarrowWaves * 64), 0, st, a);
      else hipLaunchKernelGGL((mla_attend_narrow_kernel<false, true>), dim3(ncu), dim3(kNarrowWaves * 64), 0, st, a);
      break;
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_fp8(const void* q, const void* latent_cache, const int32_t* block_table,
                          const int32_t* seq_lens, float scale, float kv_scale, void* out,
                          float* lse, int32_t B, int32_t H, int32_t NB, int32_t BS, int32_t M,
                          void* workspace, size_t workspace_bytes, void* stream) {
  mla_status s = validate_attend_fp8(q, latent_cache, block_table, scale, kv_scale, out, lse, B, H,
                                     NB, BS, M, workspace, workspace_bytes);
  if (s != MLA_OK || B == 0) return s;
  if ((s = validate_plan(seq_lens, B, H, M, BS, 0, workspace, workspace_bytes)) != MLA_OK) return s;
  if ((s = mla_decode_plan(seq_lens, B, H, M, BS, 0, workspace, workspace_bytes, stream)) != MLA_OK)
    return s;
  return mla_decode_attend_fp8(q, latent_cache, block_table, scale, kv_scale, out, lse, B, H, NB,
                               BS, M, workspace, workspace_bytes, stream);
}

mla_status mla_decode_read_error(const void* workspace, int32_t* flags, void* stream) {
  if (!workspace || !flags) return MLA_ERR_NULL_POINTER;
  if (!aligned(workspace, 256)) return MLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return MLA_ERR_HIP;
  int32_t v = 0;
  if (hipMemcpy(&v, static_cast<const char*>(workspace) + 8, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return MLA_ERR_HIP;
  *flags = v;
  return MLA_OK;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL_POINTER: return "MLA_ERR_NULL_POINTER";
    case MLA_ERR_BAD_SHAPE: return "MLA_ERR_BAD_SHAPE";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_BAD_SCALE: return "MLA_ERR_BAD_SCALE";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT";
    default: break;  // the range sentinels and any other value
  }
  return "MLA_ERR_UNKNOWN";
}

int32_t mla_decode_abi_version(void) { return 1; }

}  // extern "C"
