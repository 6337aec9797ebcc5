// qli_kernels.hip -- gfx950 (CDNA4) kernels of the quantized lightning indexer.
//
// Method: EngineX-Ascend page "VllmQuantLightningIndexer" (QLI-README),
// section 功能说明: score = sum_g W[g] * ReLU(ScaleQ[g] * ScaleK[s] * Q[g].K[s]),
// then the Top-k key indices per query token.
//
// Stage 1 scores every visible (row, key) pair of the work items:
//   * score_decode_kernel takes items of 1, 2 or 4 rows of one batch (from a
//     plan's table, a device-built table, its own split of bounded decode, or
//     for bounded runs of more rows 4-row groups that follow from the item's
//     position) and streams the item's key chunk through a 3-stage LDS ring
//     filled by direct-to-LDS loads, so the rows share every key byte read
//     from HBM; its waves raise their issue priority while behind in their
//     item, so the workgroups sharing a CU keep pace instead of finishing in
//     dispatch order;
//   * int8 keys use v_mfma_i32_16x16x64_i8 (exact int32 dots), e4m3fn
//     keys v_mfma_f32_16x16x128_f8f6f4; the 64 query heads of a row are the
//     M dimension (4 tiles of 16), 16 keys the N dimension, D=128 the K one;
//   * fused epilogue: ScaleQ is folded into W once per row (w' = W*ScaleQ,
//     exact in fp32 for fp16 inputs), so each (head, key) element costs
//     max + fma (an int8 dot enters the fma as the fp32 denormal its bits
//     spell, with w' and ScaleK carried by powers of two); the head sum
//     finishes with permlane swaps and one multiply by ScaleK[s].  This
//     reordering needs ScaleQ, ScaleK >= 0, which is the contract (dequant
//     scales are magnitudes);
//   * a row sees the entries [lo, hi) of its batch (lo > 0 only under a
//     pre_tokens window); rows that see at most sparse_count entries return
//     every visible index (the top-k of a set no larger than k is the set),
//     so their indices and scores are written straight to the outputs; other
//     rows stage fp32 scores in the workspace;
//   * bounded decode (no host plan) derives its items on the device: inside
//     score_decode_kernel for up to 256 batches (an instantiation of its
//     own, so planned runs carry none of its state), else decode_items_kernel
//     writes a plan-shaped table first; under a token window each row's range
//     is derived from its position as the planner does.
// Stage 2 selects (select_reg_kernel, select_global_kernel; one workgroup of
// 1024 threads per selection): rows of at most 8192 staged scores, and each
// 8192-score segment of longer rows, keep their top-k; a second launch
// merges a long row's segment winners.  Radix select over order-preserving
// uint32 keys held in registers (11-bit digits, starting below the bits
// every key shares, LDS histograms, block scans); ties at the threshold go to
// the lower index; the winners are written in ascending index order, and
// sort_rows_kernel reorders them by score when the caller asks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "qli_internal.h"

namespace qli {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kScoreThreads = 256;

struct ScoreParams {
  const Item* items;      // the plan's item table
  int32_t n_items;
  const int32_t* n_items_dev;  // bounded decode: the item count the device planner wrote (else null)
  int32_t plan_batches;        // bounded decode planned in the kernel: the batch count (else 0)
  int32_t chunk;          // keys per item
  int32_t reg_chunks, reg_rows, reg_maxv;  // regular decode plans (0: not regular); bounded tiles
  int32_t tiles;          // bounded runs of 4-row groups by position: item p is chunk p % reg_chunks
                          //   of group p / reg_chunks (BSND: reg_rows rows per batch; TND: the tables)
  const RowInfo* rinfo;   // the plan's row table
  const uint8_t* query;
  const uint8_t* key;
  const void* weights;
  const void* q_scale;
  const void* k_scale;
  const int32_t* block_table;
  float* ws;
  int32_t* idx_out;
  float* val_out;
  const int32_t* rows_end;     // bounded TND of many batches: the tables (TndTables), else null
  const int32_t* group_start;
  const int32_t* group_batch;
  const int32_t* aslq_tnd;     // bounded TND of few batches: the device prefix sums (tables in LDS), else null
  int32_t nbatch, trows;       //   batches, rows T
  const int32_t* aslk;  // bounded runs: key lengths on the device (else null; decode with a table: null)
  const int32_t* aslq_bsnd;  // bounded BSND: per-batch query counts (else null: all S1 rows used)
  int64_t max_len;      //   clamp for them (original tokens)
  int64_t bstride;      //   workspace elements per row
  int32_t mode, cmp;    //   sparse_mode, cmp_ratio
  int32_t pre, next;    //   pre_tokens, next_tokens clamped to kWindowCap
  int64_t stride;
  int32_t block_size;
  int32_t max_blocks;
  int32_t k;
  uint32_t bs_magic;  // floor(2^32 / block_size) + 1: j / block_size == umulhi(j, bs_magic) for j < 2^22
  int64_t d_row0, d_row1, d_cols;
  void* dots;
  float* dscores;
};

// Scale / weight element: fp16 (paired with int8 q/k) or fp32 (with fp8).
template <int QK>
__device__ __forceinline__ float load_scale(const void* base, int64_t i) {
  if constexpr (QK == QLI_QK_INT8)
    return (float)(static_cast<const _Float16*>(base)[i]);
  else
    return static_cast<const float*>(base)[i];
}

// Raw bits of a ScaleK element, converted only when staged to LDS.
template <int QK>
__device__ __forceinline__ uint32_t load_scale_bits(const void* base, int64_t i) {
  if constexpr (QK == QLI_QK_INT8)
    return static_cast<const uint16_t*>(base)[i];
  else
    return static_cast<const uint32_t*>(base)[i];
}
template <int QK>
__device__ __forceinline__ float scale_from_bits(uint32_t b) {
  if constexpr (QK == QLI_QK_INT8) {
    const uint16_t h = (uint16_t)b;
    return (float)__builtin_bit_cast(_Float16, h);
  } else {
    return __uint_as_float(b);
  }
}

// int8 epilogue without an int->float conversion.  A non-negative int32 d
// read as fp32 bits is the denormal d * 2^-149, exactly (|dot| <= 2^21).  With
// w' carried as w' * 2^95 (w' = W * ScaleQ < 2^32 for fp16 inputs, so it does
// not overflow) each product w' * 2^95 * d * 2^-149 = w' * d * 2^-54 is a
// normal float (w' >= 2^-48 when non-zero, d >= 1), so every fma rounds as it
// would on w' * d and the head sum is the same fp32 value times 2^-54; the
// 2^54 is folded into ScaleK.  The kernels run with fp32 denormals preserved
// (the code objects' float_denorm_mode_32 is 3), so the fma takes the denormal
// operand as it is: max + fma per (head, key) instead of max + convert + fma.
template <int QK>
__device__ constexpr float w_scale() { return QK == QLI_QK_INT8 ? 0x1p95f : 1.f; }
template <int QK>
__device__ constexpr float sk_scale() { return QK == QLI_QK_INT8 ? 0x1p54f : 1.f; }
__device__ __forceinline__ float relu_bits(int d) { return __int_as_float(max(d, 0)); }

// Sum over the four lane groups of per-lane partials, scattered so that lane
// (q, c) ends with the total of partial q: lane q*16 + c holds key q*16 + c
// of the 64-key tile (two permlane steps).
__device__ __forceinline__ float reduce_scatter4(float a0, float a1, float a2, float a3) {
  // halves: the lower 32 lanes keep partials 0/1, the upper 32 keep 2/3
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a2), false, false);
  auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(a1), __float_as_uint(a3), false, false);
  const float s02 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const float s13 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  // rows of 16: even rows keep the 0/2 partial, odd rows the 1/3 partial
  auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// The same for two partials: lanes of rows 0 and 1 end with the total of a0,
// rows 2 and 3 with the total of a1 (for key c of the respective n-tile).
__device__ __forceinline__ float reduce_scatter2(float a0, float a1) {
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
  const float s = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// One 32-byte operand fragment: for int8 the two halves feed two K=64
// MFMAs (dims [0,64) and [64,128)); for fp8 they form the v8i32 of one K=128
// MFMA.  Lane l covers matrix row/column l%16 and lane group q = l/16.
//   int8: lo = dims [16q, 16q+16), hi = dims [64+16q, 64+16q+16)
//   fp8:  lo = dims [32q, 32q+16), hi = dims [32q+16, 32q+32)
// A (query) and B (key) fragments use the same dim assignment, so each dot
// sums every dim exactly once.
struct Frag {
  v4i lo, hi;
};

template <int QK>
__device__ __forceinline__ int chunk_lo(int q) { return QK == QLI_QK_INT8 ? q : 2 * q; }
template <int QK>
__device__ __forceinline__ int chunk_hi(int q) { return QK == QLI_QK_INT8 ? q + 4 : 2 * q + 1; }

// Reductions over a wave.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Candidate decode chunks of the device-side split: 128, 256, .., kMaxChunk entries.
constexpr int kChunkSteps = kMaxChunk / 128;

// Workgroup barrier that orders LDS (waits for this wave's LDS accesses) but
// leaves outstanding global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Issue priority of this wave from its progress through the current item:
// 3 during the first quarter of its stages, down to 0 during the last.  Waves
// of equal priority issue oldest first, so without it the workgroups sharing
// a CU finish in dispatch order (three decode workgroups on equal items: the
// youngest ended up to 15 us after the oldest); with it a workgroup that has
// fallen behind outranks the ones ahead of it.  All waves of a workgroup are
// at the same stage, so they share the level.
__device__ __forceinline__ void progress_priority(int done, int total) {
  const int p = 3 - min(3, 4 * done / total);
  if (p == 3)
    __builtin_amdgcn_s_setprio(3);
  else if (p == 2)
    __builtin_amdgcn_s_setprio(2);
  else if (p == 1)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// w'[4m + i] = W * ScaleQ (times w_scale) for heads 16m + 4q + i of row r
// (i = 0..3 are consecutive, so one 8- or 16-byte load per tensor and m).
template <int QK>
__device__ __forceinline__ void load_wq(const ScoreParams& P, int64_t r, int q, float (&wq)[16]) {
  const int64_t e0 = r * kHeads + 4 * q;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    if constexpr (QK == QLI_QK_INT8) {
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      const h4 w = *reinterpret_cast<const h4*>(static_cast<const _Float16*>(P.weights) + e0 + 16 * m);
      const h4 sq = *reinterpret_cast<const h4*>(static_cast<const _Float16*>(P.q_scale) + e0 + 16 * m);
#pragma unroll
      for (int i = 0; i < 4; i++) wq[4 * m + i] = __builtin_fmaf((float)w[i] * w_scale<QK>(), (float)sq[i], 0.f);
    } else {
      const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(P.weights) + e0 + 16 * m);
      const float4 sq = *reinterpret_cast<const float4*>(static_cast<const float*>(P.q_scale) + e0 + 16 * m);
      wq[4 * m + 0] = w.x * sq.x;
      wq[4 * m + 1] = w.y * sq.y;
      wq[4 * m + 2] = w.z * sq.z;
      wq[4 * m + 3] = w.w * sq.w;
    }
  }
}


// ---------------------------------------------------------------------------
// Shared pieces: lane-group reductions, order keys, LDS-DMA, block selection
// ---------------------------------------------------------------------------

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);  // negative: all bits flip; else the sign bit is set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Direct-to-LDS loads, issued from inline assembly so that the compiler does
// not add waits for them: each lane's bytes land at m0 + lane * 16 (16-byte
// form) or in the lane's 4-byte slot m0 + lane * 4 (4- and 2-byte forms).
// Callers wait with wait_vm<N>() (vmcnt counts them with every other vector
// memory access; loads complete in issue order).
// These helpers write m0 behind the compiler's back.  That is sound only
// while no code in this file relies on m0 across them: gfx950 LDS accesses
// do not use it, and this file has no LDS-DMA builtins, s_sendmsg or
// dynamically indexed register arrays (the compiled code has no other m0
// access).  Code that adds one of those must switch these loads to
// __builtin_amdgcn_global_load_lds, whose m0 the compiler manages.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory");
}
__device__ __forceinline__ void dma2(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_ushort %0, off" ::"v"(g), "s"(m0) : "memory");
}
// The same from a workgroup-uniform base (an SGPR pair) plus a 32-bit byte
// offset per lane.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0) : "memory");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(m0) : "memory");
}
__device__ __forceinline__ void dma2s(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_ushort %0, %1" ::"v"(off), "s"(base), "s"(m0) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Exclusive prefix sum over the workgroup in thread order.
template <int NT>
__device__ int block_exclusive_scan(int v, int* tmp) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) before += w < wave ? tmp[w] : 0;
  __syncthreads();
  return before + incl - v;
}

// Bounded TND of at most kTndInKernelBatches batches: the batch partition of
// the T query rows from the device prefix sums, in one wave.  Batch b owns
// rows [end(b - 1), end(b)), end the running maximum of the prefix sums
// clamped to [0, T] (any input then partitions the rows; the first batch
// starts at row 0, rows from end(nb - 1) on belong to none).  Lane l holds
// e0 = end(2l) and e1 = end(2l + 1); past the last batch they repeat its end.
__device__ __forceinline__ void tnd_wave_ends(const int32_t* aslq, int nb, int t, int& e0, int& e1) {
  static_assert(kTndInKernelBatches == 128, "two batches per lane");
  const int lane = threadIdx.x & 63;
  const int b0 = 2 * lane;
  const int v0 = b0 < nb ? min(max(aslq[b0], 0), t) : 0;
  const int v1 = b0 + 1 < nb ? min(max(aslq[b0 + 1], 0), t) : 0;
  int incl = max(v0, v1);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl = max(incl, o);
  }
  int before = __shfl_up(incl, 1, 64);  // end of batch 2l - 1
  if (lane == 0) before = 0;
  e0 = max(before, v0);
  e1 = max(e0, v1);
}

// The value x of batch b (uniform, < 2 * 64) from the pair (x0, x1) that lane
// b / 2 holds for batches 2l, 2l + 1.
__device__ __forceinline__ int tnd_pick(int x0, int x1, int b) {
  return __builtin_amdgcn_readlane((b & 1) ? x1 : x0, b >> 1);
}

// Bounded runs: the entries [lo, hi) that query i of a batch (s1b used rows,
// skb key tokens after the clamp to the bound) sees under the token window
// (sides clamped to kWindowCap); without one lo = 0 and hi = visible_entries.
// Below 2^22 entries.
__device__ __forceinline__ int row_window(int mode, int cmp, int64_t skb, int s1b, int i, int pre, int next,
                                          int& lo) {
  int64_t l;
  const int64_t h = visible_window(mode, cmp, skb, s1b, i, pre, next, l);
  lo = (int)l;
  return (int)h;
}

// The entries that rows of one item see together: [start, end), start being
// the smallest lo of a row that sees something, rounded down to a multiple
// of kSpanAlign (whole stages), [0, 0) when no row does.  Chunks from start
// cover every row's range.
__device__ __forceinline__ int span_start(int lo_min, int hi_max) {
  return hi_max > 0 ? lo_min / kSpanAlign * kSpanAlign : 0;
}

// ---------------------------------------------------------------------------
// Top-k selection over staged scores.
// ---------------------------------------------------------------------------
//
// The n scores sit in the workspace, 16-byte aligned and readable up to n
// rounded up to 4.  Thread t owns the contiguous positions [t*S, t*S + S):
// up to 32768 scores are loaded once into registers as order keys (S = 4R
// per thread, R = 1, 2, 4 or 8); longer lists are re-read in every phase.
//
// Threshold: the bits every key shares are skipped, then radix passes of up
// to 11 bits histogram the keys that still match the threshold prefix (LDS
// atomics into one of two 2048-bin histograms, the other being cleared
// meanwhile); a block scan over the bins in descending digit order finds
// the digit of the kk-th largest key.  It stops once the threshold bin is
// taken whole or all 32 bits are fixed.  Three barriers per pass; cross-wave
// sums and reductions take one DPP row of 16 lanes.
// Emission: every key above the threshold and the kk lowest-positioned keys
// equal to it, each at its rank in position order (block scans of the
// per-thread counts).

// Inclusive prefix sum over the 64 lanes: DPP row shifts within rows of 16,
// then the row broadcasts.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// AND and OR over the 64 lanes (uniform results): DPP within rows of 16, then
// one lane per row.
__device__ __forceinline__ void wave_and_or(uint32_t& a, uint32_t& o) {
  int x = (int)a, y = (int)o;
  x &= __builtin_amdgcn_update_dpp(0, x, 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  y |= __builtin_amdgcn_update_dpp(0, y, 0xb1, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(0, x, 0x4e, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  y |= __builtin_amdgcn_update_dpp(0, y, 0x4e, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false);  // row_half_mirror
  y |= __builtin_amdgcn_update_dpp(0, y, 0x141, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false);  // row_mirror
  y |= __builtin_amdgcn_update_dpp(0, y, 0x140, 0xf, 0xf, false);
  a = (uint32_t)(__builtin_amdgcn_readlane(x, 0) & __builtin_amdgcn_readlane(x, 16) &
                 __builtin_amdgcn_readlane(x, 32) & __builtin_amdgcn_readlane(x, 48));
  o = (uint32_t)(__builtin_amdgcn_readlane(y, 0) | __builtin_amdgcn_readlane(y, 16) |
                 __builtin_amdgcn_readlane(y, 32) | __builtin_amdgcn_readlane(y, 48));
}

// Inclusive prefix sum over the 16 lanes of each row (row shifts only).
__device__ __forceinline__ int row_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}

// Per-wave totals tot[0 .. NW) (NW <= 16, published before a barrier): the
// sum over the waves below `wave` (uniform) and the sum over all of them.
template <int NW>
__device__ __forceinline__ void waves_prefix(const int* tot, int wave, int& below, int& total) {
  static_assert(NW <= 16, "one DPP row holds the wave totals");
  const int lane = threadIdx.x & 63;
  const int v = row_incl_scan(lane < NW ? tot[lane] : 0);
  const int b = __builtin_amdgcn_readlane(v, wave > 0 ? wave - 1 : 0);
  below = wave > 0 ? b : 0;
  total = __builtin_amdgcn_readlane(v, NW - 1);
}

// AND and OR of the per-wave values red[0][0 .. NW), red[1][0 .. NW) (uniform).
template <int NW>
__device__ __forceinline__ void waves_and_or(const uint32_t (*red)[16], uint32_t& a, uint32_t& o) {
  const int lane = threadIdx.x & 63;
  int x = lane < NW ? (int)red[0][lane] : -1, y = lane < NW ? (int)red[1][lane] : 0;
  x &= __builtin_amdgcn_update_dpp(0, x, 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  y |= __builtin_amdgcn_update_dpp(0, y, 0xb1, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(0, x, 0x4e, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  y |= __builtin_amdgcn_update_dpp(0, y, 0x4e, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false);  // row_half_mirror
  y |= __builtin_amdgcn_update_dpp(0, y, 0x141, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false);  // row_mirror
  y |= __builtin_amdgcn_update_dpp(0, y, 0x140, 0xf, 0xf, false);
  a = (uint32_t)__builtin_amdgcn_readlane(x, 0);
  o = (uint32_t)__builtin_amdgcn_readlane(y, 0);
}

struct SelShared {
  uint32_t red[2][16];  // per-wave AND / OR
  int wsum[2][16];      // per-wave scan totals
  int res[2][4];        // per-pass result: digit, keys above it, keys in it
};

// Exclusive prefix over the workgroup of two per-thread counts; also their totals.
template <int NT>
__device__ __forceinline__ void block_scan2(int x, int y, int& xb, int& yb, int& xt, int& yt, SelShared& sh) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int xi = wave_incl_scan(x), yi = wave_incl_scan(y);
  if (lane == 63) {
    sh.wsum[0][wave] = xi;
    sh.wsum[1][wave] = yi;
  }
  lds_barrier();
  int xw, yw;
  waves_prefix<NW>(sh.wsum[0], wave, xw, xt);
  waves_prefix<NW>(sh.wsum[1], wave, yw, yt);
  xb = xw + xi - x;
  yb = yw + yi - y;
}

// One radix pass over the keys that match the threshold prefix so far:
// histogram of the next digit, then the digit that holds the kk-th largest
// key.  count_into(H) adds every matching key's digit to the LDS histogram
// H; Hn (the other buffer) is cleared for the next pass.  Updates kk, mask,
// prefix and lo (uniform); false once the threshold bin is taken whole.
template <int NT, typename CountInto>
__device__ __forceinline__ bool radix_pass(int p, int& kk, uint32_t& mask, uint32_t& prefix, int& lo, int* hist,
                                           SelShared& sh, CountInto&& count_into) {
  constexpr int NW = NT / 64;
  constexpr int BPT = 2048 / NT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int width = lo < 11 ? lo : 11;
  const int shift = lo - width;
  const int nb = 1 << width;
  int* H = hist + (p & 1) * 2048;
  count_into(H, shift, nb - 1);
  int* Hn = hist + ((p + 1) & 1) * 2048;  // read last in pass p - 1, used by pass p + 1
  for (int b = tid; b < 2048; b += NT) Hn[b] = 0;
  lds_barrier();
  // Thread t owns digits nb-1-BPT*t .. nb-BPT*(t+1) (descending).
  int h[BPT];
  int local = 0;
#pragma unroll
  for (int jj = 0; jj < BPT; jj++) {
    const int d = nb - 1 - (BPT * tid + jj);
    h[jj] = d >= 0 ? H[d] : 0;
    local += h[jj];
  }
  const int incl = wave_incl_scan(local);
  if (lane == 63) sh.wsum[p & 1][wave] = incl;
  lds_barrier();
  int below, total;
  waves_prefix<NW>(sh.wsum[p & 1], wave, below, total);
  const int before = below + incl - local;
  if (before < kk && kk <= before + local) {
    int acc = before;
#pragma unroll
    for (int jj = 0; jj < BPT; jj++) {
      if (acc < kk && kk <= acc + h[jj]) {
        sh.res[p & 1][0] = nb - 1 - (BPT * tid + jj);
        sh.res[p & 1][1] = acc;
        sh.res[p & 1][2] = h[jj];
      }
      acc += h[jj];
    }
  }
  lds_barrier();
  const int digit = __builtin_amdgcn_readfirstlane(sh.res[p & 1][0]);
  const int above = __builtin_amdgcn_readfirstlane(sh.res[p & 1][1]);
  const int count = __builtin_amdgcn_readfirstlane(sh.res[p & 1][2]);
  kk -= above;
  prefix |= (uint32_t)digit << shift;
  mask |= (uint32_t)(nb - 1) << shift;
  lo = shift;
  return count != kk;
}

// Bits every key shares (a = AND, o = OR): the threshold search starts below them.
__device__ __forceinline__ void common_prefix(uint32_t a, uint32_t o, uint32_t& mask, uint32_t& prefix, int& lo) {
  const uint32_t diff = a ^ o;
  lo = diff == 0u ? 0 : 32 - __clz(diff);  // bits below lo still differ
  mask = lo == 32 ? 0u : ~((1u << lo) - 1u);
  prefix = a & mask;
}

// Top-k (k < n) of n fp32 scores read from global memory in every phase (for
// candidate lists too long to hold in registers); emit(pos, e, value) for
// each winner e with pos its rank in position order.  hist: 2 x 2048 ints.
// Thread t walks the contiguous positions [4*R*t, 4*R*t + 4*R).
template <int NT, typename Emit>
__device__ __forceinline__ void select_topk_global(const float* src, int n, int k, int* hist, SelShared& sh,
                                                   Emit&& emit) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (n + 4 * NT - 1) / (4 * NT);
  const int S = 4 * (g4 <= 1 ? 1 : 1 << (32 - __clz(g4 - 1)));
  const int beg = min(n, tid * S), end = min(n, beg + S);
  const int cnt = end - beg;
  auto group = [&](int j) __attribute__((always_inline)) {
    const float4 v = *reinterpret_cast<const float4*>(src + beg + j);
    return make_uint4(order_key(v.x), order_key(v.y), order_key(v.z), order_key(v.w));
  };

  uint32_t a = 0xFFFFFFFFu, o = 0u;
#pragma unroll 2
  for (int j = 0; j < cnt; j += 4) {
    const uint4 v = group(j);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
      a &= j + c < cnt ? q[c] : 0xFFFFFFFFu;
      o |= j + c < cnt ? q[c] : 0u;
    }
  }
  wave_and_or(a, o);
  if (lane == 0) {
    sh.red[0][wave] = a;
    sh.red[1][wave] = o;
  }
  for (int b = tid; b < 2048; b += NT) hist[b] = 0;
  lds_barrier();
  waves_and_or<NW>(sh.red, a, o);
  int kk = k, lo;
  uint32_t mask, prefix;
  common_prefix(a, o, mask, prefix, lo);
  for (int p = 0; lo > 0; p++) {
    auto count_into = [&](int* H, int shift, uint32_t dmask) __attribute__((always_inline)) {
#pragma unroll 2
      for (int j = 0; j < cnt; j += 4) {
        const uint4 v = group(j);
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; c++)
          if (j + c < cnt && (q[c] & mask) == prefix) atomicAdd(&H[(q[c] >> shift) & dmask], 1);
      }
    };
    if (!radix_pass<NT>(p, kk, mask, prefix, lo, hist, sh, count_into)) break;
  }

  int g = 0, q = 0;
#pragma unroll 2
  for (int j = 0; j < cnt; j += 4) {
    const uint4 v = group(j);
    const uint32_t f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const uint32_t m = f[c] & mask;
      g += (j + c < cnt && m > prefix) ? 1 : 0;
      q += (j + c < cnt && m == prefix) ? 1 : 0;
    }
  }
  int G, E, gt_total, eq_total;
  block_scan2<NT>(g, q, G, E, gt_total, eq_total, sh);
#pragma unroll 2
  for (int j = 0; j < cnt; j += 4) {
    const uint4 v = group(j);
    const uint32_t f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const uint32_t m = f[c] & mask;
      const bool live = j + c < cnt;
      const bool gt = live && m > prefix;
      const bool eq = live && m == prefix;
      if (gt || (eq && E < kk)) emit(G + min(E, kk), beg + j + c, key_value(f[c]));
      G += gt ? 1 : 0;
      E += eq ? 1 : 0;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode-shaped items: 1, 2 or 4 rows of one batch x a chunk of key entries.
// ---------------------------------------------------------------------------
//
// The chunk streams through a 3-stage LDS ring of 128-entry stages filled by
// direct-to-LDS loads (every wave issues exactly 4 key loads and 1 ScaleK
// load per stage, with addresses clamped into the chunk, so per-wave vmcnt
// arithmetic is exact); two stages are in flight while one is computed.
// Each wave scores its row against its n-tiles of the stage:
//   RT = 4: all 8 n-tiles, RT = 2: 4 n-tiles, RT = 1: 2 n-tiles.
template <int QK, int RT, bool DUMP, bool TILES = false, bool PLAN = false>
// Three workgroups per CU fit the LDS ring; the register budget follows (the
// dump instantiations, for parity checks only, keep two).  TILES: bounded
// runs of 4-row groups; PLAN: bounded decode planned in the kernel (planned
// runs carry neither).
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(DUMP ? 2 : 3))) void
score_decode_kernel(ScoreParams P) {
  static_assert(!TILES || (RT == kMaxItemRows && !DUMP), "4-row groups of bounded runs, no dump");
  static_assert(!PLAN || (!TILES && !DUMP), "in-kernel planning of bounded decode, no dump");
  constexpr int SC = 128;                     // entries per LDS stage
  static_assert(SC == kSpanAlign, "bounded items start on a stage");
  constexpr int NSTAGE = 3;
  constexpr int WPR = 4 / RT;                 // waves per row
  constexpr int NPW = 8 / WPR;                // n-tiles per wave per stage
  constexpr int KLOADS = SC * kDim / (kScoreThreads * 16);  // 4 key loads per thread per stage
  constexpr int PER_STAGE = KLOADS + 1;       // + the ScaleK load
  constexpr int SB = QK == QLI_QK_INT8 ? 2 : 4;

  __shared__ __attribute__((aligned(16))) uint8_t ring[NSTAGE][SC * kDim];
  __shared__ uint32_t ring_sk[NSTAGE][SC];   // ScaleK bits, one 4-byte slot per entry
  __shared__ int32_t lds_bt[kMaxChunk / 16 + 2];
  // bounded TND of few batches: row ends, then inclusive group ends (INT32_MAX
  // past the last batch), one entry per batch
  __shared__ __attribute__((aligned(8))) int32_t tnd_tab[TILES ? 2 * kTndInKernelBatches : 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;
  const int c16 = lane & 15;
  const int k = P.k;

  // Persistent workgroups over the work-sorted items, in snake order: round t
  // takes item t*G + b (t even) or t*G + G-1-b (t odd).
  const int G = gridDim.x;
  auto pos_of = [&](int t) { return t * G + ((t & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x); };
  const bool reg = !TILES && !PLAN && P.reg_chunks > 0;
  const int bs = P.block_size;
  const int u = wave / WPR;  // this wave's row of the item
  const int sub = wave % WPR;

  // State of the item being streamed (set by begin()).
  int batch = 0, key0 = 0, nkeys = 0, row0 = 0, nrows = 0, kend = 0, fb = 0;
  bool rok = false;
  int64_t r = 0;
  int rvis = 0, rlo = 0;  // this wave's row sees entries [rlo, rvis)
  int64_t coff = -1;
  // Padding deferred to the item's last stage: rows row0 + u (u < pad_n) get
  // slots [pad_from[u], k) once that stage's loads have landed, so no later
  // wait of the item drains these stores (vmcnt counts stores with loads, in
  // order), and the last stage's compute covers their latency.
  int pad_n = 0;
  int pad_from[kMaxItemRows];
  auto do_pad = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < kMaxItemRows; uu++) {
      if (uu >= pad_n) break;
      const int64_t rr = row0 + uu;
      for (int e = pad_from[uu] + tid; e < k; e += kScoreThreads) {
        P.idx_out[rr * k + e] = -1;
        if (P.val_out) P.val_out[rr * k + e] = -INFINITY;
      }
    }
    pad_n = 0;
  };
  Frag qa[4];
  float wq[16];
  int32_t* oi = nullptr;   // this row's outputs
  float* ov = nullptr;
  bool direct = false;     // the row sees at most k entries: scores go straight to the outputs
  bool whole = false;      // this item's stages each lie in one block (see issue)
  uint32_t koff[KLOADS];   // the lane's byte offsets of its stage loads within such a block
#pragma unroll
  for (int i = 0; i < KLOADS; i++) {
    const int kk = 8 * (4 * i + wave) + (lane >> 3);
    koff[i] = (uint32_t)(kk * kDim + (((lane & 7) ^ ((kk >> 1) & 7)) << 4));
  }
  const uint32_t skoff = (uint32_t)((32 * wave + (lane & 31)) * SB);

  // Bounded decode planned in the kernel (PLAN; P.plan_batches, at most one
  // batch per thread): thread t holds the entries [my_start, my_m) that batch
  // t's rows see (from entry 0 to the last used row's end without a window),
  // its used rows my_s1b and clamped key length my_skb; plan_items() picks
  // the chunk with the planner's rule (the smallest multiple of 128 entries
  // whose items fit the resident decode workgroups; for equal batches the one
  // that lowers the busiest CU's keys), gives each batch max(1,
  // ceil((my_m - my_start) / chunk)) items at the exclusive prefix my_first
  // and returns their number.  Every workgroup derives the same split; its
  // scratch lies in the ring, free until the first stage is issued.
  __shared__ int plan_sh[8];
  int my_m = 0, my_start = 0, my_s1b = 0, my_first = 0, my_n = 0, plan_chunk = 0;
  int64_t my_skb = 0;
  auto plan_items = [&]() {
    const int nb = P.plan_batches;
    if (tid < nb) {
      my_skb = min<int64_t>(max(P.aslk[tid], 0), P.max_len);
      my_s1b = P.aslq_bsnd ? min(max(P.aslq_bsnd[tid], 0), P.reg_rows) : P.reg_rows;
      int lo_min = INT32_MAX, hi_max = 0;
      for (int uu = 0; uu < my_s1b; uu++) {  // at most kMaxItemRows rows
        int lo;
        const int hi = row_window(P.mode, P.cmp, my_skb, my_s1b, uu, P.pre, P.next, lo);
        if (hi > lo) {
          lo_min = min(lo_min, lo);
          hi_max = max(hi_max, hi);
        }
      }
      my_start = span_start(lo_min, hi_max);
      my_m = hi_max;
    }
    int* sm = reinterpret_cast<int*>(&ring[0][0]);  // [256] the batches' spans
    int* part = sm + kScoreThreads;                 // [8][32] partial item counts
    int* pmm = part + kScoreThreads;                // [8] partial minima, [8] maxima
    int* scan_tmp = pmm + 16;                       // the block scan's
    sm[tid] = tid < nb ? my_m - my_start : 0;
    __syncthreads();
    {  // candidate chunk 128 (tid % 32 + 1) over batches tid / 32, tid / 32 + 8, ...
      static_assert(kChunkSteps == 32 && kScoreThreads == 256, "8 groups of the 32 candidates");
      const int c = 128 * ((tid & 31) + 1);
      int sum = 0, lo = INT32_MAX, hi = -1;
      for (int b = tid >> 5; b < nb; b += 8) {
        const int m = sm[b];
        sum += (m + c - 1) / c;
        lo = min(lo, m);
        hi = max(hi, m);
      }
      part[tid] = sum;
      if ((tid & 31) == 0) {
        pmm[tid >> 5] = lo;
        pmm[8 + (tid >> 5)] = hi;
      }
    }
    __syncthreads();
    if (wave == 0) {  // lane i < 32: candidate i's item count; the choice by ballot and a wave minimum
      const int i = lane & 31;
      int cnt = 0, lo = INT32_MAX, hi = -1;
#pragma unroll
      for (int g = 0; g < 8; g++) {
        cnt += part[32 * g + i];
        lo = min(lo, pmm[g]);
        hi = max(hi, pmm[8 + g]);
      }
      const unsigned long long fit = __ballot(lane < 32 && cnt <= kDecodeSlots);
      int best = fit ? __ffsll((long long)fit) - 1 : kChunkSteps - 1;
      if (hi >= 0 && lo == hi) {  // equal batches: the chunk >= best that lowers the busiest CU's keys
        // at most about 2^22 + 2^13 (256 batches of 2^22 entries): busiest * 32 + i fits 32 bits
        const int busiest = (cnt + kCUs - 1) / kCUs * (128 * (i + 1));
        best = wave_min(lane < 32 && i >= best ? busiest * 32 + i : INT32_MAX) & 31;
      }
      if (lane == 0) plan_sh[6] = best;
    }
    __syncthreads();
    const int best = plan_sh[6];
    plan_chunk = 128 * (best + 1);
    my_n = tid < nb ? max(1, (my_m - my_start + plan_chunk - 1) / plan_chunk) : 0;
    my_first = block_exclusive_scan<kScoreThreads>(my_n, scan_tmp);
    if (tid == kScoreThreads - 1) plan_sh[7] = my_first + my_n;
    __syncthreads();
    return plan_sh[7];
  };

  // Rows of an item that see fewer than k entries: slots count..k-1 are
  // -1 / -inf, written by do_pad.
  auto note_pad = [&](const Item& itp) __attribute__((always_inline)) {
    if (itp.flags & kItemPad) {
      pad_n = itp.nrows;
#pragma unroll
      for (int uu = 0; uu < kMaxItemRows; uu++) pad_from[uu] = uu < itp.nrows ? itp.vis[uu] - itp.lo[uu] : k;
    }
  };

  // Stage loader: wave w's load i fills stage bytes [(4i + w) * 1024, +1024),
  // lane l the 16 bytes at l*16: entry kk = 8(4i + w) + l/8, physical chunk
  // l%8 holding logical chunk (l%8) ^ ((kk>>1)&7) (conflict-free MFMA reads).
  // When a stage lies in one block (block size a multiple of SC and the
  // item's chunk starting at a multiple of SC), every load takes the block's
  // address as a uniform base plus the lane's fixed offset (koff, skoff):
  // one block-table lookup per stage instead of one per lane and load.  A
  // last, partial stage then reads past the chunk's end only inside the same
  // block; those entries are never scored.
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int slot_ = st % NSTAGE;
    const int e_base = key0 + st * SC;
    if (whole) {
      const int b = (int)__umulhi((uint32_t)e_base, P.bs_magic);
      const int blk = __builtin_amdgcn_readfirstlane(lds_bt[b - fb]);
      const int64_t at = (int64_t)blk * bs + (e_base - b * bs);  // the stage's first entry in the cache
      const uint8_t* kb = P.key + (int64_t)blk * P.stride + (int64_t)(e_base - b * bs) * kDim;
#pragma unroll
      for (int i = 0; i < KLOADS; i++)
        dma16s(kb, koff[i], __builtin_amdgcn_readfirstlane(lds_addr(&ring[slot_][(4 * i + wave) * 1024])));
      if (lane < 32) {
        const uint8_t* sb = static_cast<const uint8_t*>(P.k_scale) + at * SB;
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(&ring_sk[slot_][32 * wave]));
        if constexpr (SB == 2)
          dma2s(sb, skoff, m0);
        else
          dma4s(sb, skoff, m0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < KLOADS; i++) {
      const int kk = 8 * (4 * i + wave) + (lane >> 3);
      const int j = min(e_base + kk, kend - 1);
      const int b = (int)__umulhi((uint32_t)j, P.bs_magic);
      const int blk = lds_bt[b - fb];
      const int c = (lane & 7) ^ ((kk >> 1) & 7);
      const uint8_t* src = P.key + (int64_t)blk * P.stride + (j - b * bs) * kDim + c * 16;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(&ring[slot_][(4 * i + wave) * 1024])));
    }
    if (lane < 32) {  // entries 32w .. 32w + 31 of the stage
      const int j = min(e_base + 32 * wave + lane, kend - 1);
      const int b = (int)__umulhi((uint32_t)j, P.bs_magic);
      const uint8_t* src = static_cast<const uint8_t*>(P.k_scale) +
                           ((int64_t)lds_bt[b - fb] * bs + (j - b * bs)) * SB;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(&ring_sk[slot_][32 * wave]));
      if constexpr (SB == 2)
        dma2(src, m0);
      else
        dma4(src, m0);
    }
  };


  // Starts item pos: its fields (from the position for regular plans, so the
  // loads below need not wait for the item), its block-table slice in LDS,
  // this wave's query fragments and w' = W * ScaleQ, and the loads of its
  // stages 0 and 1.  False for an item without keys (padding only).
  auto begin = [&](int pos) __attribute__((always_inline)) {
    const Item* itp = P.items + pos;  // a plan's table or the one the bounded run built on the device
    if constexpr (TILES) {
      // bounded runs of 4-row groups: chunk pos % reg_chunks of group
      // pos / reg_chunks (BSND: ceil(reg_rows / 4) groups per batch; TND:
      // through the tables, the groups past the real ones covering the rows
      // that belong to no batch, which only receive padding)
      int g = pos / P.reg_chunks;
      const int cidx = pos - g * P.reg_chunks;  // the chunk's index from the group's start
      int b, rstart, s1b;
      if (P.aslq_tnd) {
        // the batch of group g: the number of batches whose groups all lie
        // before it (the wave's lanes hold two group ends each)
        const int2 ge = *reinterpret_cast<const int2*>(&tnd_tab[kTndInKernelBatches + 2 * lane]);
        b = (int)(__popcll(__ballot(ge.x <= g)) + __popcll(__ballot(ge.y <= g)));
        const int nb = P.nbatch;
        const int last = b < nb ? b : nb;  // rows and groups before those of batch `last`
        rstart = last > 0 ? tnd_tab[last - 1] : 0;
        g -= last > 0 ? tnd_tab[kTndInKernelBatches + last - 1] : 0;
        if (b < nb) {
          s1b = tnd_tab[b] - rstart;
        } else {  // past the real groups: rows that belong to no batch
          b = -1;
          s1b = P.trows - rstart;
        }
      } else if (P.rows_end) {
        const int real = P.group_start[P.nbatch];
        if (g < real) {
          b = P.group_batch[g];
          rstart = b > 0 ? P.rows_end[b - 1] : 0;
          s1b = P.rows_end[b] - rstart;
          g -= P.group_start[b];
        } else {
          b = -1;
          rstart = P.nbatch > 0 ? P.rows_end[P.nbatch - 1] : 0;
          s1b = P.trows - rstart;
          g -= real;
        }
      } else {
        const int per = (P.reg_rows + kMaxItemRows - 1) / kMaxItemRows;
        b = g / per;
        g -= b * per;
        rstart = b * P.reg_rows;
        s1b = P.reg_rows;
      }
      // query rows of the batch in use (BSND counts), its clamped key length
      const int s1q = P.aslq_bsnd && b >= 0 ? min(max(P.aslq_bsnd[b], 0), s1b) : s1b;
      const int64_t skb = b >= 0 ? min<int64_t>(max(P.aslk[b], 0), P.max_len) : 0;
      batch = b;
      row0 = rstart + kMaxItemRows * g;
      nrows = max(0, min(kMaxItemRows, s1b - kMaxItemRows * g));
      // row uu's entries [lo, hi): none past the batch's used rows
      auto range_of = [&](int uu, int& lo) {
        const int i = kMaxItemRows * g + uu;
        lo = 0;
        return uu < nrows && b >= 0 && i < s1q ? row_window(P.mode, P.cmp, skb, s1q, i, P.pre, P.next, lo) : 0;
      };
      int lo_min = INT32_MAX, maxv = 0, pad_to[kMaxItemRows];
#pragma unroll
      for (int uu = 0; uu < kMaxItemRows; uu++) {
        int lo;
        const int hi = range_of(uu, lo);
        pad_to[uu] = hi - lo;
        if (hi > lo) {
          lo_min = min(lo_min, lo);
          maxv = max(maxv, hi);
        }
      }
      key0 = span_start(lo_min, maxv) + cidx * P.chunk;
      nkeys = min(P.chunk, maxv - key0);
      if (cidx == 0) {  // the group's first chunk pads its rows
        pad_n = nrows;
#pragma unroll
        for (int uu = 0; uu < kMaxItemRows; uu++) pad_from[uu] = uu < nrows ? pad_to[uu] : k;
      }
      if (nkeys <= 0) {  // uniform across the workgroup
        do_pad();
        return false;
      }
      rok = u < nrows;
      r = row0 + (rok ? u : 0);
      int lo_u;
      rvis = rok ? range_of(u, lo_u) : 0;
      rlo = rok ? lo_u : 0;
      coff = rvis - rlo > k ? r * P.bstride + key0 - rlo : -1;  // entry j at slot j - lo of the row
    } else if constexpr (PLAN) {
      // bounded decode planned in the kernel: the thread of the batch whose
      // items hold pos publishes the item; the ring is free here
      if (tid < P.plan_batches && pos >= my_first && pos < my_first + my_n) {
        plan_sh[0] = tid;
        plan_sh[1] = pos - my_first;
        plan_sh[2] = my_m;
        plan_sh[3] = my_s1b;
        plan_sh[4] = (int)my_skb;  // clamped to the bound, below kMaxEntries * 128 = 2^29
        plan_sh[5] = my_start;
      }
      __syncthreads();
      batch = plan_sh[0];
      const int idx = plan_sh[1];
      const int m = plan_sh[2], s1b = plan_sh[3];
      const int64_t skb = plan_sh[4];
      key0 = plan_sh[5] + idx * plan_chunk;
      __syncthreads();  // read by every thread before the next item's owner writes them
      nkeys = min(plan_chunk, m - key0);
      row0 = batch * P.reg_rows;
      nrows = P.reg_rows;
      // the row's entries [lo, hi): none past the batch's used rows
      auto range_of = [&](int uu, int& lo) {
        lo = 0;
        return uu < s1b ? row_window(P.mode, P.cmp, skb, s1b, uu, P.pre, P.next, lo) : 0;
      };
      if (idx == 0) {  // the batch's first item pads its rows
        pad_n = nrows;
#pragma unroll
        for (int uu = 0; uu < kMaxItemRows; uu++) {
          int lo;
          const int hi = range_of(uu, lo);
          pad_from[uu] = uu < nrows ? hi - lo : k;
        }
      }
      if (nkeys <= 0) {  // uniform across the workgroup
        do_pad();
        return false;
      }
      rok = u < nrows;
      r = row0 + (rok ? u : 0);
      int lo_u;
      rvis = rok ? range_of(u, lo_u) : 0;
      rlo = rok ? lo_u : 0;
      coff = rvis - rlo > k ? r * P.bstride + key0 - rlo : -1;  // entry j at slot j - lo of the row
    } else if (reg) {
      batch = pos / P.reg_chunks;
      key0 = (pos - batch * P.reg_chunks) * P.chunk;
      nkeys = min(P.chunk, P.reg_maxv - key0);
      row0 = batch * P.reg_rows;
      nrows = P.reg_rows;
      note_pad(*itp);
    } else {
      note_pad(*itp);
      batch = itp->batch;
      key0 = itp->key0;
      nkeys = itp->nkeys;
      row0 = itp->row0;
      nrows = itp->nrows;
      if (nkeys <= 0) {  // uniform across the workgroup
        do_pad();
        return false;
      }
    }
    kend = key0 + nkeys;
    fb = (int)__umulhi((uint32_t)key0, P.bs_magic);
    whole = (bs % SC) == 0 && (key0 % SC) == 0;
    const int nblk = (int)__umulhi((uint32_t)(kend - 1), P.bs_magic) - fb + 1;
    // Block-table slice (nblk <= kMaxChunk / 16 + 2 <= 2 * kScoreThreads
    // entries): loaded now, written to LDS once the query and weight loads
    // below have been issued, so the three round trips overlap.
    static_assert(kMaxChunk / 16 + 2 <= 2 * kScoreThreads, "two block-table entries per thread");
    const int32_t* bt = P.block_table + (int64_t)batch * P.max_blocks + fb;
    const int bt0 = tid < nblk ? bt[tid] : 0;
    const int bt1 = tid + kScoreThreads < nblk ? bt[tid + kScoreThreads] : 0;
    if constexpr (!TILES && !PLAN) {
      rok = u < nrows;
      r = row0 + (rok ? u : 0);
      rvis = rok ? itp->vis[u] : 0;
      rlo = rok ? itp->lo[u] : 0;
      coff = rok ? itp->cand_off[u] : -1;
    }
    {
      const uint8_t* qrow = P.query + r * (kHeads * kDim);
  #pragma unroll
      for (int m = 0; m < 4; m++) {
        const uint8_t* qh = qrow + (16 * m + c16) * kDim;
        qa[m].lo = *reinterpret_cast<const v4i*>(qh + 16 * chunk_lo<QK>(q));
        qa[m].hi = *reinterpret_cast<const v4i*>(qh + 16 * chunk_hi<QK>(q));
      }
    }
    load_wq<QK>(P, r, q, wq);
    if (tid < nblk) lds_bt[tid] = bt0;
    if (tid + kScoreThreads < nblk) lds_bt[tid + kScoreThreads] = bt1;
    lds_barrier();  // lds_bt ready
    issue(0);
    if (nkeys > SC) issue(1);
    return true;
  };

  // Scores of 64 entries (4 n-tiles) or 32 entries (2 n-tiles) of the stage.
  auto score_group = [&](int slot_, int st, int n0, auto nt_) __attribute__((always_inline)) {
    constexpr int NTL = decltype(nt_)::value;
    float part[NTL];
#pragma unroll
    for (int n = 0; n < NTL; n++) {
      const int kk = (n0 + n) * 16 + c16;
      const uint8_t* krow = &ring[slot_][kk * kDim];
      const int sw = (kk >> 1) & 7;
      Frag b;
      b.lo = *reinterpret_cast<const v4i*>(krow + ((chunk_lo<QK>(q) ^ sw) << 4));
      b.hi = *reinterpret_cast<const v4i*>(krow + ((chunk_hi<QK>(q) ^ sw) << 4));
      float acc = 0.f;
      v4i di[4];
      v4f df[4];
      if constexpr (QK == QLI_QK_INT8) {
#pragma unroll
        for (int m = 0; m < 4; m++) {
          di[m] = v4i{0, 0, 0, 0};
          di[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[m].lo, b.lo, di[m], 0, 0, 0);
          di[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[m].hi, b.hi, di[m], 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) acc = __builtin_fmaf(wq[4 * m + i], relu_bits(di[m][i]), acc);
      } else {
        const v8i bb = __builtin_shufflevector(b.lo, b.hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int m = 0; m < 4; m++) {
          const v8i aa = __builtin_shufflevector(qa[m].lo, qa[m].hi, 0, 1, 2, 3, 4, 5, 6, 7);
          df[m] = v4f{0.f, 0.f, 0.f, 0.f};
          // format 0 (fp8 e4m3) for both operands; scale arguments 0 select the unscaled form
          df[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, df[m], 0, 0, 0, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) acc = __builtin_fmaf(wq[4 * m + i], __builtin_fmaxf(df[m][i], 0.f), acc);
      }
      part[n] = acc;
      if constexpr (DUMP) {
        const int j = key0 + st * SC + kk;
        if (r >= P.d_row0 && r < P.d_row1 && j >= rlo && j < rvis && j < P.d_cols) {
          const int64_t base = (r - P.d_row0) * kHeads;
#pragma unroll
          for (int m = 0; m < 4; m++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int64_t o = (base + 16 * m + 4 * q + i) * P.d_cols + j;
              if constexpr (QK == QLI_QK_INT8)
                static_cast<int32_t*>(P.dots)[o] = di[m][i];
              else
                static_cast<float*>(P.dots)[o] = df[m][i];
            }
        }
      }
    }
    float total;
    int kk;
    bool owner;
    if constexpr (NTL == 4) {
      total = reduce_scatter4(part[0], part[1], part[2], part[3]);
      kk = n0 * 16 + lane;
      owner = true;
    } else {
      total = reduce_scatter2(part[0], part[1]);
      kk = (n0 + (q >> 1)) * 16 + c16;
      owner = (q & 1) == 0;  // rows 0 and 2 hold the two totals
    }
    const int e = st * SC + kk;  // entry within the chunk
    const int j = key0 + e;
    const float score = total * (scale_from_bits<QK>(ring_sk[slot_][kk]) * sk_scale<QK>());
    if (owner && j >= rlo && j < rvis) {
      if (direct) {
        oi[j - rlo] = j;
        if (ov) ov[j - rlo] = score;
      } else {
        P.ws[coff + e] = score;
      }
      if constexpr (DUMP) {
        if (r >= P.d_row0 && r < P.d_row1 && j < P.d_cols) P.dscores[(r - P.d_row0) * P.d_cols + j] = score;
      }
    }
  };


  int n_items = P.n_items_dev ? *P.n_items_dev : P.n_items;
  if constexpr (PLAN) n_items = plan_items();
  if constexpr (TILES) {
    if (P.aslq_tnd) {  // the partition's tables, once per workgroup
    if (wave == 0) {
      int e0, e1;
      tnd_wave_ends(P.aslq_tnd, P.nbatch, P.trows, e0, e1);
      int before = __shfl_up(e1, 1, 64);
      if (lane == 0) before = 0;
      const int g0 = (e0 - before + kMaxItemRows - 1) / kMaxItemRows;  // groups of batches 2l, 2l + 1
      const int g1 = (e1 - e0 + kMaxItemRows - 1) / kMaxItemRows;
      const int ge1 = wave_incl_scan(g0 + g1);
      const int b0 = 2 * lane;
      *reinterpret_cast<int2*>(&tnd_tab[b0]) = int2{e0, e1};
      *reinterpret_cast<int2*>(&tnd_tab[kTndInKernelBatches + b0]) =
          int2{b0 < P.nbatch ? ge1 - g1 : INT32_MAX, b0 + 1 < P.nbatch ? ge1 : INT32_MAX};
    }
    __syncthreads();
    }
  }
  for (int round = 0;; round++) {
  const int pos = pos_of(round);
  if (pos >= n_items) break;  // uniform; positions grow with the round
  if (!begin(pos)) continue;
  const int nstages = (nkeys + SC - 1) / SC;
  oi = P.idx_out + r * k;
  ov = P.val_out ? P.val_out + r * k : nullptr;
  direct = rvis - rlo <= k;

  // Pipeline: stages st+1 and st+2 are in flight while st is computed.
  for (int st = 0; st < nstages; st++) {
    progress_priority(st, nstages);
    if (st + 2 < nstages) issue(st + 2);
    const int newer = min(st + 2, nstages - 1) - st;  // stages issued after st
    if (newer >= 2)
      wait_vm<2 * PER_STAGE>();
    else if (newer == 1)
      wait_vm<PER_STAGE>();
    else
      wait_vm<0>();
    lds_barrier();  // every wave's loads of stage st have landed
    if (st == nstages - 1 && pad_n > 0) do_pad();
    const int slot_ = st % NSTAGE;
    const int sbase = key0 + st * SC;
    if (rok && sbase < rvis) {
      if constexpr (NPW == 8) {
        score_group(slot_, st, 0, std::integral_constant<int, 4>{});
        if (sbase + 64 < rvis) score_group(slot_, st, 4, std::integral_constant<int, 4>{});
      } else if constexpr (NPW == 4) {
        if (sbase + 64 * sub < rvis) score_group(slot_, st, 4 * sub, std::integral_constant<int, 4>{});
      } else {
        if (sbase + 32 * sub < rvis) score_group(slot_, st, 2 * sub, std::integral_constant<int, 2>{});
      }
    }
    lds_barrier();  // the slot is free for stage st + 3
  }

  }  // rounds (the item's last barrier leaves the LDS free for the next one)
}

// ---------------------------------------------------------------------------
// Selection stage: one workgroup of 1024 threads per entry of the plan's
// selection table, over candidates staged in ascending position order.
// ---------------------------------------------------------------------------

constexpr int kSelThreads = 1024;  // 16 waves: the phases are latency-bound, more waves hide it
constexpr int kSelSmallThreads = 256;  // selections of at most 4 * 256 candidates
constexpr int kSelRegMax = 4 * 8 * kSelThreads;  // candidates held in registers (8 float4 per thread)

struct SelectParams {
  const SelectEntry* rows;  // this pass's entries of the plan's selection table
  float* ws;
  int32_t* ws_idx;
  int32_t* idx_out;
  float* val_out;
  int32_t k;
  // Bounded runs (aslk != null): no table; workgroup w of pass 1 takes
  // segment w / nrows of row w % nrows (every row's first segment, which exists
  // whenever the row is staged, is dispatched before any later one), workgroup
  // r of pass 2 the merge of row r.
  const int32_t* aslk;
  int64_t max_len, stride, mstride, merge_base;
  int32_t pre, next;  // pre_tokens, next_tokens clamped to kWindowCap
  int32_t s1, mode, cmp, nseg, pass;
  int32_t nrows;      //   output rows
  const int32_t* rows_end;   // bounded TND of many batches: the tables (TndTables), else null
  const int32_t* row_batch;
  const int32_t* aslq_tnd;   // bounded TND of few batches: the device prefix sums, else null
  int32_t nbatch;            //   their count
  const int32_t* aslq_bsnd;  // bounded BSND: per-batch query counts, else null (all S1 rows)
};

// The selection of this workgroup in bounded decode, from the row's key
// length: false if there is none (the row sees at most k entries, or fewer
// segments, or needs no merge).  Row r's scores sit at r * stride in key
// order; segment s keeps its winners at merge_base + r * mstride + s * k, so
// a row's merge candidates are contiguous (every segment but the last holds
// kSelSegment >= k scores).
__device__ __forceinline__ bool bounded_entry(const SelectParams& S, SelectEntry& se) {
  const int w = (int)blockIdx.x;
  const int s = S.pass == 1 ? w / S.nrows : 0;  // segment-major: every row's first segment goes first
  const int r = S.pass == 1 ? w - s * S.nrows : w;
  int b, i, s1b;
  if (S.aslq_tnd) {  // TND of few batches: the row's batch derived by each wave
    int e0, e1;
    tnd_wave_ends(S.aslq_tnd, S.nbatch, S.s1, e0, e1);
    const int lane = threadIdx.x & 63;
    b = (int)(__popcll(__ballot(2 * lane < S.nbatch && e0 <= r)) +
              __popcll(__ballot(2 * lane + 1 < S.nbatch && e1 <= r)));
    if (b >= S.nbatch) return false;  // rows of no batch need no selection
    const int rstart = b > 0 ? tnd_pick(e0, e1, b - 1) : 0;
    s1b = tnd_pick(e0, e1, b) - rstart;
    i = r - rstart;
  } else if (S.row_batch) {  // TND: the row's batch from the tables; rows of no batch need no selection
    b = S.row_batch[r];
    if (b < 0) return false;
    const int rstart = b > 0 ? S.rows_end[b - 1] : 0;
    s1b = S.rows_end[b] - rstart;
    i = r - rstart;
  } else {
    b = r / S.s1;
    s1b = S.s1;
    i = r - b * S.s1;
    if (S.aslq_bsnd) {  // rows past the batch's query count see nothing
      s1b = min(max(S.aslq_bsnd[b], 0), S.s1);
      if (i >= s1b) return false;
    }
  }
  const int64_t skb = min<int64_t>(max(S.aslk[b], 0), S.max_len);
  int lo;
  const int nv = row_window(S.mode, S.cmp, skb, s1b, i, S.pre, S.next, lo) - lo;  // entries lo.. at slots 0..
  if (nv <= S.k) return false;
  const int nsr = (nv + kSelSegment - 1) / kSelSegment;  // segments of this row
  se.row = r;
  se.base = lo;
  se.indexed = 0;
  se.dst_off = -1;
  if (S.pass == 2) {
    if (nsr == 1) return false;
    se.src_off = S.merge_base + (int64_t)r * S.mstride;
    se.n = (nsr - 1) * S.k + min(S.k, nv - (nsr - 1) * kSelSegment);
    se.base = 0;  // the candidates carry their key indices
    se.indexed = 1;
    return true;
  }
  if (nsr == 1) {
    se.src_off = (int64_t)r * S.stride;
    se.n = nv;
    return s == 0;
  }
  if (s >= nsr) return false;
  se.src_off = (int64_t)r * S.stride + (int64_t)s * kSelSegment;
  se.dst_off = S.merge_base + (int64_t)r * S.mstride + (int64_t)s * S.k;
  se.n = min(kSelSegment, nv - s * kSelSegment);
  se.base = lo + s * kSelSegment;
  return true;
}

// Where an entry's winners go: a row of the outputs, or (for a later merge)
// indexed candidates in the workspace.
struct SelectDst {
  int32_t* idx;
  float* val;  // may be null for a final row without values
  __device__ SelectDst(const SelectEntry& se, const SelectParams& S) {
    if (se.dst_off < 0) {
      idx = S.idx_out + (int64_t)se.row * S.k;
      val = S.val_out ? S.val_out + (int64_t)se.row * S.k : nullptr;
    } else {
      idx = S.ws_idx + se.dst_off;
      val = S.ws + se.dst_off;
    }
  }
  __device__ void put(int pos, int32_t key, float v) const {
    idx[pos] = key;
    if (val) val[pos] = v;
  }
};

// Up to 4*R*NT candidates: thread t loads positions [4R*t, 4R*t + 4R) once as
// order keys (and key indices when indexed) into registers; the winners are
// ranked into LDS and written out coalesced.
template <int NT, int R>
__global__ __launch_bounds__(NT) void select_reg_kernel(SelectParams S) {
  constexpr int NW = NT / 64;
  constexpr int SPT = 4 * R;
  __shared__ __attribute__((aligned(16))) int hist[2 * 2048];  // the histograms, then the ranked winners
  __shared__ SelShared sh;
  SelectEntry se;
  if (S.aslk) {
    if (!bounded_entry(S, se)) return;  // uniform
  } else {
    se = S.rows[blockIdx.x];
  }
  const int n = se.n;
  const int k = min(S.k, n);
  const float* sc = S.ws + se.src_off;
  const int32_t* ix = S.ws_idx + se.src_off;
  const bool indexed = se.indexed != 0;
  const SelectDst dst(se, S);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (n <= k) {  // every candidate is kept (a short last segment)
    for (int e = tid; e < n; e += NT) dst.put(e, indexed ? ix[e] : se.base + e, sc[e]);
    return;
  }
  const int beg = tid * SPT;
  const int cnt = max(0, min(SPT, n - beg));
  const bool full = (wave + 1) * 64 * SPT <= n;  // uniform: every position of this wave is a candidate

  float4 v[R];
  int4 w[R];
#pragma unroll
  for (int i = 0; i < R; i++) {
    const bool in = beg + 4 * i < n;  // the region is readable up to n rounded up to 4
    v[i] = in ? *reinterpret_cast<const float4*>(sc + beg + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
    w[i] = in && indexed ? *reinterpret_cast<const int4*>(ix + beg + 4 * i) : make_int4(0, 0, 0, 0);
  }
  uint32_t q[SPT];  // order keys; 0 (below every finite score) past n
  int32_t id[SPT];
  uint32_t a = 0xFFFFFFFFu, o = 0u;
#pragma unroll
  for (int i = 0; i < R; i++) {
    const float f[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    const int32_t g[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const int j = 4 * i + c;
      const bool live = j < cnt;
      q[j] = live ? order_key(f[c]) : 0u;
      id[j] = indexed ? g[c] : se.base + beg + j;
      a &= live ? q[j] : 0xFFFFFFFFu;
      o |= q[j];
    }
  }
  wave_and_or(a, o);
  if (lane == 0) {
    sh.red[0][wave] = a;
    sh.red[1][wave] = o;
  }
  for (int b = tid; b < 2048; b += NT) hist[b] = 0;
  lds_barrier();
  waves_and_or<NW>(sh.red, a, o);
  int kk = k, lo;
  uint32_t mask, prefix;
  common_prefix(a, o, mask, prefix, lo);
  for (int p = 0; lo > 0; p++) {
    auto count_into = [&](int* H, int shift, uint32_t dmask) __attribute__((always_inline)) {
      if (full) {
#pragma unroll
        for (int j = 0; j < SPT; j++)
          if ((q[j] & mask) == prefix) atomicAdd(&H[(q[j] >> shift) & dmask], 1);
      } else {
#pragma unroll
        for (int j = 0; j < SPT; j++)
          if (j < cnt && (q[j] & mask) == prefix) atomicAdd(&H[(q[j] >> shift) & dmask], 1);
      }
    };
    if (!radix_pass<NT>(p, kk, mask, prefix, lo, hist, sh, count_into)) break;
  }

  // Keys above the threshold and keys equal to it, as bit masks over j.
  uint32_t gm = 0u, em = 0u;
#pragma unroll
  for (int j = 0; j < SPT; j++) {
    const uint32_t m = q[j] & mask;
    gm |= (m > prefix ? 1u : 0u) << j;
    em |= (m == prefix && (full || j < cnt) ? 1u : 0u) << j;
  }
  int G, E, gt_total, eq_total;
  block_scan2<NT>(__builtin_popcount(gm), __builtin_popcount(em), G, E, gt_total, eq_total, sh);
  int* rank_idx = hist;  // the histograms are no longer read
  float* rank_val = reinterpret_cast<float*>(hist + 2048);
#pragma unroll
  for (int j = 0; j < SPT; j++) {
    const bool gt = (gm >> j) & 1u, eq = (em >> j) & 1u;
    if (gt || (eq && E < kk)) {
      const int pos = G + min(E, kk);
      rank_idx[pos] = id[j];
      rank_val[pos] = key_value(q[j]);
    }
    G += gt ? 1 : 0;
    E += eq ? 1 : 0;
  }
  lds_barrier();
  for (int e = tid; e < k; e += NT) dst.put(e, rank_idx[e], rank_val[e]);
}

// Longer candidate lists: every phase re-reads the scores from the workspace.
template <int NT>
__global__ __launch_bounds__(NT) void select_global_kernel(SelectParams S) {
  __shared__ int hist[2 * 2048];
  __shared__ SelShared sh;
  SelectEntry se;
  if (S.aslk) {
    if (!bounded_entry(S, se)) return;  // uniform
  } else {
    se = S.rows[blockIdx.x];
  }
  const int n = se.n;
  const int k = min(S.k, n);
  const float* sc = S.ws + se.src_off;
  const int32_t* ix = S.ws_idx + se.src_off;
  const bool indexed = se.indexed != 0;
  const SelectDst dst(se, S);
  if (n <= k) {
    for (int e = threadIdx.x; e < n; e += NT) dst.put(e, indexed ? ix[e] : se.base + e, sc[e]);
    return;
  }
  select_topk_global<NT>(sc, n, k, hist, sh, [&](int pos, int e, float v) __attribute__((always_inline)) {
    dst.put(pos, indexed ? ix[e] : se.base + e, v);
  });
}

// Workgroups of `kernel` that the current device holds at once (all CUs),
// cached per device and kernel in a fixed table (no allocation after the
// first query); 0 if it cannot be determined.
int resident_slots(const void* kernel, int threads) {
  struct Slot {
    int dev;
    const void* kernel;
    int slots;
  };
  static std::mutex mu;
  static Slot cache[256];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; i++)
    if (cache[i].dev == dev && cache[i].kernel == kernel) return cache[i].slots;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  const int slots = cus * per_cu;
  if (used < 256) cache[used++] = Slot{dev, kernel, slots};
  return slots;
}

template <typename... Args>
hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t st, Args... args) {
  hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  return hipGetLastError();
}

template <int QK, bool DUMP>
hipError_t launch_score_t(const ScoreParams& P, const PlanHeader* h, hipStream_t st) {
  const dim3 block(kScoreThreads);
  auto go = [&](void (*kern)(ScoreParams)) {
    const int slots = resident_slots(reinterpret_cast<const void*>(kern), kScoreThreads);
    const dim3 pgrid(slots > 0 ? std::min<int>(h->n_items, slots) : h->n_items);
    return launch(kern, pgrid, block, st, P);
  };
  if (P.tiles) {  // bounded runs of 4-row groups (never dumped)
    if constexpr (DUMP) return hipErrorInvalidValue;
    else return go(score_decode_kernel<QK, kMaxItemRows, false, true>);
  }
  if (P.plan_batches > 0) {  // bounded decode planned in the kernel (never dumped)
    if constexpr (DUMP) {
      return hipErrorInvalidValue;
    } else {
      switch (h->rows_per_item) {
        case 1: return go(score_decode_kernel<QK, 1, false, false, true>);
        case 2: return go(score_decode_kernel<QK, 2, false, false, true>);
        case 4: return go(score_decode_kernel<QK, 4, false, false, true>);
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (h->rows_per_item) {
    case 1: return go(score_decode_kernel<QK, 1, DUMP>);
    case 2: return go(score_decode_kernel<QK, 2, DUMP>);
    case 4: return go(score_decode_kernel<QK, 4, DUMP>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Workspace of the allocation-free bounded runs: a file-scope device array,
// one copy per GPU the library runs on, kept until the process ends.  In host
// code its name is only a stand-in; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return 0;
}

int launch_score(const RunArgs& a, bool dump) {
  const PlanHeader* h = a.hdr;
  if (h->n_items == 0) return 0;
  ScoreParams P{};
  if (a.plan_dev) {
    P.items = reinterpret_cast<const Item*>(static_cast<const uint8_t*>(a.plan_dev) + h->off_items);
    P.rinfo = reinterpret_cast<const RowInfo*>(static_cast<const uint8_t*>(a.plan_dev) + h->off_rows);
  }
  P.aslk = a.aslk;  // bounded runs (the header then describes the bound)
  P.aslq_bsnd = a.aslq_bsnd;
  if (a.aslq && a.tab_off >= 0) {
    const TndTables t = tnd_tables(a.p->batch, a.p->s1);
    const int32_t* tab = reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(a.workspace) + a.tab_off);
    P.rows_end = tab + t.rows_end;
    P.group_start = tab + t.group_start;
    P.group_batch = tab + t.group_batch;
  } else if (a.aslq) {
    if (a.p->batch > kTndInKernelBatches) return (int)hipErrorInvalidValue;  // needs the tables
    P.aslq_tnd = a.aslq;
  }
  if (a.aslq) {
    P.nbatch = a.p->batch;
    P.trows = a.p->s1;
  }
  P.max_len = a.max_len;
  P.bstride = a.stride;
  P.mode = a.p->sparse_mode;
  P.cmp = a.p->cmp_ratio;
  P.pre = window_side(a.p->pre_tokens);
  P.next = window_side(a.p->next_tokens);
  P.n_items = h->n_items;
  if (a.items_off >= 0) {  // bounded decode with a device-built item table: it reads like a plan's
    P.items = reinterpret_cast<const Item*>(static_cast<const uint8_t*>(a.workspace) + a.items_off);
    P.n_items_dev = reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(a.workspace) + a.count_off);
    P.aslk = nullptr;
  }
  if (a.plan_in_kernel) P.plan_batches = a.p->batch;
  P.chunk = h->chunk;
  P.reg_chunks = h->reg_chunks;
  P.reg_rows = h->reg_rows;
  P.reg_maxv = h->reg_maxv;
  P.tiles = h->kind == kKindTiles;
  P.query = static_cast<const uint8_t*>(a.query);
  P.key = static_cast<const uint8_t*>(a.key);
  P.weights = a.weights;
  P.q_scale = a.q_scale;
  P.k_scale = a.k_scale;
  P.block_table = a.block_table;
  P.ws = static_cast<float*>(a.workspace);
  P.idx_out = a.sparse_indices;
  P.val_out = a.sparse_values;
  P.stride = a.p->key_block_stride ? a.p->key_block_stride : (int64_t)a.p->block_size * kDim;
  P.block_size = a.p->block_size;
  P.max_blocks = a.p->max_blocks_per_seq;
  P.k = a.p->sparse_count;
  P.bs_magic = (uint32_t)((1ull << 32) / (uint64_t)a.p->block_size + 1);
  P.d_row0 = a.dump_row0;
  P.d_row1 = a.dump_row1;
  P.d_cols = a.dump_cols;
  P.dots = a.dots_out;
  P.dscores = a.scores_out;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  hipError_t e;
  if (a.p->qk_dtype == QLI_QK_INT8)
    e = dump ? launch_score_t<QLI_QK_INT8, true>(P, h, st)
             : launch_score_t<QLI_QK_INT8, false>(P, h, st);
  else
    e = dump ? launch_score_t<QLI_QK_FP8_E4M3FN, true>(P, h, st)
             : launch_score_t<QLI_QK_FP8_E4M3FN, false>(P, h, st);
  return e == hipSuccess ? 0 : (int)e;
}

int launch_select(const RunArgs& a) {
  const PlanHeader* h = a.hdr;
  if (h->n_select == 0) return 0;
  SelectParams S{};
  const SelectEntry* table =
      a.plan_dev ? reinterpret_cast<const SelectEntry*>(static_cast<const uint8_t*>(a.plan_dev) + h->off_select)
                 : nullptr;
  S.aslk = a.aslk;
  if (a.aslq && a.tab_off >= 0) {
    const TndTables t = tnd_tables(a.p->batch, a.p->s1);
    const int32_t* tab = reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(a.workspace) + a.tab_off);
    S.rows_end = tab + t.rows_end;
    S.row_batch = tab + t.row_batch;
  } else if (a.aslq) {
    if (a.p->batch > kTndInKernelBatches) return (int)hipErrorInvalidValue;  // needs the tables
    S.aslq_tnd = a.aslq;
    S.nbatch = a.p->batch;
  }
  S.aslq_bsnd = a.aslq_bsnd;
  S.max_len = a.max_len;
  S.stride = a.stride;
  S.mstride = a.mstride;
  S.merge_base = a.merge_base;
  S.s1 = a.p->s1;
  S.nrows = (int32_t)h->rows;
  S.mode = a.p->sparse_mode;
  S.cmp = a.p->cmp_ratio;
  S.pre = window_side(a.p->pre_tokens);
  S.next = window_side(a.p->next_tokens);
  S.nseg = a.nseg;
  S.ws = static_cast<float*>(a.workspace);
  S.ws_idx = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(a.workspace) + h->ws_index_offset);
  S.idx_out = a.sparse_indices;
  S.val_out = a.sparse_values;
  S.k = a.p->sparse_count;
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const dim3 block(kSelThreads);
  auto pass = [&](int which, const SelectEntry* rows, int count, int max_n) {
    S.rows = rows;
    S.pass = which;
    const dim3 grid(count);
    // Up to 1024 candidates: 256 threads hold them all, and each phase's barrier
    // waits for 4 waves instead of 16 (b1 decode's selection: 3.8 against 4.1 us).
    if (max_n <= 4 * kSelSmallThreads)
      return launch(select_reg_kernel<kSelSmallThreads, 1>, grid, dim3(kSelSmallThreads), st, S);
    if (max_n <= kSelRegMax / 8) return launch(select_reg_kernel<kSelThreads, 1>, grid, block, st, S);
    if (max_n <= kSelRegMax / 4) return launch(select_reg_kernel<kSelThreads, 2>, grid, block, st, S);
    if (max_n <= kSelRegMax / 2) return launch(select_reg_kernel<kSelThreads, 4>, grid, block, st, S);
    if (max_n <= kSelRegMax) return launch(select_reg_kernel<kSelThreads, 8>, grid, block, st, S);
    return launch(select_global_kernel<kSelThreads>, grid, block, st, S);
  };
  hipError_t e = pass(1, table, h->n_select, h->max_cand);
  if (e == hipSuccess && h->n_select2 > 0) e = pass(2, table ? table + h->n_select : nullptr, h->n_select2, h->max_cand2);
  return e == hipSuccess ? 0 : (int)e;
}

// ---------------------------------------------------------------------------
// Score-ordered output (sort_output): after the selection, one workgroup per
// row reorders the row's slots by descending score, equal scores by
// ascending index, with a bitonic sort of 64-bit keys in LDS.  Key of slot
// (index j, value v): order_key(v) above ~j, so the descending order is the
// wanted one and every listed slot's key is nonzero; -1 slots take key 0 and
// sink to the tail, where they stay -1 / -inf.
// ---------------------------------------------------------------------------
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortMax = 2048;  // sparse_count bound

__global__ __launch_bounds__(kSortThreads) void sort_rows_kernel(int32_t* idx, float* val, int k, int np2,
                                                                 int64_t rows) {
  __shared__ uint64_t key[kSortMax];
  const int tid = threadIdx.x;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    int32_t* oi = idx + r * k;
    float* ov = val + r * k;
    for (int e = tid; e < np2; e += kSortThreads) {
      uint64_t kv = 0;
      if (e < k) {
        const int32_t j = oi[e];
        if (j >= 0) kv = ((uint64_t)order_key(ov[e]) << 32) | (uint64_t)(~(uint32_t)j);
      }
      key[e] = kv;
    }
    __syncthreads();
    for (int size = 2; size <= np2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < np2 / 2; t += kSortThreads) {
          const int i = 2 * t - (t & (stride - 1));  // pair (i, i + stride)
          const bool desc = (i & size) == 0;         // runs of `size` alternate; the last is descending
          const uint64_t a = key[i], b = key[i + stride];
          if ((a < b) == desc) {
            key[i] = b;
            key[i + stride] = a;
          }
        }
        __syncthreads();
      }
    }
    for (int e = tid; e < k; e += kSortThreads) {
      const uint64_t kv = key[e];
      oi[e] = kv ? (int32_t)(~(uint32_t)kv) : -1;
      ov[e] = kv ? key_value((uint32_t)(kv >> 32)) : -INFINITY;
    }
    __syncthreads();  // the keys are free for the next row
  }
}

}  // namespace

int launch_sort(const RunArgs& a) {
  const PlanHeader* h = a.hdr;
  const int k = a.p->sparse_count;
  if (!h->sort_output || k <= 1 || h->rows == 0) return 0;
  int np2 = 2;
  while (np2 < k) np2 <<= 1;
  const int64_t grid = std::min<int64_t>(h->rows, 1 << 20);
  const hipError_t e = launch(sort_rows_kernel, dim3((unsigned)grid), dim3(kSortThreads),
                              static_cast<hipStream_t>(a.stream), a.sparse_indices, a.sparse_values, k, np2,
                              h->rows);
  return e == hipSuccess ? 0 : (int)e;
}

// ---------------------------------------------------------------------------
// Bounded decode: the item table from the device key lengths (and, for BSND
// with actual_seq_lengths_query, the query counts), so that a bounded run
// splits each batch by its own length as qli_plan would.  One workgroup:
//   1. the entries [start_b, start_b + m_b) that each batch's rows see
//      (from 0 to its last used row's visible end without a token window);
//      for every candidate chunk c = 128, 256, .., kMaxChunk the item count
//      sum ceil(m_b / c), one wave per two candidates (lanes stride the
//      batches, then a wave reduction);
//   2. the chunk: the smallest c whose items fit the decode slots (else
//      kMaxChunk); when every batch has the same m_b, the c >= it that
//      lowers ceil(items / CUs) * c, as for equal groups on the host;
//   3. max(1, ceil(m_b / c)) items per batch from start_b at an exclusive
//      prefix sum over the batches (1024 at a time with a carry), written as
//      plan items: rows b*S1 .. +S1, key range, per-row visible ranges
//      [lo, vis) (empty past the query count) and staged-score offsets
//      r * bstride + key0 - lo (rows seeing more than k entries), the first
//      item of a batch writing its padding.
// ---------------------------------------------------------------------------
namespace {

constexpr int kItemsThreads = 1024;

struct DecodeItemsParams {
  const int32_t* aslk;
  const int32_t* aslq;  // BSND query counts or null (every row used)
  int32_t batch, s1, mode, cmp, k;
  int64_t max_len, bstride;
  int32_t pre, next;    // pre_tokens, next_tokens clamped to kWindowCap
  Item* items;
  int32_t* n_items;
};

__global__ __launch_bounds__(kItemsThreads) void decode_items_kernel(DecodeItemsParams D) {
  constexpr int NW = kItemsThreads / 64;
  static_assert(kChunkSteps == 2 * NW, "two candidate chunks per wave");
  __shared__ int cnt[kChunkSteps];
  __shared__ int m_lo, m_hi, total_s;
  __shared__ int scan_tmp[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // batch b: used query rows s1b, clamped key length skb, and the entries
  // [start, start + span) its rows see (span_start)
  auto batch_info = [&](int b, int& s1b, int64_t& skb, int& start) {
    skb = min<int64_t>(max(D.aslk[b], 0), D.max_len);
    s1b = D.aslq ? min(max(D.aslq[b], 0), D.s1) : D.s1;
    int lo_min = INT32_MAX, hi_max = 0;
    for (int u = 0; u < s1b; u++) {  // at most kMaxItemRows rows
      int lo;
      const int hi = row_window(D.mode, D.cmp, skb, s1b, u, D.pre, D.next, lo);
      if (hi > lo) {
        lo_min = min(lo_min, lo);
        hi_max = max(hi_max, hi);
      }
    }
    start = span_start(lo_min, hi_max);
    return hi_max - start;
  };
  // 1. wave w sums the items of candidate chunks 128 (w + 1) and 128 (w + NW + 1)
  //    over every batch (lanes stride the batches); wave 0 also takes the
  //    smallest and largest visible maximum
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int i = wave + NW * h, c = 128 * (i + 1);
    int sum = 0, lo = INT32_MAX, hi = -1;
    for (int b = lane; b < D.batch; b += 64) {
      int s1b, start;
      int64_t skb;
      const int m = batch_info(b, s1b, skb, start);
      sum += (m + c - 1) / c;
      lo = min(lo, m);
      hi = max(hi, m);
    }
    sum = wave_sum(sum);
    if (lane == 0) cnt[i] = sum;
    if (h == 0 && wave == 0) {
      lo = wave_min(lo);
      hi = wave_max(hi);
      if (lane == 0) {
        m_lo = lo;
        m_hi = hi;
      }
    }
  }
  __syncthreads();
  // 2. the chunk (every thread reads the same counters)
  int best = kChunkSteps - 1;
  for (int i = 0; i < kChunkSteps; i++)
    if (cnt[i] <= kDecodeSlots) {
      best = i;
      break;
    }
  if (m_hi >= 0 && m_lo == m_hi) {
    auto busiest = [&](int i) { return (int64_t)((cnt[i] + kCUs - 1) / kCUs) * (128 * (i + 1)); };
    for (int i = best + 1; i < kChunkSteps; i++)
      if (busiest(i) < busiest(best)) best = i;
  }
  const int c = 128 * (best + 1);
  // 3. the items, batch b's at the exclusive prefix sum of the batches before it
  int carry = 0;
  for (int b0 = 0; b0 < D.batch; b0 += kItemsThreads) {  // uniform
    const int b = b0 + tid;
    int s1b = 0, m = 0, n = 0, start = 0;
    int64_t skb = 0;
    if (b < D.batch) {
      m = batch_info(b, s1b, skb, start);
      n = max(1, (m + c - 1) / c);
    }
    const int first = carry + block_exclusive_scan<kItemsThreads>(n, scan_tmp);
    if (tid == kItemsThreads - 1) total_s = first + n;
    Item it;
    it.row0 = b * D.s1;
    it.nrows = D.s1;
    it.batch = b;
    it.reserved[0] = it.reserved[1] = 0;
#pragma unroll
    for (int u = 0; u < kMaxItemRows; u++) {
      int lo = 0;
      it.vis[u] = u < s1b ? row_window(D.mode, D.cmp, skb, s1b, u, D.pre, D.next, lo) : 0;
      it.lo[u] = lo;
    }
    for (int i = 0; i < n; i++) {
      it.key0 = start + i * c;
      it.nkeys = max(0, min(c, m - i * c));
      it.flags = i == 0 ? kItemPad : 0;
#pragma unroll
      for (int u = 0; u < kMaxItemRows; u++)  // entry j of a staged row at slot j - lo
        it.cand_off[u] = it.vis[u] - it.lo[u] > D.k
                             ? (int64_t)(b * D.s1 + u) * D.bstride + it.key0 - it.lo[u] : -1;
      D.items[first + i] = it;
    }
    __syncthreads();  // total_s written
    carry = total_s;
    __syncthreads();  // read before the next chunk of batches overwrites it
  }
  if (tid == 0) *D.n_items = carry;
}

}  // namespace

int launch_decode_items(const RunArgs& a) {
  if (a.items_off < 0) return 0;
  DecodeItemsParams D{};
  D.aslk = a.aslk;
  D.aslq = a.aslq_bsnd;
  D.batch = a.p->batch;
  D.s1 = a.p->s1;
  D.mode = a.p->sparse_mode;
  D.cmp = a.p->cmp_ratio;
  D.k = a.p->sparse_count;
  D.max_len = a.max_len;
  D.bstride = a.stride;
  D.pre = window_side(a.p->pre_tokens);
  D.next = window_side(a.p->next_tokens);
  D.items = reinterpret_cast<Item*>(static_cast<uint8_t*>(a.workspace) + a.items_off);
  D.n_items = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(a.workspace) + a.count_off);
  const hipError_t e =
      launch(decode_items_kernel, dim3(1), dim3(kItemsThreads), static_cast<hipStream_t>(a.stream), D);
  return e == hipSuccess ? 0 : (int)e;
}

// ---------------------------------------------------------------------------
// Bounded TND runs: the row and group tables (TndTables) from the device
// actual_seq_lengths_query.  One workgroup: inclusive scans over the
// batches, 1024 at a time with a carry (a running maximum clamped to [0, T]
// makes any input a valid partition of the rows), then a binary search per
// group and per row over the prefix tables held in LDS.
// ---------------------------------------------------------------------------
namespace {

constexpr int kTabThreads = 1024;

__device__ int block_incl_scan(int v, bool use_max, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTabThreads; off <<= 1) {
    const int o = tid >= off ? buf[tid - off] : 0;  // 0 is the identity of both (values are >= 0)
    __syncthreads();
    buf[tid] = use_max ? max(buf[tid], o) : buf[tid] + o;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTabThreads) void tnd_tables_kernel(const int32_t* aslq, int32_t nb, int32_t t,
                                                                 int32_t groups, int32_t* tab, TndTables lay) {
  __shared__ int32_t s_end[kTndMaxBatch];
  __shared__ int32_t s_grp[kTndMaxBatch + 1];
  __shared__ int32_t buf[kTabThreads];
  const int tid = threadIdx.x;
  int carry_end = 0, carry_grp = 0;
  if (tid == 0) s_grp[0] = 0;
  for (int base = 0; base < nb; base += kTabThreads) {
    const int b = base + tid;
    const int v = b < nb ? min(max(aslq[b], 0), t) : 0;
    const int end = max(block_incl_scan(v, true, buf), carry_end);
    if (b < nb) s_end[b] = end;
    __syncthreads();
    const int before = b == 0 ? 0 : (tid > 0 ? s_end[b - 1] : carry_end);
    const int rows_b = b < nb ? end - before : 0;
    const int grp = block_incl_scan((rows_b + kMaxItemRows - 1) / kMaxItemRows, false, buf) + carry_grp;
    if (b < nb) s_grp[b + 1] = grp;
    __syncthreads();
    const int last = min(nb - 1, base + kTabThreads - 1);
    carry_end = s_end[last];
    carry_grp = s_grp[last + 1];
    __syncthreads();
  }
  __syncthreads();  // s_grp[0] (no batches: the loop above has no barrier)
  for (int b = tid; b < nb; b += kTabThreads) tab[lay.rows_end + b] = s_end[b];
  for (int b = tid; b <= nb; b += kTabThreads) tab[lay.group_start + b] = s_grp[b];
  const int real = s_grp[nb];
  for (int g = tid; g < groups; g += kTabThreads) {
    int b = -1;
    if (g < real) {  // the batch with s_grp[b] <= g < s_grp[b + 1]: the last b with s_grp[b] <= g
      int lo = 0, hi = nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_grp[mid] <= g) lo = mid; else hi = mid - 1;
      }
      b = lo;
    }
    tab[lay.group_batch + g] = b;
  }
  const int used = nb > 0 ? s_end[nb - 1] : 0;
  for (int r = tid; r < t; r += kTabThreads) {
    int b = -1;
    if (r < used) {  // the first b with s_end[b] > r
      int lo = 0, hi = nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_end[mid] > r) hi = mid; else lo = mid + 1;
      }
      b = lo;
    }
    tab[lay.row_batch + r] = b;
  }
}

}  // namespace

int launch_tnd_tables(const RunArgs& a) {
  const TndTables lay = tnd_tables(a.p->batch, a.p->s1);
  int32_t* tab = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(a.workspace) + a.tab_off);
  const int groups = (int)tnd_groups(a.p->batch, a.p->s1);
  const hipError_t e = launch(tnd_tables_kernel, dim3(1), dim3(kTabThreads), static_cast<hipStream_t>(a.stream),
                              a.aslq, (int32_t)a.p->batch, (int32_t)a.p->s1, (int32_t)groups, tab, lay);
  return e == hipSuccess ? 0 : (int)e;
}

}  // namespace qli
