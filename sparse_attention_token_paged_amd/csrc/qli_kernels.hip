// qli_kernels.hip -- gfx950 (CDNA4) kernels of the quantized lightning indexer.
//
// Method: EngineX-Ascend page "VllmQuantLightningIndexer" (QLI-README),
// section 功能说明: score = sum_g W[g] * ReLU(ScaleQ[g] * ScaleK[s] * Q[g].K[s]),
// then the Top-k key indices per query token.
//
// Stage 1, score_kernel (one work item per workgroup, 4 waves):
//   * the item's key chunk is walked in tiles of 64 entries; each tile is
//     gathered through block_table with 16-byte loads (8 lanes per 128-byte
//     key row, so every row is one fully used cache line) and staged in a
//     double-buffered, XOR-swizzled LDS tile;
//   * int8 keys use v_mfma_i32_16x16x64_i8 (exact int32 dots), e4m3fn keys
//     v_mfma_f32_16x16x128_f8f6f4; the 64 query heads of a row are the M
//     dimension (4 tiles of 16), 16 keys the N dimension, D=128 the K one;
//   * fused epilogue: ScaleQ is folded into W once per row (w' = W*ScaleQ,
//     exact in fp32 for fp16 inputs), so each (head, key) element costs
//     max + convert + fma; the head sum finishes with two permlane swaps and
//     one multiply by ScaleK[s].  This reordering needs ScaleQ, ScaleK >= 0,
//     which is the contract (dequant scales are magnitudes).
//   * rows that see at most sparse_count entries return every visible index
//     (the top-k of a set no larger than k is the set), so their indices and
//     scores are written straight to the outputs; other rows stage fp32
//     scores in the workspace.
// Stage 2, select_kernel (one workgroup of 1024 threads per staged row):
//   radix select over order-preserving uint32 keys of the scores with 11-bit
//   digits, starting below the bits every score shares; LDS histograms; the
//   threshold digit found with a block scan; ties at the threshold resolved
//   towards the lower index with wave ballots and mbcnt prefix counts; the
//   selected entries written in ascending index order.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "qli_internal.h"

namespace qli {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kScoreThreads = 256;

struct ScoreParams {
  const uint8_t* plan;
  const uint8_t* query;
  const uint8_t* key;
  const void* weights;
  const void* q_scale;
  const void* k_scale;
  const int32_t* block_table;
  float* ws;
  int32_t* idx_out;
  float* val_out;
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

// Sum of the four lanes {l%16 + 16m}: permlane32 then permlane16 swaps.
__device__ __forceinline__ float sum_lane_groups(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

template <int QK, int RW, int WPR, bool DUMP>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(RW == 1 ? 4 : 2)))
void score_kernel(ScoreParams P) {
  constexpr int NT = 4 / WPR;  // 16-key n-tiles per wave per 64-key tile
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(P.plan);
  const RowInfo* rinfo = reinterpret_cast<const RowInfo*>(P.plan + hdr->off_rows);
  const Item it = reinterpret_cast<const Item*>(P.plan + hdr->off_items)[blockIdx.x];

  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][kTileKeys * kDim];
  __shared__ float lds_sk[2][kTileKeys];
  __shared__ int32_t lds_blk[kMaxChunkBlocks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;
  const int c16 = lane & 15;
  const int k = P.k;

  // Rows that see fewer than k entries: slots vis..k-1 are -1 / -inf.
  if (it.flags & kItemPad) {
    for (int u = 0; u < it.nrows; u++) {
      const int64_t r = it.row0 + u;
      const int vis = rinfo[r].vis;
      if (vis >= k) continue;
      for (int pos = vis + tid; pos < k; pos += kScoreThreads) {
        P.idx_out[r * k + pos] = -1;
        if (P.val_out) P.val_out[r * k + pos] = -INFINITY;
      }
    }
  }
  if (it.nkeys <= 0) return;  // uniform across the workgroup

  const int bs = P.block_size;
  const int key0 = it.key0;
  const int kend = key0 + it.nkeys;
  const int fb = key0 / bs;
  const int nblk = (kend - 1) / bs - fb + 1;
  {
    const int32_t* bt = P.block_table + (int64_t)it.batch * P.max_blocks + fb;
    for (int t = tid; t < nblk; t += kScoreThreads) lds_blk[t] = bt[t];
  }

  // This wave's rows: query fragments and folded weights w' = W * ScaleQ.
  const int wr = wave / WPR;
  const int wk = wave % WPR;
  bool rok[RW];
  int64_t rowid[RW];
  int rvis[RW];
  int64_t rws[RW];
  Frag qa[RW][4];
  float wq[RW][16];
#pragma unroll
  for (int rr = 0; rr < RW; rr++) {
    const int u = wr * RW + rr;
    rok[rr] = u < it.nrows;
    const int64_t r = it.row0 + (rok[rr] ? u : 0);
    rowid[rr] = r;
    const RowInfo ri = rinfo[r];
    rvis[rr] = rok[rr] ? ri.vis : 0;
    rws[rr] = ri.ws_off;
    const uint8_t* qrow = P.query + r * (kHeads * kDim);
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const uint8_t* qh = qrow + (16 * m + c16) * kDim;
      qa[rr][m].lo = *reinterpret_cast<const v4i*>(qh + 16 * chunk_lo<QK>(q));
      qa[rr][m].hi = *reinterpret_cast<const v4i*>(qh + 16 * chunk_hi<QK>(q));
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t e = r * kHeads + 16 * m + 4 * q + i;
        wq[rr][4 * m + i] = load_scale<QK>(P.weights, e) * load_scale<QK>(P.q_scale, e);
      }
    }
  }

  // Loader: thread tid fetches two 16-byte pieces of each 64-key tile, at LDS
  // bytes tid*16 and 4096 + tid*16, i.e. key rows tid/8 and 32 + tid/8, physical
  // chunk tid%8.  The logical chunk stored there is XOR-swizzled with bits 1..3
  // of the key row so that the MFMA-layout reads (16 rows, same chunk) hit
  // distinct banks.  Block / slot positions advance incrementally per tile.
  // Two register sets hold the tiles in flight (tile j uses set j % 2); the
  // ScaleK bits stay raw until the stash so no wait is forced at issue time.
  const int cfetch = (tid & 7) ^ ((tid >> 4) & 7);
  int bi[2], slot[2];
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int j = key0 + 32 * p + (tid >> 3);
    bi[p] = j / bs - fb;
    slot[p] = j % bs;
  }
  int sbi = 0, sslot = 0;
  if (tid < kTileKeys) {
    const int j = key0 + tid;
    sbi = j / bs - fb;
    sslot = j % bs;
  }
  int4 kr[2][2];
  uint32_t skr[2] = {0u, 0u};
  __syncthreads();  // lds_blk is ready

  auto fetch = [&](int t, auto set_) __attribute__((always_inline)) {
    constexpr int S = decltype(set_)::value;
    const int tb = key0 + t * kTileKeys;
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const int j = tb + 32 * p + (tid >> 3);
      if (j < kend) {
        const uint8_t* src = P.key + (int64_t)lds_blk[bi[p]] * P.stride + slot[p] * kDim + cfetch * 16;
        kr[S][p] = *reinterpret_cast<const int4*>(src);
      } else {
        kr[S][p] = make_int4(0, 0, 0, 0);
      }
      slot[p] += kTileKeys;
      while (slot[p] >= bs) {
        slot[p] -= bs;
        bi[p]++;
      }
    }
    if (tid < kTileKeys) {
      const int j = tb + tid;
      skr[S] = j < kend ? load_scale_bits<QK>(P.k_scale, (int64_t)lds_blk[sbi] * bs + sslot) : 0u;
      sslot += kTileKeys;
      while (sslot >= bs) {
        sslot -= bs;
        sbi++;
      }
    }
  };
  auto stash = [&](int s, auto set_) __attribute__((always_inline)) {
    constexpr int S = decltype(set_)::value;
    int4* dst = reinterpret_cast<int4*>(&lds_k[s][0]);
    dst[tid] = kr[S][0];
    dst[kScoreThreads + tid] = kr[S][1];
    if (tid < kTileKeys) lds_sk[s][tid] = scale_from_bits<QK>(skr[S]);
  };

  auto compute = [&](int t, int s) __attribute__((always_inline)) {
    const int tb = key0 + t * kTileKeys;
#pragma unroll
    for (int n = 0; n < NT; n++) {
      const int kk = (wk * NT + n) * 16 + c16;
      const uint8_t* krow = &lds_k[s][kk * kDim];
      const int sw = (kk >> 1) & 7;
      Frag b;
      b.lo = *reinterpret_cast<const v4i*>(krow + ((chunk_lo<QK>(q) ^ sw) << 4));
      b.hi = *reinterpret_cast<const v4i*>(krow + ((chunk_hi<QK>(q) ^ sw) << 4));
      const float skv = lds_sk[s][kk];
      const int j = tb + kk;
#pragma unroll
      for (int rr = 0; rr < RW; rr++) {
        if (!rok[rr]) break;  // valid rows of a wave are a prefix
        float acc = 0.f;
        v4i di[4];
        v4f df[4];
        if constexpr (QK == QLI_QK_INT8) {
#pragma unroll
          for (int m = 0; m < 4; m++) {
            di[m] = v4i{0, 0, 0, 0};
            di[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[rr][m].lo, b.lo, di[m], 0, 0, 0);
            di[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[rr][m].hi, b.hi, di[m], 0, 0, 0);
          }
#pragma unroll
          for (int m = 0; m < 4; m++)
#pragma unroll
            for (int i = 0; i < 4; i++)
              acc = __builtin_fmaf(wq[rr][4 * m + i], (float)max(di[m][i], 0), acc);
        } else {
          const v8i bb = __builtin_shufflevector(b.lo, b.hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int m = 0; m < 4; m++) {
            const v8i aa = __builtin_shufflevector(qa[rr][m].lo, qa[rr][m].hi, 0, 1, 2, 3, 4, 5, 6, 7);
            df[m] = v4f{0.f, 0.f, 0.f, 0.f};
            // format 0 = fp8 e4m3 for both operands; scale arguments 0 select the unscaled form
            df[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, df[m], 0, 0, 0, 0, 0, 0);
          }
#pragma unroll
          for (int m = 0; m < 4; m++)
#pragma unroll
            for (int i = 0; i < 4; i++)
              acc = __builtin_fmaf(wq[rr][4 * m + i], __builtin_fmaxf(df[m][i], 0.f), acc);
        }
        acc = sum_lane_groups(acc);
        const float score = acc * skv;
        const int64_t r = rowid[rr];
        if (q == 0 && j < rvis[rr]) {
          if (rws[rr] >= 0) {
            P.ws[rws[rr] + j] = score;
          } else {
            P.idx_out[r * k + j] = j;
            if (P.val_out) P.val_out[r * k + j] = score;
          }
        }
        if constexpr (DUMP) {
          if (r >= P.d_row0 && r < P.d_row1 && j < rvis[rr] && j < P.d_cols) {
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
            if (q == 0) P.dscores[(r - P.d_row0) * P.d_cols + j] = score;
          }
        }
      }
    }
  };

  // Pipeline: LDS stages alternate per tile; while tile t is computed, the
  // loads of tiles t+1 and t+2 are in flight in the two register sets.
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  const int ntiles = (it.nkeys + kTileKeys - 1) / kTileKeys;
  fetch(0, Set0{});
  if (ntiles > 1) fetch(1, Set1{});
  stash(0, Set0{});
  if (ntiles > 2) fetch(2, Set0{});
  __syncthreads();
  auto step = [&](int t, auto set_next) __attribute__((always_inline)) {
    // set_next holds tile t+1; after its stash it receives tile t+3
    compute(t, t & 1);
    if (t + 1 < ntiles) stash((t + 1) & 1, set_next);
    if (t + 3 < ntiles) fetch(t + 3, set_next);
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, Set1{});
    if (t + 1 < ntiles) step(t + 1, Set0{});
  }
}

// ---------------------------------------------------------------------------
// Decode-shaped items: one chunk of kDecodeChunk entries, 1, 2 or 4 rows.
// ---------------------------------------------------------------------------

// Sum over the four lane groups of four per-lane partials, scattered so that
// lane (q, c) ends with the total of partial q (a reduce-scatter in two
// permlane steps): after it, lane q*16 + c holds key q*16 + c of the tile.
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

template <int QK, int RT, bool DUMP>
__global__ __launch_bounds__(kScoreThreads) void score_decode_kernel(ScoreParams P) {
  constexpr int CH = kDecodeChunk;
  constexpr int NTILE = CH / kTileKeys;   // 64-entry tiles per chunk
  constexpr int WPR = 4 / RT;             // waves per row
  constexpr int LOADS = CH * kDim / (kScoreThreads * 16);  // 16-byte key loads per thread
  constexpr int SB = QK == QLI_QK_INT8 ? 2 : 4;           // scale bytes
  typedef __attribute__((address_space(3))) void lds_t;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(P.plan);
  const RowInfo* rinfo = reinterpret_cast<const RowInfo*>(P.plan + hdr->off_rows);
  const Item it = reinterpret_cast<const Item*>(P.plan + hdr->off_items)[blockIdx.x];

  __shared__ __attribute__((aligned(16))) uint8_t lds_k[CH * kDim];
  // A 2-byte direct-to-LDS load fills a 4-byte slot per lane (value in the
  // low half), so ScaleK takes 4 bytes per entry for both dtypes.
  __shared__ __attribute__((aligned(16))) uint32_t lds_sk[CH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;
  const int c16 = lane & 15;
  const int k = P.k;

  if (it.flags & kItemPad) {
    for (int u = 0; u < it.nrows; u++) {
      const int64_t r = it.row0 + u;
      const int vis = rinfo[r].vis;
      if (vis >= k) continue;
      for (int pos = vis + tid; pos < k; pos += kScoreThreads) {
        P.idx_out[r * k + pos] = -1;
        if (P.val_out) P.val_out[r * k + pos] = -INFINITY;
      }
    }
  }
  if (it.nkeys <= 0) return;  // uniform across the workgroup

  // Block ids of the chunk: lane l of every wave holds entry fb + l.
  const int bs = P.block_size;
  const int key0 = it.key0;
  const int kend = key0 + it.nkeys;
  const int fb = (int)__umulhi((uint32_t)key0, P.bs_magic);
  const int nblk = (int)__umulhi((uint32_t)(kend - 1), P.bs_magic) - fb + 1;
  const int32_t btv = lane < nblk ? P.block_table[(int64_t)it.batch * P.max_blocks + fb + lane] : 0;

  // The whole chunk goes to LDS with direct-to-LDS loads.  Wave w's load i
  // fills LDS bytes [(4i + w) * 1024, +1024), lane l the 16 bytes at l*16:
  // key row kk = 32i + 8w + l/8, physical chunk l%8, which holds logical
  // chunk (l%8) ^ ((kk>>1)&7) so that MFMA-layout reads are conflict-free.
#pragma unroll
  for (int i = 0; i < LOADS; i++) {
    const int kk = 32 * i + 8 * wave + (lane >> 3);
    const int j = key0 + kk;
    // the block id comes from another lane: shuffle with every lane active
    const int jc = min(j, kend - 1);
    const int b = (int)__umulhi((uint32_t)jc, P.bs_magic);
    const int blk = __shfl(btv, b - fb, 64);
    if (j < kend) {
      const int slot = j - b * bs;
      const int c = (lane & 7) ^ ((kk >> 1) & 7);
      const uint8_t* src = P.key + (int64_t)blk * P.stride + slot * kDim + c * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_t*)&lds_k[(4 * i + wave) * 1024], 16, 0, 0);
    }
  }
  // ScaleK of every entry of the chunk: thread tid fetches entry tid.
  {
    const int j = key0 + tid;
    const int jc = min(j, kend - 1);
    const int b = (int)__umulhi((uint32_t)jc, P.bs_magic);
    const int blk = __shfl(btv, b - fb, 64);
    if (j < kend) {
      const int slot = j - b * bs;
      const uint8_t* src = static_cast<const uint8_t*>(P.k_scale) + ((int64_t)blk * bs + slot) * SB;
      if constexpr (SB == 2)
        __builtin_amdgcn_global_load_lds(src, (lds_t*)&lds_sk[wave * 64], 2, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(src, (lds_t*)&lds_sk[wave * 64], 4, 0, 0);
    }
  }

  // This wave's row: query fragments and folded weights w' = W * ScaleQ.
  const int u = wave / WPR;
  const int sub = wave % WPR;
  const bool rok = u < it.nrows;
  const int64_t r = it.row0 + (rok ? u : 0);
  const RowInfo ri = rinfo[r];
  const int rvis = rok ? ri.vis : 0;
  const int64_t rws = ri.ws_off;
  Frag qa[4];
  float wq[16];
  {
    const uint8_t* qrow = P.query + r * (kHeads * kDim);
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const uint8_t* qh = qrow + (16 * m + c16) * kDim;
      qa[m].lo = *reinterpret_cast<const v4i*>(qh + 16 * chunk_lo<QK>(q));
      qa[m].hi = *reinterpret_cast<const v4i*>(qh + 16 * chunk_hi<QK>(q));
    }
    // heads 16m + 4q + i, i = 0..3, are consecutive: one vector load per m
    const int64_t e0 = r * kHeads + 4 * q;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      if constexpr (QK == QLI_QK_INT8) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 w = *reinterpret_cast<const h4*>(static_cast<const _Float16*>(P.weights) + e0 + 16 * m);
        const h4 sq = *reinterpret_cast<const h4*>(static_cast<const _Float16*>(P.q_scale) + e0 + 16 * m);
#pragma unroll
        for (int i = 0; i < 4; i++) wq[4 * m + i] = (float)w[i] * (float)sq[i];
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
  __syncthreads();  // every direct-to-LDS load has landed

  int32_t* oi = P.idx_out + r * k;
  float* ov = P.val_out ? P.val_out + r * k : nullptr;
  // This wave's tiles: sub, sub + WPR, ... (64 entries each).
#pragma unroll
  for (int tt = 0; tt < NTILE / WPR; tt++) {
    const int t = sub + tt * WPR;
    const int tb = key0 + t * kTileKeys;
    if (!rok || tb >= kend || tb >= rvis) break;  // uniform per wave
    float part[4];
#pragma unroll
    for (int n = 0; n < 4; n++) {
      const int kk = t * kTileKeys + n * 16 + c16;
      const uint8_t* krow = &lds_k[kk * kDim];
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
          for (int i = 0; i < 4; i++) acc = __builtin_fmaf(wq[4 * m + i], (float)max(di[m][i], 0), acc);
      } else {
        const v8i bb = __builtin_shufflevector(b.lo, b.hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int m = 0; m < 4; m++) {
          const v8i aa = __builtin_shufflevector(qa[m].lo, qa[m].hi, 0, 1, 2, 3, 4, 5, 6, 7);
          df[m] = v4f{0.f, 0.f, 0.f, 0.f};
          df[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, df[m], 0, 0, 0, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) acc = __builtin_fmaf(wq[4 * m + i], __builtin_fmaxf(df[m][i], 0.f), acc);
      }
      part[n] = acc;
      if constexpr (DUMP) {
        const int j = key0 + kk;
        if (r >= P.d_row0 && r < P.d_row1 && j < rvis && j < P.d_cols) {
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
    // lane l now owns entry t*64 + l of the chunk
    const int kk = t * kTileKeys + lane;
    const int j = key0 + kk;
    const float score = reduce_scatter4(part[0], part[1], part[2], part[3]) * scale_from_bits<QK>(lds_sk[kk]);
    if (j < rvis) {
      if (rws >= 0) {
        P.ws[rws + j] = score;
      } else {
        oi[j] = j;
        if (ov) ov[j] = score;
      }
      if constexpr (DUMP) {
        if (r >= P.d_row0 && r < P.d_row1 && j < P.d_cols) P.dscores[(r - P.d_row0) * P.d_cols + j] = score;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelCache = 32768;  // scores cached in LDS (128 KiB)

struct SelectParams {
  const uint8_t* plan;
  const float* ws;
  int32_t* idx_out;
  float* val_out;
  int32_t k;
};

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum over the workgroup in thread order.
__device__ int block_exclusive_scan(int v, int* tmp) {
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
  for (int w = 0; w < wave; w++) before += tmp[w];
  __syncthreads();
  return before + incl - v;
}

constexpr int kSelBatch = 8;  // independent loads in flight per thread

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams S) {
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(S.plan);
  const RowInfo* rinfo = reinterpret_cast<const RowInfo*>(S.plan + hdr->off_rows);
  const int32_t* sel_rows = reinterpret_cast<const int32_t*>(S.plan + hdr->off_select);
  const int64_t row = sel_rows[blockIdx.x];
  const RowInfo ri = rinfo[row];
  const int n = ri.vis;
  const float* sc = S.ws + ri.ws_off;
  const int k = S.k;

  __shared__ uint32_t cache[kSelCache];
  __shared__ int hist[2048];
  __shared__ uint32_t red_and[kSelWaves], red_or[kSelWaves];
  __shared__ int scan_tmp[kSelWaves];
  __shared__ int res[3];
  __shared__ int cnt_gt[kSelWaves], cnt_eq[kSelWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool cached = n <= kSelCache;

  // Visits every score this thread owns (e = tid + i * kSelThreads) as its
  // order key, kSelBatch loads at a time.
  auto for_each_key = [&](auto&& f) {
    for (int base = 0; base < n; base += kSelThreads * kSelBatch) {
      uint32_t u[kSelBatch];
#pragma unroll
      for (int i = 0; i < kSelBatch; i++) {
        const int e = base + i * kSelThreads + tid;
        u[i] = e < n ? (cached ? cache[e] : order_key(sc[e])) : 0u;
      }
#pragma unroll
      for (int i = 0; i < kSelBatch; i++) {
        const int e = base + i * kSelThreads + tid;
        if (e < n) f(e, u[i]);
      }
    }
  };

  // First pass: stage the keys in LDS when they fit, and find the bits every
  // key shares (AND == OR there), which need no radix pass.
  uint32_t a = 0xFFFFFFFFu, o = 0u;
  for (int base = 0; base < n; base += kSelThreads * kSelBatch) {
    float v[kSelBatch];
#pragma unroll
    for (int i = 0; i < kSelBatch; i++) {
      const int e = base + i * kSelThreads + tid;
      v[i] = e < n ? sc[e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kSelBatch; i++) {
      const int e = base + i * kSelThreads + tid;
      if (e < n) {
        const uint32_t u = order_key(v[i]);
        if (cached) cache[e] = u;
        a &= u;
        o |= u;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a &= __shfl_xor(a, off, 64);
    o |= __shfl_xor(o, off, 64);
  }
  if (lane == 0) {
    red_and[wave] = a;
    red_or[wave] = o;
  }
  __syncthreads();
  a = 0xFFFFFFFFu;
  o = 0u;
  for (int w = 0; w < kSelWaves; w++) {
    a &= red_and[w];
    o |= red_or[w];
  }
  const uint32_t diff = a ^ o;
  uint32_t mask, prefix;
  int lo;
  if (diff == 0u) {
    mask = 0xFFFFFFFFu;
    prefix = a;
    lo = 0;
  } else {
    const int hb = 31 - __clz(diff);
    mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    prefix = a & mask;
    lo = hb + 1;
  }
  // Invariant: the kk-th largest key has the top bits `prefix` under `mask`,
  // and kk <= the number of keys that do.
  int kk = k;
  bool whole_bin = diff == 0u;
  while (!whole_bin && lo > 0) {
    const int width = lo < 11 ? lo : 11;
    const int shift = lo - width;
    const int nb = 1 << width;
    for (int b = tid; b < nb; b += kSelThreads) hist[b] = 0;
    __syncthreads();
    for_each_key([&](int, uint32_t u) {
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1);
    });
    __syncthreads();
    // Thread t owns digits nb-1-2t and nb-2-2t (descending order).
    const int d0 = nb - 1 - 2 * tid, d1 = d0 - 1;
    const int h0 = d0 >= 0 ? hist[d0] : 0;
    const int h1 = d1 >= 0 ? hist[d1] : 0;
    const int before = block_exclusive_scan(h0 + h1, scan_tmp);
    if (before < kk && kk <= before + h0 + h1) {
      if (kk <= before + h0) {
        res[0] = d0;
        res[1] = before;
        res[2] = h0;
      } else {
        res[0] = d1;
        res[1] = before + h0;
        res[2] = h1;
      }
    }
    __syncthreads();
    const int digit = res[0], above = res[1], count = res[2];
    __syncthreads();  // res and hist are rewritten by the next pass
    kk -= above;
    prefix |= (uint32_t)digit << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    lo = shift;
    whole_bin = count == kk;
  }

  // Emit in ascending index order: each wave owns one contiguous segment,
  // walked 64 entries per step, kSelBatch steps per batch of loads.
  const int seg = (((n + kSelWaves - 1) / kSelWaves) + 63) & ~63;
  const int beg = min(n, wave * seg);
  const int end = min(n, beg + seg);
  auto segment = [&](auto&& f) {
    for (int e0 = beg; e0 < end; e0 += 64 * kSelBatch) {
      uint32_t u[kSelBatch];
#pragma unroll
      for (int i = 0; i < kSelBatch; i++) {
        const int e = e0 + 64 * i + lane;
        u[i] = e < end ? (cached ? cache[e] : order_key(sc[e])) : 0u;
      }
#pragma unroll
      for (int i = 0; i < kSelBatch; i++) {
        const int e = e0 + 64 * i + lane;
        if (e0 + 64 * i < end) f(e, e < end, u[i]);
      }
    }
  };
  int ngt = 0, neq = 0;
  segment([&](int, bool live, uint32_t u) {
    const uint32_t m = u & mask;
    ngt += __popcll(__ballot(live && m > prefix));
    neq += __popcll(__ballot(live && m == prefix));
  });
  if (lane == 0) {
    cnt_gt[wave] = ngt;
    cnt_eq[wave] = neq;
  }
  __syncthreads();
  int eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; w++) {
    sel_before += cnt_gt[w] + min(cnt_eq[w], max(0, kk - eq_before));
    eq_before += cnt_eq[w];
  }
  int32_t* oi = S.idx_out + row * k;
  float* ov = S.val_out ? S.val_out + row * k : nullptr;
  int run_eq = eq_before, run_sel = sel_before;
  segment([&](int e, bool live, uint32_t u) {
    const uint32_t m = u & mask;
    const bool gt = live && m > prefix;
    const bool eq = live && m == prefix;
    const uint64_t beq = __ballot(eq);
    const bool take = gt || (eq && run_eq + lanes_below(beq) < kk);
    const uint64_t btake = __ballot(take);
    const int pos = run_sel + lanes_below(btake);
    if (take && pos < k) {  // exactly k are taken; the bound only guards the row's slots
      oi[pos] = e;
      if (ov) ov[pos] = key_value(u);
    }
    run_eq += __popcll(beq);
    run_sel += __popcll(btake);
  });
}

template <typename... Args>
hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t st, void* const* ev, int e0,
                  Args... args) {
  void* argv[] = {(void*)&args...};
  hipEvent_t start = ev ? static_cast<hipEvent_t>(ev[e0]) : nullptr;
  hipEvent_t stop = ev ? static_cast<hipEvent_t>(ev[e0 + 1]) : nullptr;
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, st,
                                          start, stop, 0);
  return e != hipSuccess ? e : hipGetLastError();
}

template <int QK, bool DUMP>
hipError_t launch_score_t(const ScoreParams& P, int kind, int rt, int items, hipStream_t st, void* const* ev) {
  const dim3 grid(items), block(kScoreThreads);
  if (kind == kKindDecode) {
    switch (rt) {
      case 1: return launch(score_decode_kernel<QK, 1, DUMP>, grid, block, st, ev, 0, P);
      case 2: return launch(score_decode_kernel<QK, 2, DUMP>, grid, block, st, ev, 0, P);
      case 4: return launch(score_decode_kernel<QK, 4, DUMP>, grid, block, st, ev, 0, P);
      default: return hipErrorInvalidValue;
    }
  }
  if (rt != 8) return hipErrorInvalidValue;
  return launch(score_kernel<QK, 2, 1, DUMP>, grid, block, st, ev, 0, P);
}

}  // namespace

int launch_score(const RunArgs& a, bool dump, void* const* events) {
  const PlanHeader* h = a.hdr;
  if (h->n_items == 0) return 0;
  ScoreParams P{};
  P.plan = static_cast<const uint8_t*>(a.plan_dev);
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
    e = dump ? launch_score_t<QLI_QK_INT8, true>(P, h->kind, h->rows_per_item, h->n_items, st, events)
             : launch_score_t<QLI_QK_INT8, false>(P, h->kind, h->rows_per_item, h->n_items, st, events);
  else
    e = dump ? launch_score_t<QLI_QK_FP8_E4M3FN, true>(P, h->kind, h->rows_per_item, h->n_items, st, events)
             : launch_score_t<QLI_QK_FP8_E4M3FN, false>(P, h->kind, h->rows_per_item, h->n_items, st, events);
  return e == hipSuccess ? 0 : (int)e;
}

int launch_select(const RunArgs& a, void* const* events) {
  const PlanHeader* h = a.hdr;
  if (h->n_select == 0) return 0;
  SelectParams S{};
  S.plan = static_cast<const uint8_t*>(a.plan_dev);
  S.ws = static_cast<const float*>(a.workspace);
  S.idx_out = a.sparse_indices;
  S.val_out = a.sparse_values;
  S.k = a.p->sparse_count;
  const hipError_t e = launch(select_kernel, dim3(h->n_select), dim3(kSelThreads),
                              static_cast<hipStream_t>(a.stream), events, 2, S);
  return e == hipSuccess ? 0 : (int)e;
}

}  // namespace qli
