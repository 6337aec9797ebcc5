// qli_attention.hip -- gfx950 sparse attention over the indexer's selected
// entries (the consumer of sparse_indices).
//
// The page (EngineX-Ascend "VllmQuantLightningIndexer", QLI-README) calls the
// indexer the preprocessing of sparse attention: its Top-k indices are the
// input of Attention (功能说明 step 3), sparse_indices are the tokens that take
// part in the sparse attention and block_table maps the KV storage of
// PageAttention (参数说明).  It does not write the attention out; the reading
// implemented here: for query row r of batch b and head h, softmax attention
// restricted to the listed entries S_r (slots holding -1 are skipped),
//   out[r][h] = sum_{j in S_r} softmax_j(scale * q[r][h] . K_b[j]) * V_b[j],
//   lse[r][h] = log sum_{j in S_r} exp(scale * q[r][h] . K_b[j]),
// with one bf16 key / value head shared by every query head, entry j of batch
// b at block block_table[b][j / block_size], slot j % block_size.
//
// attention_kernel: one workgroup per (row, split of the row's list).  The
// split's valid entries are compacted into LDS (block id and slot), then
// streamed through a 4-stage LDS ring of 32 entries (three stages load while
// one is computed): keys and values both land by direct-to-LDS loads into
// row-major tiles whose 16-byte chunks are XOR-swizzled by entry, so the
// MFMA operand reads are conflict-free; the V^T operands come from the value
// tile by LDS transpose reads (ds_read_b64_tr_b16, two per d-tile).  Waves
// raise their issue priority while behind in their stages, so the workgroups
// sharing a CU keep pace.  Wave w owns query heads
// [w*HPW, (w+1)*HPW); per 32 entries and 16 heads: S^T = K Q^T
// (8 x v_mfma_f32_16x16x32_bf16, lanes hold one head and 4 keys), an online
// softmax in the exp2 domain (max across the 4 lanes of a head by permlane
// swaps), P^T packed to bf16 in place, O^T += V^T P^T (8 MFMAs over the 8
// d-tiles; the key order inside the 32-entry K dimension is the one the S^T
// lanes already hold, applied to V^T as well).  A row finished by one
// workgroup writes bf16 out and fp32 lse; split rows write fp32 partials
// (unnormalized O, running max, sum) that combine_kernel merges.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "../../include/qli.h"

#define QLI_EXPORT extern "C" __attribute__((visibility("default")))

namespace qla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kDim = 128;         // head dim (the same D as the indexer's)
constexpr int kStage = 32;        // entries per LDS stage
constexpr int kRing = 4;          // stages in the LDS ring (three load while one is computed)
constexpr int kMaxList = 2048;    // entries one workgroup compacts (sparse_count <= 2048)
constexpr int kMaxSplit = kMaxList / 256;  // splits of a row (each at least 256 entries)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const uint16_t* q;          // [rows, H, 128] bf16
  const uint16_t* kc;         // [num_blocks, block_size, 128] bf16, block stride `stride` elements
  const uint16_t* vc;
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* indices;     // [rows, k]
  const int32_t* aslq;        // TND prefix sums (device) or null
  uint16_t* out;              // [rows, H, 128] bf16
  float* lse;                 // [rows, H] or null
  float* part_o;              // split rows: [rows, nsplit, H, 128] fp32
  float* part_ml;             // split rows: [rows, nsplit, H, 2] fp32 (max in log2 units, sum)
  int64_t stride;
  int32_t batch, s1, layout, heads;
  int32_t block_size, max_blocks, num_blocks, k;
  int32_t nsplit, chunk;
  float scale_log2;           // softmax_scale * log2(e)
};

// Max and sum over the four lanes of each head (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float max4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Batch of output row r: BSND r / S1; TND the b with aslq[b-1] <= r < aslq[b]
// (binary search over the prefix sums; -1 past the last one).
__device__ int row_batch(const Params& P, int r) {
  if (P.layout == QLI_LAYOUT_BSND) return r / P.s1;
  int lo = 0, hi = P.batch;  // first b with aslq[b] > r
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (P.aslq[mid] > r) hi = mid; else lo = mid + 1;
  }
  return lo < P.batch ? lo : -1;
}

// Workgroup barrier without a memory fence: waits for this wave's LDS
// accesses only, so direct-to-LDS loads of later stages stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Issue priority of this wave from its progress through its entries: 3 during
// the first quarter of its stages, down to 0 during the last.  Waves of equal
// priority issue oldest first, so the workgroups sharing a CU would otherwise
// finish in dispatch order; this lets one that has fallen behind catch up.
// All waves of a workgroup are at the same stage, so they share the level.
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
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Direct-to-LDS load of 16 bytes per lane (landing at the wave-uniform LDS
// address lds + lane * 16), issued from inline assembly: the compiler then
// adds no waits of its own between these loads and the LDS reads of other
// ring slots (with the builtin it put a vmcnt(0) into one slot's reads);
// the ring's waits are the explicit wait_vm<N>() above.  The helper writes
// m0 behind the compiler's back, which is sound only while nothing else in
// this file relies on m0 (gfx950 LDS reads and writes do not use it, and
// this file has no LDS-DMA builtin, s_sendmsg or dynamically indexed
// register array).
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory");
}

template <int HPW, int NW>
__global__ __launch_bounds__(64 * NW) void attention_kernel(Params P) {
  constexpr int NT = 64 * NW;
  constexpr int HG = HPW / 16;                   // 16-head groups per wave
  constexpr int KL = kStage * 256 / (NT * 16);   // 16-byte loads per thread per stage, of keys and of values
  constexpr int PER = 2 * KL;                    // vector memory operations per thread per stage
  constexpr int IPT = 8;                         // list slots per thread per compaction pass

  // The ring: kRing stages of kStage entries, keys and values as separate
  // arrays per slot (row-major, 256 bytes per entry, 16-byte chunks stored at
  // position chunk ^ (entry % 16)).
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kRing][kStage * 256];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[kRing][kStage * 256];
  __shared__ int32_t lds_blk[kMaxList];
  __shared__ uint16_t lds_slot[kMaxList];
  __shared__ int32_t lds_cnt[IPT][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int r = (int)blockIdx.x / P.nsplit;
  const int split = (int)blockIdx.x - r * P.nsplit;
  const int p0 = split * P.chunk;
  const int p1 = min(P.k, p0 + P.chunk);
  const int jmax = P.max_blocks * P.block_size;

  // 1. This wave's query heads as MFMA B operands (Q^T: K = d, N = head),
  //    requested first: they do not depend on the list.
  bf16x8 qf[HG][4];
  const int h0 = wave * HPW;
#pragma unroll
  for (int g = 0; g < HG; g++) {
    const uint16_t* qh = P.q + ((int64_t)r * P.heads + h0 + 16 * g + c16) * kDim + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) qf[g][ks] = *reinterpret_cast<const bf16x8*>(qh + 32 * ks);
  }

  // 2. Compact the split's valid entries (listed, inside the block table, on a
  //    block of the cache) into LDS in list order: per pass, every list slot
  //    and its block-table entry are requested at once, then one barrier.
  const int b = row_batch(P, r);
  int nvalid = 0;
  for (int base = p0; base < p1; base += IPT * NT) {
    int jv[IPT], bv[IPT];
#pragma unroll
    for (int i = 0; i < IPT; i++) {
      const int pos = base + i * NT + tid;
      jv[i] = (b >= 0 && pos < p1) ? P.indices[(int64_t)r * P.k + pos] : -1;
    }
#pragma unroll
    for (int i = 0; i < IPT; i++) {
      const int j = jv[i];
      bv[i] = (j >= 0 && j < jmax) ? P.block_table[(int64_t)b * P.max_blocks + j / P.block_size] : -1;
    }
    unsigned long long m[IPT];
#pragma unroll
    for (int i = 0; i < IPT; i++) {
      const bool v = bv[i] >= 0 && bv[i] < P.num_blocks;
      m[i] = __ballot(v);
      if (lane == 0) lds_cnt[i][wave] = __popcll(m[i]);
    }
    __syncthreads();
    int before = nvalid;
#pragma unroll
    for (int i = 0; i < IPT; i++) {
      int below_w = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; w++) {
        below_w += w < wave ? lds_cnt[i][w] : 0;
        tot += lds_cnt[i][w];
      }
      if ((m[i] >> lane) & 1ull) {
        const int at = before + below_w + __popcll(m[i] & ((1ull << lane) - 1ull));
        lds_blk[at] = bv[i];
        lds_slot[at] = (uint16_t)(jv[i] % P.block_size);
      }
      before += tot;
    }
    nvalid = before;
    __syncthreads();
  }

  v4f o[HG][8];
  float m_run[HG], l_run[HG];
#pragma unroll
  for (int g = 0; g < HG; g++) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; t++) o[g][t] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  // Loader: piece i of a stage is entry kk = 4 (i NW + wave) + lane / 16 of
  // the stage, 16-byte chunk lane % 16; the chunk stored at position
  // lane % 16 of the entry's row is the logical chunk (lane % 16) ^ (kk % 16).
  // Entries past the list load its last entry again (masked when scored).
  const int nst = (nvalid + kStage - 1) / kStage;
  auto issue = [&](int st, auto slot_) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_)::value;
#pragma unroll
    for (int i = 0; i < KL; i++) {
      const int kk = 4 * (i * NW + wave) + q4;
      const int e = min(st * kStage + kk, nvalid - 1);
      const int64_t off = (int64_t)lds_blk[e] * P.stride + (int64_t)lds_slot[e] * kDim + 8 * (c16 ^ (kk & 15));
      dma16(P.kc + off, &lds_k[S][(i * NW + wave) * 1024]);
      dma16(P.vc + off, &lds_v[S][(i * NW + wave) * 1024]);
    }
  };

  // Stage st: computed from ring slot st % kRing once its loads have landed.
  auto compute = [&](int st, auto slot_) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_)::value;
    const int live = nvalid - st * kStage;  // entries of this stage that exist (>= 1)
    const uint8_t* kt = lds_k[S];
    const uint8_t* vt = lds_v[S];
    // S^T for kStage entries x 16 heads per group: A = keys (rows), B = Q^T.
    bf16x8 ka[2][4];
#pragma unroll
    for (int kt2 = 0; kt2 < 2; kt2++) {
      const int key = 16 * kt2 + c16;
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        const int pc = (4 * ks + q4) ^ c16;
        ka[kt2][ks] = *reinterpret_cast<const bf16x8*>(kt + key * 256 + pc * 16);
      }
    }
    // V^T operands of the 8 d-tiles: row d = 16 t + lane % 16, K positions
    // 8 q .. 8 q + 7 <-> entries 4 q + {0..3} and 16 + 4 q + {0..3}; element
    // (entry e, dim d) sits in chunk (d / 8) ^ (e % 16) of row e.  Two LDS
    // transpose reads (ds_read_b64_tr_b16) per d-tile: within each group of
    // 16 lanes, lane j receives as its element c element j % 4 of the four
    // that lane 4 c + j / 4 addressed.  Lane i of group q addresses entry
    // 4 q + i / 4 (then 16 + 4 q + i / 4), dims 16 t + 4 (i % 4) .. + 3 (8
    // contiguous bytes of one chunk), so lane j receives V[4 q + c][16 t + j].
    bf16x8 va[8];
    {
      const int ea = 4 * q4 + (c16 >> 2), eb = ea + 16;
      const uint8_t* ra = vt + ea * 256 + 8 * (c16 & 1);
      const uint8_t* rb = vt + eb * 256 + 8 * (c16 & 1);
#pragma unroll
      for (int t = 0; t < 8; t++) {
        const int lc = 2 * t + ((c16 & 3) >> 1);  // logical chunk of dims 16 t + 4 (i % 4)
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(ra + ((lc ^ (ea & 15)) << 4)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(rb + ((lc ^ (eb & 15)) << 4)));
        va[t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
#pragma unroll
    for (int g = 0; g < HG; g++) {
      v4f sc[2];
#pragma unroll
      for (int kt2 = 0; kt2 < 2; kt2++) {
        sc[kt2] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
          sc[kt2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kt2][ks], qf[g][ks], sc[kt2], 0, 0, 0);
      }
      // lane: head 16 g + lane % 16; entries 16 kt2 + 4 q + i
      float x[8];
      float mt = -INFINITY;
#pragma unroll
      for (int kt2 = 0; kt2 < 2; kt2++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int e = 16 * kt2 + 4 * q4 + i;
          const float v = e < live ? sc[kt2][i] * P.scale_log2 : -INFINITY;
          x[4 * kt2 + i] = v;
          mt = fmaxf(mt, v);
        }
      mt = max4(mt);
      const float m_new = fmaxf(m_run[g], mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // nothing seen yet: every p is 0
      const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_use);
      m_run[g] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        x[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
        ps += x[e];
      }
      l_run[g] = l_run[g] * alpha + ps;
#pragma unroll
      for (int t = 0; t < 8; t++) o[g][t] *= alpha;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e++) pb[e] = (__bf16)x[e];
#pragma unroll
      for (int t = 0; t < 8; t++) o[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[t], pb, o[g][t], 0, 0, 0);
    }
  };

  // 3. The ring: stages st + 1 .. st + kRing - 1 load while stage st is
  //    computed.  At the top of step st, this wave's pieces of stages st ..
  //    min(st + kRing - 2, nst - 1) are outstanding; waiting until only the
  //    newer ones are leaves stage st landed, and the barrier makes every
  //    wave's pieces visible and frees the slot computed in step st - 1, which
  //    then receives stage st + kRing - 1.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  static_assert(kRing == 4, "the step below names four slots");
  if (nst > 0) issue(0, S0{});
  if (nst > 1) issue(1, S1{});
  if (nst > 2) issue(2, S2{});
  auto step = [&](int st, auto slot_, auto prev_) __attribute__((always_inline)) {
    const int newer = min(st + kRing - 2, nst - 1) - st;
    if (newer >= 2)
      wait_vm<2 * PER>();
    else if (newer == 1)
      wait_vm<PER>();
    else
      wait_vm<0>();
    lds_barrier();
    if (st + kRing - 1 < nst) issue(st + kRing - 1, prev_);
    compute(st, slot_);
  };
  for (int st = 0; st < nst; st += kRing) {
    progress_priority(st, nst);
    step(st, S0{}, S3{});
    if (st + 1 < nst) step(st + 1, S1{}, S0{});
    if (st + 2 < nst) step(st + 2, S2{}, S1{});
    if (st + 3 < nst) step(st + 3, S3{}, S2{});
  }

  // 4. Finish: lane holds head h0 + 16 g + lane % 16, dims 16 t + 4 q + {0..3}.
#pragma unroll
  for (int g = 0; g < HG; g++) {
    const int h = h0 + 16 * g + c16;
    const float l = sum4(l_run[g]);
    if (P.nsplit == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* orow = P.out + ((int64_t)r * P.heads + h) * kDim + 4 * q4;
#pragma unroll
      for (int t = 0; t < 8; t++) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = (__bf16)(o[g][t][i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * t) = v;
      }
      if (P.lse && q4 == 0)
        P.lse[(int64_t)r * P.heads + h] = l > 0.f ? (m_run[g] + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    } else {
      const int64_t slot = ((int64_t)r * P.nsplit + split) * P.heads + h;
      float* po = P.part_o + slot * kDim + 4 * q4;
#pragma unroll
      for (int t = 0; t < 8; t++) *reinterpret_cast<v4f*>(po + 16 * t) = o[g][t];
      if (q4 == 0) {
        P.part_ml[2 * slot] = l > 0.f ? m_run[g] : -INFINITY;
        P.part_ml[2 * slot + 1] = l;
      }
    }
  }
}

// Merge of a split row's partials: M = max_s m_s, L = sum_s l_s 2^(m_s - M),
// out = sum_s O_s 2^(m_s - M) / L, lse = (M + log2 L) ln 2.  32 threads per
// (row, head), one float4 of dims each; workgroups of 8 heads.
__global__ __launch_bounds__(256) void combine_kernel(Params P) {
  const int64_t pair = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);  // row * heads + head
  const int d4 = threadIdx.x & 31;
  const int64_t rows_heads = (int64_t)gridDim.x * 8;
  if (pair >= rows_heads) return;
  const int r = (int)(pair / P.heads), h = (int)(pair - (int64_t)r * P.heads);
  // every split's (max, sum) and O slice requested at once (nsplit <= kMaxSplit)
  float ms[kMaxSplit], ls[kMaxSplit];
  v4f os[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; s++) {
    const int64_t slot = ((int64_t)r * P.nsplit + s) * P.heads + h;
    const bool in = s < P.nsplit;
    ms[s] = in ? P.part_ml[2 * slot] : -INFINITY;
    ls[s] = in ? P.part_ml[2 * slot + 1] : 0.f;
    os[s] = in ? *reinterpret_cast<const v4f*>(P.part_o + slot * kDim + 4 * d4) : v4f{0.f, 0.f, 0.f, 0.f};
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplit; s++) M = fmaxf(M, ms[s]);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kMaxSplit; s++) {
      if (ms[s] == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(ms[s] - M);
      L += ls[s] * w;
      acc += os[s] * w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; i++) v[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x4*>(P.out + pair * kDim + 4 * d4) = v;
  if (P.lse && d4 == 0) P.lse[pair] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

// Split of each row's list: as many workgroups as the chip holds at once
// (two per CU) without going below 256 entries per split.
struct Split {
  int nsplit, chunk;
};
Split choose_split(int64_t rows, int k) {
  const int64_t target = 2 * 256;  // resident workgroups: every split runs in one round
  int64_t ns = rows > 0 ? target / rows : 1;
  const int64_t cap = (k + 255) / 256;
  ns = ns < 1 ? 1 : (ns > cap ? cap : ns);
  int chunk = (int)((k + ns - 1) / ns);
  chunk = (chunk + kStage - 1) / kStage * kStage;
  Split s;
  s.chunk = chunk;
  s.nsplit = (k + chunk - 1) / chunk;
  return s;
}

int validate(const qli_attn_problem* p) {
  if (!p) return QLI_ERR_ARG;
  if (p->layout_query != QLI_LAYOUT_BSND && p->layout_query != QLI_LAYOUT_TND) return QLI_ERR_ARG;
  if (p->batch < 0 || p->s1 < 0) return QLI_ERR_ARG;
  if (p->num_heads != 16 && p->num_heads != 32 && p->num_heads != 64 && p->num_heads != 128)
    return QLI_ERR_UNSUPPORTED;
  if (p->head_dim != kDim) return QLI_ERR_UNSUPPORTED;
  if (p->num_blocks < 1 || p->max_blocks_per_seq < 1) return QLI_ERR_ARG;
  if (p->block_size < 16 || p->block_size > 1024 || p->block_size % 16 != 0) return QLI_ERR_ARG;
  if (p->kv_block_stride != 0) {
    if (p->kv_block_stride < (int64_t)p->block_size * kDim) return QLI_ERR_ARG;
    if (p->kv_block_stride % 8 != 0) return QLI_ERR_UNSUPPORTED;  // 16-byte entry loads
  }
  if (p->sparse_count < 1 || p->sparse_count > kMaxList) return QLI_ERR_ARG;
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale)) return QLI_ERR_ARG;
  if (p->return_lse != 0 && p->return_lse != 1) return QLI_ERR_ARG;
  if (p->reserved0 || p->reserved1 || p->reserved2) return QLI_ERR_ARG;
  const int64_t rows = p->layout_query == QLI_LAYOUT_BSND ? (int64_t)p->batch * p->s1 : p->s1;
  if (rows > INT32_MAX / 8) return QLI_ERR_SIZE;
  if ((int64_t)p->max_blocks_per_seq * p->block_size > INT32_MAX) return QLI_ERR_SIZE;
  return QLI_OK;
}

int64_t rows_of(const qli_attn_problem* p) {
  return p->layout_query == QLI_LAYOUT_BSND ? (int64_t)p->batch * p->s1 : (int64_t)p->s1;
}

size_t workspace_bytes(const qli_attn_problem* p) {
  const int64_t rows = rows_of(p);
  const Split s = choose_split(rows, p->sparse_count);
  if (s.nsplit <= 1 || rows == 0) return 0;
  return (size_t)rows * s.nsplit * p->num_heads * (kDim + 2) * sizeof(float);
}

template <int HPW, int NW>
hipError_t launch_attention(const Params& P, int64_t rows, hipStream_t st) {
  hipLaunchKernelGGL((attention_kernel<HPW, NW>), dim3((unsigned)(rows * P.nsplit)), dim3(64 * NW), 0, st, P);
  return hipGetLastError();
}

}  // namespace
}  // namespace qla

using namespace qla;

QLI_EXPORT int qli_sparse_attention_workspace(const qli_attn_problem* p, size_t* bytes) {
  const int rc = validate(p);
  if (rc != QLI_OK) return rc;
  if (!bytes) return QLI_ERR_ARG;
  *bytes = workspace_bytes(p);
  return QLI_OK;
}

QLI_EXPORT int qli_sparse_attention(const qli_attn_problem* p, const int32_t* aslq, const void* q,
                                    const void* k_cache, const void* v_cache, const int32_t* block_table,
                                    const int32_t* sparse_indices, void* workspace, void* out, float* lse,
                                    void* stream) {
  int rc = validate(p);
  if (rc != QLI_OK) return rc;
  const int64_t rows = rows_of(p);
  if (rows == 0) return QLI_OK;
  auto aligned = [](const void* ptr, uintptr_t n) { return ((uintptr_t)ptr % n) == 0; };
  if (!q || !k_cache || !v_cache || !block_table || !sparse_indices || !out) return QLI_ERR_ARG;
  if (p->layout_query == QLI_LAYOUT_TND && (!aslq || !aligned(aslq, 4))) return QLI_ERR_ARG;
  if (p->return_lse && !lse) return QLI_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4) ||
      !aligned(sparse_indices, 4) || !aligned(out, 8) || !aligned(lse, 4))
    return QLI_ERR_ARG;
  const Split s = choose_split(rows, p->sparse_count);
  if (s.nsplit > kMaxSplit) return QLI_ERR_SIZE;  // combine_kernel holds at most kMaxSplit partials
  const size_t ws = workspace_bytes(p);
  if (ws > 0 && (!workspace || !aligned(workspace, 16))) return QLI_ERR_ARG;
  Params P{};
  P.q = static_cast<const uint16_t*>(q);
  P.kc = static_cast<const uint16_t*>(k_cache);
  P.vc = static_cast<const uint16_t*>(v_cache);
  P.block_table = block_table;
  P.indices = sparse_indices;
  P.aslq = p->layout_query == QLI_LAYOUT_TND ? aslq : nullptr;
  P.out = static_cast<uint16_t*>(out);
  P.lse = p->return_lse ? lse : nullptr;
  P.stride = p->kv_block_stride ? p->kv_block_stride : (int64_t)p->block_size * kDim;
  P.batch = p->batch;
  P.s1 = p->s1;
  P.layout = p->layout_query;
  P.heads = p->num_heads;
  P.block_size = p->block_size;
  P.max_blocks = p->max_blocks_per_seq;
  P.num_blocks = p->num_blocks;
  P.k = p->sparse_count;
  P.nsplit = s.nsplit;
  P.chunk = s.chunk;
  P.scale_log2 = p->softmax_scale * kLog2e;
  if (s.nsplit > 1) {
    P.part_o = static_cast<float*>(workspace);
    P.part_ml = P.part_o + rows * s.nsplit * p->num_heads * kDim;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (p->num_heads) {
    case 16: e = launch_attention<16, 1>(P, rows, st); break;
    case 32: e = launch_attention<16, 2>(P, rows, st); break;
    case 64: e = launch_attention<16, 4>(P, rows, st); break;
    default: e = launch_attention<32, 4>(P, rows, st); break;
  }
  if (e == hipSuccess && s.nsplit > 1) {
    // rows * heads is a multiple of 8 (heads is)
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(rows * p->num_heads / 8)), dim3(256), 0, st, P);
    e = hipGetLastError();
  }
  return e == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}
