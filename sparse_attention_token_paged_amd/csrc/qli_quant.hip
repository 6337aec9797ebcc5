// qli_quant.hip -- gfx950 kernels of the producer side: per-token-head
// quantization of the index query and key into the indexer's 8-bit inputs.
//
// Method: EngineX-Ascend page "VllmQuantLightningIndexer" (QLI-README),
// section 功能说明 (query and key stored and computed in 8 bits) and 参数说明
// (query_quant_mode / key_quant_mode: per-token-head).  The quantizer itself
// is not given by the page; include/qli.h states the symmetric absmax form
// implemented here, with every rounding step fixed in fp32.
//
// One 128-element head vector per row.  A row is spread over 16 lanes of 8
// elements (one 16-byte load of bf16 values per lane), so a wave quantizes 4
// rows at a time and its 64 lanes read 1 KiB contiguous (query) or 4 rows of
// 256 bytes (key entries).  The row's absmax is reduced over its 16 lanes
// with DPP; every lane then forms the same scale and reciprocal and writes
// its 8 codes with one 8-byte store (a row of codes is 128 contiguous bytes:
// one cache line).  Memory bound: 256 bytes read and 128 + 2 (or 4) bytes
// written per row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "qli.h"

#define QLI_EXPORT extern "C" __attribute__((visibility("default")))

namespace qli {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantMaxGrid = 256 * 8;  // persistent grid: 8 workgroups per CU of one MI355X

struct QuantParams {
  const uint16_t* x;  // bf16 rows [n, 128]
  int64_t n;
  // contiguous destination (query)
  uint8_t* q_out;
  void* s_out;
  // paged destination (key entries)
  const int32_t* batch_idx;
  const int32_t* pos;
  const int32_t* block_table;
  int32_t batch_count, max_blocks, num_blocks, block_size;
  int64_t stride;
};

// Maximum over the 16 lanes of each DPP row (every lane ends with its row's
// maximum); non-negative floats order like their bit patterns.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  int x = (int)v;
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false));  // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false));  // row_mirror
  return (uint32_t)x;
}

// OCP E4M3FN code of a finite y with |y| <= 448, nearest, ties to even.
// Below 2^-6 the representable magnitudes are the multiples of 2^-9 (a code
// of 8 is the smallest normal, 2^-6, so the carry is the right code); above,
// 3 of the 23 mantissa bits are kept with round-to-nearest-even on the 20
// dropped ones, a mantissa carry moving into the exponent, and the exponent is
// rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3fn_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = __builtin_fabsf(y);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t u = __float_as_uint(a);
    mag = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return sign | mag;
}

// Codes and scale of one row piece (8 values) from the row's absmax.
template <int QK>
__device__ __forceinline__ uint2 encode8(const float (&f)[8], float amax, uint32_t& scale_bits) {
  uint32_t c[8];
  if constexpr (QK == QLI_QK_INT8) {
    _Float16 s16 = (_Float16)(amax / 127.0f);
    if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
    const float s = (float)s16;
    scale_bits = __builtin_bit_cast(uint16_t, s16);
    const float r = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int q = s == 0.0f ? 0 : (int)__builtin_amdgcn_fmed3f(__builtin_rintf(f[i] * r), -127.0f, 127.0f);
      c[i] = (uint32_t)q & 0xFFu;
    }
  } else {
    const float s = amax / 448.0f;
    scale_bits = __float_as_uint(s);
    const float r = 1.0f / s;
    const bool zero = s == 0.0f || __builtin_isinf(r);
#pragma unroll
    for (int i = 0; i < 8; i++)
      c[i] = zero ? 0u : e4m3fn_code(__builtin_amdgcn_fmed3f(f[i] * r, -448.0f, 448.0f));
  }
  return make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24, c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
}

// Each wave takes groups of 4 rows (16 lanes per row), kGroups groups per
// iteration so that that many 16-byte loads per lane are in flight; the trip
// count is uniform per wave and rows past n are masked at the loads and
// stores.  For key entries the destination (sequence, position, then the
// block-table entry) is requested before the row data, so the dependent
// block-table load waits only for the destination loads (vector loads
// complete in issue order).  Two groups (39 VGPRs, 8 waves per SIMD) beat
// deeper ones, whose registers cost occupancy: the headline decode cache's
// append took 21.6, 20.6, 23.7 and 25.1 us with 1, 2, 4 and 8 groups, and
// the prefill query 40.9 us with 2 groups against 44.8 with 4.
constexpr int kGroups = 2;

template <int QK, bool PAGED>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(QuantParams P) {
  const int lane = threadIdx.x & 63;
  const int piece = lane & 15;  // elements [8 * piece, 8 * piece + 8) of the row
  const int64_t waves = (int64_t)gridDim.x * (kQuantThreads / 64);
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t groups = (P.n + 3) / 4;
  for (int64_t g0 = wave; g0 < groups; g0 += kGroups * waves) {
    int64_t row[kGroups];
    bool ok[kGroups];
    uint4 raw[kGroups];
    int32_t bsel[kGroups], psel[kGroups], blk[kGroups];
#pragma unroll
    for (int h = 0; h < kGroups; h++) {
      row[h] = (g0 + h * waves) * 4 + (lane >> 4);
      ok[h] = row[h] < P.n;
      if constexpr (PAGED) {
        bsel[h] = ok[h] ? P.batch_idx[row[h]] : -1;
        psel[h] = ok[h] ? P.pos[row[h]] : -1;
      }
    }
    if constexpr (PAGED) {
#pragma unroll
      for (int h = 0; h < kGroups; h++) {
        const int32_t b = bsel[h], p = psel[h];
        const bool in = b >= 0 && b < P.batch_count && p >= 0 && p / P.block_size < P.max_blocks;
        blk[h] = in ? P.block_table[(int64_t)b * P.max_blocks + p / P.block_size] : -1;
      }
    }
#pragma unroll
    for (int h = 0; h < kGroups; h++)
      raw[h] = ok[h] ? *reinterpret_cast<const uint4*>(P.x + row[h] * 128 + piece * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int h = 0; h < kGroups; h++) {
      const uint32_t w[4] = {raw[h].x, raw[h].y, raw[h].z, raw[h].w};
      float f[8];
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        f[2 * i] = __uint_as_float(w[i] << 16);  // bf16 -> fp32 is exact
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        m = max(m, (w[i] << 16) & 0x7FFFFFFFu);
        m = max(m, w[i] & 0x7FFF0000u);
      }
      const float amax = __uint_as_float(row16_max(m));
      uint32_t sbits;
      const uint2 codes = encode8<QK>(f, amax, sbits);
      if (!ok[h]) continue;
      uint8_t* dst;
      int64_t sidx;
      if constexpr (PAGED) {
        // entries outside the sequence table or the cache are skipped
        if (blk[h] < 0 || blk[h] >= P.num_blocks) continue;
        const int32_t o = psel[h] % P.block_size;
        dst = P.q_out + (int64_t)blk[h] * P.stride + (int64_t)o * 128;
        sidx = (int64_t)blk[h] * P.block_size + o;
      } else {
        dst = P.q_out + row[h] * 128;
        sidx = row[h];
      }
      *reinterpret_cast<uint2*>(dst + piece * 8) = codes;
      if (piece == 0) {
        if constexpr (QK == QLI_QK_INT8)
          static_cast<uint16_t*>(P.s_out)[sidx] = (uint16_t)sbits;
        else
          static_cast<uint32_t*>(P.s_out)[sidx] = sbits;
      }
    }
  }
}

int launch_quantize(int32_t qk, bool paged, const QuantParams& P, void* stream) {
  const int64_t groups = (P.n + 3) / 4;
  const int64_t per_wg = (kQuantThreads / 64) * kGroups;  // row groups per workgroup and iteration
  const int64_t wgs = std::min<int64_t>((groups + per_wg - 1) / per_wg, kQuantMaxGrid);
  if (wgs <= 0) return QLI_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)wgs), block(kQuantThreads);
  if (qk == QLI_QK_INT8) {
    if (paged)
      hipLaunchKernelGGL((quantize_kernel<QLI_QK_INT8, true>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((quantize_kernel<QLI_QK_INT8, false>), grid, block, 0, st, P);
  } else {
    if (paged)
      hipLaunchKernelGGL((quantize_kernel<QLI_QK_FP8_E4M3FN, true>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((quantize_kernel<QLI_QK_FP8_E4M3FN, false>), grid, block, 0, st, P);
  }
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace
}  // namespace qli

QLI_EXPORT int qli_quantize_query(int32_t qk_dtype, int64_t rows, const void* x, void* q_out, void* scale_out,
                                  void* stream) {
  using namespace qli;
  if (qk_dtype != QLI_QK_INT8 && qk_dtype != QLI_QK_FP8_E4M3FN) return QLI_ERR_UNSUPPORTED;
  if (rows < 0 || rows > (INT64_MAX >> 8)) return QLI_ERR_ARG;
  if (rows == 0) return QLI_OK;
  if (!x || !q_out || !scale_out || !aligned(x, 16) || !aligned(q_out, 8) ||
      !aligned(scale_out, qk_dtype == QLI_QK_INT8 ? 2 : 4))
    return QLI_ERR_ARG;
  QuantParams P{};
  P.x = static_cast<const uint16_t*>(x);
  P.n = rows;
  P.q_out = static_cast<uint8_t*>(q_out);
  P.s_out = scale_out;
  return launch_quantize(qk_dtype, false, P, stream);
}

QLI_EXPORT int qli_append_keys(int32_t qk_dtype, int64_t n, const void* x, const int32_t* batch_idx,
                               const int32_t* pos, const int32_t* block_table, int32_t batch_count,
                               int32_t max_blocks_per_seq, int32_t num_blocks, int32_t block_size,
                               int64_t key_block_stride, void* key_cache, void* k_scale, void* stream) {
  using namespace qli;
  if (qk_dtype != QLI_QK_INT8 && qk_dtype != QLI_QK_FP8_E4M3FN) return QLI_ERR_UNSUPPORTED;
  // cache geometry as for qli_problem (约束说明: block_size a multiple of 16 in 16..1024)
  if (block_size < 16 || block_size > 1024 || block_size % 16 != 0) return QLI_ERR_ARG;
  if (num_blocks < 1 || batch_count < 0 || max_blocks_per_seq < 1) return QLI_ERR_ARG;
  const int64_t stride = key_block_stride == 0 ? (int64_t)block_size * 128 : key_block_stride;
  if (stride < (int64_t)block_size * 128 || stride % 16 != 0) return QLI_ERR_ARG;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return QLI_ERR_ARG;
  if (n < 0 || n > (INT64_MAX >> 8)) return QLI_ERR_ARG;
  if (n == 0) return QLI_OK;
  if (!x || !batch_idx || !pos || !block_table || !key_cache || !k_scale || !aligned(x, 16) ||
      !aligned(key_cache, 16) || !aligned(k_scale, qk_dtype == QLI_QK_INT8 ? 2 : 4))
    return QLI_ERR_ARG;
  QuantParams P{};
  P.x = static_cast<const uint16_t*>(x);
  P.n = n;
  P.q_out = static_cast<uint8_t*>(key_cache);
  P.s_out = k_scale;
  P.batch_idx = batch_idx;
  P.pos = pos;
  P.block_table = block_table;
  P.batch_count = batch_count;
  P.max_blocks = max_blocks_per_seq;
  P.num_blocks = num_blocks;
  P.block_size = block_size;
  P.stride = stride;
  return launch_quantize(qk_dtype, true, P, stream);
}
