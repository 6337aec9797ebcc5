// qli_api.cpp -- the C ABI: validation, the host work-split planner and the
// launch sequence.  Semantics are documented in include/qli.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <new>
#include <vector>

#include "qli_internal.h"

#define QLI_EXPORT extern "C" __attribute__((visibility("default")))

namespace qli {
namespace {

bool is_pow2_upto(int v, int hi) {
  return v >= 1 && v <= hi && (v & (v - 1)) == 0;
}

// Scalar validation shared by qli_plan and qli_run.  Each rule cites the
// QLI-README passage it enforces.
int validate_problem(const qli_problem* p) {
  if (!p) return QLI_ERR_ARG;
  // 约束说明: query N = 64, key N = 1, D = 128.
  if (p->num_heads_q != kHeads || p->num_heads_k != 1 || p->head_dim != kDim) return QLI_ERR_ARG;
  // 参数说明 layout_query: BSND or TND.
  if (p->layout_query != QLI_LAYOUT_BSND && p->layout_query != QLI_LAYOUT_TND) return QLI_ERR_ARG;
  if (p->qk_dtype != QLI_QK_INT8 && p->qk_dtype != QLI_QK_FP8_E4M3FN) return QLI_ERR_ARG;
  if (p->scale_dtype != QLI_SCALE_F16 && p->scale_dtype != QLI_SCALE_F32) return QLI_ERR_ARG;
  // 参数说明 notes: INT8 q/k with FLOAT16 scales, FLOAT8_e4m3fn with FLOAT32.
  if (!((p->qk_dtype == QLI_QK_INT8 && p->scale_dtype == QLI_SCALE_F16) ||
        (p->qk_dtype == QLI_QK_FP8_E4M3FN && p->scale_dtype == QLI_SCALE_F32)))
    return QLI_ERR_UNSUPPORTED;
  if (p->batch < 0 || p->s1 < 0) return QLI_ERR_ARG;
  if (p->num_blocks < 1 || p->max_blocks_per_seq < 1) return QLI_ERR_ARG;
  // 约束说明: block_size a multiple of 16, at most 1024.
  if (p->block_size < 16 || p->block_size > 1024 || p->block_size % 16 != 0) return QLI_ERR_ARG;
  // 参数说明 stride: step of key's first axis; at least one whole block.
  if (p->key_block_stride != 0) {
    if (p->key_block_stride < (int64_t)p->block_size * kDim) return QLI_ERR_ARG;
    if (p->key_block_stride % 16 != 0) return QLI_ERR_UNSUPPORTED;  // 16-byte row loads
  }
  // 参数说明 sparse_count: [1, 2048].
  if (p->sparse_count < 1 || p->sparse_count > 2048) return QLI_ERR_ARG;
  // 参数说明 sparse_mode: 0 or 3.
  if (p->sparse_mode != 0 && p->sparse_mode != 3) return QLI_ERR_ARG;
  // 参数说明 cmp_ratio: 1/2/4/8/16/32/64/128.
  if (!is_pow2_upto(p->cmp_ratio, 128)) return QLI_ERR_ARG;
  // 参数说明 pre_tokens / next_tokens: reserved there (only 2^63-1); other
  // values are taken as a token window around the query (visible_window),
  // whose bounds are >= 0.
  if (p->pre_tokens < 0 || p->next_tokens < 0) return QLI_ERR_ARG;
  // 参数说明 query_quant_mode / key_quant_mode: only 0 (per-token-head).
  if (p->query_quant_mode != 0 || p->key_quant_mode != 0) return QLI_ERR_UNSUPPORTED;
  if (p->return_value != 0 && p->return_value != 1) return QLI_ERR_ARG;
  if (p->sort_output != 0 && p->sort_output != 1) return QLI_ERR_ARG;
  if (p->reserved0 || p->reserved1) return QLI_ERR_ARG;
  const int64_t rows = p->layout_query == QLI_LAYOUT_BSND ? (int64_t)p->batch * p->s1 : p->s1;
  if (rows > INT32_MAX / 2) return QLI_ERR_SIZE;
  return QLI_OK;
}

constexpr uint32_t kFnvPrime = 16777619u;

uint64_t fnv_mix(uint64_t h, int64_t v) {
  for (int b = 0; b < 8; b++) {
    h ^= (uint64_t)((v >> (8 * b)) & 0xFF);
    h *= 1099511628211ull;
  }
  return h;
}

}  // namespace

uint64_t problem_fingerprint(const qli_problem& p) {
  uint64_t h = 1469598103934665603ull ^ kFnvPrime;
  const int64_t fields[] = {p.batch, p.s1, p.layout_query, p.qk_dtype, p.scale_dtype,
                            p.num_blocks, p.block_size, p.max_blocks_per_seq,
                            p.sparse_count, p.sparse_mode, p.cmp_ratio, p.pre_tokens, p.next_tokens,
                            p.return_value, p.sort_output};
  for (int64_t f : fields) h = fnv_mix(h, f);
  return h;
}

namespace {

struct Built {
  PlanHeader hdr;
  std::vector<RowInfo> rows;
  std::vector<Item> items;
  std::vector<SelectEntry> select;
};

int64_t align16(int64_t v) { return (v + 15) & ~int64_t(15); }

// Score-ordered output: the reordering reads each row's values, so a caller
// that takes none gets a [rows, k] fp32 region at the end of the workspace.
void add_values_region(const qli_problem& p, PlanHeader& h) {
  h.sort_output = p.sort_output;
  h.ws_values_offset = -1;
  if (p.sort_output && !p.return_value && h.rows > 0) {
    h.ws_values_offset = align16(h.workspace_bytes);
    h.workspace_bytes = h.ws_values_offset + h.rows * p.sparse_count * 4;
  }
}

// Decode chunk for row groups with visible maxima maxv (all alike when
// equal): the smallest multiple of 128 entries for which the items fit the
// decode kernel's resident workgroups on one MI355X (256 CUs x 3) in a
// single round; for equal groups, a longer chunk if it lowers the keys of the
// busiest CU, the items being dealt evenly over the CUs (e.g. 512 items of
// 512 keys, 2 per CU, rather than 688 of 384, 3 on most CUs).
template <typename ItemsFor>
int decode_chunk_for(ItemsFor&& items_for, bool equal) {
  int c = 128;
  while (c < kMaxChunk && items_for(c) > kDecodeSlots) c += 128;
  if (equal) {
    auto busiest = [&](int cc) { return (items_for(cc) + kCUs - 1) / kCUs * cc; };
    int best = c;
    for (int cc = c + 128; cc <= kMaxChunk; cc += 128)
      if (busiest(cc) < busiest(best)) best = cc;
    c = best;
  }
  return c;
}

int decode_chunk(const std::vector<int32_t>& maxv, bool equal) {
  return decode_chunk_for(
      [&](int c) {
        int64_t n = 0;
        for (int32_t m : maxv) n += (m + c - 1) / c;
        return n;
      },
      equal);
}

// The same for `groups` equal groups of maxv entries (no allocation).
int decode_chunk_equal(int64_t groups, int32_t maxv) {
  return decode_chunk_for([&](int c) { return groups * ((maxv + c - 1) / c); }, groups > 0);
}

int build_plan(const qli_problem& p, const int32_t* aslq, const int32_t* aslk, Built& out) {
  const bool bsnd = p.layout_query == QLI_LAYOUT_BSND;
  if (p.batch > 0 && !aslk) return QLI_ERR_ARG;  // 约束说明: required for PA_BSND keys
  if (!bsnd && p.batch > 0 && !aslq) return QLI_ERR_ARG;  // 约束说明: required for TND
  const int64_t rows = bsnd ? (int64_t)p.batch * p.s1 : p.s1;

  // Per-batch query ranges (约束说明: TND prefix sums non-decreasing, >= 0).
  std::vector<int64_t> qbeg(p.batch), qcnt(p.batch);
  int64_t prev = 0;
  for (int b = 0; b < p.batch; b++) {
    if (aslk[b] < 0) return QLI_ERR_ARG;
    const int64_t stored = aslk[b] / p.cmp_ratio;
    if (stored >= kMaxEntries) return QLI_ERR_SIZE;  // exact reciprocal division in the kernels
    const int64_t need = (stored + p.block_size - 1) / p.block_size;
    if (need > p.max_blocks_per_seq) return QLI_ERR_ARG;  // 约束说明: block_table second dim
    if (bsnd) {
      const int64_t n = aslq ? aslq[b] : p.s1;
      if (n < 0 || n > p.s1) return QLI_ERR_ARG;
      qbeg[b] = (int64_t)b * p.s1;
      qcnt[b] = n;
    } else {
      if (aslq[b] < prev || aslq[b] > p.s1) return QLI_ERR_ARG;
      qbeg[b] = prev;
      qcnt[b] = aslq[b] - prev;
      prev = aslq[b];
    }
  }

  // Row r sees entries [lo, vis) (visible_window; lo = 0 without a window).
  out.rows.assign(rows, RowInfo{-1, 0, -1, 0, 0});
  int64_t max_s1b = 0, visible = 0, max_vis = 0, key_entries = 0, table_entries = 0, active = 0;
  for (int b = 0; b < p.batch; b++) {
    max_s1b = std::max(max_s1b, qcnt[b]);
    int64_t batch_lo = INT64_MAX, batch_hi = 0;
    for (int64_t i = 0; i < qcnt[b]; i++) {
      int64_t lo = 0;
      const int64_t hi = visible_window(p.sparse_mode, p.cmp_ratio, aslk[b], qcnt[b], i, p.pre_tokens,
                                        p.next_tokens, lo);
      const int64_t v = hi - lo;
      RowInfo& ri = out.rows[qbeg[b] + i];
      ri.batch = b;
      ri.vis = (int32_t)hi;
      ri.lo = (int32_t)lo;
      visible += v;
      active += v > 0;
      max_vis = std::max(max_vis, v);
      if (v > 0) {
        batch_lo = std::min(batch_lo, lo);
        batch_hi = std::max(batch_hi, hi);
      }
    }
    if (batch_hi > 0) {  // the entries some row of the batch sees lie in [batch_lo, batch_hi)
      key_entries += batch_hi - batch_lo;
      table_entries += (batch_hi - 1) / p.block_size - batch_lo / p.block_size + 1;
    }
  }
  const bool windowed = p.pre_tokens != INT64_MAX || p.next_tokens != INT64_MAX;

  // Tile shape: items of 1, 2 or 4 rows of one batch (the most a batch has,
  // up to 4), so the key chunk is read once for all of them.  Prefill-like
  // problems take 4-row items too, chunked by the same slot-filling rule
  // (measured against 8-row tiles walking whole rows: the 4 x 2048 TND
  // prefill 113 against 123 us, 16 sequences of 16 tokens over 8192 keys 28
  // against 107 us, with the same bits).
  const int rt = max_s1b <= 1 ? 1 : (max_s1b <= 2 ? 2 : 4);

  // A group's items cover the entries [start, start + maxv) that some row of
  // it sees (start: the smallest lo rounded down to a 64-entry tile).
  struct Group { int32_t row0, nrows, batch, maxv, start; };
  std::vector<Group> groups;
  for (int b = 0; b < p.batch; b++) {
    for (int64_t i = 0; i < qcnt[b]; i += rt) {
      const int32_t n = (int32_t)std::min<int64_t>(rt, qcnt[b] - i);
      int32_t lo = INT32_MAX, hi = 0;
      for (int32_t u = 0; u < n; u++) {
        const RowInfo& ri = out.rows[qbeg[b] + i + u];
        if (ri.vis > ri.lo) {
          lo = std::min(lo, ri.lo);
          hi = std::max(hi, ri.vis);
        }
      }
      const int32_t start = hi > 0 ? lo / kTileKeys * kTileKeys : 0;
      groups.push_back({(int32_t)(qbeg[b] + i), n, b, hi - start, start});
    }
  }
  // Rows that belong to no query token only receive padding.
  for (int64_t r = 0; r < rows;) {
    if (out.rows[r].batch >= 0) { r++; continue; }
    int64_t e = r;
    while (e < rows && e - r < rt && out.rows[e].batch < 0) e++;
    groups.push_back({(int32_t)r, (int32_t)(e - r), -1, 0, 0});
    r = e;
  }

  // Chunk size: decode_chunk (items fill the resident decode workgroups).
  const int k = p.sparse_count;
  int chunk;
  bool equal = !groups.empty();
  {
    std::vector<int32_t> maxv;
    for (const Group& g : groups) {
      maxv.push_back(g.maxv);
      equal = equal && g.batch >= 0 && g.nrows == groups[0].nrows && g.maxv == groups[0].maxv;
    }
    chunk = decode_chunk(maxv, equal);
  }
  // Items per group.  Groups of unequal length split their entries into
  // ceil(maxv / chunk) items, and while the items leave decode slots free the
  // group with the longest items takes one more; each group's items are then
  // near-equal runs of 128-entry blocks (never longer than the chunk), so no
  // CU is left with several full chunks while others hold remainders (the
  // 64 ragged fp8 decode rows: 740 items become 768, the busiest CU's entries
  // 9984 -> 9472 against a mean of 9188, scoring 70.4 -> 69.4 us).  Equal
  // groups keep whole chunks (decode_chunk already balances them).
  std::vector<int32_t> nitems(groups.size(), 0);
  {
    int64_t used = 0;
    for (size_t i = 0; i < groups.size(); i++) {
      nitems[i] = groups[i].maxv > 0 ? (groups[i].maxv + chunk - 1) / chunk : 0;
      used += nitems[i];
    }
    auto blocks_of = [&](size_t i) { return (groups[i].maxv + kSpanAlign - 1) / kSpanAlign; };
    if (!equal && used < kDecodeSlots) {
      std::vector<std::pair<int32_t, size_t>> heap;  // (blocks per item, group), longest on top
      for (size_t i = 0; i < groups.size(); i++)
        if (nitems[i] > 0) heap.push_back({(blocks_of(i) + nitems[i] - 1) / nitems[i], i});
      std::make_heap(heap.begin(), heap.end());
      while (used < kDecodeSlots && !heap.empty()) {
        std::pop_heap(heap.begin(), heap.end());
        const auto [longest, i] = heap.back();
        const int32_t next = (blocks_of(i) + nitems[i]) / (nitems[i] + 1);  // with one item more
        if (next >= longest) break;  // one-block items: nothing gets shorter
        nitems[i]++;
        used++;
        heap.back().first = next;
        std::push_heap(heap.begin(), heap.end());
      }
    }
  }

  // Per-row workspace offsets.  A row that sees more than k entries stages
  // every score for the selection stage, in ascending key order.
  int64_t ws = 0, max_cand = 0, max_cand2 = 0;
  std::vector<SelectEntry> pass2;
  std::vector<std::pair<size_t, size_t>> pass2_segments;  // each merge's pass-1 entries
  auto pad4 = [](int64_t n) { return (n + 3) & ~int64_t(3); };  // 16-byte aligned regions
  for (int64_t r = 0; r < rows; r++) {
    RowInfo& ri = out.rows[r];
    ri.ncand = 0;
    if (ri.vis - ri.lo > k) {
      const int64_t n = ri.vis - ri.lo;
      ri.ws_off = ws;
      ri.ncand = (int32_t)n;
      ws += pad4(n);
      if (n <= kSelSegment) {
        SelectEntry se{};
        se.src_off = ri.ws_off;
        se.dst_off = -1;
        se.row = (int32_t)r;
        se.n = ri.ncand;
        se.base = ri.lo;
        out.select.push_back(se);
        max_cand = std::max<int64_t>(max_cand, n);
      } else {
        // Segments of kSelSegment candidates first keep their top-k each,
        // then one selection merges them (regions placed below).
        const size_t first = out.select.size();
        int64_t m = 0;
        for (int64_t s0 = 0; s0 < n; s0 += kSelSegment) {
          const int64_t sn = std::min<int64_t>(kSelSegment, n - s0);
          SelectEntry se{};
          se.src_off = ri.ws_off + s0;
          se.dst_off = m;  // relative to the row's merge region for now
          se.row = (int32_t)r;
          se.n = (int32_t)sn;
          se.base = (int32_t)(ri.lo + s0);
          out.select.push_back(se);
          max_cand = std::max<int64_t>(max_cand, sn);
          m += std::min<int64_t>(k, sn);
        }
        SelectEntry fin{};
        fin.dst_off = -1;
        fin.row = (int32_t)r;
        fin.n = (int32_t)m;
        fin.indexed = 1;
        pass2.push_back(fin);
        pass2_segments.push_back({first, out.select.size()});
        max_cand2 = std::max<int64_t>(max_cand2, m);
      }
    }
  }
  // The merge regions (scores, and key indices in the index region) follow
  // every row's candidate region; only they carry key indices.
  const int64_t merge_start = ws;
  for (size_t i = 0; i < pass2.size(); i++) {
    pass2[i].src_off = ws;
    for (size_t e = pass2_segments[i].first; e < pass2_segments[i].second; e++) out.select[e].dst_off += ws;
    ws += pad4(pass2[i].n);
  }
  const size_t n_pass1 = out.select.size();
  out.select.insert(out.select.end(), pass2.begin(), pass2.end());

  for (const Group& g : groups) {
    Item base{};
    base.row0 = g.row0;
    base.nrows = g.nrows;
    base.batch = g.batch;
    for (int u = 0; u < kMaxItemRows; u++) {
      base.vis[u] = 0;
      base.lo[u] = 0;
      base.cand_off[u] = -1;
    }
    for (int u = 0; u < g.nrows; u++) {
      base.vis[u] = out.rows[g.row0 + u].vis;
      base.lo[u] = out.rows[g.row0 + u].lo;
    }
    if (g.maxv == 0) {
      base.flags = kItemPad;
      out.items.push_back(base);
      continue;
    }
    const int32_t n_it = nitems[&g - groups.data()];  // >= 1 and at most blocks here
    const int32_t blocks = (g.maxv + kSpanAlign - 1) / kSpanAlign;
    for (int32_t i = 0, c0 = 0; c0 < g.maxv; i++) {
      // whole chunks for equal groups; else near-equal runs of blocks
      const int32_t len = equal ? chunk : (blocks / n_it + (i < blocks % n_it ? 1 : 0)) * kSpanAlign;
      Item it = base;
      it.key0 = g.start + c0;
      it.nkeys = std::min(len, g.maxv - c0);
      it.flags = c0 == 0 ? kItemPad : 0;
      c0 += len;
      for (int u = 0; u < g.nrows; u++) {
        const RowInfo& ri = out.rows[g.row0 + u];
        if (ri.ws_off >= 0) it.cand_off[u] = ri.ws_off + it.key0 - ri.lo;
      }
      out.items.push_back(it);
    }
  }
  // Regular decode plans: every batch has the same query rows (one group) and
  // the same visible maximum, so an item's batch, key range and rows follow
  // from its position, and the kernel can start its block-table and query
  // loads without waiting for the item.  They keep batch-major order.
  bool regular = !windowed && p.layout_query == QLI_LAYOUT_BSND && p.batch > 0 &&
                 (int64_t)groups.size() == p.batch;
  for (int b = 0; regular && b < p.batch; b++) {
    const Group& g = groups[b];
    regular = g.batch == b && g.nrows == p.s1 && g.row0 == (int64_t)b * p.s1 && g.maxv == groups[0].maxv &&
              g.maxv > 0;
  }
  const int32_t reg_chunks = regular ? (groups[0].maxv + chunk - 1) / chunk : 0;
  if (!regular)  // longest items first: the kernels hand them out in snake order
    std::stable_sort(out.items.begin(), out.items.end(),
                     [](const Item& a, const Item& b) { return a.nkeys * a.nrows > b.nkeys * b.nrows; });
  if (out.items.size() > (size_t)INT32_MAX) return QLI_ERR_SIZE;

  PlanHeader& h = out.hdr;
  std::memset(&h, 0, sizeof(h));
  h.magic = kPlanMagic;
  h.version = kPlanVersion;
  h.fingerprint = problem_fingerprint(p);
  h.rows = rows;
  h.visible_pairs = visible;
  h.ws_scores = ws;
  // Index region: the key indices of the merge regions [merge_start, ws),
  // placed after the scores so that candidate e's index sits at byte
  // ws_index_offset + 4e (merge_start is a multiple of 4 elements).
  h.ws_index_offset = align16(ws * 4) - merge_start * 4;
  h.workspace_bytes = n_pass1 < out.select.size() ? align16(ws * 4) + (ws - merge_start) * 4 : ws * 4;
  h.kind = kKindDecode;
  h.rows_per_item = rt;
  h.n_items = (int32_t)out.items.size();
  h.n_select = (int32_t)n_pass1;
  h.chunk = chunk;
  h.max_vis = (int32_t)max_vis;
  h.max_cand = (int32_t)max_cand;
  h.n_select2 = (int32_t)pass2.size();
  h.max_cand2 = (int32_t)max_cand2;
  h.reg_chunks = reg_chunks;
  h.reg_rows = regular ? p.s1 : 0;
  h.reg_maxv = regular ? groups[0].maxv : 0;
  h.key_entries = key_entries;
  h.table_entries = table_entries;
  h.active_rows = active;
  add_values_region(p, h);
  h.off_rows = align16(sizeof(PlanHeader));
  h.off_items = align16(h.off_rows + (int64_t)sizeof(RowInfo) * rows);
  h.off_select = align16(h.off_items + (int64_t)sizeof(Item) * h.n_items);
  h.plan_bytes = align16(h.off_select + (int64_t)sizeof(SelectEntry) * (h.n_select + h.n_select2));
  return QLI_OK;
}

bool plan_matches(const qli_problem* p, const void* plan_host) {
  if (!plan_host) return false;
  const PlanHeader* h = plan_header(plan_host);
  return h->magic == kPlanMagic && h->version == kPlanVersion &&
         h->fingerprint == problem_fingerprint(*p);
}

// internal_ws: the workspace is the library's own (checked by the caller).
int check_run_args(const RunArgs& a, bool internal_ws = false) {
  const PlanHeader* h = a.hdr;
  if (!a.plan_dev && !a.aslk) return QLI_ERR_ARG;  // a plan, or bounded decode
  if (h->rows == 0) return QLI_OK;
  if (!a.sparse_indices) return QLI_ERR_ARG;
  if (a.p->return_value && !a.sparse_values) return QLI_ERR_ARG;
  if (h->n_items > 0 && (!a.query || !a.key || !a.weights || !a.q_scale || !a.k_scale || !a.block_table))
    return QLI_ERR_ARG;
  if (!internal_ws && h->workspace_bytes > 0 && !a.workspace) return QLI_ERR_ARG;
  // Vector loads need aligned bases: 16 bytes for query, key, the fp32
  // weights / q_scale, plan and workspace; the element size elsewhere.
  auto aligned = [](const void* ptr, uintptr_t n) { return ((uintptr_t)ptr % n) == 0; };
  const uintptr_t sb = a.p->scale_dtype == QLI_SCALE_F16 ? 2 : 4;
  if ((a.plan_dev && !aligned(a.plan_dev, 16)) || (!internal_ws && !aligned(a.workspace, 16)) || !aligned(a.query, 16) ||
      !aligned(a.key, 16) || !aligned(a.weights, 4 * sb) || !aligned(a.q_scale, 4 * sb) ||
      !aligned(a.k_scale, sb) || !aligned(a.block_table, 4) || !aligned(a.sparse_indices, 4) ||
      !aligned(a.sparse_values, 4))
    return QLI_ERR_ARG;
  return QLI_OK;
}

}  // namespace
}  // namespace qli

using namespace qli;

QLI_EXPORT const char* qli_status_string(int status) {
  switch (status) {
    case QLI_OK: return "ok";
    case QLI_ERR_ARG: return "invalid argument";
    case QLI_ERR_UNSUPPORTED: return "unsupported configuration";
    case QLI_ERR_SIZE: return "buffer too small or size overflow";
    case QLI_ERR_HIP: return "HIP runtime error";
    case QLI_ERR_PLAN: return "plan does not match the problem";
    default: return "unknown status";
  }
}

QLI_EXPORT int qli_plan(const qli_problem* p, const int32_t* aslq, const int32_t* aslk,
                        void* plan, size_t plan_capacity, size_t* plan_bytes,
                        size_t* workspace_bytes) {
  try {
    int rc = validate_problem(p);
    if (rc != QLI_OK) return rc;
    Built b;
    rc = build_plan(*p, aslq, aslk, b);
    if (rc != QLI_OK) return rc;
    if (plan_bytes) *plan_bytes = (size_t)b.hdr.plan_bytes;
    if (workspace_bytes) *workspace_bytes = (size_t)b.hdr.workspace_bytes;
    if (!plan) return QLI_OK;
    if (plan_capacity < (size_t)b.hdr.plan_bytes) return QLI_ERR_SIZE;
    uint8_t* dst = static_cast<uint8_t*>(plan);
    std::memset(dst, 0, (size_t)b.hdr.plan_bytes);
    std::memcpy(dst, &b.hdr, sizeof(PlanHeader));
    if (!b.rows.empty()) std::memcpy(dst + b.hdr.off_rows, b.rows.data(), sizeof(RowInfo) * b.rows.size());
    if (!b.items.empty()) std::memcpy(dst + b.hdr.off_items, b.items.data(), sizeof(Item) * b.items.size());
    if (!b.select.empty()) std::memcpy(dst + b.hdr.off_select, b.select.data(), sizeof(SelectEntry) * b.select.size());
    return QLI_OK;
  } catch (const std::bad_alloc&) {
    return QLI_ERR_SIZE;
  } catch (...) {
    return QLI_ERR_ARG;
  }
}

QLI_EXPORT int qli_plan_info_get(const void* plan_host, qli_plan_info* info) {
  if (!plan_host || !info) return QLI_ERR_ARG;
  const PlanHeader* h = plan_header(plan_host);
  if (h->magic != kPlanMagic || h->version != kPlanVersion) return QLI_ERR_PLAN;
  info->rows = h->rows;
  info->visible_pairs = h->visible_pairs;
  info->plan_bytes = h->plan_bytes;
  info->workspace_bytes = h->workspace_bytes;
  info->key_entries = h->key_entries;
  info->table_entries = h->table_entries;
  info->active_rows = h->active_rows;
  info->score_items = h->n_items;
  {  // rows with a final selection: pass-1 entries that write a row, plus the merges
    const SelectEntry* table = reinterpret_cast<const SelectEntry*>(static_cast<const uint8_t*>(plan_host) + h->off_select);
    int32_t finals = h->n_select2;
    for (int32_t i = 0; i < h->n_select; i++) finals += table[i].dst_off < 0 ? 1 : 0;
    info->select_rows = finals;
  }
  info->rows_per_item = h->rows_per_item;
  info->keys_per_chunk = h->chunk;
  info->kind = h->kind;
  info->reserved = 0;
  return QLI_OK;
}

// Launch geometry of bounded decode (no plan): the regular decode mapping
// over B batches of S1 rows and nmax = max_len / cmp_ratio entries (at least
// one item per batch, so rows that see nothing are still padded); row r's
// scores at element r * stride when it may see more than k entries, nseg
// segments per row, merge candidates at merge_base + r * mstride.
struct Bounded {
  PlanHeader h;
  int64_t stride, mstride, merge_base;
  int32_t nseg;
  int64_t tab_off;  // TND of many batches: byte offset of the row and group tables in the workspace, else -1
  int64_t items_off, count_off;  // decode: the device-built item table and its count (-1: none)
  bool plan_in_kernel;           // decode with few batches: the scoring kernel splits the work itself
  int64_t span;                  // the most entries an item's rows see together
};

// Bounded runs: the most entries that `rows` consecutive query rows of a
// batch see together (nmax without a token window).  Row i sees entries in
// [ceil((pos_i - pre) / cmp), floor((pos_i + next' + 1) / cmp)) with next' = 0
// under mode 3, whose causal cut binds first (visible_window), so rows
// pos_0 .. pos_0 + rows - 1 see at most (pre + next' + rows) / cmp + 1
// entries; items, which start at a multiple of kSpanAlign below the first of
// them (aligned), cover up to kSpanAlign - 1 more.
int64_t window_span(const qli_problem& p, int64_t nmax, int64_t rows, bool aligned) {
  if (p.pre_tokens == INT64_MAX && p.next_tokens == INT64_MAX) return nmax;
  const int64_t next = p.sparse_mode == 3 ? 0 : p.next_tokens;
  constexpr int64_t kBeyond = int64_t(1) << 40;  // past any key length: the window bounds nothing
  if (p.pre_tokens >= kBeyond || next >= kBeyond) return nmax;
  const int64_t span = (p.pre_tokens + next + rows) / p.cmp_ratio + 1 + (aligned ? kSpanAlign - 1 : 0);
  return std::min(nmax, span);
}

int bounded_geometry_scores(const qli_problem& p, int64_t max_len, Bounded& g) {
  if (max_len < 0) return QLI_ERR_ARG;
  const bool tnd = p.layout_query == QLI_LAYOUT_TND;
  if (tnd && p.batch > kTndMaxBatch) return QLI_ERR_UNSUPPORTED;
  const int64_t nmax = max_len / p.cmp_ratio;
  if (nmax >= kMaxEntries) return QLI_ERR_SIZE;
  if ((nmax + p.block_size - 1) / p.block_size > p.max_blocks_per_seq) return QLI_ERR_ARG;
  std::memset(&g, 0, sizeof(g));
  g.tab_off = -1;
  PlanHeader& h = g.h;
  const int64_t rows = tnd ? (int64_t)p.s1 : (int64_t)p.batch * p.s1;
  const int k = p.sparse_count;
  h.rows = rows;
  // More than 4 query rows per batch (and TND, whose rows per batch are known
  // only on the device): groups of 4 rows that follow from the item's
  // position, each chunked like the decode items of qli_plan, all batches
  // sized for the bound.  Otherwise decode items derived on the device.
  const bool tiles = tnd || p.s1 > kMaxItemRows;
  h.kind = tiles ? kKindTiles : kKindDecode;
  h.rows_per_item = tiles ? kMaxItemRows : (p.s1 <= 1 ? 1 : (p.s1 <= 2 ? 2 : 4));
  if (rows == 0) return QLI_OK;
  // Entries one row sees (its workspace region) and an item's rows see
  // together (its chunks, from the item's start): nmax without a window.
  const int64_t row_span = window_span(p, nmax, 1, false);
  const int64_t span = window_span(p, nmax, tiles ? kMaxItemRows : p.s1, true);
  g.span = span;
  // TND: at most tnd_groups groups (the real ones, then padding-only ones)
  const int64_t groups = tnd ? tnd_groups(p.batch, p.s1)
                             : (int64_t)p.batch * ((p.s1 + kMaxItemRows - 1) / kMaxItemRows);
  h.chunk = tiles ? decode_chunk_for([&](int c) { return groups * ((span + c - 1) / c); }, true)
                  : decode_chunk_equal(p.batch, (int32_t)span);
  h.reg_chunks = (int32_t)std::max<int64_t>(1, (span + h.chunk - 1) / h.chunk);
  h.reg_rows = p.s1;
  h.reg_maxv = (int32_t)nmax;
  const int64_t items = (tiles ? groups : (int64_t)p.batch) * h.reg_chunks;
  if (items > INT32_MAX) return QLI_ERR_SIZE;
  h.n_items = (int32_t)items;
  // TND of many batches: the row and group tables follow whatever the
  // selection needs (fewer batches: the kernels derive the partition)
  auto add_tables = [&]() {
    if (!tnd || p.batch <= kTndInKernelBatches) return;
    g.tab_off = align16(h.workspace_bytes);
    h.workspace_bytes = g.tab_off + 4 * tnd_tables(p.batch, p.s1).total;
  };
  if (row_span <= k) {  // every row is written by the scoring kernel
    add_tables();
    return QLI_OK;
  }
  auto pad4 = [](int64_t n) { return (n + 3) & ~int64_t(3); };
  g.nseg = (int32_t)((row_span + kSelSegment - 1) / kSelSegment);
  g.stride = pad4(row_span);
  g.merge_base = rows * g.stride;
  g.mstride = g.nseg > 1 ? pad4((int64_t)g.nseg * k) : 0;
  const int64_t total = g.merge_base + rows * g.mstride;
  if (rows * g.nseg > INT32_MAX) return QLI_ERR_SIZE;
  h.n_select = (int32_t)(rows * g.nseg);
  h.max_cand = (int32_t)std::min<int64_t>(row_span, kSelSegment);
  if (g.nseg > 1) {
    h.n_select2 = (int32_t)rows;
    h.max_cand2 =
        (g.nseg - 1) * k + (int32_t)std::min<int64_t>(k, row_span - (int64_t)(g.nseg - 1) * kSelSegment);
  }
  h.ws_scores = total;
  // key indices for the merge regions only (see build_plan)
  h.ws_index_offset = align16(total * 4) - g.merge_base * 4;
  h.workspace_bytes = g.nseg > 1 ? align16(total * 4) + (total - g.merge_base) * 4 : total * 4;
  add_tables();
  return QLI_OK;
}

int bounded_geometry(const qli_problem& p, int64_t max_len, Bounded& g) {
  const int rc = bounded_geometry_scores(p, max_len, g);
  if (rc != QLI_OK) return rc;
  g.items_off = -1;
  g.plan_in_kernel = false;
  PlanHeader& h = g.h;
  if (h.kind == kKindDecode && h.rows > 0) {
    // decode: items derived on the device from the lengths, by every scoring
    // workgroup for few batches, else by decode_items_kernel into a table
    // after the scores; h.n_items bounds their number for the launch
    const int64_t cap = device_items_capacity(p.batch, g.span);
    if (cap > INT32_MAX) return QLI_ERR_SIZE;
    h.n_items = (int32_t)cap;
    h.reg_chunks = 0;
    if (p.batch <= kPlanInKernelBatches) {
      // The launch only bounds the persistent grid: size it as for every batch
      // at the bound (each workgroup runs the split's prologue, so idle ones
      // are not free); items beyond it run in later rounds.
      g.plan_in_kernel = true;
      const int c = decode_chunk_equal(p.batch, (int32_t)g.span);
      h.n_items = (int32_t)std::min<int64_t>(cap, std::max<int64_t>(1, (g.span + c - 1) / c) * p.batch);
    } else {
      g.items_off = align16(h.workspace_bytes);
      g.count_off = g.items_off + (int64_t)sizeof(Item) * cap;
      h.workspace_bytes = g.count_off + 16;
    }
  }
  add_values_region(p, h);
  return QLI_OK;
}

// The values the kernels write: the caller's, or the workspace region kept
// for the score ordering.
float* values_target(const RunArgs& a, float* sparse_values) {
  if (a.p->return_value) return sparse_values;
  if (a.hdr->ws_values_offset >= 0)
    return reinterpret_cast<float*>(static_cast<uint8_t*>(a.workspace) + a.hdr->ws_values_offset);
  return nullptr;
}

static int run_common(const qli_problem* p, const void* plan_host, const void* plan_dev,
                      const void* query, const void* key, const void* weights,
                      const void* q_scale, const void* k_scale, const int32_t* block_table,
                      void* workspace, int32_t* sparse_indices, float* sparse_values,
                      int64_t row0, int64_t row1, int64_t cols, void* dots_out,
                      float* scores_out, bool dump, int stages, void* stream) {
  int rc = validate_problem(p);
  if (rc != QLI_OK) return rc;
  if (!plan_matches(p, plan_host)) return QLI_ERR_PLAN;
  RunArgs a;
  a.p = p;
  a.plan_dev = plan_dev;
  a.hdr = plan_header(plan_host);
  a.query = query;
  a.key = key;
  a.weights = weights;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.block_table = block_table;
  a.workspace = workspace;
  a.sparse_indices = sparse_indices;
  a.sparse_values = p->return_value ? sparse_values : nullptr;
  a.dump_row0 = row0;
  a.dump_row1 = row1;
  a.dump_cols = cols;
  a.dots_out = dots_out;
  a.scores_out = scores_out;
  a.stream = stream;
  rc = check_run_args(a);
  if (rc != QLI_OK) return rc;
  if (dump) {
    if (row0 < 0 || row1 < row0 || row1 > a.hdr->rows || cols < 0) return QLI_ERR_ARG;
    if (row1 > row0 && cols > 0 && (!dots_out || !scores_out)) return QLI_ERR_ARG;
  }
  if (stages < 1 || stages > 3) return QLI_ERR_ARG;
  if (a.hdr->rows == 0) return QLI_OK;
  a.sparse_values = values_target(a, a.sparse_values);
  if ((stages & 1) && launch_score(a, dump) != 0) return QLI_ERR_HIP;
  if ((stages & 2) && a.hdr->n_select > 0 && launch_select(a) != 0) return QLI_ERR_HIP;
  if ((stages & 2) && a.hdr->sort_output && launch_sort(a) != 0) return QLI_ERR_HIP;
  return QLI_OK;
}

QLI_EXPORT int qli_run(const qli_problem* p, const void* plan_host, const void* plan_dev,
                       const void* query, const void* key, const void* weights,
                       const void* q_scale, const void* k_scale, const int32_t* block_table,
                       void* workspace, int32_t* sparse_indices, float* sparse_values,
                       void* stream) {
  return run_common(p, plan_host, plan_dev, query, key, weights, q_scale, k_scale, block_table,
                    workspace, sparse_indices, sparse_values, 0, 0, 0, nullptr, nullptr, false,
                    3, stream);
}

QLI_EXPORT int qli_run_stage(const qli_problem* p, const void* plan_host, const void* plan_dev,
                             const void* query, const void* key, const void* weights,
                             const void* q_scale, const void* k_scale,
                             const int32_t* block_table, void* workspace,
                             int32_t* sparse_indices, float* sparse_values, int32_t stages,
                             void* stream) {
  return run_common(p, plan_host, plan_dev, query, key, weights, q_scale, k_scale, block_table,
                    workspace, sparse_indices, sparse_values, 0, 0, 0, nullptr, nullptr, false,
                    stages, stream);
}

QLI_EXPORT int qli_bounded_workspace(const qli_problem* p, int64_t max_seq_len_key, size_t* workspace_bytes) {
  try {
    int rc = validate_problem(p);
    if (rc != QLI_OK) return rc;
    if (!workspace_bytes) return QLI_ERR_ARG;
    Bounded g;
    rc = bounded_geometry(*p, max_seq_len_key, g);
    if (rc != QLI_OK) return rc;
    *workspace_bytes = (size_t)g.h.workspace_bytes;
    return QLI_OK;
  } catch (...) {
    return QLI_ERR_SIZE;
  }
}

// static_ws: use the library's static workspace (workspace is ignored).
static int run_bounded_common(const qli_problem* p, int64_t max_seq_len_key, const int32_t* aslq_dev,
                              const int32_t* aslk_dev, const void* query, const void* key, const void* weights,
                              const void* q_scale, const void* k_scale, const int32_t* block_table,
                              void* workspace, int32_t* sparse_indices, float* sparse_values, void* stream,
                              bool static_ws = false) {
  int rc = validate_problem(p);
  if (rc != QLI_OK) return rc;
  Bounded g;
  rc = bounded_geometry(*p, max_seq_len_key, g);
  if (rc != QLI_OK) return rc;
  if (static_ws && g.h.workspace_bytes > (int64_t)kScratchBytes) return QLI_ERR_SIZE;
  if (g.h.rows == 0) return QLI_OK;
  if (!aslk_dev || ((uintptr_t)aslk_dev % 4) != 0) return QLI_ERR_ARG;
  const bool tnd = p->layout_query == QLI_LAYOUT_TND;
  if (tnd && (!aslq_dev || ((uintptr_t)aslq_dev % 4) != 0)) return QLI_ERR_ARG;
  if (aslq_dev && ((uintptr_t)aslq_dev % 4) != 0) return QLI_ERR_ARG;
  RunArgs a;
  a.p = p;
  a.plan_dev = nullptr;
  a.hdr = &g.h;
  a.query = query;
  a.key = key;
  a.weights = weights;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.block_table = block_table;
  a.workspace = workspace;
  a.sparse_indices = sparse_indices;
  a.sparse_values = p->return_value ? sparse_values : nullptr;
  a.dump_row0 = a.dump_row1 = a.dump_cols = 0;
  a.dots_out = nullptr;
  a.scores_out = nullptr;
  a.stream = stream;
  a.aslk = aslk_dev;
  a.max_len = max_seq_len_key;
  a.stride = g.stride;
  a.mstride = g.mstride;
  a.merge_base = g.merge_base;
  a.nseg = g.nseg;
  if (tnd) {
    a.aslq = aslq_dev;
    a.tab_off = g.tab_off;
  } else {
    a.aslq_bsnd = aslq_dev;  // null: every row of every batch is used
  }
  a.items_off = g.items_off;
  a.count_off = g.count_off;
  a.plan_in_kernel = g.plan_in_kernel;
  rc = check_run_args(a, static_ws);
  if (rc != QLI_OK) return rc;
  if (static_ws && g.h.workspace_bytes > 0 && scratch_address(&a.workspace) != 0) return QLI_ERR_HIP;
  a.sparse_values = values_target(a, a.sparse_values);
  if (tnd && g.tab_off >= 0 && launch_tnd_tables(a) != 0) return QLI_ERR_HIP;
  if (launch_decode_items(a) != 0) return QLI_ERR_HIP;
  if (launch_score(a, false) != 0) return QLI_ERR_HIP;
  if (g.h.n_select > 0 && launch_select(a) != 0) return QLI_ERR_HIP;
  if (g.h.sort_output && launch_sort(a) != 0) return QLI_ERR_HIP;
  return QLI_OK;
}

QLI_EXPORT int qli_run_bounded(const qli_problem* p, int64_t max_seq_len_key, const int32_t* aslk_dev,
                               const void* query, const void* key, const void* weights,
                               const void* q_scale, const void* k_scale, const int32_t* block_table,
                               void* workspace, int32_t* sparse_indices, float* sparse_values,
                               void* stream) {
  try {
    if (p && p->layout_query == QLI_LAYOUT_TND) return QLI_ERR_UNSUPPORTED;  // needs the query lengths
    return run_bounded_common(p, max_seq_len_key, nullptr, aslk_dev, query, key, weights, q_scale, k_scale,
                              block_table, workspace, sparse_indices, sparse_values, stream);
  } catch (...) {
    return QLI_ERR_ARG;
  }
}

QLI_EXPORT int qli_run_bounded_aslq(const qli_problem* p, int64_t max_seq_len_key, const int32_t* aslq_dev,
                                    const int32_t* aslk_dev, const void* query, const void* key,
                                    const void* weights, const void* q_scale, const void* k_scale,
                                    const int32_t* block_table, void* workspace, int32_t* sparse_indices,
                                    float* sparse_values, void* stream) {
  try {
    if (p && p->layout_query != QLI_LAYOUT_BSND) return QLI_ERR_UNSUPPORTED;
    if (!aslq_dev) return QLI_ERR_ARG;
    return run_bounded_common(p, max_seq_len_key, aslq_dev, aslk_dev, query, key, weights, q_scale, k_scale,
                              block_table, workspace, sparse_indices, sparse_values, stream);
  } catch (...) {
    return QLI_ERR_ARG;
  }
}

QLI_EXPORT int qli_run_bounded_tnd(const qli_problem* p, int64_t max_seq_len_key, const int32_t* aslq_dev,
                                   const int32_t* aslk_dev, const void* query, const void* key,
                                   const void* weights, const void* q_scale, const void* k_scale,
                                   const int32_t* block_table, void* workspace, int32_t* sparse_indices,
                                   float* sparse_values, void* stream) {
  try {
    if (p && p->layout_query != QLI_LAYOUT_TND) return QLI_ERR_UNSUPPORTED;
    return run_bounded_common(p, max_seq_len_key, aslq_dev, aslk_dev, query, key, weights, q_scale, k_scale,
                              block_table, workspace, sparse_indices, sparse_values, stream);
  } catch (...) {
    return QLI_ERR_ARG;
  }
}

QLI_EXPORT int qli_run_bounded_static(const qli_problem* p, int64_t max_seq_len_key, const int32_t* aslk_dev,
                                      const void* query, const void* key, const void* weights,
                                      const void* q_scale, const void* k_scale, const int32_t* block_table,
                                      int32_t* sparse_indices, float* sparse_values, void* stream) {
  try {
    if (p && p->layout_query == QLI_LAYOUT_TND) return QLI_ERR_UNSUPPORTED;  // needs the query lengths
    return run_bounded_common(p, max_seq_len_key, nullptr, aslk_dev, query, key, weights, q_scale, k_scale,
                              block_table, nullptr, sparse_indices, sparse_values, stream, true);
  } catch (...) {
    return QLI_ERR_ARG;
  }
}

QLI_EXPORT int qli_run_debug(const qli_problem* p, const void* plan_host, const void* plan_dev,
                             const void* query, const void* key, const void* weights,
                             const void* q_scale, const void* k_scale,
                             const int32_t* block_table, void* workspace,
                             int32_t* sparse_indices, float* sparse_values, int64_t row0,
                             int64_t row1, int64_t cols, void* dots_out, float* scores_out,
                             void* stream) {
  return run_common(p, plan_host, plan_dev, query, key, weights, q_scale, k_scale, block_table,
                    workspace, sparse_indices, sparse_values, row0, row1, cols, dots_out,
                    scores_out, true, 3, stream);
}
