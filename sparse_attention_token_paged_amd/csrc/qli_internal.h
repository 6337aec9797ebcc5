// qli_internal.h -- plan layout shared by the host planner and the kernels.
//
// A plan is position-independent bytes: a header, then a row table, a
// score-item table and the list of rows that need a selection.  The host
// reads the header for launch geometry; the kernels read the device copy.
#pragma once
#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "../../include/qli.h"

namespace qli {

constexpr uint32_t kPlanMagic = 0x504C4951u;  // "QILP"
constexpr uint32_t kPlanVersion = 8;
constexpr int kHeads = 64;       // query heads (QLI-README 约束说明)
constexpr int kDim = 128;        // head dim of query and key (约束说明)
constexpr int kTileKeys = 64;    // keys per MFMA tile step (4 n-tiles of 16)
constexpr int kMaxChunk = 4096;  // keys per work item, upper bound
constexpr int kCUs = 256;                 // compute units of one MI355X
constexpr int kDecodeSlots = 3 * kCUs;    // decode workgroups resident at once (3 per CU)
constexpr int kMaxEntries = 1 << 22;      // compressed entries per sequence (exact reciprocal division)
constexpr int kMaxItemRows = 4;           // rows carried inline by a decode item

// kKindDecode: items of 1, 2 or 4 rows from a plan's table, a device-built
// table or the scoring kernel's own split.  kKindTiles: bounded runs of more
// than 4 query rows per batch (and TND), whose 4-row groups follow from the
// item's position.  One kernel scores both.
enum PlanKind : int32_t { kKindDecode = 0, kKindTiles = 1 };
enum ItemFlags : int32_t { kItemPad = 1 };

struct PlanHeader {
  uint32_t magic;
  uint32_t version;
  uint64_t fingerprint;      // hash of the problem fields the plan depends on
  int64_t plan_bytes;
  int64_t workspace_bytes;
  int64_t rows;              // output rows
  int64_t visible_pairs;     // sum of visible counts
  int64_t ws_scores;         // fp32 candidate scores staged in the workspace
  int64_t off_rows;          // byte offset of RowInfo[rows]
  int64_t off_items;         // byte offset of Item[n_items]
  int64_t off_select;        // byte offset of SelectEntry[n_select]
  int32_t kind;              // PlanKind
  int32_t rows_per_item;     // 1, 2 or 4
  int32_t n_items;
  int32_t n_select;
  int32_t chunk;             // the chunk rule's length: no work item covers more keys
  int32_t max_vis;
  int32_t reserved1;
  int32_t max_cand;          // largest candidate count of a pass-1 selection
  int64_t key_entries;       // sum over batches of the entries some row of the batch sees
  int64_t table_entries;     // block-table entries spanned by those entries
  int64_t active_rows;       // rows with at least one visible entry
  int64_t ws_index_offset;   // the int32 key index of merge candidate e (an element offset of a
                             // merge region) sits at workspace byte ws_index_offset + 4e; only
                             // merge regions carry indices, stored after every score
  // Regular decode plans (every batch: the same rows, one group, the same
  // visible maximum): item i covers batch i / reg_chunks, keys from
  // (i % reg_chunks) * chunk, rows batch * reg_rows .. + reg_rows.  0 = not regular.
  int32_t reg_chunks;
  int32_t reg_rows;
  int32_t reg_maxv;
  int32_t n_select2;         // pass-2 selections (after the n_select pass-1 entries)
  int32_t max_cand2;         // largest candidate count of a pass-2 selection
  int32_t sort_output;       // 1: each row's slots are reordered by score after the selection
  int32_t reserved2[2];
  int64_t ws_values_offset;  // byte offset of [rows, k] fp32 values kept in the workspace for the
                             // reordering when the caller takes no values; -1 = none
  int64_t reserved3;
};
static_assert(sizeof(PlanHeader) % 16 == 0, "header keeps the tables aligned");

// Row r sees the compressed entries [lo, vis): vis - lo of them (lo = 0
// without a pre_tokens window).
struct RowInfo {
  int32_t batch;   // -1 for rows that belong to no query token
  int32_t vis;     // end of the visible range
  int64_t ws_off;  // element offset of the row's candidates in the workspace, -1 = direct output;
                   // candidate e is entry lo + e
  int32_t ncand;   // scores the row stages for the selection stage (0: direct output)
  int32_t lo;      // start of the visible range
};

// One selection of the selection stage: the top min(k, n) of n candidates.
// Pass 1 holds the rows of at most kSelSegment candidates (final) and the
// segments of longer rows; pass 2 merges each long row's segment results.
struct SelectEntry {
  int64_t src_off;  // element offset of the candidate scores (a multiple of 4); their
                    // key indices sit at the same offset of the index region when indexed
  int64_t dst_off;  // >= 0: write the winners as indexed candidates here; -1: final, to row `row`
  int32_t row;      // output row
  int32_t n;        // candidates
  int32_t base;     // key index of candidate 0 when they carry no indices
  int32_t indexed;  // 1: the candidates carry key indices (pass-2 merges)
};
constexpr int kSelSegment = 8192;  // candidates per first-pass selection of a long row
constexpr int kSpanAlign = 128;    // bounded runs: items start at a multiple of this many entries (one stage)

// Visible compressed entries of query i (of s1b) in a batch with skb original
// key tokens (QLI-README 参数说明 cmp_ratio and sparse_mode; the planner and
// the bounded decode kernels both use it).  Only floor(skb / cmp) whole
// entries exist; under mode 3 query i sits at token position skb - s1b + i
// and sees entry j once all of its tokens [j*cmp, (j+1)*cmp) are at or
// before that position.
#if defined(__HIPCC__)
__host__ __device__
#endif
inline int64_t visible_entries(int mode, int cmp, int64_t skb, int64_t s1b, int64_t i) {
  const int sh = __builtin_ctz((unsigned)cmp);  // cmp is a power of two: x / cmp == x >> sh for x >= 0
  const int64_t stored = skb >> sh;             // skb >= 0
  if (mode == 0) return stored;
  const int64_t through = skb - s1b + i + 1;  // tokens at or before the query
  if (through <= 0) return 0;
  return (through >> sh) < stored ? (through >> sh) : stored;
}

// The same query with pre_tokens / next_tokens windows (QLI-README 参数说明
// marks both reserved, default 2^63-1; reading for other values: the query
// sits at token position pos = skb - s1b + i in both modes and sees an entry
// only when all of its tokens lie in [pos - pre, pos + next]).  Returns the
// end of the visible range and sets lo to its start; an empty range is
// [0, 0).  pre, next >= 0.  Entry j's first token j*cmp >= pos - pre holds
// from j = ceil((pos - pre) / cmp); its last token (j+1)*cmp - 1 <= pos + next
// holds below floor((pos + next + 1) / cmp), a bound that cuts nothing once
// next >= s1b (then pos + next + 1 >= skb).
#if defined(__HIPCC__)
__host__ __device__
#endif
inline int64_t visible_window(int mode, int cmp, int64_t skb, int64_t s1b, int64_t i, int64_t pre, int64_t next,
                              int64_t& lo) {
  const int sh = __builtin_ctz((unsigned)cmp);  // the divisions below take positive operands
  int64_t hi = visible_entries(mode, cmp, skb, s1b, i);
  const int64_t pos = skb - s1b + i;
  lo = pre < pos ? (pos - pre + cmp - 1) >> sh : 0;
  if (next < s1b) {
    const int64_t end = pos + next + 1;  // tokens before end are inside the window
    const int64_t cut = end > 0 ? end >> sh : 0;
    if (cut < hi) hi = cut;
  }
  if (hi <= lo) lo = hi = 0;
  return hi;
}
static_assert(sizeof(SelectEntry) == 32, "select table layout");

// Window sides as the bounded kernels take them: clamped to 2^30, which
// changes no visible range, since positions and row counts stay below it
// (keys below 2^22 entries of at most 128 tokens; rows below 2^30).
constexpr int32_t kWindowCap = int32_t(1) << 30;
inline int32_t window_side(int64_t v) { return v < kWindowCap ? (int32_t)v : kWindowCap; }

struct Item {
  int32_t row0;    // first global row
  int32_t nrows;   // rows in the item (same batch), <= rows_per_item
  int32_t batch;   // batch whose keys are scored (-1: padding only)
  int32_t key0;    // first key entry of the chunk
  int32_t nkeys;   // entries in the chunk (0: padding only)
  int32_t flags;   // kItemPad: this item writes the -1 padding of its rows
  int32_t reserved[2];
  int32_t vis[kMaxItemRows];       // decode items: end of the visible range of row row0 + u
  int64_t cand_off[kMaxItemRows];  // decode items: workspace slot of entry key0 of row u
                                   // (the row's region starts at its entry lo), -1 = direct output
  int32_t lo[kMaxItemRows];        // decode items: start of the visible range of row row0 + u
};
static_assert(sizeof(Item) == 96, "item layout");

// Bounded TND runs of at most kTndInKernelBatches batches derive the batch
// partition inside the kernels (the scoring kernel keeps row ends and group
// starts in LDS, two per lane of a wave; the selection re-derives a row's
// batch in one wave).  More batches (up to kTndMaxBatch): tables written into
// the workspace (at byte offset tab_off, int32 elements) by a one-workgroup
// kernel from the device actual_seq_lengths_query, before the scoring kernel:
//   rows_end[B]          running maximum of the prefix sums clamped to [0, T]:
//                        batch b owns rows [rows_end[b-1], rows_end[b])
//   group_start[B + 1]   4-row groups of the batches before b
//   group_batch[groups]  batch of each group, -1 past the last real group
//   row_batch[T]         batch of each row, -1 for rows past rows_end[B-1]
// groups = T / 4 + B + 2 bounds the real groups (at most T/4 + B) plus the
// groups of rows that belong to no batch (padding only).
constexpr int kTndMaxBatch = 4096;  // the table kernel keeps both prefix tables in LDS
// 1 KB of LDS per scoring workgroup, which still fits three per CU
constexpr int kTndInKernelBatches = 128;
struct TndTables {
  int64_t rows_end, group_start, group_batch, row_batch, total;  // element offsets, element count
};
inline int64_t tnd_groups(int64_t batch, int64_t t) { return t / kMaxItemRows + batch + 2; }
inline TndTables tnd_tables(int64_t batch, int64_t t) {
  TndTables x;
  x.rows_end = 0;
  x.group_start = (batch + 3) & ~int64_t(3);
  x.group_batch = x.group_start + ((batch + 1 + 3) & ~int64_t(3));
  x.row_batch = x.group_batch + ((tnd_groups(batch, t) + 3) & ~int64_t(3));
  x.total = x.row_batch + t;
  return x;
}

inline const PlanHeader* plan_header(const void* plan) {
  return static_cast<const PlanHeader*>(plan);
}

uint64_t problem_fingerprint(const qli_problem& p);

// Kernel launchers (qli_kernels.hip).  Return a hipError_t value.
struct RunArgs {
  const qli_problem* p;
  const void* plan_dev;
  const PlanHeader* hdr;
  const void* query;
  const void* key;
  const void* weights;
  const void* q_scale;
  const void* k_scale;
  const int32_t* block_table;
  void* workspace;
  int32_t* sparse_indices;
  float* sparse_values;
  int64_t dump_row0, dump_row1, dump_cols;
  void* dots_out;
  float* scores_out;
  void* stream;
  // Bounded runs (no host plan; aslk != nullptr): the kernels read the key
  // lengths and clamp them to max_len tokens; decode items come from the
  // table decode_items_kernel builds, prefill items and each selection are
  // derived from the lengths directly.  Row r's scores sit at element
  // r * stride, its merge candidates at merge_base + r * mstride; nseg
  // segments per row.
  const int32_t* aslk = nullptr;
  int64_t max_len = 0;
  int64_t stride = 0, mstride = 0, merge_base = 0;
  int32_t nseg = 0;
  // Bounded TND runs: device actual_seq_lengths_query and the byte offset of
  // the tables (TndTables) in the workspace, -1 for none (few batches: the
  // kernels derive the partition themselves).
  const int32_t* aslq = nullptr;
  int64_t tab_off = -1;
  // Bounded BSND runs with actual_seq_lengths_query on the device (rows past a
  // batch's count see nothing), else null.
  const int32_t* aslq_bsnd = nullptr;
  // Bounded decode: byte offsets in the workspace of the item table the device
  // planner builds (decode_items_kernel) and of its item count; -1 = none.
  int64_t items_off = -1, count_off = 0;
  // Bounded decode with at most kPlanInKernelBatches batches: every scoring
  // workgroup derives the same split itself (no table, no extra launch).
  bool plan_in_kernel = false;
};

// Batches up to which bounded decode plans inside the scoring kernel (one
// batch per thread of a 256-thread workgroup); larger batches use the table.
constexpr int kPlanInKernelBatches = 256;

// Bounded decode's device-built item table: one workgroup picks the chunk as
// qli_plan does (the smallest multiple of 128 entries whose items fit the
// decode slots; for equal batches the one that lowers the busiest CU's keys)
// and writes max(1, ceil(span / chunk)) items per batch, span being the
// entries its rows see together.  Upper bound on their number, for the
// workspace, when no batch's span exceeds `span`.
inline int64_t device_items_capacity(int64_t batch, int64_t span) {
  const int64_t most = batch * std::max<int64_t>(1, (span + kMaxChunk - 1) / kMaxChunk);
  return std::max<int64_t>(kDecodeSlots + batch, most);
}
int launch_score(const RunArgs& a, bool dump);

// The allocation-free bounded runs' workspace: kScratchBytes of device memory
// per GPU (a file-scope array of qli_kernels.hip).  scratch_address() writes
// the current device's address of it (looked up once per device); returns a
// hipError_t value.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
int scratch_address(void** out);
int launch_select(const RunArgs& a);
int launch_sort(const RunArgs& a);
int launch_decode_items(const RunArgs& a);
int launch_tnd_tables(const RunArgs& a);

}  // namespace qli
