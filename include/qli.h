/*
 * qli.h -- C ABI of the quantized lightning indexer for AMD MI355X (gfx950).
 *
 * The operation is the one defined on the EngineX-Ascend page
 * "VllmQuantLightningIndexer" (csrc/attention/vllm_quant_lightning_indexer/
 * README.md; cited below as QLI-README with its section headings):
 *
 *   out = Top-k{ [1]_{1xg} @ [ (W @ [1]_{1xSk}) (.) ReLU( (ScaleQ @ ScaleK^T)
 *                                                  (.) (Q_index @ K_index^T) ) ] }
 *   (QLI-README, section 功能说明, formula and steps 1-3)
 *
 * For every query token (row) and every key entry it may see, the score is
 *   score[r][j] = sum_{g<64} W[r][g] * max(0, ScaleQ[r][g] * ScaleK[j] * dot(Q[r][g], K[j]))
 * and the row returns the indices of its sparse_count highest scores.
 *
 * Two calls, as on the page (metadata op, then indexer op):
 *   qli_plan  host only: validates the scalar problem and the sequence
 *             lengths and writes a work-split plan (our replacement for the
 *             page's int32[1024] metadata, QLI-README 参数说明 "metadata").
 *   qli_run   stream-ordered GPU execution of the whole hot path.
 *
 * Conventions for every entry point:
 *   - All buffers are owned by the caller.  The library allocates no device
 *     memory at run time and keeps no state between calls; calls are
 *     thread-safe.  One exception, for callers that cannot allocate:
 *     qli_run_bounded_static works in a static device workspace that every
 *     GPU the library is loaded on holds from load to process exit.
 *   - Device pointers are plain HIP device addresses; "stream" is a
 *     hipStream_t passed as void* (NULL = the default stream).
 *   - Every scalar argument is validated before anything is launched; a
 *     violation returns a distinct qli_status and touches nothing.
 *   - Device-resident data (tensor contents, block_table entries) is not
 *     validated.  Out-of-contract values (NaN/Inf inputs, negative or
 *     non-finite dequant scales, block ids outside [0, num_blocks)) give
 *     undefined results, as the page leaves NaN ordering undefined
 *     (QLI-README 约束说明).
 *   - No C++ exception crosses the ABI.
 */
#ifndef QLI_H
#define QLI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum qli_status {
    QLI_OK = 0,
    QLI_ERR_ARG = 1,         /* an argument breaks a constraint of the page or of this ABI */
    QLI_ERR_UNSUPPORTED = 2, /* allowed by the page on some hardware, not supported here */
    QLI_ERR_SIZE = 3,        /* a caller buffer is too small, or a size overflows */
    QLI_ERR_HIP = 4,         /* the HIP runtime reported an error (launch, device) */
    QLI_ERR_PLAN = 5         /* the plan does not belong to this problem or is corrupt */
} qli_status;

/* query / key element type (QLI-README 参数说明: INT8, FLOAT8_e4m3fn). */
typedef enum qli_qk_dtype { QLI_QK_INT8 = 0, QLI_QK_FP8_E4M3FN = 1 } qli_qk_dtype;
/* weights / dequant-scale element type (QLI-README 参数说明: FLOAT16, FLOAT32).
 * Pairings accepted (the page's per-product notes): INT8 with FLOAT16 and
 * FLOAT8_e4m3fn with FLOAT32; other mixes return QLI_ERR_UNSUPPORTED. */
typedef enum qli_scale_dtype { QLI_SCALE_F16 = 0, QLI_SCALE_F32 = 1 } qli_scale_dtype;
/* layout_query (QLI-README 参数说明: BSND or TND).  layout_key is always
 * PA_BSND (paged). */
typedef enum qli_layout { QLI_LAYOUT_BSND = 0, QLI_LAYOUT_TND = 1 } qli_layout;

/* The scalar problem (QLI-README 参数说明 attributes and shapes).  Fields
 * are fixed-width and explicitly padded so that the struct has the same
 * layout from every language. */
/* pre_tokens / next_tokens: the page lists both as reserved attributes that
 * bound how many tokens before (after) a query the attention relates to, and
 * accepts only 2^63-1.  Other values (>= 0; negative ones are QLI_ERR_ARG)
 * are taken as a token window: query i of a batch with S1 query and Sk key
 * tokens sits at position pos = Sk - S1 + i (both sparse modes), and sees a
 * compressed entry only when sparse_mode lets it and every token the entry
 * covers lies in [pos - pre_tokens, pos + next_tokens].  A row's visible
 * entries are then consecutive, [lo, hi); its outputs list the top
 * min(k, hi - lo) of them, padded as usual.  Planned and bounded runs. */
typedef struct qli_problem {
    int32_t batch;              /* B.  TND: number of entries of actual_seq_lengths_query */
    int32_t s1;                 /* BSND: S1 (query tokens per batch); TND: T (total tokens) */
    int32_t num_heads_q;        /* must be 64 (约束说明) */
    int32_t num_heads_k;        /* must be 1 (约束说明) */
    int32_t head_dim;           /* must be 128 (约束说明) */
    int32_t layout_query;       /* qli_layout */
    int32_t qk_dtype;           /* qli_qk_dtype */
    int32_t scale_dtype;        /* qli_scale_dtype */
    int32_t num_blocks;         /* key cache blocks, >= 1 */
    int32_t block_size;         /* multiple of 16, 16..1024 (约束说明) */
    int32_t max_blocks_per_seq; /* second dim of block_table, >= blocks any sequence needs */
    int32_t reserved0;          /* must be 0 */
    int64_t key_block_stride;   /* "stride" of key's first axis (参数说明) in elements (= bytes);
                                   0 = block_size*128; else >= block_size*128 and a multiple of 16 */
    int32_t sparse_count;       /* k, 1..2048 (参数说明 sparse_count) */
    int32_t sparse_mode;        /* 0 defaultMask, 3 rightDownCausal (参数说明 sparse_mode) */
    int32_t cmp_ratio;          /* 1,2,4,...,128 (参数说明 cmp_ratio) */
    int32_t reserved1;          /* must be 0 */
    int64_t pre_tokens;         /* token window, >= 0; INT64_MAX (the page's default) = none */
    int64_t next_tokens;        /* token window, >= 0; INT64_MAX (the page's default) = none */
    int32_t query_quant_mode;   /* must be 0 (per-token-head) */
    int32_t key_quant_mode;     /* must be 0 (per-token-head) */
    int32_t return_value;       /* 1: also write sparse_values; 0: sparse_values may be NULL */
    int32_t sort_output;        /* 0: slots in ascending index order; 1: in descending score order */
} qli_problem;

/* Static description of the string for a status code (never NULL). */
const char *qli_status_string(int status);

/*
 * qli_plan -- host-side work split (QLI-README 参数说明 "metadata" and the
 * VllmQuantLightningIndexerMetadata call of the page's examples).
 *
 *   p          the problem; validated as qli_run validates it.
 *   aslq       host int32[batch]: actual_seq_lengths_query.  BSND: query
 *              tokens used per batch (each in 0..S1); NULL means S1 for all.
 *              TND: required; non-decreasing prefix sums, last <= T
 *              (约束说明).  Rows past a batch's count are padded outputs.
 *   aslk       host int32[batch], required: actual_seq_lengths_key, the
 *              ORIGINAL key tokens per batch (>= 0).  The cache stores
 *              floor(aslk / cmp_ratio) compressed entries per batch, which
 *              must fit in max_blocks_per_seq blocks.
 *   plan       host buffer of plan_capacity bytes, or NULL to query sizes.
 *   plan_bytes       out: bytes the plan needs (always written on QLI_OK or
 *                    QLI_ERR_SIZE).
 *   workspace_bytes  out: device workspace qli_run needs (may be 0).
 *
 * Returns QLI_ERR_SIZE when plan != NULL and plan_capacity < *plan_bytes.
 * The plan is position-independent bytes: copy it verbatim to the device
 * and pass both copies to qli_run.
 */
int qli_plan(const qli_problem *p, const int32_t *aslq, const int32_t *aslk,
             void *plan, size_t plan_capacity, size_t *plan_bytes,
             size_t *workspace_bytes);

/* Summary of a plan, for callers that size buffers or report throughput. */
typedef struct qli_plan_info {
    int64_t rows;            /* output rows: B*S1 (BSND) or T (TND) */
    int64_t visible_pairs;   /* sum over rows of visible key entries (scored pairs) */
    int64_t plan_bytes;
    int64_t workspace_bytes;
    int64_t key_entries;     /* key entries some row sees: sum over batches of the span from
                                the smallest window start to the largest visible end (each is
                                read once per batch) */
    int64_t table_entries;   /* block_table entries those key entries span */
    int64_t active_rows;     /* rows that see at least one key entry */
    int32_t score_items;     /* work items of the scoring stage */
    int32_t select_rows;     /* rows whose visible count exceeds sparse_count */
    int32_t rows_per_item;
    int32_t keys_per_chunk;
    int32_t kind;            /* 0 (qli_plan's items: rows_per_item rows of one batch x a key
                                chunk); other values are reserved */
    int32_t reserved;
} qli_plan_info;

int qli_plan_info_get(const void *plan_host, qli_plan_info *info);

/*
 * qli_run -- the indexer (QLI-README 功能说明 formula; 参数说明 inputs and
 * outputs).  Stream-ordered, no host synchronisation.
 *
 *   plan_host     the bytes qli_plan wrote (host), for launch geometry.
 *   plan_dev      a device copy of the same bytes (read by the kernels).
 *   query         device [B,S1,64,128] (BSND) or [T,64,128] (TND), 8-bit.
 *   key           device paged cache [num_blocks, block_size, 1, 128],
 *                 consecutive blocks key_block_stride bytes apart, 16-byte
 *                 aligned.
 *   weights       device [B,S1,64] or [T,64], scale dtype, contiguous.
 *   q_scale       device query_dequant_scale, same shape/dtype as weights.
 *   k_scale       device key_dequant_scale [num_blocks, block_size, 1],
 *                 contiguous.
 *   block_table   device int32 [B, max_blocks_per_seq]; entry [b][i] is the
 *                 cache block holding entries i*block_size .. of batch b.
 *   workspace     device, workspace_bytes from qli_plan (NULL if 0).
 *   Alignment (QLI_ERR_ARG otherwise): plan_dev, workspace, query and key
 *   16 bytes; weights / q_scale 8 bytes (FLOAT16) or 16 bytes (FLOAT32);
 *   k_scale its element size; block_table and the outputs 4 bytes.
 *   sparse_indices device int32 [rows, sparse_count] (out).
 *   sparse_values  device float [rows, sparse_count] (out) or NULL when
 *                  return_value == 0.
 *
 * Output contract per row r with n = min(sparse_count, visible(r)), where
 * visible(r) counts the row's visible entries (window applied):
 *   sparse_indices[r][0:n] = the indices of the n highest scores, ties at
 *   the threshold broken towards the lower index, listed in ascending index
 *   order (sort_output = 0) or in descending fp32 score order, equal scores
 *   by ascending index (sort_output = 1: the order in which the page's
 *   Top-k step ranks them); sparse_values[r][i] = the fp32 score of
 *   sparse_indices[r][i]; slots n..sparse_count-1 hold -1 and -INFINITY.
 *   With sort_output = 1 and return_value = 0 the workspace also holds the
 *   rows' values ([rows, sparse_count] fp32, counted in workspace_bytes).
 */
int qli_run(const qli_problem *p, const void *plan_host, const void *plan_dev,
            const void *query, const void *key, const void *weights,
            const void *q_scale, const void *k_scale,
            const int32_t *block_table, void *workspace,
            int32_t *sparse_indices, float *sparse_values, void *stream);

/*
 * qli_run_debug -- parity instrumentation: runs the same scoring kernels
 * with a dump epilogue for rows [row0, row1) and writes, for each visible
 * entry j < cols of row r (entry index j, window applied):
 *   dots_out   [(row1-row0), 64, cols]: int32 dot products (INT8 path) or
 *              float (FP8 path), exactly as the matrix cores produced them;
 *   scores_out [(row1-row0), cols] float scores.
 * Slots of entries the row does not see are left untouched.  It also performs
 * the full qli_run (same outputs).
 */
int qli_run_debug(const qli_problem *p, const void *plan_host,
                  const void *plan_dev, const void *query, const void *key,
                  const void *weights, const void *q_scale,
                  const void *k_scale, const int32_t *block_table,
                  void *workspace, int32_t *sparse_indices,
                  float *sparse_values, int64_t row0, int64_t row1,
                  int64_t cols, void *dots_out, float *scores_out,
                  void *stream);

/*
 * qli_run_stage -- qli_run restricted to one of its two stages, for
 * measuring each on its own: stages = 1 runs only the scoring kernel
 * (gather, contraction and epilogue; rows that see at most sparse_count
 * entries are finished here, the others stage every score in the
 * workspace), 2 only the selection (the segment top-k launch, then the
 * merge launch for rows longer than one segment), 3 both (= qli_run).
 * Stage 2 alone reads whatever the workspace holds from the last stage-1
 * run with the same plan and workspace; its outputs are meaningful only
 * after one.  Returns QLI_ERR_ARG for other values of stages; otherwise
 * errors are those of qli_run.
 */
int qli_run_stage(const qli_problem *p, const void *plan_host,
                  const void *plan_dev, const void *query, const void *key,
                  const void *weights, const void *q_scale,
                  const void *k_scale, const int32_t *block_table,
                  void *workspace, int32_t *sparse_indices,
                  float *sparse_values, int32_t stages, void *stream);

/*
 * Bounded runs: the indexer without a host plan, for serving loops that
 * keep actual_seq_lengths_key on the device and capture the call in a graph
 * once.  The page's metadata op runs on the device for the same reason
 * (QLI-README 参数说明 "metadata"; the operator supports graph mode); here the
 * launch geometry comes from a host bound on the key length alone, and the
 * kernels read the lengths themselves.
 *
 * Scope: qli_run_bounded takes the BSND query layout with every one of the
 * S1 query rows of every batch active (no actual_seq_lengths_query); any S1.
 * qli_run_bounded_aslq takes BSND with actual_seq_lengths_query
 * on the device; qli_run_bounded_tnd the TND layout with
 * actual_seq_lengths_query on the device too (batch <= 4096).  Every other
 * parameter as for qli_plan, pre_tokens / next_tokens windows included:
 * each row's range [lo, hi) is derived on the device from its position.
 *
 * Decode problems (BSND, S1 <= 4): every batch is split by its own length
 * into items with the chunk rule of qli_plan, by the scoring kernel itself
 * for up to 256 batches, else by a first one-workgroup kernel into an item
 * table in the workspace, so ragged lengths cost what they cost under
 * qli_plan.  More query rows per batch (and TND): groups of 4 rows whose
 * place follows from the item's position, every batch sized for the bound.
 * Under a window a batch's or group's items start at the smallest lo of its
 * rows (rounded down to 128 entries), and the workspace holds a row's window
 * rather than every entry up to the bound.
 *
 * qli_bounded_workspace -- workspace bytes that qli_run_bounded needs for
 *   these problem sizes and any key lengths in [0, max_seq_len_key] original
 *   tokens.  QLI_ERR_ARG if the bound breaks a constraint (it must be >= 0,
 *   its compressed entries must fit max_blocks_per_seq blocks),
 *   QLI_ERR_UNSUPPORTED outside the scope above.
 *
 * qli_run_bounded -- the same outputs as qli_plan + qli_run would give for
 *   actual_seq_lengths_key = aslk_dev[0..B) (device int32; each value is
 *   clamped to [0, max_seq_len_key], so reads stay within the bound).
 *   Stream-ordered, no host synchronisation, no host reads of device data:
 *   a graph captured once replays correctly after aslk_dev (or any input)
 *   changes.  workspace: qli_bounded_workspace bytes, 16-byte aligned.
 *   Other arguments, alignment and the output contract as for qli_run.
 */
int qli_bounded_workspace(const qli_problem *p, int64_t max_seq_len_key,
                          size_t *workspace_bytes);

int qli_run_bounded(const qli_problem *p, int64_t max_seq_len_key,
                    const int32_t *aslk_dev, const void *query,
                    const void *key, const void *weights,
                    const void *q_scale, const void *k_scale,
                    const int32_t *block_table, void *workspace,
                    int32_t *sparse_indices, float *sparse_values,
                    void *stream);

/*
 * qli_run_bounded_aslq -- qli_run_bounded for BSND with
 *   actual_seq_lengths_query on the device: aslq_dev (device int32[B], 4-byte
 *   aligned, required) gives the query rows used per batch; each value is
 *   clamped to [0, S1], so any contents are safe.  Rows past a batch's count
 *   see no entry and return only padding; the used rows' visibility follows
 *   from the count as in qli_plan (sparse_mode 3 aligns the last used row
 *   with the last key).  The workspace is qli_bounded_workspace's.  Returns
 *   QLI_ERR_UNSUPPORTED for TND; otherwise as qli_run_bounded.
 */
int qli_run_bounded_aslq(const qli_problem *p, int64_t max_seq_len_key,
                         const int32_t *aslq_dev, const int32_t *aslk_dev,
                         const void *query, const void *key,
                         const void *weights, const void *q_scale,
                         const void *k_scale, const int32_t *block_table,
                         void *workspace, int32_t *sparse_indices,
                         float *sparse_values, void *stream);

/*
 * qli_run_bounded_tnd -- the same for the TND layout: aslq_dev (device int32[B],
 *   actual_seq_lengths_query as prefix sums, 4-byte aligned) and aslk_dev are
 *   both read on the device, so a graph captured once replays correctly after
 *   either changes.  The prefix sums are taken as their running maximum
 *   clamped to [0, T], so any contents give a valid partition of the T rows;
 *   rows past the last prefix sum are padding.  Up to 128 batches the kernels
 *   derive the partition themselves; for more, a first small kernel turns
 *   aslq into row and group tables in the workspace.  Query rows are scored
 *   in 4-row groups within each batch.  Returns QLI_ERR_UNSUPPORTED for BSND
 *   or batch > 4096; otherwise as qli_run_bounded.
 */
int qli_run_bounded_tnd(const qli_problem *p, int64_t max_seq_len_key,
                        const int32_t *aslq_dev, const int32_t *aslk_dev,
                        const void *query, const void *key,
                        const void *weights, const void *q_scale,
                        const void *k_scale, const int32_t *block_table,
                        void *workspace, int32_t *sparse_indices,
                        float *sparse_values, void *stream);

/*
 * qli_run_bounded_static -- qli_run_bounded for callers that cannot allocate
 *   device memory: code under HIP graph capture, tight serving loops, hosts
 *   that forbid hipMalloc.  Same arguments, semantics and outputs as
 *   qli_run_bounded (BSND layout), minus the workspace: the library uses its
 *   own static device workspace of 32 MiB per GPU (a file-scope device array,
 *   allocated when the library is loaded on a device and held until the
 *   process ends).  The call itself allocates nothing, host or device.
 *   Limit: QLI_ERR_SIZE when qli_bounded_workspace reports more than
 *   33554432 bytes for the problem and bound (e.g. 64 sequences of 65536 key
 *   entries at sparse_count 512 need about 18 MiB).  QLI_ERR_UNSUPPORTED for
 *   the TND layout.  QLI_ERR_HIP if the workspace's device address cannot be
 *   obtained.
 *   Every call on one GPU shares that GPU's workspace, and nothing in it needs
 *   to start at zero (each call writes what it later reads).  Calls that may
 *   overlap on one GPU -- on different streams, or from different host threads
 *   -- race on the workspace and give undefined outputs: serialize them (one
 *   stream, or events).
 */
int qli_run_bounded_static(const qli_problem *p, int64_t max_seq_len_key,
                           const int32_t *aslk_dev, const void *query,
                           const void *key, const void *weights,
                           const void *q_scale, const void *k_scale,
                           const int32_t *block_table, int32_t *sparse_indices,
                           float *sparse_values, void *stream);

/*
 * Producer side: per-token-head quantization of the index query and key, the
 * step before the indexer.  QLI-README 功能说明 states that query and key are
 * quantized so that both are stored and computed in 8 bits, and 参数说明
 * names per-token-head as the only quantization mode (query_quant_mode,
 * key_quant_mode = 0); it gives no formula.  The reading adopted here is
 * symmetric absmax quantization of each 128-element head vector, matching the
 * indexer's dequantization ScaleQ * ScaleK * (q . k).  Every step is fixed in
 * fp32 so that the codes are reproducible bit for bit:
 *
 *   x      the row's 128 bf16 values, widened exactly to fp32
 *   amax   max_i |x_i|
 *   int8 codes, fp16 scale (the page's INT8 + FLOAT16 pairing):
 *     s    = fp16(amax / 127)     fp32 division, rounded to nearest-even fp16,
 *                                 65504 if that overflows
 *     r    = 1 / float(s)         fp32 division (correctly rounded)
 *     q_i  = clamp(rint(x_i * r), -127, 127), rint = nearest, ties to even;
 *            all q_i = 0 when s == 0
 *   e4m3fn codes, fp32 scale (the FLOAT8_e4m3fn + FLOAT32 pairing):
 *     s    = amax / 448           fp32 division
 *     r    = 1 / s                fp32 division
 *     q_i  = e4m3fn(clamp(x_i * r, -448, 448)), rounded to nearest, ties to
 *            even (OCP E4M3FN: bias 7, subnormals m * 2^-9, max 448);
 *            all q_i = 0 when s == 0 or r is not finite (amax < 448 * 2^-128)
 *   s is the dequant scale written beside the codes; s * q_i approximates x_i.
 *
 * Inputs must be finite (NaN / Inf give undefined codes).  Pointers are
 * device addresses; x 16-byte aligned, q_out 8-byte aligned; nothing is
 * allocated; a row count of 0 launches nothing.  Errors: QLI_ERR_ARG for a
 * negative count, a NULL or misaligned pointer, or a cache geometry that
 * breaks the indexer's constraints; QLI_ERR_UNSUPPORTED for another
 * qk_dtype; QLI_ERR_HIP if the launch fails.
 */

/*
 * qli_quantize_query -- rows = tokens * 64 head vectors of a query
 *   [tokens, 64, 128] bf16 (row-major) -> q_out [rows, 128] codes (qli_qk_dtype)
 *   and scale_out [rows] (fp16 for int8, fp32 for e4m3fn): the query and
 *   query_dequant_scale inputs of qli_run, row for row.
 */
int qli_quantize_query(int32_t qk_dtype, int64_t rows, const void *x,
                       void *q_out, void *scale_out, void *stream);

/*
 * qli_append_keys -- quantizes n key entries (bf16 [n, 128]; when cmp_ratio >
 *   1 these are compressed entries, produced upstream) and writes entry e into
 *   the paged key cache at entry position pos[e] of sequence batch_idx[e]:
 *   block blk = block_table[batch_idx[e] * max_blocks_per_seq + pos[e] /
 *   block_size], slot o = pos[e] % block_size; codes at key_cache + blk *
 *   stride + o * 128, scale at k_scale[blk * block_size + o] (the key and
 *   key_dequant_scale layouts of qli_run; stride = key_block_stride, or
 *   block_size * 128 when 0).  An entry whose batch_idx is outside
 *   [0, batch_count), whose pos is negative or past max_blocks_per_seq *
 *   block_size, or whose block id is outside [0, num_blocks) is skipped, so no
 *   write leaves the cache.  Entries must address distinct slots (two entries
 *   for one slot race).  block_size, stride and num_blocks follow the
 *   constraints of qli_problem.
 */
int qli_append_keys(int32_t qk_dtype, int64_t n, const void *x,
                    const int32_t *batch_idx, const int32_t *pos,
                    const int32_t *block_table, int32_t batch_count,
                    int32_t max_blocks_per_seq, int32_t num_blocks,
                    int32_t block_size, int64_t key_block_stride,
                    void *key_cache, void *k_scale, void *stream);

/*
 * Consumer: sparse attention over the indexer's output.  The page calls the
 * indexer the preprocessing of sparse attention: its Top-k indices are the
 * input of Attention (QLI-README 功能说明 step 3), sparse_indices are the
 * tokens taking part in the sparse attention, and block_table maps the KV
 * storage of PageAttention (参数说明).  The page does not write the attention
 * out; the reading implemented here is, for query row r of batch b and query
 * head h,
 *   S_r       = { sparse_indices[r][i] : i < sparse_count, value >= 0 }
 *   out[r][h] = sum_{j in S_r} softmax_j(softmax_scale * q[r][h] . K_b[j]) * V_b[j]
 *   lse[r][h] = log sum_{j in S_r} exp(softmax_scale * q[r][h] . K_b[j])
 * with one key / value head shared by every query head; K_b[j], V_b[j] is
 * entry j of batch b in the paged caches: block block_table[b][j / block_size],
 * slot j % block_size (the index space of the indexer's output).  A row with
 * no listed entry gets out = 0 and lse = -INFINITY.  Rows map to batches as
 * in the indexer: BSND row r is batch r / S1; TND rows follow the prefix sums
 * of actual_seq_lengths_query (rows past the last one attend to nothing).
 */
typedef struct qli_attn_problem {
    int32_t batch;              /* B (TND: entries of actual_seq_lengths_query) */
    int32_t s1;                 /* BSND: S1; TND: T */
    int32_t layout_query;       /* qli_layout */
    int32_t num_heads;          /* query heads H: 16, 32, 64 or 128 (else QLI_ERR_UNSUPPORTED) */
    int32_t head_dim;           /* must be 128 (else QLI_ERR_UNSUPPORTED) */
    int32_t num_blocks;         /* blocks of the key and value caches, >= 1 */
    int32_t block_size;         /* multiple of 16, 16..1024 (as the indexer's key cache) */
    int32_t max_blocks_per_seq; /* second dim of block_table */
    int64_t kv_block_stride;    /* elements (bf16) between consecutive blocks of either cache;
                                   0 = block_size * 128; else >= that and a multiple of 8 */
    int32_t sparse_count;       /* columns of sparse_indices, 1..2048 */
    float softmax_scale;        /* > 0 and finite (e.g. 1 / sqrt(128)) */
    int32_t return_lse;         /* 1: write lse */
    int32_t reserved0;          /* must be 0 */
    int32_t reserved1;          /* must be 0 */
    int32_t reserved2;          /* must be 0 */
} qli_attn_problem;

/*
 * qli_sparse_attention_workspace -- device workspace bytes qli_sparse_attention
 *   needs (0 when every row is finished by one workgroup; otherwise fp32
 *   partials of rows whose list is split across workgroups).
 */
int qli_sparse_attention_workspace(const qli_attn_problem *p, size_t *workspace_bytes);

/*
 * qli_sparse_attention -- stream-ordered, no host synchronisation.
 *   aslq            device int32[B] prefix sums (TND only; NULL for BSND)
 *   q               device bf16 [rows, H, 128], 16-byte aligned
 *   k_cache, v_cache device bf16 [num_blocks, block_size, 128] (block stride
 *                   kv_block_stride), 16-byte aligned
 *   block_table     device int32 [B, max_blocks_per_seq]
 *   sparse_indices  device int32 [rows, sparse_count] (the indexer's output)
 *   workspace       device, qli_sparse_attention_workspace bytes, 16-byte
 *                   aligned (NULL if 0)
 *   out             device bf16 [rows, H, 128] (written), 8-byte aligned
 *   lse             device float [rows, H] (written when return_lse), or NULL
 * Listed entries at or past max_blocks_per_seq * block_size, or whose block
 * id lies outside [0, num_blocks), are skipped, so no read leaves the caches;
 * listing an entry the batch does not store (a block-table slot of another
 * sequence) is out of contract.  Errors: QLI_ERR_ARG / QLI_ERR_UNSUPPORTED for
 * a scalar or pointer that breaks the rules above, before anything is
 * launched; QLI_ERR_HIP if a launch fails.
 */
int qli_sparse_attention(const qli_attn_problem *p, const int32_t *aslq, const void *q,
                         const void *k_cache, const void *v_cache, const int32_t *block_table,
                         const int32_t *sparse_indices, void *workspace, void *out, float *lse,
                         void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QLI_H */
