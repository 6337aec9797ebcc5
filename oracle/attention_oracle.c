/*
 * attention_oracle.c -- plain, slow CPU oracle for the sparse attention that
 * consumes the indexer's output.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under sparse_attention_token_paged_amd/) never calls it
 * and shares no code with it.
 *
 * Source ("QLI-README" below): the EngineX-Ascend page
 * "VllmQuantLightningIndexer".  Its section 功能说明 calls the operator the
 * preprocessing of sparse attention: it selects the important sparse tokens,
 * and step 3 says the selected Top-k indices are the input of Attention.
 * Section 参数说明 defines sparse_indices as the indices of the tokens that
 * take part in the sparse attention computation, and block_table as the
 * block map of the KV storage of PageAttention.  The page does not write the
 * attention out.  reading: the plainest attention the rest supports --
 * for query row r of batch b and head h, softmax attention restricted to the
 * listed entries:
 *   S        = { sparse_indices[r][i] : 0 <= i < k, sparse_indices[r][i] >= 0 }
 *   logit_j  = scale * sum_d q[r][h][d] * K_b[j][d]            (j in S)
 *   p_j      = exp(logit_j - m) / sum_{j' in S} exp(logit_j' - m),  m = max logit
 *   out[r][h] = sum_{j in S} p_j * V_b[j]
 *   lse[r][h] = m + log(sum_{j in S} exp(logit_j - m))
 * where K_b[j] and V_b[j] are entry j of batch b's paged key and value caches
 * (entry j at block block_table[b][j / block_size], slot j % block_size, the
 * same index space as the indexer's sparse_indices).  One key/value head is
 * shared by every query head.  An entry listed twice counts twice (the
 * indexer lists each at most once).  A row with no listed entry, or one that
 * belongs to no batch, gets out = 0 and lse = -infinity.
 *
 * Precision: bf16 inputs decoded exactly; everything else in fp64 in the
 * literal order above (indices in list order, dims ascending).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { QLAO_OK = 0, QLAO_E_ARG = 1 };

/* bf16: the upper 16 bits of an IEEE binary32 value; widened exactly. */
double qlao_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Batch of output row r, or -1.  BSND: r / s1.  TND: the batch whose
 * prefix-sum range [aslq[b-1], aslq[b]) holds r (QLI-README 约束说明: in TND
 * actual_seq_lengths_query holds prefix sums). */
static int row_batch(int layout, int batch, int s1_or_t, const int32_t *aslq, int64_t r)
{
    int b;
    if (layout == 0)
        return (int)(r / s1_or_t);
    for (b = 0; b < batch; b++)
        if (r < aslq[b])
            return b;
    return -1;
}

/* Entry j of batch b in a paged cache: block block_table[b][j / bs], slot
 * j % bs; consecutive blocks are stride elements apart. */
static const uint16_t *entry(const uint16_t *cache, const int32_t *block_table, int max_blocks,
                             int block_size, int64_t stride, int head_dim, int b, int64_t j)
{
    int32_t blk = block_table[(int64_t)b * max_blocks + j / block_size];
    return cache + (int64_t)blk * stride + (j % block_size) * head_dim;
}

/* The whole consumer over every row.  q: [rows, heads, head_dim] bf16;
 * k_cache, v_cache: [num_blocks, block_size, head_dim] bf16 with block stride
 * kv_stride elements (0: block_size * head_dim); indices: [rows, k] int32.
 * out: [rows, heads, head_dim] fp64; lse: [rows, heads] fp64 (may be NULL).
 * Entries at or past max_blocks * block_size are rejected (QLAO_E_ARG). */
int qlao_sparse_attention(int layout, int batch, int s1_or_t, const int32_t *aslq, int heads,
                          int head_dim, int block_size, int max_blocks, int64_t kv_stride,
                          const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                          const int32_t *block_table, const int32_t *indices, int sparse_count,
                          double scale, double *out, double *lse, int nthreads)
{
    int64_t rows = layout == 0 ? (int64_t)batch * s1_or_t : (int64_t)s1_or_t;
    int64_t r;
    int bad = 0;
    int64_t stride = kv_stride > 0 ? kv_stride : (int64_t)block_size * head_dim;
    if (heads < 1 || head_dim < 1 || block_size < 1 || sparse_count < 1 || (layout == 1 && !aslq))
        return QLAO_E_ARG;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (r = 0; r < rows; r++) {
        int b = row_batch(layout, batch, s1_or_t, aslq, r);
        const int32_t *list = indices + r * sparse_count;
        double *logit = (double *)malloc(sizeof(double) * (size_t)sparse_count);
        int h, i, d;
        if (!logit) {
            bad = 1;
            continue;
        }
        for (h = 0; h < heads; h++) {
            const uint16_t *qh = q + (r * heads + h) * head_dim;
            double *o = out + (r * heads + h) * head_dim;
            double m = -INFINITY, l = 0.0;
            int n = 0;
            for (d = 0; d < head_dim; d++)
                o[d] = 0.0;
            if (b >= 0) {
                for (i = 0; i < sparse_count; i++) {
                    int64_t j = list[i];
                    const uint16_t *kj;
                    double dot = 0.0;
                    if (j < 0)
                        continue;
                    if (j >= (int64_t)max_blocks * block_size) {
                        bad = 1;
                        continue;
                    }
                    kj = entry(k_cache, block_table, max_blocks, block_size, stride, head_dim, b, j);
                    for (d = 0; d < head_dim; d++)
                        dot += qlao_bf16_value(qh[d]) * qlao_bf16_value(kj[d]);
                    logit[n] = scale * dot;
                    if (logit[n] > m)
                        m = logit[n];
                    n++;
                }
            }
            if (n == 0) {
                if (lse)
                    lse[r * heads + h] = -INFINITY;
                continue;
            }
            n = 0;
            for (i = 0; i < sparse_count; i++) {
                int64_t j = list[i];
                const uint16_t *vj;
                double w;
                if (j < 0 || j >= (int64_t)max_blocks * block_size)
                    continue;
                w = exp(logit[n++] - m);
                l += w;
                vj = entry(v_cache, block_table, max_blocks, block_size, stride, head_dim, b, j);
                for (d = 0; d < head_dim; d++)
                    o[d] += w * qlao_bf16_value(vj[d]);
            }
            for (d = 0; d < head_dim; d++)
                o[d] /= l;
            if (lse)
                lse[r * heads + h] = m + log(l);
        }
        free(logit);
    }
    return bad ? QLAO_E_ARG : QLAO_OK;
}
