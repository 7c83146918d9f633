/*
 * pa_oracle.c -- plain, slow, obviously correct CPU reference for attention
 * over a block-paged KV cache, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two are compared on the
 * same seeded inputs.
 *
 * What it follows (pages are cited by title and section):
 *  - "nano-vllm deep dive" (LLM-101-CN), Step 4, "Triton Kernel: write KV
 *    Cache": a token's K/V row goes to flat slot s of the cache, slot -1 is a
 *    padding token that is skipped; the slot is block_table[i]*block_size +
 *    offset inside the block.
 *  - same page, Step 1, "why block_table": logical token j of a sequence
 *    lives in physical block block_table[j / block_size], slot j % block_size.
 *  - same page, Step 5, "KV Cache memory layout": each layer's cache is
 *    [num_blocks, block_size, kv_heads, head_dim].
 *  - same page, Step 5, prepare_prefill / prepare_decode: a prefill sequence
 *    contributes len - num_cached query tokens at absolute positions
 *    num_cached .. len-1 and len keys; a decode sequence has one query at
 *    position len-1 and context length len.
 *  - "推理系统" notes (notes.cassieliang.com), KV-cache demo: new token i of T
 *    new tokens over S keys sees the first S-T+i+1 keys (bottom-right causal
 *    alignment); the attention itself is softmax(q k^T / sqrt(D)) v.
 *  - "vLLM/SGLang interview source labs", section 2: a prompt of N tokens has
 *    N(N+1)/2 valid causal (query, key) pairs.
 *
 * The attention is the plain definition: for each query row and head, walk
 * the block table key by key, form every visible score in fp64, subtract the
 * maximum, exponentiate, normalise and take the weighted sum of V.  No
 * tiling, no online rescaling, no reordering.
 *
 * Element types: 0 = fp32, 1 = bf16 (raw 16-bit patterns; widened exactly to
 * fp64 by placing the bits in the top half of an fp32), 3 = IEEE binary16
 * (raw 16-bit patterns; widened exactly from sign, 5-bit exponent and 10-bit
 * fraction).  Code 2 is unused here: the INT8 reference dequantizes in Python
 * and hands this file fp32 pools.
 *
 * Return codes: 0 ok, 1 null argument, 2 bad shape / sizes,
 *               3 bad element type, 4 index out of range in the metadata.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_NULL = 1, OR_SHAPE = 2, OR_DTYPE = 3, OR_RANGE = 4 };

static int elem_bytes_of(int dtype)
{
    if (dtype == 0) return 4;
    if (dtype == 1 || dtype == 3) return 2;
    return 0;
}

/* Exact widening of one stored element to fp64. */
static double widen(const void *base, int64_t index, int dtype)
{
    if (dtype == 0) {
        float f;
        memcpy(&f, (const char *)base + index * 4, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char *)base + index * 2, 2);
    if (dtype == 3) {
        /* binary16: (-1)^s * 2^(e-15) * (1 + f/1024) for 0 < e < 31,
         * (-1)^s * 2^-14 * (f/1024) for e == 0, inf / NaN for e == 31. */
        int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
        double mag;
        if (e == 31) mag = f ? NAN : INFINITY;
        else if (e == 0) mag = ldexp((double)f, -24);
        else mag = ldexp((double)(1024 + f), e - 25);
        return sign ? -mag : mag;
    }
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Host threads the attention loops use from now on (n >= 1); returns the
 * number in effect.  Timing only: results do not depend on it. */
int oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/*
 * Store: for every token t whose slot is not -1, copy its K row and V row
 * (num_kv_heads * head_dim elements, taken at t * row_stride elements) to
 * flat slot `slot` of the pools, i.e. block slot / block_size, offset
 * slot % block_size.  Bytes are copied unchanged.
 */
int oracle_store_kv(const void *k, int64_t k_row_stride,
                    const void *v, int64_t v_row_stride,
                    const int32_t *slot_mapping, int32_t num_tokens,
                    void *k_pool, void *v_pool,
                    int64_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype)
{
    int eb = elem_bytes_of(dtype);
    if (!eb) return OR_DTYPE;
    if (num_tokens < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0)
        return OR_SHAPE;
    if (num_tokens == 0) return OR_OK;
    if (!k || !v || !slot_mapping || !k_pool || !v_pool) return OR_NULL;
    int64_t row = (int64_t)num_kv_heads * head_dim;
    if (k_row_stride < row || v_row_stride < row) return OR_SHAPE;
    int64_t num_slots = num_blocks * block_size;
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot == -1) continue;
        if (slot < 0 || slot >= num_slots) return OR_RANGE;
        int64_t block = slot / block_size;
        int64_t offset = slot % block_size;
        int64_t dst = (block * block_size + offset) * row; /* element index */
        memcpy((char *)k_pool + dst * eb, (const char *)k + (int64_t)t * k_row_stride * eb, (size_t)(row * eb));
        memcpy((char *)v_pool + dst * eb, (const char *)v + (int64_t)t * v_row_stride * eb, (size_t)(row * eb));
    }
    return OR_OK;
}

/*
 * Gather: for each sequence s and each key j < k_len(s), walk the block
 * table: physical block p = block_table[s][j / block_size], offset
 * j % block_size, and copy that token's K and V rows to packed output row
 * cu_seqlens_k[s] + j.  Output is [total_k, num_kv_heads, head_dim].
 */
int oracle_gather_kv(const void *k_pool, const void *v_pool,
                     int64_t num_blocks, int32_t block_size,
                     int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                     const int32_t *cu_seqlens_k, const int32_t *block_table,
                     int32_t block_table_stride, int32_t num_seqs,
                     void *k_out, void *v_out)
{
    int eb = elem_bytes_of(dtype);
    if (!eb) return OR_DTYPE;
    if (num_seqs < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return OR_SHAPE;
    if (num_seqs == 0) return OR_OK;
    if (!k_pool || !v_pool || !cu_seqlens_k || !block_table || !k_out || !v_out) return OR_NULL;
    int64_t row = (int64_t)num_kv_heads * head_dim;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int64_t base = cu_seqlens_k[s];
        int64_t k_len = (int64_t)cu_seqlens_k[s + 1] - cu_seqlens_k[s];
        if (k_len < 0) return OR_SHAPE;
        if (k_len > (int64_t)block_table_stride * block_size) return OR_RANGE;
        for (int64_t j = 0; j < k_len; ++j) {
            int64_t p = block_table[(int64_t)s * block_table_stride + j / block_size];
            int64_t o = j % block_size;
            if (p < 0 || p >= num_blocks) return OR_RANGE;
            int64_t src = (p * block_size + o) * row;
            memcpy((char *)k_out + (base + j) * row * eb, (const char *)k_pool + src * eb, (size_t)(row * eb));
            memcpy((char *)v_out + (base + j) * row * eb, (const char *)v_pool + src * eb, (size_t)(row * eb));
        }
    }
    return OR_OK;
}

/*
 * One query row, one query head: attend to keys 0..last of sequence s.
 * kv head g = h / (num_q_heads / num_kv_heads).  Keys are fetched one at a
 * time through the block table.  Writes head_dim fp64 values to out.
 * Returns OR_RANGE if a block id the row needs is out of range.
 */
static int attend_one(const void *q_row, int32_t h, int32_t num_q_heads, int32_t dtype,
                      const void *k_pool, const void *v_pool, int64_t num_blocks,
                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                      const int32_t *table_row, int64_t last, double scale, double *out)
{
    int64_t d;
    for (d = 0; d < head_dim; ++d) out[d] = 0.0;
    if (last < 0) return OR_OK; /* no visible key: defined as zero output */
    int32_t group = num_q_heads / num_kv_heads;
    int32_t g = h / group;
    int64_t n = last + 1;
    double *z = (double *)malloc((size_t)n * sizeof(double));
    double *qd = (double *)malloc((size_t)head_dim * sizeof(double));
    if (!z || !qd) { free(z); free(qd); return OR_SHAPE; }
    for (d = 0; d < head_dim; ++d) qd[d] = widen(q_row, (int64_t)h * head_dim + d, dtype);

    /* scores z_j = scale * <q, k_j> */
    double zmax = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        int64_t p = table_row[j / block_size];
        if (p < 0 || p >= num_blocks) { free(z); free(qd); return OR_RANGE; }
        int64_t base = ((p * block_size + j % block_size) * num_kv_heads + g) * (int64_t)head_dim;
        double dot = 0.0;
        for (d = 0; d < head_dim; ++d) dot += qd[d] * widen(k_pool, base + d, dtype);
        z[j] = scale * dot;
        if (z[j] > zmax) zmax = z[j];
    }
    /* softmax weights, then the weighted sum of V rows */
    double denom = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        z[j] = exp(z[j] - zmax);
        denom += z[j];
    }
    for (int64_t j = 0; j < n; ++j) {
        int64_t p = table_row[j / block_size];
        int64_t base = ((p * block_size + j % block_size) * num_kv_heads + g) * (int64_t)head_dim;
        double w = z[j] / denom;
        for (d = 0; d < head_dim; ++d) out[d] += w * widen(v_pool, base + d, dtype);
    }
    free(z);
    free(qd);
    return OR_OK;
}

static int check_common(int32_t num_q_heads, int32_t dtype, int64_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim)
{
    if (!elem_bytes_of(dtype)) return OR_DTYPE;
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return OR_SHAPE;
    if (num_q_heads % num_kv_heads) return OR_SHAPE;
    return OR_OK;
}

/*
 * Varlen causal prefill over the paged cache.
 *   q: [total_q, num_q_heads, head_dim] with row stride q_row_stride elements.
 *   Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and
 *   k_len = cu_seqlens_k[s+1] - cu_seqlens_k[s] keys; query i of s sits at
 *   absolute position q_offsets[s] + i and sees keys
 *   0 .. min(q_offsets[s] + i, k_len - 1).
 *   rows: the packed query rows to compute (NULL = all rows 0..total_q-1,
 *   num_rows = total_q).  out: [num_rows, num_q_heads, head_dim] fp64.
 *   pairs (may be NULL): receives the number of visible (query, key) pairs
 *   summed over the computed rows (per head, i.e. counted once per row).
 */
int oracle_prefill(const void *q, int64_t q_row_stride, int32_t num_q_heads, int32_t dtype,
                   const void *k_pool, const void *v_pool, int64_t num_blocks,
                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                   const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                   const int32_t *q_offsets, const int32_t *block_table,
                   int32_t block_table_stride, int32_t num_seqs, double scale,
                   const int32_t *rows, int32_t num_rows, double *out, int64_t *pairs)
{
    int rc = check_common(num_q_heads, dtype, num_blocks, block_size, num_kv_heads, head_dim);
    if (rc) return rc;
    if (num_seqs < 0 || num_rows < 0) return OR_SHAPE;
    if (num_rows == 0 || num_seqs == 0) { if (pairs) *pairs = 0; return OR_OK; }
    if (!q || !k_pool || !v_pool || !cu_seqlens_q || !cu_seqlens_k || !q_offsets || !block_table || !out)
        return OR_NULL;
    if (q_row_stride < (int64_t)num_q_heads * head_dim) return OR_SHAPE;
    int32_t total_q = cu_seqlens_q[num_seqs];
    int64_t npairs = 0;
    int err = OR_OK;
    int64_t work = (int64_t)num_rows * num_q_heads;

#pragma omp parallel for schedule(dynamic, 1) reduction(+ : npairs)
    for (int64_t w = 0; w < work; ++w) {
        int32_t r_idx = (int32_t)(w / num_q_heads);
        int32_t h = (int32_t)(w % num_q_heads);
        int32_t r = rows ? rows[r_idx] : r_idx;
        double *dst = out + ((int64_t)r_idx * num_q_heads + h) * head_dim;
        if (r < 0 || r >= total_q) {
#pragma omp atomic write
            err = OR_RANGE;
            continue;
        }
        /* the sequence that owns packed row r: plain linear scan */
        int32_t s = 0;
        while (!(cu_seqlens_q[s] <= r && r < cu_seqlens_q[s + 1])) ++s;
        int64_t i = r - cu_seqlens_q[s];
        int64_t k_len = (int64_t)cu_seqlens_k[s + 1] - cu_seqlens_k[s];
        int64_t last = (int64_t)q_offsets[s] + i;
        if (last > k_len - 1) last = k_len - 1;
        if (last + 1 > (int64_t)block_table_stride * block_size) {
#pragma omp atomic write
            err = OR_RANGE;
            continue;
        }
        int rc1 = attend_one((const char *)q + (int64_t)r * q_row_stride * elem_bytes_of(dtype), h,
                             num_q_heads, dtype, k_pool, v_pool, num_blocks, block_size,
                             num_kv_heads, head_dim, block_table + (int64_t)s * block_table_stride,
                             last, scale, dst);
        if (rc1) {
#pragma omp atomic write
            err = rc1;
        }
        if (h == 0 && last >= 0) npairs += last + 1;
    }
    if (pairs) *pairs = npairs;
    return err;
}

/*
 * Decode: one query row per sequence.  q: [num_seqs, num_q_heads, head_dim]
 * (row stride q_row_stride); context_lens[s] counts every key of sequence s,
 * the new token included, and the query sits at position context_lens[s]-1,
 * so it sees keys 0 .. context_lens[s]-1.  A context length of 0 (a padding
 * row) gives a zero output.  seqs: sequences to compute (NULL = all,
 * num_rows = num_seqs).  out: [num_rows, num_q_heads, head_dim] fp64.
 */
int oracle_decode(const void *q, int64_t q_row_stride, int32_t num_q_heads, int32_t dtype,
                  const void *k_pool, const void *v_pool, int64_t num_blocks,
                  int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                  const int32_t *context_lens, const int32_t *block_table,
                  int32_t block_table_stride, int32_t num_seqs, double scale,
                  const int32_t *seqs, int32_t num_rows, double *out, int64_t *pairs)
{
    int rc = check_common(num_q_heads, dtype, num_blocks, block_size, num_kv_heads, head_dim);
    if (rc) return rc;
    if (num_seqs < 0 || num_rows < 0) return OR_SHAPE;
    if (num_rows == 0 || num_seqs == 0) { if (pairs) *pairs = 0; return OR_OK; }
    if (!q || !k_pool || !v_pool || !context_lens || !block_table || !out) return OR_NULL;
    if (q_row_stride < (int64_t)num_q_heads * head_dim) return OR_SHAPE;
    int64_t npairs = 0;
    int err = OR_OK;
    int64_t work = (int64_t)num_rows * num_q_heads;

#pragma omp parallel for schedule(dynamic, 1) reduction(+ : npairs)
    for (int64_t w = 0; w < work; ++w) {
        int32_t r_idx = (int32_t)(w / num_q_heads);
        int32_t h = (int32_t)(w % num_q_heads);
        int32_t s = seqs ? seqs[r_idx] : r_idx;
        double *dst = out + ((int64_t)r_idx * num_q_heads + h) * head_dim;
        if (s < 0 || s >= num_seqs || context_lens[s] < 0 ||
            (int64_t)context_lens[s] > (int64_t)block_table_stride * block_size) {
#pragma omp atomic write
            err = OR_RANGE;
            continue;
        }
        int64_t last = (int64_t)context_lens[s] - 1;
        int rc1 = attend_one((const char *)q + (int64_t)s * q_row_stride * elem_bytes_of(dtype), h,
                             num_q_heads, dtype, k_pool, v_pool, num_blocks, block_size,
                             num_kv_heads, head_dim, block_table + (int64_t)s * block_table_stride,
                             last, scale, dst);
        if (rc1) {
#pragma omp atomic write
            err = rc1;
        }
        if (h == 0 && last >= 0) npairs += last + 1;
    }
    if (pairs) *pairs = npairs;
    return err;
}
