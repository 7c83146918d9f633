// pa_api.cpp -- the extern "C" entry points of libpa (see include/pa.h).
// Host-side argument checks, launch planning and dispatch.  Nothing here
// synchronises the device, allocates, or reads device memory.
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "pa.h"
#include "pa_kernels.h"

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
    int s = 0;
    while ((int64_t(1) << s) < x) ++s;
    return s;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_BF16 || dtype == PA_F16 ? 2 : 0); }

// Element types of the queries and of the rows quantized into INT8 pools.
bool float_dtype(int dtype) { return dtype == PA_F32 || dtype == PA_BF16 || dtype == PA_F16; }

// Checks shared by every call that reads the pools.
pa_status check_pool(const pa_pool *pool, pa::PoolGeom *g) {
    if (!pool) return PA_ERR_NULL_ARG;
    if (!elem_bytes(pool->dtype)) return PA_ERR_BAD_DTYPE;
    if (pool->num_blocks < 0 || pool->block_size <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0)
        return PA_ERR_BAD_SHAPE;
    if (!is_pow2(pool->block_size) || pool->block_size > 65536) return PA_ERR_UNSUPPORTED;
    // a block's (slot, head) rows are indexed in 32 bits, offset * heads in 24
    if (pool->num_kv_heads > 65536 || (int64_t)pool->num_kv_heads * pool->block_size >= (int64_t(1) << 31))
        return PA_ERR_UNSUPPORTED;
    g->num_blocks = pool->num_blocks;
    g->block_size = pool->block_size;
    g->block_shift = log2i(pool->block_size);
    g->hkv = pool->num_kv_heads;
    g->d = pool->head_dim;
    g->dtype = pool->dtype;
    return PA_OK;
}

// INT8 pools: the same geometry checks for dtype PA_INT8.
pa_status check_pool_int8(const pa_pool *pool, pa::PoolGeom *g) {
    if (!pool) return PA_ERR_NULL_ARG;
    if (pool->dtype != PA_INT8) return PA_ERR_BAD_DTYPE;
    pa_pool p = *pool;
    p.dtype = PA_BF16;  // geometry only
    pa_status st = check_pool(&p, g);
    g->dtype = PA_INT8;
    return st;
}

pa_status check_attention_shape(const pa_pool *pool, int32_t num_q_heads, pa::PoolGeom *g) {
    pa_status st = check_pool(pool, g);
    if (st != PA_OK) return st;
    if (num_q_heads <= 0 || num_q_heads % g->hkv) return PA_ERR_BAD_SHAPE;
    const int group = num_q_heads / g->hkv;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
    if (g->d != 32 && g->d != 64 && g->d != 128 && g->d != 256) return PA_ERR_UNSUPPORTED;
    if (g->num_blocks < 1) return PA_ERR_BAD_SHAPE;  // attention needs a non-empty pool
    return PA_OK;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// The kernels track a running max of the raw scores, which orders the scaled
// scores the same way only for a positive scale.
bool scale_ok(float s) { return s > 0.f && s <= 3.0e38f; }

void say(char *why, size_t why_len, const char *fmt, long long a, long long b) {
    if (why && why_len) snprintf(why, why_len, fmt, a, b);
}

// INT8 decode: the float decode's checks, with int8 code pools, fp16 scale
// pools and q / out of q_dtype; query groups of 1, 2, 4 or 8.
pa_status check_decode_int8_shape(const pa_pool *pool, int32_t num_q_heads, int32_t q_dtype, pa::PoolGeom *g) {
    pa_status st = check_pool_int8(pool, g);
    if (st != PA_OK) return st;
    if (!float_dtype(q_dtype)) return PA_ERR_BAD_DTYPE;
    if (num_q_heads <= 0 || num_q_heads % g->hkv) return PA_ERR_BAD_SHAPE;
    const int group = num_q_heads / g->hkv;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
    if (g->d != 32 && g->d != 64 && g->d != 128 && g->d != 256) return PA_ERR_UNSUPPORTED;
    if (g->num_blocks < 1) return PA_ERR_BAD_SHAPE;
    return PA_OK;
}

// pa_decode's host checks and split plan, shared with pa_decode_static.
// PA_OK with num_seqs == 0 means nothing to do; *need is the partials' size.
pa_status check_decode(const void *q, int64_t q_row_stride, int32_t num_q_heads, const void *k_pool,
                       const void *v_pool, const pa_pool *pool, const int32_t *context_lens,
                       const int32_t *block_table, int32_t block_table_stride, int32_t num_seqs,
                       int32_t max_context_len, float softmax_scale, const void *out, pa::PoolGeom *g,
                       pa::RowAttnPlan *plan, size_t *need) {
    pa_status st = check_attention_shape(pool, num_q_heads, g);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || max_context_len < 0) return PA_ERR_BAD_SHAPE;
    if (!scale_ok(softmax_scale)) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_pool || !v_pool || !context_lens || !block_table || !out) return PA_ERR_NULL_ARG;
    if (block_table_stride <= 0) return PA_ERR_BAD_SHAPE;
    if (q_row_stride < (int64_t)num_q_heads * g->d) return PA_ERR_BAD_SHAPE;
    const int eb = elem_bytes(g->dtype);
    if (!aligned16(q) || (q_row_stride * eb) % 16 || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_UNSUPPORTED;
    const int group = num_q_heads / g->hkv;
    *plan = pa::plan_row_attention(num_seqs, *g, group, max_context_len);
    *need = pa::row_attention_workspace_bytes(*plan, num_q_heads, g->d);
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char *pa_status_string(pa_status s) {
    switch (s) {
        case PA_OK: return "ok";
        case PA_ERR_NULL_ARG: return "null argument";
        case PA_ERR_BAD_SHAPE: return "bad shape or size";
        case PA_ERR_BAD_DTYPE: return "unsupported element type";
        case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, group size or alignment";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_HIP: return "HIP launch error";
        case PA_ERR_BAD_METADATA: return "invalid metadata";
    }
    return "unknown status";
}

pa_status pa_store_kv(const void *k, int64_t k_row_stride, const void *v, int64_t v_row_stride,
                      const int32_t *slot_mapping, int32_t num_tokens, void *k_pool, void *v_pool,
                      const pa_pool *pool, void *stream) {
    pa::PoolGeom g;
    pa_status st = check_pool(pool, &g);
    if (st != PA_OK) return st;
    if (num_tokens < 0) return PA_ERR_BAD_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PA_ERR_NULL_ARG;
    const int64_t row = (int64_t)g.hkv * g.d;
    if (k_row_stride < row || v_row_stride < row) return PA_ERR_BAD_SHAPE;
    return from_hip(pa::launch_store_kv(k, k_row_stride, v, v_row_stride, slot_mapping, num_tokens,
                                        k_pool, v_pool, g, (hipStream_t)stream));
}

pa_status pa_store_kv_int8(const void *k, int64_t k_row_stride, const void *v, int64_t v_row_stride,
                           int32_t src_dtype, const int32_t *slot_mapping, int32_t num_tokens, void *k_pool,
                           void *v_pool, void *k_scale, void *v_scale, const pa_pool *pool, void *stream) {
    pa::PoolGeom g;
    pa_status st = check_pool_int8(pool, &g);
    if (st != PA_OK) return st;
    if (!float_dtype(src_dtype)) return PA_ERR_BAD_DTYPE;
    if (num_tokens < 0) return PA_ERR_BAD_SHAPE;
    // a head vector is d/8 (16-bit rows) or d/4 (fp32 rows) lanes that reduce
    // max |x| with xor shuffles: the group must be a power of two
    if (g.d < 8 || g.d > 256 || !is_pow2(g.d)) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_pool || !v_pool || !k_scale || !v_scale) return PA_ERR_NULL_ARG;
    const int64_t row = (int64_t)g.hkv * g.d;
    if (k_row_stride < row || v_row_stride < row) return PA_ERR_BAD_SHAPE;
    if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 7) return PA_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 1) return PA_ERR_UNSUPPORTED;
    return from_hip(pa::launch_store_kv_int8(k, k_row_stride, v, v_row_stride, src_dtype, slot_mapping, num_tokens,
                                             k_pool, v_pool, k_scale, v_scale, g, (hipStream_t)stream));
}

pa_status pa_copy_blocks(void *k_pool, void *v_pool, void *k_scale, void *v_scale, const pa_pool *pool,
                         const int32_t *src_blocks, const int32_t *dst_blocks, const int32_t *num_valid,
                         int32_t num_pairs, void *stream) {
    pa::PoolGeom g;
    if (!pool) return PA_ERR_NULL_ARG;
    const bool i8 = pool->dtype == PA_INT8;
    pa_status st = i8 ? check_pool_int8(pool, &g) : check_pool(pool, &g);
    if (st != PA_OK) return st;
    if (num_pairs < 0) return PA_ERR_BAD_SHAPE;
    if (num_pairs == 0) return PA_OK;
    if (!k_pool || !v_pool || !src_blocks || !dst_blocks || !num_valid) return PA_ERR_NULL_ARG;
    if (i8 && (!k_scale || !v_scale)) return PA_ERR_NULL_ARG;
    const int64_t slot = (int64_t)g.hkv * g.d * (i8 ? 1 : elem_bytes(g.dtype));
    hipError_t e = pa::launch_copy_blocks(k_pool, slot, g, src_blocks, dst_blocks, num_valid, num_pairs,
                                          (hipStream_t)stream);
    if (e == hipSuccess)
        e = pa::launch_copy_blocks(v_pool, slot, g, src_blocks, dst_blocks, num_valid, num_pairs, (hipStream_t)stream);
    if (e == hipSuccess && i8) {
        const int64_t sslot = (int64_t)g.hkv * 2;
        e = pa::launch_copy_blocks(k_scale, sslot, g, src_blocks, dst_blocks, num_valid, num_pairs,
                                   (hipStream_t)stream);
        if (e == hipSuccess)
            e = pa::launch_copy_blocks(v_scale, sslot, g, src_blocks, dst_blocks, num_valid, num_pairs,
                                       (hipStream_t)stream);
    }
    return from_hip(e);
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k, const pa_pool *pool) {
    (void)max_seqlen_q;
    pa::PoolGeom g;
    if (check_attention_shape(pool, num_q_heads, &g) != PA_OK) return 0;
    if (num_seqs <= 0 || total_q <= 0) return 0;
    const int group = num_q_heads / g.hkv;
    if (pa::prefill_mfma_supported(g, group)) return 0;
    const pa::RowAttnPlan plan = pa::plan_row_attention(total_q, g, group, max_seqlen_k);
    return pa::row_attention_workspace_bytes(plan, num_q_heads, g.d);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 const pa_pool *pool) {
    pa::PoolGeom g;
    if (check_attention_shape(pool, num_q_heads, &g) != PA_OK) return 0;
    if (num_seqs <= 0 || max_context_len <= 0) return 0;
    const int group = num_q_heads / g.hkv;
    const pa::RowAttnPlan plan = pa::plan_row_attention(num_seqs, g, group, max_context_len);
    return pa::row_attention_workspace_bytes(plan, num_q_heads, g.d);
}

pa_status pa_prefill_varlen(const void *q, int64_t q_row_stride, int32_t num_q_heads,
                            const void *k_pool, const void *v_pool, const pa_pool *pool,
                            const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                            const int32_t *q_offsets, const int32_t *block_table,
                            int32_t block_table_stride, int32_t num_seqs, int32_t total_q,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                            void *out, void *workspace, size_t workspace_bytes, void *stream) {
    pa::PoolGeom g;
    pa_status st = check_attention_shape(pool, num_q_heads, &g);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return PA_ERR_BAD_SHAPE;
    if (!scale_ok(softmax_scale)) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0 || total_q == 0) return PA_OK;
    if (!q || !k_pool || !v_pool || !cu_seqlens_q || !cu_seqlens_k || !q_offsets || !block_table || !out)
        return PA_ERR_NULL_ARG;
    if (block_table_stride <= 0) return PA_ERR_BAD_SHAPE;
    if (q_row_stride < (int64_t)num_q_heads * g.d) return PA_ERR_BAD_SHAPE;
    const int eb = elem_bytes(g.dtype);
    if (!aligned16(q) || (q_row_stride * eb) % 16 || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_UNSUPPORTED;
    const int group = num_q_heads / g.hkv;
    if (pa::prefill_mfma_supported(g, group)) {
        if (!aligned16(out)) return PA_ERR_UNSUPPORTED;
        return from_hip(pa::launch_prefill_mfma(q, q_row_stride, num_q_heads, k_pool, v_pool, g,
                                                cu_seqlens_q, cu_seqlens_k, q_offsets, block_table,
                                                block_table_stride, num_seqs, total_q, max_seqlen_q,
                                                softmax_scale, out, (hipStream_t)stream));
    }
    const pa::RowAttnPlan plan = pa::plan_row_attention(total_q, g, group, max_seqlen_k);
    const size_t need = pa::row_attention_workspace_bytes(plan, num_q_heads, g.d);
    if (need && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    return from_hip(pa::launch_prefill_rows(q, q_row_stride, num_q_heads, k_pool, v_pool, g,
                                            cu_seqlens_q, cu_seqlens_k, q_offsets, block_table,
                                            block_table_stride, num_seqs, plan, softmax_scale, out,
                                            workspace, (hipStream_t)stream));
}

pa_status pa_decode(const void *q, int64_t q_row_stride, int32_t num_q_heads, const void *k_pool,
                    const void *v_pool, const pa_pool *pool, const int32_t *context_lens,
                    const int32_t *block_table, int32_t block_table_stride, int32_t num_seqs,
                    int32_t max_context_len, float softmax_scale, const int32_t *row_order, void *out,
                    void *workspace, size_t workspace_bytes, void *stream) {
    pa::PoolGeom g;
    pa::RowAttnPlan plan;
    size_t need = 0;
    pa_status st = check_decode(q, q_row_stride, num_q_heads, k_pool, v_pool, pool, context_lens, block_table,
                                block_table_stride, num_seqs, max_context_len, softmax_scale, out, &g, &plan, &need);
    if (st != PA_OK || num_seqs == 0) return st;
    if (need && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    return from_hip(pa::launch_decode(q, q_row_stride, num_q_heads, k_pool, v_pool, g, context_lens,
                                      block_table, block_table_stride, plan, softmax_scale, row_order,
                                      out, workspace, (hipStream_t)stream));
}

pa_status pa_decode_static(const void *q, int64_t q_row_stride, int32_t num_q_heads, const void *k_pool,
                           const void *v_pool, const pa_pool *pool, const int32_t *context_lens,
                           const int32_t *block_table, int32_t block_table_stride, int32_t num_seqs,
                           int32_t max_context_len, float softmax_scale, const int32_t *row_order, void *out,
                           void *stream) {
    pa::PoolGeom g;
    pa::RowAttnPlan plan;
    size_t need = 0;
    pa_status st = check_decode(q, q_row_stride, num_q_heads, k_pool, v_pool, pool, context_lens, block_table,
                                block_table_stride, num_seqs, max_context_len, softmax_scale, out, &g, &plan, &need);
    if (st != PA_OK || num_seqs == 0) return st;
    if (need > pa::kStaticScratchBytes) return PA_ERR_WORKSPACE;  // before any device call
    void *ws = nullptr;
    if (need && pa::static_scratch(&ws) != hipSuccess) return PA_ERR_HIP;
    return from_hip(pa::launch_decode(q, q_row_stride, num_q_heads, k_pool, v_pool, g, context_lens,
                                      block_table, block_table_stride, plan, softmax_scale, row_order,
                                      out, ws, (hipStream_t)stream));
}

size_t pa_decode_int8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                      const pa_pool *pool) {
    pa::PoolGeom g;
    if (check_decode_int8_shape(pool, num_q_heads, PA_BF16, &g) != PA_OK) return 0;
    if (num_seqs <= 0 || max_context_len <= 0) return 0;
    const pa::RowAttnPlan plan = pa::plan_row_attention(num_seqs, g, num_q_heads / g.hkv, max_context_len);
    return pa::row_attention_workspace_bytes(plan, num_q_heads, g.d);
}

pa_status pa_decode_int8(const void *q, int64_t q_row_stride, int32_t num_q_heads, int32_t q_dtype,
                         const void *k_pool, const void *v_pool, const void *k_scale, const void *v_scale,
                         const pa_pool *pool, const int32_t *context_lens, const int32_t *block_table,
                         int32_t block_table_stride, int32_t num_seqs, int32_t max_context_len, float softmax_scale,
                         const int32_t *row_order, void *out, void *workspace, size_t workspace_bytes,
                         void *stream) {
    pa::PoolGeom g;
    pa_status st = check_decode_int8_shape(pool, num_q_heads, q_dtype, &g);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || max_context_len < 0) return PA_ERR_BAD_SHAPE;
    if (!scale_ok(softmax_scale)) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !context_lens || !block_table || !out)
        return PA_ERR_NULL_ARG;
    if (block_table_stride <= 0) return PA_ERR_BAD_SHAPE;
    if (q_row_stride < (int64_t)num_q_heads * g.d) return PA_ERR_BAD_SHAPE;
    const int eb = elem_bytes(q_dtype);
    if (!aligned16(q) || (q_row_stride * eb) % 16 || !aligned16(k_pool) || !aligned16(v_pool) ||
        ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 1))
        return PA_ERR_UNSUPPORTED;
    const int group = num_q_heads / g.hkv;
    const pa::RowAttnPlan plan = pa::plan_row_attention(num_seqs, g, group, max_context_len);
    const size_t need = pa::row_attention_workspace_bytes(plan, num_q_heads, g.d);
    if (need && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    return from_hip(pa::launch_decode_int8(q, q_row_stride, num_q_heads, q_dtype, k_pool, v_pool, k_scale, v_scale,
                                           g, context_lens, block_table, block_table_stride, plan, softmax_scale,
                                           row_order, out, workspace, (hipStream_t)stream));
}

size_t pa_prefill_int8_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                                       int32_t max_seqlen_k, const pa_pool *pool) {
    pa::PoolGeom g;
    if (check_decode_int8_shape(pool, num_q_heads, PA_BF16, &g) != PA_OK) return 0;
    if (num_seqs <= 0 || total_q <= 0 || max_seqlen_k <= 0) return 0;
    // the row path's split partials (the MFMA path for bf16 and fp16 queries
    // needs none; fp32 queries and unsupported shapes take the row path, so
    // the size covers it)
    const pa::RowAttnPlan plan = pa::plan_row_attention(total_q, g, num_q_heads / g.hkv, max_seqlen_k);
    return pa::row_attention_workspace_bytes(plan, num_q_heads, g.d);
}

pa_status pa_prefill_varlen_int8(const void *q, int64_t q_row_stride, int32_t num_q_heads, int32_t q_dtype,
                                 const void *k_pool, const void *v_pool, const void *k_scale, const void *v_scale,
                                 const pa_pool *pool, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                 const int32_t *q_offsets, const int32_t *block_table, int32_t block_table_stride,
                                 int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 float softmax_scale, void *out, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    (void)max_seqlen_q;
    pa::PoolGeom g;
    pa_status st = check_decode_int8_shape(pool, num_q_heads, q_dtype, &g);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return PA_ERR_BAD_SHAPE;
    if (!scale_ok(softmax_scale)) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0 || total_q == 0) return PA_OK;
    if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !cu_seqlens_q || !cu_seqlens_k || !q_offsets ||
        !block_table || !out)
        return PA_ERR_NULL_ARG;
    if (block_table_stride <= 0) return PA_ERR_BAD_SHAPE;
    if (q_row_stride < (int64_t)num_q_heads * g.d) return PA_ERR_BAD_SHAPE;
    const int eb = elem_bytes(q_dtype);
    if (!aligned16(q) || (q_row_stride * eb) % 16 || !aligned16(k_pool) || !aligned16(v_pool) ||
        ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 1))
        return PA_ERR_UNSUPPORTED;
    const int group = num_q_heads / g.hkv;
    if ((q_dtype == PA_BF16 || q_dtype == PA_F16) && pa::prefill_mfma_int8_supported(g, group) && aligned16(out) &&
        !((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3))
        return from_hip(pa::launch_prefill_mfma_int8(q, q_row_stride, num_q_heads, q_dtype, k_pool, v_pool, k_scale,
                                                     v_scale,
                                                     g, cu_seqlens_q, cu_seqlens_k, q_offsets, block_table,
                                                     block_table_stride, num_seqs, total_q, max_seqlen_q, softmax_scale,
                                                     out, (hipStream_t)stream));
    const pa::RowAttnPlan plan = pa::plan_row_attention(total_q, g, group, max_seqlen_k);
    const size_t need = pa::row_attention_workspace_bytes(plan, num_q_heads, g.d);
    if (need && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    return from_hip(pa::launch_prefill_rows_int8(q, q_row_stride, num_q_heads, q_dtype, k_pool, v_pool, k_scale,
                                                 v_scale, g, cu_seqlens_q, cu_seqlens_k, q_offsets, block_table,
                                                 block_table_stride, num_seqs, plan, softmax_scale, out, workspace,
                                                 (hipStream_t)stream));
}

pa_status pa_decode_order(const int32_t *context_lens, int32_t num_seqs, int32_t *row_order, void *stream) {
    if (num_seqs < 0) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!context_lens || !row_order) return PA_ERR_NULL_ARG;
    if (num_seqs > pa::kDecodeOrderMax) return PA_ERR_UNSUPPORTED;
    return from_hip(pa::launch_decode_order(context_lens, num_seqs, row_order, (hipStream_t)stream));
}

pa_status pa_gather_kv(const void *k_pool, const void *v_pool, const pa_pool *pool,
                       const int32_t *cu_seqlens_k, const int32_t *block_table,
                       int32_t block_table_stride, int32_t num_seqs, int32_t total_k, void *k_out,
                       void *v_out, void *stream) {
    pa::PoolGeom g;
    pa_status st = check_pool(pool, &g);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || total_k < 0) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0 || total_k == 0) return PA_OK;
    if (!k_pool || !v_pool || !cu_seqlens_k || !block_table || !k_out || !v_out) return PA_ERR_NULL_ARG;
    if (block_table_stride <= 0) return PA_ERR_BAD_SHAPE;
    if (((int64_t)g.hkv * g.d * elem_bytes(g.dtype)) % 16) return PA_ERR_UNSUPPORTED;
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_out) || !aligned16(v_out))
        return PA_ERR_UNSUPPORTED;
    return from_hip(pa::launch_gather_kv(k_pool, v_pool, g, cu_seqlens_k, block_table,
                                         block_table_stride, num_seqs, total_k, k_out, v_out,
                                         (hipStream_t)stream));
}

static pa_status check_slots(const int32_t *slot_mapping, int32_t num_slots, const pa_pool *pool,
                             char *why, size_t why_len) {
    if (!slot_mapping || num_slots <= 0) return PA_OK;
    const int64_t cap = pool->num_blocks * (int64_t)pool->block_size;
    std::vector<int32_t> seen;
    seen.reserve((size_t)num_slots);
    for (int32_t t = 0; t < num_slots; ++t) {
        const int32_t s = slot_mapping[t];
        if (s == -1) continue;
        if (s < 0 || s >= cap) {
            say(why, why_len, "slot_mapping[%lld] = %lld out of range", t, s);
            return PA_ERR_BAD_METADATA;
        }
        seen.push_back(s);
    }
    std::sort(seen.begin(), seen.end());
    for (size_t i = 1; i < seen.size(); ++i)
        if (seen[i] == seen[i - 1]) {
            say(why, why_len, "slot %lld stored twice (%lld)", seen[i], seen[i]);
            return PA_ERR_BAD_METADATA;
        }
    return PA_OK;
}

static pa_status check_table_row(const int32_t *block_table, int32_t stride, int32_t s, int64_t keys,
                                 const pa_pool *pool, char *why, size_t why_len) {
    const int64_t need = (keys + pool->block_size - 1) / pool->block_size;
    if (need > stride) {
        say(why, why_len, "sequence %lld needs %lld blocks, more than the table width", s, need);
        return PA_ERR_BAD_METADATA;
    }
    for (int64_t b = 0; b < need; ++b) {
        const int32_t p = block_table[(int64_t)s * stride + b];
        if (p < 0 || p >= pool->num_blocks) {
            say(why, why_len, "sequence %lld block id %lld out of range", s, p);
            return PA_ERR_BAD_METADATA;
        }
    }
    return PA_OK;
}

pa_status pa_validate_prefill_metadata(const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                       const int32_t *q_offsets, const int32_t *block_table,
                                       int32_t block_table_stride, int32_t num_seqs,
                                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                                       const int32_t *slot_mapping, int32_t num_slots,
                                       const pa_pool *pool, char *why, size_t why_len) {
    if (why && why_len) why[0] = 0;
    if (!pool) return PA_ERR_NULL_ARG;
    if (num_seqs < 0) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return check_slots(slot_mapping, num_slots, pool, why, why_len);
    if (!cu_seqlens_q || !cu_seqlens_k || !q_offsets || !block_table) return PA_ERR_NULL_ARG;
    if (pool->block_size <= 0) return PA_ERR_BAD_SHAPE;
    if (cu_seqlens_q[0] != 0 || cu_seqlens_k[0] != 0) {
        say(why, why_len, "cu_seqlens must start at 0 (q %lld, k %lld)", cu_seqlens_q[0], cu_seqlens_k[0]);
        return PA_ERR_BAD_METADATA;
    }
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t ql = (int64_t)cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        const int64_t kl = (int64_t)cu_seqlens_k[s + 1] - cu_seqlens_k[s];
        if (ql < 0 || kl < 0) {
            say(why, why_len, "sequence %lld has a negative length (%lld)", s, ql < 0 ? ql : kl);
            return PA_ERR_BAD_METADATA;
        }
        if (ql > max_seqlen_q || kl > max_seqlen_k) {
            say(why, why_len, "sequence %lld longer than max_seqlen (%lld)", s, ql > max_seqlen_q ? ql : kl);
            return PA_ERR_BAD_METADATA;
        }
        if ((int64_t)q_offsets[s] + ql != kl) {
            say(why, why_len, "sequence %lld: q_offset + q_len != k_len (k_len %lld)", s, kl);
            return PA_ERR_BAD_METADATA;
        }
        pa_status st = check_table_row(block_table, block_table_stride, s, kl, pool, why, why_len);
        if (st != PA_OK) return st;
    }
    return check_slots(slot_mapping, num_slots, pool, why, why_len);
}

pa_status pa_validate_decode_metadata(const int32_t *context_lens, const int32_t *block_table,
                                      int32_t block_table_stride, int32_t num_seqs,
                                      int32_t max_context_len, const int32_t *slot_mapping,
                                      const int32_t *row_order, const pa_pool *pool, char *why,
                                      size_t why_len) {
    if (why && why_len) why[0] = 0;
    if (!pool) return PA_ERR_NULL_ARG;
    if (num_seqs < 0) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!context_lens || !block_table) return PA_ERR_NULL_ARG;
    if (pool->block_size <= 0) return PA_ERR_BAD_SHAPE;
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (context_lens[s] < 0 || context_lens[s] > max_context_len) {
            say(why, why_len, "context_lens[%lld] = %lld outside [0, max_context_len]", s, context_lens[s]);
            return PA_ERR_BAD_METADATA;
        }
        pa_status st = check_table_row(block_table, block_table_stride, s, context_lens[s], pool, why, why_len);
        if (st != PA_OK) return st;
    }
    if (row_order) {  // a permutation of the rows
        std::vector<char> seen((size_t)num_seqs, 0);
        for (int32_t r = 0; r < num_seqs; ++r) {
            const int32_t s = row_order[r];
            if (s < 0 || s >= num_seqs || seen[(size_t)s]) {
                say(why, why_len, "row_order[%lld] = %lld is out of range or repeated", r, s);
                return PA_ERR_BAD_METADATA;
            }
            seen[(size_t)s] = 1;
        }
    }
    return check_slots(slot_mapping, num_seqs, pool, why, why_len);
}

}  // extern "C"
