// pa_kernels.h -- internal launchers of libpa (host side).  Not part of the
// C ABI; the extern "C" entry points in pa_api.cpp validate arguments and
// call these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Geometry of one layer's K (and V) pool: [num_blocks][block_size][hkv][d].
struct PoolGeom {
    int64_t num_blocks;
    int block_size;    // power of two
    int block_shift;   // log2(block_size)
    int hkv;
    int d;
    int dtype;         // 0 fp32, 1 bf16, 2 int8 (with fp16 scale pools), 3 fp16
};

// Store / gather ---------------------------------------------------------
hipError_t launch_store_kv(const void *k, int64_t k_row_stride, const void *v, int64_t v_row_stride,
                           const int32_t *slot_mapping, int num_tokens, void *k_pool, void *v_pool,
                           const PoolGeom &g, hipStream_t stream);

// INT8 pools: quantize K/V rows (src_dtype 0 fp32, 1 bf16, 3 fp16) per (token, KV
// head) into int8 codes and fp16 scales.
hipError_t launch_store_kv_int8(const void *k, int64_t k_row_stride, const void *v, int64_t v_row_stride,
                                int src_dtype, const int32_t *slot_mapping, int num_tokens, void *k_pool,
                                void *v_pool, void *k_scale, void *v_scale, const PoolGeom &g,
                                hipStream_t stream);

// Copy slots 0 .. num_valid[i]-1 of block src_blocks[i] to block
// dst_blocks[i] in one pool whose slots are slot_bytes bytes.
hipError_t launch_copy_blocks(void *pool, int64_t slot_bytes, const PoolGeom &g, const int32_t *src_blocks,
                              const int32_t *dst_blocks, const int32_t *num_valid, int num_pairs,
                              hipStream_t stream);

hipError_t launch_gather_kv(const void *k_pool, const void *v_pool, const PoolGeom &g,
                            const int32_t *cu_seqlens_k, const int32_t *block_table, int bt_stride,
                            int num_seqs, int total_k, void *k_out, void *v_out, hipStream_t stream);

// Split-K row attention (decode, and the vector-ALU prefill path) ---------
// A "row" is one query token: row r of a decode batch is sequence r; row r
// of a prefill batch is packed query token r.
struct RowAttnPlan {
    int num_rows;
    int num_splits;     // split slots per row (grid dimension)
    int round_tokens;   // keys a workgroup takes per round; splits are whole rounds
    int split_cap;      // most keys one split may cover (a multiple of round_tokens)
    int waves;          // waves per workgroup
};

// The number of split slots is chosen from host sizes only (rows, KV heads,
// an upper bound of the keys per row), so workspace size and launch agree.
// Each row's own split length is chosen on the device from its key count
// (split_tokens_of in the kernels): a launch planned for a capacity serves
// every shorter row, which keeps one captured graph valid for any lengths.
RowAttnPlan plan_row_attention(int num_rows, const PoolGeom &g, int group, int max_keys);
size_t row_attention_workspace_bytes(const RowAttnPlan &p, int hq, int d);

hipError_t launch_decode(const void *q, int64_t q_row_stride, int hq, const void *k_pool,
                         const void *v_pool, const PoolGeom &g, const int32_t *context_lens,
                         const int32_t *block_table, int bt_stride, const RowAttnPlan &plan,
                         float softmax_scale, const int32_t *row_order, void *out, void *workspace,
                         hipStream_t stream);

// Decode over INT8 pools (int8 codes, fp16 scales per (token, KV head));
// q and out are q_dtype (0 fp32, 1 bf16, 3 fp16); query groups of 1, 2, 4 or
// 8 (8 runs as two virtual KV heads of 4 query heads per pool head).
hipError_t launch_decode_int8(const void *q, int64_t q_row_stride, int hq, int q_dtype, const void *k_pool,
                              const void *v_pool, const void *k_scale, const void *v_scale, const PoolGeom &g,
                              const int32_t *context_lens, const int32_t *block_table, int bt_stride,
                              const RowAttnPlan &plan, float softmax_scale, const int32_t *row_order, void *out,
                              void *workspace, hipStream_t stream);

// Query-tiled MFMA prefill over INT8 pools with bf16 or fp16 queries
// (q_dtype 1 or 3): each step's codes are dequantized to the query type in
// LDS (d 64/128, even hkv, groups 1/2/4/8).
bool prefill_mfma_int8_supported(const PoolGeom &g, int group);
hipError_t launch_prefill_mfma_int8(const void *q, int64_t q_row_stride, int hq, int q_dtype, const void *k_pool,
                                    const void *v_pool, const void *k_scale, const void *v_scale, const PoolGeom &g,
                                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                    const int32_t *q_offsets, const int32_t *block_table, int bt_stride,
                                    int num_seqs, int total_q, int max_seqlen_q, float softmax_scale, void *out,
                                    hipStream_t stream);

// Prefill over INT8 pools, one packed query token per row.
hipError_t launch_prefill_rows_int8(const void *q, int64_t q_row_stride, int hq, int q_dtype, const void *k_pool,
                                    const void *v_pool, const void *k_scale, const void *v_scale,
                                    const PoolGeom &g, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                    const int32_t *q_offsets, const int32_t *block_table, int bt_stride,
                                    int num_seqs, const RowAttnPlan &plan, float softmax_scale, void *out,
                                    void *workspace, hipStream_t stream);

// The device array that pa_decode_static uses in place of a caller
// workspace: kStaticScratchBytes per GPU, held until the process ends and
// shared by every such call on that GPU.  static_scratch() returns its
// address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(void **ptr);

// Longest-context-first permutation of decode rows (one workgroup).
constexpr int kDecodeOrderMax = 2048;
hipError_t launch_decode_order(const int32_t *context_lens, int num_rows, int32_t *row_order,
                               hipStream_t stream);

hipError_t launch_prefill_rows(const void *q, int64_t q_row_stride, int hq, const void *k_pool,
                               const void *v_pool, const PoolGeom &g, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, const int32_t *q_offsets,
                               const int32_t *block_table, int bt_stride, int num_seqs,
                               const RowAttnPlan &plan, float softmax_scale, void *out,
                               void *workspace, hipStream_t stream);

// MFMA prefill (bf16, head_dim 64 / 128) ----------------------------------
bool prefill_mfma_supported(const PoolGeom &g, int group);
hipError_t launch_prefill_mfma(const void *q, int64_t q_row_stride, int hq, const void *k_pool,
                               const void *v_pool, const PoolGeom &g, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, const int32_t *q_offsets,
                               const int32_t *block_table, int bt_stride, int num_seqs, int total_q,
                               int max_seqlen_q, float softmax_scale, void *out, hipStream_t stream);

}  // namespace pa
