/*
 * pa.h -- attention over a block-paged KV cache on AMD Instinct MI355X
 * (gfx950).  C ABI of libpa.so.
 *
 * The operations are the ones an LLM inference engine runs in every
 * attention layer (nano-vllm deep dive, Step 4 "Attention -- Triton Kernel +
 * Flash Attention"): write this step's K/V rows into the paged cache, then
 * run causal attention for a packed prefill batch or for one decode token per
 * sequence, reading keys and values through a per-sequence block table.
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless marked (host).  Buffers are owned by
 *    the caller and must stay alive until the work enqueued on `stream`
 *    completes.  `stream` is a hipStream_t (NULL = the default stream).
 *  - Calls only enqueue work on `stream`: no device synchronisation, no
 *    device-to-host copy, no allocation, no global mutable state (except
 *    pa_decode_static's per-GPU scratch array, see there).  They may be
 *    called from several host threads and captured in a HIP graph.
 *  - Errors: a pa_status is returned synchronously for problems visible on
 *    the host (null pointers, sizes, unsupported shapes, a workspace that is
 *    too small) and nothing is enqueued.  PA_ERR_HIP means a launch failed
 *    (hipGetLastError; no synchronisation).  The CONTENTS of device index
 *    arrays are preconditions that the hot path does not check on the host
 *    (checking them would need a sync): pa_validate_prefill_metadata and
 *    pa_validate_decode_metadata check host copies.  The kernels still never
 *    read a block-table entry past a sequence's last needed block, skip
 *    block ids outside [0, num_blocks) and slots outside the pool, so bad
 *    contents give wrong numbers, not out-of-bounds accesses of the pools.
 *  - No C++ exception crosses this interface.
 *
 * KV pool layout (nano-vllm deep dive, Step 5, "KV Cache memory layout"):
 * one K pool and one V pool per layer, each a contiguous
 *     [num_blocks][block_size][num_kv_heads][head_dim]
 * array of `dtype` elements.  Token j of a sequence lives in physical block
 * block_table[s][j / block_size] at offset j % block_size (same page,
 * Step 1, "why block_table"); its flat slot is block * block_size + offset.
 *
 * Supported: dtype PA_F32, PA_BF16 or PA_F16 (IEEE binary16, the element
 * type of the fork's fused-dequantization microbenchmark: LLM inference
 * interview notes (nano-vllm fork), Q3, the INT8-versus-FP16 latency table);
 * head_dim 32, 64, 128 or 256;
 * block_size a power of two (1 .. 65536); num_kv_heads at most 65536, with
 * num_kv_heads * block_size below 2^31 (PA_ERR_UNSUPPORTED otherwise: the
 * kernels index a block's (slot, head) rows in 32 bits); num_q_heads a multiple of
 * num_kv_heads with group size num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * The bf16 and fp16 prefills run on MFMA for head_dim 64, 128 and 256 with
 * block_size >= 4; every other supported shape runs on the vector ALU path.
 * Outputs of a 16-bit type are
 * the fp32 result rounded to nearest even (fp16: beyond +-65504 it is +-inf).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 6

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                      */
    PA_ERR_BAD_SHAPE = 2,    /* a size or stride is negative or inconsistent    */
    PA_ERR_BAD_DTYPE = 3,    /* dtype not supported by this call                */
    PA_ERR_UNSUPPORTED = 4,  /* head_dim, block_size or group size not built    */
    PA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the *_bytes call */
    PA_ERR_HIP = 6,          /* a kernel launch failed                          */
    PA_ERR_BAD_METADATA = 7  /* (validators only) host copy of metadata invalid */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_INT8 = 2, PA_F16 = 3 } pa_dtype;

/* Shape of one layer's K pool (the V pool has the same shape). Host struct. */
typedef struct {
    int64_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype; /* pa_dtype */
} pa_pool;

/*
 * pa_store_kv -- scatter this step's K/V rows into the paged pools.
 * (nano-vllm deep dive, Step 4, "Triton Kernel: write KV Cache", and the
 * slot_mapping note there: slot = block_table[block] * block_size + offset.)
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim] rows, `pool->dtype`;
 *                 row t starts at element t * k_row_stride (v_row_stride);
 *                 strides are in elements and >= num_kv_heads * head_dim.
 *   slot_mapping  int32 [num_tokens]; slot -1 = padding token, skipped.
 *   k_pool,v_pool the layer's pools (see layout above), written in place.
 * Row t is copied bit-for-bit to flat slot slot_mapping[t].  Slots must be
 * unique within one call (precondition).  num_tokens == 0 is a no-op.
 */
pa_status pa_store_kv(const void *k, int64_t k_row_stride,
                      const void *v, int64_t v_row_stride,
                      const int32_t *slot_mapping, int32_t num_tokens,
                      void *k_pool, void *v_pool, const pa_pool *pool /* host */,
                      void *stream);

/*
 * INT8 KV cache (LLM inference interview notes (nano-vllm fork), Q3: how
 * quantization and dequantization are done).  An INT8 layer has, per K and
 * per V, a code pool and a scale pool indexed by the same slot:
 *   codes   int8    [num_blocks][block_size][num_kv_heads][head_dim]
 *   scales  float16 [num_blocks][block_size][num_kv_heads]  (IEEE binary16)
 * described by a pa_pool with dtype PA_INT8.  One (token, KV head) takes
 * head_dim + 2 bytes (130 B at head_dim 128, against 256 B in bf16).
 *
 * pa_store_kv_int8 -- quantize this step's K/V rows into INT8 pools (part 1
 * of that answer: quantization happens on write, inside the store).  For
 * each token t with slot_mapping[t] != -1 and each KV head h, over the
 * head_dim values x of that head:
 *   scale   = max(max_i |x_i| / 127, 1e-8)     fp32; IEEE division
 *   code_i  = trunc(x_i / scale + 0.5)  if x_i / scale >= 0
 *             trunc(x_i / scale - 0.5)  otherwise            (fp32)
 * and the scale is stored as fp16 (round to nearest even; 1e-8 and other
 * scales below fp16's range store as 0, whose codes are all 0 anyway).
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim] rows of src_dtype
 *                 (PA_BF16, PA_F16 or PA_F32), strides in elements as in
 *                 pa_store_kv;
 *                 values must be finite and |x| <= 65504 * 127.
 *   slot_mapping  int32 [num_tokens]; -1 = padding token, skipped.
 *   k_pool,v_pool int8 code pools, 8-byte aligned; k_scale,v_scale fp16
 *                 scale pools; all written in place.
 *   pool          dtype PA_INT8; head_dim a power of two from 8 to 256 (a
 *                 head vector's lanes reduce its max |x| as one group).
 * Errors: PA_ERR_BAD_DTYPE (pool not PA_INT8, src_dtype not bf16/fp16/fp32),
 * PA_ERR_UNSUPPORTED (head_dim, block_size, misaligned pools), the checks of
 * pa_store_kv otherwise.  Slots must be unique within one call.
 */
pa_status pa_store_kv_int8(const void *k, int64_t k_row_stride,
                           const void *v, int64_t v_row_stride, int32_t src_dtype,
                           const int32_t *slot_mapping, int32_t num_tokens,
                           void *k_pool, void *v_pool, void *k_scale, void *v_scale,
                           const pa_pool *pool /* host */, void *stream);

/*
 * pa_decode_int8 -- pa_decode over INT8 pools, with the dequantization fused
 * into the attention (the same answer, part 2: K/V are read as int8, widened
 * and scaled in registers; no float copy of the cache is made).  It computes
 * pa_decode's result with K and V replaced by their dequantized values
 * code * float(scale).  As the pages suggest, the K scale multiplies each
 * finished dot product and the V scale is folded into the probability.
 *
 *   q, out        [num_seqs][num_q_heads][head_dim] of q_dtype (PA_BF16,
 *                 PA_F16 or PA_F32); q rows at q_row_stride elements, 16-byte
 *                 aligned;
 *                 bf16 q values must lie within fp16's range (|q| <= 65504;
 *                 the K dot products run on fp16 pairs).
 *   k_pool,v_pool int8 code pools, 16-byte aligned; k_scale,v_scale fp16
 *                 scale pools (layout above); pool->dtype PA_INT8.
 *   everything else as pa_decode (context_lens, block_table, row_order,
 *                 workspace from pa_decode_int8_workspace_bytes).
 * Query groups (num_q_heads / num_kv_heads) of 1, 2, 4 or 8 (a group of 8
 * reads each K/V byte twice, once per half of its query heads); head_dim 32,
 * 64, 128 or 256 (else PA_ERR_UNSUPPORTED).  Errors as pa_decode.
 */
size_t pa_decode_int8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_context_len, const pa_pool *pool /* host */);
pa_status pa_decode_int8(const void *q, int64_t q_row_stride, int32_t num_q_heads, int32_t q_dtype,
                         const void *k_pool, const void *v_pool,
                         const void *k_scale, const void *v_scale, const pa_pool *pool /* host */,
                         const int32_t *context_lens, const int32_t *block_table,
                         int32_t block_table_stride, int32_t num_seqs, int32_t max_context_len,
                         float softmax_scale, const int32_t *row_order, void *out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_prefill_varlen_int8 -- pa_prefill_varlen over INT8 pools, with the
 * dequantization fused into the attention instead of first gathering the
 * referenced K/V into a float tensor (the slow path the same answer, part 3,
 * describes for prefill).  Same arguments, semantics and errors as
 * pa_prefill_varlen, plus q_dtype (PA_BF16 / PA_F16 / PA_F32, also out's
 * type) and the fp16 scale pools; INT8 pools as for pa_decode_int8 (query
 * groups 1, 2, 4, 8).  bf16 or fp16 queries with head_dim 64 or 128, an even
 * number of KV heads, a 16-byte aligned out and 4-byte aligned scale pools
 * run on the matrix cores (each key step's codes are dequantized to the query
 * type in LDS; for fp16 they saturate at +-65504); every other call takes
 * each packed query token as one row of the INT8 decode pass over its
 * visible keys (vector ALU).
 */
size_t pa_prefill_int8_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                                       int32_t max_seqlen_k, const pa_pool *pool /* host */);
pa_status pa_prefill_varlen_int8(const void *q, int64_t q_row_stride, int32_t num_q_heads, int32_t q_dtype,
                                 const void *k_pool, const void *v_pool,
                                 const void *k_scale, const void *v_scale, const pa_pool *pool /* host */,
                                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                 const int32_t *q_offsets, const int32_t *block_table,
                                 int32_t block_table_stride, int32_t num_seqs, int32_t total_q,
                                 int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                                 void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_copy_blocks -- copy-on-write of shared, mutable last blocks (vLLM/SGLang
 * interview labs, section 4, the follow-up on a native block-table fork: the
 * parent and child share block ids; an append that would land in a shared,
 * still-mutable last block first gives the child a new block holding a copy
 * of the valid KV; full immutable blocks are never copied).  For each pair i,
 * slots 0 .. num_valid[i]-1 of physical block src_blocks[i] are copied bit for
 * bit to the same slots of block dst_blocks[i], in the K and V pools and, for
 * PA_INT8 pools, in the scale pools; every other slot is left unchanged.
 *
 *   k_pool, v_pool   the layer's pools (any dtype); k_scale, v_scale the fp16
 *                    scale pools of a PA_INT8 layer (ignored otherwise).
 *   src_blocks, dst_blocks, num_valid   device int32 [num_pairs].
 * Preconditions: destination blocks are distinct and none is a source in the
 * same call.  Pairs with ids outside [0, num_blocks) or num_valid outside
 * [1, block_size] are skipped.  Errors: the pool checks of pa_store_kv /
 * pa_store_kv_int8; num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(void *k_pool, void *v_pool, void *k_scale, void *v_scale,
                         const pa_pool *pool /* host */, const int32_t *src_blocks,
                         const int32_t *dst_blocks, const int32_t *num_valid, int32_t num_pairs,
                         void *stream);

/*
 * pa_prefill_varlen -- causal attention for a packed variable-length batch
 * over the paged cache (nano-vllm deep dive, Step 4, flash_attn_varlen_func
 * with cu_seqlens_q / cu_seqlens_k / block_table, causal; Step 5,
 * prepare_prefill: query tokens are the uncached ones, keys are all tokens).
 *
 *   q             [total_q][num_q_heads][head_dim], row stride q_row_stride
 *                 elements (>= num_q_heads * head_dim), `pool->dtype`.
 *   cu_seqlens_q  int32 [num_seqs + 1], cu_seqlens_q[0] = 0, non-decreasing,
 *                 cu_seqlens_q[num_seqs] = total_q.  Sequence s owns query
 *                 rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1.
 *   cu_seqlens_k  int32 [num_seqs + 1]: k_len(s) = cu_seqlens_k[s+1] -
 *                 cu_seqlens_k[s] keys, ALL already in the pools (call
 *                 pa_store_kv for the new tokens first, on the same stream).
 *   q_offsets     int32 [num_seqs]: cached-prefix length of sequence s;
 *                 query i of s sits at absolute position q_offsets[s] + i
 *                 and sees keys 0 .. min(q_offsets[s] + i, k_len(s) - 1)
 *                 (bottom-right causal alignment).  Normally q_offsets[s] +
 *                 q_len(s) == k_len(s).
 *   block_table   int32 [num_seqs][block_table_stride] physical block ids;
 *                 only the first ceil(k_len(s) / block_size) entries of a
 *                 row are read.
 *   max_seqlen_q, max_seqlen_k  host upper bounds of q_len(s) and k_len(s)
 *                 (they size the launch; no device read is needed, so a
 *                 call captured in a HIP graph with bounds stays valid for
 *                 any lengths within them).
 *   softmax_scale multiplies q . k before the softmax (usually 1/sqrt(d));
 *                 it must be finite and > 0 (else PA_ERR_BAD_SHAPE).
 *   out           [total_q][num_q_heads][head_dim] contiguous, `pool->dtype`
 *                 (bf16 output is rounded to nearest-even).
 *   workspace     device scratch of at least pa_prefill_workspace_bytes(...)
 *                 bytes (may be NULL when that returns 0).
 * Sequences with q_len 0 are no-ops; a query row with no visible key
 * (k_len 0) gets a zero output.
 */
pa_status pa_prefill_varlen(const void *q, int64_t q_row_stride, int32_t num_q_heads,
                            const void *k_pool, const void *v_pool, const pa_pool *pool /* host */,
                            const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                            const int32_t *q_offsets, const int32_t *block_table,
                            int32_t block_table_stride, int32_t num_seqs, int32_t total_q,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                            void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode -- one query token per sequence against its paged context
 * (nano-vllm deep dive, Step 4, flash_attn_with_kvcache with cache_seqlens
 * and block_table; Step 5, prepare_decode: context length = len(seq), the
 * new token included; its K/V must already be stored).
 *
 *   q             [num_seqs][num_q_heads][head_dim], row stride q_row_stride.
 *   context_lens  int32 [num_seqs]; sequence s attends to keys
 *                 0 .. context_lens[s]-1.  0 marks a padding row (output 0).
 *   block_table   int32 [num_seqs][block_table_stride].
 *   max_context_len  host upper bound of context_lens: it sizes the launch
 *                 and the workspace; each row's split count is then chosen
 *                 on the device from its own context length.  So a call
 *                 captured in a HIP graph with max_context_len = the table's
 *                 capacity (block_table_stride * block_size) stays valid for
 *                 every context length up to it (fork Q&A, general Q&A: the
 *                 graph-versus-kernel-choice trade-off).
 *   softmax_scale as for pa_prefill_varlen (finite, > 0).
 *   row_order     NULL, or int32 [num_seqs]: a permutation of 0..num_seqs-1
 *                 (precondition; pa_validate_decode_metadata checks a host
 *                 copy) giving the order in which rows are scheduled, e.g.
 *                 from pa_decode_order.  It changes the launch order only:
 *                 outputs are bit-identical with or without it.
 *   out           [num_seqs][num_q_heads][head_dim] contiguous.
 *   workspace     >= pa_decode_workspace_bytes(...) bytes: split-K partial
 *                 results (running max, normaliser and fp32 accumulator per
 *                 split), merged by log-sum-exp (fork Q&A, general Q&A,
 *                 "what is split-K").
 */
pa_status pa_decode(const void *q, int64_t q_row_stride, int32_t num_q_heads,
                    const void *k_pool, const void *v_pool, const pa_pool *pool /* host */,
                    const int32_t *context_lens, const int32_t *block_table,
                    int32_t block_table_stride, int32_t num_seqs, int32_t max_context_len,
                    float softmax_scale, const int32_t *row_order, void *out, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * pa_decode_static -- pa_decode without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It computes pa_decode's result
 * with the same kernels and the same split plan; the split-K partials go to a
 * device array the library defines at file scope, 16 MiB per GPU (held by
 * each GPU the library runs on until the process ends).  Its address on the
 * current device is looked up once per device (hipGetSymbolAddress, no
 * allocation); the call itself allocates and frees nothing.
 *
 * Arguments as pa_decode, minus workspace and workspace_bytes.
 * Errors: those of pa_decode; PA_ERR_WORKSPACE when the partials this call
 * needs (pa_decode_workspace_bytes with the same sizes) exceed 16 MiB,
 * returned before any device call; PA_ERR_HIP if the lookup fails.
 * Every call on one GPU shares that GPU's array and leaves its partials in
 * it: calls that overlap on one GPU (several streams or host threads at once)
 * race and give wrong results; calls ordered on one stream are safe.  The
 * array needs no clearing: each call writes every partial it reads.
 */
pa_status pa_decode_static(const void *q, int64_t q_row_stride, int32_t num_q_heads,
                           const void *k_pool, const void *v_pool, const pa_pool *pool /* host */,
                           const int32_t *context_lens, const int32_t *block_table,
                           int32_t block_table_stride, int32_t num_seqs, int32_t max_context_len,
                           float softmax_scale, const int32_t *row_order, void *out, void *stream);

/*
 * pa_decode_order -- scheduling aid for pa_decode, not an operation of the
 * pages: writes row_order (int32 [num_seqs], device) = the rows sorted by
 * decreasing context_lens, ties by row index.  A decode step has the same
 * context lengths in every layer, so one call per step serves all layers'
 * pa_decode calls.  With ragged contexts and more (row, KV head) work items
 * than the GPU runs at once, longest-first scheduling keeps a long row from
 * running alone at the end of the launch.  num_seqs <= 2048 (else
 * PA_ERR_UNSUPPORTED: pass row_order = NULL); 0 is a no-op.
 */
pa_status pa_decode_order(const int32_t *context_lens, int32_t num_seqs, int32_t *row_order,
                          void *stream);

/* Workspace sizes (bytes) for the matching calls with the same host sizes. */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  const pa_pool *pool /* host */);
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 const pa_pool *pool /* host */);

/*
 * pa_gather_kv -- test and debug helper, not on the hot path: copy every
 * sequence's keys/values out of the pools, walking the block table, into
 * packed [total_k][num_kv_heads][head_dim] arrays (row cu_seqlens_k[s] + j
 * holds key j of sequence s).  Bit-exact.  (mini-infer 03, section 2: the
 * dense gather that paged attention avoids.)
 */
pa_status pa_gather_kv(const void *k_pool, const void *v_pool, const pa_pool *pool /* host */,
                       const int32_t *cu_seqlens_k, const int32_t *block_table,
                       int32_t block_table_stride, int32_t num_seqs, int32_t total_k,
                       void *k_out, void *v_out, void *stream);

/*
 * Host-side validators of HOST copies of the metadata (never called by the
 * hot path).  They return PA_OK or PA_ERR_BAD_METADATA / PA_ERR_BAD_SHAPE and
 * write a short reason into `why` (host buffer of why_len bytes, may be NULL).
 * Prefill: cu_seqlens monotone from 0, q_len <= k_len, q_offsets[s] + q_len
 * == k_len, lengths within the maxima and the block table width, block ids of
 * every needed entry in range.  slot_mapping (may be NULL): ids in range or
 * -1, no duplicates.  Decode: 0 <= context_lens <= max_context_len, ids in
 * range; row_order (may be NULL) a permutation of the rows.
 */
pa_status pa_validate_prefill_metadata(const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                       const int32_t *q_offsets, const int32_t *block_table,
                                       int32_t block_table_stride, int32_t num_seqs,
                                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                                       const int32_t *slot_mapping, int32_t num_slots,
                                       const pa_pool *pool, char *why, size_t why_len);
pa_status pa_validate_decode_metadata(const int32_t *context_lens, const int32_t *block_table,
                                      int32_t block_table_stride, int32_t num_seqs,
                                      int32_t max_context_len, const int32_t *slot_mapping,
                                      const int32_t *row_order, const pa_pool *pool, char *why,
                                      size_t why_len);

const char *pa_status_string(pa_status status);
int pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
