// pa_store.hip -- KV scatter into the paged pools, and the gather helper.
//
// Store (nano-vllm deep dive, Step 4, "Triton Kernel: write KV Cache"): the
// K row and V row of token t go to flat slot slot_mapping[t] of the pools;
// slot -1 is a padding token and is skipped.  Bits are copied unchanged.
//
// Design for gfx950: one lane moves one 16-byte chunk of K and one of V, so a
// wave moves 1 KiB of each per instruction; a token row of Hkv*d elements
// (2 KiB at 8 heads x 128 x bf16) is 128 lanes.  When the rows or the
// pointers are not 16-byte aligned a lane copies single elements instead.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kStoreThreads = 256;

__global__ __launch_bounds__(kStoreThreads) void store_kv_vec16(
    const char *__restrict__ k, int64_t k_stride_bytes, const char *__restrict__ v,
    int64_t v_stride_bytes, const int32_t *__restrict__ slot_mapping, int64_t num_chunks,
    int chunks_per_row, char *__restrict__ k_pool, char *__restrict__ v_pool, int64_t num_slots) {
    const int64_t i = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x;
    if (i >= num_chunks) return;
    const int64_t t = i / chunks_per_row;
    const int c = (int)(i - t * chunks_per_row);
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;  // -1: padding token
    const int64_t row_bytes = (int64_t)chunks_per_row * 16;
    const uint4 kv = ld16(k + t * k_stride_bytes + c * 16);
    const uint4 vv = ld16(v + t * v_stride_bytes + c * 16);
    *reinterpret_cast<uint4 *>(k_pool + slot * row_bytes + c * 16) = kv;
    *reinterpret_cast<uint4 *>(v_pool + slot * row_bytes + c * 16) = vv;
}

template <typename W>
__global__ __launch_bounds__(kStoreThreads) void store_kv_elem(
    const W *__restrict__ k, int64_t k_stride, const W *__restrict__ v, int64_t v_stride,
    const int32_t *__restrict__ slot_mapping, int64_t num_elems, int row_elems,
    W *__restrict__ k_pool, W *__restrict__ v_pool, int64_t num_slots) {
    const int64_t i = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x;
    if (i >= num_elems) return;
    const int64_t t = i / row_elems;
    const int e = (int)(i - t * row_elems);
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    k_pool[slot * row_elems + e] = k[t * k_stride + e];
    v_pool[slot * row_elems + e] = v[t * v_stride + e];
}

// Gather (test helper): packed row cu_seqlens_k[s] + j <- key j of sequence s,
// found through block_table[s][j / block_size].
__global__ __launch_bounds__(kStoreThreads) void gather_kv_vec16(
    const char *__restrict__ k_pool, const char *__restrict__ v_pool, int64_t num_blocks,
    int block_shift, int chunks_per_row, const int32_t *__restrict__ cu_seqlens_k,
    const int32_t *__restrict__ block_table, int bt_stride, int num_seqs, int64_t num_chunks,
    char *__restrict__ k_out, char *__restrict__ v_out) {
    const int64_t i = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x;
    if (i >= num_chunks) return;
    const int64_t row = i / chunks_per_row;
    const int c = (int)(i - row * chunks_per_row);
    // owning sequence: largest s with cu_seqlens_k[s] <= row
    int lo = 0, hi = num_seqs;  // invariant: cu[lo] <= row < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_seqlens_k[mid] <= row) lo = mid; else hi = mid;
    }
    const int64_t j = row - cu_seqlens_k[lo];
    if ((j >> block_shift) >= bt_stride) return;
    const int64_t blk = block_table[(int64_t)lo * bt_stride + (j >> block_shift)];
    if (blk < 0 || blk >= num_blocks) return;
    const int64_t slot = (blk << block_shift) + (j & ((1 << block_shift) - 1));
    const int64_t row_bytes = (int64_t)chunks_per_row * 16;
    *reinterpret_cast<uint4 *>(k_out + row * row_bytes + c * 16) = ld16(k_pool + slot * row_bytes + c * 16);
    *reinterpret_cast<uint4 *>(v_out + row * row_bytes + c * 16) = ld16(v_pool + slot * row_bytes + c * 16);
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_store_kv(const void *k, int64_t k_row_stride, const void *v, int64_t v_row_stride,
                           const int32_t *slot_mapping, int num_tokens, void *k_pool, void *v_pool,
                           const PoolGeom &g, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int eb = g.dtype == 0 ? 4 : 2;
    const int row_elems = g.hkv * g.d;
    const int64_t row_bytes = (int64_t)row_elems * eb;
    const int64_t num_slots = g.num_blocks << g.block_shift;
    const bool vec = row_bytes % 16 == 0 && (k_row_stride * eb) % 16 == 0 &&
                     (v_row_stride * eb) % 16 == 0 && aligned16(k) && aligned16(v) &&
                     aligned16(k_pool) && aligned16(v_pool);
    if (vec) {
        const int cpr = (int)(row_bytes / 16);
        const int64_t n = (int64_t)num_tokens * cpr;
        const unsigned grid = (unsigned)((n + kStoreThreads - 1) / kStoreThreads);
        hipLaunchKernelGGL(store_kv_vec16, dim3(grid), dim3(kStoreThreads), 0, stream,
                           (const char *)k, k_row_stride * eb, (const char *)v, v_row_stride * eb,
                           slot_mapping, n, cpr, (char *)k_pool, (char *)v_pool, num_slots);
    } else {
        const int64_t n = (int64_t)num_tokens * row_elems;
        const unsigned grid = (unsigned)((n + kStoreThreads - 1) / kStoreThreads);
        if (eb == 4)
            hipLaunchKernelGGL(store_kv_elem<uint32_t>, dim3(grid), dim3(kStoreThreads), 0, stream,
                               (const uint32_t *)k, k_row_stride, (const uint32_t *)v, v_row_stride,
                               slot_mapping, n, row_elems, (uint32_t *)k_pool, (uint32_t *)v_pool,
                               num_slots);
        else
            hipLaunchKernelGGL(store_kv_elem<uint16_t>, dim3(grid), dim3(kStoreThreads), 0, stream,
                               (const uint16_t *)k, k_row_stride, (const uint16_t *)v, v_row_stride,
                               slot_mapping, n, row_elems, (uint16_t *)k_pool, (uint16_t *)v_pool,
                               num_slots);
    }
    return hipGetLastError();
}

hipError_t launch_gather_kv(const void *k_pool, const void *v_pool, const PoolGeom &g,
                            const int32_t *cu_seqlens_k, const int32_t *block_table, int bt_stride,
                            int num_seqs, int total_k, void *k_out, void *v_out, hipStream_t stream) {
    if (total_k == 0 || num_seqs == 0) return hipSuccess;
    const int eb = g.dtype == 0 ? 4 : 2;
    const int cpr = g.hkv * g.d * eb / 16;  // supported head_dim keeps rows a multiple of 16 B
    const int64_t n = (int64_t)total_k * cpr;
    const unsigned grid = (unsigned)((n + kStoreThreads - 1) / kStoreThreads);
    hipLaunchKernelGGL(gather_kv_vec16, dim3(grid), dim3(kStoreThreads), 0, stream,
                       (const char *)k_pool, (const char *)v_pool, g.num_blocks, g.block_shift, cpr,
                       cu_seqlens_k, block_table, bt_stride, num_seqs, n, (char *)k_out,
                       (char *)v_out);
    return hipGetLastError();
}

}  // namespace pa
