// pa_store.hip -- KV scatter into the paged pools, and the gather helper.
//
// Store (nano-vllm deep dive, Step 4, "Triton Kernel: write KV Cache"): the
// K row and V row of token t go to flat slot slot_mapping[t] of the pools;
// slot -1 is a padding token and is skipped.  Bits are copied unchanged.
//
// Design for gfx950: a wave-wide 16-byte load moves 1 KiB of K (or V); a
// token row of Hkv*d elements (2 KiB at 8 heads x 128 x bf16) is 128 lanes.
// A lane moves kStoreChunks such chunks of K and of V, 256 lanes apart, with
// all of its loads issued before its first store, so each lane keeps
// 2 * kStoreChunks * 16 bytes in flight; the rows are read before (not
// after) their slots are known, and a workgroup's row index is one scalar
// division.  When the rows or the pointers are
// not 16-byte aligned a lane copies single elements instead.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kStoreThreads = 256;
constexpr int kStoreChunks = 4;  // 16-byte chunks of K (and of V) per lane

// Chunk u of lane x in workgroup b is chunk (b * kStoreChunks + u) * 256 + x
// of the flat [num_tokens][chunks_per_row] view: every load and store
// instruction of a wave covers 1 KiB of consecutive bytes of a row.
__global__ __launch_bounds__(kStoreThreads) void store_kv_vec16(
    const char *__restrict__ k, int64_t k_stride_bytes, const char *__restrict__ v,
    int64_t v_stride_bytes, const int32_t *__restrict__ slot_mapping, int64_t num_chunks,
    int chunks_per_row, char *__restrict__ k_pool, char *__restrict__ v_pool, int64_t num_slots) {
    const int64_t row_bytes = (int64_t)chunks_per_row * 16;
    // the workgroup's first chunk as (row, chunk) once, in scalar registers;
    // each lane's chunks from there with 32-bit arithmetic
    const int64_t base = (int64_t)blockIdx.x * (kStoreChunks * kStoreThreads);
    const int64_t t_base = base / chunks_per_row;
    const uint32_t c_base = (uint32_t)(base - t_base * chunks_per_row);
    int64_t dst[kStoreChunks];
    uint4 kv[kStoreChunks], vv[kStoreChunks];
#pragma unroll
    for (int u = 0; u < kStoreChunks; ++u) {
        const int64_t i = base + u * kStoreThreads + threadIdx.x;
        dst[u] = -1;
        if (i >= num_chunks) continue;
        const uint32_t cu = c_base + u * kStoreThreads + threadIdx.x;  // < chunks_per_row + 1024
        const uint32_t dt = cu / (uint32_t)chunks_per_row;
        const int64_t t = t_base + dt;
        const int c = (int)(cu - dt * (uint32_t)chunks_per_row);
        // the rows are read whatever the slot holds, so their loads do not
        // wait for the slot's
        kv[u] = ld16(k + t * k_stride_bytes + c * 16);
        vv[u] = ld16(v + t * v_stride_bytes + c * 16);
        const int64_t slot = slot_mapping[t];
        if (slot >= 0 && slot < num_slots) dst[u] = slot * row_bytes + c * 16;  // -1: padding token
    }
#pragma unroll
    for (int u = 0; u < kStoreChunks; ++u) {
        if (dst[u] < 0) continue;
        *reinterpret_cast<uint4 *>(k_pool + dst[u]) = kv[u];
        *reinterpret_cast<uint4 *>(v_pool + dst[u]) = vv[u];
    }
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
    if (j < 0 || (j >> block_shift) >= bt_stride) return;  // cu_seqlens_k not covering this row
    const int64_t blk = block_table[(int64_t)lo * bt_stride + (j >> block_shift)];
    if (blk < 0 || blk >= num_blocks) return;
    const int64_t slot = (blk << block_shift) + (j & ((1 << block_shift) - 1));
    const int64_t row_bytes = (int64_t)chunks_per_row * 16;
    *reinterpret_cast<uint4 *>(k_out + row * row_bytes + c * 16) = ld16(k_pool + slot * row_bytes + c * 16);
    *reinterpret_cast<uint4 *>(v_out + row * row_bytes + c * 16) = ld16(v_pool + slot * row_bytes + c * 16);
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Quantizing store (LLM inference interview notes (nano-vllm fork), Q3 part
// 1: quantization happens on write, fused into the store).  For each token t
// with a valid slot and each KV head h, the head_dim values x of K (and of V)
// become int8 codes with one scale:
//   scale = max(max_i |x_i| / 127, 1e-8)              (fp32)
//   code_i = trunc(x_i / scale + (x_i / scale >= 0 ? 0.5 : -0.5))
// and the scale is stored as fp16 (round to nearest even).  The division is
// IEEE fp32 (the compiler's default for HIP), so the codes are exactly those
// of the same steps on a CPU.
//
// Mapping: a group of L lanes owns one head vector; each lane loads 16 bytes
// of it (E = 8 bf16 or 4 fp32 values), the group reduces max |x| with xor
// shuffles, then each lane writes its E codes and lane 0 the scale.  All lanes
// run the shuffles; only loads and stores are guarded.
template <typename SrcT, bool VEC>
__global__ __launch_bounds__(kStoreThreads) void store_kv_int8(
    const SrcT *__restrict__ k, int64_t k_stride, const SrcT *__restrict__ v, int64_t v_stride,
    const int32_t *__restrict__ slot_mapping, int64_t num_vectors, int hkv, int d, int lanes,
    int8_t *__restrict__ k_pool, int8_t *__restrict__ v_pool, _Float16 *__restrict__ k_scale,
    _Float16 *__restrict__ v_scale, int64_t num_slots) {
    constexpr int E = 16 / sizeof(SrcT);
    const int64_t gid = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x;
    const int64_t vec = gid / lanes;  // t * hkv + h
    const int li = (int)(gid - vec * lanes);
    const int64_t t = vec / hkv;
    const int h = (int)(vec - t * hkv);
    int64_t slot = -1;
    if (vec < num_vectors) slot = slot_mapping[t];
    const bool ok = slot >= 0 && slot < num_slots;

    auto quantize = [&](const SrcT *src, int8_t *dst_pool, _Float16 *dst_scale) {
        float x[E];
        if (ok) {
            const SrcT *p = src + h * d + li * E;
            if constexpr (VEC) {
                unpack16<SrcT>(ld16(p), x);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = to_float(p[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = 0.f;
        }
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
        for (int o = lanes >> 1; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float scale = fmaxf(amax / 127.0f, 1.0e-8f);
        uint32_t packed[E / 4];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float qf = x[e] / scale;
            const int code = (int)truncf(qf >= 0.f ? qf + 0.5f : qf - 0.5f);
            if (e % 4 == 0) packed[e / 4] = 0;
            packed[e / 4] |= ((uint32_t)code & 0xFFu) << (8 * (e % 4));
        }
        if (ok) {
            int8_t *q = dst_pool + (slot * hkv + h) * d + li * E;
            if constexpr (E == 8)
                *reinterpret_cast<uint2 *>(q) = make_uint2(packed[0], packed[1]);
            else
                *reinterpret_cast<uint32_t *>(q) = packed[0];
            if (li == 0) dst_scale[slot * hkv + h] = (_Float16)scale;
        }
    };
    quantize(k + t * k_stride, k_pool, k_scale);
    quantize(v + t * v_stride, v_pool, v_scale);
}

// Copy-on-write of shared, mutable last blocks (vLLM/SGLang interview labs,
// section 4, the follow-up on a native block-table fork: the child gets a new
// block holding a copy of the valid KV; full immutable blocks are never
// copied).  For pair i, slots 0 .. n-1 (n = num_valid[i]) of block src[i] go
// to block dst[i].  In the [num_blocks][block_size][...] layout they are one
// contiguous run of n * slot_bytes bytes, so a pair is a contiguous copy:
// workgroup (pair, part) moves the 16-byte chunks part*kCopyPer*256 + i*256 +
// thread (coalesced); a tail shorter than 16 bytes (scale pools) moves in
// 2-byte pieces.  VEC = false (blocks not 16-byte aligned): 2-byte pieces only.
// Pairs with ids outside the pool or n outside [1, block_size] are skipped.
constexpr int kCopyPer = 4;  // 16-byte chunks per thread per workgroup
template <bool VEC>
__global__ __launch_bounds__(kStoreThreads) void copy_blocks_kernel(
    char *__restrict__ pool, int64_t block_bytes, int64_t slot_bytes, int64_t num_blocks, int block_size,
    const int32_t *__restrict__ src, const int32_t *__restrict__ dst, const int32_t *__restrict__ num_valid,
    int parts) {
    const int pair = blockIdx.x / parts, part = blockIdx.x % parts;
    const int64_t sb = src[pair], db = dst[pair];
    const int n = num_valid[pair];
    if (sb < 0 || sb >= num_blocks || db < 0 || db >= num_blocks || n <= 0 || n > block_size) return;
    const int64_t bytes = (int64_t)n * slot_bytes;
    const char *from = pool + sb * block_bytes;
    char *to = pool + db * block_bytes;
    if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < kCopyPer; ++i) {
            const int64_t off = ((int64_t)(part * kCopyPer + i) * kStoreThreads + threadIdx.x) * 16;
            if (off + 16 <= bytes) {
                *reinterpret_cast<uint4 *>(to + off) = ld16(from + off);
            } else if (off < bytes) {
                for (int64_t b = off; b < bytes; b += 2)
                    *reinterpret_cast<uint16_t *>(to + b) = *reinterpret_cast<const uint16_t *>(from + b);
            }
        }
    } else {
        for (int64_t b = ((int64_t)part * kStoreThreads + threadIdx.x) * 2; b < bytes;
             b += (int64_t)parts * kStoreThreads * 2)
            *reinterpret_cast<uint16_t *>(to + b) = *reinterpret_cast<const uint16_t *>(from + b);
    }
}

}  // namespace

hipError_t launch_copy_blocks(void *pool, int64_t slot_bytes, const PoolGeom &g, const int32_t *src_blocks,
                              const int32_t *dst_blocks, const int32_t *num_valid, int num_pairs,
                              hipStream_t stream) {
    if (num_pairs == 0 || !pool) return hipSuccess;
    const int64_t block_bytes = slot_bytes * g.block_size;
    const bool vec = block_bytes % 16 == 0 && aligned16(pool);
    if (vec) {
        const int64_t chunks = (block_bytes + 15) / 16;
        const int parts = (int)((chunks + kStoreThreads * kCopyPer - 1) / (kStoreThreads * kCopyPer));
        hipLaunchKernelGGL(copy_blocks_kernel<true>, dim3((unsigned)((int64_t)num_pairs * parts)), dim3(kStoreThreads),
                           0, stream, (char *)pool, block_bytes, slot_bytes, g.num_blocks, g.block_size, src_blocks,
                           dst_blocks, num_valid, parts);
    } else {
        const int64_t pieces = (block_bytes + 1) / 2;
        const int parts = (int)((pieces + kStoreThreads * kCopyPer - 1) / (kStoreThreads * kCopyPer));
        hipLaunchKernelGGL(copy_blocks_kernel<false>, dim3((unsigned)((int64_t)num_pairs * parts)), dim3(kStoreThreads),
                           0, stream, (char *)pool, block_bytes, slot_bytes, g.num_blocks, g.block_size, src_blocks,
                           dst_blocks, num_valid, parts);
    }
    return hipGetLastError();
}

hipError_t launch_store_kv_int8(const void *k, int64_t k_row_stride, const void *v, int64_t v_row_stride,
                                int src_dtype, const int32_t *slot_mapping, int num_tokens, void *k_pool,
                                void *v_pool, void *k_scale, void *v_scale, const PoolGeom &g,
                                hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int eb = src_dtype == 0 ? 4 : 2;
    const int E = 16 / eb;
    const int lanes = g.d / E;  // a power of two, at most 64: head_dim is one from 8 to 256 (checked by the caller)
    const int64_t vectors = (int64_t)num_tokens * g.hkv;
    const int64_t threads = vectors * lanes;
    const unsigned grid = (unsigned)((threads + kStoreThreads - 1) / kStoreThreads);
    const int64_t num_slots = g.num_blocks << g.block_shift;
    const bool vec = (k_row_stride * eb) % 16 == 0 && (v_row_stride * eb) % 16 == 0 && aligned16(k) &&
                     aligned16(v);
    auto go = [&](auto src_tag, auto vec_tag) {
        using S = decltype(src_tag);
        constexpr bool V = decltype(vec_tag)::value;
        hipLaunchKernelGGL((store_kv_int8<S, V>), dim3(grid), dim3(kStoreThreads), 0, stream,
                           (const S *)k, k_row_stride, (const S *)v, v_row_stride, slot_mapping, vectors,
                           g.hkv, g.d, lanes, (int8_t *)k_pool, (int8_t *)v_pool, (_Float16 *)k_scale,
                           (_Float16 *)v_scale, num_slots);
    };
    if (src_dtype == 0) {
        if (vec) go(float{}, std::true_type{}); else go(float{}, std::false_type{});
    } else if (src_dtype == 3) {
        if (vec) go(f16_t{}, std::true_type{}); else go(f16_t{}, std::false_type{});
    } else {
        if (vec) go(bf16_t{}, std::true_type{}); else go(bf16_t{}, std::false_type{});
    }
    return hipGetLastError();
}

hipError_t launch_store_kv(const void *k, int64_t k_row_stride, const void *v, int64_t v_row_stride,
                           const int32_t *slot_mapping, int num_tokens, void *k_pool, void *v_pool,
                           const PoolGeom &g, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int eb = g.dtype == 0 ? 4 : 2;  // fp32, else bf16 / fp16
    const int row_elems = g.hkv * g.d;
    const int64_t row_bytes = (int64_t)row_elems * eb;
    const int64_t num_slots = g.num_blocks << g.block_shift;
    const bool vec = row_bytes % 16 == 0 && (k_row_stride * eb) % 16 == 0 &&
                     (v_row_stride * eb) % 16 == 0 && aligned16(k) && aligned16(v) &&
                     aligned16(k_pool) && aligned16(v_pool);
    if (vec) {
        const int cpr = (int)(row_bytes / 16);
        const int64_t n = (int64_t)num_tokens * cpr;
        const int64_t per_wg = (int64_t)kStoreThreads * kStoreChunks;
        const unsigned grid = (unsigned)((n + per_wg - 1) / per_wg);
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
    const int eb = g.dtype == 0 ? 4 : 2;  // fp32, else bf16 / fp16
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
