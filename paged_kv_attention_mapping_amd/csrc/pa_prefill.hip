// pa_prefill.hip -- query-tiled flash-attention prefill over the paged KV
// cache on bf16 MFMA (gfx950), for head_dim 64 and 128.
//
// What it computes (nano-vllm deep dive, Step 4 path A/B, flash_attn_varlen_func
// with cu_seqlens and block_table, causal): query i of sequence s sits at
// absolute position q_offsets[s] + i and attends to keys 0 .. min(q_off + i,
// k_len - 1), read through block_table[s][key / block_size].
// How (vLLM/SGLang interview labs, section 2, "the main gains of
// FlashAttention"): score tiles live in registers only, tiles are merged by an
// online softmax, key tiles wholly above the causal diagonal are skipped and
// masks are applied only on boundary tiles, and the products run on the
// matrix cores.  The fork's kernel was one query per program with no matrix
// dots (fork Q&A, Q1 section 4, and the follow-up on query tiling); this
// kernel tiles the query dimension, so tiles that straddle the diagonal need
// in-tile masks.
//
// Mapping on gfx950 (wave64, v_mfma_f32_32x32x16_bf16):
//  * a wave owns 32 query positions of ONE query head; a workgroup of four
//    waves owns NH query heads that share one KV head (GQA) times 4/NH
//    position sub-tiles, so one K/V tile in LDS serves all of them.
//  * scores are computed transposed, S^T = K . Q^T (A = K rows from LDS,
//    B = the wave's Q held in registers all along), so each lane owns one
//    query's column: row max / sum need one exchange between the two lane
//    halves only.
//  * K rows are fed to the MFMA in an order that swaps bits 2 and 3 of the
//    row index inside each 32-row block.  With the 32x32 accumulator layout
//    (lane half h, register r -> row 8*(r/4) + 4h + r%4) this puts the scores
//    of keys 16s + 8h + (0..7) in registers 8s..8s+7 of lane half h, which is
//    exactly the B operand layout of O^T = V^T . P^T: P never leaves registers.
//  * V is written to LDS transposed (V^T[d][key]) so the A operand of the PV
//    product is one 16-byte LDS read per lane.
//  * a workgroup processes a PAIR of query tiles of one sequence, tile p and
//    tile T-1-p, so every workgroup of a sequence does the same causal work.
//  * the KV head index varies fastest across workgroups; with 8 KV heads and
//    workgroups dealt round-robin to the 8 XCDs, all tiles of one KV head run
//    on one XCD and re-read its K/V from that XCD's L2.
//  * K/V tiles are double-buffered in LDS: the global loads of tile j+1 are in
//    flight while tile j is computed.  Block ids are staged in LDS per window.
//  * rows past k_len are zero-filled, so masked probabilities (0) never meet
//    uninitialised pool contents (0 * NaN).
#include <math.h>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfThreads = 256;
constexpr int kBN = 64;       // keys per tile
constexpr int kBlkWin = 1024;  // block ids staged in LDS at a time
constexpr float kLog2eF = 1.4426950408889634f;

template <int D, int NH>
struct Pf {
    static constexpr int SUB = 4 / NH;                     // position sub-tiles per workgroup
    static constexpr int BM = 32 * SUB;                    // positions per workgroup tile
    static constexpr int KS = D / 16;                      // MFMA k-steps over head_dim
    static constexpr int DT = D / 32;                      // 32-wide output tiles over head_dim
    static constexpr int KLD = D + 8;                      // LDS row stride (elements), K tile
    static constexpr int VLD = kBN + 8;                    // LDS row stride (elements), V^T tile
    static constexpr int CPR = D / 8;                      // 16-byte chunks per K row
    static constexpr int KCH = kBN * CPR / kPfThreads;     // K chunks per thread
    static constexpr int VIT = (D / 4) * (kBN / 4);        // 4 keys x 4 dims items per V tile
    static constexpr int VPT = (VIT + kPfThreads - 1) / kPfThreads;
    static_assert(KCH >= 1 && kBN * CPR % kPfThreads == 0, "K tile split");
};

struct PfArgs {
    const uint16_t *q;
    int64_t q_row_stride;   // elements
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    int64_t num_blocks;
    int block_shift;
    int hkv;
    int group;              // query heads per KV head
    int head_groups;        // group / NH
    const int32_t *block_table;
    int bt_stride;
    const int32_t *cu_q;
    const int32_t *cu_k;
    const int32_t *q_off;
    int pairs_per_seq;
    float scale_log2;
    uint16_t *out;
};

__device__ __forceinline__ int swap_bits_2_3(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

template <int D, int NH>
struct Tile {
    using C = Pf<D, NH>;
    uint4 kreg[C::KCH];
    uint2 vreg[C::VPT][4];
};

template <int D, int NH>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_mfma_kernel(PfArgs a) {
    using C = Pf<D, NH>;
    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kBN * C::KLD];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[2][D * C::VLD];
    __shared__ int s_blk[kBlkWin];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hf = lane >> 5;

    int64_t wg = blockIdx.x;
    const int g = (int)(wg % a.hkv);
    wg /= a.hkv;
    const int hgrp = (int)(wg % a.head_groups);
    wg /= a.head_groups;
    const int pair = (int)(wg % a.pairs_per_seq);
    const int s = (int)(wg / a.pairs_per_seq);

    const int q_start = a.cu_q[s];
    const int q_len = a.cu_q[s + 1] - q_start;
    const int k_len = a.cu_k[s + 1] - a.cu_k[s];
    const int q_off = a.q_off[s];
    const int T = (q_len + C::BM - 1) / C::BM;
    if (pair >= (T + 1) / 2) return;

    const int hh = w % NH, sub = w / NH;
    const int h = g * a.group + hgrp * NH + hh;
    const int hq = a.hkv * a.group;
    const int shift = a.block_shift;
    const int bmask = (1 << shift) - 1;
    const int32_t *bt = a.block_table + (int64_t)s * a.bt_stride;
    // keys that may be indexed: within k_len and within the table row
    const int kcap = (int)min((int64_t)k_len, (int64_t)a.bt_stride << shift);
    const float c = a.scale_log2;
    const int64_t kv_row = (int64_t)a.hkv * D;      // elements per pool slot
    const int64_t kv_head = (int64_t)g * D;

    for (int it = 0; it < 2; ++it) {
        const int tile = it == 0 ? T - 1 - pair : pair;
        if (it == 1 && tile == T - 1 - pair) break;

        const int i_wg0 = tile * C::BM;
        const int i_wg_last = min(i_wg0 + C::BM, q_len) - 1;
        const int kmax_wg = min(q_off + i_wg_last, kcap - 1);
        const int i0 = i_wg0 + sub * 32;
        const bool wave_active = i0 < q_len;
        const int kmax_w = wave_active ? min(q_off + min(i0 + 31, q_len - 1), kcap - 1) : -1;
        const int kfull_w = min(q_off + i0, kcap - 1);  // keys <= this: visible to all rows of the wave
        const int i_me = i0 + n;
        const bool row_ok = i_me < q_len;
        const int lim_me = min(q_off + i_me, kcap - 1);
        uint16_t *orow = a.out + ((int64_t)(q_start + i_me) * hq + h) * D;

        if (kmax_wg < 0) {  // no keys at all (k_len == 0): zero output
            if (row_ok && hf == 0)
                for (int d = 0; d < D; ++d) orow[d] = 0;
            continue;
        }
        const int ntiles = kmax_wg / kBN + 1;
        const int last_blk = kmax_wg >> shift;

        // the wave's queries, B operand layout: lane (n, hf), k-step ks holds d = 16ks + 8hf .. +7
        bf16x8 qf[C::KS];
        {
            const uint16_t *qrow = a.q + (int64_t)(q_start + i_me) * a.q_row_stride + (int64_t)h * D;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                uint4 v = row_ok ? ld16(qrow + 16 * ks + 8 * hf) : make_uint4(0, 0, 0, 0);
                qf[ks] = __builtin_bit_cast(bf16x8, v);
            }
        }
        f32x16 o[C::DT];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
        float m = -INFINITY, l = 0.f;

        // block-id window staging (every thread reads ids only after a barrier)
        int win0 = 0;
        auto stage_ids = [&](int first_blk) {
            win0 = first_blk;
            const int cnt = min(kBlkWin, last_blk - first_blk + 1);
            for (int i = tid; i < cnt; i += kPfThreads) {
                const int p = bt[first_blk + i];
                s_blk[i] = (p >= 0 && (int64_t)p < a.num_blocks) ? p : -1;
            }
        };
        // keys past kmax_wg are masked for every row and their blocks are not staged
        auto blk_of = [&](int key) -> int {
            return key <= kmax_wg ? s_blk[(key >> shift) - win0] : -1;
        };

        Tile<D, NH> reg;
        auto load_tile = [&](int kt) {
            const int kb = kt * kBN;
#pragma unroll
            for (int ci = 0; ci < C::KCH; ++ci) {
                const int qi = tid + kPfThreads * ci;
                const int key = kb + qi / C::CPR, ch = qi % C::CPR;
                const int p = blk_of(key);
                reg.kreg[ci] = p >= 0 ? ld16(a.k_pool + (((int64_t)p << shift) + (key & bmask)) * kv_row +
                                                 kv_head + ch * 8)
                                      : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int vi = 0; vi < C::VPT; ++vi) {
                const int item = tid + kPfThreads * vi;
                const int dg = item % (D / 4), kg = item / (D / 4);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int key = kb + 4 * kg + kk;
                    const int p = (item < C::VIT) ? blk_of(key) : -1;
                    reg.vreg[vi][kk] =
                        p >= 0 ? *reinterpret_cast<const uint2 *>(
                                     a.v_pool + (((int64_t)p << shift) + (key & bmask)) * kv_row + kv_head + 4 * dg)
                               : make_uint2(0, 0);
                }
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int ci = 0; ci < C::KCH; ++ci) {
                const int qi = tid + kPfThreads * ci;
                const int key = qi / C::CPR, ch = qi % C::CPR;
                *reinterpret_cast<uint4 *>(&s_k[buf][key * C::KLD + ch * 8]) = reg.kreg[ci];
            }
#pragma unroll
            for (int vi = 0; vi < C::VPT; ++vi) {
                const int item = tid + kPfThreads * vi;
                if (item < C::VIT) {
                    const int dg = item % (D / 4), kg = item / (D / 4);
                    const uint2 *x = reg.vreg[vi];
                    // 4 keys x 4 dims -> for each dim, 4 consecutive keys (8 bytes)
                    const uint2 d0 = make_uint2((x[0].x & 0xffffu) | (x[1].x << 16),
                                                (x[2].x & 0xffffu) | (x[3].x << 16));
                    const uint2 d1 = make_uint2((x[0].x >> 16) | (x[1].x & 0xffff0000u),
                                                (x[2].x >> 16) | (x[3].x & 0xffff0000u));
                    const uint2 d2 = make_uint2((x[0].y & 0xffffu) | (x[1].y << 16),
                                                (x[2].y & 0xffffu) | (x[3].y << 16));
                    const uint2 d3 = make_uint2((x[0].y >> 16) | (x[1].y & 0xffff0000u),
                                                (x[2].y >> 16) | (x[3].y & 0xffff0000u));
                    uint16_t *base = &s_v[buf][(4 * dg) * C::VLD + 4 * kg];
                    *reinterpret_cast<uint2 *>(base) = d0;
                    *reinterpret_cast<uint2 *>(base + C::VLD) = d1;
                    *reinterpret_cast<uint2 *>(base + 2 * C::VLD) = d2;
                    *reinterpret_cast<uint2 *>(base + 3 * C::VLD) = d3;
                }
            }
        };

        stage_ids(0);
        __syncthreads();
        load_tile(0);
        store_tile(0);
        __syncthreads();

        const int pn = swap_bits_2_3(n);
        for (int j = 0; j < ntiles; ++j) {
            const int buf = j & 1;
            if (j + 1 < ntiles) {
                const int kb1 = (j + 1) * kBN;
                if (((kb1 + kBN - 1) >> shift) >= win0 + kBlkWin) {  // leave the staged window
                    stage_ids(kb1 >> shift);
                    __syncthreads();
                }
                load_tile(j + 1);
            }
            const int kb = j * kBN;
            if (wave_active && kb <= kmax_w) {
                // ---- S^T = K . Q^T for the 64 keys of this tile (two 32-key blocks)
                f32x16 sacc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                            &s_k[buf][(32 * t + pn) * C::KLD + 16 * ks + 8 * hf]);
                        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sacc[t], 0, 0, 0);
                    }
                }
                // ---- mask (only tiles that cross the diagonal or the key end)
                // register r of block t holds key kb + 32t + 16(r/8) + 8hf + r%8
                if (kb + kBN - 1 > kfull_w) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kb + 32 * t + 16 * (r >> 3) + 8 * hf + (r & 7);
                            if (key > lim_me) sacc[t][r] = -INFINITY;
                        }
                }
                // ---- online softmax (log2 domain; scores scaled inside exp2)
                float mx = -INFINITY;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m, mx);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = exp2f((m - m_use) * c);
                const float mc = m_use * c;
                float rs = 0.f;
                bf16x8 pb[4];
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    uint32_t w4[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float p0 = exp2f(fmaf(sacc[st >> 1][8 * (st & 1) + 2 * jj], c, -mc));
                        const float p1 = exp2f(fmaf(sacc[st >> 1][8 * (st & 1) + 2 * jj + 1], c, -mc));
                        rs += p0 + p1;
                        w4[jj] = pack_bf16x2(p0, p1);
                    }
                    pb[st] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
                }
                l = l * alpha + rs;
                m = m_new;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                // ---- O^T += V^T . P^T
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const bf16x8 va = *reinterpret_cast<const bf16x8 *>(
                            &s_v[buf][(32 * dt + n) * C::VLD + 16 * st + 8 * hf]);
                        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[st], o[dt], 0, 0, 0);
                    }
                }
            }
            if (j + 1 < ntiles) store_tile(buf ^ 1);
            __syncthreads();
        }

        // ---- epilogue: O = O^T / l; lane (n, hf) holds d = 32dt + 8b + 4hf + a at register a + 4b
        const float l_tot = l + __shfl_xor(l, 32);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (row_ok) {
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint2 v = make_uint2(pack_bf16x2(o[dt][4 * b] * inv, o[dt][4 * b + 1] * inv),
                                               pack_bf16x2(o[dt][4 * b + 2] * inv, o[dt][4 * b + 3] * inv));
                    *reinterpret_cast<uint2 *>(orow + 32 * dt + 8 * b + 4 * hf) = v;
                }
        }
    }
}

template <int D, int NH>
hipError_t run(const PfArgs &a, int num_seqs, int max_seqlen_q, hipStream_t stream) {
    using C = Pf<D, NH>;
    PfArgs b = a;
    const int max_tiles = (max_seqlen_q + C::BM - 1) / C::BM;
    b.pairs_per_seq = (max_tiles + 1) / 2;
    b.head_groups = a.group / NH;
    const int64_t wgs = (int64_t)num_seqs * b.pairs_per_seq * b.head_groups * a.hkv;
    if (wgs == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_mfma_kernel<D, NH>), dim3((unsigned)wgs), dim3(kPfThreads), 0, stream, b);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_nh(const PfArgs &a, int num_seqs, int max_seqlen_q, hipStream_t stream) {
    switch (a.group) {
        case 1: return run<D, 1>(a, num_seqs, max_seqlen_q, stream);
        case 2: return run<D, 2>(a, num_seqs, max_seqlen_q, stream);
        case 4: return run<D, 4>(a, num_seqs, max_seqlen_q, stream);
        case 8: return run<D, 4>(a, num_seqs, max_seqlen_q, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool prefill_mfma_supported(const PoolGeom &g, int group) {
    return g.dtype == 1 && (g.d == 64 || g.d == 128) && g.block_size >= 4 &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill_mfma(const void *q, int64_t q_row_stride, int hq, const void *k_pool,
                               const void *v_pool, const PoolGeom &g, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, const int32_t *q_offsets,
                               const int32_t *block_table, int bt_stride, int num_seqs, int total_q,
                               int max_seqlen_q, float softmax_scale, void *out, hipStream_t stream) {
    (void)total_q;
    PfArgs a{};
    a.q = reinterpret_cast<const uint16_t *>(q);
    a.q_row_stride = q_row_stride;
    a.k_pool = reinterpret_cast<const uint16_t *>(k_pool);
    a.v_pool = reinterpret_cast<const uint16_t *>(v_pool);
    a.num_blocks = g.num_blocks;
    a.block_shift = g.block_shift;
    a.hkv = g.hkv;
    a.group = hq / g.hkv;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.q_off = q_offsets;
    a.scale_log2 = softmax_scale * kLog2eF;
    a.out = reinterpret_cast<uint16_t *>(out);
    if (max_seqlen_q <= 0) return hipSuccess;
    return g.d == 128 ? dispatch_nh<128>(a, num_seqs, max_seqlen_q, stream)
                      : dispatch_nh<64>(a, num_seqs, max_seqlen_q, stream);
}

}  // namespace pa
