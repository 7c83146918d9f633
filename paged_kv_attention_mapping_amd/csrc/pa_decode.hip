// pa_decode.hip -- split-K ("flash-decoding") attention of single query rows
// over the paged KV cache, plus the log-sum-exp merge of the split partials.
//
// What it computes (nano-vllm deep dive, Step 4 path C, flash_attn_with_kvcache;
// Step 5 prepare_decode): for query row r of sequence s with context length
// ctx, and query head h of KV head g = h / G,
//     o = sum_j softmax_j(scale * q . k_j) v_j,   j = 0 .. ctx-1,
// with k_j, v_j found through block_table[s][j / block_size].
// Split-K (fork Q&A, general Q&A, "what is split-K"): the keys of a row are cut
// into segments; each segment keeps its own running max m, normaliser l and
// fp32 accumulator; a second kernel merges the segments by log-sum-exp.
//
// Layout on gfx950: one workgroup (8 waves for groups of up to 2 query heads,
// else 4; chosen by the planner) per (row, KV head g, split).  A token's K row
// for head g is head_dim contiguous elements; LPT lanes each load 16 bytes of
// it, so a wave covers 64/LPT tokens per load instruction (bf16, d=128: 16
// lanes x 16 B = 256 B per token, 4 tokens per wave).  The G query heads that
// share KV head g are all served from the same K/V bytes (GQA reuse, fork Q&A
// Q3 section 2), so every K/V byte is read from HBM once.  One pass: before
// scoring a round, a lane issues the next round's 16-byte loads (2 K and 2 V,
// into the second of two register buffers); the scores are summed across the
// LPT lanes with DPP row operations (bf16 q.k on v_dot2_f32_bf16), and a
// running max, normaliser and fp32 accumulator per lane group absorb the round
// (online softmax in the log2 domain).  The groups of a wave and then the
// waves are combined by log-sum-exp.  Block ids of a split are staged in LDS
// once.
//
// The same kernel also serves as the vector-ALU prefill path: a prefill row is
// one packed query token whose context is min(q_offset + i + 1, k_len) keys.
#include <limits.h>
#include <type_traits>
#include <math.h>

#include <atomic>
#include <mutex>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kNW = 4;        // waves per merge workgroup
constexpr int kThreads = kNW * kWave;
constexpr int kUnroll = 2;    // tokens per lane per round (K and V loads each)
constexpr int kSplitMax = 1 << 20;   // keys per split, upper bound
constexpr int kBlkIds = 4096;        // block ids a split may span (LDS staging)
// Fewest rounds a split covers at the planned key bound.  Shorter splits
// spread small batches over more workgroups but each then pays the fixed
// cost of a workgroup (block ids, queries, the cross-wave reduction, its
// partials and their merge) for little streaming: on MI355X, 16 rounds (1024
// keys at bf16, head_dim 128) measured fastest for one row of 20000 keys
// (51 -> 30 us), 32 rows of 1024 (32 -> 26 us) and 8 of 4096 (37 -> 32 us),
// against 1, 2, 4, 8, 32, 64 and 128, and left the large batches unchanged.
constexpr int kMinRoundsPerSplit = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kOrderThreads = 1024;

template <typename T, int D, int NW>
struct RowCfg {
    static constexpr int EPV = 16 / Elem<T>::bytes;  // elements per 16-byte vector
    static constexpr int LPT = D / EPV;              // lanes per token row
    static constexpr int TPW = kWave / LPT;          // tokens per wave per load
    static constexpr int TPR = NW * TPW * kUnroll;   // tokens per round
    static_assert(LPT >= 1 && LPT <= kWave && kWave % LPT == 0, "head_dim");
};

// Decode rows.  `order`, when given, is a permutation of the rows: the
// workgroups of row slot r (dispatched in index order) serve row order[r].
// With the longest-first order of decode_order_kernel the long rows start
// first and the short ones fill the end of the launch, instead of a long row
// streaming on alone at the end.  Results do not depend on the order.
struct DecodeRows {
    const int32_t *context_lens;
    const int32_t *order;
    int num_rows;
    // an entry of order outside [0, num_rows) (not a permutation: a broken
    // precondition) falls back to the slot itself, so no row is out of bounds
    __device__ __forceinline__ int row_of(int slot) const {
        if (!order) return slot;
        const int r = order[slot];
        return (unsigned)r < (unsigned)num_rows ? r : slot;
    }
    __device__ __forceinline__ void get(int r, int &seq, int &ctx) const {
        seq = r;
        ctx = context_lens[r];
    }
};

// order[rank] = row, for the rows ranked by decreasing context length with
// ties by row index (a strict total order, so every row gets its own rank).
// One workgroup; n <= kDecodeOrderMax.
__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(const int32_t *__restrict__ context_lens, int n,
                                                                     int32_t *__restrict__ order) {
    __shared__ __attribute__((aligned(16))) int s_len[kDecodeOrderMax];
    const int n4 = (n + 3) & ~3;
    for (int i = threadIdx.x; i < n4; i += kOrderThreads) s_len[i] = i < n ? context_lens[i] : INT_MIN;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kOrderThreads) {
        const int li = s_len[i];
        int rank = 0;
        for (int j = 0; j < n4; j += 4) {
            const int4 v = *reinterpret_cast<const int4 *>(s_len + j);
            // padding (INT_MIN at index >= n > i) never ranks ahead of row i
            rank += (v.x > li) | ((v.x == li) & (j < i));
            rank += (v.y > li) | ((v.y == li) & (j + 1 < i));
            rank += (v.z > li) | ((v.z == li) & (j + 2 < i));
            rank += (v.w > li) | ((v.w == li) & (j + 3 < i));
        }
        order[rank] = i;
    }
}

struct PrefillRows {
    const int32_t *cu_q;
    const int32_t *cu_k;
    const int32_t *q_off;
    int num_seqs;
    __device__ __forceinline__ int row_of(int slot) const { return slot; }
    __device__ __forceinline__ void get(int r, int &seq, int &ctx) const {
        int lo = 0, hi = num_seqs;  // cu_q[lo] <= r < cu_q[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu_q[mid] <= r) lo = mid; else hi = mid;
        }
        seq = lo;
        const int i = r - cu_q[lo];
        const int k_len = cu_k[lo + 1] - cu_k[lo];
        ctx = min(q_off[lo] + i + 1, k_len);
    }
};

struct RowArgs {
    const void *q;
    int64_t q_row_stride;      // elements
    const void *k_pool;
    const void *v_pool;
    int64_t num_blocks;
    int block_shift;
    int hkv;
    const int32_t *block_table;
    int bt_stride;
    int num_rows;
    int num_splits;            // split slots per row
    int round_tokens;          // splits are whole rounds of this many keys
    int split_cap;             // keys per split, upper bound
    float scale_log2;          // softmax_scale * log2(e)
    void *out;
    float *ws_acc;             // [rows][hq][splits][D]
    float *ws_m;               // [rows][hq][splits]
    float *ws_l;
    const _Float16 *k_scale;   // INT8 pools only: [slots][hkv] fp16 scales
    const _Float16 *v_scale;
    int kv_shift;              // INT8 only: hkv counts 2^kv_shift virtual heads per pool head
};

// Keys per split of a row with ctx keys: the row cut into at most
// num_splits pieces of whole rounds, none longer than split_cap.  The split
// kernel and the merge both derive a row's split length and count from its
// own key count this way, so the split count follows each row on the device.
// ctx must be at most num_splits * split_cap (the callers clamp it).
__device__ __forceinline__ int split_tokens_of(int ctx, int num_splits, int round_tokens, int split_cap) {
    const int per = (int)(((int64_t)ctx + num_splits - 1) / num_splits);
    const int st = (per + round_tokens - 1) / round_tokens * round_tokens;
    return min(max(st, round_tokens), split_cap);
}

// Index of the (slot, KV head) row that offset `off` of physical block `blk`
// holds for KV head `head` in a [num_blocks][block_size][hkv][...] pool: one
// 32 x 32 -> 64-bit multiply-add (the pool checks keep blk_rows = hkv *
// block_size below 2^31 and hkv at most 65536, so off * hkv fits 24-bit
// operands).  A masked token (blk < 0) maps to row `head` of slot 0: every
// such load hits one cached line.
__device__ __forceinline__ uint64_t kv_row_index(int blk, int off, uint32_t blk_rows, int hkv, int head) {
    const bool ok = blk >= 0;
    const uint32_t r = (ok ? __umul24((uint32_t)off, (uint32_t)hkv) : 0u) + (uint32_t)head;
    return (uint64_t)(ok ? (uint32_t)blk : 0u) * blk_rows + r;
}

// This lane's slice of one query head, kept in the form the dot product wants:
// bf16 and fp16 stay packed (two elements per 32-bit word, consumed by
// v_dot2_f32_bf16 / v_dot2_f32_f16); fp32 is kept as floats.
template <typename T> struct QSlice;
template <> struct QSlice<bf16_t> {
    uint4 w;
    __device__ __forceinline__ void load(const bf16_t *p) { w = ld16(p); }
    __device__ __forceinline__ float dot(const uint4 &k) const {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        float acc = 0.f;
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, k.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, k.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, k.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, k.w), acc, false);
        return acc;
    }
};
template <> struct QSlice<f16_t> {   // fp16: v_dot2_f32_f16 on the packed pairs
    uint4 w;
    __device__ __forceinline__ void load(const f16_t *p) { w = ld16(p); }
    __device__ __forceinline__ float dot(const uint4 &k) const {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        float acc = 0.f;
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.x), __builtin_bit_cast(f16x2, k.x), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.y), __builtin_bit_cast(f16x2, k.y), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.z), __builtin_bit_cast(f16x2, k.z), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w.w), __builtin_bit_cast(f16x2, k.w), acc, false);
        return acc;
    }
};
template <> struct QSlice<float> {
    float f[4];
    __device__ __forceinline__ void load(const float *p) { unpack16<float>(ld16(p), f); }
    __device__ __forceinline__ float dot(const uint4 &k) const {
        float kf[4];
        unpack16<float>(k, kf);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(f[e], kf[e], acc);
        return acc;
    }
};

// One pass over the split's keys with an online softmax kept per lane group:
// every round each lane issues kUnroll K loads and kUnroll V loads at once,
// scores them (DPP sum over the LPT lanes of a token), rescales its running
// (m, l, acc) once per round and accumulates p * v.  At the end the token
// groups of a wave and then the waves are combined by log-sum-exp.
template <typename T, int D, int G, int NW, class Rows>
__global__ __launch_bounds__(NW * kWave) void row_attn_split(RowArgs a, Rows rows) {
    using C = RowCfg<T, D, NW>;
    constexpr int EPV = C::EPV, LPT = C::LPT, TPW = C::TPW, TPR = C::TPR;
    constexpr int kNW = NW, kThreads = NW * kWave;
    __shared__ int s_blk[kBlkIds];           // physical block ids of this split
    __shared__ float s_acc[NW][G][D];
    __shared__ float s_m[NW][G], s_l[NW][G];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), w = tid >> 6;
    const int tg = lane / LPT, c = lane % LPT;
    const int hkv = a.hkv, hq = hkv * G;

    const int64_t wg = blockIdx.x;
    const int g = (int)(wg % hkv);
    const int64_t rest = wg / hkv;
    const int split = (int)(rest % a.num_splits);
    const int row = rows.row_of((int)(rest / a.num_splits));
    int seq, ctx;
    rows.get(row, seq, ctx);
    // Never index past the table row or past the splits the launch covers.
    ctx = (int)min((int64_t)ctx, min((int64_t)a.bt_stride << a.block_shift,
                                     (int64_t)a.num_splits * a.split_cap));
    const int st = split_tokens_of(ctx, a.num_splits, a.round_tokens, a.split_cap);

    T *out_row = reinterpret_cast<T *>(a.out) + ((int64_t)row * hq + (int64_t)g * G) * D;
    if ((int64_t)split * st >= ctx) {
        if (split == 0)  // no visible key: defined as a zero output
            for (int i = tid; i < G * D; i += kThreads) store_elem<T>(out_row + i, 0.f);
        return;
    }
    const int t0 = split * st;
    const int t1 = min(t0 + st, ctx);
    const int nsplit_row = (ctx + st - 1) / st;
    const int shift = a.block_shift;
    const int bmask = (1 << shift) - 1;
    const int b0 = t0 >> shift;

    {   // stage the block ids this split needs; ids outside the pool are masked
        const int32_t *bt = a.block_table + (int64_t)seq * a.bt_stride;
        const int nb = ((t1 - 1) >> shift) - b0 + 1;
        for (int i = tid; i < nb; i += kThreads) {
            const int p = bt[b0 + i];
            s_blk[i] = (p >= 0 && (int64_t)p < a.num_blocks) ? p : -1;
        }
    }
    QSlice<T> qv[G];
    {
        const T *qrow = reinterpret_cast<const T *>(a.q) + (int64_t)row * a.q_row_stride + (int64_t)g * G * D;
#pragma unroll
        for (int j = 0; j < G; ++j) qv[j].load(qrow + j * D + c * EPV);
    }
    __syncthreads();

    const T *kp = reinterpret_cast<const T *>(a.k_pool);
    const T *vp = reinterpret_cast<const T *>(a.v_pool);
    const uint32_t blk_rows = (uint32_t)hkv << a.block_shift;

    float m[G], l[G], acc[G][EPV];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[j][e] = 0.f;
    }

    // Software pipeline over rounds of TPR tokens: the loads of round r+1 are
    // issued before round r is scored, from two register buffers.  Tokens past
    // t1 (and ids outside the pool) are masked; their loads all hit slot 0 of
    // the pool, one cached line, so the trailing prefetch costs no HBM traffic.
    auto issue = [&](uint4 (&kr)[kUnroll], uint4 (&vr)[kUnroll], int (&blk)[kUnroll], int base) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tok = base + (u * kNW + w) * TPW + tg;
            blk[u] = tok < t1 ? s_blk[(tok >> shift) - b0] : -1;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tok = base + (u * kNW + w) * TPW + tg;
            const uint64_t e = kv_row_index(blk[u], tok & bmask, blk_rows, hkv, g) * D + c * EPV;
            kr[u] = ld16_stream(kp + e);
            vr[u] = ld16_stream(vp + e);
        }
    };
    auto consume = [&](const uint4 (&kr)[kUnroll], const uint4 (&vr)[kUnroll], const int (&blk)[kUnroll]) {
        float sc[kUnroll][G];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float dot = group_sum<LPT>(qv[j].dot(kr[u]));
                sc[u][j] = blk[u] >= 0 ? dot * a.scale_log2 : -INFINITY;
            }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = m[j];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, sc[u][j]);
            const float m_use = (mx == -INFINITY) ? 0.f : mx;
            const float alpha = __builtin_amdgcn_exp2f(m[j] - m_use);
            m[j] = mx;
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                sc[u][j] = __builtin_amdgcn_exp2f(sc[u][j] - m_use);
                ps += sc[u][j];
            }
            l[j] = l[j] * alpha + ps;
            // rescale only if the max moved for some lane of the wave (after the
            // first rounds it seldom does; a skipped rescale is by alpha = 1)
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f))
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[j][e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float vf[EPV];
            unpack16<T>(blk[u] >= 0 ? vr[u] : make_uint4(0, 0, 0, 0), vf);
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[j][e] = fmaf(sc[u][j], vf[e], acc[j][e]);
        }
    };
    {
        uint4 kA[kUnroll], vA[kUnroll], kB[kUnroll], vB[kUnroll];
        int bA[kUnroll], bB[kUnroll];
        issue(kA, vA, bA, t0);
        for (int base = t0; base < t1; base += 2 * TPR) {
            issue(kB, vB, bB, base + TPR);
            consume(kA, vA, bA);
            if (base + TPR >= t1) break;
            issue(kA, vA, bA, base + 2 * TPR);
            consume(kB, vB, bB);
        }
    }

    // ---- combine the token groups of the wave (lanes sharing c) -----------
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float M = m[j];
#pragma unroll
        for (int sft = LPT; sft < kWave; sft <<= 1) M = fmaxf(M, __shfl_xor(M, sft));
        const float f = (m[j] == -INFINITY) ? 0.f : exp2f(m[j] - M);
        l[j] = cross_group_sum<LPT>(l[j] * f);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[j][e] = cross_group_sum<LPT>(acc[j][e] * f);
        m[j] = M;
    }
    if (tg == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) s_acc[w][j][c * EPV + e] = acc[j][e];
            if (c == 0) {
                s_m[w][j] = m[j];
                s_l[w][j] = l[j];
            }
        }
    }
    __syncthreads();
    // ---- combine the waves, then write the output or the split's partials --
    for (int i = tid; i < G * D; i += kThreads) {
        const int j = i / D, d = i - j * D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, s_m[ww][j]);
        float A = 0.f, L = 0.f;
#pragma unroll
        for (int ww = 0; ww < kNW; ++ww) {
            const float f = (s_m[ww][j] == -INFINITY) ? 0.f : exp2f(s_m[ww][j] - M);
            A += s_acc[ww][j][d] * f;
            L += s_l[ww][j] * f;
        }
        if (nsplit_row == 1) {
            store_elem<T>(out_row + i, L > 0.f ? A / L : 0.f);
        } else {
            const int64_t idx = ((int64_t)row * hq + g * G + j) * a.num_splits + split;
            a.ws_acc[idx * D + d] = A;
            if (d == 0) {
                a.ws_m[idx] = M;
                a.ws_l[idx] = L;
            }
        }
    }
}

// INT8 pools (LLM inference interview notes (nano-vllm fork), Q3 part 2:
// dequantization fused into the decode kernel, no float copy of the cache).
// The same pass as row_attn_split over int8 codes with one fp16 scale per
// (token, KV head): a lane loads 16 codes of K and 16 of V (LPT = D/16 lanes
// per token) and the token's two scales.  Following the algebra the pages
// suggest, the K scale multiplies the finished dot product instead of every
// element, and the V scale is folded into the probability p (l keeps the
// unscaled p):
//     s_t = k_scale_t * sum_i q_i k_code_ti,   acc += (p_t * v_scale_t) * v_code_t.
// Codes are used in their offset form u = code + 128 (one XOR per 4 codes).
// K, with bf16 or fp16 queries: a byte permute turns two codes into the fp16
// pair (1024 + u0, 1024 + u1), exact integers, and v_dot2_f32_f16 takes them
// against the queries in fp16 (exact for bf16 values inside fp16's range);
// the dot is sum q (1152 + code) - 1152 sum q.  fp32 queries use fp32
// products of the widened u.  V, with bf16 or fp16 queries: the lane's two
// tokens of a round meet in v_dot2_f32_f16, the folded p of both rounded to
// an fp16 pair, against each element's two codes as the fp16 pair (1024 +
// u_t0, 1024 + u_t1) (one byte permute and one XOR): half the instructions of
// widening the codes and accumulating in fp32.  The accumulator then holds
// sum p' (1152 + code) and subtracts 1152 * sum p' over the same rounded p'.
// fp32 queries keep fp32 products of the widened u and subtract 128 * sum p.
//
// Workgroup order: the virtual heads of one (row, split) are dealt to
// workgroups 8 apart, which the dispatcher places on one XCD (workgroups go
// round-robin over the 8 XCDs): a token's scales, one 16-byte run for all its
// KV heads, are then fetched from HBM once, into that XCD's L2, rather than
// once per head.  The grid is padded to whole groups of 8 (row, split) units.
template <typename TQ, int D, int G, int NW, class Rows>
__global__ __launch_bounds__(NW * kWave) void row_attn_int8(RowArgs a, Rows rows) {
    constexpr int EPV = 16, LPT = D / EPV, TPW = kWave / LPT, TPR = NW * TPW * kUnroll;
    constexpr int kT = NW * kWave;
    static_assert(LPT >= 1 && LPT <= kWave && kWave % LPT == 0, "head_dim");
    __shared__ int s_blk[kBlkIds];
    __shared__ float s_acc[NW][G][D];
    __shared__ float s_m[NW][G], s_l[NW][G];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), w = tid >> 6;
    const int tg = lane / LPT, c = lane % LPT;
    // g indexes the G query heads this workgroup serves (a "virtual" KV head);
    // gp = g >> kv_shift is the pool's KV head they read (groups of 8 run as
    // two virtual heads of 4 query heads each, which keeps the per-lane
    // state within the 4-wave register budget)
    const int hkv = a.hkv, hq = hkv * G;
    const int hkv_p = hkv >> a.kv_shift;

    const int64_t r8 = (int64_t)blockIdx.x >> 3;
    const int g = (int)(r8 % hkv);
    const int gp = g >> a.kv_shift;
    const int64_t rest = (blockIdx.x & 7) + 8 * (r8 / hkv);
    if (rest >= (int64_t)a.num_rows * a.num_splits) return;  // grid padding
    const int split = (int)(rest % a.num_splits);
    const int row = rows.row_of((int)(rest / a.num_splits));
    int seq, ctx;
    rows.get(row, seq, ctx);
    ctx = (int)min((int64_t)ctx, min((int64_t)a.bt_stride << a.block_shift,
                                     (int64_t)a.num_splits * a.split_cap));
    const int st = split_tokens_of(ctx, a.num_splits, a.round_tokens, a.split_cap);

    TQ *out_row = reinterpret_cast<TQ *>(a.out) + ((int64_t)row * hq + (int64_t)g * G) * D;
    if ((int64_t)split * st >= ctx) {
        if (split == 0)
            for (int i = tid; i < G * D; i += kT) store_elem<TQ>(out_row + i, 0.f);
        return;
    }
    const int t0 = split * st;
    const int t1 = min(t0 + st, ctx);
    const int nsplit_row = (ctx + st - 1) / st;
    const int shift = a.block_shift;
    const int bmask = (1 << shift) - 1;
    const int b0 = t0 >> shift;
    {
        const int32_t *bt = a.block_table + (int64_t)seq * a.bt_stride;
        const int nb = ((t1 - 1) >> shift) - b0 + 1;
        for (int i = tid; i < nb; i += kT) {
            const int p = bt[b0 + i];
            s_blk[i] = (p >= 0 && (int64_t)p < a.num_blocks) ? p : -1;
        }
    }
    // this lane's 16 elements of each query head, as fp32, and their sum
    // (bf16 and fp16 queries: as fp16 pairs for v_dot2_f32_f16, summed as fp16
    // values; exact for fp16 queries)
    constexpr bool kF16Dot = std::is_same<TQ, bf16_t>::value || std::is_same<TQ, f16_t>::value;
    // fp16 V pairs: the folded p carry a factor 64, removed at the end (exact):
    // p <= 1 and a scale <= 65504/127 keep p * scale * 64 below 33030, inside
    // fp16, while small scales stay clear of fp16's subnormals 64 times longer
    constexpr float kVsFold = kF16Dot ? 64.f : 1.f;
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    float qv[G][EPV], qsum[G];
    half2_t qh[G][EPV / 2];
    {
        const TQ *qrow = reinterpret_cast<const TQ *>(a.q) + (int64_t)row * a.q_row_stride + (int64_t)g * G * D;
        constexpr int QE = 16 / Elem<TQ>::bytes;
#pragma unroll
        for (int j = 0; j < G; ++j) {
#pragma unroll
            for (int h = 0; h < EPV / QE; ++h) unpack16<TQ>(ld16(qrow + j * D + c * EPV + h * QE), &qv[j][h * QE]);
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                if constexpr (kF16Dot) qv[j][e] = (float)(_Float16)qv[j][e];
                sq += qv[j][e];
            }
            qsum[j] = sq;
            if constexpr (kF16Dot) {
#pragma unroll
                for (int e = 0; e < EPV; e += 2) qh[j][e / 2] = (half2_t){(_Float16)qv[j][e], (_Float16)qv[j][e + 1]};
            }
        }
    }
    __syncthreads();

    const int8_t *kp = reinterpret_cast<const int8_t *>(a.k_pool);
    const int8_t *vp = reinterpret_cast<const int8_t *>(a.v_pool);
    const uint32_t blk_rows = (uint32_t)hkv_p << a.block_shift;

    // ps: sum of the folded p (fp32 V path); vsum: sum of the same p rounded
    // to fp16 (fp16 V pairs)
    float m[G], l[G], ps[G], vsum[G], acc[G][EPV];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
        ps[j] = 0.f;
        vsum[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[j][e] = 0.f;
    }

    // u_e = code_e + 128 as fp32 (byte e of the 16 after flipping each sign bit)
    auto widen = [](const uint4 &x, float (&u)[EPV]) {
        const uint32_t wd[4] = {x.x ^ 0x80808080u, x.y ^ 0x80808080u, x.z ^ 0x80808080u, x.w ^ 0x80808080u};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) u[4 * i + b] = (float)((wd[i] >> (8 * b)) & 0xffu);
    };
    auto issue = [&](uint4 (&kr)[kUnroll], uint4 (&vr)[kUnroll], float (&ks)[kUnroll], float (&vs)[kUnroll],
                     int (&blk)[kUnroll], int base) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tok = base + (u * NW + w) * TPW + tg;
            blk[u] = tok < t1 ? s_blk[(tok >> shift) - b0] : -1;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tok = base + (u * NW + w) * TPW + tg;
            const uint64_t ri = kv_row_index(blk[u], tok & bmask, blk_rows, hkv_p, gp);
            kr[u] = ld16_stream(kp + ri * D + c * EPV);
            vr[u] = ld16_stream(vp + ri * D + c * EPV);
            ks[u] = (float)a.k_scale[ri] * a.scale_log2;  // K scale and softmax scale, once per token
            vs[u] = (float)a.v_scale[ri] * kVsFold;
        }
    };
    auto consume = [&](const uint4 (&kr)[kUnroll], const uint4 (&vr)[kUnroll], const float (&ks)[kUnroll],
                       const float (&vs)[kUnroll], const int (&blk)[kUnroll]) {
        float sc[kUnroll][G];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if constexpr (kF16Dot) {
                // code pairs as fp16 (1024 + code + 128): one byte permute per pair
                const uint32_t wd[4] = {kr[u].x ^ 0x80808080u, kr[u].y ^ 0x80808080u, kr[u].z ^ 0x80808080u,
                                        kr[u].w ^ 0x80808080u};
                half2_t kp2[EPV / 2];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kp2[2 * i] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, wd[i], 0x05010400u));
                    kp2[2 * i + 1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, wd[i], 0x05030402u));
                }
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    float d0 = 0.f;
#pragma unroll
                    for (int i = 0; i < EPV / 2; ++i) d0 = __builtin_amdgcn_fdot2(qh[j][i], kp2[i], d0, false);
                    const float dot = group_sum<LPT>(fmaf(-1152.f, qsum[j], d0));
                    sc[u][j] = blk[u] >= 0 ? dot * ks[u] : -INFINITY;
                }
            } else {
                float ku[EPV];
                widen(kr[u], ku);
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    float d0 = 0.f;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) d0 = fmaf(qv[j][e], ku[e], d0);
                    const float dot = group_sum<LPT>(fmaf(-128.f, qsum[j], d0));
                    sc[u][j] = blk[u] >= 0 ? dot * ks[u] : -INFINITY;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = m[j];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, sc[u][j]);
            const float m_use = (mx == -INFINITY) ? 0.f : mx;
            const float alpha = __builtin_amdgcn_exp2f(m[j] - m_use);
            m[j] = mx;
            float pl = 0.f, pv = 0.f;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float p = __builtin_amdgcn_exp2f(sc[u][j] - m_use);
                pl += p;
                sc[u][j] = blk[u] >= 0 ? p * vs[u] : 0.f;  // V scale folded into p
                pv += sc[u][j];
            }
            l[j] = l[j] * alpha + pl;
            ps[j] = ps[j] * alpha + pv;
            vsum[j] *= alpha;
            // rescale only if the max moved for some lane of the wave (after the
            // first rounds it seldom does; a skipped rescale is by alpha = 1)
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f))
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[j][e] *= alpha;
        }
        if constexpr (kF16Dot) {
            static_assert(kUnroll % 2 == 0, "tokens of a round pair up");
#pragma unroll
            for (int u = 0; u < kUnroll; u += 2) {
                half2_t pp[G];
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const _Float16 p0 = (_Float16)sc[u][j], p1 = (_Float16)sc[u + 1][j];
                    pp[j] = (half2_t){p0, p1};
                    vsum[j] = __builtin_amdgcn_fdot2(pp[j], (half2_t){(_Float16)1.f, (_Float16)1.f}, vsum[j], false);
                }
                const uint32_t c0[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
                const uint32_t c1[4] = {vr[u + 1].x, vr[u + 1].y, vr[u + 1].z, vr[u + 1].w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // byte b of each token's word i into the low bytes of the two
                        // halves (zeros above), then sign flip and fp16 exponent at once
                        const uint32_t pair = __builtin_amdgcn_perm(c1[i], c0[i], 0x0c040c00u + 0x00010001u * b);
                        const half2_t vv = __builtin_bit_cast(half2_t, pair ^ 0x64806480u);
#pragma unroll
                        for (int j = 0; j < G; ++j)
                            acc[j][4 * i + b] = __builtin_amdgcn_fdot2(pp[j], vv, acc[j][4 * i + b], false);
                    }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float vu[EPV];
                widen(vr[u], vu);
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc[j][e] = fmaf(sc[u][j], vu[e], acc[j][e]);
            }
        }
    };
    {
        uint4 kA[kUnroll], vA[kUnroll], kB[kUnroll], vB[kUnroll];
        float ksA[kUnroll], vsA[kUnroll], ksB[kUnroll], vsB[kUnroll];
        int bA[kUnroll], bB[kUnroll];
        issue(kA, vA, ksA, vsA, bA, t0);
        for (int base = t0; base < t1; base += 2 * TPR) {
            issue(kB, vB, ksB, vsB, bB, base + TPR);
            consume(kA, vA, ksA, vsA, bA);
            if (base + TPR >= t1) break;
            issue(kA, vA, ksA, vsA, bA, base + 2 * TPR);
            consume(kB, vB, ksB, vsB, bB);
        }
    }
    // codes were offset by 1152 (fp16 pairs) or 128 (fp32): remove that times
    // the sum of the folded p from every element
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            if constexpr (kF16Dot) acc[j][e] = fmaf(-1152.f, vsum[j], acc[j][e]) * (1.f / kVsFold);
            else acc[j][e] = fmaf(-128.f, ps[j], acc[j][e]);
        }

    // ---- combine the token groups of the wave, then the waves (as row_attn_split)
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float M = m[j];
#pragma unroll
        for (int sft = LPT; sft < kWave; sft <<= 1) M = fmaxf(M, __shfl_xor(M, sft));
        const float f = (m[j] == -INFINITY) ? 0.f : exp2f(m[j] - M);
        l[j] = cross_group_sum<LPT>(l[j] * f);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[j][e] = cross_group_sum<LPT>(acc[j][e] * f);
        m[j] = M;
    }
    if (tg == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) s_acc[w][j][c * EPV + e] = acc[j][e];
            if (c == 0) {
                s_m[w][j] = m[j];
                s_l[w][j] = l[j];
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kT) {
        const int j = i / D, d = i - j * D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, s_m[ww][j]);
        float A = 0.f, L = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float f = (s_m[ww][j] == -INFINITY) ? 0.f : exp2f(s_m[ww][j] - M);
            A += s_acc[ww][j][d] * f;
            L += s_l[ww][j] * f;
        }
        if (nsplit_row == 1) {
            store_elem<TQ>(out_row + i, L > 0.f ? A / L : 0.f);
        } else {
            const int64_t idx = ((int64_t)row * hq + g * G + j) * a.num_splits + split;
            a.ws_acc[idx * D + d] = A;
            if (d == 0) {
                a.ws_m[idx] = M;
                a.ws_l[idx] = L;
            }
        }
    }
}

struct MergeArgs {
    int num_rows;
    int hq;
    int num_splits;
    int round_tokens;
    int split_cap;
    int bt_stride;
    int block_shift;
    const float *ws_acc;
    const float *ws_m;
    const float *ws_l;
    void *out;
};

// One wave per (row, query head): out = sum_c acc_c 2^(m_c - m*) / sum_c l_c 2^(m_c - m*).
// Lane s holds split s's (m, l); the split weights are reduced across the wave
// and broadcast with shuffles, so the whole merge is one round trip to memory.
template <typename T, int D, class Rows>
__global__ __launch_bounds__(kThreads) void row_attn_merge(MergeArgs a, Rows rows) {
    constexpr int DPL = (D + kWave - 1) / kWave;  // output elements per lane
    const int64_t wave = (int64_t)blockIdx.x * kNW + (threadIdx.x >> 6);
    const int lane = threadIdx.x & (kWave - 1);
    if (wave >= (int64_t)a.num_rows * a.hq) return;
    const int row = (int)(wave / a.hq), h = (int)(wave % a.hq);
    int seq, ctx;
    rows.get(row, seq, ctx);
    ctx = (int)min((int64_t)ctx, min((int64_t)a.bt_stride << a.block_shift,
                                     (int64_t)a.num_splits * a.split_cap));
    const int st = split_tokens_of(ctx, a.num_splits, a.round_tokens, a.split_cap);
    const int ns = (ctx + st - 1) / st;
    if (ns <= 1) return;  // written directly by the split kernel
    const int64_t base = ((int64_t)row * a.hq + h) * a.num_splits;
    T *o = reinterpret_cast<T *>(a.out) + ((int64_t)row * a.hq + h) * D;
    float A[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) A[k] = 0.f;
    float L = 0.f;
    // splits in chunks of 64 (one per lane); the running max rescales earlier chunks
    float M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += kWave) {
        const int sl = s0 + lane;
        const float ms = sl < ns ? a.ws_m[base + sl] : -INFINITY;
        const float ls = sl < ns ? a.ws_l[base + sl] : 0.f;
        const float cm = group_max<kWave>(ms);
        const float Mn = fmaxf(M, cm);
        if (Mn == -INFINITY) continue;
        const float r = M == -INFINITY ? 0.f : exp2f(M - Mn);
        const float wl = ms == -INFINITY ? 0.f : exp2f(ms - Mn);
        L = L * r + group_sum<kWave>(ls * wl);
#pragma unroll
        for (int k = 0; k < DPL; ++k) A[k] *= r;
        const int cnt = min(kWave, ns - s0);
        for (int s = 0; s < cnt; ++s) {
            const float ws = __shfl(wl, s);
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
                const int d = lane + k * kWave;
                if (d < D) A[k] = fmaf(a.ws_acc[(base + s0 + s) * D + d], ws, A[k]);
            }
        }
        M = Mn;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        const int d = lane + k * kWave;
        if (d < D) store_elem<T>(o + d, L > 0.f ? A[k] / L : 0.f);
    }
}

int tokens_per_round(int dtype, int d, int nw) {
    const int epv = dtype == 0 ? 4 : (dtype == 2 ? 16 : 8);  // fp32, int8, else 16-bit
    const int lpt = d / epv;
    return nw * (kWave / lpt) * kUnroll;
}

template <typename T, int D, int G, int NW, class Rows, bool I8 = false>
hipError_t run_rows(const RowArgs &a, const Rows &rows, hipStream_t stream) {
    int64_t wgs = (int64_t)a.num_rows * a.num_splits * a.hkv;
    if (wgs == 0) return hipSuccess;
    if constexpr (I8) wgs = ((int64_t)a.num_rows * a.num_splits + 7) / 8 * 8 * a.hkv;  // whole groups of 8 units
    if constexpr (I8)
        hipLaunchKernelGGL((row_attn_int8<T, D, G, NW, Rows>), dim3((unsigned)wgs), dim3(NW * kWave), 0,
                           stream, a, rows);
    else
        hipLaunchKernelGGL((row_attn_split<T, D, G, NW, Rows>), dim3((unsigned)wgs), dim3(NW * kWave), 0,
                           stream, a, rows);
    if (a.num_splits > 1) {
        MergeArgs m{a.num_rows, a.hkv * G, a.num_splits, a.round_tokens, a.split_cap, a.bt_stride, a.block_shift,
                    a.ws_acc, a.ws_m, a.ws_l, a.out};
        const int64_t waves = (int64_t)a.num_rows * a.hkv * G;
        hipLaunchKernelGGL((row_attn_merge<T, D, Rows>), dim3((unsigned)((waves + kNW - 1) / kNW)),
                           dim3(kThreads), 0, stream, m, rows);
    }
    return hipGetLastError();
}

template <typename T, int D, int G, class Rows, bool I8 = false>
hipError_t dispatch_waves(int waves, const RowArgs &a, const Rows &rows, hipStream_t s) {
    if constexpr (G <= 2) {  // wider workgroups only where the registers allow them
        if (waves == 16) return run_rows<T, D, G, 16, Rows, I8>(a, rows, s);
        if (waves == 8) return run_rows<T, D, G, 8, Rows, I8>(a, rows, s);
    }
    if (waves == 4) return run_rows<T, D, G, 4, Rows, I8>(a, rows, s);
    return hipErrorInvalidValue;
}

template <typename T, int D, class Rows, bool I8 = false>
hipError_t dispatch_group(int group, int waves, const RowArgs &a, const Rows &rows, hipStream_t s) {
    switch (group) {
        case 1: return dispatch_waves<T, D, 1, Rows, I8>(waves, a, rows, s);
        case 2: return dispatch_waves<T, D, 2, Rows, I8>(waves, a, rows, s);
        case 4: return dispatch_waves<T, D, 4, Rows, I8>(waves, a, rows, s);
        case 8:
            if constexpr (!I8) return dispatch_waves<T, D, 8, Rows, I8>(waves, a, rows, s);
            break;
    }
    return hipErrorInvalidValue;
}

template <typename T, class Rows, bool I8 = false>
hipError_t dispatch_dim(int d, int group, int waves, const RowArgs &a, const Rows &rows, hipStream_t s) {
    switch (d) {
        case 32: return dispatch_group<T, 32, Rows, I8>(group, waves, a, rows, s);
        case 64: return dispatch_group<T, 64, Rows, I8>(group, waves, a, rows, s);
        case 128: return dispatch_group<T, 128, Rows, I8>(group, waves, a, rows, s);
        case 256: return dispatch_group<T, 256, Rows, I8>(group, waves, a, rows, s);
    }
    return hipErrorInvalidValue;
}

template <class Rows>
hipError_t dispatch(const PoolGeom &g, int group, int waves, const RowArgs &a, const Rows &rows,
                    hipStream_t s) {
    if (g.dtype == 0) return dispatch_dim<float>(g.d, group, waves, a, rows, s);
    if (g.dtype == 3) return dispatch_dim<f16_t>(g.d, group, waves, a, rows, s);
    return dispatch_dim<bf16_t>(g.d, group, waves, a, rows, s);
}

RowArgs make_args(const void *q, int64_t q_row_stride, int hq, const void *k_pool, const void *v_pool,
                  const PoolGeom &g, const int32_t *block_table, int bt_stride,
                  const RowAttnPlan &plan, float softmax_scale, void *out, void *workspace) {
    RowArgs a{};
    a.q = q;
    a.q_row_stride = q_row_stride;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.num_blocks = g.num_blocks;
    a.block_shift = g.block_shift;
    a.hkv = g.hkv;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.num_rows = plan.num_rows;
    a.num_splits = plan.num_splits;
    a.round_tokens = plan.round_tokens;
    a.split_cap = plan.split_cap;
    a.scale_log2 = softmax_scale * kLog2e;
    a.out = out;
    if (plan.num_splits > 1) {
        const int64_t n = (int64_t)plan.num_rows * hq * plan.num_splits;
        float *ws = reinterpret_cast<float *>(workspace);
        a.ws_acc = ws;
        a.ws_m = ws + n * g.d;
        a.ws_l = a.ws_m + n;
    }
    return a;
}

}  // namespace

RowAttnPlan plan_row_attention(int num_rows, const PoolGeom &g, int group, int max_keys) {
    // Waves per workgroup: 8 when the per-lane state of the G heads stays
    // within 128 registers (G <= 2; two 512-thread workgroups per CU), else 4.
    // Wider workgroups stream one (row, KV head) faster, which shortens the
    // tail when context lengths are ragged; two per CU keep one streaming
    // while the other starts up or reduces.
    // INT8 pools: 4 waves.  The int8 kernel (about 122 registers) also fits 8
    // waves, but measured slower on MI355X there: the 256-sequence decode
    // 125-128 against 112-114 us, the 8 x 512 batch unchanged.
    const int waves = (group <= 2 && g.dtype != 2) ? 8 : 4;
    const int tpr = tokens_per_round(g.dtype, g.d, waves);
    // A split's keys may start anywhere in a block, so it spans at most
    // ceil(keys / block_size) + 1 blocks: keep that within the kBlkIds block
    // ids a workgroup stages in LDS.  Whole rounds (tpr is a power of two).
    const int64_t cap = min((int64_t)kSplitMax, (int64_t)(kBlkIds - 1) << g.block_shift) & ~(int64_t)(tpr - 1);
    RowAttnPlan p{num_rows, 1, tpr, (int)cap, waves};
    if (num_rows <= 0 || max_keys <= 0) return p;
    // Split slots per row: enough (row, KV head, split) workgroups for two
    // waves of resident workgroups, but at least kMinRoundsPerSplit rounds of
    // keys per split at max_keys, and no split longer than cap.
    const int64_t slots = 256LL * 16 / waves;        // resident workgroups on 256 CUs
    const int64_t target_wgs = 2 * slots;
    const int64_t units = (int64_t)num_rows * g.hkv;
    int64_t ns = (target_wgs + units - 1) / units;
    ns = min(ns, ((int64_t)max_keys + kMinRoundsPerSplit * tpr - 1) / (kMinRoundsPerSplit * tpr));
    ns = max(ns, ((int64_t)max_keys + cap - 1) / cap);
    p.num_splits = (int)max(ns, (int64_t)1);
    return p;
}

size_t row_attention_workspace_bytes(const RowAttnPlan &p, int hq, int d) {
    if (p.num_splits <= 1) return 0;
    const size_t n = (size_t)p.num_rows * hq * p.num_splits;
    return n * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_decode(const void *q, int64_t q_row_stride, int hq, const void *k_pool,
                         const void *v_pool, const PoolGeom &g, const int32_t *context_lens,
                         const int32_t *block_table, int bt_stride, const RowAttnPlan &plan,
                         float softmax_scale, const int32_t *row_order, void *out, void *workspace,
                         hipStream_t stream) {
    const RowArgs a = make_args(q, q_row_stride, hq, k_pool, v_pool, g, block_table, bt_stride, plan,
                                softmax_scale, out, workspace);
    return dispatch(g, hq / g.hkv, plan.waves, a, DecodeRows{context_lens, row_order, plan.num_rows}, stream);
}

hipError_t launch_decode_int8(const void *q, int64_t q_row_stride, int hq, int q_dtype, const void *k_pool,
                              const void *v_pool, const void *k_scale, const void *v_scale, const PoolGeom &g,
                              const int32_t *context_lens, const int32_t *block_table, int bt_stride,
                              const RowAttnPlan &plan, float softmax_scale, const int32_t *row_order, void *out,
                              void *workspace, hipStream_t stream) {
    RowArgs a = make_args(q, q_row_stride, hq, k_pool, v_pool, g, block_table, bt_stride, plan, softmax_scale,
                          out, workspace);
    a.k_scale = reinterpret_cast<const _Float16 *>(k_scale);
    a.v_scale = reinterpret_cast<const _Float16 *>(v_scale);
    const DecodeRows rows{context_lens, row_order, plan.num_rows};
    int group = hq / g.hkv;
    if (group == 8) {  // two virtual KV heads of 4 query heads each per pool head
        a.hkv = g.hkv * 2;
        a.kv_shift = 1;
        group = 4;
    }
    if (q_dtype == 0) return dispatch_dim<float, DecodeRows, true>(g.d, group, plan.waves, a, rows, stream);
    if (q_dtype == 3) return dispatch_dim<f16_t, DecodeRows, true>(g.d, group, plan.waves, a, rows, stream);
    return dispatch_dim<bf16_t, DecodeRows, true>(g.d, group, plan.waves, a, rows, stream);
}

// pa_decode_static's scratch: the split partials of a decode call live in
// this file-scope device array instead of a caller workspace.  In host code
// `scratch` names a host-side stand-in, so kernels get the device address
// that hipGetSymbolAddress returns, looked up once per device with that
// device current and kept per device (each GPU holds its own copy).
namespace {
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_decode_order(const int32_t *context_lens, int num_rows, int32_t *row_order,
                               hipStream_t stream) {
    hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, context_lens, num_rows,
                       row_order);
    return hipGetLastError();
}

hipError_t launch_prefill_rows(const void *q, int64_t q_row_stride, int hq, const void *k_pool,
                               const void *v_pool, const PoolGeom &g, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, const int32_t *q_offsets,
                               const int32_t *block_table, int bt_stride, int num_seqs,
                               const RowAttnPlan &plan, float softmax_scale, void *out,
                               void *workspace, hipStream_t stream) {
    const RowArgs a = make_args(q, q_row_stride, hq, k_pool, v_pool, g, block_table, bt_stride, plan,
                                softmax_scale, out, workspace);
    return dispatch(g, hq / g.hkv, plan.waves, a,
                    PrefillRows{cu_seqlens_q, cu_seqlens_k, q_offsets, num_seqs}, stream);
}

// Prefill over INT8 pools, one packed query token per row (the decode pass
// above with the INT8 dequantization fused in; no float copy of the cache).
hipError_t launch_prefill_rows_int8(const void *q, int64_t q_row_stride, int hq, int q_dtype, const void *k_pool,
                                    const void *v_pool, const void *k_scale, const void *v_scale,
                                    const PoolGeom &g, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                    const int32_t *q_offsets, const int32_t *block_table, int bt_stride,
                                    int num_seqs, const RowAttnPlan &plan, float softmax_scale, void *out,
                                    void *workspace, hipStream_t stream) {
    RowArgs a = make_args(q, q_row_stride, hq, k_pool, v_pool, g, block_table, bt_stride, plan, softmax_scale,
                          out, workspace);
    a.k_scale = reinterpret_cast<const _Float16 *>(k_scale);
    a.v_scale = reinterpret_cast<const _Float16 *>(v_scale);
    const PrefillRows rows{cu_seqlens_q, cu_seqlens_k, q_offsets, num_seqs};
    int group = hq / g.hkv;
    if (group == 8) {  // two virtual KV heads of 4 query heads each per pool head
        a.hkv = g.hkv * 2;
        a.kv_shift = 1;
        group = 4;
    }
    if (q_dtype == 0) return dispatch_dim<float, PrefillRows, true>(g.d, group, plan.waves, a, rows, stream);
    if (q_dtype == 3) return dispatch_dim<f16_t, PrefillRows, true>(g.d, group, plan.waves, a, rows, stream);
    return dispatch_dim<bf16_t, PrefillRows, true>(g.d, group, plan.waves, a, rows, stream);
}

}  // namespace pa
