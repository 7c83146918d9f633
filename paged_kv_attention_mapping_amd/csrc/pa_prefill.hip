// pa_prefill.hip -- query-tiled flash-attention prefill over the paged KV
// cache on bf16 or fp16 MFMA (gfx950), for head_dim 64, 128 and 256 (256 in
// the 4-wave layout only), and over INT8 pools at head_dim 64 and 128.
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
//  * a wave owns 32 query positions of ONE query head; four (head, position
//    sub-tile) slots cover NH query heads that share one KV head (GQA) times
//    4/NH sub-tiles, so one K/V tile in LDS serves all of them.
//  * two workgroup layouts.  8 waves, two per SIMD, one workgroup per CU:
//    each slot is held by two waves that split the keys.  A step stages 128
//    keys; the first key half takes keys 0..63 of it, the second keys
//    64..127.  At the end the second half hands its (O, m, l) to the first
//    through LDS, which merges them.  4 waves, one per SIMD: 64-key steps,
//    one wave per slot, half the LDS, so two workgroups share a CU and one's
//    prologue, barriers and epilogue overlap the other's matrix work.  The
//    host takes the 8-wave layout when the launch fits the CUs in one round
//    (long prompts) and the 4-wave one otherwise (many or short sequences).
//  * scores are computed transposed, S^T = K . Q^T (A = K rows from LDS,
//    B = the wave's Q held in registers all along), so each lane owns one
//    query's column: sums need one exchange between the two lane halves.
//  * K rows are fed to the MFMA in an order that swaps bits 2 and 3 of the
//    row index inside each 32-row block.  With the 32x32 accumulator layout
//    (lane half h, register r -> row 8*(r/4) + 4h + r%4) this puts the scores
//    of keys 16s + 8h + (0..7) in registers 8s..8s+7 of lane half h, which is
//    exactly the B operand layout of O^T = V^T . P^T: P never leaves registers.
//  * K and V rows go from HBM/L2 straight into LDS (16-byte direct loads, no
//    staging registers), row-major with a 16-byte XOR swizzle per row, so both
//    the K reads (ds_read_b128) and the V^T reads are free of bank conflicts.
//    Each wave loads 16 rows of a step; when they are 16 visible keys of one
//    valid block, a buffer resource over them (scalar registers) and fixed
//    per-lane offsets make the loads free of per-lane address arithmetic.
//  * the A operand of the PV product, V^T, is read with the gfx950 LDS
//    transpose load ds_read_b64_tr_b16: in each 16-lane group, lane i gets
//    element i%4 of the 8-byte chunks named by lanes 4r + i/4 (r = 0..3), so
//    if lane 4r+q names V[key_r][d0 + 4q] it receives V[key_0..3][d0 + i].
//  * softmax runs against a running reference max that moves only when a
//    block's probabilities would grow too large (see attend_tile), so the hot
//    path computes no per-tile max.
//  * a long prompt (one round of 8-wave workgroups) gives each workgroup a
//    PAIR of query tiles of one sequence, tile p and tile T-1-p, so every
//    workgroup of the sequence does the same causal work; other launches give
//    each workgroup one tile, longest tiles dispatched first (see
//    plan_prefill).
//  * the KV head index varies fastest across workgroups; with 8 KV heads and
//    workgroups dealt round-robin to the 8 XCDs, all tiles of one KV head run
//    on one XCD and re-read its K/V from that XCD's L2.
//  * steps are double-buffered in LDS: the direct loads of step j+1 are in
//    flight while step j is computed.  Block ids are staged in LDS per window.
//  * rows a tile holds past the last needed key are loaded from the sequence's
//    key 0 (finite data), so masked probabilities (exact zeros) never meet
//    uninitialised pool contents (0 * NaN).
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr int kBN = 64;                       // keys per wave tile
constexpr int kRowsPerWave = 16;              // step rows each wave loads (both layouts)
constexpr int kNumCUs = 256;                  // MI355X compute units
constexpr int kBlkWin = 1024;                 // block ids staged in LDS at a time

// Workgroup layouts.  NW = 8: two waves per SIMD, one workgroup per CU; each
// slot's two waves split every 128-key step into key halves and merge their
// partial results at the end of a tile.  NW = 4: one wave per SIMD, 64-key
// steps, no merge, and half the LDS, so two workgroups share a CU and their
// phases (prologues, barriers, epilogues) overlap each other's matrix work.
template <int D, int NH, typename E = bf16_t, int NW = 8>
struct Pf {
    using M = Mm<E>;
    static constexpr int WAVES = NW;
    static constexpr int THREADS = 64 * NW;
    static constexpr int KH = NW == 8 ? 2 : 1;         // key halves per step
    static constexpr int STEP = KH * kBN;              // keys per workgroup step
    static_assert((NW == 8 || NW == 4) && STEP / NW == kRowsPerWave, "layout");
    typedef typename M::x8 x8;
    typedef typename M::x4 x4;
    typedef typename M::x2 x2;
    static constexpr int SUB = 4 / NH;                 // position sub-tiles per workgroup
    static constexpr int BM = 32 * SUB;                // positions per workgroup tile
    static constexpr int KS = D / 16;                  // MFMA k-steps over head_dim
    static constexpr int DT = D / 32;                  // 32-wide output tiles over head_dim
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int ROWB = D * 2;                 // bytes per LDS row (bf16)
    static constexpr int TILEB = kBN * ROWB;           // bytes of one wave tile (K or V)
    static constexpr int STEPB = STEP * ROWB;          // bytes of one step (K or V)
    static constexpr int RPI = 64 / CPR;               // rows per wave-wide 16-byte load
    static constexpr int LPW = kRowsPerWave / RPI;     // 16-byte loads per lane per step (K or V)
    static constexpr int MERGE = DT * 16 + 2;          // floats per lane handed between key halves
    // INT8 pools: one bf16 step buffer, an int8 staging step (D bytes per row)
    // and the rows' scale words
    static constexpr int DIM = D;
    static constexpr int CPR8 = D / 16;                // 16-byte chunks per int8 row
    static constexpr int STAGEB = STEP * D;            // bytes of one int8 step (K or V)
    static constexpr int RPI8 = 64 / CPR8;             // int8 rows per wave-wide 16-byte load
    static constexpr int LPW8 = kRowsPerWave / RPI8;   // such loads per lane per step (K or V)
    static constexpr int CONV = STEP * CPR8 / THREADS;  // int8 chunks each thread converts (K or V)
    static constexpr int SCLB = STEP * 4;              // bytes of one step's scale words (K or V)
    // the INT8 staging: 2 * STEP / 64 waves fetch 64 scale words each
    static_assert(LPW8 * RPI8 == kRowsPerWave && CONV * THREADS == STEP * CPR8 && 2 * STEP / 64 <= NW,
                  "int8 row split");
    static_assert(NW != 8 || 4 * MERGE * 64 * 4 <= 2 * STEPB + 2 * STAGEB, "merge area fits in the INT8 layout");
    static_assert(LPW * RPI == kRowsPerWave && LPW >= 1, "row split");
    // V rows swizzle by 4r mod min(CPR, 16): the same for every wave-wide load
    // when 4*RPI is a multiple of that (d <= 128), else each load has its own
    // lane offset
    static constexpr int VOFFS = (4 * RPI) % (CPR < 16 ? CPR : 16) == 0 ? 1 : LPW;
    static_assert(D <= 128 || NW == 4, "head_dim 256: the 4-wave layout only (its LDS)");
    static_assert(NW != 8 || 4 * MERGE * 64 * 4 <= 4 * STEPB, "merge area fits in the K/V buffers");
};

// Direct HBM/L2 -> LDS loads of this wave's 16 rows of one step (keys
// kb_step + 16w .. +15) into the step buffers dk / dv.  Slot q of the wave's
// rows (16 bytes) is written by lane q%64 of its wave-instruction q/64 and
// holds chunk (slot ^ swizzle) of row q / CPR.
//  * fast path: when all 16 rows are visible keys of one valid block (block
//    size >= 16), a buffer resource over the 16 pool rows (wave-uniform, in
//    scalar registers) is read at per-lane 32-bit offsets (koff / voff: row
//    lane/CPR of each RPI-row group, swizzled chunk of slot lane%CPR) plus a
//    scalar offset of RPI rows per load;
//  * otherwise each lane resolves its own row: keys past kmax (masked for
//    every row; their blocks are not staged) and keys in blocks outside the
//    pool are read from key 0 of the sequence (blk0) instead, finite data
//    that the zero probabilities cancel;
//  * rows of a wave tile that no wave computes are not loaded.
template <class C>
__device__ __forceinline__ void load_wave_rows(const PfArgs &a, int kb_step, int kmax, int shift, int bmask,
                                               int win0, int blk0, int64_t kv_row, int64_t kv_head,
                                               const uint32_t (&koff)[C::LPW], const uint32_t (&voff)[C::VOFFS], int w,
                                               int lane, const int *s_blk, unsigned char *dk, unsigned char *dv) {
    if (kb_step + kBN * (C::KH == 2 ? w / (C::WAVES / 2) : 0) > kmax) return;
    const int row0 = __builtin_amdgcn_readfirstlane(kb_step + kRowsPerWave * w);
    if (shift >= 4 && row0 + kRowsPerWave - 1 <= kmax) {
        const int p = __builtin_amdgcn_readfirstlane(s_blk[(row0 >> shift) - win0]);
        if (p >= 0) {
            const int row_bytes = (int)(kv_row * 2);
            const int64_t sbase = ((((int64_t)p << shift) + (row0 & bmask)) * kv_row + kv_head) * 2;
            const i32x4 rk =
                raw_rsrc(reinterpret_cast<const unsigned char *>(a.k_pool) + sbase, kRowsPerWave * row_bytes);
            const i32x4 rv =
                raw_rsrc(reinterpret_cast<const unsigned char *>(a.v_pool) + sbase, kRowsPerWave * row_bytes);
            const uint32_t lk = __builtin_amdgcn_readfirstlane(lds_addr(dk) + w * C::LPW * 1024);
            const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_addr(dv) + w * C::LPW * 1024);
#pragma unroll
            for (int u = 0; u < C::LPW; ++u) {
                const int soff = __builtin_amdgcn_readfirstlane(u * C::RPI * row_bytes);
                buffer_lds16(rk, koff[u], soff, lk + u * 1024);
                buffer_lds16(rv, voff[C::VOFFS == 1 ? 0 : u], soff, lv + u * 1024);
            }
            return;
        }
    }
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
        const int blk_i = w * C::LPW + u;  // 1 KiB block of the step
        const int q = blk_i * 64 + lane;
        const int r = q / C::CPR, sl = q % C::CPR;
        const int key = kb_step + r;
        const int p = key <= kmax ? s_blk[(key >> shift) - win0] : -1;
        const int64_t slot = p >= 0 ? ((int64_t)p << shift) + (key & bmask)
                                    : (blk0 >= 0 ? ((int64_t)blk0 << shift) : 0);
        const int64_t eoff = slot * kv_row + kv_head;
        global_lds16(a.k_pool + eoff + k_slot<C::CPR>(r, sl) * 8,
                     __builtin_amdgcn_readfirstlane(lds_addr(dk) + blk_i * 1024));
        global_lds16(a.v_pool + eoff + v_slot<C::CPR>(r, sl) * 8,
                     __builtin_amdgcn_readfirstlane(lds_addr(dv) + blk_i * 1024));
    }
}

// INT8 pools (LLM inference interview notes (nano-vllm fork), Q3: K/V stored
// as int8 codes with one fp16 scale per (token, KV head)).  Direct loads of
// this wave's 16 code rows of one step into the int8 staging buffers dk / dv
// (row-major, D bytes a row), rows resolved as in load_wave_rows; and, from
// waves 0..3, one 4-byte scale word per step row (K for waves 0, 1, V for 2,
// 3): the word holding the fp16 scales of heads g & ~1 and g | 1 (hkv is
// even, so it is 4-byte aligned).
template <class C>
__device__ __forceinline__ void load_wave_rows_i8(const PfArgs &a, int kb_step, int kmax, int shift, int bmask,
                                                  int win0, int blk0, int g, int w, int lane, const int *s_blk,
                                                  unsigned char *dk, unsigned char *dv, unsigned char *dsk,
                                                  unsigned char *dsv) {
    const int64_t row_bytes = (int64_t)a.hkv * C::DIM;  // bytes of one pool slot
    const int64_t head = (int64_t)g * C::DIM;
    const unsigned char *kp = reinterpret_cast<const unsigned char *>(a.k_pool);
    const unsigned char *vp = reinterpret_cast<const unsigned char *>(a.v_pool);
    auto slot_of = [&](int key) -> int64_t {
        const int p = key <= kmax ? s_blk[(key >> shift) - win0] : -1;
        return p >= 0 ? ((int64_t)p << shift) + (key & bmask) : (blk0 >= 0 ? ((int64_t)blk0 << shift) : 0);
    };
    constexpr int SW = C::STEP / 64;  // waves fetching each of K's and V's scale words, 64 rows each
    if (w < 2 * SW) {
        const int r = (w % SW) * 64 + lane;
        const uint16_t *sp = w < SW ? a.k_scale : a.v_scale;
        global_lds4(sp + slot_of(kb_step + r) * a.hkv + (g & ~1),
                    __builtin_amdgcn_readfirstlane(lds_addr(w < SW ? dsk : dsv) + (w % SW) * 256));
    }
    if (kb_step + kBN * (C::KH == 2 ? w / (C::WAVES / 2) : 0) > kmax) return;
    const int row0 = __builtin_amdgcn_readfirstlane(kb_step + kRowsPerWave * w);
    if (shift >= 4 && row0 + kRowsPerWave - 1 <= kmax) {
        const int p = __builtin_amdgcn_readfirstlane(s_blk[(row0 >> shift) - win0]);
        if (p >= 0) {
            const int64_t sbase = (((int64_t)p << shift) + (row0 & bmask)) * row_bytes + head;
            const i32x4 rk = raw_rsrc(kp + sbase, (uint32_t)(kRowsPerWave * row_bytes));
            const i32x4 rv = raw_rsrc(vp + sbase, (uint32_t)(kRowsPerWave * row_bytes));
            const uint32_t off = (uint32_t)((lane / C::CPR8) * row_bytes + (lane % C::CPR8) * 16);
            const uint32_t lk = __builtin_amdgcn_readfirstlane(lds_addr(dk) + w * C::LPW8 * 1024);
            const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_addr(dv) + w * C::LPW8 * 1024);
#pragma unroll
            for (int u = 0; u < C::LPW8; ++u) {
                const int soff = __builtin_amdgcn_readfirstlane((int)(u * C::RPI8 * row_bytes));
                buffer_lds16(rk, off, soff, lk + u * 1024);
                buffer_lds16(rv, off, soff, lv + u * 1024);
            }
            return;
        }
    }
#pragma unroll
    for (int u = 0; u < C::LPW8; ++u) {
        const int blk_i = w * C::LPW8 + u;  // 1 KiB block of the staging step
        const int q = blk_i * 64 + lane;
        const int r = q / C::CPR8, c8 = q % C::CPR8;
        const int64_t eoff = slot_of(kb_step + r) * row_bytes + head + c8 * 16;
        global_lds16(kp + eoff, __builtin_amdgcn_readfirstlane(lds_addr(dk) + blk_i * 1024));
        global_lds16(vp + eoff, __builtin_amdgcn_readfirstlane(lds_addr(dv) + blk_i * 1024));
    }
}

// Dequantize one staged INT8 step into the 16-bit step buffer: code * scale,
// exact in fp32, rounded once to the element type (nearest even), written in
// the same swizzled layout the direct loads produce (K rows XOR r, V rows XOR
// 4r).  Codes are widened in their +128 offset form: (u - 128) s =
// fma(u, s, -128 s).  fp16: values saturate at +-65504 (127 times a scale
// rounded up can pass fp16's largest finite value by up to 0.05%).
template <class C>
__device__ __forceinline__ void convert_step_i8(const unsigned char *k8, const unsigned char *v8,
                                                const uint32_t *sk, const uint32_t *sv, int g, unsigned char *kt,
                                                unsigned char *vt, int tid) {
    constexpr bool kF16 = std::is_same<typename C::x8, Mm<f16_t>::x8>::value;
#pragma unroll
    for (int t = 0; t < C::CONV; ++t) {
        const int cid = tid + C::THREADS * t;
        const int r = cid / C::CPR8, c8 = cid % C::CPR8;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            const uint4 codes = *reinterpret_cast<const uint4 *>((kv ? v8 : k8) + r * C::DIM + c8 * 16);
            const uint32_t word = (kv ? sv : sk)[r];
            const uint16_t bits = (uint16_t)((g & 1) ? (word >> 16) : (word & 0xffffu));
            const float sc = (float)__builtin_bit_cast(_Float16, bits);
            const float nsc = -128.f * sc;
            const uint32_t wd[4] = {codes.x ^ 0x80808080u, codes.y ^ 0x80808080u, codes.z ^ 0x80808080u,
                                    codes.w ^ 0x80808080u};
            f32x8 lo, hi;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                lo[b] = fmaf((float)((wd[b / 4] >> (8 * (b % 4))) & 0xffu), sc, nsc);
                hi[b] = fmaf((float)((wd[2 + b / 4] >> (8 * (b % 4))) & 0xffu), sc, nsc);
                if constexpr (kF16) {
                    lo[b] = __builtin_amdgcn_fmed3f(lo[b], -65504.f, 65504.f);
                    hi[b] = __builtin_amdgcn_fmed3f(hi[b], -65504.f, 65504.f);
                }
            }
            const int c0 = 2 * c8;
            const int s0 = kv ? v_slot<C::CPR>(r, c0) : k_slot<C::CPR>(r, c0);
            const int s1 = kv ? v_slot<C::CPR>(r, c0 + 1) : k_slot<C::CPR>(r, c0 + 1);
            unsigned char *tile = kv ? vt : kt;
            *reinterpret_cast<typename C::x8 *>(tile + r * C::ROWB + s0 * 16) =
                __builtin_convertvector(lo, typename C::x8);
            *reinterpret_cast<typename C::x8 *>(tile + r * C::ROWB + s1 * 16) =
                __builtin_convertvector(hi, typename C::x8);
        }
    }
}

// Probabilities of one 32-key block of the tile (scores sacc), scaled by
// the running reference max m: P = exp2(s*c - m*c), rounded to bf16 once so
// that the PV product and the row sum (dot products with ones) see the same
// weights.  Returns this lane's sum over its 16 keys of the block.
template <class C>
__device__ __forceinline__ float block_probs(const f32x16 &sacc, float c, float mc, typename C::x8 &p_lo,
                                             typename C::x8 &p_hi) {
    const typename C::x2 ones = {1.f, 1.f};
    f32x8 lo, hi;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        lo[jj] = __builtin_amdgcn_exp2f(fmaf(sacc[jj], c, -mc));
        hi[jj] = __builtin_amdgcn_exp2f(fmaf(sacc[8 + jj], c, -mc));
    }
    p_lo = __builtin_convertvector(lo, typename C::x8);
    p_hi = __builtin_convertvector(hi, typename C::x8);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        s0 = C::M::dot2((typename C::x2){p_lo[k], p_lo[k + 1]}, ones, s0);
        s1 = C::M::dot2((typename C::x2){p_hi[k], p_hi[k + 1]}, ones, s1);
    }
    return s0 + s1;
}

// Cold path of one block: move the reference max to the block max (the same
// in both lane halves of each query column), rescale O and l, and
// exponentiate the block again.
template <class C>
__device__ __forceinline__ float rebase_block(const f32x16 &sacc, f32x16 (&o)[C::DT], float &m, float &l,
                                             float c, typename C::x8 &p_lo, typename C::x8 &p_hi) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    const float mc = (m == -INFINITY) ? 0.f : m * c;
    return block_probs<C>(sacc, c, mc, p_lo, p_hi);
}

// Sets the scores of keys hidden from the lane's position to -inf in block
// t: register r holds key kb + 32t + 16(r/8) + 8hf + r%8, hidden when
// 32t + 16(r/8) + r%8 > thr.  The empty asm keeps the guarded call a real
// branch (no selects on tiles that need no mask).
__device__ __forceinline__ void mask_block(f32x16 &sacc, int t, int thr) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (32 * t + 16 * (r >> 3) + (r & 7) > thr) sacc[r] = -INFINITY;
}

// One wave tile: 64 keys (rows of kt / vt in LDS) against the wave's 32
// query positions, in two 32-key blocks.  need_mask: the tile crosses the
// causal diagonal or the key end of some position (thr = last visible key -
// kb - 8hf).
//
// Online softmax without a max per tile: each block is exponentiated against
// the running reference max m (log2 domain, scores scaled inside exp2).
// Only if some lane's block sum exceeds kBlockSumMax (or no m is set yet)
// does the wave take the cold path (rebase_block).  O / l is exact
// whatever m is, since both use it.  The hot path has no branch between
// block 1's QK MFMAs and block 0's exponentials, nor between block 0's PV
// MFMAs and block 1's exponentials, so the two can be issued interleaved.
// V^T operand of the PV MFMA for 16-key group st and d block dt: two LDS
// transpose reads at the lane's base vofs[dt] plus an immediate offset (see
// the kernel for the lane mapping).
template <class C>
__device__ __forceinline__ typename C::x8 read_vt(const unsigned char *vbuf, const int (&vofs)[C::DT], int st, int dt) {
    i16x4 part[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
        part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(vbuf + vofs[dt] + (16 * st + 4 * x) * C::ROWB));
    return __builtin_bit_cast(typename C::x8, (i16x8){part[0][0], part[0][1], part[0][2], part[0][3], part[1][0],
                                             part[1][1], part[1][2], part[1][3]});
}

// Probabilities of scores 2i, 2i+1 of a block's 16 against the scaled
// reference max mc (one slice of block_probs).
__device__ __forceinline__ void probs_step(const f32x16 &sacc, float c, float mc, int i, f32x16 &pf) {
    pf[2 * i] = __builtin_amdgcn_exp2f(fmaf(sacc[2 * i], c, -mc));
    pf[2 * i + 1] = __builtin_amdgcn_exp2f(fmaf(sacc[2 * i + 1], c, -mc));
}

// 16-bit probabilities and the lane's sum of them (see block_probs).
template <class C>
__device__ __forceinline__ float probs_finish(const f32x16 &pf, typename C::x8 &p_lo, typename C::x8 &p_hi) {
    const typename C::x2 ones = {1.f, 1.f};
    p_lo = __builtin_convertvector(__builtin_shufflevector(pf, pf, 0, 1, 2, 3, 4, 5, 6, 7), typename C::x8);
    p_hi = __builtin_convertvector(__builtin_shufflevector(pf, pf, 8, 9, 10, 11, 12, 13, 14, 15), typename C::x8);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        s0 = C::M::dot2((typename C::x2){p_lo[k], p_lo[k + 1]}, ones, s0);
        s1 = C::M::dot2((typename C::x2){p_hi[k], p_hi[k + 1]}, ones, s1);
    }
    return s0 + s1;
}

// Running softmax state of one wave: reference max m (raw score units), mc =
// m * c (0 while m is -inf), O^T accumulators, row-sum l, and whether any
// block has set m yet (wave-uniform).
template <class C>
struct SoftState {
    f32x16 o[C::DT];
    float m, mc, l;
    bool m_set;
};

// One wave tile: 64 keys against the wave's 32 query positions, in two
// 32-key blocks.  kbuf / vbuf: bases of the step buffer (compile-time
// offsets); kofs / vofs: the lane's byte offsets of its K rows and V^T pieces
// from them (key half included).  need_mask: the tile crosses the causal diagonal
// or the key end of some position (thr = last visible key - kb - 8hf).
//
// Online softmax without a max per tile: each block is exponentiated against
// the running reference max (log2 domain, scores scaled inside exp2).  Only
// if some lane's block sum exceeds kBlockSumMax (or no max is set yet) does
// the wave take the cold path (rebase_block).  O / l is exact whatever the
// reference is, since both use it.  Issue order: block 0's QK MFMAs; block
// 1's QK MFMAs, then block 0's exponentials (the compiler's order here: the
// second wave of the SIMD fills the gap, and interleaving them one by one
// measured no faster); block 0's PV MFMAs, each followed by two of block 1's
// exponentials and the V^T reads of block 1; block 1's PV MFMAs
// (sched_barrier keeps the groups in that order).
template <class C>
__device__ __forceinline__ void attend_tile(const unsigned char *kbuf, const unsigned char *vbuf,
                                            const int (&kofs)[C::KS], const int (&vofs)[C::DT],
                                            const typename C::x8 (&qf)[C::KS], SoftState<C> &st_, bool need_mask, int thr,
                                            float c) {
    constexpr int NPV = 2 * C::DT;  // PV MFMAs per block
    const f32x16 zero = {};
    f32x16 sacc[2];
    typename C::x8 ka[2][C::KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            ka[t][ks] = *reinterpret_cast<const typename C::x8 *>(kbuf + kofs[ks] + t * 32 * C::ROWB);
    __builtin_amdgcn_sched_barrier(0);
    sacc[0] = C::M::mfma(ka[0][0], qf[0], zero);
#pragma unroll
    for (int ks = 1; ks < C::KS; ++ks)
        sacc[0] = C::M::mfma(ka[0][ks], qf[ks], sacc[0]);
    __builtin_amdgcn_sched_barrier(0);
    if (need_mask) mask_block(sacc[0], 0, thr);

    // ---- block 1's QK MFMAs; block 0's probabilities
    f32x16 pf;
    sacc[1] = C::M::mfma(ka[1][0], qf[0], zero);
#pragma unroll
    for (int ks = 1; ks < C::KS; ++ks)
        sacc[1] = C::M::mfma(ka[1][ks], qf[ks], sacc[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) probs_step(sacc[0], c, st_.mc, i, pf);
    typename C::x8 p0_lo, p0_hi, p1_lo, p1_hi;
    float ls = probs_finish<C>(pf, p0_lo, p0_hi);
    if (__builtin_expect(!st_.m_set || __any(!(ls <= C::M::kBlockSumMax)), 0)) {
        ls = rebase_block<C>(sacc[0], st_.o, st_.m, st_.l, c, p0_lo, p0_hi);
        st_.m_set = true;
        st_.mc = (st_.m == -INFINITY) ? 0.f : st_.m * c;
    }
    st_.l += ls;
    if (need_mask) mask_block(sacc[1], 1, thr);

    // ---- block 0's PV MFMAs, block 1's probabilities and V^T reads between them
    typename C::x8 va0[NPV], va1[NPV];
#pragma unroll
    for (int k = 0; k < NPV; ++k) va0[k] = read_vt<C>(vbuf, vofs, k / C::DT, k % C::DT);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NPV; ++k) {
        st_.o[k % C::DT] = C::M::mfma(va0[k], k < C::DT ? p0_lo : p0_hi, st_.o[k % C::DT]);
        va1[k] = read_vt<C>(vbuf, vofs, 2 + k / C::DT, k % C::DT);
#pragma unroll
        for (int i = k * 8 / NPV; i < (k + 1) * 8 / NPV; ++i) probs_step(sacc[1], c, st_.mc, i, pf);
        __builtin_amdgcn_sched_barrier(0);
    }
    ls = probs_finish<C>(pf, p1_lo, p1_hi);
    if (__builtin_expect(__any(!(ls <= C::M::kBlockSumMax)), 0)) {
        ls = rebase_block<C>(sacc[1], st_.o, st_.m, st_.l, c, p1_lo, p1_hi);
        st_.mc = (st_.m == -INFINITY) ? 0.f : st_.m * c;
    }
    st_.l += ls;

    // ---- block 1's PV MFMAs
#pragma unroll
    for (int k = 0; k < NPV; ++k)
        st_.o[k % C::DT] = C::M::mfma(va1[k], k < C::DT ? p1_lo : p1_hi, st_.o[k % C::DT]);
}

// The same tile for head_dim 256 (KS = 16 k-steps, DT = 8 output blocks):
// the K operands of the two 32-key blocks (64 registers each) and the V^T
// operands of a block (64) are not all held at once; each block's operands
// are read just before its MFMAs, which leaves room for the wave's 128
// output accumulators and 64 query registers.
template <class C>
__device__ __forceinline__ void attend_tile_wide(const unsigned char *kbuf, const unsigned char *vbuf,
                                                 const int (&kofs)[C::KS], const int (&vofs)[C::DT],
                                                 const typename C::x8 (&qf)[C::KS], SoftState<C> &st_, bool need_mask,
                                                 int thr, float c) {
    constexpr int NPV = 2 * C::DT;
    const f32x16 zero = {};
    f32x16 sacc[2];
    typename C::x8 p_lo[2], p_hi[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        sacc[t] = zero;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const typename C::x8 ka = *reinterpret_cast<const typename C::x8 *>(kbuf + kofs[ks] + t * 32 * C::ROWB);
            sacc[t] = C::M::mfma(ka, qf[ks], sacc[t]);
        }
        if (need_mask) mask_block(sacc[t], t, thr);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        f32x16 pf;
#pragma unroll
        for (int i = 0; i < 8; ++i) probs_step(sacc[t], c, st_.mc, i, pf);
        float ls = probs_finish<C>(pf, p_lo[t], p_hi[t]);
        const bool big = __any(!(ls <= C::M::kBlockSumMax));
        if (__builtin_expect((!st_.m_set) | big, 0)) {
            if (t == 1) {  // block 0's products use the reference block 1 moves: finish them first
#pragma unroll
                for (int k = 0; k < NPV; ++k)
                    st_.o[k % C::DT] = C::M::mfma(read_vt<C>(vbuf, vofs, k / C::DT, k % C::DT),
                                                  k < C::DT ? p_lo[0] : p_hi[0], st_.o[k % C::DT]);
            }
            ls = rebase_block<C>(sacc[t], st_.o, st_.m, st_.l, c, p_lo[t], p_hi[t]);
            st_.m_set = true;
            st_.mc = (st_.m == -INFINITY) ? 0.f : st_.m * c;
            if (t == 1) {
                st_.l += ls;
#pragma unroll
                for (int k = 0; k < NPV; ++k)
                    st_.o[k % C::DT] = C::M::mfma(read_vt<C>(vbuf, vofs, 2 + k / C::DT, k % C::DT),
                                                  k < C::DT ? p_lo[1] : p_hi[1], st_.o[k % C::DT]);
                return;
            }
        }
        st_.l += ls;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int k = 0; k < NPV; ++k)
            st_.o[k % C::DT] = C::M::mfma(read_vt<C>(vbuf, vofs, 2 * t + k / C::DT, k % C::DT),
                                          k < C::DT ? p_lo[t] : p_hi[t], st_.o[k % C::DT]);
}

// One step of a wave: the direct loads of the next step into (nk, nv), if
// `load`, then the wave's tile of this step from cur, if `tile`.  The three
// step buffers are distinct (restrict), which tells the compiler that the
// tile's LDS reads do not depend on the loads in flight: it then issues them
// without waiting for those loads (the caller's s_waitcnt and barrier after
// the step order every buffer's loads before its reads).
template <class C>
__device__ __forceinline__ void load_and_attend(const PfArgs &a, bool load, int kb1, int kmax, int shift, int bmask,
                                                int win0, int blk0, int64_t kv_row, int64_t kv_head,
                                                const uint32_t (&koff)[C::LPW], const uint32_t (&voff)[C::VOFFS],
                                                int w, int lane,
                                                const int *s_blk, unsigned char *__restrict__ nk,
                                                unsigned char *__restrict__ nv, bool tile,
                                                const unsigned char *__restrict__ cur, const int (&kofs)[C::KS],
                                                const int (&vofs)[C::DT], const typename C::x8 (&qf)[C::KS],
                                                SoftState<C> &st, bool need_mask, int thr, float c) {
    if (load) load_wave_rows<C>(a, kb1, kmax, shift, bmask, win0, blk0, kv_row, kv_head, koff, voff, w, lane, s_blk, nk, nv);
    if (tile) {
        if constexpr (C::KS > 8) attend_tile_wide<C>(cur, cur, kofs, vofs, qf, st, need_mask, thr, c);
        else attend_tile<C>(cur, cur, kofs, vofs, qf, st, need_mask, thr, c);
    }
}

template <int D, int NH, bool I8, typename E, int NW>
__global__ __launch_bounds__(64 * NW, (NW == 8 || D > 128) ? 1 : 2) void prefill_mfma_kernel(PfArgs a) {
    using C = Pf<D, NH, E, NW>;
    constexpr int kStep = C::STEP;
    constexpr int kPfThreads = C::THREADS;
    // [K, V][buffer][step rows] bf16 step buffers: every buffer and block
    // offset of an LDS read is an immediate.  bf16 pools: two buffers, the
    // next step loading while this one is computed.  INT8 pools: one bf16
    // buffer, then the int8 staging step (K, V) and its scale words: the next
    // step's codes load while this one is computed, and are dequantized into
    // the buffer between two barriers.  After the key loop the same memory
    // carries the second key half's partial results to the first.
    constexpr int NB = I8 ? 1 : 2;
    constexpr int MEMB = I8 ? 2 * C::STEPB + 2 * C::STAGEB + 2 * C::SCLB : 4 * C::STEPB;
    __shared__ __attribute__((aligned(1024))) unsigned char s_mem[MEMB];
    __shared__ int s_blk[kBlkWin];
    auto kbuf = [&](int b) { return s_mem + b * C::STEPB; };
    auto vbuf = [&](int b) { return s_mem + (NB + b) * C::STEPB; };
    unsigned char *const s_k8 = s_mem + 2 * C::STEPB;  // INT8 only (past the end otherwise: never used)
    unsigned char *const s_v8 = s_k8 + C::STAGEB;
    uint32_t *const s_sk = reinterpret_cast<uint32_t *>(s_v8 + C::STAGEB);
    uint32_t *const s_sv = s_sk + kStep;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = tid >> 6;
    const int n = lane & 31, hf = lane >> 5;
    const int kh = C::KH == 2 ? w / (C::WAVES / 2) : 0;  // key half: tile kh of every step
    const int wl = w % (C::WAVES / C::KH);               // (head, position sub-tile) slot

    int64_t wg = blockIdx.x;
    const int g = (int)(wg % a.hkv);
    wg /= a.hkv;
    const int hgrp = (int)(wg % a.head_groups);
    wg /= a.head_groups;
    // single tiles: the sequences in groups of seq_group (all of them when
    // 0), and inside a group unit u of every sequence before unit u + 1,
    // unit u being tile T-1-u, so the group's longest tiles are dispatched
    // first; pairs: sequence-major
    int pair, s;
    if (a.single) {
        const int sg = a.seq_group > 0 ? a.seq_group : a.num_seqs;
        const int64_t per = (int64_t)sg * a.units_per_seq;
        const int64_t k = wg / per, loc = wg % per;
        const int sgk = (int)min((int64_t)sg, (int64_t)a.num_seqs - k * sg);  // the last group may be short
        pair = (int)(loc / sgk);
        s = (int)(k * sg + loc % sgk);
    } else {
        pair = (int)(wg % a.units_per_seq);
        s = (int)(wg / a.units_per_seq);
    }

    // rows outside [0, total_q) are never read or written, whatever cu_seqlens_q holds
    const int q_start = min(max(a.cu_q[s], 0), a.total_q);
    const int q_len = min(max(a.cu_q[s + 1], 0), a.total_q) - q_start;
    const int k_len = a.cu_k[s + 1] - a.cu_k[s];
    const int q_off = a.q_off[s];
    const int T = (q_len + C::BM - 1) / C::BM;
    if (pair >= (a.single ? T : (T + 1) / 2)) return;

    const int hh = wl % NH, sub = wl / NH;
    const int h = g * a.group + hgrp * NH + hh;
    const int hq = a.hkv * a.group;
    const int shift = a.block_shift;
    const int bmask = (1 << shift) - 1;
    const int32_t *bt = a.block_table + (int64_t)s * a.bt_stride;
    // keys that may be indexed: within k_len and within the table row
    const int kcap = (int)min((int64_t)k_len, (int64_t)a.bt_stride << shift);
    const float c = a.scale_log2;
    const int64_t kv_row = (int64_t)a.hkv * D;  // elements per pool slot
    const int64_t kv_head = (int64_t)g * D;
    const int pn = swap_bits_2_3(n);
    // byte offsets, from the K buffer of a step, of this lane's K reads (row
    // pn of its key half's tile, chunk 2ks + hf, swizzled; block 1 adds 32
    // rows, which keeps the swizzle) and V^T transpose reads (the V buffers
    // start 2*STEPB further), one per 32-wide d block: row 8hf + i/4, chunk
    // (4dt + 2(grp&1) + (i&3)/2) ^ 4(i/4), byte 8(i&1) inside the chunk (i =
    // lane%16, grp = lane/16).  What remains of each LDS address is an
    // immediate offset.
    int kofs[C::KS], vofs[C::DT];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kofs[ks] = kh * C::TILEB + pn * C::ROWB + k_slot<C::CPR>(pn, 2 * ks + hf) * 16;
    {
        const int li = lane & 15, grp = lane >> 4;
        const int row = 8 * hf + (li >> 2);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const int chunk = 4 * dt + 2 * (grp & 1) + ((li & 3) >> 1);
            vofs[dt] = NB * C::STEPB + kh * C::TILEB + row * C::ROWB + v_slot<C::CPR>(row, chunk) * 16 + 8 * (li & 1);
        }
    }
    // byte offsets, inside the pool, of this lane's 16-byte pieces of the
    // wave's 16 rows (fast load path): row RPI*u + lane/CPR of the wave,
    // swizzled chunk of slot lane%CPR
    // (the row RPI*u itself is a scalar offset; the V swizzle is the same for
    // every u because 4*RPI is a multiple of CPR)
    uint32_t koff[C::LPW];
    uint32_t voff[C::VOFFS];
#pragma unroll
    for (int u = 0; u < C::VOFFS; ++u)
        voff[u] = (uint32_t)((lane / C::CPR) * kv_row * 2 +
                             v_slot<C::CPR>(C::RPI * u + lane / C::CPR, lane % C::CPR) * 16);
#pragma unroll
    for (int u = 0; u < C::LPW; ++u)  // (the wave's first row, 16w, matters for the K swizzle when CPR = 32)
        koff[u] = (uint32_t)((lane / C::CPR) * kv_row * 2 +
                             k_slot<C::CPR>(kRowsPerWave * w + C::RPI * u + lane / C::CPR, lane % C::CPR) * 16);
    float *merge = reinterpret_cast<float *>(s_mem) + wl * (C::MERGE * 64);

    for (int it = 0; it < 2; ++it) {
        const int tile = (a.single || it == 0) ? T - 1 - pair : pair;
        if (it == 1 && (a.single || tile == T - 1 - pair)) break;

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
            if (kh == 0 && row_ok && hf == 0)
                for (int d = 0; d < D; ++d) orow[d] = 0;
            continue;
        }
        const int nsteps = kmax_wg / kStep + 1;
        const int last_blk = kmax_wg >> shift;

        // the wave's queries, B operand layout: lane (n, hf), k-step ks holds d = 16ks + 8hf .. +7
        typename C::x8 qf[C::KS];
        {
            const uint16_t *qrow = a.q + (int64_t)(q_start + i_me) * a.q_row_stride + (int64_t)h * D;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                uint4 v = row_ok ? ld16(qrow + 16 * ks + 8 * hf) : make_uint4(0, 0, 0, 0);
                qf[ks] = __builtin_bit_cast(typename C::x8, v);
            }
        }
        SoftState<C> sm;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.o[dt][r] = 0.f;
        sm.m = -INFINITY;
        sm.mc = 0.f;
        sm.l = 0.f;
        sm.m_set = false;

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
        stage_ids(0);
        __syncthreads();
        const int blk0 = s_blk[0];  // physical block of key 0 (finite stand-in for masked rows)
        if constexpr (I8) {
            load_wave_rows_i8<C>(a, 0, kmax_wg, shift, bmask, win0, blk0, g, w, lane, s_blk, s_k8, s_v8,
                                 reinterpret_cast<unsigned char *>(s_sk), reinterpret_cast<unsigned char *>(s_sv));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            convert_step_i8<C>(s_k8, s_v8, s_sk, s_sv, g, kbuf(0), vbuf(0), tid);
        } else {
            load_wave_rows<C>(a, 0, kmax_wg, shift, bmask, win0, blk0, kv_row, kv_head, koff, voff, w, lane, s_blk,
                              kbuf(0), vbuf(0));
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();

        // one step j in buffer BUF (compile-time): issue the loads of step
        // j+1 into the other buffer, compute this wave's tile of step j, wait
        // for the loads and synchronise
        auto step = [&](int j, auto buf_c) {
            constexpr int BUF = decltype(buf_c)::value;
            const bool load = j + 1 < nsteps;
            const int kb1 = (j + 1) * kStep;
            if (load && (min(kb1 + kStep - 1, kmax_wg) >> shift) >= win0 + kBlkWin) {  // leave the staged window
                stage_ids(kb1 >> shift);
                __syncthreads();
            }
            const int kb = j * kStep + kh * kBN;
            if constexpr (I8) {
                // codes of step j+1 load into the staging step while step j is
                // computed; after the barrier they are dequantized into the
                // (now free) buffer
                if (load)
                    load_wave_rows_i8<C>(a, kb1, kmax_wg, shift, bmask, win0, blk0, g, w, lane, s_blk, s_k8, s_v8,
                                         reinterpret_cast<unsigned char *>(s_sk),
                                         reinterpret_cast<unsigned char *>(s_sv));
                if (wave_active && kb <= kmax_w)
                    attend_tile<C>(kbuf(0), kbuf(0), kofs, vofs, qf, sm, kb + kBN - 1 > kfull_w, lim_me - kb - 8 * hf,
                                   c);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (load) {
                    convert_step_i8<C>(s_k8, s_v8, s_sk, s_sv, g, kbuf(0), vbuf(0), tid);
                    __syncthreads();
                }
            } else {
                load_and_attend<C>(a, load, kb1, kmax_wg, shift, bmask, win0, blk0, kv_row, kv_head, koff, voff, w,
                                   lane, s_blk, kbuf(BUF ^ 1), vbuf(BUF ^ 1), wave_active && kb <= kmax_w, kbuf(BUF),
                                   kofs, vofs, qf, sm, kb + kBN - 1 > kfull_w, lim_me - kb - 8 * hf, c);
                __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of step j+1 have landed
                __syncthreads();
            }
        };
        if constexpr (I8) {
            for (int j = 0; j < nsteps; ++j) step(j, std::integral_constant<int, 0>{});
        } else {
            for (int j = 0; j < nsteps; j += 2) {
                step(j, std::integral_constant<int, 0>{});
                if (j + 1 < nsteps) step(j + 1, std::integral_constant<int, 1>{});
            }
        }

        if constexpr (C::KH == 2) {
            // ---- the second key half hands (O, m, l) to the first through LDS
            if (kh == 1) {
    #pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) merge[(dt * 16 + r) * 64 + lane] = sm.o[dt][r];
                merge[(C::DT * 16) * 64 + lane] = sm.m;
                merge[(C::DT * 16 + 1) * 64 + lane] = sm.l;
            }
            __syncthreads();
            if (kh == 0) {
                const float m2 = merge[(C::DT * 16) * 64 + lane];
                const float l2 = merge[(C::DT * 16 + 1) * 64 + lane];
                const float mn = fmaxf(sm.m, m2);
                const float a1 = (sm.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sm.m - mn) * c);
                const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m2 - mn) * c);
                const float l = sm.l * a1 + l2 * a2;
                // ---- epilogue: O = O^T / l; lane (n, hf) holds d = 32dt + 8b + 4hf + a at register a + 4b
                const float l_tot = halves_sum(l);
                const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                if (row_ok) {
    #pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt)
    #pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            f32x4 v;
    #pragma unroll
                            for (int a4 = 0; a4 < 4; ++a4) {
                                const int r = 4 * b + a4;
                                v[a4] = (sm.o[dt][r] * a1 + merge[(dt * 16 + r) * 64 + lane] * a2) * inv;
                            }
                            *reinterpret_cast<typename C::x4 *>(orow + 32 * dt + 8 * b + 4 * hf) =
                                __builtin_convertvector(v, typename C::x4);
                        }
                }
            }
        } else {  // one wave per slot: O^T / l straight out
            const float l_tot = halves_sum(sm.l);
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            if (row_ok) {
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        f32x4 v;
#pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4) v[a4] = sm.o[dt][4 * b + a4] * inv;
                        *reinterpret_cast<typename C::x4 *>(orow + 32 * dt + 8 * b + 4 * hf) =
                            __builtin_convertvector(v, typename C::x4);
                    }
            }
        }
        __syncthreads();  // the merge area is the next tile's K/V buffer
    }
}

template <int D, int NH, bool I8, typename E, int NW>
hipError_t run(const PfArgs &a, int num_seqs, int max_seqlen_q, hipStream_t stream) {
    using C = Pf<D, NH, E, NW>;
    PfArgs b = a;
    const int max_tiles = (max_seqlen_q + C::BM - 1) / C::BM;
    b.num_seqs = num_seqs;
    b.units_per_seq = a.single ? max_tiles : (max_tiles + 1) / 2;
    b.head_groups = a.group / NH;
    const int64_t wgs = (int64_t)num_seqs * b.units_per_seq * b.head_groups * a.hkv;
    if (wgs == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_mfma_kernel<D, NH, I8, E, NW>), dim3((unsigned)wgs), dim3(C::THREADS), 0, stream, b);
    return hipGetLastError();
}

template <int D, bool I8 = false, typename E = bf16_t, int NW = 8>
hipError_t dispatch_nh(const PfArgs &a, int num_seqs, int max_seqlen_q, hipStream_t stream) {
    switch (a.group) {
        case 1: return run<D, 1, I8, E, NW>(a, num_seqs, max_seqlen_q, stream);
        case 2: return run<D, 2, I8, E, NW>(a, num_seqs, max_seqlen_q, stream);
        case 4: return run<D, 4, I8, E, NW>(a, num_seqs, max_seqlen_q, stream);
        case 8: return run<D, 4, I8, E, NW>(a, num_seqs, max_seqlen_q, stream);
    }
    return hipErrorInvalidValue;
}

// Workgroups of a launch (the same in both layouts): sequences x work units
// at max_seqlen_q x head groups x KV heads, a unit being a pair of query
// tiles, or a single tile.
int64_t prefill_grid(int group, int hkv, int num_seqs, int max_seqlen_q, bool single) {
    const int nh = group >= 4 ? 4 : group;
    const int bm = 32 * (4 / nh);
    const int64_t tiles = ((int64_t)max_seqlen_q + bm - 1) / bm;
    return (int64_t)num_seqs * (single ? tiles : (tiles + 1) / 2) * (group / nh) * hkv;
}

// Work units and layout of a launch.
//  * Layout: the 8-wave workgroup while the launch's tile pairs fit the CUs in
//    one round (every workgroup streams its keys alone on a CU); the 4-wave
//    one, two per CU, once they do not (many or short sequences), so one
//    workgroup's prologue and epilogue overlap another's matrix work.
//  * Units: pairs of query tiles (p, T-1-p) give the workgroups of a
//    sequence equal causal work; they serve the one case where equal work
//    matters, a single round of 8-wave workgroups that single tiles would
//    overflow (a long prompt).  Otherwise a workgroup takes one tile: when the
//    tiles all fit the CUs at once, the launch then costs one tile's latency
//    chain (metadata, block ids, first keys, epilogue) rather than two in a
//    row; with more tiles than slots, the smaller units, longest first, fill
//    the slots more evenly (4-wave layout, measured on MI355X: 8192 new
//    tokens over 17 sequences of 35 to 842, 56 -> 45 us against tile pairs).
//  * Order of single tiles: longest first across the whole batch balances a
//    ragged batch; when every sequence has the same number of new tokens
//    (total_q = num_seqs * max_seqlen_q, known on the host) there is nothing
//    to balance, and groups of 4 sequences keep their K/V in L2 while their
//    tiles run (64 sequences of 128 tokens: 39 -> 32 us).  For the ragged
//    batch the groups cut the HBM reads from 1.29x to 1.0x the Q+K+V bytes
//    but left long tiles of later groups to run alone at the end (52 -> 62
//    us with groups of 8, 70 us with 4), so it keeps the batch-wide order.
void plan_prefill(PfArgs &a, int num_seqs, int max_seqlen_q, bool &w4) {
    const bool singles_fit = prefill_grid(a.group, a.hkv, num_seqs, max_seqlen_q, true) <= kNumCUs;
    w4 = prefill_grid(a.group, a.hkv, num_seqs, max_seqlen_q, false) > kNumCUs;
    a.single = (singles_fit || w4) ? 1 : 0;
    a.seq_group = (int64_t)a.total_q == (int64_t)num_seqs * max_seqlen_q ? 4 : 0;
}

}  // namespace

bool prefill_mfma_supported(const PoolGeom &g, int group) {
    // 16 pool rows (one wave's share of a step) must span < 2^31 bytes for
    // the 32-bit buffer offsets
    return (g.dtype == 1 || g.dtype == 3) && (g.d == 64 || g.d == 128 || g.d == 256) && g.block_size >= 4 &&
           (group == 1 || group == 2 || group == 4 || group == 8) &&
           (int64_t)g.hkv * g.d * 2 * kRowsPerWave < ((int64_t)1 << 31);
}

hipError_t launch_prefill_mfma(const void *q, int64_t q_row_stride, int hq, const void *k_pool,
                               const void *v_pool, const PoolGeom &g, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, const int32_t *q_offsets,
                               const int32_t *block_table, int bt_stride, int num_seqs, int total_q,
                               int max_seqlen_q, float softmax_scale, void *out, hipStream_t stream) {
    PfArgs a{};
    a.total_q = total_q;
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
    bool w4;
    plan_prefill(a, num_seqs, max_seqlen_q, w4);
    if (g.d == 256) {  // 4-wave layout only: its 64-key steps of 512-byte rows fill 128 KB of LDS
        a.single = 1;
        return g.dtype == 3 ? dispatch_nh<256, false, f16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                            : dispatch_nh<256, false, bf16_t, 4>(a, num_seqs, max_seqlen_q, stream);
    }
    if (g.dtype == 3)
        return g.d == 128 ? (w4 ? dispatch_nh<128, false, f16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                                : dispatch_nh<128, false, f16_t, 8>(a, num_seqs, max_seqlen_q, stream))
                          : (w4 ? dispatch_nh<64, false, f16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                                : dispatch_nh<64, false, f16_t, 8>(a, num_seqs, max_seqlen_q, stream));
    return g.d == 128 ? (w4 ? dispatch_nh<128, false, bf16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                            : dispatch_nh<128, false, bf16_t, 8>(a, num_seqs, max_seqlen_q, stream))
                      : (w4 ? dispatch_nh<64, false, bf16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                            : dispatch_nh<64, false, bf16_t, 8>(a, num_seqs, max_seqlen_q, stream));
}

bool prefill_mfma_int8_supported(const PoolGeom &g, int group) {
    // INT8 pools with bf16 or fp16 queries: the scale words are 4-byte pairs of heads
    // (even hkv); 16 pool rows span < 2^31 bytes
    return g.dtype == 2 && (g.d == 64 || g.d == 128) && g.block_size >= 4 && g.hkv % 2 == 0 &&
           (group == 1 || group == 2 || group == 4 || group == 8) &&
           (int64_t)g.hkv * g.d * kRowsPerWave < ((int64_t)1 << 31);
}

hipError_t launch_prefill_mfma_int8(const void *q, int64_t q_row_stride, int hq, int q_dtype, const void *k_pool,
                                    const void *v_pool, const void *k_scale, const void *v_scale, const PoolGeom &g,
                                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                    const int32_t *q_offsets, const int32_t *block_table, int bt_stride,
                                    int num_seqs, int total_q, int max_seqlen_q, float softmax_scale, void *out,
                                    hipStream_t stream) {
    PfArgs a{};
    a.total_q = total_q;
    a.q = reinterpret_cast<const uint16_t *>(q);
    a.q_row_stride = q_row_stride;
    a.k_pool = reinterpret_cast<const uint16_t *>(k_pool);
    a.v_pool = reinterpret_cast<const uint16_t *>(v_pool);
    a.k_scale = reinterpret_cast<const uint16_t *>(k_scale);
    a.v_scale = reinterpret_cast<const uint16_t *>(v_scale);
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
    bool w4;
    plan_prefill(a, num_seqs, max_seqlen_q, w4);  // as for 16-bit pools
    if (q_dtype == 3)  // fp16 queries: the codes dequantize to fp16, fp16 MFMA
        return g.d == 128 ? (w4 ? dispatch_nh<128, true, f16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                                : dispatch_nh<128, true, f16_t, 8>(a, num_seqs, max_seqlen_q, stream))
                          : (w4 ? dispatch_nh<64, true, f16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                                : dispatch_nh<64, true, f16_t, 8>(a, num_seqs, max_seqlen_q, stream));
    return g.d == 128 ? (w4 ? dispatch_nh<128, true, bf16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                            : dispatch_nh<128, true, bf16_t, 8>(a, num_seqs, max_seqlen_q, stream))
                      : (w4 ? dispatch_nh<64, true, bf16_t, 4>(a, num_seqs, max_seqlen_q, stream)
                            : dispatch_nh<64, true, bf16_t, 8>(a, num_seqs, max_seqlen_q, stream));
}

}  // namespace pa
