// pa_mfma.h -- device pieces shared by the MFMA prefill kernels of libpa
// (gfx950, wave64): the 16-bit operand types of the 32x32x16 matrix-core
// products, the LDS swizzles of K and V rows, lane-half reductions, and the
// direct HBM -> LDS loads.
#pragma once

#include <math.h>

#include "pa_device.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2eF = 1.4426950408889634f;

// The 16-bit element type of the pools, the queries and the matrix-core
// operands: bf16 (v_mfma_f32_32x32x16_bf16) or IEEE fp16
// (v_mfma_f32_32x32x16_f16), with the same 32x32x16 operand layouts.  The
// probabilities are rounded to the same type; kBlockSumMax bounds them (see
// attend_tile) below the type's largest finite value.
template <typename E> struct Mm;
template <> struct Mm<bf16_t> {
    typedef __bf16 x8 __attribute__((ext_vector_type(8)));
    typedef __bf16 x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 x2 __attribute__((ext_vector_type(2)));
    // every P <= 2^20: O and l stay far inside fp32 range
    static constexpr float kBlockSumMax = 1048576.f;
    static __device__ __forceinline__ f32x16 mfma(const x8 &a, const x8 &b, const f32x16 &c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(const x2 &a, const x2 &b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
    }
};
template <> struct Mm<f16_t> {
    typedef _Float16 x8 __attribute__((ext_vector_type(8)));
    typedef _Float16 x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 x2 __attribute__((ext_vector_type(2)));
    // every P <= 2^14, inside fp16's range (largest finite 65504)
    static constexpr float kBlockSumMax = 16384.f;
    static __device__ __forceinline__ f32x16 mfma(const x8 &a, const x8 &b, const f32x16 &c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(const x2 &a, const x2 &b, float c) {
        return __builtin_amdgcn_fdot2(a, b, c, false);
    }
};

// Arguments of the MFMA prefill kernels (one struct, passed by value).
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
    int num_seqs;
    int units_per_seq;      // work units (tile pairs, or single tiles) per sequence
    int single;             // 1: a unit is one query tile; 0: the pair (p, T-1-p)
    int seq_group;          // single tiles: sequences dealt together, longest tile first (0: all of them)
    int total_q;            // rows of q and out: packed rows past it are never touched
    float scale_log2;
    uint16_t *out;
    const uint16_t *k_scale;   // INT8 pools: fp16 scales [slots][hkv]
    const uint16_t *v_scale;
};

__device__ __forceinline__ int swap_bits_2_3(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// 16-byte slot of logical chunk c in LDS row r.  K rows XOR with r: the 16
// lanes of a K read name 16 different rows at one chunk.  V rows XOR with 4r
// (mod 16): a transpose read of 32 lanes names 4 consecutive rows x 4
// adjacent chunks, which 4r spreads over 16 different slots (all 64 banks);
// the V swizzle repeats every 4 rows, so a read 4k rows further is the same
// lane offset plus an immediate.
template <int CPR> __device__ __forceinline__ int k_slot(int r, int c) { return c ^ (r & (CPR - 1)); }
template <int CPR> __device__ __forceinline__ int v_slot(int r, int c) {
    return c ^ ((4 * r) & (CPR < 16 ? CPR - 1 : 15));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Max / sum of x over lanes i and i^32 (the two 32-lane halves), in every
// lane, with one v_permlane32_swap: it exchanges lanes 32..63 of its first
// operand with lanes 0..31 of its second, so with x in both, one result holds
// the lane's own x and the other its partner's.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Words of a buffer resource over `bytes` bytes from p (wave-uniform): raw
// (stride 0) addressing with 32-bit data format, the gfx9 default for
// untyped buffer loads.
__device__ __forceinline__ i32x4 raw_rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return (i32x4){__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
                   __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p) {
    return (uint32_t)(uintptr_t)(const lds_u8 *)p;
}

// Direct loads to LDS, 16 bytes per lane, lane i writing lds_base + 16 i.
// They are issued from inline assembly so that the compiler does not track
// them: it would otherwise make every later LDS read wait for them (it
// cannot tell which buffer they fill).  The kernel orders them itself: an
// s_waitcnt on all counters and a barrier separate every buffer's loads from
// its reads, and its reuse from earlier reads.
// (M0, which they write, is used by nothing else in the kernels that include
// this file.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buffer_lds16(i32x4 rsrc, uint32_t voff, int soff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_base)
                 : "memory", "m0");
}
__device__ __forceinline__ void global_lds16(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}
// 4 bytes per lane, lane i writing lds_base + 4 i.
__device__ __forceinline__ void global_lds4(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace
}  // namespace pa
