// pa_device.h -- device-side helpers shared by the gfx950 kernels of libpa.
// Wave64 throughout (CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;

// Storage tags: the kernels move raw bits and widen to fp32 themselves.
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };   // IEEE binary16

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int bytes = 4; };
template <> struct Elem<bf16_t> { static constexpr int bytes = 2; };
template <> struct Elem<f16_t> { static constexpr int bytes = 2; };

// ---- conversions ----------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary16 halves of a 32-bit word, widened exactly (v_cvt_f32_f16).
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// One stored element as fp32 (exact).
__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(bf16_t x) { return bf16_lo(x.bits); }
__device__ __forceinline__ float to_float(f16_t x) { return f16_lo(x.bits); }

// Unpack one 16-byte vector into its elements as fp32.
template <typename T> __device__ __forceinline__ void unpack16(const uint4 &v, float *f);
template <> __device__ __forceinline__ void unpack16<float>(const uint4 &v, float *f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
template <> __device__ __forceinline__ void unpack16<bf16_t>(const uint4 &v, float *f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
template <> __device__ __forceinline__ void unpack16<f16_t>(const uint4 &v, float *f) {
    f[0] = f16_lo(v.x); f[1] = f16_hi(v.x); f[2] = f16_lo(v.y); f[3] = f16_hi(v.y);
    f[4] = f16_lo(v.z); f[5] = f16_hi(v.z); f[6] = f16_lo(v.w); f[7] = f16_hi(v.w);
}

template <typename T> __device__ __forceinline__ void store_elem(T *p, float x);
template <> __device__ __forceinline__ void store_elem<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_elem<bf16_t>(bf16_t *p, float x) {
    p->bits = (uint16_t)f32_to_bf16_bits(x);
}
// fp32 -> binary16, round to nearest even (v_cvt_f16_f32 in the default mode);
// beyond the largest finite value the result is infinite.
template <> __device__ __forceinline__ void store_elem<f16_t>(f16_t *p, float x) {
    p->bits = __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---- cross-lane reductions (DPP inside a row of 16 lanes) -----------------
// DPP controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.  After the steps up to N every
// lane of an aligned group of N lanes holds the same (commutative) sum.

// Every lane of a row is a valid source for these controls, so bound_ctrl
// never applies; with it set (and no old value) the compiler folds the move
// into the consuming add or max (v_add_f32_dpp), one instruction per step.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <int N> __device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
    if constexpr (N >= 2) x += dpp_f<0xB1>(x);
    if constexpr (N >= 4) x += dpp_f<0x4E>(x);
    if constexpr (N >= 8) x += dpp_f<0x141>(x);
    if constexpr (N >= 16) x += dpp_f<0x140>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

template <int N> __device__ __forceinline__ float group_max(float x) {
    if constexpr (N >= 2) x = fmaxf(x, dpp_f<0xB1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp_f<0x4E>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp_f<0x141>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp_f<0x140>(x));
    if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
    if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

// Sum over lanes that share (lane % STRIDE), i.e. across the 64/STRIDE groups.
template <int STRIDE> __device__ __forceinline__ float cross_group_sum(float x) {
#pragma unroll
    for (int s = STRIDE; s < kWave; s <<= 1) x += __shfl_xor(x, s);
    return x;
}

// Plain 16-byte global load.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// 16-byte global load marked nontemporal: for data read exactly once (the
// decode stream of K/V), so it does not displace reusable lines in the caches.
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace pa
