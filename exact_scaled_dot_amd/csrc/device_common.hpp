// Device-side helpers shared by the libsdpa HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte global load as four dwords.
__device__ __forceinline__ u32x4 ldg128(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Pack the low (resp. high) 16-bit halves of two dwords: result = lo16(a) | lo16(b) << 16.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// fp32 -> bf16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 -> packed bf16 pair (lo = a, hi = b), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32 on gfx950 (RNE)
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 positions away (lanes l and l^32 swap values).
__device__ __forceinline__ float swap_half_wave(float x) {
    return __shfl_xor(x, 32);
}

// max(x[l], x[l^32]) in every lane, without the LDS: v_permlane32_swap on two
// copies of x yields (x_lo, x_lo) and (x_hi, x_hi).
__device__ __forceinline__ float max_half_waves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                   __builtin_bit_cast(unsigned, x), false, false);
    // The two results are copied to scalars before the bit casts: this hipcc
    // folds __builtin_bit_cast of a vector element to element 0.
    const unsigned r0 = r[0], r1 = r[1];
    return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// Three-input maximum as one v_max3_f32 (the inputs are MFMA results or -inf,
// so the NaN canonicalisation the compiler adds around fmaxf is not needed).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// ---------------------------------------------------------------------------
// 16-bit element types of the MFMA paths (bf16 and fp16 inputs).  Operands
// travel as raw 32-bit words; these wrappers pick the instruction.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

struct Bf16T {
    static constexpr bool kF16 = false;
};
struct F16T {
    static constexpr bool kF16 = true;
};

template <class T>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (T::kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <class T>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (T::kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <class T>
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    if constexpr (T::kF16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
// Two fp32 values -> packed 16-bit pair (lo = a, hi = b), round to nearest even.
template <class T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (T::kF16) {
        const f16x2 r = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, r);
    } else {
        return pack_bf16x2(a, b);
    }
}
// Element `hi` (0: low half, 1: high half) of a packed 16-bit pair as fp32 (exact).
template <class T>
__device__ __forceinline__ float bias_elem(uint32_t w, int hi) {
    if constexpr (T::kF16) {
        const uint16_t h = (uint16_t)(hi ? (w >> 16) : (w & 0xffffu));
        return (float)__builtin_bit_cast(_Float16, h);
    } else {
        return __builtin_bit_cast(float, hi ? (w & 0xffff0000u) : (w << 16));
    }
}
// acc + lo + hi of a packed pair, in fp32 (v_dot2 with (1, 1)).
template <class T>
__device__ __forceinline__ float sum2(uint32_t w, float acc) {
    if constexpr (T::kF16) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
    } else {
        const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
    }
}
// fp32 -> 16-bit bits in the low half, round to nearest even.
template <class T>
__device__ __forceinline__ uint32_t to16(float f) {
    if constexpr (T::kF16)
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
    else
        return f32_to_bf16_bits(f);
}

}  // namespace sdpa
