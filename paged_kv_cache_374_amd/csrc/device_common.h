// Device-side helpers shared by the kernels: element types, conversions, vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

// Storage tags for the 16-bit element types (raw bit patterns in memory).
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

template <typename T> struct Elt;
template <> struct Elt<float> {
    static __device__ __forceinline__ float to_float(float x) { return x; }
    static __device__ __forceinline__ float from_float(float x) { return x; }
};
template <> struct Elt<bf16_t> {
    // bfloat16 is the top half of a binary32.
    static __device__ __forceinline__ float to_float(bf16_t x) {
        return __uint_as_float((uint32_t)x.bits << 16);
    }
    // Round to nearest even (hardware conversion on gfx950).
    static __device__ __forceinline__ bf16_t from_float(float x) {
        __bf16 h = (__bf16)x;
        return bf16_t{__builtin_bit_cast(uint16_t, h)};
    }
};
template <> struct Elt<f16_t> {
    static __device__ __forceinline__ float to_float(f16_t x) {
        return (float)__builtin_bit_cast(_Float16, x.bits);
    }
    static __device__ __forceinline__ f16_t from_float(float x) {
        _Float16 h = (_Float16)x;
        return f16_t{__builtin_bit_cast(uint16_t, h)};
    }
};

// Unpack a 16-byte vector into floats.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Vec16<f16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        }
    }
};

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x combined with x of lane l ^ 32, through the gfx950 lane swap (a VALU operation, no
// LDS round trip as for a general shuffle). The swap exchanges the upper half of its
// first operand with the lower half of its second; with x in both, one result holds x
// and the other x of lane l ^ 32 in every lane, in an order that max and sum ignore.
__device__ __forceinline__ float max_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// binary32 -> OCP FP8 E4M3 code (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
// bits; largest finite value 448; S.1111.111 is NaN): nearest, ties to an even
// mantissa; magnitudes of 448 or more (infinity included) give 448; NaN stays NaN.
// Integer arithmetic on the binary32 fields, plus one exact power-of-two scaling and
// a round-to-nearest-even in the subnormal range.
__device__ __forceinline__ uint32_t fp8_e4m3_code(float y) {
    // Every case is computed and the right one selected, with no branches: as a chain
    // of early returns this compiled to divergent branches costing ~2 us of a decode
    // step's prologue per 16 codes.
    const uint32_t b = __float_as_uint(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7fffffffu;
    // |y| < 2^-6: multiples of 2^-9; |y| * 2^9 is exact, a result of 8 is the code of
    // 2^-6 (the smallest normal). The operand is clamped so the conversion stays in
    // range when another case applies.
    const uint32_t sub =
        (uint32_t)__builtin_rintf(__builtin_fminf(__uint_as_float(a), 0x1p-6f) * 512.0f);
    // normal range: the E4M3 biased exponent (1..15) and the top 3 mantissa bits,
    // rounded to nearest even on the 20 bits dropped; a carry moves to the exponent
    const uint32_t expo = (a >> 23) - 120u;
    const uint32_t mant = a & 0x7fffffu;
    const uint32_t keep = mant >> 20;
    const uint32_t rest = mant & 0xfffffu;
    const uint32_t up = (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u;
    const uint32_t normal = (expo << 3) + keep + up;
    uint32_t code = a < 0x3c800000u ? sub : normal;
    code = a >= 0x43e00000u ? 0x7eu : code;                // |y| >= 448 (infinity too)
    code = a > 0x7f800000u ? 0x7fu : code;                 // NaN
    return sign | code;
}

}  // namespace pkv
