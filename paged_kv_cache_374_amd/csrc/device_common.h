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

}  // namespace pkv
