// Device helpers shared by the gfx950 kernels.
//
// Lane layout used for per-token work on d = 128: a wavefront holds 16 tokens;
// lane l works on token (l & 15) and owns the 32 consecutive coordinates
// 32*(l >> 4) .. 32*(l >> 4) + 31.  Coordinate bits 0..4 therefore live inside
// a lane and bits 5, 6 across lanes l ^ 16 and l ^ 32.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return float(__builtin_bit_cast(_Float16, uint16_t(bits16)));
}
__device__ __forceinline__ uint32_t f2h(float f) {
    return uint32_t(__builtin_bit_cast(uint16_t, _Float16(f)));
}

// Walsh-Hadamard butterflies over the five in-lane coordinate bits.
__device__ __forceinline__ void fwht_inlane32(float (&v)[32]) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

// Butterflies over coordinate bits 5 and 6 (partner lanes l^16 and l^32):
// the lower lane keeps a + b, the upper lane b' - a' = (partner) - (own).
__device__ __forceinline__ void fwht_crosslane(float (&v)[32], int lane) {
#pragma unroll
    for (int s = 16; s <= 32; s <<= 1) {
        const float sg = (lane & s) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float p = __shfl_xor(v[i], s);
            v[i] = fmaf(sg, v[i], p);
        }
    }
}

__device__ __forceinline__ float quad_sum(float x) {  // sum over lanes l, l^16, l^32, l^48
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Code i (compile-time) of width B from an LSB-first bitstream held in dwords.
template <int B, int I>
__device__ __forceinline__ uint32_t code_at(const uint32_t *w) {
    constexpr int bit = I * B, wi = bit / 32, sh = bit % 32;
    if constexpr (sh + B <= 32) {
        return (w[wi] >> sh) & ((1u << B) - 1u);
    } else {
        return ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & ((1u << B) - 1u);
    }
}

template <int B, int I>
__device__ __forceinline__ void put_code(uint32_t *w, uint32_t c) {
    constexpr int bit = I * B, wi = bit / 32, sh = bit % 32;
    w[wi] |= c << sh;
    if constexpr (sh + B > 32) w[wi + 1] |= c >> (32 - sh);
}

template <int N, int I = 0>
struct Unroll {
    template <typename F>
    __device__ __forceinline__ static void run(F &&f) {
        if constexpr (I < N) {
            f(std::integral_constant<int, I>{});
            Unroll<N, I + 1>::run(f);
        }
    }
};

// binary64 -> binary16 with one rounding (nearest, ties to even), from the
// bit pattern; used for per-group scales that must match an exact reference.
__device__ __forceinline__ uint32_t double_to_half_bits(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t sign = uint32_t((b >> 48) & 0x8000u);
    const int exp = int((b >> 52) & 0x7FF);
    const uint64_t frac = b & ((1ull << 52) - 1);
    if (exp == 0x7FF) return sign | 0x7C00u | (frac ? 0x200u : 0u);
    if (exp == 0) return sign;
    const int e = exp - 1023;
    const uint64_t m = (1ull << 52) | frac;
    if (e > 15) return sign | 0x7C00u;
    if (e >= -14) {
        uint64_t hm = m >> 42;
        const uint64_t rem = m & ((1ull << 42) - 1), half = 1ull << 41;
        if (rem > half || (rem == half && (hm & 1))) ++hm;
        int he = e + 15;
        if (hm == (1ull << 11)) { hm >>= 1; ++he; }
        if (he >= 31) return sign | 0x7C00u;
        return sign | uint32_t(he << 10) | uint32_t(hm & 0x3FF);
    }
    const int shift = 28 - e;
    if (shift > 53) return sign;
    uint64_t hm = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (hm & 1))) ++hm;
    return sign | uint32_t(hm);
}

}  // namespace tq
