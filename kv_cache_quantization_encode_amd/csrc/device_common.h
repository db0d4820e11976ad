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
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

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

// The two cross-lane butterfly stages as register swaps (gfx950
// v_permlane32_swap / v_permlane16_swap).  permlane32_swap(a, b) leaves lanes
// 0..31 holding both halves (lanes l and l+32) of element a and lanes 32..63
// both halves of element b; the butterfly then runs in-lane.  Each stage
// therefore trades one lane bit for one register bit:
//   stage 1: lane bit 5 <-> register bit 4 (pairs r, r+16),
//   stage 2: lane bit 4 <-> register bit 3 (pairs r, r+8).
// Applied after the five in-lane stages, the whole sequence is the full
// 128-point transform and maps
//   layout A: lane bits (4,5) = coord bits (3,4), register bits = (0,1,2,5,6)
//   layout N: lane bits (4,5) = coord bits (5,6), register bits = (0,1,2,3,4)
// onto each other in either direction (N is the natural "32 consecutive
// coordinates per lane" layout).
__device__ __forceinline__ void swap_butterfly32(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const float x = __uint_as_float(r[0]), y = __uint_as_float(r[1]);
    a = x + y;
    b = x - y;
}
__device__ __forceinline__ void swap_butterfly16(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const float x = __uint_as_float(r[0]), y = __uint_as_float(r[1]);
    a = x + y;
    b = x - y;
}

__device__ __forceinline__ void fwht128_swap(float (&v)[32]) {
    fwht_inlane32(v);
#pragma unroll
    for (int r = 0; r < 16; ++r) swap_butterfly32(v[r], v[r + 16]);
#pragma unroll
    for (int r = 0; r < 32; ++r)
        if ((r & 8) == 0) swap_butterfly16(v[r], v[r + 8]);
}

// Sum over lanes l, l^16, l^32, l^48 (result in every lane).
__device__ __forceinline__ float quad_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Coordinate held in register r by lane quarter q in layout A.
__host__ __device__ constexpr int layoutA_coord(int q, int r) { return 8 * q + (r & 7) + 32 * (r >> 3); }

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

// Blocks of `kernel` that can be resident at once on the current device (the
// occupancy calculator's per-CU count times the CU count), cached per device
// in `cache` (kMaxDevices entries, zero-initialised).  Persistent kernels size
// their grids with it so that no block waits for a second round.
constexpr int kMaxDevices = 64;
template <typename Kernel>
inline int resident_blocks(Kernel kernel, int threads, int *cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
    if (dev >= 0) {
        const int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
        if (v > 0) return v;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kernel), threads, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess ||
        cus < 1)
        cus = 1;
    const int v = per_cu * cus;
    if (dev >= 0) __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    return v;
}

// Grid of a persistent kernel whose waves (4 per block) stride over n_items
// tiles: as few rounds as the resident capacity allows, with the tiles spread
// evenly over the blocks of the last round count.
inline int64_t persistent_grid(int64_t n_items, int resident) {
    const int64_t per_round = int64_t(resident) * 4;
    const int64_t rounds = (n_items + per_round - 1) / per_round;
    if (rounds < 1) return 1;
    return (n_items + 4 * rounds - 1) / (4 * rounds);
}

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
