// Per-group asymmetric min-max baseline (gfx950).
//
// mac-code GitHub issue #1, technical analysis, section 2.1: groups of 64,
// scale = (max - min)/(2^b - 1), zero = min, code = round((x - zero)/scale),
// x_hat = code * scale + zero; scale and zero stored as fp16 (two fp16 per 64
// values = 0.5 bit per element).
//
// Two lanes per group, 32 consecutive elements (64 bytes) per lane; the codes
// of one lane are 32*b bits = b whole dwords of the global LSB-first stream.
// The fp16 scale is formed from the exact fp16 extremes in float64 and
// rounded once; the code is decided in float32 from the stored fp16 scale and
// zero (round half to even), then clamped.
#include <type_traits>

#include "device_common.h"

namespace tq {

template <int BITS>
__global__ __launch_bounds__(256) void minmax_quant_kernel(const uint16_t *__restrict__ x, int64_t n_half,
                                                           uint32_t *__restrict__ codes,
                                                           uint16_t *__restrict__ scale_out,
                                                           uint16_t *__restrict__ zero_out) {
    constexpr float kQmax = float((1 << BITS) - 1);
    const int64_t h = int64_t(blockIdx.x) * 256 + threadIdx.x;  // half-group index
    const bool valid = h < n_half;                               // n_half is even
    float v[32];
    float mn = INFINITY, mx = -INFINITY;
    if (valid) {
        const uint4 *src = reinterpret_cast<const uint4 *>(x + h * 32);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 u = src[c];
            const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                v[8 * c + 2 * p] = h2f(ww[p] & 0xFFFFu);
                v[8 * c + 2 * p + 1] = h2f(ww[p] >> 16);
            }
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) { mn = fminf(mn, v[j]); mx = fmaxf(mx, v[j]); }
    }
    // partner lane holds the other half of the group (h ^ 1 = lane ^ 1)
    mn = fminf(mn, __shfl_xor(mn, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    if (!valid) return;
    const uint32_t sbits = double_to_half_bits((double(mx) - double(mn)) / double(kQmax));
    const float scale = h2f(sbits);
    const float zero = mn;  // already an fp16 value
    // code = rint(fl32(v - zero) / scale), the quotient rounded to float32
    // first.  With rs = fl32(1/scale) the product (v - zero) rs is within
    // three float32 ulps of that quotient, so both round to the same integer
    // unless the product lies within 2^-17 of a half-integer (an ulp is at
    // most 2^-19 below 32); only then, in any of the lane's 32 values, the
    // lane redoes its values with the division itself.
    const float rs = scale > 0.0f ? 1.0f / scale : 0.0f;
    float code[32];
    bool tie = false;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float q = (v[j] - zero) * rs;
        code[j] = rintf(q);
        tie |= !(fabsf(fabsf(q - code[j]) - 0.5f) > 0x1p-17f);  // also NaN
    }
    if (tie && scale > 0.0f) {
#pragma unroll
        for (int j = 0; j < 32; ++j) code[j] = rintf((v[j] - zero) / scale);
    }
    uint32_t packed[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) packed[i] = 0;
    Unroll<32>::run([&](auto I) {
        constexpr int j = decltype(I)::value;
        put_code<BITS, j>(packed, uint32_t(fminf(fmaxf(code[j], 0.0f), kQmax)));
    });
#pragma unroll
    for (int i = 0; i < BITS; ++i) codes[h * BITS + i] = packed[i];
    if ((h & 1) == 0) {
        scale_out[h >> 1] = uint16_t(sbits);
        zero_out[h >> 1] = uint16_t(f2h(zero));
    }
}

// Dequant: a wave's 64 lanes write 64 consecutive half-groups (4 KB of
// fp16).  Each lane forms its 32 outputs (64 contiguous bytes) in LDS, and
// the wave stores them as 16-byte pieces, lane l taking bytes 16 l + 1024 c
// (c = 0..3), so that every store instruction writes one contiguous 1 KB.
template <int BITS>
__global__ __launch_bounds__(256) void minmax_dequant_kernel(const uint32_t *__restrict__ codes,
                                                             const uint16_t *__restrict__ scale_in,
                                                             const uint16_t *__restrict__ zero_in,
                                                             int64_t n_half, uint16_t *__restrict__ out) {
    __shared__ uint4 s_o[4][256];  // per wave: 4 KB
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t h0 = (int64_t(blockIdx.x) * 4 + wave) * 64;
    const int64_t h = h0 + lane;
    if (h0 >= n_half) return;  // uniform over the wave
    if (h < n_half) {
        uint32_t w[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[i] = codes[h * BITS + i];
        const float scale = h2f(scale_in[h >> 1]);
        const float zero = h2f(zero_in[h >> 1]);
        uint32_t o[16];
        Unroll<16>::run([&](auto I) {
            constexpr int p = decltype(I)::value;
            const float a = fmaf(float(code_at<BITS, 2 * p>(w)), scale, zero);
            const float b = fmaf(float(code_at<BITS, 2 * p + 1>(w)), scale, zero);
            o[p] = f2h(a) | (f2h(b) << 16);
        });
#pragma unroll
        for (int c = 0; c < 4; ++c) s_o[wave][4 * lane + c] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    uint4 *dst = reinterpret_cast<uint4 *>(out + h0 * 32);
    const int64_t n16 = (n_half - h0) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int i = lane + 64 * c;
        if (i < n16) dst[i] = s_o[wave][i];
    }
}

int launch_minmax_quant(const void *x, int64_t n, int bits, void *codes, void *scale, void *zero,
                        void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n_half = n / 32;
    const unsigned blocks = unsigned((n_half + 255) / 256);
    auto xs = static_cast<const uint16_t *>(x);
    auto cs = static_cast<uint32_t *>(codes);
    auto ss = static_cast<uint16_t *>(scale);
    auto zs = static_cast<uint16_t *>(zero);
    switch (bits) {
        case 2: hipLaunchKernelGGL(minmax_quant_kernel<2>, dim3(blocks), dim3(256), 0, s, xs, n_half, cs, ss, zs); break;
        case 3: hipLaunchKernelGGL(minmax_quant_kernel<3>, dim3(blocks), dim3(256), 0, s, xs, n_half, cs, ss, zs); break;
        case 4: hipLaunchKernelGGL(minmax_quant_kernel<4>, dim3(blocks), dim3(256), 0, s, xs, n_half, cs, ss, zs); break;
        default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}

int launch_minmax_dequant(const void *codes, const void *scale, const void *zero, int64_t n, int bits,
                          void *out, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n_half = n / 32;
    const unsigned blocks = unsigned((n_half + 255) / 256);
    auto cs = static_cast<const uint32_t *>(codes);
    auto ss = static_cast<const uint16_t *>(scale);
    auto zs = static_cast<const uint16_t *>(zero);
    auto os = static_cast<uint16_t *>(out);
    switch (bits) {
        case 2: hipLaunchKernelGGL(minmax_dequant_kernel<2>, dim3(blocks), dim3(256), 0, s, cs, ss, zs, n_half, os); break;
        case 3: hipLaunchKernelGGL(minmax_dequant_kernel<3>, dim3(blocks), dim3(256), 0, s, cs, ss, zs, n_half, os); break;
        case 4: hipLaunchKernelGGL(minmax_dequant_kernel<4>, dim3(blocks), dim3(256), 0, s, cs, ss, zs, n_half, os); break;
        default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}

}  // namespace tq
