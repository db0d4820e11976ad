// Per-token KV encode for gfx950.
//
// quidproquo.cc, "TurboQuant+ KV cache compression":
//   Stage 1 (PolarQuant): n = ||x||, random-sign Walsh-Hadamard rotation,
//   nearest Lloyd-Max level per coordinate, store indices + norm.
//   Stage 2 (QJL, K only): residual, its norm, 1 sign bit per projection.
// yeyulingfeng.com TurboQuant+ introduction, core item 3: boundary layers
// kept at q8_0 (symmetric absmax int8 per block of 32 here).
//
// Work split: one wavefront = 16 tokens, lane l owns token l&15.  A lane
// loads the 32 coordinates 8*(l>>4) + [0,8) + 32k (k = 0..3), runs the five
// in-register butterfly stages, then two permlane-swap stages that finish the
// 128-point transform and leave it holding coordinates 32*(l>>4) + [0,32).
// The standardised coordinates z = H (D x) / n are quantised against the fp32
// Lloyd-Max boundaries (bucket lookup for 3-4 bits).  For K the rotated
// residual e = z - c[idx] is projected on the MFMA units: P = S e for the 16
// tokens of the wave as a [128 x 128] x [128 x 16] fp16 product with fp32
// accumulation, e split into hi + lo fp16 halves (scaled by 2^8 first so the
// lo half stays normal) so that the product keeps ~22 mantissa bits.
#include <type_traits>

#include "device_common.h"

namespace tq {

constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

// idx = #{t_k <= z} and the level c[idx].  1 bit: sign test; 2 bits: three
// compares; 3-4 bits: one bucket lookup (base + one compare) from LDS.
template <int BITS>
__device__ __forceinline__ uint32_t quantise(float z, const float *bnd, const float *s_levels,
                                             const QBucket *s_lut, float &zhat) {
    if constexpr (BITS == 1) {
        const bool up = z >= 0.0f;
        zhat = up ? s_levels[1] : s_levels[0];
        return up ? 1u : 0u;
    } else if constexpr (BITS == 2) {
        const uint32_t c = (z >= bnd[0] ? 1u : 0u) + (z >= bnd[1] ? 1u : 0u) + (z >= bnd[2] ? 1u : 0u);
        zhat = s_levels[c];
        return c;
    } else {
        int j = int(fmaf(z, 4.0f, 12.5f));
        j = j < 0 ? 0 : (j > kBuckets - 1 ? kBuckets - 1 : j);
        const QBucket qb = s_lut[j];
        const bool up = z >= qb.thr;
        zhat = up ? qb.c_hi : qb.c_lo;
        return qb.base + (up ? 1u : 0u);
    }
}

template <int BITS, bool PROD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void encode_tq_kernel(const DevTables *__restrict__ tab, const uint16_t *__restrict__ x, int64_t n_vec,
                      uint8_t *__restrict__ idx_plane, uint8_t *__restrict__ sign_plane,
                      uint8_t *__restrict__ norm_plane, int64_t n_tiles) {
    __shared__ float s_levels[16];
    __shared__ QBucket s_lut[kBuckets];
    __shared__ half8 s_frag[PROD ? 32 * 64 : 1];
    __shared__ uint4 s_sx[4][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < 16) s_levels[tid] = tab->levels[BITS - 1][tid];
    if (tid < kBuckets) s_lut[tid] = tab->qlut[BITS - 1][tid];
    if (tid < 16) s_sx[tid >> 2][tid & 3] = reinterpret_cast<const uint4 *>(tab->sign_pair_xor)[tid];
    if constexpr (PROD) {
        const half8 *src = reinterpret_cast<const half8 *>(tab->S_enc);
        for (int i = tid; i < 32 * 64; i += 256) s_frag[i] = src[i];
    }
    __syncthreads();

    const int t = lane & 15, q = lane >> 4;
    float bnd[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) bnd[k] = tab->bounds[BITS - 1][k];

    // row counts are below 2^31 (checked on the host), so 32-bit indices
    const int ntl = int(n_tiles), nv = int(n_vec);
    for (int tile = int(blockIdx.x) * 4 + wave; tile < ntl; tile += int(gridDim.x) * 4) {
        const int tok = tile * 16 + t;
        const bool valid = tok < nv;
        // load layout A: register r holds coordinate 8q + (r&7) + 32(r>>3)
        uint32_t w[16];
        if (valid) {
            const uint16_t *row = x + size_t(tok) * kHeadDim + 8 * q;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 u = *reinterpret_cast<const uint4 *>(row + 32 * k);
                w[4 * k + 0] = u.x; w[4 * k + 1] = u.y; w[4 * k + 2] = u.z; w[4 * k + 3] = u.w;
            }
        } else {
#pragma unroll
            for (int p = 0; p < 16; ++p) w[p] = 0;
        }
        uint32_t sx[16];  // sign flips of D for this lane's coordinates (LDS, per tile)
        {
            int qq = q;
            asm volatile("" : "+v"(qq));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 u = s_sx[qq][k];
                sx[4 * k] = u.x; sx[4 * k + 1] = u.y; sx[4 * k + 2] = u.z; sx[4 * k + 3] = u.w;
            }
        }
        float v[32];
        float ss = 0.0f;
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const uint32_t sgn = w[p] ^ sx[p];  // D x on the packed fp16 pair
            v[2 * p] = h2f(sgn & 0xFFFFu);
            v[2 * p + 1] = h2f(sgn >> 16);
            ss = fmaf(v[2 * p], v[2 * p], ss);
            ss = fmaf(v[2 * p + 1], v[2 * p + 1], ss);
        }
        ss = quad_sum(ss);
        const float n = sqrtf(ss);
        fwht128_swap(v);  // now lane q holds coordinates 32q + r
        const float inv = n > 0.0f ? 1.0f / n : 0.0f;
        uint32_t packed[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) packed[i] = 0;
        // K: residual e = z - c[idx], scaled by 2^8 so that its fp16 lo half
        // stays normal, split into the hi/lo MFMA operands as it is produced
        half8 bhi[PROD ? 4 : 1], blo[PROD ? 4 : 1];
        float se = 0.0f;
        Unroll<32>::run([&](auto J) {
            constexpr int j = decltype(J)::value;
            const float z = v[j] * inv;  // z = H(Dx)/n = sqrt(d) R x / n
            float zhat;
            const uint32_t c = quantise<BITS>(z, bnd, s_levels, s_lut, zhat);
            put_code<BITS, j>(packed, c);
            if constexpr (PROD) {
                const float e = z - zhat;
                se = fmaf(e, e, se);
                const float es = e * 256.0f;
                const _Float16 hi = _Float16(es);
                bhi[j >> 3][j & 7] = hi;
                blo[j >> 3][j & 7] = _Float16(es - float(hi));
            }
        });
        if (valid) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(idx_plane + size_t(tok) * (16 * BITS) + q * (4 * BITS));
#pragma unroll
            for (int i = 0; i < BITS; ++i) dst[i] = packed[i];
        }
        if constexpr (!PROD) {
            if (valid && q == 0)
                reinterpret_cast<uint16_t *>(norm_plane)[tok] = uint16_t(f2h(n));
        } else {
            se = quad_sum(se);
            const float gamma = n * sqrtf(se) * kInvSqrtD;
            floatx4 acc[8];
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) acc[mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
            // read the S fragments from LDS at their use: an opaque index keeps
            // the compiler from hoisting all 32 of them out of the tile loop
            int fl = lane;
            asm volatile("" : "+v"(fl));
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) {
                    const half8 a = s_frag[(mb * 4 + s) * 64 + fl];
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bhi[s], acc[mb], 0, 0, 0);
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, blo[s], acc[mb], 0, 0, 0);
                }
            }
            // lane (t, q) now holds projections 32q + 4mb + j of token t
            uint32_t bits = 0;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int j = 0; j < 4; ++j) bits |= (acc[mb][j] > 0.0f ? 1u : 0u) << (4 * mb + j);
            if (valid) {
                reinterpret_cast<uint32_t *>(sign_plane + size_t(tok) * 16)[q] = bits;
                if (q == 0)
                    reinterpret_cast<uint32_t *>(norm_plane)[tok] = f2h(n) | (f2h(gamma) << 16);
            }
        }
    }
}

// q8 boundary blocks: lane l owns token l&15, block (l>>4) of 32 elements.
__global__ __launch_bounds__(256) void encode_q8_kernel(const uint16_t *__restrict__ x, int64_t n_vec,
                                                        int8_t *__restrict__ qplane,
                                                        uint16_t *__restrict__ scale_plane) {
    const int64_t gl = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t tok = gl >> 2;
    const int blk = int(gl & 3);
    if (tok >= n_vec) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + tok * kHeadDim + 32 * blk);
    float v[32];
    float amax = 0.0f;
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
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    // scale = fp16(max|x| / 127): the quotient is formed in float64 and rounded once
    const uint32_t sbits = double_to_half_bits(double(amax) / 127.0);
    const float scale = h2f(sbits);
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        float r = scale > 0.0f ? rintf(v[j] / scale) : 0.0f;
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        out[j >> 2] |= (uint32_t(int32_t(r)) & 0xFFu) << (8 * (j & 3));
    }
    uint4 *dst = reinterpret_cast<uint4 *>(qplane + tok * kHeadDim + 32 * blk);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    scale_plane[tok * 4 + blk] = uint16_t(sbits);
}

template <int BITS, bool PROD>
static int launch_tq(const DevTables *tab, const uint16_t *x, int64_t n_vec, uint8_t *base,
                     const tq_planes_desc &lay, hipStream_t s) {
    const int64_t n_tiles = (n_vec + 15) / 16;
    int64_t blocks = (n_tiles + 3) / 4;
    if (PROD && blocks > 1024) blocks = 1024;  // amortise the 32 KB fragment load
    if (blocks > (int64_t(1) << 30)) blocks = int64_t(1) << 30;
    hipLaunchKernelGGL((encode_tq_kernel<BITS, PROD>), dim3(unsigned(blocks)), dim3(256), 0, s, tab, x,
                       n_vec, base + lay.idx_offset, PROD ? base + lay.sign_offset : nullptr,
                       base + lay.norm_offset, n_tiles);
    return int(hipGetLastError());
}

int launch_encode(const DevTables *tab, const void *xv, int64_t n_vec, tq_format f, void *packed,
                  const tq_planes_desc &lay, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t *x = static_cast<const uint16_t *>(xv);
    uint8_t *base = static_cast<uint8_t *>(packed);
    if (f.kind == TQ_KIND_Q8) {
        const int64_t threads = n_vec * 4;
        const int64_t blocks = (threads + 255) / 256;
        hipLaunchKernelGGL(encode_q8_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, x, n_vec,
                           reinterpret_cast<int8_t *>(base + lay.idx_offset),
                           reinterpret_cast<uint16_t *>(base + lay.norm_offset));
        return int(hipGetLastError());
    }
    if (f.kind == TQ_KIND_PROD) {
        switch (f.bits) {
            case 1: return launch_tq<1, true>(tab, x, n_vec, base, lay, s);
            case 2: return launch_tq<2, true>(tab, x, n_vec, base, lay, s);
            case 3: return launch_tq<3, true>(tab, x, n_vec, base, lay, s);
        }
    } else {
        switch (f.bits) {
            case 1: return launch_tq<1, false>(tab, x, n_vec, base, lay, s);
            case 2: return launch_tq<2, false>(tab, x, n_vec, base, lay, s);
            case 3: return launch_tq<3, false>(tab, x, n_vec, base, lay, s);
            case 4: return launch_tq<4, false>(tab, x, n_vec, base, lay, s);
        }
    }
    return int(hipErrorInvalidValue);
}

}  // namespace tq
