// The per-tile TurboQuant encode (gfx950), shared by the encode kernels and
// by the attention kernels that append a decode step's new token.
//
// quidproquo.cc, "TurboQuant+ KV cache compression":
//   Stage 1 (PolarQuant): n = ||x||, random-sign Walsh-Hadamard rotation,
//   nearest Lloyd-Max level per coordinate, store indices + norm.
//   Stage 2 (QJL, K only): residual, its norm, 1 sign bit per projection.
//
// One wavefront encodes a tile of 16 rows.  Both dense products run on the
// MFMA units (v_mfma_f32_16x16x32_f16, columns = the 16 rows):
//   y = H diag(D) x  with the +-1 matrix as A operand (exact in fp16; built
//   from four per-lane register patterns, see encode_lane) and the
//   sign-flipped fp16 input rows as B operand; lane (t, q) receives
//   coordinates 32q + [0,32) of row t;
//   P = S e  (K only) with the rotated residual e split into hi + lo fp16
//   halves (scaled by 2^8 first so the lo half stays normal), ~22 mantissa bits.
// The norm is a packed fp16 dot product of the row with itself (fp32
// accumulation); z = y / n is quantised against the fp32 Lloyd-Max
// boundaries (bucket lookup for 3-4 bits).  Every caller runs this same
// code, so a row gets the same bytes whichever kernel encodes it.
// Block-32 norm storage (yeyulingfeng.com "TurboQuant+: 3.8x compression
// ...", technical highlights): lane group q holds exactly the rotated block
// q, so its norm ||y_q|| is a sum over the lane's own 32 values and
// z = sqrt(32) y / ||y_q||; K's residual enters the projection in units of
// the whole vector, scaled per block by rho_q = 2 ||y_q|| / ||y||.
#pragma once

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
        // bucket floor(4 z + 48.5): 4 z + 48 + 1.5 * 2^23 rounded to an integer
        // (a tie lands in either neighbour, both give the same index) leaves
        // the bucket number in the low mantissa bits; |z| <= 12.125 always
        const uint32_t j = __float_as_uint(fmaf(z, 4.0f, 12582960.0f)) - 0x4B400000u;
        const uint4 qb = reinterpret_cast<const uint4 *>(s_lut)[j];  // {thr, base, c_lo, c_hi}
        const bool up = z >= __uint_as_float(qb.x);
        zhat = __uint_as_float(up ? qb.w : qb.z);
        return qb.y + (up ? 1u : 0u);
    }
}

// Quantiser tables of one format in LDS; K (PROD) works with 2^8-scaled
// levels, because its residual is formed scaled.
struct EncodeTables {
    float levels[16];
    __attribute__((aligned(16))) QBucket lut[kBuckets];
};

// Thread i of n fills entries i, i + n, ... (a barrier must follow).
template <int BITS, bool PROD>
__device__ __forceinline__ void fill_encode_tables(const DevTables *__restrict__ tab, EncodeTables *t, int i,
                                                   int n) {
    const float lscale = PROD ? 256.0f : 1.0f;
    for (int e = i; e < 16 + kBuckets; e += n) {
        if (e < 16) {
            t->levels[e] = tab->levels[BITS - 1][e] * lscale;
        } else {
            QBucket qb = tab->qlut[BITS - 1][e - 16];
            qb.c_lo *= lscale;
            qb.c_hi *= lscale;
            t->lut[e - 16] = qb;
        }
    }
}

// Per-lane constants of the tile encode.
struct EncodeLane {
    half8 pat[2][2];       // the four +-1 A operands of the rotation
    uint32_t dmask[4][4];  // sign flips of D on the lane's fp16 pairs
    float bnd[3];          // the first three boundaries (2-bit quantiser)
};

// Rotation operands.  k-step s of lane group q carries input coordinates
// k = 32q + 8s + j (j = 0..7); MFMA row i of block rb is output coordinate
// c = 32(i>>2) + 4rb + (i&3), so lane group q receives c = 32q + [0,32).
// Sylvester H[c][k] = (-1)^popcount(c & k) then factors as
//   (-1)^popcount(((i&3) | (rb&1)<<2) & j) * (-1)^popcount((rb>>1) & s)
//   * (-1)^popcount((i>>2) & q):
// an 8-entry pattern chosen by rb&1, a sign fixed by (rb, s) at compile
// time and a sign fixed per lane, so every A operand is one of four
// register constants (pat[rb&1][sign]).  D is applied to the fp16 inputs
// by flipping their sign bits (dmask).
template <int BITS>
__device__ __forceinline__ void encode_lane(const DevTables *__restrict__ tab, int lane, EncodeLane &el) {
    const int q = lane >> 4;
#pragma unroll
    for (int k = 0; k < 3; ++k) el.bnd[k] = tab->bounds[BITS - 1][k];
    const int ri = lane & 15;
    const int tau = __builtin_popcount(unsigned((ri >> 2) & q)) & 1;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int cl = (ri & 3) | (p << 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool neg = ((__builtin_popcount(unsigned(cl & j)) & 1) ^ tau) != 0;
            el.pat[p][0][j] = neg ? _Float16(-1.0f) : _Float16(1.0f);
            el.pat[p][1][j] = neg ? _Float16(1.0f) : _Float16(-1.0f);
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int c0 = 32 * q + 8 * s + 2 * w;
            el.dmask[s][w] =
                (tab->signs[c0] < 0.0f ? 0x8000u : 0u) | (tab->signs[c0 + 1] < 0.0f ? 0x80000000u : 0u);
        }
}

// Output planes of one packed tensor.  B32: norm holds four fp16 block norms
// per row and rnorm the K residual norms (one fp16 per row).
struct EncodePlanes {
    uint8_t *idx, *sign, *norm, *rnorm;
};

// Encodes the tile whose rows lane (t, q) holds in xb (input coordinates
// 32q + 8s + [0,8) of row t in xb[s]); the row of lane t is stored at
// destination row dst when `valid`.  frag(i) returns S fragment i (K only).
// before_store() runs after the arithmetic and before the first store
// (callers take delivery of prefetched rows there: loads and stores share one
// completion counter).
template <int BITS, bool PROD, bool B32, typename Frag, typename BeforeStore>
__device__ __forceinline__ void encode_tile(const half8 (&xb)[4], const EncodeLane &el, const float *s_levels,
                                            const QBucket *s_lut, Frag frag, int lane, bool valid, int dst,
                                            const EncodePlanes &pl, BeforeStore before_store) {
    const int q = lane >> 4;
    // n^2: packed fp16 products, fp32 accumulation, then over the 4 lanes
    float ss = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const half2v h = half2v{xb[s][2 * p], xb[s][2 * p + 1]};
            ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        }
    ss = quad_sum(ss);
    float n = sqrtf(ss);
    float inv = n > 0.0f ? 1.0f / n : 0.0f;
    // y = H D x; lane (t, q) ends with coordinates 32q + 4rb + j in yb[rb][j]
    floatx4 yb[8];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) yb[rb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint4 u = __builtin_bit_cast(uint4, xb[s]);
        u.x ^= el.dmask[s][0];
        u.y ^= el.dmask[s][1];
        u.z ^= el.dmask[s][2];
        u.w ^= el.dmask[s][3];
        const half8 xd = __builtin_bit_cast(half8, u);
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
            yb[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                el.pat[rb & 1][__builtin_popcount(unsigned((rb >> 1) & s)) & 1], xd, yb[rb], 0, 0, 0);
    }
    // block-32: this lane's block norm from its rotated values
    float rho = 1.0f, nb = 0.0f;
    if constexpr (B32) {
        float sb = 0.0f;
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
            for (int j = 0; j < 4; ++j) sb = fmaf(yb[rb][j], yb[rb][j], sb);
        const float yq = sqrtf(sb), yall = sqrtf(quad_sum(sb));
        nb = yq * kInvSqrtD;                               // ||(R x)_q||
        inv = yq > 0.0f ? 5.656854249492381f / yq : 0.0f;  // sqrt(32) / ||y_q||
        rho = yall > 0.0f ? 2.0f * yq / yall : 0.0f;
        n = yall * kInvSqrtD;                              // ||x||, for gamma
    }
    uint32_t packed[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) packed[i] = 0;
    // K: residual e = z - c[idx], scaled by 2^8 so that its fp16 lo half
    // stays normal (levels in s_levels / s_lut are pre-scaled by 2^8 for
    // K), split into the hi/lo MFMA operands a pair at a time.  The
    // coordinates of QJL k-step s (32q + 8s + [0,8), i.e. yb[2s], yb[2s+1])
    // are quantised together and their 16 products issued right away, so
    // only one k-step's operands are live and the matrix work overlaps the
    // quantiser of the next k-step.
    float se = 0.0f;  // sum of (2^8 e)^2
    floatx4 acc[PROD ? 8 : 1];
#pragma unroll
    for (int mb = 0; mb < (PROD ? 8 : 1); ++mb) acc[mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    int fl = lane;
    asm volatile("" : "+v"(fl));
    Unroll<4>::run([&](auto S) {
        constexpr int s = decltype(S)::value;
        // this k-step's S fragments are requested first and land while its
        // coordinates are quantised; nothing moves across k-steps
        __builtin_amdgcn_sched_barrier(0);
        half8 sa[PROD ? 8 : 1];
        if constexpr (PROD) {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) sa[mb] = frag((mb * 4 + s) * 64 + fl);
        }
        uint32_t bhi[4], blo[4];
        float es_prev = 0.0f;
        Unroll<8>::run([&](auto J) {
            constexpr int j = 8 * s + decltype(J)::value;
            const float z = yb[j >> 2][j & 3] * inv;  // z = H(Dx)/n = sqrt(d) R x / n
            float zhat;
            const uint32_t c = quantise<BITS>(z, el.bnd, s_levels, s_lut, zhat);
            put_code<BITS, j>(packed, c);
            if constexpr (PROD) {
                const float es = B32 ? rho * fmaf(z, 256.0f, -zhat) : fmaf(z, 256.0f, -zhat);
                se = fmaf(es, es, se);
                if constexpr (j & 1) {
                    const half2v hi = __builtin_convertvector(float2v{es_prev, es}, half2v);
                    const half2v lo =
                        __builtin_convertvector(float2v{es_prev - float(hi[0]), es - float(hi[1])}, half2v);
                    bhi[(j >> 1) & 3] = __builtin_bit_cast(uint32_t, hi);
                    blo[(j >> 1) & 3] = __builtin_bit_cast(uint32_t, lo);
                } else {
                    es_prev = es;
                }
            }
        });
        if constexpr (PROD) {
            const half8 bh = __builtin_bit_cast(half8, make_uint4(bhi[0], bhi[1], bhi[2], bhi[3]));
            const half8 bl = __builtin_bit_cast(half8, make_uint4(blo[0], blo[1], blo[2], blo[3]));
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa[mb], bh, acc[mb], 0, 0, 0);
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa[mb], bl, acc[mb], 0, 0, 0);
            }
        }
    });
    before_store();
    if (valid) {
        uint32_t *out = reinterpret_cast<uint32_t *>(pl.idx + size_t(dst) * (16 * BITS) + q * (4 * BITS));
#pragma unroll
        for (int i = 0; i < BITS; ++i) out[i] = packed[i];
    }
    if constexpr (B32) {
        if (valid) reinterpret_cast<uint16_t *>(pl.norm)[size_t(dst) * 4 + q] = uint16_t(f2h(nb));
    }
    if constexpr (!PROD) {
        if (!B32 && valid && q == 0) reinterpret_cast<uint16_t *>(pl.norm)[dst] = uint16_t(f2h(n));
    } else {
        se = quad_sum(se);
        const float gamma = n * sqrtf(se) * (kInvSqrtD / 256.0f);
        // lane (t, q) now holds projections 32q + 4mb + j of row t.  Bit
        // (4mb + j) = [P > 0]: shift the sign bits in from the top, from
        // projection 31 down to 0, then invert; a zero residual (all P = 0)
        // gives no set bit.
        uint32_t neg = 0;
#pragma unroll
        for (int mb = 7; mb >= 0; --mb)
#pragma unroll
            for (int j = 3; j >= 0; --j) neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(acc[mb][j]), 31);
        const uint32_t bits = se > 0.0f ? ~neg : 0u;
        if (valid) {
            reinterpret_cast<uint32_t *>(pl.sign + size_t(dst) * 16)[q] = bits;
            if (q == 0) {
                if constexpr (B32) reinterpret_cast<uint16_t *>(pl.rnorm)[dst] = uint16_t(f2h(gamma));
                else reinterpret_cast<uint32_t *>(pl.norm)[dst] = f2h(n) | (f2h(gamma) << 16);
            }
        }
    }
}

// One decode step's new token: the K row (Stage 1 + QJL, KB bits) or the V
// row (Stage 1, VB bits) of input row `in_row` encoded by one wavefront into
// cache row `dst` with exactly the arithmetic of the encode kernels.  All
// 16 columns of the tile carry the same row; column 0 stores it.  `t` must
// hold this format's tables (fill_encode_tables, then a barrier); the S
// fragments are read from global memory.
template <int BITS, bool PROD>
__device__ __forceinline__ void encode_new_row(const DevTables *__restrict__ tab, const EncodeTables *t,
                                               const uint16_t *__restrict__ x, int in_row, int dst,
                                               const EncodePlanes &pl, int lane) {
    const int q = lane >> 4;
    half8 xb[4];
    const uint16_t *row = x + size_t(in_row) * kHeadDim + 32 * q;
#pragma unroll
    for (int s = 0; s < 4; ++s) xb[s] = *reinterpret_cast<const half8 *>(row + 8 * s);
    EncodeLane el;
    encode_lane<BITS>(tab, lane, el);
    const half8 *fr = reinterpret_cast<const half8 *>(tab->S_enc);
    encode_tile<BITS, PROD, false>(
        xb, el, t->levels, t->lut, [&](int i) { return fr[i]; }, lane, (lane & 15) == 0, dst, pl, [] {});
}

}  // namespace tq
