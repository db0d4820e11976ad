// Per-token KV encode for gfx950.
//
// quidproquo.cc, "TurboQuant+ KV cache compression":
//   Stage 1 (PolarQuant): n = ||x||, random-sign Walsh-Hadamard rotation,
//   nearest Lloyd-Max level per coordinate, store indices + norm.
//   Stage 2 (QJL, K only): residual, its norm, 1 sign bit per projection.
// yeyulingfeng.com TurboQuant+ introduction, core item 3: boundary layers
// kept at q8_0 (symmetric absmax int8 per block of 32 here).
//
// Work split: one wavefront = 16 tokens.  Both dense products run on the
// MFMA units (v_mfma_f32_16x16x32_f16, columns = the 16 tokens):
//   y = H diag(D) x  with the +-1 matrix as A operand (exact in fp16; built
//   from four per-lane register patterns, see below) and the sign-flipped
//   fp16 input rows as B operand, so no conversion or butterfly is spent on
//   the rotation; lane (t, q) receives coordinates 32q + [0,32) of token t;
//   P = S e  (K only) with the rotated residual e split into hi + lo fp16
//   halves (scaled by 2^8 first so the lo half stays normal), ~22 mantissa bits.
// The norm is a packed fp16 dot product of the row with itself (fp32
// accumulation); z = y / n is quantised against the fp32 Lloyd-Max
// boundaries (bucket lookup for 3-4 bits).
// Block-32 norm storage (yeyulingfeng.com "TurboQuant+: 3.8x compression
// ...", technical highlights): lane group q holds exactly the rotated block
// q, so its norm ||y_q|| is a sum over the lane's own 32 values and
// z = sqrt(32) y / ||y_q||; K's residual enters the projection in units of
// the whole vector, scaled per block by rho_q = 2 ||y_q|| / ||y||.
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

// Destination rows of an append: input row r = b*hkv + h (one new token per
// sequence and KV head) goes to cache row r*tcap + pos[b]; a position outside
// [0, tcap) writes nothing.  Without APPEND the destination is the input row.
struct RowMap {
    const int32_t *pos;
    int hkv, tcap;
};

template <bool APPEND>
__device__ __forceinline__ int dest_row(const RowMap &m, int tok, bool &valid) {
    if constexpr (!APPEND) {
        return tok;
    } else {
        if (!valid) return 0;
        const int p = m.pos[tok / m.hkv];
        valid = p >= 0 && p < m.tcap;
        return valid ? tok * m.tcap + p : 0;
    }
}

// The encode of one packed tensor by a block of 256 threads (4 waves), the
// waves of the grid striding over 16-row tiles.
// B32: block-32 norms (norm_plane: four fp16 per row; rnorm_plane: the K
// residual norms, one fp16 per row).
template <int BITS, bool PROD, bool APPEND, bool B32 = false>
__device__ __forceinline__ void encode_rows(const DevTables *__restrict__ tab, const uint16_t *__restrict__ x,
                                            int64_t n_vec, uint8_t *__restrict__ idx_plane,
                                            uint8_t *__restrict__ sign_plane, uint8_t *__restrict__ norm_plane,
                                            int64_t n_tiles, const RowMap &map,
                                            uint8_t *__restrict__ rnorm_plane = nullptr) {
    __shared__ float s_levels[16];
    __shared__ __attribute__((aligned(16))) QBucket s_lut[kBuckets];
    __shared__ half8 s_frag[PROD ? 32 * 64 : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = lane & 15, q = lane >> 4;
    // row counts are below 2^31 (checked on the host), so 32-bit indices.
    // B operand of k-step s: input coordinates 32q + 8s + [0,8) of token t.
    // The next tile's rows are loaded while this one is processed; rows past
    // the end (and the prefetch after the last tile) read row nv - 1, whose
    // results are not stored.  The first tile's rows are in flight while the
    // tables are set up.
    const int ntl = int(n_tiles), nv = int(n_vec);
    const int stride = int(gridDim.x) * 4;
    auto load_rows = [&](int tl, half8 (&xr)[4]) {
        const int tk = min(tl * 16 + t, nv - 1);
        const uint16_t *row = x + size_t(tk) * kHeadDim + 32 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) xr[s] = *reinterpret_cast<const half8 *>(row + 8 * s);
    };
    half8 xb[4], xn[4];
    load_rows(min(int(blockIdx.x) * 4 + wave, ntl - 1), xb);
    // K works with 2^8-scaled levels (the residual is formed scaled)
    const float lscale = PROD ? 256.0f : 1.0f;
    if (tid < 16) s_levels[tid] = tab->levels[BITS - 1][tid] * lscale;
    if (tid < kBuckets) {
        QBucket qb = tab->qlut[BITS - 1][tid];
        qb.c_lo *= lscale;
        qb.c_hi *= lscale;
        s_lut[tid] = qb;
    }
    if constexpr (PROD) {
        const half8 *src = reinterpret_cast<const half8 *>(tab->S_enc);
        for (int i = tid; i < 32 * 64; i += 256) s_frag[i] = src[i];
    }
    __syncthreads();

    float bnd[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) bnd[k] = tab->bounds[BITS - 1][k];

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
    half8 pat[2][2];
    {
        const int ri = lane & 15;
        const int tau = __builtin_popcount(unsigned((ri >> 2) & q)) & 1;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int cl = (ri & 3) | (p << 2);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool neg = ((__builtin_popcount(unsigned(cl & j)) & 1) ^ tau) != 0;
                pat[p][0][j] = neg ? _Float16(-1.0f) : _Float16(1.0f);
                pat[p][1][j] = neg ? _Float16(1.0f) : _Float16(-1.0f);
            }
        }
    }
    uint32_t dmask[4][4];  // sign flips of D on the lane's fp16 pairs
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int c0 = 32 * q + 8 * s + 2 * w;
            dmask[s][w] = (tab->signs[c0] < 0.0f ? 0x8000u : 0u) | (tab->signs[c0 + 1] < 0.0f ? 0x80000000u : 0u);
        }

    for (int tile = int(blockIdx.x) * 4 + wave; tile < ntl; tile += stride) {
        const int tok = tile * 16 + t;
        bool valid = tok < nv;
        const int dst = dest_row<APPEND>(map, tok, valid);
        load_rows(min(tile + stride, ntl - 1), xn);
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
            u.x ^= dmask[s][0];
            u.y ^= dmask[s][1];
            u.z ^= dmask[s][2];
            u.w ^= dmask[s][3];
            const half8 xd = __builtin_bit_cast(half8, u);
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
                yb[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    pat[rb & 1][__builtin_popcount(unsigned((rb >> 1) & s)) & 1], xd, yb[rb], 0, 0, 0);
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
            nb = yq * kInvSqrtD;                           // ||(R x)_q||
            inv = yq > 0.0f ? 5.656854249492381f / yq : 0.0f;  // sqrt(32) / ||y_q||
            rho = yall > 0.0f ? 2.0f * yq / yall : 0.0f;
            n = yall * kInvSqrtD;                          // ||x||, for gamma
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
                for (int mb = 0; mb < 8; ++mb) sa[mb] = s_frag[(mb * 4 + s) * 64 + fl];
            }
            uint32_t bhi[4], blo[4];
            float es_prev = 0.0f;
            Unroll<8>::run([&](auto J) {
                constexpr int j = 8 * s + decltype(J)::value;
                const float z = yb[j >> 2][j & 3] * inv;  // z = H(Dx)/n = sqrt(d) R x / n
                float zhat;
                const uint32_t c = quantise<BITS>(z, bnd, s_levels, s_lut, zhat);
                put_code<BITS, j>(packed, c);
                if constexpr (PROD) {
                    const float es = B32 ? rho * fmaf(z, 256.0f, -zhat) : fmaf(z, 256.0f, -zhat);
                    se = fmaf(es, es, se);
                    if constexpr (j & 1) {
                        const half2v hi = __builtin_convertvector(float2v{es_prev, es}, half2v);
                        const half2v lo = __builtin_convertvector(
                            float2v{es_prev - float(hi[0]), es - float(hi[1])}, half2v);
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
        // the prefetched rows become the next tile's operands here, before any
        // store of this tile: loads and stores share one completion counter,
        // so waiting for them after a (possibly skipped) store would wait for
        // the stores as well
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            xb[s] = xn[s];
            asm volatile("" : "+v"(xb[s]));
        }
        if (valid) {
            uint32_t *out = reinterpret_cast<uint32_t *>(idx_plane + size_t(dst) * (16 * BITS) + q * (4 * BITS));
#pragma unroll
            for (int i = 0; i < BITS; ++i) out[i] = packed[i];
        }
        if constexpr (B32) {
            if (valid) reinterpret_cast<uint16_t *>(norm_plane)[size_t(dst) * 4 + q] = uint16_t(f2h(nb));
        }
        if constexpr (!PROD) {
            if (!B32 && valid && q == 0)
                reinterpret_cast<uint16_t *>(norm_plane)[dst] = uint16_t(f2h(n));
        } else {
            se = quad_sum(se);
            const float gamma = n * sqrtf(se) * (kInvSqrtD / 256.0f);
            // lane (t, q) now holds projections 32q + 4mb + j of token t.  Bit
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
                reinterpret_cast<uint32_t *>(sign_plane + size_t(dst) * 16)[q] = bits;
                if (q == 0) {
                    if constexpr (B32) reinterpret_cast<uint16_t *>(rnorm_plane)[dst] = uint16_t(f2h(gamma));
                    else reinterpret_cast<uint32_t *>(norm_plane)[dst] = f2h(n) | (f2h(gamma) << 16);
                }
            }
        }
    }
}

template <int BITS, bool PROD, bool APPEND, bool B32>
__global__ __launch_bounds__(256) void encode_tq_kernel(const DevTables *__restrict__ tab,
                                                        const uint16_t *__restrict__ x, int64_t n_vec,
                                                        uint8_t *__restrict__ idx_plane,
                                                        uint8_t *__restrict__ sign_plane,
                                                        uint8_t *__restrict__ norm_plane, int64_t n_tiles,
                                                        RowMap map, uint8_t *__restrict__ rnorm_plane) {
    encode_rows<BITS, PROD, APPEND, B32>(tab, x, n_vec, idx_plane, sign_plane, norm_plane, n_tiles, map,
                                         rnorm_plane);
}

// K (Stage 1 + QJL) and V (Stage 1) rows in a single launch, for encodes
// small enough that one launch each would leave most of the GPU idle (a
// decode step's append, short prompts): blocks with blockIdx.y = 0 encode the
// K rows, = 1 the V rows.
struct PairPlanes {
    const uint16_t *x;
    uint8_t *idx, *sign, *norm;
};

template <int KB, int VB, bool APPEND>
__global__ __launch_bounds__(256) void encode_pair_kernel(const DevTables *__restrict__ tab, int64_t n_vec,
                                                          int64_t n_tiles, PairPlanes k, PairPlanes v,
                                                          RowMap map) {
    if (blockIdx.y == 0)
        encode_rows<KB, true, APPEND>(tab, k.x, n_vec, k.idx, k.sign, k.norm, n_tiles, map);
    else
        encode_rows<VB, false, APPEND>(tab, v.x, n_vec, v.idx, nullptr, v.norm, n_tiles, map);
}

// q8 boundary blocks: four consecutive lanes share a token, lane l taking
// block (l & 3) of 32 elements.
template <bool APPEND>
__global__ __launch_bounds__(256) void encode_q8_kernel(const uint16_t *__restrict__ x, int64_t n_vec,
                                                        int8_t *__restrict__ qplane,
                                                        uint16_t *__restrict__ scale_plane, RowMap map) {
    const int64_t gl = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t tok = gl >> 2;
    const int blk = int(gl & 3);
    if (tok >= n_vec) return;
    bool valid = true;
    const int64_t dst = dest_row<APPEND>(map, int(tok), valid);
    if (!valid) return;
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
    uint4 *qd = reinterpret_cast<uint4 *>(qplane + dst * kHeadDim + 32 * blk);
    qd[0] = make_uint4(out[0], out[1], out[2], out[3]);
    qd[1] = make_uint4(out[4], out[5], out[6], out[7]);
    scale_plane[dst * 4 + blk] = uint16_t(sbits);
}

template <int BITS, bool PROD, bool APPEND, bool B32 = false>
static int launch_tq(const DevTables *tab, const uint16_t *x, int64_t n_vec, uint8_t *base,
                     const tq_planes_desc &lay, const RowMap &map, hipStream_t s) {
    const int64_t n_tiles = (n_vec + 15) / 16;
    // persistent blocks amortise the 32 KB of S fragments (K) in LDS: as many
    // as are resident at once, each wave striding over the tiles
    static int cache[kMaxDevices];
    const int64_t blocks =
        persistent_grid(n_tiles, resident_blocks(encode_tq_kernel<BITS, PROD, APPEND, B32>, 256, cache));
    // block-32 K: the residual norms follow the block norms of every row of
    // the packed tensor (lay.norm_bytes = rows * 10)
    uint8_t *rnorm = B32 && PROD ? base + lay.norm_offset + lay.norm_bytes / 10 * 8 : nullptr;
    hipLaunchKernelGGL((encode_tq_kernel<BITS, PROD, APPEND, B32>), dim3(unsigned(blocks)), dim3(256), 0, s, tab,
                       x, n_vec, base + lay.idx_offset, PROD ? base + lay.sign_offset : nullptr,
                       base + lay.norm_offset, n_tiles, map, rnorm);
    return int(hipGetLastError());
}

template <bool APPEND>
static int launch_format(const DevTables *tab, const uint16_t *x, int64_t n_vec, tq_format f, uint8_t *base,
                         const tq_planes_desc &lay, const RowMap &map, hipStream_t s) {
    if (f.kind == TQ_KIND_Q8) {
        const int64_t threads = n_vec * 4;
        const int64_t blocks = (threads + 255) / 256;
        hipLaunchKernelGGL(encode_q8_kernel<APPEND>, dim3(unsigned(blocks)), dim3(256), 0, s, x, n_vec,
                           reinterpret_cast<int8_t *>(base + lay.idx_offset),
                           reinterpret_cast<uint16_t *>(base + lay.norm_offset), map);
        return int(hipGetLastError());
    }
    if (f.kind == TQ_KIND_PROD32) {
        switch (f.bits) {
            case 1: return launch_tq<1, true, APPEND, true>(tab, x, n_vec, base, lay, map, s);
            case 2: return launch_tq<2, true, APPEND, true>(tab, x, n_vec, base, lay, map, s);
            case 3: return launch_tq<3, true, APPEND, true>(tab, x, n_vec, base, lay, map, s);
        }
        return int(hipErrorInvalidValue);
    }
    if (f.kind == TQ_KIND_MSE32) {
        switch (f.bits) {
            case 1: return launch_tq<1, false, APPEND, true>(tab, x, n_vec, base, lay, map, s);
            case 2: return launch_tq<2, false, APPEND, true>(tab, x, n_vec, base, lay, map, s);
            case 3: return launch_tq<3, false, APPEND, true>(tab, x, n_vec, base, lay, map, s);
            case 4: return launch_tq<4, false, APPEND, true>(tab, x, n_vec, base, lay, map, s);
        }
        return int(hipErrorInvalidValue);
    }
    if (f.kind == TQ_KIND_PROD) {
        switch (f.bits) {
            case 1: return launch_tq<1, true, APPEND>(tab, x, n_vec, base, lay, map, s);
            case 2: return launch_tq<2, true, APPEND>(tab, x, n_vec, base, lay, map, s);
            case 3: return launch_tq<3, true, APPEND>(tab, x, n_vec, base, lay, map, s);
        }
    } else {
        switch (f.bits) {
            case 1: return launch_tq<1, false, APPEND>(tab, x, n_vec, base, lay, map, s);
            case 2: return launch_tq<2, false, APPEND>(tab, x, n_vec, base, lay, map, s);
            case 3: return launch_tq<3, false, APPEND>(tab, x, n_vec, base, lay, map, s);
            case 4: return launch_tq<4, false, APPEND>(tab, x, n_vec, base, lay, map, s);
        }
    }
    return int(hipErrorInvalidValue);
}

int launch_encode(const DevTables *tab, const void *xv, int64_t n_vec, tq_format f, void *packed,
                  const tq_planes_desc &lay, void *stream) {
    return launch_format<false>(tab, static_cast<const uint16_t *>(xv), n_vec, f, static_cast<uint8_t *>(packed),
                                lay, RowMap{nullptr, 1, 1}, static_cast<hipStream_t>(stream));
}

// Returns kPairDeclined (nothing launched) when the encode is too large for
// one joint launch: each of K and V then gets a full persistent grid.
template <int KB, int VB, bool APPEND>
static int launch_pair(const DevTables *tab, int64_t n_vec, const PairPlanes &k, const PairPlanes &v,
                       const RowMap &map, hipStream_t s) {
    const int64_t n_tiles = (n_vec + 15) / 16;
    static int cache[kMaxDevices];
    const int resident = resident_blocks(encode_pair_kernel<KB, VB, APPEND>, 256, cache);
    // one tile per wave and both halves of the grid resident at once
    if (n_tiles > int64_t(resident) * 2) return kPairDeclined;
    const int64_t blocks = (n_tiles + 3) / 4;
    hipLaunchKernelGGL((encode_pair_kernel<KB, VB, APPEND>), dim3(unsigned(blocks), 2), dim3(256), 0, s, tab, n_vec,
                       n_tiles, k, v, map);
    return int(hipGetLastError());
}

template <int KB, bool APPEND>
static int dispatch_pair_v(const DevTables *tab, int64_t n_vec, int vbits, const PairPlanes &k,
                           const PairPlanes &v, const RowMap &map, hipStream_t s) {
    switch (vbits) {
        case 1: return launch_pair<KB, 1, APPEND>(tab, n_vec, k, v, map, s);
        case 2: return launch_pair<KB, 2, APPEND>(tab, n_vec, k, v, map, s);
        case 3: return launch_pair<KB, 3, APPEND>(tab, n_vec, k, v, map, s);
        case 4: return launch_pair<KB, 4, APPEND>(tab, n_vec, k, v, map, s);
    }
    return int(hipErrorInvalidValue);
}

template <bool APPEND>
static int dispatch_pair(const DevTables *tab, const void *k, const void *v, int64_t n_vec, tq_format kf,
                         tq_format vf, void *kp, void *vp, const tq_planes_desc &kl, const tq_planes_desc &vl,
                         const RowMap &map, void *stream) {
    if (kf.kind != TQ_KIND_PROD || vf.kind != TQ_KIND_MSE) return kPairDeclined;
    uint8_t *kb = static_cast<uint8_t *>(kp), *vb = static_cast<uint8_t *>(vp);
    const PairPlanes ka{static_cast<const uint16_t *>(k), kb + kl.idx_offset, kb + kl.sign_offset,
                        kb + kl.norm_offset};
    const PairPlanes va{static_cast<const uint16_t *>(v), vb + vl.idx_offset, nullptr, vb + vl.norm_offset};
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kf.bits) {
        case 1: return dispatch_pair_v<1, APPEND>(tab, n_vec, vf.bits, ka, va, map, s);
        case 2: return dispatch_pair_v<2, APPEND>(tab, n_vec, vf.bits, ka, va, map, s);
        case 3: return dispatch_pair_v<3, APPEND>(tab, n_vec, vf.bits, ka, va, map, s);
    }
    return int(hipErrorInvalidValue);
}

int launch_encode_pair(const DevTables *tab, const void *k, const void *v, int64_t n_vec, tq_format kf,
                       tq_format vf, void *kp, void *vp, const tq_planes_desc &kl, const tq_planes_desc &vl,
                       void *stream) {
    return dispatch_pair<false>(tab, k, v, n_vec, kf, vf, kp, vp, kl, vl, RowMap{nullptr, 1, 1}, stream);
}

int launch_append_kv(const DevTables *tab, const void *k, const void *v, int B, int hkv, int tcap,
                     const int32_t *pos, tq_format kf, tq_format vf, void *kp, void *vp,
                     const tq_planes_desc &kl, const tq_planes_desc &vl, void *stream) {
    return dispatch_pair<true>(tab, k, v, int64_t(B) * hkv, kf, vf, kp, vp, kl, vl, RowMap{pos, hkv, tcap},
                               stream);
}

int launch_append(const DevTables *tab, const void *xv, int B, int hkv, int tcap, const int32_t *pos,
                  tq_format f, void *packed, const tq_planes_desc &lay, void *stream) {
    return launch_format<true>(tab, static_cast<const uint16_t *>(xv), int64_t(B) * hkv, f,
                               static_cast<uint8_t *>(packed), lay, RowMap{pos, hkv, tcap},
                               static_cast<hipStream_t>(stream));
}

}  // namespace tq
