// Device code shared by the attention kernels (gfx950): kernel arguments,
// row mapping of decode and prefill, lane exchanges, the 128-point FWHT
// across a wavefront, the query operands of the scores MFMAs and the K tile
// loads.  Included by attn.hip (two-pass kernels) and attn_fused.hip.
#pragma once

#include <algorithm>
#include <type_traits>

#include "encode_common.h"

namespace tq {

constexpr float kRsqrtD = 0.08838834764831845f;  // 1/sqrt(128)
constexpr float kQjlOverSqrtD = 1.2533141373155003f / 128.0f * 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSliceTiles = 4;            // 16-token tiles per wave and slice
constexpr int kSlice = 64 * kSliceTiles;  // tokens per slice of the scores pass (4 waves)
constexpr int kVThreads = 512;            // threads per values block
constexpr int kVWaves = kVThreads / 64;

struct AttnArgs {
    const DevTables *tab;
    const uint16_t *q;
    const uint8_t *kidx, *ksign, *knorm;  // K planes
    const uint8_t *vidx, *vnorm;          // V planes
    const int32_t *seq_lens;
    float *scores, *stats;
    float *out;
    float tau;
    int B, Hq, Hkv, T, chunk, n_chunks;
    int ld_scores;  // score row stride (floats)
    int vsub;       // tokens per block of the MFMA values pass (multiple of 32)
    // Prefill: tq queries per sequence, taken qp at a time.  Virtual sequence
    // b holds queries qp * (b % (tq / qp)) + [0, qp) of sequence b / (tq / qp);
    // its G = qg * qp rows are those queries' qg heads of one kv head (query
    // u = row / qg, head row % qg), so the queries share every K load.  Hq is
    // the virtual head count (real heads x qp), hq_io the real one.  Decode:
    // tq = qp = 1.
    int tq, qp, qg, hq_io;
    int k_rotated;  // K codec works in the rotated domain
    int v_rotated;  // V codec works in the rotated domain
    // single-launch path: nblk blocks of tb tokens per (sequence, kv head)
    // row; a departure counter per row at sync, and stats holds one 64-bit
    // (max, sum) slot per block and head
    uint32_t *sync;
    int nblk, tb;
    // decode step with append (chenxutan.com, "TurboQuant+ deep dive", 3.4:
    // the backends write each step's new K/V rows into the quantised cache):
    // the new token of row (b, kv head) goes to position seq_lens[b] of the
    // cache, encoded in the attention launch itself by one block of its row.
    //   append 1: that block is an extra one of the scores pass (its
    //             statistics are the last of a.n_chunks columns) which
    //             scores only the new token; the other chunks scan the
    //             seq_lens[b] tokens before it;
    //   append 2: the block whose token range holds the new position.
    // len_add: added to seq_lens[b] before clamping to [0, T].
    int append, len_add, vbits;
    const uint16_t *k_new, *v_new;  // [B * Hkv][128] fp16
    EncodePlanes kw, vw;            // the K and V planes, writable
};

// Query i of sequence s sits at position L_s - tq + i and sees the first
// L_s - tq + i + 1 tokens (causal prefill; with tq = 1 the whole sequence).
// seq_len_of gives what the last query of virtual sequence b sees; row_shift
// how many tokens fewer its row g sees.
__device__ __forceinline__ int seq_len_of(const AttnArgs &a, int b) {
    if (a.tq == 1) {  // decode: no integer divisions on the setup path
        if (!a.seq_lens) return a.T;
        int L = a.seq_lens[b];
        if (L >= a.T) return a.T;
        L += a.len_add;
        return L < 0 ? 0 : (L > a.T ? a.T : L);
    }
    const int groups = a.tq / a.qp;
    const int s = b / groups, grp = b - s * groups;
    int L = a.seq_lens ? a.seq_lens[s] : a.T;
    L = L < 0 ? 0 : (L > a.T ? a.T : L);
    L -= a.tq - a.qp * (grp + 1);
    return L < 0 ? 0 : L;
}
__device__ __forceinline__ int row_shift(const AttnArgs &a, int g) { return a.qp - 1 - g / a.qg; }

// The new token of decode row `row` (b * Hkv + kv head) encoded into cache
// row row * T + pos: K (Stage 1 + QJL, KB bits) by wave 0, V (Stage 1, VB
// bits) by wave 1, with the encode kernels' own tile code, so the bytes are
// those of tq_append_kv.  Every global read (quantiser tables, the 32 KB of
// S fragments, the two new rows, the lane constants) is issued before one
// barrier; et (two EncodeTables) and frag (2048 half8) are LDS scratch.
// Every thread of the block (NT threads) calls this; after the barrier that
// the caller places next, the block's own loads see the stored rows (no other
// block reads them in this launch).
template <int KB, int VB, int NT>
__device__ __forceinline__ void append_new_token(const AttnArgs &a, int row, int pos, EncodeTables *et,
                                                 half8 *frag, int tid) {
    static_assert(2048 % NT == 0, "S fragments split evenly over the threads");
    constexpr int kPer = 2048 / NT;
    const int wave = tid >> 6, lane = tid & 63, q = lane >> 4;
    half8 fr[kPer];
    const half8 *src = reinterpret_cast<const half8 *>(a.tab->S_enc);
#pragma unroll
    for (int i = 0; i < kPer; ++i) fr[i] = src[tid + i * NT];
    half8 xb[4];
    EncodeLane el;
    if (wave < 2) {
        const uint16_t *x = (wave == 0 ? a.k_new : a.v_new) + size_t(row) * kHeadDim + 32 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[s] = *reinterpret_cast<const half8 *>(x + 8 * s);
        if (wave == 0) encode_lane<KB>(a.tab, lane, el);
        else encode_lane<VB>(a.tab, lane, el);
    }
    fill_encode_tables<KB, true>(a.tab, &et[0], tid, NT);
    fill_encode_tables<VB, false>(a.tab, &et[1], tid, NT);
#pragma unroll
    for (int i = 0; i < kPer; ++i) frag[tid + i * NT] = fr[i];
    __syncthreads();
    const int dst = row * a.T + pos;  // cache rows < 2^31 (checked on the host)
    const bool first = (lane & 15) == 0;
    auto fget = [&](int i) { return frag[i]; };
    if (wave == 0)
        encode_tile<KB, true, false>(xb, el, et[0].levels, et[0].lut, fget, lane, first, dst, a.kw, [] {});
    else if (wave == 1)
        encode_tile<VB, false, false>(xb, el, et[1].levels, et[1].lut, fget, lane, first, dst, a.vw, [] {});
}

// Packed K/V row (batch * Hkv + kv head) of virtual row b * Hkv + kvh: the
// queries of one sequence share its cache.
__device__ __forceinline__ int kv_row(const AttnArgs &a, int row) {
    if (a.tq == 1) return row;
    const int b = row / a.Hkv;
    return (b / (a.tq / a.qp)) * a.Hkv + (row - b * a.Hkv);
}

// Row of q and out ([B, tq, Hq, d]) of row g of (virtual sequence b, kv head kvh).
__device__ __forceinline__ int64_t io_row(const AttnArgs &a, int b, int kvh, int g) {
    if (a.tq == 1) return int64_t(b) * a.hq_io + int64_t(kvh) * a.qg + g;
    const int groups = a.tq / a.qp;
    const int s = b / groups, grp = b - s * groups, u = g / a.qg;
    return (int64_t(s) * a.tq + a.qp * grp + u) * a.hq_io + int64_t(kvh) * a.qg + (g - u * a.qg);
}

// 2^x on the transcendental unit (v_exp_f32); only used for softmax weights
// of arguments <= 0, where its flush of results below 2^-126 is immaterial.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the 16 lanes of a DPP row: quad_perm xor 1, quad_perm
// xor 2, row_half_mirror, row_mirror; every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));
    x = fmaxf(x, dpp_mov<0x4E>(x));
    x = fmaxf(x, dpp_mov<0x141>(x));
    return fmaxf(x, dpp_mov<0x140>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    x += dpp_mov<0x141>(x);
    return x + dpp_mov<0x140>(x);
}
// Max over lanes l, l^16, l^32, l^48 (result in every lane).
__device__ __forceinline__ float quad_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The value of lane l ^ S (S = 1 .. 32) without LDS traffic: DPP quad
// permutes (1, 2) and row rotate (8), a bit-mode swizzle (4), and the
// permlane swaps (16, 32), whose pair holds both halves of the exchange.
template <int S>
__device__ __forceinline__ float lane_xor(float x, int lane) {
    if constexpr (S == 1) {
        return dpp_mov<0xB1>(x);
    } else if constexpr (S == 2) {
        return dpp_mov<0x4E>(x);
    } else if constexpr (S == 4) {
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));  // and 31, xor 4
    } else if constexpr (S == 8) {
        return dpp_mov<0x128>(x);  // rotate a row of 16 by 8
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
    } else {
        static_assert(S == 32, "lane bit");
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float((lane & 32) ? r[0] : r[1]);
    }
}

// Unnormalised 128-point Walsh-Hadamard transform of the coordinates held
// as v0 = coordinate lane, v1 = coordinate lane + 64 (bit 6 in-lane, bits
// 0..5 across lanes).
__device__ __forceinline__ void fwht128_lanes(float &v0, float &v1, int lane) {
    const float s0 = v0 + v1, s1 = v0 - v1;
    v0 = s0;
    v1 = s1;
    Unroll<6>::run([&](auto I) {
        constexpr int S = 1 << decltype(I)::value;
        const float sg = (lane & S) ? -1.0f : 1.0f;
        const float p0 = lane_xor<S>(v0, lane), p1 = lane_xor<S>(v1, lane);
        v0 = fmaf(sg, v0, p0);
        v1 = fmaf(sg, v1, p1);
    });
}

// ------------------------------------------------------------ query operands
// The MFMA A operands of the scores pass hold each query twice: row h < G is
// the fp16 hi half and row G + h the fp16 lo half of head h (rows >= 2G are
// zero), so that the two rows together carry the fp32 value to about 2^-22.
//   s_a:  q_rot = H D q / sqrt(d) for rotated keys, q itself for q8 keys;
//   s_ap: q_proj = S q_rot (unscaled; the score scales are applied per token).
// q_proj runs on the MFMA units: rows = 128 projections (wave w takes row
// blocks 2w, 2w+1), columns = heads (hi rows, then lo rows), k = coordinates;
// S is exact in fp16.  All global reads of this setup are issued at kernel
// entry (QueryLoads) and consumed after the lookup tables are built.
// NW = waves per block (4 or 8): wave w forms the query rows of heads
// w, w + NW, ... and the q_proj row blocks RB w .. RB w + RB - 1 (RB = 8 / NW).
template <int G, bool PROJ, int NW = 4>
struct QueryLoads {
    static_assert(NW == 4 || NW == 8, "4 or 8 waves per block");
    static constexpr int NH = (G + NW - 1) / NW;  // heads per wave
    static constexpr int RB = 8 / NW;             // q_proj row blocks of 16 per wave
    uint32_t q0[NH], q1[NH];                      // fp16 bits of coordinates lane, lane + 64
    float sg0, sg1;                               // D entries of those coordinates
    half8 sf[PROJ ? 4 * RB : 1];                  // S fragments (row block, k-step)
};

template <int G, bool PROJ, int NW>
__device__ __forceinline__ void load_query(QueryLoads<G, PROJ, NW> &ql, const AttnArgs &a, int b, int kvh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < ql.NH; ++i) {
        const int g = wave + NW * i;
        const uint16_t *q = a.q + io_row(a, b, kvh, g < G ? g : 0) * 128;
        ql.q0[i] = q[lane];
        ql.q1[i] = q[lane + 64];
    }
    ql.sg0 = a.tab->signs[lane];
    ql.sg1 = a.tab->signs[lane + 64];
    if constexpr (PROJ) {
        const int h = lane & 15, kq = lane >> 4;
        const half8 *S8 = reinterpret_cast<const half8 *>(a.tab->S);  // row-major [128][128]
#pragma unroll
        for (int rb2 = 0; rb2 < ql.RB; ++rb2)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                ql.sf[4 * rb2 + st] = S8[(16 * (ql.RB * wave + rb2) + h) * 16 + 4 * kq + st];
    }
}

__device__ __forceinline__ void put_hi_lo(_Float16 *hi, _Float16 *lo, float x) {
    const _Float16 h = _Float16(x);
    *hi = h;
    *lo = _Float16(x - float(h));
}

// Fills s_a (and s_ap) rows 0 .. 2G-1; rows 2G .. 15 must already be zero.
// Ends with a barrier.
template <int G, bool PROJ, int NW>
__device__ __forceinline__ void build_query_rows(const QueryLoads<G, PROJ, NW> &ql, const AttnArgs &a,
                                                 _Float16 (*s_a)[128], _Float16 (*s_ap)[128]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < ql.NH; ++i) {
        const int g = wave + NW * i;
        if (g >= G) break;
        float v0 = h2f(ql.q0[i]), v1 = h2f(ql.q1[i]);
        if (a.k_rotated) {
            v0 *= ql.sg0;
            v1 *= ql.sg1;
            fwht128_lanes(v0, v1, lane);
            v0 *= kRsqrtD;
            v1 *= kRsqrtD;
        }
        put_hi_lo(&s_a[g][lane], &s_a[G + g][lane], v0);
        put_hi_lo(&s_a[g][lane + 64], &s_a[G + g][lane + 64], v1);
    }
    __syncthreads();
    if constexpr (PROJ) {
        const int c = lane & 15, kq = lane >> 4;
        // B operand: column c = hi row c of s_a for c < G, lo row c - G + G
        // (= row c) for G <= c < 2G, zero above; i.e. simply row c of s_a
        half8 bq[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) bq[st] = *reinterpret_cast<const half8 *>(&s_a[c][32 * kq + 8 * st]);
#pragma unroll
        for (int rb2 = 0; rb2 < ql.RB; ++rb2) {
            const int rb = ql.RB * wave + rb2;
            floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql.sf[4 * rb2 + st], bq[st], acc, 0, 0, 0);
            // lane (c, kq) holds projections 16 rb + 4 kq + j of column c;
            // q_proj of head h = column h + column G + h (lanes c and c + G)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float other = __shfl_down(acc[j], G, 16);
                if (c < G) put_hi_lo(&s_ap[c][16 * rb + 4 * kq + j], &s_ap[G + c][16 * rb + 4 * kq + j],
                                     acc[j] + other);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ scores
// One wavefront scores 16 tokens of one kv head at a time with
// v_mfma_f32_16x16x32_f16: columns = tokens, k = coordinates, and the 16 rows
// carry the query of the G heads twice, as fp16 hi halves (rows h) and fp16
// lo halves (rows G + h), so that row h plus row G + h is the fp32 query to
// about 2^-22.  Lane l supplies token l&15 and the 32 coordinates
// 32*(l>>4)+[0,32) of its packed row (8 per MFMA k-step), so a lane unpacks
// exactly the b dwords it loaded.  Codebook levels enter as fp16 hi + lo
// halves (two MFMAs into one accumulator); the QJL operand is +-1, exact in
// fp16.  q8 keys use k-steps = the four 32-element scale blocks.
template <int KIND, int BITS>
struct KTiles {
    static constexpr int NT = kSliceTiles;  // tiles of 16 tokens per wave per slice
    static constexpr int W = KIND == TQ_KIND_Q8 ? 8 : BITS;
    uint32_t wk[NT][W], sw[NT], nn[NT];
    uint2 q8s[NT];
};

// Loads the K tiles of one slice (kSlice tokens).  Tokens at or past t1 read row
// tmax instead (any valid row: the scores of such tokens are discarded), so
// every call issues the same loads and the waits before scoring stay exact.
// NW = waves per block: tile i of wave w covers tokens base + 16 w + 16 NW i + [0, 16).
template <int NW = 4, int KIND, int BITS>
__device__ __forceinline__ void load_ktiles(KTiles<KIND, BITS> &d, int base, int tmax, int wave, int t, int kq,
                                            const uint8_t *kid, const uint8_t *ksg, const uint8_t *knm) {
    using KT = KTiles<KIND, BITS>;
    // byte offsets within the row are non-negative and below 2^32: unsigned
    // 32-bit offsets from the uniform row pointers, so each load is one
    // scalar-base + vector-offset access with no 64-bit address arithmetic
#pragma unroll
    for (int i = 0; i < KT::NT; ++i) {
        const uint32_t tok = uint32_t(min(base + wave * 16 + 16 * NW * i + t, tmax));
        if constexpr (KIND == TQ_KIND_Q8) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint2 u = *reinterpret_cast<const uint2 *>(kid + (tok * 128u + uint32_t(32 * s + 8 * kq)));
                d.wk[i][2 * s] = u.x;
                d.wk[i][2 * s + 1] = u.y;
            }
            d.q8s[i] = *reinterpret_cast<const uint2 *>(knm + tok * 8u);
        } else {
            const uint32_t *src =
                reinterpret_cast<const uint32_t *>(kid + (tok * uint32_t(16 * BITS) + uint32_t(4 * BITS * kq)));
#pragma unroll
            for (int w = 0; w < KT::W; ++w) d.wk[i][w] = src[w];
            if constexpr (KIND == TQ_KIND_PROD) {
                d.sw[i] = *reinterpret_cast<const uint32_t *>(ksg + (tok * 16u + uint32_t(4 * kq)));
                d.nn[i] = *reinterpret_cast<const uint32_t *>(knm + tok * 4u);
            } else {
                d.nn[i] = *reinterpret_cast<const uint16_t *>(knm + tok * 2u);
            }
        }
    }
}

// Adds row G + h of the MFMA result to row h: lane (t, kq) holds rows
// 4 kq + j, so for G <= 2 both rows are in the lane, for G = 4 in lanes l and
// l ^ 16, for G = 8 in lanes l and l ^ 32.
template <int G>
__device__ __forceinline__ void fold_rows(float (&e)[4]) {
    if constexpr (G == 1) {
        e[0] += e[1];
    } else if constexpr (G == 2) {
        e[0] += e[2];
        e[1] += e[3];
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = __float_as_uint(e[j]);
            const auto r = G == 4 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                                  : __builtin_amdgcn_permlane32_swap(x, x, false, false);
            e[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    }
}

// The value of x in lane l ^ 16 (resp. l ^ 32).  permlane16_swap(x, x)
// leaves a lane of an even 16-lane row with (x[l], x[l + 16]) and one of an
// odd row with (x[l - 16], x[l]); permlane32_swap likewise with halves.
__device__ __forceinline__ float partner16(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float partner32(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
}

// After fold_rows, each lane group kq (lanes 16 kq .. 16 kq + 15, one token
// per lane) takes over kOwn<G> heads: for G = 8, groups 0 and 2 hold heads
// 0..3 and groups 1 and 3 heads 4..7 in e[0..3], and group kq keeps heads
// 4 (kq & 1) + 2 (kq >> 1) + {0, 1}; G = 4: head kq (via a lane swap); below,
// head kq % G (duplicated across groups).  own_scores moves the scores there.
template <int G>
constexpr int kOwn = G >= 8 ? 2 : 1;
template <int G>
__device__ __forceinline__ int own_head(int kq, int i) {
    if constexpr (G >= 8) return 4 * (kq & 1) + 2 * (kq >> 1) + i;
    return G >= 4 ? kq + 4 * i : kq % G;
}
template <int G>
__device__ __forceinline__ void own_scores(const float (&e)[4], int lane, float (&o)[kOwn<G>]) {
    const int kq = lane >> 4;
    if constexpr (G == 1) {
        // head 0 sits in e[0] of group 0; every other group holds zero there
        o[0] = quad_sum(e[0]);
    } else if constexpr (G == 2) {
        // heads 0, 1 in e[0], e[1] of group 0, zeros elsewhere
        const float h0 = quad_sum(e[0]), h1 = quad_sum(e[1]);
        o[0] = (kq & 1) ? h1 : h0;
    } else if constexpr (G == 4) {
        // groups 0 and 1 both hold heads 0..3 in e[0..3]; groups 2, 3 zeros
        const float lo = (kq & 1) ? e[1] : e[0];
        const float hi = partner32((kq & 1) ? e[3] : e[2], lane);
        o[0] = kq < 2 ? lo : hi;
    } else {
        const bool up = (kq & 2) != 0;
        o[0] = up ? e[2] : e[0];
        o[1] = up ? e[3] : e[1];
    }
}

// Scores one slice (NT tiles per wave) and folds it into the running (max,
// sum) of each own head; store(h, tok, s) receives the score of head h (in
// the block's head numbering) and token tok, -inf past a row's causal limit.
// NW = waves per block (token layout as in load_ktiles).
template <bool FULL, bool ROWLIM, int G, int NW = 4, int KIND, int BITS, typename Store>
__device__ __forceinline__ void score_ktiles(const KTiles<KIND, BITS> &d, int base, int t1, int wave, int t,
                                             int kq, const uint2 *s_pair, const half8 *s_sgn,
                                             const half8 (&aq)[8], const half8 (&ap)[4], Store &&store,
                                             const int (&lim)[kOwn<G>], float (&m)[kOwn<G>],
                                             float (&l)[kOwn<G>]) {
    using KT = KTiles<KIND, BITS>;
    float scv[KT::NT][kOwn<G>];  // this lane's scores of the slice in log2 units, -inf where absent
    // B operands of the rotated-key path.  Field f (codes 2f, 2f+1 of the
    // lane) gives (hi(c0) hi(c1) | lo(c0) lo(c1)); fields 2u and 2u+1 side by
    // side are the B operand of k-step u, whose A operand repeats each query
    // value against its level's hi and lo half.  The table reads of tile i+1
    // are issued before the MFMAs of tile i, so LDS latency overlaps them.
    struct Ops {
        uint2 ef[16];
        half8 sg[4];
    };
    Ops ops[1];
    auto fetch = [&](int i, Ops &o) {
        Unroll<16>::run([&](auto P) {
            constexpr int pr = decltype(P)::value;
            o.ef[pr] = s_pair[code_at<2 * BITS, pr>(d.wk[i])];
        });
        if constexpr (KIND == TQ_KIND_PROD) {
#pragma unroll
            for (int s = 0; s < 4; ++s) o.sg[s] = s_sgn[(d.sw[i] >> (8 * s)) & 0xFFu];
        }
    };
    Unroll<KT::NT>::run([&](auto I) {
        constexpr int i = decltype(I)::value;
        const int tok = base + wave * 16 + 16 * NW * i + t;
        const bool valid = FULL || tok < t1;
        float e[4];
        if constexpr (KIND == TQ_KIND_Q8) {
            const uint2 scl = d.q8s[i];
            const float bs[4] = {h2f(scl.x & 0xFFFFu), h2f(scl.x >> 16), h2f(scl.y & 0xFFFFu), h2f(scl.y >> 16)};
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = 0.0f;
            // int8 q as fp16, exactly: byte q ^ 0x80 = q + 128 as the low
            // mantissa byte under exponent byte 0x64 is 1024 + q + 128, then
            // one packed subtract of 1152 (one XOR per four bytes, one permute
            // and one subtract per two)
            const half2v k1152 = half2v{_Float16(1152.0f), _Float16(1152.0f)};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint32_t bw[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t x = d.wk[i][2 * s + h] ^ 0x80808080u;
                    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);  // q0, q1
                    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);  // q2, q3
                    bw[2 * h] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, lo) - k1152);
                    bw[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, hi) - k1152);
                }
                const half8 bv = __builtin_bit_cast(half8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
                floatx4 ds = {0.0f, 0.0f, 0.0f, 0.0f};
                ds = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[s], bv, ds, 0, 0, 0);  // aq[0..3] only
                // scale of block s of token t
#pragma unroll
                for (int j = 0; j < 4; ++j) e[j] = fmaf(bs[s], ds[j], e[j]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] *= kRsqrtD;
        } else {
            fetch(i, ops[0]);
            __builtin_amdgcn_sched_barrier(0);
            const Ops &o = ops[0];
            floatx4 d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint4 bv = make_uint4(o.ef[2 * u].x, o.ef[2 * u].y, o.ef[2 * u + 1].x, o.ef[2 * u + 1].y);
                d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[u], __builtin_bit_cast(half8, bv), d0, 0, 0, 0);
            }
            if constexpr (KIND == TQ_KIND_PROD) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[s], o.sg[s], d1, 0, 0, 0);
            }
            // s = (1/sqrt d)(n/sqrt d)<q_rot, c> + (1/sqrt d) sqrt(pi/2)/m gamma <q_proj, sign>
            const float n = h2f(d.nn[i] & 0xFFFFu) * (1.0f / 128.0f);
            const float gq = h2f(d.nn[i] >> 16) * kQjlOverSqrtD;
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = (KIND == TQ_KIND_PROD) ? fmaf(n, d0[j], gq * d1[j]) : n * d0[j];
        }
        fold_rows<G>(e);
        float o[kOwn<G>];
        own_scores<G>(e, 16 * kq + t, o);
        // lane (t, kq) now holds the scores of its own heads for token tok;
        // one store per head and lane (on the whole-slice path without a
        // branch, so the memory counters stay exact).  A row whose query sees
        // fewer tokens (the earlier queries of a prefill group) stores -inf
        // past its limit, so the values pass gives those tokens no weight.
#pragma unroll
        for (int j = 0; j < kOwn<G>; ++j) {
            const bool vj = valid && (!ROWLIM || tok < lim[j]);
            if (valid) store(own_head<G>(kq, j), tok, vj ? o[j] : -INFINITY);
            scv[i][j] = vj ? o[j] * kLog2e : -INFINITY;
        }
    });
    // running (max, sum) per lane and own head, once per slice, in log2 units
    // (no branch: with every value -inf the base is 0 and each term exp2(-inf))
#pragma unroll
    for (int j = 0; j < kOwn<G>; ++j) {
        float mx = scv[0][j];
#pragma unroll
        for (int i = 1; i < KT::NT; ++i) mx = fmaxf(mx, scv[i][j]);
        const float nm = fmaxf(m[j], mx);
        const float mb = nm == -INFINITY ? 0.0f : nm;
        float acc = l[j] * fast_exp2(m[j] - mb);
#pragma unroll
        for (int i = 0; i < KT::NT; ++i) acc += fast_exp2(scv[i][j] - mb);
        l[j] = acc;
        m[j] = nm;
    }
}


// ------------------------------------------------- compacting values pass
// LDS of the compacting V accumulation (kSuper tokens compacted at a time;
// the per-wave partial sums of the end reuse the compaction buffers).
template <int G, int KIND, int BITS, int kSuper>
struct ValuesLds {
    static constexpr int kVPairs = KIND == TQ_KIND_Q8 ? 1 : 1 << (2 * BITS);
    static constexpr int R = kSuper / kVThreads;
    float2 vpair[kVPairs];  // the two levels of a 2-code field f = c0 | c1 << BITS (filled by the caller)
    int wcount[R][kVWaves];
    // the kept list: up to two super-slices of kept rows (weights per head,
    // token), drained when the next super-slice might not fit
    union {
        struct {
            float w[G][2 * kSuper];
            int tok[2 * kSuper];
        } c;
        float acc[kVWaves][G][128];
    } u;
};

// Accumulates weight x V over the kept tokens of [t0, t1) of one (sequence,
// kv head) row in the rotated domain (chenxutan.com, "TurboQuant+ deep
// dive", 3.3, and yeyulingfeng.com TurboQuant+ introduction, core item 4:
// rows whose weight p = exp(s - M)/L is below tau are skipped, the kept
// weights are not renormalised), then rotates each head's sum back and adds
// it into the output (ATOMIC) or stores it.  kVThreads threads; sv / vraw
// hold the first super-slice's scores (natural units) and V scale words,
// loaded by load_super(t0) before the call; load_super(base) refills them;
// s_M / s_invL are the exact statistics per head (natural-log max, 1/sum).
template <int G, int KIND, int BITS, int kSuper, bool ATOMIC, typename LoadSuper>
__device__ __forceinline__ void values_compact(const AttnArgs &a, int b, int kvh, int vrow, int t0, int t1,
                                               const float *s_M, const float *s_invL,
                                               float (&sv)[kSuper / kVThreads][G],
                                               uint32_t (&vraw)[kSuper / kVThreads], LoadSuper &&load_super,
                                               ValuesLds<G, KIND, BITS, kSuper> &lds) {
    constexpr int R = kSuper / kVThreads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // V accumulation layout: CPL coordinates per lane, LPT lanes per token,
    // TPW tokens per wave and pass (fewer coordinates per lane for 8 heads,
    // whose accumulators take twice the registers)
    constexpr int CPL = G >= 8 ? 4 : 8, LPT = 128 / CPL, TPW = 64 / LPT;
    const int tk = lane / LPT, cg = lane % LPT;  // token slot within the wave, coordinate group
    float acc[G][CPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < CPL; ++j) acc[g][j] = 0.0f;

    bool kept_any = false;  // uniform over the block
    int total = 0;          // rows in the kept list, uniform over the block
    for (int base = t0; base < t1; base += kSuper) {
        // 1) weights and the keep decision, R tokens per thread
        bool keep[R];
        uint64_t bal[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            keep[r] = false;
            if (base + kVThreads * r < t1) {  // uniform
                const bool ok = base + kVThreads * r + tid < t1;
                const float vsc = KIND == TQ_KIND_Q8 ? 1.0f : h2f(vraw[r]) * kRsqrtD;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float p = fast_exp2((sv[r][g] - s_M[g]) * kLog2e) * s_invL[g];
                    const bool k = ok && p >= a.tau;
                    keep[r] |= k;
                    sv[r][g] = k ? p * vsc : 0.0f;  // reuse as the weight
                }
            }
            bal[r] = __ballot(keep[r]);
            if (lane == 0) lds.wcount[r][wave] = __popcll(bal[r]);
        }
        __syncthreads();
        // 2) compaction in token order, appended to the kept list
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int off = total + cnt;
#pragma unroll
            for (int w = 0; w < kVWaves; ++w) {
                const int c = lds.wcount[r][w];
                off += (w < wave) ? c : 0;
                cnt += c;
            }
            if (keep[r]) {
                const int slot = off + __popcll(bal[r] & ((uint64_t(1) << lane) - 1));
                lds.u.c.tok[slot] = base + kVThreads * r + tid;
#pragma unroll
                for (int g = 0; g < G; ++g) lds.u.c.w[g][slot] = sv[r][g];
            }
        }
        total += cnt;
        kept_any |= cnt > 0;
        __syncthreads();
        if (base + kSuper < t1) load_super(base + kSuper);  // next super-slice in flight
        // the list is drained after the last super-slice and whenever the
        // next might not fit, so that with peaked attention the kept rows of
        // many super-slices share one round of V row loads
        if (total <= kSuper && base + kSuper < t1) continue;  // uniform
        // 3) accumulate kept rows: TPW tokens per wave and pass, CPL
        //    coordinates per lane.  All row loads of a batch are issued before
        //    any is used (a slot past `total` reads a kept row), and passes run
        //    four at a time without branches (such slots carry weight 0); the
        //    number of groups of four is uniform over the block.
        constexpr int PASSES = 8, PER_PASS = TPW * kVWaves;
        // codes of this lane: CPL * BITS bits from bit CPL * BITS * cg of the
        // row; within one dword unless 3-bit codes straddle two
        constexpr int NB = CPL * (KIND == TQ_KIND_Q8 ? 8 : BITS);
        constexpr bool TWO = (32 % NB) != 0;
        const int bit0 = NB * cg;
        for (int k0 = 0; k0 < total; k0 += PER_PASS * PASSES) {
            const int npass = min((total - k0 + PER_PASS - 1) / PER_PASS, PASSES);
            uint32_t raw[PASSES][2];
            float bsc[PASSES];
            Unroll<PASSES>::run([&](auto P) {
                constexpr int ps = decltype(P)::value;
                {
                    const int slot = min(k0 + PER_PASS * ps + wave * TPW + tk, total - 1);
                    const int64_t vec = int64_t(vrow) * a.T + lds.u.c.tok[slot];
                    raw[ps][1] = 0u;
                    if constexpr (KIND == TQ_KIND_Q8) {
                        if constexpr (CPL == 8) {
                            const uint2 u = *reinterpret_cast<const uint2 *>(a.vidx + vec * 128 + 8 * cg);
                            raw[ps][0] = u.x;
                            raw[ps][1] = u.y;
                        } else {
                            raw[ps][0] = *reinterpret_cast<const uint32_t *>(a.vidx + vec * 128 + 4 * cg);
                        }
                        bsc[ps] = h2f(reinterpret_cast<const uint16_t *>(a.vnorm)[vec * 4 + ((CPL * cg) >> 5)]);
                    } else {
                        const uint32_t *wp = reinterpret_cast<const uint32_t *>(a.vidx + vec * (16 * BITS));
                        raw[ps][0] = wp[bit0 >> 5];
                        if constexpr (TWO) raw[ps][1] = wp[(bit0 + NB - 1) >> 5];
                    }
                }
            });
            // every row load above is issued before the first use below
            asm volatile("" ::: "memory");
            Unroll<PASSES / 4>::run([&](auto Q) {
                constexpr int q4 = decltype(Q)::value;
                if (4 * q4 < npass) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int ps = 4 * q4 + u;
                        const int slot = k0 + PER_PASS * ps + wave * TPW + tk;
                        const bool live = slot < total;
                        float val[CPL];
                        if constexpr (KIND == TQ_KIND_Q8) {
#pragma unroll
                            for (int j = 0; j < CPL; ++j)
                                val[j] = float(int8_t((raw[ps][j >> 2] >> (8 * (j & 3))) & 0xFFu)) * bsc[ps];
                        } else {
                            uint32_t bitsw;
                            if constexpr (TWO) {
                                bitsw = __builtin_amdgcn_alignbit(raw[ps][1], raw[ps][0], bit0 & 31);
                            } else {
                                bitsw = raw[ps][0] >> (bit0 & 31);
                            }
                            // 2-code fields: one table read gives two levels
#pragma unroll
                            for (int f = 0; f < CPL / 2; ++f) {
                                const float2 lv = lds.vpair[(bitsw >> (2 * BITS * f)) & ((1u << (2 * BITS)) - 1u)];
                                val[2 * f] = lv.x;
                                val[2 * f + 1] = lv.y;
                            }
                        }
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            const float wg = live ? lds.u.c.w[g][slot] : 0.0f;
#pragma unroll
                            for (int j = 0; j < CPL; ++j) acc[g][j] = fmaf(wg, val[j], acc[g][j]);
                        }
                    }
                }
            });
        }
        total = 0;
        __syncthreads();
    }
    // reduce over the token slots of each wave, then over the waves
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            if constexpr (TPW == 4) {
                acc[g][j] = quad_sum(acc[g][j]);
            } else {
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[g][j]),
                                                                __float_as_uint(acc[g][j]), false, false);
                acc[g][j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            }
        }
    if (tk == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < CPL; ++j) lds.u.acc[wave][g][CPL * cg + j] = acc[g][j];
    }
    __syncthreads();
    // the block's share of each head, rotated back (out = R^T acc = D H acc /
    // sqrt(d) for rotated V codecs; R^T is linear, so shares rotate one by
    // one) and added into the output, which an earlier step zeroed (ATOMIC;
    // a block that kept no row adds nothing), or stored (a block that owns
    // the whole row)
    if (kept_any || !ATOMIC) {
        for (int g = wave; g < G; g += kVWaves) {
            float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
            for (int w = 0; w < kVWaves; ++w) {
                v0 += lds.u.acc[w][g][lane];
                v1 += lds.u.acc[w][g][lane + 64];
            }
            if (a.v_rotated) {
                fwht128_lanes(v0, v1, lane);
                v0 *= a.tab->signs[lane] * kRsqrtD;
                v1 *= a.tab->signs[lane + 64] * kRsqrtD;
            }
            float *o = a.out + io_row(a, b, kvh, g) * 128;
            if constexpr (ATOMIC) {
                __hip_atomic_fetch_add(o + lane, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(o + lane + 64, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                o[lane] = v0;
                o[lane + 64] = v1;
            }
        }
    }
}

}  // namespace tq
