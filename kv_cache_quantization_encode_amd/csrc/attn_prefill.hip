// Causal prefill attention at prompt scale over a packed TurboQuant cache
// (gfx950).
//
// The computation of the prefill path in attn.hip, where every one of the
// last Tq positions of a sequence attends to its own prefix exactly as a
// decode step does (chenxutan.com, "TurboQuant+ deep dive", 1.1; sparse V:
// yeyulingfeng.com TurboQuant+ introduction, core item 4, and chenxutan.com
// 3.3; the QJL term of the K score: quidproquo.cc, "TurboQuant+ KV cache
// compression", Stage 2), organised so that many queries share every K and
// V load and every operand decode:
//
//   block   64 (query, head) rows of one (sequence, kv head) x one token
//           range; row r is query r / g, head r % g of the kv head's g query
//           heads.  Wave w holds rows 16 w .. 16 w + 15 as two MFMA row
//           blocks of 8 rows, each carried as fp16 hi rows 0..7 and lo rows
//           8..15 (the query operands of the decode scan), so one decode of
//           a 16-token K tile feeds both row blocks.
//   pass 1  attn_prefill_stats_kernel scores the range and writes each
//           row's (max, sum exp) over it.
//   pass 2  attn_prefill_values_kernel merges the ranges' statistics into
//           the exact (M, L) of each row, scores the range again 32 tokens
//           at a time and keeps the weights p >= tau (dropped ones are not
//           renormalised).  The block stages w = p n_v (n_v: the V norm) in
//           LDS and the group's V levels transposed ([coordinate][token],
//           fp16 hi and lo), and each wave accumulates
//             O_rot[row][x] += sum_t w[row][t] c[idx(t, x)]
//           on the matrix cores (A = w as fp16 hi and lo rows, B = the level
//           hi or lo halves).  A group in which no row keeps a token is
//           skipped.  Each row's rotated sum is rotated back (R^T) and
//           stored (one range) or added with fp32 atomics (several ranges;
//           pass 1's first range zeroes the rows first).
// K: TurboQuant (codebook + QJL) or codebook only; V: codebook.  The
// statistics live in the workspace, [B, Tq, Hq, ranges] (max, sum) pairs.
#include "attn_common.h"

namespace tq {

constexpr int kPThreads = 256;  // 4 waves x 16 rows
constexpr int kPRows = 64;      // (query, head) rows per block
constexpr int kPGroup = 32;     // tokens per step of the values pass
constexpr int kVS = 40;         // LDS stride (halves) of a transposed V row: 16-byte aligned token octets

// The K operands of one 16-token tile, for the lane's token: its code words
// (lane group kq: coordinates 32 kq .. 32 kq + 31), QJL sign word, norms,
// and the token's V norm.
template <int KB>
struct PTile {
    uint32_t wk[KB], sw, nn, vn;
};

template <int KK, int KB>
__device__ __forceinline__ void load_ptile(PTile<KB> &d, const AttnArgs &a, int64_t kvbase, int tok, int kq) {
    const int64_t r = kvbase + tok;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(a.kidx + r * (16 * KB) + 4 * KB * kq);
#pragma unroll
    for (int w = 0; w < KB; ++w) d.wk[w] = src[w];
    if constexpr (KK == TQ_KIND_PROD) {
        d.sw = reinterpret_cast<const uint32_t *>(a.ksign + r * 16)[kq];
        d.nn = reinterpret_cast<const uint32_t *>(a.knorm)[r];
    } else {
        d.sw = 0;
        d.nn = reinterpret_cast<const uint16_t *>(a.knorm)[r];
    }
    d.vn = reinterpret_cast<const uint16_t *>(a.vnorm)[r];
}

// Block geometry: rows of queries qb * QB .. of sequence b, kv head kvh; the
// token range [t0, t1) of range `split` (t1 clipped to what the block's last
// query sees).
struct PBlock {
    int b, kvh, qb, split, L, t0, t1;
    int64_t kvbase;  // packed row of token 0 of this (sequence, kv head)
};

__device__ __forceinline__ PBlock prefill_block(const AttnArgs &a) {
    PBlock p;
    p.qb = int(blockIdx.x);
    p.split = int(blockIdx.y);
    const int row = int(blockIdx.z);  // b * Hkv + kvh
    p.b = row / a.Hkv;
    p.kvh = row - p.b * a.Hkv;
    int L = a.seq_lens ? a.seq_lens[p.b] : a.T;
    L = L < 0 ? 0 : (L > a.T ? a.T : L);
    p.L = L;
    const int qpb = kPRows / a.qg;
    const int qlast = min(p.qb * qpb + qpb - 1, a.tq - 1);
    const int lim = min(max(L - a.tq + qlast + 1, 0), L);
    p.t0 = p.split * a.chunk;
    p.t1 = min(p.t0 + a.chunk, lim);
    p.kvbase = int64_t(row) * a.T;
    return p;
}

// Row r of the block: query index (within the sequence's Tq) and head, and
// its offset in q / out ([B, Tq, Hq, d]); qi >= Tq marks a padding row.
__device__ __forceinline__ void prefill_row(const AttnArgs &a, const PBlock &p, int r, int &qi, int64_t &io) {
    const int u = r / a.qg, h = r - u * a.qg;
    qi = p.qb * (kPRows / a.qg) + u;
    const int qc = qi < a.tq ? qi : a.tq - 1;
    io = (int64_t(p.b) * a.tq + qc) * a.hq_io + int64_t(p.kvh) * a.qg + h;
}

// Query operands of this wave's 16 rows.  sa / sap: this wave's 32 LDS rows
// (row block rb: hi rows 16 rb .. 16 rb + 7, lo rows 16 rb + 8 ..).  Fills
// aq, ap (A operands of the codebook and QJL products, as in the decode
// scan) and, per own row (after the fold, lane group kq owns rows
// own_head<8>(kq, j) of each row block), the number of tokens it sees.
template <bool PROJ>
__device__ __forceinline__ void prefill_query(const AttnArgs &a, const PBlock &p, _Float16 (*sa)[128],
                                              _Float16 (*sap)[128], half8 (&aq)[2][8], half8 (&ap)[2][4],
                                              int (&lim)[2][2]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, kq = lane >> 4;
    uint32_t q0[16], q1[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        int qi;
        int64_t io;
        prefill_row(a, p, 16 * wave + rr, qi, io);
        const uint16_t *q = a.q + io * 128;
        q0[rr] = q[lane];
        q1[rr] = q[lane + 64];
    }
    const float sg0 = a.tab->signs[lane], sg1 = a.tab->signs[lane + 64];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        int qi;
        int64_t io;
        prefill_row(a, p, 16 * wave + rr, qi, io);
        float v0 = qi < a.tq ? h2f(q0[rr]) * sg0 : 0.0f;
        float v1 = qi < a.tq ? h2f(q1[rr]) * sg1 : 0.0f;
        fwht128_lanes(v0, v1, lane);
        const int rb = rr >> 3, i = rr & 7;
        put_hi_lo(&sa[16 * rb + i][lane], &sa[16 * rb + 8 + i][lane], v0 * kRsqrtD);
        put_hi_lo(&sa[16 * rb + i][lane + 64], &sa[16 * rb + 8 + i][lane + 64], v1 * kRsqrtD);
    }
    if constexpr (PROJ) {
        // q_proj = S q_rot on the matrix cores: rows = 128 projections (8
        // blocks of 16), columns = the 16 rows of a row block (hi, then lo),
        // k = coordinates; S fragments from global memory, four row blocks
        // of S at a time
        const half8 *S8 = reinterpret_cast<const half8 *>(a.tab->S);  // row-major [128][128]
        half8 bq[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                bq[rb][st] = *reinterpret_cast<const half8 *>(&sa[16 * rb + c][32 * kq + 8 * st]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            half8 sf[4][4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int st = 0; st < 4; ++st) sf[s4][st] = S8[(16 * (4 * half + s4) + c) * 16 + 4 * kq + st];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int sb = 4 * half + s4;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int st = 0; st < 4; ++st)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf[s4][st], bq[rb][st], acc, 0, 0, 0);
                    // lane (c, kq) holds projections 16 sb + 4 kq + j of
                    // column c; row i's q_proj = column i + column 8 + i
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float other = __shfl_down(acc[j], 8, 16);
                        if (c < 8)
                            put_hi_lo(&sap[16 * rb + c][16 * sb + 4 * kq + j],
                                      &sap[16 * rb + 8 + c][16 * sb + 4 * kq + j], acc[j] + other);
                    }
                }
            }
        }
    }
    // A operands (row = lane & 15 of each row block): codebook k-step u of
    // lane group kq covers coordinates 32 kq + 4u .. +3 as (q0 q1 q0 q1 q2 q3
    // q2 q3) against the levels' (hi hi lo lo hi hi lo lo); QJL k-step s
    // covers projections 32 kq + 8 s .. +7
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint2 v = *reinterpret_cast<const uint2 *>(&sa[16 * rb + c][32 * kq + 4 * u]);
            aq[rb][u] = __builtin_bit_cast(half8, make_uint4(v.x, v.x, v.y, v.y));
        }
        if constexpr (PROJ) {
#pragma unroll
            for (int s = 0; s < 4; ++s) ap[rb][s] = *reinterpret_cast<const half8 *>(&sap[16 * rb + c][32 * kq + 8 * s]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int qi;
            int64_t io;
            prefill_row(a, p, 16 * wave + 8 * rb + own_head<8>(kq, j), qi, io);
            lim[rb][j] = qi < a.tq ? min(max(p.L - a.tq + qi + 1, 0), p.L) : 0;
        }
    }
}

// The level-pair table of the K codebook (field f = codes c0 | c1 << KB:
// fp16 hi halves of both levels, then lo halves) and the QJL sign table
// (byte -> eight fp16 +-1), built by the block's threads (barrier after).
template <int KK, int KB>
__device__ __forceinline__ void prefill_tables(const AttnArgs &a, uint2 *s_pair, half8 *s_sgn, int tid) {
    constexpr int kPairs = 1 << (2 * KB);
    if (tid < kPairs) {
        const float l0 = a.tab->levels[KB - 1][tid & ((1 << KB) - 1)];
        const float l1 = a.tab->levels[KB - 1][tid >> KB];
        const _Float16 h0 = _Float16(l0), h1 = _Float16(l1);
        const _Float16 o0 = _Float16(l0 - float(h0)), o1 = _Float16(l1 - float(h1));
        s_pair[tid] = uint2{uint32_t(__builtin_bit_cast(uint16_t, h0)) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16),
                            uint32_t(__builtin_bit_cast(uint16_t, o0)) | (uint32_t(__builtin_bit_cast(uint16_t, o1)) << 16)};
    }
    if constexpr (KK == TQ_KIND_PROD) {
        half8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ((tid >> j) & 1) ? _Float16(1.0f) : _Float16(-1.0f);
        s_sgn[tid] = v;
    }
}

// Scores of one 16-token tile for this lane's token and its own rows:
// o[rb][j] = score of row own_head<8>(kq, j) of row block rb (natural units).
template <int KK, int KB>
__device__ __forceinline__ void prefill_score(const PTile<KB> &d, const uint2 *s_pair, const half8 *s_sgn,
                                              const half8 (&aq)[2][8], const half8 (&ap)[2][4], int lane,
                                              float (&o)[2][2]) {
    uint2 ef[16];
    Unroll<16>::run([&](auto P) {
        constexpr int pr = decltype(P)::value;
        ef[pr] = s_pair[code_at<2 * KB, pr>(d.wk)];
    });
    half8 sg[4];
    if constexpr (KK == TQ_KIND_PROD) {
#pragma unroll
        for (int s = 0; s < 4; ++s) sg[s] = s_sgn[(d.sw >> (8 * s)) & 0xFFu];
    }
    // s = (1/sqrt d)(n/sqrt d)<q_rot, c> + (1/sqrt d) sqrt(pi/2)/m gamma <q_proj, sign>
    const float n = h2f(d.nn & 0xFFFFu) * (1.0f / 128.0f);
    const float gq = KK == TQ_KIND_PROD ? h2f(d.nn >> 16) * kQjlOverSqrtD : 0.0f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        floatx4 d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint4 bv = make_uint4(ef[2 * u].x, ef[2 * u].y, ef[2 * u + 1].x, ef[2 * u + 1].y);
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[rb][u], __builtin_bit_cast(half8, bv), d0, 0, 0, 0);
        }
        if constexpr (KK == TQ_KIND_PROD) {
#pragma unroll
            for (int s = 0; s < 4; ++s) d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[rb][s], sg[s], d1, 0, 0, 0);
        }
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = KK == TQ_KIND_PROD ? fmaf(n, d0[j], gq * d1[j]) : n * d0[j];
        fold_rows<8>(e);
        own_scores<8>(e, lane, o[rb]);
    }
}

// ------------------------------------------------------------------ pass 1
template <int KK, int KB>
__global__ __launch_bounds__(kPThreads) void attn_prefill_stats_kernel(AttnArgs a) {
    constexpr bool PROJ = KK == TQ_KIND_PROD;
    __shared__ uint2 s_pair[1 << (2 * KB)];
    __shared__ half8 s_sgn[PROJ ? 256 : 1];
    __shared__ __attribute__((aligned(16))) _Float16 s_a[4 * 32][128];
    __shared__ __attribute__((aligned(16))) _Float16 s_ap[PROJ ? 4 * 32 : 1][128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = lane & 15, kq = lane >> 4;
    const PBlock p = prefill_block(a);
    // several ranges add their shares into the output: the first range's
    // block zeroes its rows (this pass ends before the values pass starts)
    if (a.n_chunks > 1 && p.split == 0) {
        for (int i = tid; i < kPRows * 128; i += kPThreads) {
            int qi;
            int64_t io;
            prefill_row(a, p, i >> 7, qi, io);
            if (qi < a.tq) a.out[io * 128 + (i & 127)] = 0.0f;
        }
    }
    prefill_tables<KK, KB>(a, s_pair, s_sgn, tid);
    half8 aq[2][8], ap[2][4];
    int lim[2][2];
    prefill_query<PROJ>(a, p, &s_a[32 * wave], PROJ ? &s_ap[32 * wave] : nullptr, aq, ap, lim);
    __syncthreads();  // tables
    float m[2][2], l[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            m[rb][j] = -INFINITY;
            l[rb][j] = 0.0f;
        }
    if (p.t0 < p.t1) {
        const int tmax = p.t1 - 1;
        // tiles of 16 tokens, two ahead of the one scored
        PTile<KB> ta, tb, tc;
        load_ptile<KK, KB>(ta, a, p.kvbase, min(p.t0 + t, tmax), kq);
        load_ptile<KK, KB>(tb, a, p.kvbase, min(p.t0 + 16 + t, tmax), kq);
        // two tiles' scores, then one update of the running (max, sum)
        float sv[2][2][2];  // [tile][rb][j], log2 units
        auto score = [&](PTile<KB> &cur, PTile<KB> &nxt2, int base, int k) {
            load_ptile<KK, KB>(nxt2, a, p.kvbase, min(base + 32 + t, tmax), kq);
            float o[2][2];
            prefill_score<KK, KB>(cur, s_pair, s_sgn, aq, ap, lane, o);
            const int tok = base + t;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    sv[k][rb][j] = (tok < p.t1 && tok < lim[rb][j]) ? o[rb][j] * kLog2e : -INFINITY;
        };
        auto update = [&]() {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float nm = fmaxf(m[rb][j], fmaxf(sv[0][rb][j], sv[1][rb][j]));
                    const float mb = nm == -INFINITY ? 0.0f : nm;
                    l[rb][j] = l[rb][j] * fast_exp2(m[rb][j] - mb) + fast_exp2(sv[0][rb][j] - mb) +
                               fast_exp2(sv[1][rb][j] - mb);
                    m[rb][j] = nm;
                }
        };
        // tiles rotate through ta, tb, tc (two loads ahead); a pair of tiles
        // per update, the second of a last odd tile scoring nothing
        for (int base = p.t0;;) {
            score(ta, tc, base, 0);
            if (base + 16 < p.t1) score(tb, ta, base + 16, 1);
            else sv[1][0][0] = sv[1][0][1] = sv[1][1][0] = sv[1][1][1] = -INFINITY;
            update();
            base += 32;
            if (base >= p.t1) break;
            score(tc, tb, base, 0);
            if (base + 16 < p.t1) score(ta, tc, base + 16, 1);
            else sv[1][0][0] = sv[1][0][1] = sv[1][1][0] = sv[1][1][1] = -INFINITY;
            update();
            base += 32;
            if (base >= p.t1) break;
            score(tb, ta, base, 0);
            if (base + 16 < p.t1) score(tc, tb, base + 16, 1);
            else sv[1][0][0] = sv[1][0][1] = sv[1][1][0] = sv[1][1][1] = -INFINITY;
            update();
            base += 32;
            if (base >= p.t1) break;
        }
    }
    // (max, sum) of each own row over its 16 token lanes, natural units
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float mx = row16_max(m[rb][j]);
            const float ll = row16_sum(m[rb][j] == -INFINITY ? 0.0f : l[rb][j] * fast_exp2(m[rb][j] - mx));
            int qi;
            int64_t io;
            prefill_row(a, p, 16 * wave + 8 * rb + own_head<8>(kq, j), qi, io);
            if (t == 0 && qi < a.tq) {
                float *st = a.stats + (io * a.n_chunks + p.split) * 2;
                st[0] = mx == -INFINITY ? mx : mx / kLog2e;
                st[1] = ll;
            }
        }
}

// ------------------------------------------------------------------ pass 2
// V codes for the transposed staging of a 32-token group: the 4 VB-bit
// codes of coordinates 4 j .. 4 j + 3 of packed row r (low bits first).
// The V norms enter the weights.
template <int VB>
__device__ __forceinline__ uint32_t load_vcodes(const AttnArgs &a, int64_t r, int j) {
    const uint32_t *row = reinterpret_cast<const uint32_t *>(a.vidx + r * (16 * VB));
    const int bit = 4 * VB * j, dw = bit >> 5, sh = bit & 31;
    uint32_t v = row[dw] >> sh;
    if (sh + 4 * VB > 32) v |= row[dw + 1] << (32 - sh);
    return v;
}

template <int KK, int KB, int VB>
__global__ __launch_bounds__(kPThreads) void attn_prefill_values_kernel(AttnArgs a) {
    constexpr bool PROJ = KK == TQ_KIND_PROD;
    __shared__ uint2 s_pair[1 << (2 * KB)];
    __shared__ half8 s_sgn[PROJ ? 256 : 1];
    __shared__ uint32_t s_vlev[16];  // V levels as fp16 hi | lo << 16
    __shared__ int s_flag[2][4];
    __shared__ float s_ml[kPRows][2];  // per row: M (log2 units), 1/L
    // one region, three uses: the query set-up (s_a, s_ap), the per-group
    // staging (weights and transposed V, two buffers), the rotated outputs
    struct Setup {
        _Float16 a[4 * 32][128];
        _Float16 ap[PROJ ? 4 * 32 : 1][128];
    };
    struct Stage {
        float w[2][kPRows][kPGroup];
        _Float16 vh[2][128][kVS], vl[2][128][kVS];
    };
    struct Outs {
        float o[kPRows][128];
    };
    constexpr size_t kRegion = sizeof(Setup) > sizeof(Stage) ? (sizeof(Setup) > sizeof(Outs) ? sizeof(Setup) : sizeof(Outs))
                                                             : (sizeof(Stage) > sizeof(Outs) ? sizeof(Stage) : sizeof(Outs));
    __shared__ __attribute__((aligned(16))) unsigned char s_region[kRegion];
    Setup &su = *reinterpret_cast<Setup *>(s_region);
    Stage &sg = *reinterpret_cast<Stage *>(s_region);
    Outs &so = *reinterpret_cast<Outs *>(s_region);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = lane & 15, kq = lane >> 4;
    const PBlock p = prefill_block(a);
    prefill_tables<KK, KB>(a, s_pair, s_sgn, tid);
    if (tid < 16) {
        const float lv = a.tab->levels[VB - 1][tid & ((1 << VB) - 1)];
        const _Float16 h = _Float16(lv), o = _Float16(lv - float(h));
        s_vlev[tid] = uint32_t(__builtin_bit_cast(uint16_t, h)) | (uint32_t(__builtin_bit_cast(uint16_t, o)) << 16);
    }
    half8 aq[2][8], ap[2][4];
    int lim[2][2];
    prefill_query<PROJ>(a, p, &su.a[32 * wave], PROJ ? &su.ap[32 * wave] : nullptr, aq, ap, lim);
    // the exact (M, 1/L) of each of the wave's rows from every range's
    // statistics: lane s holds range s (ranges s + 64, ... folded into it),
    // all 16 rows' loads in flight together; M in log2 units
    {
        float ms[16], ls[16];
        const float *st[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            int qi;
            int64_t io;
            prefill_row(a, p, 16 * wave + rr, qi, io);
            st[rr] = a.stats + io * a.n_chunks * 2;
            float2 v = make_float2(-INFINITY, 0.0f);
            if (lane < a.n_chunks) v = *reinterpret_cast<const float2 *>(st[rr] + 2 * lane);
            ms[rr] = v.x;
            ls[rr] = v.y;
        }
        for (int s = lane + 64; s < a.n_chunks; s += 64) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const float m2 = st[rr][2 * s], l2 = st[rr][2 * s + 1];
                const float mm = fmaxf(ms[rr], m2);
                if (mm != -INFINITY) {
                    ls[rr] = ls[rr] * __expf(ms[rr] - mm) + l2 * __expf(m2 - mm);
                    ms[rr] = mm;
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float mm = quad_max(row16_max(ms[rr]));
            const float ll = quad_sum(row16_sum(mm == -INFINITY || ms[rr] == -INFINITY ? 0.0f
                                                                                       : ls[rr] * __expf(ms[rr] - mm)));
            if (lane == 0) {
                s_ml[16 * wave + rr][0] = mm == -INFINITY ? 0.0f : mm * kLog2e;
                s_ml[16 * wave + rr][1] = ll > 0.0f ? 1.0f / ll : 0.0f;
            }
        }
    }
    __syncthreads();  // tables and row statistics ready; the set-up rows are consumed
    float M2[2][2], invL[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 16 * wave + 8 * rb + own_head<8>(kq, j);
            M2[rb][j] = s_ml[r][0];
            invL[rb][j] = s_ml[r][1];
        }

    floatx4 acc[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) acc[rb][cb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    const int tq4 = tid & 7, jv = tid >> 3;  // V staging: token quad, coordinate quad
    if (p.t0 < p.t1) {
        const int tmax = p.t1 - 1;
        // a group's loads one group ahead, in two named buffers (no copies,
        // so no wait is forced before the data is used)
        struct Grp {
            PTile<KB> k[2];
            uint32_t vc[4];
        };
        Grp g0, g1;
        auto load_group = [&](int base, Grp &g) {
#pragma unroll
            for (int i = 0; i < 2; ++i) load_ptile<KK, KB>(g.k[i], a, p.kvbase, min(base + 16 * i + t, tmax), kq);
#pragma unroll
            for (int u = 0; u < 4; ++u) g.vc[u] = load_vcodes<VB>(a, p.kvbase + min(base + 4 * tq4 + u, tmax), jv);
        };
        auto process = [&](const Grp &g, int base, int buf) {
            // transposed V levels of the group (before its weights are known,
            // so one barrier per group serves both stagings; a group whose
            // weights all drop is then skipped at the products): rows =
            // coordinates 4 jv + i, columns = tokens 4 tq4 .. 4 tq4 + 3 (fp16
            // hi and lo, 8 bytes a store: rows 4 apart fall 16 banks apart).
            // Buffer buf was last read by the products two groups back, which
            // every wave finished before the previous group's barrier.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t lv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) lv[u] = s_vlev[(g.vc[u] >> (VB * i)) & ((1u << VB) - 1u)];
                *reinterpret_cast<uint2 *>(&sg.vh[buf][4 * jv + i][4 * tq4]) =
                    make_uint2((lv[0] & 0xFFFFu) | (lv[1] << 16), (lv[2] & 0xFFFFu) | (lv[3] << 16));
                *reinterpret_cast<uint2 *>(&sg.vl[buf][4 * jv + i][4 * tq4]) =
                    make_uint2((lv[0] >> 16) | (lv[1] & 0xFFFF0000u), (lv[2] >> 16) | (lv[3] & 0xFFFF0000u));
            }
            // weights of the group's 32 tokens for this lane's own rows
            bool any = false;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float o[2][2];
                prefill_score<KK, KB>(g.k[i], s_pair, s_sgn, aq, ap, lane, o);
                const int tok = base + 16 * i + t;
                const float nv = h2f(g.k[i].vn);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const bool in = tok < p.t1 && tok < lim[rb][j];
                        const float pw = fast_exp2(fmaf(o[rb][j], kLog2e, -M2[rb][j])) * invL[rb][j];
                        const float w = in && pw >= a.tau ? pw * nv : 0.0f;
                        any |= w != 0.0f;
                        sg.w[buf][16 * wave + 8 * rb + own_head<8>(kq, j)][16 * i + t] = w;
                    }
            }
            const bool wave_any = __builtin_amdgcn_ballot_w64(any) != 0;
            if (lane == 0) s_flag[buf][wave] = wave_any ? 1 : 0;
            __syncthreads();
            if ((s_flag[buf][0] | s_flag[buf][1] | s_flag[buf][2] | s_flag[buf][3]) == 0) return;
            // O_rot += w V on the matrix cores: A row mr = lane & 15 is row
            // mr & 7 of the row block as the fp16 hi (mr < 8) or lo half of
            // its weights, k = tokens 8 kq .. 8 kq + 7
            const int mr = lane & 15;
            half8 A[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const float *wr = &sg.w[buf][16 * wave + 8 * rb + (mr & 7)][8 * kq];
                const float4 w0 = *reinterpret_cast<const float4 *>(wr);
                const float4 w1 = *reinterpret_cast<const float4 *>(wr + 4);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const _Float16 h = _Float16(wv[k]);
                    A[rb][k] = mr < 8 ? h : _Float16(wv[k] - float(h));
                }
            }
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const half8 bh = *reinterpret_cast<const half8 *>(&sg.vh[buf][16 * cb + mr][8 * kq]);
                const half8 bl = *reinterpret_cast<const half8 *>(&sg.vl[buf][16 * cb + mr][8 * kq]);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[rb], bh, acc[rb][cb], 0, 0, 0);
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[rb], bl, acc[rb][cb], 0, 0, 0);
                }
            }
        };
        load_group(p.t0, g0);
        for (int base = p.t0;;) {
            if (base + kPGroup < p.t1) load_group(base + kPGroup, g1);
            process(g0, base, 0);
            base += kPGroup;
            if (base >= p.t1) break;
            if (base + kPGroup < p.t1) load_group(base + kPGroup, g0);
            process(g1, base, 1);
            base += kPGroup;
            if (base >= p.t1) break;
        }
    }
    __syncthreads();  // the staging buffers are done with
    // rows i and 8 + i of each product are row i's hi- and lo-weight parts
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            float e[4] = {acc[rb][cb][0], acc[rb][cb][1], acc[rb][cb][2], acc[rb][cb][3]};
            fold_rows<8>(e);
            if (kq < 2) {
#pragma unroll
                for (int j = 0; j < 4; ++j) so.o[16 * wave + 8 * rb + 4 * kq + j][16 * cb + t] = e[j];
            }
        }
    __syncthreads();
    // each wave rotates its rows back: out = D H O_rot / d (the V levels
    // carry no 1/sqrt(d), the weights carry the V norms)
    const float d0 = a.tab->signs[lane] * (kRsqrtD * kRsqrtD), d1 = a.tab->signs[lane + 64] * (kRsqrtD * kRsqrtD);
    for (int rr = 0; rr < 16; ++rr) {
        const int r = 16 * wave + rr;
        int qi;
        int64_t io;
        prefill_row(a, p, r, qi, io);
        if (qi >= a.tq) continue;
        float v0 = so.o[r][lane], v1 = so.o[r][lane + 64];
        fwht128_lanes(v0, v1, lane);
        float *o = a.out + io * 128;
        if (a.n_chunks > 1) {
            if (p.t0 < p.t1) {
                __hip_atomic_fetch_add(o + lane, v0 * d0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(o + lane + 64, v1 * d1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            o[lane] = v0 * d0;
            o[lane + 64] = v1 * d1;
        }
    }
}

// ------------------------------------------------------------------ launch
template <int KK, int KB, int VB>
static int launch_prefill_t(const AttnArgs &a, int qblocks, hipStream_t s) {
    const dim3 grid(unsigned(qblocks), unsigned(a.n_chunks), unsigned(a.B * a.Hkv));
    hipLaunchKernelGGL((attn_prefill_stats_kernel<KK, KB>), grid, dim3(kPThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return int(e);
    hipLaunchKernelGGL((attn_prefill_values_kernel<KK, KB, VB>), grid, dim3(kPThreads), 0, s, a);
    return int(hipGetLastError());
}

template <int KK, int KB>
static int prefill_dispatch_v(const AttnArgs &a, int qblocks, tq_format vf, hipStream_t s) {
    switch (vf.bits) {
        case 1: return launch_prefill_t<KK, KB, 1>(a, qblocks, s);
        case 2: return launch_prefill_t<KK, KB, 2>(a, qblocks, s);
        case 3: return launch_prefill_t<KK, KB, 3>(a, qblocks, s);
        case 4: return launch_prefill_t<KK, KB, 4>(a, qblocks, s);
    }
    return int(hipErrorInvalidValue);
}

int launch_attn_prefill(const AttnArgs &a, tq_format kf, tq_format vf, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t rows = int64_t(a.tq) * a.qg;
    const int qblocks = int((rows + kPRows - 1) / kPRows);
    if (vf.kind != TQ_KIND_MSE) return int(hipErrorInvalidValue);
    if (kf.kind == TQ_KIND_PROD) {
        switch (kf.bits) {
            case 1: return prefill_dispatch_v<TQ_KIND_PROD, 1>(a, qblocks, vf, s);
            case 2: return prefill_dispatch_v<TQ_KIND_PROD, 2>(a, qblocks, vf, s);
            case 3: return prefill_dispatch_v<TQ_KIND_PROD, 3>(a, qblocks, vf, s);
        }
    } else if (kf.kind == TQ_KIND_MSE) {
        switch (kf.bits) {
            case 1: return prefill_dispatch_v<TQ_KIND_MSE, 1>(a, qblocks, vf, s);
            case 2: return prefill_dispatch_v<TQ_KIND_MSE, 2>(a, qblocks, vf, s);
            case 3: return prefill_dispatch_v<TQ_KIND_MSE, 3>(a, qblocks, vf, s);
            case 4: return prefill_dispatch_v<TQ_KIND_MSE, 4>(a, qblocks, vf, s);
        }
    }
    return int(hipErrorInvalidValue);
}

}  // namespace tq
