// Single-launch decode attention for 8 query heads per KV head (gfx950).
//
// The same computation as the two passes of attn.hip (chenxutan.com,
// "TurboQuant+ deep dive", 1.1 cached decode attention; quidproquo.cc,
// "TurboQuant+ KV cache compression", Stage 2: the QJL term of the K score;
// yeyulingfeng.com TurboQuant+ introduction, core item 4, and chenxutan.com
// 3.3: V rows below the weight threshold are skipped, kept weights are not
// renormalised), in one kernel:
//
//   phase 1  each block scores its token range [t0, t1) of one (sequence, KV
//            head) row exactly as the scores pass does (query rows on the
//            matrix cores, 16-token MFMA tiles) and keeps the scores in LDS;
//            its (max, sum exp) per head go to the workspace.
//   barrier  the nblk blocks of a row wait for each other (one counter per
//            row, bounded spin): exact sparse V needs the row's global softmax
//            statistics before any V row is skipped.  The launcher sizes the
//            grid so that every block is resident at once (one block per CU).
//   phase 2  the exact (M, L) from all blocks' statistics; the V products of
//            the block's range on the matrix cores, reading the scores from
//            LDS; the block's share is rotated back (R^T) and added into the
//            output (fp32 atomics; block 0 zeroes the output before the
//            barrier).  A row served by one block stores its output directly.
//
// V products, 2-bit codebook: the symmetric 4-level codebook is exactly
// c[2 b1 + b0] = a1 (2 b1 - 1) + a0 (2 b0 - 1) (a1 = (c3 + c2) / 2,
// a0 = (c3 - c2) / 2), so the rotated-domain sum of head h over coordinate x
//   y[h][x] = sum_t w_ht n_t c[code_tx] = 2 a1 X1 + 2 a0 X0 - (a1 + a0) W,
//   X_p[h][x] = sum_t w_ht n_t bit_p(code_tx),  W[h] = sum_t w_ht n_t,
// and each X_p is an MFMA product whose A operand carries w_ht n_t (fp16 hi
// and lo rows, scaled below 2^14 by the block's largest V norm) and whose B
// operand is the code bit itself: a half with only bit k set is the exact
// fp16 power of two bitval(k), so B = (two tokens' code words) & (bit k of
// each half) costs one AND per two k-slots, and the product's power of two is
// divided out of its accumulator at the end.  q8 V keeps the int8-as-fp16 B
// operand of attn.hip with the per-32 block scales in A.
#include "attn_common.h"

namespace tq {

constexpr int kFW = 8;                           // waves per block
constexpr int kFThreads = 64 * kFW;
constexpr int kFSlice = 16 * kFW * kSliceTiles;  // tokens scored per slice (512)
static_assert(kFSlice == kFusedSlice, "slice size shared with the host plan");
constexpr int kFTokens = kFusedMaxTokens;        // most tokens per block (scores held in LDS)
constexpr int kFLd = kFTokens + 16;              // LDS score row stride: head rows 16 banks apart
constexpr float kAMax = 16384.0f;                // V-product A operands stay below 2^14
constexpr uint64_t kSpinTicks = 25000000;        // barrier spin budget: 0.25 s of the 100 MHz clock
constexpr int kQRow = 132;                       // fp32 query row stride of the setup scratch

// fp16 value of a half whose only set bit is bit k (k <= 14)
__host__ __device__ constexpr float bitval(int k) {
    return k <= 9 ? 1.0f / float(1 << (24 - k))
                  : (k == 10 ? 1.0f / 16384.0f
                             : (k == 11 ? 1.0f / 8192.0f : (k == 12 ? 1.0f / 2048.0f : (k == 13 ? 1.0f / 128.0f : 2.0f))));
}

// ------------------------------------------------------- bit-plane scoring
// 1- and 2-bit codebooks are sums of signed constants chosen by single code
// bits: c[b] = a (2b - 1) (1 bit, a = c1) and c[2 b1 + b0] = a1 (2 b1 - 1) +
// a0 (2 b0 - 1) (2 bits, a1 = (c3 + c2) / 2, a0 = (c3 - c2) / 2).  So the
// codebook product of a key is
//   sum over bits of (2 coef q) x bit  -  (a1 + a0) sum q   (1 bit: a sum q),
// and its MFMA B operand is the packed code word itself: w & (bit k of both
// 16-bit halves) is two fp16 halves whose only set bit is bit k, i.e. the
// code bit times the exact power of two 2^(k - 24) (subnormal for k <= 9;
// bits 10..15 are first shifted down to 4..9).  The query operand of each
// k-slot carries 2 coef q 2^(S0 - k), so every product has the same scale
// 2^(S0 - 24), divided out in the epilogue.  One AND per two k-slots, no
// table reads.  Lane (r, kq) of source dword j, product u (0..3) holds k-slot
// pairs i = 0..3 from bit k = 4u + i of the dword's low half (slot 2i) and
// high half (slot 2i + 1).  The QJL term takes its +-1 B operands from the
// 256-entry sign table against the q_proj rows.
//
// Rows of these products come in head pairs: row 2h is the fp16 hi half of
// head h, row 2h + 1 its lo half, so lane group kq (output rows 4kq..4kq+3)
// holds both halves of heads 2kq and 2kq + 1, its own heads: the hi + lo
// fold is two adds in the lane.
template <int G, int BITS>
struct PlaneOps {
    half8 ab[4 * BITS];  // codebook products
    float sc_cb;         // log2(e) 2^(24 - S0) / 128: accumulator to log2-unit score per unit of norm
    float ccb[2];        // log2(e) (a1 + a0) sum q / 128 of the own heads
};
struct NoPlanes {};

// Bit k of a 16-bit half after the shift that brings bits 10..15 to 4..9.
__device__ __forceinline__ constexpr int plane_pos(int k) { return k <= 9 ? k : k - 6; }

// Coordinate of k-slot half h (0 low, 1 high) for bit k of source dword j of
// lane group kq.
template <int BITS>
__device__ __forceinline__ int plane_coord(int kq, int j, int k, int h) {
    if constexpr (BITS == 2) return 32 * kq + 16 * j + 8 * h + (k >> 1);
    return 32 * kq + 16 * h + k;  // 1-bit codes: one bit per coordinate
}

// Own head j (0, 1) of lane group kq: on the bit-plane path the head pair of
// the group's output rows, else the layout of own_scores.
template <bool PLANES>
__device__ __forceinline__ int fused_own_head(int kq, int j) {
    if constexpr (PLANES) return 2 * kq + j;
    return own_head<8>(kq, j);
}

// MFMA row r of the bit-plane products: head r / 2, lo half when r is odd.
__device__ __forceinline__ int plane_row(int r) { return (r & 1) ? 8 + (r >> 1) : (r >> 1); }

// Query operands of the single-launch kernel: 8 heads, 8 waves, wave w
// owns head w (its q_rot in registers) and the q_proj rows 16 w .. 16 w + 15.
// Fills s_a / s_ap (fp16 hi and lo rows of q_rot and q_proj, as the scores
// MFMAs of every key format read them) and, for bit-plane keys, this lane's
// PlaneOps.  Scratch (all of it may alias the score area; a barrier must
// follow before the area is reused): fq: fp32 q_rot [8][128] in rows of kQRow
// floats (the padding puts the 8 rows in different banks); red: 16 floats of
// per-head sums and maxima; tab: the plane operand table, 4 BITS x 64 half8
// (operand u of lane l at u * 64 + l).  Four steps and three barriers:
// rotation, projection, table, each lane's operands.
template <bool PROJ, bool PLANES, int BITS, typename PO>
__device__ __forceinline__ void fused_query_setup(const QueryLoads<8, PROJ, 8> &ql, const AttnArgs &a,
                                                  _Float16 (*s_a)[128], _Float16 (*s_ap)[128], float (*fq)[kQRow],
                                                  float *red, half8 *tab, PO &po) {
    constexpr int G = 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, kq = lane >> 4;
    // q_rot = H D q / sqrt(d) of head `wave` (q itself for unrotated keys)
    {
        float v0 = h2f(ql.q0[0]), v1 = h2f(ql.q1[0]);
        if (a.k_rotated) {
            v0 *= ql.sg0;
            v1 *= ql.sg1;
            fwht128_lanes(v0, v1, lane);
            v0 *= kRsqrtD;
            v1 *= kRsqrtD;
        }
        put_hi_lo(&s_a[wave][lane], &s_a[G + wave][lane], v0);
        put_hi_lo(&s_a[wave][lane + 64], &s_a[G + wave][lane + 64], v1);
        if constexpr (PLANES) {
            fq[wave][lane] = v0;
            fq[wave][lane + 64] = v1;
            const float sx = quad_sum(row16_sum(v0 + v1));
            const float mx = quad_max(row16_max(fmaxf(fabsf(v0), fabsf(v1))));
            if (lane == 0) {
                red[wave] = sx;
                red[G + wave] = mx;
            }
        }
    }
    __syncthreads();
    // q_proj = S q_rot on the matrix cores: rows = projections 16 wave + [0, 16),
    // columns = the hi (c < 8) and lo (c >= 8) rows of every head
    if constexpr (PROJ) {
        half8 bq[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) bq[st] = *reinterpret_cast<const half8 *>(&s_a[c][32 * kq + 8 * st]);
        floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql.sf[st], bq[st], acc, 0, 0, 0);
        // lane (c, kq) holds projections 16 wave + 4 kq + j of column c; the
        // head's value is column c plus column c + 8 (row rotate by 8)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p = acc[j] + dpp_mov<0x128>(acc[j]);
            const int idx = 16 * wave + 4 * kq + j;
            if (c < G) put_hi_lo(&s_ap[c][idx], &s_ap[G + c][idx], p);
        }
        __syncthreads();
    }
    if constexpr (PLANES) {
        float mq = 0.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) mq = fmaxf(mq, red[G + h]);
        float a1, a0;
        if constexpr (BITS == 2) {
            a1 = 0.5f * (a.tab->levels[1][3] + a.tab->levels[1][2]);
            a0 = 0.5f * (a.tab->levels[1][3] - a.tab->levels[1][2]);
        } else {
            a1 = a0 = a.tab->levels[0][1];
        }
        int e_cb = 0;
        (void)frexpf(mq * 2.0f * fmaxf(a1, a0), &e_cb);
        const int s0_cb = 14 - e_cb;  // every |A| < 2^14
        // the epilogue scales by the fp16 norm itself: 1/128 = 1/sqrt(d)^2
        // and the change to log2 units go into the constants
        po.sc_cb = ldexpf(1.0f, 24 - s0_cb) * (kLog2e / 128.0f);
        const float f1 = 2.0f * a1 * ldexpf(1.0f, s0_cb), f0 = 2.0f * a0 * ldexpf(1.0f, s0_cb);
        // table entry e = (operand u, lane 16 ekq + r); row r is half r & 1
        // (hi, lo) of head r / 2
        for (int e = tid; e < 4 * BITS * 64; e += 8 * 64) {
            const int u = e >> 6, ekq = (e >> 4) & 3, r = e & 15;
            const bool lo = (r & 1) != 0;
            const int hr = r >> 1;
            half8 v;
            const int j = u >> 2, uu = u & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = 4 * uu + i;
                    const float f = (BITS == 2 && (k & 1)) ? f1 : f0;
                    const float x = fq[hr][plane_coord<BITS>(ekq, j, k, h)] * f * ldexpf(1.0f, -plane_pos(k));
                    const _Float16 xh = _Float16(x);
                    v[2 * i + h] = lo ? _Float16(x - float(xh)) : xh;
                }
            tab[e] = v;
        }
        // head constants: sum_i q c[idx] = sum (2 coef q) bit - (a1 + a0) sum q
        // (1 bit: a sum q)
#pragma unroll
        for (int jo = 0; jo < 2; ++jo)
            po.ccb[jo] = (BITS == 2 ? a1 + a0 : a1) * red[fused_own_head<true>(kq, jo)] * (kLog2e / 128.0f);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4 * BITS; ++u) po.ab[u] = tab[u * 64 + lane];
    }
}

// Scores one slice of 1- or 2-bit codebook keys on the bit-plane path (the
// products and epilogue of score_ktiles with its PlaneOps) with the tiles
// software-pipelined: the matrix products of tile i + 1 are issued before
// the epilogue of tile i (token scales, row fold, head constants, LDS
// store), so that the epilogue's vector work runs while the matrix cores are
// busy instead of after them.  Then the slice's (max, sum) update.
template <bool FULL, int BITS, bool PROJ, typename KT, typename Store, typename PO>
__device__ __forceinline__ void score_planes_slice(const KT &d, int base, int t1, int wave, int t, int kq,
                                                   const half8 *s_sgn, const half8 (&ap)[4], Store &&store,
                                                   float (&m)[2], float (&l)[2], const PO &po) {
    constexpr int G = 8, NT = KT::NT;
    static_assert(kOwn<G> == 2, "two own heads per lane");
    float scv[NT][2];
    floatx4 d0[NT], d1[NT];
    auto products = [&](auto I) {
        constexpr int i = decltype(I)::value;
        d0[i] = d1[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < BITS; ++j) {
            const uint32_t w = d.wk[i][j], ws = w >> 6;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t bw[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int k = 4 * u + q4;
                    bw[q4] = (k <= 9 ? w : ws) & (0x00010001u << plane_pos(k));
                }
                d0[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    po.ab[4 * j + u], __builtin_bit_cast(half8, make_uint4(bw[0], bw[1], bw[2], bw[3])), d0[i], 0, 0,
                    0);
            }
        }
        if constexpr (PROJ) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                d1[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[s], s_sgn[(d.sw[i] >> (8 * s)) & 0xFFu], d1[i], 0, 0,
                                                               0);
        }
    };
    // scores in log2 units: log2(e) s, with s = (n/d) <q_rot, c> +
    // (sqrt(pi/2)/m)(gamma/sqrt d) <q_proj, sign>
    auto epilogue = [&](auto I) {
        constexpr int i = decltype(I)::value;
        const int tok = base + wave * 16 + 16 * kFW * i + t;
        const bool valid = FULL || tok < t1;
        const float cn = h2f(d.nn[i] & 0xFFFFu);
        const float cg = PROJ ? h2f(d.nn[i] >> 16) * (kQjlOverSqrtD * kLog2e) : 0.0f;
        const float n = cn * po.sc_cb;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // rows 4kq + 2j (hi) and 4kq + 2j + 1 (lo) of head 2kq + j
            const float cb = d0[i][2 * j] + d0[i][2 * j + 1];
            float o = PROJ ? fmaf(n, cb, cg * (d1[i][2 * j] + d1[i][2 * j + 1])) : n * cb;
            o = fmaf(-cn, po.ccb[j], o);
            if (valid) store(2 * kq + j, tok, o);
            scv[i][j] = valid ? o : -INFINITY;
        }
    };
    constexpr int kMfma = 4 * BITS + (PROJ ? 4 : 0);
    Unroll<NT>::run([&](auto I) {
        constexpr int i = decltype(I)::value;
        products(I);
        if constexpr (i > 0) {
            epilogue(std::integral_constant<int, i - 1>{});
            // ask the scheduler to spread the vector work over the products:
            // the table reads first, then one product after every few
            // vector instructions
            if constexpr (PROJ) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int r = 0; r < kMfma; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
    });
    epilogue(std::integral_constant<int, NT - 1>{});
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float mx = scv[0][j];
#pragma unroll
        for (int i = 1; i < NT; ++i) mx = fmaxf(mx, scv[i][j]);
        const float nm = fmaxf(m[j], mx);
        const float mb = nm == -INFINITY ? 0.0f : nm;
        float acc = l[j] * fast_exp2(m[j] - mb);
#pragma unroll
        for (int i = 0; i < NT; ++i) acc += fast_exp2(scv[i][j] - mb);
        l[j] = acc;
        m[j] = nm;
    }
}

// Fused kernel for rows whose tokens fit the block range; rows of the grid y
// = (sequence, kv head), x = block of the row.  a.sync: a departure counter
// per row; a.stats: [rows][nblk][8] 64-bit (max, sum) slots; both zero
// between calls.
// APPEND: a decode step that also appends the new token (AttnArgs::append
// 2): the block whose range holds the new position encodes it first.
template <int KK, int KB, int VK, bool APPEND = false>
__global__ __launch_bounds__(kFThreads) void attn_fused_kernel(AttnArgs a, const uint8_t *__restrict__ kidx,
                                                               const uint8_t *__restrict__ ksign,
                                                               const uint8_t *__restrict__ knorm) {
    constexpr int G = 8;
    static_assert(!APPEND || (KK == TQ_KIND_PROD && VK == TQ_KIND_MSE), "the append encodes TurboQuant K and V");
    constexpr bool PROJ = KK == TQ_KIND_PROD;
    constexpr bool VQ8 = VK == TQ_KIND_Q8;
    static_assert(VK == TQ_KIND_Q8 || VK == TQ_KIND_MSE, "2-bit codebook V or q8 V");
    constexpr int kPairs = KK == TQ_KIND_Q8 ? 1 : 1 << (2 * KB);
    // one LDS block, small lookup tables first: their addresses then fit the
    // 16-bit offset of ds_read and need no per-lookup address arithmetic
    struct Lds {
        uint2 pair[kPairs];
        half8 sgn[PROJ ? 256 : 1];
        float red[kFW][G][2];
        float M[G], invL[G], W[kFW][G], vmax[kFW];
        int ok, last, okw[G];
        __attribute__((aligned(16))) _Float16 a[16][128];
        __attribute__((aligned(16))) _Float16 ap[PROJ ? 16 : 1][128];
        // scores of the block: head h, token t0 + i at sc[h * kFLd + i]
        // (log2 units on the bit-plane path, natural units otherwise);
        // after the V products, the per-wave partial sums [kFW][G][128]
        __attribute__((aligned(16))) float sc[G * kFLd];
    };
    __shared__ Lds lds;
    uint2 *s_pair = lds.pair;
    half8 *s_sgn = lds.sgn;
    auto &s_red = lds.red;
    _Float16 (*s_a)[128] = lds.a;
    _Float16 (*s_ap)[128] = lds.ap;
    float *s_sc = lds.sc;
    float *s_M = lds.M, *s_invL = lds.invL, *s_vmax = lds.vmax;
    auto &s_W = lds.W;
    int &s_ok = lds.ok;
    static_assert(kFW * G * 128 <= G * kFLd, "partial sums fit the score area");

    // every kernel argument of the first loads, requested together so that
    // one wait covers them (else the compiler spreads them over several
    // dependent round trips before the first query load)
    asm volatile("" ::"s"(a.tab), "s"(a.q), "s"(a.vnorm), "s"(kidx), "s"(ksign), "s"(knorm), "s"(a.seq_lens),
                 "s"(a.Hq), "s"(a.Hkv), "s"(a.T), "s"(a.tb), "s"(a.nblk), "s"(a.k_rotated));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = lane & 15, kq = lane >> 4;
    const int blk = blockIdx.x, row = blockIdx.y;  // row = b * Hkv + kvh
    const int b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int64_t head0 = int64_t(b) * a.Hq + int64_t(kvh) * G;
    const int L = seq_len_of(a, b);
    const int t0 = blk * a.tb;
    const int t1 = min(t0 + a.tb, L);
    const int n_tok = max(t1 - t0, 0);
    const int tmax = max(t1 - 1, 0);
    const uint8_t *kid = kidx + int64_t(row) * a.T * (KK == TQ_KIND_Q8 ? 128 : 16 * KB);
    const uint8_t *ksg = ksign + int64_t(row) * a.T * 16;
    const uint8_t *knm = knorm + int64_t(row) * a.T * (KK == TQ_KIND_Q8 ? 8 : (PROJ ? 4 : 2));

    // ---- global reads first: query, tables, V scale words, first K slices
    QueryLoads<G, PROJ, kFW> ql;
    load_query(ql, a, b, kvh);
    float lv[2] = {0.0f, 0.0f};
    if constexpr (KK != TQ_KIND_Q8) {
        if (tid < kPairs) {
            lv[0] = a.tab->levels[KB - 1][tid & ((1 << KB) - 1)];
            lv[1] = a.tab->levels[KB - 1][tid >> KB];
        }
    }
    if constexpr (APPEND) {
        // the new token at position seq_lens[b] (none outside [0, T); L
        // counts it: len_add = 1): the block whose range holds it encodes it
        // before any load of its range; its reads travel with the query's
        const int pos = a.seq_lens[b];
        if (pos >= 0 && pos < a.T && pos >= blk * a.tb && pos < (blk + 1) * a.tb) {
            append_new_token<KB, 2, kFThreads>(a, row, pos, reinterpret_cast<EncodeTables *>(lds.sc),
                                               reinterpret_cast<half8 *>(lds.sc + 1024), tid);
            __syncthreads();
        }
    }
    // largest V norm (codebook V) or block scale (q8 V) of the block's tokens,
    // as fp16 bits (non-negative halves order like their bit patterns):
    // thread i takes tokens t0 + 8 i .. t0 + 8 i + 7, in one or four 16-byte
    // loads when they all lie in the range and the address is 16-byte
    // aligned (else one clamped load each)
    static_assert(8 * kFThreads >= kFTokens, "eight scale words per thread cover the block");
    constexpr int kVW = VQ8 ? 16 : 4;  // dwords per thread
    uint32_t vraw[kVW];
    {
        const int tk = t0 + 8 * tid;
        const uint8_t *vp = a.vnorm + (int64_t(row) * a.T + tk) * (VQ8 ? 8 : 2);
        if (tk + 8 <= t1 && (reinterpret_cast<uintptr_t>(vp) & 15) == 0) {
            const uint4 *src = reinterpret_cast<const uint4 *>(vp);
#pragma unroll
            for (int i = 0; i < kVW / 4; ++i) {
                const uint4 u = src[i];
                vraw[4 * i] = u.x;
                vraw[4 * i + 1] = u.y;
                vraw[4 * i + 2] = u.z;
                vraw[4 * i + 3] = u.w;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int tok = min(tk + r, tmax);
                if constexpr (VQ8) {
                    const uint2 u = reinterpret_cast<const uint2 *>(a.vnorm)[int64_t(row) * a.T + tok];
                    vraw[2 * r] = u.x;
                    vraw[2 * r + 1] = u.y;
                } else {
                    const uint32_t h = reinterpret_cast<const uint16_t *>(a.vnorm)[int64_t(row) * a.T + tok];
                    if (r & 1) vraw[r >> 1] |= h << 16;
                    else vraw[r >> 1] = h;
                }
            }
        }
    }
    asm volatile("" ::: "memory");
    const bool whole = n_tok % kFSlice == 0;
    // K slices in flight ahead of the one being scored
    constexpr int kAhead = 2;
    KTiles<KK, KB> kt[kAhead + 1];
    Unroll<kAhead>::run([&](auto I) {
        constexpr int i = decltype(I)::value;
        if (i == 0 || t0 + i * kFSlice < t1) load_ktiles<kFW>(kt[i], t0 + i * kFSlice, tmax, wave, t, kq, kid, ksg, knm);
    });

    // a row shared by several blocks is summed with atomics: block 0 zeroes
    // it before the barrier
    if (a.nblk > 1 && blk == 0) {
        for (int i = tid; i < G * 128; i += kFThreads)
            __hip_atomic_store(a.out + (head0 + (i >> 7)) * 128 + (i & 127), 0.0f, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int i = tid; i < (16 - 2 * G) * 32; i += kFThreads) {
        reinterpret_cast<uint2 *>(&s_a[2 * G][0])[i] = uint2{0u, 0u};
        if constexpr (PROJ) reinterpret_cast<uint2 *>(&s_ap[2 * G][0])[i] = uint2{0u, 0u};
    }
    if constexpr (PROJ) {
        if (tid < 256) {
            half8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = ((tid >> j) & 1) ? _Float16(1.0f) : _Float16(-1.0f);
            s_sgn[tid] = v;
        }
    }
    if constexpr (KK != TQ_KIND_Q8) {
        if (tid < kPairs) {
            uint32_t hp = 0, lp = 0;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const _Float16 hi = _Float16(lv[u]);
                const _Float16 lo = _Float16(lv[u] - float(hi));
                hp |= uint32_t(__builtin_bit_cast(uint16_t, hi)) << (16 * u);
                lp |= uint32_t(__builtin_bit_cast(uint16_t, lo)) << (16 * u);
            }
            s_pair[tid] = uint2{hp, lp};
        }
    }
    // query operands; 1- and 2-bit codebook keys take bit-plane products
    // (code words as B operands).  Scratch in the score area: fp32 q_rot and
    // q_proj rows (8.25 KB), sums (512 B), the plane operand table (12 KB).
    constexpr bool USE_PLANES = KK != TQ_KIND_Q8 && KB <= 2;
    using PO = typename std::conditional<USE_PLANES, PlaneOps<G, (KB <= 2 ? KB : 1)>, NoPlanes>::type;
    PO po;
    static_assert(8 * kQRow + 128 + 4 * 2 * 64 * 4 <= G * kFLd, "setup scratch fits the score area");
    fused_query_setup<PROJ, USE_PLANES, (KB <= 2 ? KB : 1)>(ql, a, s_a, s_ap, reinterpret_cast<float (*)[kQRow]>(s_sc),
                                                           s_sc + 8 * kQRow,
                                                           reinterpret_cast<half8 *>(s_sc + 8 * kQRow + 128), po);
    // V scale bound of the block (its words were requested before the K
    // tiles, so they have long landed)
    uint32_t vmx = 0;
#pragma unroll
    for (int r = 0; r < kVW; ++r) vmx = max(vmx, max(vraw[r] & 0xFFFFu, vraw[r] >> 16));

    half8 aq[8], ap[4];
    {
        const _Float16 *ra = s_a[lane & 15];
        if constexpr (KK == TQ_KIND_Q8) {
#pragma unroll
            for (int s = 0; s < 4; ++s) aq[s] = *reinterpret_cast<const half8 *>(ra + 32 * s + 8 * kq);
#pragma unroll
            for (int s = 4; s < 8; ++s) aq[s] = half8{};
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint2 v = *reinterpret_cast<const uint2 *>(ra + 32 * kq + 4 * u);
                aq[u] = __builtin_bit_cast(half8, make_uint4(v.x, v.x, v.y, v.y));
            }
        }
        if constexpr (PROJ) {
            // the bit-plane products take their rows in head pairs
            const _Float16 *rp = s_ap[USE_PLANES ? plane_row(lane & 15) : lane & 15];
#pragma unroll
            for (int s = 0; s < 4; ++s) ap[s] = *reinterpret_cast<const half8 *>(rp + 32 * kq + 8 * s);
        }
    }

    __syncthreads();  // the setup scratch in the score area is free again

    // ---- phase 1: scores into LDS, running (max, sum) per own head
    float m[kOwn<G>], l[kOwn<G>];
    int lim[kOwn<G>];
#pragma unroll
    for (int j = 0; j < kOwn<G>; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
        lim[j] = L;
    }
    auto sink = [&](int h, int tok, float v) { s_sc[h * kFLd + (tok - t0)] = v; };
    auto scan = [&](auto full_c) {
        constexpr bool F = decltype(full_c)::value;
        if (t0 >= t1) return;
        // slices are requested kAhead ahead, and only inside the range: the
        // arrival below waits for every outstanding access of the block
        constexpr int NS = kAhead + 1, A = kAhead * kFSlice;
        for (int base = t0;;) {
            bool done = false;
            Unroll<NS>::run([&](auto I) {
                constexpr int i = decltype(I)::value;
                if (done) return;
                if (base + A < t1) load_ktiles<kFW>(kt[(i + kAhead) % NS], base + A, tmax, wave, t, kq, kid, ksg, knm);
                if constexpr (USE_PLANES)
                    score_planes_slice<F, KB, PROJ>(kt[i], base, t1, wave, t, kq, s_sgn, ap, sink, m, l, po);
                else
                    score_ktiles<F, false, G, kFW>(kt[i], base, t1, wave, t, kq, s_pair, s_sgn, aq, ap, sink, lim, m,
                                                   l);
                base += kFSlice;
                done = base >= t1;
            });
            if (done) break;
        }
    };
    if (whole) scan(std::true_type{});
    else scan(std::false_type{});
#pragma unroll
    for (int j = 0; j < kOwn<G>; ++j) {
        const float mx = row16_max(m[j]);
        l[j] = row16_sum(m[j] == -INFINITY ? 0.0f : l[j] * fast_exp2(m[j] - mx));
        m[j] = mx;
        if (t == 0) {
            s_red[wave][fused_own_head<USE_PLANES>(kq, j)][0] = m[j];
            s_red[wave][fused_own_head<USE_PLANES>(kq, j)][1] = l[j];
        }
    }
    // V scale bound of the block
    {
        const float vf = quad_max(row16_max(h2f(vmx)));
        if (lane == 0) s_vmax[wave] = vf;
    }
    __syncthreads();
    // block statistics per head, in natural-log units
    if (a.nblk > 1 && blk == 0) {
        // the zeroed output is visible before this block's statistics are
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    }
    uint64_t *slots = reinterpret_cast<uint64_t *>(a.stats) + int64_t(row) * a.nblk * G;  // [nblk][G]
    float bm = -INFINITY, bl = 0.0f;
    if (tid < G) {
        for (int w = 0; w < kFW; ++w) bm = fmaxf(bm, s_red[w][tid][0]);
        if (bm != -INFINITY)
            for (int w = 0; w < kFW; ++w) bl += s_red[w][tid][1] * fast_exp2(s_red[w][tid][0] - bm);
        bm = bm == -INFINITY ? bm : bm / kLog2e;
        if (a.nblk > 1) {
            // one 64-bit slot carries both values and marks them written: a
            // written slot is never zero (an empty block stores -inf, 0)
            const uint64_t v = uint64_t(__float_as_uint(bm)) | (uint64_t(__float_as_uint(bl)) << 32);
            __hip_atomic_store(slots + int64_t(blk) * G + tid, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- barrier of the row's blocks: wave h waits (bounded spin) until
    // every block's slot of head h is written and reduces them to the exact
    // softmax statistics; the poll returns the data itself, so the wait ends
    // one device-coherent round trip after the last block's store lands.
    // Everything exchanged between blocks goes through device-coherent
    // atomic accesses; acquire/release fences would write back and
    // invalidate the whole L2 instead.
    if (a.nblk > 1) {
        if (wave < G) {
            const uint64_t *sl = slots + wave;
            uint64_t v[4];
            const uint64_t tstart = __builtin_amdgcn_s_memrealtime();
            int ok = 1;
            for (;;) {
                bool missing = false;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = lane + 64 * i;
                    v[i] = c < a.nblk ? __hip_atomic_load(sl + int64_t(c) * G, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : ~uint64_t(0);
                    missing |= v[i] == 0;
                }
                if (__ballot(missing) == 0) break;
                __builtin_amdgcn_s_sleep(1);
                if (__builtin_amdgcn_s_memrealtime() - tstart > kSpinTicks) {
                    ok = 0;
                    break;
                }
            }
            float mc[4], lc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool real = lane + 64 * i < a.nblk;
                mc[i] = real ? __uint_as_float(uint32_t(v[i])) : -INFINITY;
                lc[i] = real ? __uint_as_float(uint32_t(v[i] >> 32)) : 0.0f;
            }
            float mm = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
            mm = quad_max(row16_max(mm));
            float ll = 0.0f;
            if (mm != -INFINITY)
#pragma unroll
                for (int i = 0; i < 4; ++i) ll += mc[i] == -INFINITY ? 0.0f : lc[i] * fast_exp2((mc[i] - mm) * kLog2e);
            ll = quad_sum(row16_sum(ll));
            if (lane == 0) {
                s_M[wave] = mm;
                s_invL[wave] = ll > 0.0f ? 1.0f / ll : 0.0f;
                lds.okw[wave] = ok;
            }
        }
    } else {
        if (tid < G) {
            s_M[tid] = bm;
            s_invL[tid] = bl > 0.0f ? 1.0f / bl : 0.0f;
            lds.okw[tid] = 1;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int ok = 1;
        for (int w = 0; w < G; ++w) ok &= lds.okw[w];
        s_ok = ok;
    }
    __syncthreads();

    // ---- phase 2: V products of the block's range
    float vmaxf = 0.0f;
#pragma unroll
    for (int w = 0; w < kFW; ++w) vmaxf = fmaxf(vmaxf, s_vmax[w]);
    // A operands: weight x (V norm | q8 block scale) x vsh < 2^14
    int vexp = 0;
    (void)frexpf(vmaxf, &vexp);
    const float vsh = ldexpf(kAMax, -vexp);
    const int n = lane & 15;
    const bool lo_half = n >= G;
    const int hn = n & (G - 1);
    const int jo = lo_half ? 4 : 0;  // lanes n and n + 8 weigh tokens 0-3 and 4-7 of their eight
    // A value of a token = p vsh = exp2(s log2(e) - Cy) with p = exp(s - M)/L
    // (1/L and vsh = 2^(14 - vexp) in the exponent); kept when p >= tau, i.e.
    // when the exponent is at least log2(tau) + 14 - vexp
    const float lsh = float(14 - vexp);
    const float Cy = s_M[hn] * kLog2e - log2f(s_invL[hn]) - lsh;
    const float keep_y = log2f(a.tau) + lsh;
    const int vrow = row;
    // uniform row bases and unsigned 32-bit byte offsets (one scalar-base +
    // vector-offset access per load)
    const uint8_t *vrow_codes = a.vidx + int64_t(vrow) * a.T * (VQ8 ? 128 : 32);
    const uint32_t lane_cw = VQ8 ? uint32_t(4 * n) : uint32_t(4 * (n >> 1));  // this lane's word of a token row
    const uint32_t half_sel = (n & 1) ? 0x07060302u : 0x05040100u;
    const uint8_t *vrow_scl = a.vnorm + int64_t(vrow) * a.T * (VQ8 ? 8 : 2);
    auto code_word = [&](int tok, uint32_t w) {
        return *reinterpret_cast<const uint32_t *>(vrow_codes + (uint32_t(tok) * (VQ8 ? 128u : 32u) + lane_cw + w));
    };
    constexpr int NC = VQ8 ? 16 : 8;  // code dwords per lane and group
    constexpr int NA = VQ8 ? 16 : 4;  // A-operand dwords

    const int nfull = n_tok >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int ng = wv < nfull ? (nfull - 1 - wv) / kFW + 1 : 0;
    auto gbase = [&](int k) { return t0 + 32 * (wv + kFW * min(k, ng - 1)); };
    // q8 scales need all four blocks of each token: kept as four uint2
    auto load_q8scl = [&](int tbs, uint2 (&sc)[4], bool tail) {
        const int tk = tbs + 8 * kq + jo;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sc[j] = *reinterpret_cast<const uint2 *>(vrow_scl + uint32_t(tail ? min(tk + j, tmax) : tk + j) * 8u);
    };
    auto load_norms = [&](int tbs, uint32_t (&nr)[2], bool tail) {
        const int tk = tbs + 8 * kq + jo;
        if (tail) {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                h[j] = *reinterpret_cast<const uint16_t *>(vrow_scl + uint32_t(min(tk + j, tmax)) * 2u);
            nr[0] = h[0] | (h[1] << 16);
            nr[1] = h[2] | (h[3] << 16);
        } else {
            __builtin_memcpy(nr, vrow_scl + uint32_t(tk) * 2u, 8);
        }
    };
    auto load_codes = [&](int tbs, bool real, uint32_t (&c)[NC]) {
        const int tk = real ? tbs + 8 * kq : t0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (VQ8) {
                c[2 * j] = code_word(tk + j, 0);
                c[2 * j + 1] = code_word(tk + j, 64);
            } else {
                c[j] = code_word(tk + j, 0);
            }
        }
    };
    auto load_tail_codes = [&](int tbs, uint32_t (&c)[NC]) {
        const int tk = tbs + 8 * kq;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tok = min(tk + j, tmax);
            if constexpr (VQ8) {
                c[2 * j] = code_word(tok, 0);
                c[2 * j + 1] = code_word(tok, 64);
            } else {
                c[j] = code_word(tok, 0);
            }
        }
    };

    floatx4 acc[8][2];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) acc[mm][0] = acc[mm][1] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;  // this lane's sum of A values (head hn), codebook V
    // weights of head hn for tokens tbs + 8kq + jo + [0, 4): p = exp(s - M)/L,
    // kept when p >= tau, times the token's V scale, as this row's fp16 half;
    // returns whether any lane of the wave keeps a token (uniform)
    auto read_sd = [&](int tbs) -> float4 {
        return *reinterpret_cast<const float4 *>(&s_sc[hn * kFLd + (tbs - t0) + 8 * kq + jo]);
    };
    auto weights = [&](int tbs, const float4 &sd, const uint32_t (&nr)[2], const uint2 (&sc)[4], uint32_t (&aw)[NA],
                       auto whole_c) -> bool {
        const float sv[4] = {sd.x, sd.y, sd.z, sd.w};
        float y[4];
        bool kj[4], kept = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            y[j] = fmaf(sv[j], USE_PLANES ? 1.0f : kLog2e, -Cy);
            kj[j] = y[j] >= keep_y;
            if constexpr (!decltype(whole_c)::value) kj[j] = kj[j] && tbs + 8 * kq + jo + j < t1;
            kept |= kj[j];
        }
        if (__ballot(kept) == 0) return false;
        float ws[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ws[j] = kj[j] ? fast_exp2(y[j]) : 0.0f;
#pragma unroll
        for (int blkq = 0; blkq < NA / 4; ++blkq) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (VQ8) {
                    const uint32_t sp = blkq < 2 ? sc[j].x : sc[j].y;
                    v[j] = ws[j] * h2f((sp >> (16 * (blkq & 1))) & 0xFFFFu);
                } else {
                    v[j] = ws[j] * h2f((nr[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
                    wsum += v[j];  // lanes n and n + 8 weigh different tokens
                }
            }
            uint32_t hi[2], lo[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const half2v h = __builtin_convertvector(float2v{v[2 * i], v[2 * i + 1]}, half2v);
                const half2v lw =
                    __builtin_convertvector(float2v{v[2 * i] - float(h[0]), v[2 * i + 1] - float(h[1])}, half2v);
                hi[i] = __builtin_bit_cast(uint32_t, h);
                lo[i] = __builtin_bit_cast(uint32_t, lw);
            }
            uint32_t got[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                got[i] = uint32_t(__builtin_amdgcn_mov_dpp(int(lo_half ? hi[i] : lo[i]), 0x128, 0xF, 0xF, false));
            aw[4 * blkq + 0] = lo_half ? got[0] : hi[0];
            aw[4 * blkq + 1] = lo_half ? got[1] : hi[1];
            aw[4 * blkq + 2] = lo_half ? lo[0] : got[0];
            aw[4 * blkq + 3] = lo_half ? lo[1] : got[1];
        }
        return true;
    };
    auto products = [&](const uint32_t (&aw)[NA], const uint32_t (&c)[NC]) {
        if constexpr (VQ8) {
            half8 A[4];
#pragma unroll
            for (int blkq = 0; blkq < 4; ++blkq)
                A[blkq] = __builtin_bit_cast(half8, make_uint4(aw[4 * blkq], aw[4 * blkq + 1], aw[4 * blkq + 2],
                                                               aw[4 * blkq + 3]));
            const half2v k1152 = half2v{_Float16(1152.0f), _Float16(1152.0f)};
#pragma unroll
            for (int mq = 0; mq < 8; ++mq) {
                const int w = mq >> 2, by = mq & 3;
                const uint32_t sel = uint32_t(by) | (12u << 8) | (uint32_t(4 + by) << 16) | (12u << 24);
                uint32_t bw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x = __builtin_amdgcn_perm(c[4 * i + 2 + w], c[4 * i + w], sel) ^ 0x64806480u;
                    bw[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, x) - k1152);
                }
                const half8 Bv = __builtin_bit_cast(half8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    acc[mq][p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2 * w + p], Bv, acc[mq][p], 0, 0, 0);
            }
        } else {
            const half8 A = __builtin_bit_cast(half8, make_uint4(aw[0], aw[1], aw[2], aw[3]));
            uint32_t cwd[4], cwd1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cwd[i] = __builtin_amdgcn_perm(c[2 * i + 1], c[2 * i], half_sel);
                cwd1[i] = cwd[i] >> 1;
            }
#pragma unroll
            for (int mq = 0; mq < 8; ++mq)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    // bit 2m + p of both token halves, alone in its half: an
                    // exact fp16 power of two (bit 15, the sign, via bit 14)
                    const int k = 2 * mq + p;
                    const uint32_t mask = k == 15 ? 0x40004000u : (0x00010001u << k);
                    uint32_t bw[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) bw[i] = (k == 15 ? cwd1[i] : cwd[i]) & mask;
                    acc[mq][p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A, __builtin_bit_cast(half8, make_uint4(bw[0], bw[1], bw[2], bw[3])), acc[mq][p], 0, 0, 0);
                }
        }
    };
    auto take = [&](const uint32_t (&c)[NC]) {
        asm volatile("" ::"v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(c[4]), "v"(c[5]), "v"(c[6]), "v"(c[7]));
        if constexpr (VQ8)
            asm volatile("" ::"v"(c[8]), "v"(c[9]), "v"(c[10]), "v"(c[11]), "v"(c[12]), "v"(c[13]), "v"(c[14]),
                         "v"(c[15]));
    };
    if (s_ok && ng > 0) {
        // software pipeline two groups deep: step k starts the scale words of
        // group k + 4 and the LDS read of group k + 3's scores, forms the A
        // operands of group k + 2 (scale words issued two steps earlier, its
        // scores one step earlier), starts its code words, and runs the
        // products of group k; three register sets rotate with k mod 3 (the
        // early score read: middle layer ~0.25 us faster over five A/B pairs)
        uint32_t aw[3][NA], c[3][NC];
        uint32_t NR[3][2];
        float4 SD[3];  // scores of group g in slot g mod 3, read one step ahead
        SD[0] = read_sd(gbase(0));
        uint2 SC[3][4];
        bool kp[3] = {false, false, false};
        auto load_scale = [&](int tbs, int p) {
            if constexpr (VQ8) load_q8scl(tbs, SC[p], false);
            else load_norms(tbs, NR[p], false);
        };
        load_scale(gbase(0), 0);
        load_scale(gbase(1), 1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        auto step = [&](int k, auto P) {
            constexpr int p = decltype(P)::value, p1 = (p + 1) % 3, p2 = (p + 2) % 3;
            load_scale(gbase(k + 4), p1);
            asm volatile("" ::: "memory");
            const bool more = k + 2 < ng;
            SD[p] = read_sd(gbase(k + 3));
            kp[p2] = more && weights(gbase(k + 2), SD[p2], NR[p2], SC[p2], aw[p2], std::true_type{});
            load_codes(gbase(k + 2), kp[p2], c[p2]);
            asm volatile("" ::: "memory");
            if (kp[p]) {
                products(aw[p], c[p]);
            } else {
                take(c[p]);
            }
        };
        for (int k = -2; k < ng; k += 3) {
            step(k, std::integral_constant<int, 1>{});
            step(k + 1, std::integral_constant<int, 2>{});
            step(k + 2, std::integral_constant<int, 0>{});
        }
    }
    if (s_ok && (n_tok & 31) != 0 && wv == (nfull & (kFW - 1))) {
        const int tbs = t0 + 32 * nfull;
        // the partial group's scores past t1 are not in LDS: the weights test
        // masks them by position before any use of their value
        uint32_t aw[NA], c[NC], nr[2] = {0u, 0u};
        uint2 sc[4] = {};
        if constexpr (VQ8) load_q8scl(tbs, sc, true);
        else load_norms(tbs, nr, true);
        if (weights(tbs, read_sd(tbs), nr, sc, aw, std::false_type{})) {
            load_tail_codes(tbs, c);
            products(aw, c);
        }
    }

    // ---- combine: rows 4kq + j of column n; rows G + h are the lo halves
    float y[8][4];
    if constexpr (VQ8) {
#pragma unroll
        for (int mq = 0; mq < 8; ++mq)
#pragma unroll
            for (int j = 0; j < 4; ++j) y[mq][j] = n >= 8 ? acc[mq][1][j] : acc[mq][0][j];
    } else {
        const float c2 = a.tab->levels[1][2], c3 = a.tab->levels[1][3];
        const float a1 = 0.5f * (c3 + c2), a0 = 0.5f * (c3 - c2);
#pragma unroll
        for (int mq = 0; mq < 8; ++mq)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                y[mq][j] = (2.0f * a1 / bitval(2 * mq + 1)) * acc[mq][1][j] + (2.0f * a0 / bitval(2 * mq)) * acc[mq][0][j];
    }
#pragma unroll
    for (int mq = 0; mq < 8; ++mq)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const auto r =
                __builtin_amdgcn_permlane32_swap(__float_as_uint(y[mq][j]), __float_as_uint(y[mq][j]), false, false);
            y[mq][j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    // W of head hn: lanes n, n ^ 8 and the four lane groups
    if constexpr (!VQ8) {
        wsum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(wsum), 0x128, 0xF, 0xF, false));
        wsum = quad_sum(wsum);
    }
    __syncthreads();  // every wave is done with the scores in LDS
    float *s_acc = s_sc;  // [kFW][G][128]
    if (kq < 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float *hrow = s_acc + (wave * G + 4 * kq + j) * 128;
            float4 *d0 = reinterpret_cast<float4 *>(hrow + (VQ8 ? 4 * n : 8 * n));
            float4 *d1 = reinterpret_cast<float4 *>(hrow + (VQ8 ? 64 + 4 * n : 8 * n + 4));
            *d0 = make_float4(y[0][j], y[1][j], y[2][j], y[3][j]);
            *d1 = make_float4(y[4][j], y[5][j], y[6][j], y[7][j]);
        }
    }
    if (lane < G) s_W[wave][lane] = VQ8 ? 0.0f : wsum;
    __syncthreads();
    // the block's share of head `wave`, rotated back (R^T = D H / sqrt(d);
    // q8 V is not rotated)
    {
        const int g = wave;
        float v0 = 0.0f, v1 = 0.0f, wt = 0.0f;
#pragma unroll
        for (int w = 0; w < kFW; ++w) {
            v0 += s_acc[(w * G + g) * 128 + lane];
            v1 += s_acc[(w * G + g) * 128 + lane + 64];
            wt += s_W[w][g];
        }
        const float unsh = 1.0f / vsh;
        if constexpr (VQ8) {
            v0 *= unsh;
            v1 *= unsh;
        } else {
            const float wc = a.tab->levels[1][3] * wt;  // (a1 + a0) W = c3 W
            v0 -= wc;
            v1 -= wc;
            fwht128_lanes(v0, v1, lane);
            const float sc = kRsqrtD * kRsqrtD * unsh;
            v0 *= a.tab->signs[lane] * sc;
            v1 *= a.tab->signs[lane + 64] * sc;
        }
        if (!s_ok) {
            v0 = __builtin_nanf("");
            v1 = v0;
        }
        float *o = a.out + (head0 + g) * 128;
        if (a.nblk > 1) {
            if (n_tok > 0 || !s_ok) {
                __hip_atomic_fetch_add(o + lane, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(o + lane + 64, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            o[lane] = v0;
            o[lane + 64] = v1;
        }
    }
    // departure: the last block of the row to leave clears the row's slots
    // and its counter for the next call (no block reads them any more)
    if (a.nblk > 1) {
        uint32_t *depart = a.sync + row;
        if (tid == 0)
            lds.last = __hip_atomic_fetch_add(depart, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       uint32_t(a.nblk) - 1;
        __syncthreads();
        if (lds.last) {
            for (int i = tid; i < a.nblk * G; i += kFThreads)
                __hip_atomic_store(slots + i, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0) __hip_atomic_store(depart, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------------------------ launch
template <int KK, int KB, int VK>
static int launch_fused_t(const AttnArgs &a, hipStream_t s) {
    dim3 grid(unsigned(a.nblk), unsigned(a.B * a.Hkv));
    if constexpr (KK == TQ_KIND_PROD && VK == TQ_KIND_MSE) {
        if (a.append) {
            hipLaunchKernelGGL((attn_fused_kernel<KK, KB, VK, true>), grid, dim3(kFThreads), 0, s, a, a.kidx,
                               a.ksign, a.knorm);
            return int(hipGetLastError());
        }
    }
    hipLaunchKernelGGL((attn_fused_kernel<KK, KB, VK>), grid, dim3(kFThreads), 0, s, a, a.kidx, a.ksign, a.knorm);
    return int(hipGetLastError());
}

template <int VK>
static int fused_dispatch_k(const AttnArgs &a, tq_format kf, hipStream_t s) {
    if (kf.kind == TQ_KIND_Q8) return launch_fused_t<TQ_KIND_Q8, 8, VK>(a, s);
    if (kf.kind == TQ_KIND_PROD) {
        switch (kf.bits) {
            case 1: return launch_fused_t<TQ_KIND_PROD, 1, VK>(a, s);
            case 2: return launch_fused_t<TQ_KIND_PROD, 2, VK>(a, s);
            case 3: return launch_fused_t<TQ_KIND_PROD, 3, VK>(a, s);
        }
    } else {
        switch (kf.bits) {
            case 1: return launch_fused_t<TQ_KIND_MSE, 1, VK>(a, s);
            case 2: return launch_fused_t<TQ_KIND_MSE, 2, VK>(a, s);
            case 3: return launch_fused_t<TQ_KIND_MSE, 3, VK>(a, s);
            case 4: return launch_fused_t<TQ_KIND_MSE, 4, VK>(a, s);
        }
    }
    return int(hipErrorInvalidValue);
}

int launch_attn_fused(const AttnArgs &a, tq_format kf, tq_format vf, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (vf.kind == TQ_KIND_Q8) return fused_dispatch_k<TQ_KIND_Q8>(a, kf, s);
    if (vf.kind == TQ_KIND_MSE && vf.bits == 2) return fused_dispatch_k<TQ_KIND_MSE>(a, kf, s);
    return int(hipErrorInvalidValue);
}

// Blocks of the fused kernel resident at once on the current device (the
// occupancy calculator's per-CU count times the CU count), cached per device;
// 0 when the kernel cannot be resident.  The grid of the fused path never
// exceeds it when a row spans several blocks.
int fused_capacity() {
    static int cache[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    const int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v != 0) return v > 0 ? v : 0;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(attn_fused_kernel<TQ_KIND_PROD, 2, TQ_KIND_MSE>), kFThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        per_cu = cus = 0;
    const int cap = per_cu > 0 && cus > 0 ? per_cu * cus : 0;
    __atomic_store_n(&cache[dev], cap > 0 ? cap : -1, __ATOMIC_RELAXED);
    return cap;
}

}  // namespace tq
