// Single-token decode attention over a packed TurboQuant KV cache (gfx950).
//
// chenxutan.com, "TurboQuant+ deep dive", 1.1: one query per step against all
// cached keys/values; 3.3 and yeyulingfeng.com TurboQuant+ introduction, core
// item 4: V rows whose softmax weight is below 1e-6 are not dequantised, and
// the kept weights are not renormalised.  quidproquo.cc, "TurboQuant+ KV cache
// compression", Stage 2: the K score carries the QJL inner-product estimate.
//
// The packed K rows are never dequantised.  With q_rot = R q and
// q_proj = S q_rot, the score of token j is
//   s_j = (1/sqrt d) [ n_j/sqrt(d) <q_rot, c[idx_j]>
//                      + sqrt(pi/2)/m * gamma_j <q_proj, 2 bit_j - 1> ],
// which equals <q, k_hat_j>/sqrt(d) for the dequantised row.  V is
// accumulated in the rotated domain and rotated back once per head.
//
// Passes (one stream, no host synchronisation):
//   1. scores   grid (chunk, batch*kv head).  Each block first forms q_rot and
//               q_proj of the g query heads of its kv head (q_proj on MFMA)
//               while its first K tiles are being fetched, then scores 16-token
//               tiles with v_mfma_f32_16x16x32_f16 (rows = query heads), two
//               slices of kSlice tokens in flight ahead of the one scored.
//               Scores go to the workspace with per-chunk (max, sum exp) per
//               head; the block of chunk 0 zeroes the output.
//   2. values   combines the chunk statistics into the exact softmax
//               normaliser and accumulates the kept weights times V in the
//               rotated domain, then rotates each block's share back (R^T) and
//               adds it into the output with fp32 atomics.  Two kernels:
//               - compacting (same grid): keeps tokens with some weight >= tau,
//                 compacts them (up to 1024 at a time, all loads issued
//                 together) and accumulates weight * level per coordinate;
//               - matrix cores (8 query heads, 2-bit codebook V): every 32-token
//                 group is one set of MFMA products, see below.
// Exact sparse V needs the global softmax statistics before any V row is
// skipped, hence the kernel boundary between passes 1 and 2.
#include "attn_common.h"

namespace tq {

// The extra block of an appending decode step (256 threads): encodes the
// new token of its row at position pos (K by wave 0, V by wave 1, with the
// encode kernels' tile code) while waves 2 and 3 form the query operands of
// the row's G heads, q_rot = R q and q_proj = S q_rot, in fp32; then wave 0
// scores the stored token for every head with the rotated-domain formula of
// the scan,
//   s_h = (1/sqrt d) [ n/sqrt(d) <q_rot, c[idx]> + sqrt(pi/2)/m gamma <q_proj, 2 bit - 1> ],
// and writes the scores at position pos and the statistics (max = the score,
// sum = 1) of the extra chunk column.  LDS scratch: et (two EncodeTables),
// frag (2048 half8), qr ([2G][128] fp32: q_rot rows, then q_proj rows).
template <int G, int KB, int VB>
__device__ __forceinline__ void append_and_score(const AttnArgs &a, int b, int kvh, int row, int pos,
                                                 int64_t head0, float *scores, EncodeTables *et, half8 *frag,
                                                 float (*qr)[128], int tid) {
    constexpr float kQjl = 1.2533141373155003f / 128.0f;  // sqrt(pi/2) / m
    const int wave = tid >> 6, lane = tid & 63;
    // waves 2 and 3: the query rows of heads wave - 2, wave, ... (in flight
    // with the encode's loads)
    constexpr int kH = (G + 1) / 2;
    uint32_t q0[kH], q1[kH];
    float d0 = 0.0f, d1 = 0.0f;
    if (wave >= 2) {
#pragma unroll
        for (int i = 0; i < kH; ++i) {
            const int h = wave - 2 + 2 * i;
            const uint16_t *q = a.q + io_row(a, b, kvh, h < G ? h : 0) * kHeadDim;
            q0[i] = q[lane];
            q1[i] = q[lane + 64];
        }
        d0 = a.tab->signs[lane];
        d1 = a.tab->signs[lane + 64];
    }
    append_new_token<KB, VB, 256>(a, row, pos, et, frag, tid);
    if (wave >= 2) {
#pragma unroll
        for (int i = 0; i < kH; ++i) {
            const int h = wave - 2 + 2 * i;
            if (h >= G) break;
            float v0 = h2f(q0[i]) * d0, v1 = h2f(q1[i]) * d1;
            fwht128_lanes(v0, v1, lane);
            qr[h][lane] = v0 * kRsqrtD;
            qr[h][lane + 64] = v1 * kRsqrtD;
        }
        // q_proj rows p = lane, lane + 64 of this wave's heads, S from row-major [m][d]
        const half8 *S8 = reinterpret_cast<const half8 *>(a.tab->S);
        float pr[kH][2];
#pragma unroll
        for (int i = 0; i < kH; ++i) pr[i][0] = pr[i][1] = 0.0f;
#pragma unroll 2
        for (int k8 = 0; k8 < 16; ++k8) {
            const half8 sa = S8[lane * 16 + k8], sb = S8[(lane + 64) * 16 + k8];
#pragma unroll
            for (int i = 0; i < kH; ++i) {
                const int h = wave - 2 + 2 * i;
                if (h >= G) break;
                const float4 qa = *reinterpret_cast<const float4 *>(&qr[h][8 * k8]);
                const float4 qb = *reinterpret_cast<const float4 *>(&qr[h][8 * k8 + 4]);
                const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pr[i][0] = fmaf(float(sa[j]), qv[j], pr[i][0]);
                    pr[i][1] = fmaf(float(sb[j]), qv[j], pr[i][1]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kH; ++i) {
            const int h = wave - 2 + 2 * i;
            if (h >= G) break;
            qr[G + h][lane] = pr[i][0];
            qr[G + h][lane + 64] = pr[i][1];
        }
    }
    __syncthreads();  // the new rows are stored, the query rows are in LDS
    if (wave != 0) return;
    const int dst = row * a.T + pos;
    const uint32_t *iw = reinterpret_cast<const uint32_t *>(a.kw.idx + size_t(dst) * (16 * KB));
    const uint4 sg = *reinterpret_cast<const uint4 *>(a.kw.sign + size_t(dst) * 16);
    const uint32_t nn = reinterpret_cast<const uint32_t *>(a.kw.norm)[dst];
    const float n = h2f(nn & 0xFFFFu), gamma = h2f(nn >> 16);
    float lev[2], sgn[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = lane + 64 * u;
        // code i: bits i*KB .. i*KB + KB - 1 of the row's bitstream
        const int o = i * KB, w = o >> 5, sh = o & 31;
        uint32_t c = iw[w] >> sh;
        if (sh + KB > 32) c |= iw[w + 1] << (32 - sh);
        lev[u] = a.tab->levels[KB - 1][c & ((1u << KB) - 1u)];
        const uint32_t word = u == 0 ? (lane < 32 ? sg.x : sg.y) : (lane < 32 ? sg.z : sg.w);
        sgn[u] = ((word >> (lane & 31)) & 1u) ? 1.0f : -1.0f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float dc = quad_sum(row16_sum(qr[h][lane] * lev[0] + qr[h][lane + 64] * lev[1]));
        const float dq = quad_sum(row16_sum(qr[G + h][lane] * sgn[0] + qr[G + h][lane + 64] * sgn[1]));
        const float sc = kRsqrtD * (n * kRsqrtD * dc + kQjl * gamma * dq);
        if (lane == 0) {
            scores[(head0 + h) * a.ld_scores + pos] = sc;
            float *stt = a.stats + ((head0 + h) * a.n_chunks + a.n_chunks - 1) * 2;
            stt[0] = sc;
            stt[1] = 1.0f;
        }
    }
}

// APPEND: a decode step that also appends the new token (AttnArgs::append
// 1): one extra block per row, in grid rows after the chunks' rows, encodes
// it and scores only it (append_and_score).
template <int G, int KIND, int BITS, bool APPEND = false>
__global__ __launch_bounds__(256) void attn_scores_kernel(AttnArgs a, const uint8_t *kidx,
                                                          const uint8_t *ksign,
                                                          const uint8_t *knorm,
                                                          float *__restrict__ scores) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "1, 2, 4 or 8 query heads per kv head");
    static_assert(!APPEND || KIND == TQ_KIND_PROD, "the append encodes TurboQuant K");
    // s_pair[f]: fp16 hi halves and fp16 lo halves of the two levels of a
    // 2-code field f = c0 | c1 << BITS; s_sgn[byte]: eight fp16 +-1 (bit set -> +1)
    constexpr int kPairs = KIND == TQ_KIND_Q8 ? 1 : 1 << (2 * BITS);
    __shared__ uint2 s_pair[kPairs];
    __shared__ half8 s_sgn[KIND == TQ_KIND_PROD ? 256 : 1];
    __shared__ float s_red[4][16][2];  // per wave, per head: (max, sum)
    __shared__ __attribute__((aligned(16))) _Float16 s_a[16][128];
    __shared__ __attribute__((aligned(16))) _Float16 s_ap[KIND == TQ_KIND_PROD ? 16 : 1][128];
    __shared__ EncodeTables s_et[APPEND ? 2 : 1];
    __shared__ half8 s_fr[APPEND ? 2048 : 1];
    __shared__ float s_qr[APPEND ? 2 * G : 1][128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = lane & 15, kq = lane >> 4;
    if constexpr (APPEND) {
        // the extra blocks (grid rows past the B * Hkv rows of chunks, so
        // that they are dispatched last): block r of them encodes the new
        // token of row r at position seq_lens[b] (none outside [0, T)) and
        // scores it as the one-token chunk a.n_chunks - 1; the other chunks
        // end before it (L = the clamped seq_lens[b])
        const int rows = a.B * a.Hkv;
        if (int(blockIdx.y) >= rows) {
            const int row = (int(blockIdx.y) - rows) * int(gridDim.x) + int(blockIdx.x);
            if (row >= rows) return;
            const int b = row / a.Hkv, kvh = row - b * a.Hkv;
            const int64_t head0 = int64_t(b) * a.Hq + int64_t(kvh) * G;
            const int chunk_id = a.n_chunks - 1;
            const int pos = a.seq_lens[b];
            if (pos >= 0 && pos < a.T) {
                switch (a.vbits) {
                    case 1: append_and_score<G, BITS, 1>(a, b, kvh, row, pos, head0, scores, s_et, s_fr, s_qr, tid); break;
                    case 2: append_and_score<G, BITS, 2>(a, b, kvh, row, pos, head0, scores, s_et, s_fr, s_qr, tid); break;
                    case 3: append_and_score<G, BITS, 3>(a, b, kvh, row, pos, head0, scores, s_et, s_fr, s_qr, tid); break;
                    default: append_and_score<G, BITS, 4>(a, b, kvh, row, pos, head0, scores, s_et, s_fr, s_qr, tid); break;
                }
            } else if (tid < G) {
                float *st = a.stats + ((head0 + tid) * a.n_chunks + chunk_id) * 2;
                st[0] = -INFINITY;
                st[1] = 0.0f;
            }
            return;
        }
    }
    const int chunk_id = blockIdx.x, row = blockIdx.y;  // row = b*Hkv + kvh
    const int b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int64_t head0 = int64_t(b) * a.Hq + int64_t(kvh) * G;
    const int L = seq_len_of(a, b);
    const int t0 = chunk_id * a.chunk;
    const int t1 = min(t0 + a.chunk, L);
    // per-(batch, kv head) bases of the planes; token offsets below are 32-bit
    // (T * 128 < 2^31 is checked on the host)
    const int krow = kv_row(a, row);
    const uint8_t *kid = kidx + int64_t(krow) * a.T * (KIND == TQ_KIND_Q8 ? 128 : 16 * BITS);
    const uint8_t *ksg = ksign + int64_t(krow) * a.T * 16;
    const uint8_t *knm = knorm + int64_t(krow) * a.T * (KIND == TQ_KIND_Q8 ? 8 : (KIND == TQ_KIND_PROD ? 4 : 2));

    // global reads first: query, D, S fragments, levels and the first slice's
    // K tiles are all in flight while the tables are built.  A chunk whose
    // length is a multiple of 512 has only whole slices and takes the path
    // without per-token bounds checks.
    QueryLoads<G, KIND == TQ_KIND_PROD> ql;
    load_query(ql, a, b, kvh);
    float lv[2] = {0.0f, 0.0f};
    if constexpr (KIND != TQ_KIND_Q8) {
        if (tid < kPairs) {
            lv[0] = a.tab->levels[BITS - 1][tid & ((1 << BITS) - 1)];
            lv[1] = a.tab->levels[BITS - 1][tid >> BITS];
        }
    }
    // keep these small loads ahead of the K tiles in the memory queue, so
    // the query setup below does not wait for the (slower) K tiles
    asm volatile("" ::: "memory");
    // rows past the sequence (or of an empty chunk) read row tmax instead.
    // Three slices rotate through ta, tb, tc: two are in flight while the
    // third is scored, enough bytes in flight to cover the memory latency.
    const int n_tok = max(t1 - t0, 0);
    const bool whole = n_tok % kSlice == 0;
    const int tmax = max(t1 - 1, 0);
    KTiles<KIND, BITS> ta, tb, tc;
    load_ktiles(ta, t0, tmax, wave, t, kq, kid, ksg, knm);
    load_ktiles(tb, t0 + kSlice, tmax, wave, t, kq, kid, ksg, knm);

    // the output rows of this kv head start at zero; the values pass adds
    // every chunk's share into them
    if (chunk_id == 0) {
        for (int i = tid; i < G * 128; i += 256) a.out[io_row(a, b, kvh, i >> 7) * 128 + (i & 127)] = 0.0f;
    }
    // zero stacked rows 2G .. 15
    for (int i = tid; i < (16 - 2 * G) * 32; i += 256) {
        reinterpret_cast<uint2 *>(&s_a[2 * G][0])[i] = uint2{0u, 0u};
        if constexpr (KIND == TQ_KIND_PROD) reinterpret_cast<uint2 *>(&s_ap[2 * G][0])[i] = uint2{0u, 0u};
    }
    if constexpr (KIND == TQ_KIND_PROD) {
        half8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ((tid >> j) & 1) ? _Float16(1.0f) : _Float16(-1.0f);
        s_sgn[tid] = v;
    }
    if constexpr (KIND != TQ_KIND_Q8) {
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
    build_query_rows<G>(ql, a, s_a, s_ap);

    // A operands, row r = l&15 of the stacked rows.  Rotated keys: k-step
    // u of lane group kq covers coordinates c0 = 32 kq + 4u .. c0+3 as
    // (q0 q1 q0 q1 q2 q3 q2 q3) against (hi hi lo lo hi hi lo lo) of the
    // levels; the QJL k-step s covers 32 kq + 8s .. +7.  q8 keys: k-step s
    // covers 32 s + 8 kq .. +7.
    half8 aq[8], ap[4];
    {
        const _Float16 *ra = s_a[lane & 15];
        if constexpr (KIND == TQ_KIND_Q8) {
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
        if constexpr (KIND == TQ_KIND_PROD) {
            const _Float16 *rp = s_ap[lane & 15];
#pragma unroll
            for (int s = 0; s < 4; ++s) ap[s] = *reinterpret_cast<const half8 *>(rp + 32 * kq + 8 * s);
        }
    }
    float m[kOwn<G>], l[kOwn<G>];
    int lim[kOwn<G>];  // tokens seen by the row of each own head
#pragma unroll
    for (int j = 0; j < kOwn<G>; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
        lim[j] = L - row_shift(a, own_head<G>(kq, j));
    }

    auto sink = [&](int h, int tok, float v) { scores[(head0 + h) * a.ld_scores + tok] = v; };
    // the scan: every load is unconditional (clamped rows), so the wait
    // before scoring a slice covers exactly that slice's loads.  The K planes
    // are not declared __restrict__, and a compiler barrier follows each
    // request: otherwise the compiler is free to move a slice's loads past
    // the loop exits to just before the slice is scored, and the scan then
    // waits for each slice's loads in turn (the needle batch's scores pass:
    // 84 us with the loads kept in place, 91 us with them moved)
    auto scan = [&](auto full_c, auto rowlim_c) {
        constexpr bool F = decltype(full_c)::value;
        constexpr bool RL = decltype(rowlim_c)::value;
        if (t0 >= t1) return;
        for (int base = t0;;) {
            load_ktiles(tc, base + 2 * kSlice, tmax, wave, t, kq, kid, ksg, knm);
            asm volatile("" ::: "memory");  // issued here, two slices ahead
            score_ktiles<F, RL, G>(ta, base, t1, wave, t, kq, s_pair, s_sgn, aq, ap, sink, lim, m, l);
            base += kSlice;
            if (base >= t1) break;
            load_ktiles(ta, base + 2 * kSlice, tmax, wave, t, kq, kid, ksg, knm);
            asm volatile("" ::: "memory");  // issued here, two slices ahead
            score_ktiles<F, RL, G>(tb, base, t1, wave, t, kq, s_pair, s_sgn, aq, ap, sink, lim, m, l);
            base += kSlice;
            if (base >= t1) break;
            load_ktiles(tb, base + 2 * kSlice, tmax, wave, t, kq, kid, ksg, knm);
            asm volatile("" ::: "memory");  // issued here, two slices ahead
            score_ktiles<F, RL, G>(tc, base, t1, wave, t, kq, s_pair, s_sgn, aq, ap, sink, lim, m, l);
            base += kSlice;
            if (base >= t1) break;
        }
    };
    // rows with their own causal limit only in multi-query prefill groups
    if (a.qp > 1) {
        if (whole) scan(std::true_type{}, std::true_type{});
        else scan(std::false_type{}, std::true_type{});
    } else {
        if (whole) scan(std::true_type{}, std::false_type{});
        else scan(std::false_type{}, std::false_type{});
    }
    // (max, sum) per head: over the 16 token lanes of each lane group, then
    // over the waves; m is kept in log2 units and stored in natural units
#pragma unroll
    for (int j = 0; j < kOwn<G>; ++j) {
        const float mx = row16_max(m[j]);
        l[j] = row16_sum(m[j] == -INFINITY ? 0.0f : l[j] * fast_exp2(m[j] - mx));
        m[j] = mx;
        if (t == 0 && (G >= 4 || kq < G)) {
            s_red[wave][own_head<G>(kq, j)][0] = m[j];
            s_red[wave][own_head<G>(kq, j)][1] = l[j];
        }
    }
    __syncthreads();
    if (tid < G) {
        float mm = -INFINITY;
        for (int w = 0; w < 4; ++w) mm = fmaxf(mm, s_red[w][tid][0]);
        float ll = 0.0f;
        if (mm != -INFINITY)
            for (int w = 0; w < 4; ++w) ll += s_red[w][tid][1] * fast_exp2(s_red[w][tid][0] - mm);
        float *st = a.stats + ((head0 + tid) * a.n_chunks + chunk_id) * 2;
        st[0] = mm == -INFINITY ? mm : mm / kLog2e;
        st[1] = ll;
    }
}

// ------------------------------------------------------------------ values
template <int G, int KIND, int BITS>
__global__ __launch_bounds__(kVThreads) void attn_values_kernel(AttnArgs a) {
    // tokens compacted together (one super-slice); fewer for 8 heads, whose
    // accumulators take twice the registers
    constexpr int kSuper = G >= 8 ? 512 : 1024;
    constexpr int R = kSuper / kVThreads;  // tokens per thread per super-slice
    // s_vpair[f]: the two levels of a 2-code field f = c0 | c1 << BITS
    constexpr int kVPairs = KIND == TQ_KIND_Q8 ? 1 : 1 << (2 * BITS);
    __shared__ float s_M[G], s_invL[G];
    __shared__ ValuesLds<G, KIND, BITS, kSuper> lds;
    float2 *s_vpair = lds.vpair;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk_id = blockIdx.x, row = blockIdx.y;
    const int b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int64_t head0 = int64_t(b) * a.Hq + int64_t(kvh) * G;
    const int L = seq_len_of(a, b);
    const int t0 = chunk_id * a.chunk;
    const int t1 = min(t0 + a.chunk, L);
    if (t0 >= t1) return;  // an empty chunk adds nothing (uniform over the block)
    const int tmax = t1 - 1;
    const float *sc_base = a.scores + head0 * a.ld_scores;
    const int vrow = kv_row(a, row);
    const uint16_t *vn_base = reinterpret_cast<const uint16_t *>(a.vnorm) + int64_t(vrow) * a.T;

    // every global read of the prologue is issued before any is used: the
    // levels, the chunk statistics of head `wave`, and the scores and V norms
    // of the first super-slice (tokens past the chunk read row tmax and are
    // masked out later)
    float2 lv = make_float2(0.0f, 0.0f);
    if constexpr (KIND != TQ_KIND_Q8) {
        const int f = tid & (kVPairs - 1);
        lv = make_float2(a.tab->levels[BITS - 1][f & ((1 << BITS) - 1)], a.tab->levels[BITS - 1][f >> BITS]);
    }
    const float *st = a.stats + (head0 + min(wave, G - 1)) * a.n_chunks * 2;
    const float2 st0 = *reinterpret_cast<const float2 *>(st + 2 * min(lane, a.n_chunks - 1));
    float sv[R][G];
    uint32_t vraw[R];
    auto load_super = [&](int base) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tt = min(base + kVThreads * r + tid, tmax);
#pragma unroll
            for (int g = 0; g < G; ++g) sv[r][g] = sc_base[int64_t(g) * a.ld_scores + tt];
            if constexpr (KIND != TQ_KIND_Q8) vraw[r] = vn_base[tt];
        }
    };
    load_super(t0);
    asm volatile("" ::: "memory");

    if constexpr (KIND != TQ_KIND_Q8) {
        if (tid < kVPairs) s_vpair[tid] = lv;
    }
    // exact softmax statistics from all chunks of this (batch, kv head)
    if (wave < G) {
        float mm = lane < a.n_chunks ? st0.x : -INFINITY;
        for (int c = lane + 64; c < a.n_chunks; c += 64) mm = fmaxf(mm, st[2 * c]);
        mm = quad_max(row16_max(mm));
        float ll = 0.0f;
        if (mm != -INFINITY) {
            if (lane < a.n_chunks) ll = st0.y * fast_exp2((st0.x - mm) * kLog2e);
            for (int c = lane + 64; c < a.n_chunks; c += 64) ll += st[2 * c + 1] * fast_exp2((st[2 * c] - mm) * kLog2e);
        }
        ll = quad_sum(row16_sum(ll));
        if (lane == 0) {
            s_M[wave] = mm;
            s_invL[wave] = ll > 0.0f ? 1.0f / ll : 0.0f;
        }
    }
    __syncthreads();
    values_compact<G, KIND, BITS, kSuper, true>(a, b, kvh, vrow, t0, t1, s_M, s_invL, sv, vraw, load_super, lds);
}

// ------------------------------------- values pass on MFMA: 2-bit V and q8 V
// A symmetric 4-level codebook (c0 = -c3, c1 = -c2) is a sum of two signed
// constants chosen by the two bits of the code:
//   c[2 b1 + b0] = a1 (2 b1 - 1) + a0 (2 b0 - 1),  a1 = (c3 + c2) / 2,  a0 = (c3 - c2) / 2.
// The rotated-domain V sum of head h over coordinate x is therefore
//   sum_t w_ht n_t c[code_tx] / sqrt(d) = -(a1 X1 + a0 X0) / sqrt(d),
//   X_p[h][x] = sum_t w_ht n_t (1 - 2 bit_p(code_tx)),
// and each X_p is a [2G x T] x [T x 128] product on the matrix cores
// (v_mfma_f32_16x16x32_f16, 32 tokens per step): A = the kept weights as fp16
// hi (rows h) and lo (rows G + h) halves, scaled by 2^15 so both stay in
// range; B = the token's fp16 norm with the code bit as its sign, exact.
// Lane (kq, n) of a wave holds tokens 8kq + [0, 8) of the 32-token group as
// k-slots, for A row n and for B column n; column n of product m is
// coordinate 8n + m, whose two code bits are bits 2m, 2m + 1 of the 16-bit
// word n of the token's row.  Every token of a chunk is stepped over; a group
// in which no head keeps a token is skipped as a whole.
//
// 3- and 4-bit codebook V: B = the level of the token's code, as fp16 hi
// and lo halves (two products per column block), two tokens at a time from
// an LDS table indexed by both codes (64 / 256 entries);
// the token's norm goes into A (weight x norm, scaled below 2^14 by the
// block's largest norm); the sum is the rotated-domain V sum times that
// scale and sqrt(d).  Coordinates 8n + [0, 8) of a token are dword n of its
// 64-byte row (4-bit), or bits 24n + [0, 24) of its 48-byte row (3-bit: two
// dwords, the second clamped to the row, joined by one funnel shift).
//
// q8 V (boundary layers): x = q s_blk with int8 q and one fp16 scale per 32
// coordinates.  B = q as fp16 (exact: the byte becomes the mantissa of
// 1024 + (q + 128) through v_perm and an xor, then one packed fp16 subtract
// of 1152), and the scale goes into A: four A operands per group, the kept
// weights times the scale of block 0..3, each as hi/lo halves.  Column n of
// product m is coordinate 4n + (m & 3) + 64 (m >> 2), so product m needs the
// blocks 2 (m >> 2) and 2 (m >> 2) + 1: two products per m, and lane n keeps
// the one for its own block (n < 8 or n >= 8).
constexpr int kMThreads = 256;
constexpr int kMWaves = kMThreads / 64;
constexpr float kWScale = 32768.0f;  // 2^15

// (the 4-bit instance is held to three waves per SIMD, 168 registers: the
// grouped prefill at Tq 2048 takes 9.0-9.1 ms against 9.8-10.0 ms at two;
// the 3-bit one, with twice the code dwords in flight, would spill there)
template <int G, int VK, int VB>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(VK == TQ_KIND_MSE && VB == 4 ? 3 : 1)))
void attn_values_mfma_kernel(AttnArgs a) {
    static_assert(G == 8, "rows: 8 heads x (hi, lo)");
    static_assert(VK == TQ_KIND_Q8 || (VK == TQ_KIND_MSE && VB >= 2 && VB <= 4), "2/3/4-bit codebook V or q8 V");
    constexpr bool Q8 = VK == TQ_KIND_Q8;
    constexpr bool LUT = VK == TQ_KIND_MSE && VB >= 3;  // levels from the table, norms in A
    constexpr bool SCL = Q8 || LUT;                     // A = weight x a per-token factor
    constexpr int NC = Q8 || VB == 3 ? 16 : 8;  // code dwords per lane and group
    constexpr int NN = LUT || Q8 ? 1 : 4;  // norm dwords per lane and group (2-bit: in B)
    constexpr int NA = Q8 ? 16 : 4;  // A-operand dwords (q8: one operand per block)
    constexpr int NS = Q8 ? 4 : 1;   // q8 scale pairs or (4-bit) four norms, uint2, per lane and group
    __shared__ float s_M[G], s_invL[G], s_qmax[kMWaves];
    // 3/4-bit: entry c0 | c1 << VB = the levels of codes c0, c1 as fp16 (hi
    // halves, lo halves): one B dword of a token pair for each product
    __shared__ uint2 s_lv2[LUT ? 1 << (2 * VB) : 1];
    __shared__ int s_any[kMWaves];
    __shared__ __attribute__((aligned(16))) float s_acc[kMWaves][G][128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.y;
    const int b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int64_t head0 = int64_t(b) * a.Hq + int64_t(kvh) * G;
    const int L = seq_len_of(a, b);
    const int t0 = int(blockIdx.x) * a.vsub;
    const int t1 = min(t0 + a.vsub, L);
    if (t0 >= t1) return;  // uniform over the block
    const int tmax = t1 - 1;
    const int kq = lane >> 4, n = lane & 15;
    // A row n: head hn, fp16 hi half (n < G) or lo half (G <= n < 2G); rows
    // from 2G on stay zero
    const bool arow = n < 2 * G;
    const bool lo_half = n >= G;
    const int hn = n < G ? n : (n < 2 * G ? n - G : 0);
    const float *srow = a.scores + (head0 + hn) * int64_t(a.ld_scores);
    const int vrow = kv_row(a, row);
    // 2-bit: the dword that holds 16-bit word n of each 32-byte row; 4-bit:
    // dword n of each 64-byte row; 3-bit: the dword that holds bit 24n of
    // each 48-byte row (and the next one, clamped to the row: c3n1)
    constexpr int kRowDw = 4 * VB;  // code dwords per row (codebook V)
    const int c3n0 = VB == 3 ? (3 * n) >> 2 : 0, c3n1 = VB == 3 ? min(c3n0 + 1, kRowDw - 1) - c3n0 : 0;
    const uint32_t c3sh = VB == 3 ? uint32_t(24 * n) & 31u : 0u;
    const uint32_t *cwd32 = reinterpret_cast<const uint32_t *>(a.vidx) + int64_t(vrow) * a.T * kRowDw +
                            (VB == 4 ? n : VB == 3 ? c3n0 : (n >> 1));
    // v_perm selector joining half (n & 1) of two dwords: that half of the
    // second operand (bytes 0-3) in bits 0-15, of the first (bytes 4-7) in 16-31
    const uint32_t half_sel = (n & 1) ? 0x07060302u : 0x05040100u;
    const uint16_t *vn = reinterpret_cast<const uint16_t *>(a.vnorm) + int64_t(vrow) * a.T;
    // q8: dwords n and 16 + n of each 128-byte row (coordinates 4n.. and
    // 64 + 4n..), and the four fp16 block scales of each token
    const uint32_t *q8w = reinterpret_cast<const uint32_t *>(a.vidx) + int64_t(vrow) * a.T * 32 + n;
    const uint2 *q8s = reinterpret_cast<const uint2 *>(a.vnorm) + int64_t(vrow) * a.T;

    // 32-token groups: lane (kq, n) reads the scores of head hn for tokens
    // 8kq + [0, 8) (score rows are padded to 32 tokens, so a group is always
    // in bounds), and code word n and the fp16 norm of the same tokens.  Whole
    // groups lie inside [t0, t1); only the last group of a block may be
    // partial, and its code words and norms clamp to the last token.
    const int nfull = (t1 - t0) >> 5;  // whole groups of the block
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int ng = wv < nfull ? (nfull - 1 - wv) / kMWaves + 1 : 0;  // whole groups of this wave
    auto gbase = [&](int k) { return t0 + 32 * (wv + kMWaves * min(k, ng - 1)); };
    // scores (and q8 scales) of three consecutive groups rotate through
    // three register sets
    float4 S[3];
    uint2 SC[3][NS];
    // lanes n and n + 8 (the hi and lo rows of head hn) each take four of
    // the eight tokens 8kq + [0, 8): tokens jo + [0, 4)
    const int jo = lo_half ? 4 : 0;
    auto load_scores = [&](int tb, float4 &sd, uint2 (&sc)[NS]) {
        sd = *reinterpret_cast<const float4 *>(srow + tb + 8 * kq + jo);
        if constexpr (Q8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[j] = q8s[min(tb + 8 * kq + jo + j, tmax)];
        } else if constexpr (LUT) {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = vn[min(tb + 8 * kq + jo + j, tmax)];
            sc[0] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
    };
    // code words and norms of a whole group; a group that keeps no token
    // reads the block's first tokens instead (the same cache lines every
    // time), so that every step issues the same loads and the memory waits
    // stay exact
    // (the code words come in as the dword that holds word n; products()
    // picks the half)
    auto load_codes = [&](int tb, bool real, uint32_t (&c)[NC], uint32_t (&nr)[NN]) {
        const int tk = real ? tb + 8 * kq : t0;
        if constexpr (Q8) {
            const uint32_t *cp = q8w + int64_t(tk) * 32;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c[2 * j] = cp[32 * j];
                c[2 * j + 1] = cp[32 * j + 16];
            }
        } else if constexpr (LUT && VB == 3) {
            const uint32_t *cp = cwd32 + int64_t(tk) * kRowDw;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c[2 * j] = cp[kRowDw * j];
                c[2 * j + 1] = cp[kRowDw * j + c3n1];
            }
        } else if constexpr (LUT) {
            const uint32_t *cp = cwd32 + int64_t(tk) * 16;
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = cp[16 * j];
        } else {
            const uint32_t *cp = cwd32 + int64_t(tk) * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = cp[8 * j];
            __builtin_memcpy(nr, vn + tk, 16);
        }
    };
    auto load_tail = [&](int tb, uint32_t (&c)[NC], uint32_t (&nr)[NN]) {
        const int tk = tb + 8 * kq;
        if constexpr (Q8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t *cp = q8w + int64_t(min(tk + j, tmax)) * 32;
                c[2 * j] = cp[0];
                c[2 * j + 1] = cp[16];
            }
        } else if constexpr (LUT && VB == 3) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t *cp = cwd32 + int64_t(min(tk + j, tmax)) * kRowDw;
                c[2 * j] = cp[0];
                c[2 * j + 1] = cp[c3n1];
            }
        } else if constexpr (LUT) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = cwd32[int64_t(min(tk + j, tmax)) * 16];
        } else {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tj = min(tk + j, tmax);
                c[j] = cwd32[int64_t(tj) * 8];
                h[j] = vn[tj];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) nr[i] = h[2 * i] | (h[2 * i + 1] << 16);
        }
    };
    if (ng > 0) {
        load_scores(gbase(0), S[0], SC[0]);
        load_scores(gbase(1), S[1], SC[1]);
    }
    const float c2 = SCL ? 0.0f : a.tab->levels[1][2], c3 = SCL ? 0.0f : a.tab->levels[1][3];
    if constexpr (LUT) {
        static_assert(kMThreads >= (1 << (2 * VB)), "one pair-table entry per thread");
        if (tid < (1 << (2 * VB))) {
            uint32_t h2[2], l2[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float lv = a.tab->levels[VB - 1][(tid >> (VB * u)) & ((1 << VB) - 1)];
                const _Float16 hi = _Float16(lv);
                const _Float16 lo = _Float16(lv - float(hi));
                h2[u] = __builtin_bit_cast(uint16_t, hi);
                l2[u] = __builtin_bit_cast(uint16_t, lo);
            }
            s_lv2[tid] = make_uint2(h2[0] | (h2[1] << 16), l2[0] | (l2[1] << 16));
        }
    }
    const float *st = a.stats + (head0 + min(wave, G - 1)) * a.n_chunks * 2;
    const float2 st0 = *reinterpret_cast<const float2 *>(st + 2 * min(lane, a.n_chunks - 1));
    asm volatile("" ::: "memory");
    // q8 V: the A operands are weight x block scale, 4-bit V weight x norm;
    // the block's largest scale or norm bounds them (fp16 bits of
    // non-negative halves order like the values; 2-bit V: weights <= 1,
    // scaled by 2^15)
    if constexpr (SCL) {
        uint32_t mx = 0;
        for (int tk = t0 + tid; tk < t1; tk += kMThreads) {
            if constexpr (Q8) {
                const uint2 u = q8s[tk];
                mx = max(mx, max(max(u.x & 0xFFFFu, u.x >> 16), max(u.y & 0xFFFFu, u.y >> 16)));
            } else {
                mx = max(mx, uint32_t(vn[tk]));
            }
        }
        const float mf = quad_max(row16_max(h2f(mx)));
        if (lane == 0) s_qmax[wave] = mf;
    }

    // exact softmax statistics of every head from all chunk statistics
    for (int h = wave; h < G; h += kMWaves) {
        const float *sth = a.stats + (head0 + h) * a.n_chunks * 2;
        const float2 f0 = h == wave ? st0 : *reinterpret_cast<const float2 *>(sth + 2 * min(lane, a.n_chunks - 1));
        float mm = lane < a.n_chunks ? f0.x : -INFINITY;
        for (int c = lane + 64; c < a.n_chunks; c += 64) mm = fmaxf(mm, sth[2 * c]);
        mm = quad_max(row16_max(mm));
        float ll = 0.0f;
        if (mm != -INFINITY) {
            if (lane < a.n_chunks) ll = f0.y * fast_exp2((f0.x - mm) * kLog2e);
            for (int c = lane + 64; c < a.n_chunks; c += 64) ll += sth[2 * c + 1] * fast_exp2((sth[2 * c] - mm) * kLog2e);
        }
        ll = quad_sum(row16_sum(ll));
        if (lane == 0) {
            s_M[h] = mm;
            s_invL[h] = ll > 0.0f ? 1.0f / ll : 0.0f;
        }
    }
    __syncthreads();
    const float Ml2 = s_M[hn] * kLog2e;
    float ash = kWScale;
    if constexpr (SCL) {
        float mf = 0.0f;
#pragma unroll
        for (int w = 0; w < kMWaves; ++w) mf = fmaxf(mf, s_qmax[w]);
        int e = 0;
        (void)frexpf(mf, &e);
        ash = ldexpf(16384.0f, -e);  // weight x scale x ash < 2^14
    }
    const float invL = s_invL[hn] * ash;  // weights leave scaled by ash
    // p = 2^x / L >= tau  <=>  x >= log2(tau L), x = (s - M) log2(e): the keep
    // test needs no exponential (rows >= 2G keep nothing)
    const float keep_x = arow ? log2f(a.tau) - log2f(s_invL[hn]) : INFINITY;

    floatx4 acc[8][2];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m][0] = acc[m][1] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    bool any = false;  // uniform over the wave
    // weights of head hn for tokens tb + 8kq + j: p = exp(s - M) / L, kept
    // when p >= tau, as this row's fp16 half; returns whether any lane of the
    // wave keeps a token (uniform)
    auto weights = [&](int tb, const float4 &sd, const uint2 (&sc)[NS], uint32_t (&aw)[NA], auto whole) -> bool {
        const float sv[4] = {sd.x, sd.y, sd.z, sd.w};
        float x[4];
        bool kj[4], kept = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = fmaf(sv[j], kLog2e, -Ml2);
            kj[j] = x[j] >= keep_x;
            if constexpr (!decltype(whole)::value) kj[j] = kj[j] && tb + 8 * kq + jo + j < t1;
            kept |= kj[j];
        }
        if (__ballot(kept) == 0) return false;
        float ws[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ws[j] = kj[j] ? fast_exp2(x[j]) * invL : 0.0f;
        // one A operand per block scale (q8) or a single one (2-bit)
#pragma unroll
        for (int blk = 0; blk < NA / 4; ++blk) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (Q8) {  // the token's scale of block blk
                    const uint32_t sp = blk < 2 ? sc[j].x : sc[j].y;
                    v[j] = ws[j] * h2f((sp >> (16 * (blk & 1))) & 0xFFFFu);
                } else if constexpr (LUT) {  // the token's norm
                    const uint32_t sp = j < 2 ? sc[0].x : sc[0].y;
                    v[j] = ws[j] * h2f((sp >> (16 * (j & 1))) & 0xFFFFu);
                } else {
                    v[j] = ws[j];
                }
            }
            uint32_t hi[2], lo[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const half2v h = __builtin_convertvector(float2v{v[2 * i], v[2 * i + 1]}, half2v);
                const half2v l =
                    __builtin_convertvector(float2v{v[2 * i] - float(h[0]), v[2 * i + 1] - float(h[1])}, half2v);
                hi[i] = __builtin_bit_cast(uint32_t, h);
                lo[i] = __builtin_bit_cast(uint32_t, l);
            }
            // the partner lane (n ^ 8, same DPP row) needs the other half of
            // these four tokens: hi rows take tokens 4-7's hi halves from
            // their lo partner, lo rows tokens 0-3's lo halves from their hi
            // partner
            uint32_t got[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                got[i] = uint32_t(__builtin_amdgcn_mov_dpp(int(lo_half ? hi[i] : lo[i]), 0x128, 0xF, 0xF, false));
            aw[4 * blk + 0] = lo_half ? got[0] : hi[0];
            aw[4 * blk + 1] = lo_half ? got[1] : hi[1];
            aw[4 * blk + 2] = lo_half ? lo[0] : got[0];
            aw[4 * blk + 3] = lo_half ? lo[1] : got[1];
        }
        return true;
    };
    auto products = [&](const uint32_t (&aw)[NA], const uint32_t (&c)[NC], const uint32_t (&nr)[NN]) {
        if constexpr (Q8) {
            half8 A[4];
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
                A[blk] = __builtin_bit_cast(half8, make_uint4(aw[4 * blk], aw[4 * blk + 1], aw[4 * blk + 2],
                                                              aw[4 * blk + 3]));
            const half2v k1152 = half2v{_Float16(1152.0f), _Float16(1152.0f)};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                // byte m & 3 of dword (m >> 2) of tokens 2i and 2i + 1 as the
                // low bytes of two fp16 halves 0x64..: 1024 + (q + 128)
                const int w = m >> 2, by = m & 3;
                const uint32_t sel = uint32_t(by) | (12u << 8) | (uint32_t(4 + by) << 16) | (12u << 24);
                uint32_t bw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x = __builtin_amdgcn_perm(c[4 * i + 2 + w], c[4 * i + w], sel) ^ 0x64806480u;
                    bw[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, x) - k1152);
                }
                const half8 B = __builtin_bit_cast(half8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    acc[m][p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2 * w + p], B, acc[m][p], 0, 0, 0);
            }
        } else if constexpr (LUT) {
            const half8 A = __builtin_bit_cast(half8, make_uint4(aw[0], aw[1], aw[2], aw[3]));
            // 4-bit, token pair i (tokens 2i, 2i + 1): byte k of pe[i] is
            // code 2k of the first | code 2k of the second << 4, of po[i] the
            // same for code 2k + 1 (coordinates 8n + 2k and 8n + 2k + 1).
            // 3-bit: f[j] = the eight 3-bit codes of token j.
            uint32_t pe[4], po[4], f[8];
            if constexpr (VB == 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pe[i] = (c[2 * i] & 0x0F0F0F0Fu) | ((c[2 * i + 1] & 0x0F0F0F0Fu) << 4);
                    po[i] = ((c[2 * i] >> 4) & 0x0F0F0F0Fu) | (c[2 * i + 1] & 0xF0F0F0F0u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] = __builtin_amdgcn_alignbit(c[2 * j + 1], c[2 * j], c3sh);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                // coordinate 8n + m of the eight tokens: hi halves into one B
                // operand, lo halves into another, a token pair per table read
                uint32_t bh[4], bl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t e;
                    if constexpr (VB == 4)
                        e = (((m & 1) ? po[i] : pe[i]) >> (8 * (m >> 1))) & 0xFFu;
                    else
                        e = ((f[2 * i] >> (3 * m)) & 7u) | (((f[2 * i + 1] >> (3 * m)) & 7u) << 3);
                    const uint2 v = s_lv2[e];
                    bh[i] = v.x;
                    bl[i] = v.y;
                }
                acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    A, __builtin_bit_cast(half8, make_uint4(bh[0], bh[1], bh[2], bh[3])), acc[m][0], 0, 0, 0);
                acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    A, __builtin_bit_cast(half8, make_uint4(bl[0], bl[1], bl[2], bl[3])), acc[m][1], 0, 0, 0);
            }
        } else {
            const half8 A = __builtin_bit_cast(half8, make_uint4(aw[0], aw[1], aw[2], aw[3]));
            uint32_t cwd[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) cwd[i] = __builtin_amdgcn_perm(c[2 * i + 1], c[2 * i], half_sel);
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    // bit p of coordinate 8n + m moved to the fp16 sign bit of
                    // both token halves, over the (positive) norms
                    const int sh = 15 - 2 * m - p;
                    uint32_t bw[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) bw[i] = ((cwd[i] << sh) & 0x80008000u) | nr[i];
                    acc[m][p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A, __builtin_bit_cast(half8, make_uint4(bw[0], bw[1], bw[2], bw[3])), acc[m][p], 0, 0, 0);
                }
        }
    };
    // a group that keeps no token still takes delivery of its (cache-resident)
    // loads, so that no later reuse of these registers has to wait for
    // everything in flight
    auto take = [&](const uint32_t (&c)[NC], const uint32_t (&nr)[NN]) {
        asm volatile("" ::"v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(c[4]), "v"(c[5]), "v"(c[6]), "v"(c[7]));
        if constexpr (NC == 16)
            asm volatile("" ::"v"(c[8]), "v"(c[9]), "v"(c[10]), "v"(c[11]), "v"(c[12]), "v"(c[13]), "v"(c[14]),
                         "v"(c[15]));
        else if constexpr (!LUT)
            asm volatile("" ::"v"(nr[0]), "v"(nr[1]), "v"(nr[2]), "v"(nr[3]));
    };
    // software pipeline over this wave's whole groups k = 0 .. ng-1, two
    // groups deep.  Step k starts the scores of group k+4, forms the weights
    // of group k+2 (scores issued two steps earlier), starts its code words
    // and norms, and runs the products of group k (code words issued two
    // steps earlier); steps -2 and -1 only fill the pipeline.  Three register
    // sets rotate with k mod 3, so nothing is copied while its load is
    // outstanding.
    if (ng > 0) {
        uint32_t aw[3][NA], c[3][NC], nr[3][NN];
        bool kp[3] = {false, false, false};
        // the loop starts with nothing in flight but its own loads (so the
        // compiler's memory waits inside it stay exact): vmcnt(0)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        auto step = [&](int k, auto P) {
            constexpr int p = decltype(P)::value, p1 = (p + 1) % 3, p2 = (p + 2) % 3;
            load_scores(gbase(k + 4), S[p1], SC[p1]);
            asm volatile("" ::: "memory");
            const bool more = k + 2 < ng;
            kp[p2] = more && weights(gbase(k + 2), S[p2], SC[p2], aw[p2], std::true_type{});
            load_codes(gbase(k + 2), kp[p2], c[p2], nr[p2]);
            asm volatile("" ::: "memory");
            if (kp[p]) {
                any = true;
                products(aw[p], c[p], nr[p]);
            } else {
                take(c[p], nr[p]);
            }
        };
        // steps run in threes (the last ones may lie past ng and only issue
        // cache-resident loads), so the loop has a single exit
        for (int k = -2; k < ng; k += 3) {
            step(k, std::integral_constant<int, 1>{});
            step(k + 1, std::integral_constant<int, 2>{});
            step(k + 2, std::integral_constant<int, 0>{});
        }
    }
    if (((t1 - t0) & 31) != 0 && wv == (nfull & (kMWaves - 1))) {
        const int tb = t0 + 32 * nfull;
        uint32_t aw[NA], c[NC], nr[NN];
        load_scores(tb, S[0], SC[0]);
        if (weights(tb, S[0], SC[0], aw, std::false_type{})) {
            any = true;
            load_tail(tb, c, nr);
            products(aw, c, nr);
        }
    }
    // lane (kq, n) holds rows 4kq + j, column n of every product: coordinate
    // 8n + m of row 4kq + j is -(a1 X1 + a0 X0) (times 2^-15 / sqrt(d), applied
    // with R^T below); add each head's lo row to its hi row
    // (q8: the product of this lane's own block, 2^15 sum w s q)
    const float a1 = 0.5f * (c3 + c2), a0 = 0.5f * (c3 - c2);
    float y[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            y[m][j] = Q8    ? (n >= 8 ? acc[m][1][j] : acc[m][0][j])
                      : LUT ? acc[m][0][j] + acc[m][1][j]
                            : fmaf(a1, acc[m][1][j], a0 * acc[m][0][j]);
    // rows 4kq + j and 4(kq + 2) + j are the hi and lo rows of head 4kq + j
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const auto r =
                __builtin_amdgcn_permlane32_swap(__float_as_uint(y[m][j]), __float_as_uint(y[m][j]), false, false);
            y[m][j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    // heads 4kq + j (kq < 2) go to this wave's slot
    if (kq < 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float *hrow = &s_acc[wave][4 * kq + j][0];
            float4 *d0 = reinterpret_cast<float4 *>(hrow + (Q8 ? 4 * n : 8 * n));
            float4 *d1 = reinterpret_cast<float4 *>(hrow + (Q8 ? 64 + 4 * n : 8 * n + 4));
            *d0 = make_float4(y[0][j], y[1][j], y[2][j], y[3][j]);
            *d1 = make_float4(y[4][j], y[5][j], y[6][j], y[7][j]);
        }
    }
    if (lane == 0) s_any[wave] = any ? 1 : 0;
    __syncthreads();
    bool kept_any = false;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) kept_any |= s_any[w] != 0;
    // the block's share of each head, rotated back (R^T = D H / sqrt(d); q8
    // V is not rotated) and added into the output, which the scores pass
    // zeroed
    if (kept_any) {
        // 2-bit: -(a1 X1 + a0 X0); 4-bit: the sum itself
        const float sc = (LUT ? kRsqrtD : -kRsqrtD) * kRsqrtD / ash;
        for (int g = wave; g < G; g += kMWaves) {
            float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
            for (int w = 0; w < kMWaves; ++w) {
                v0 += s_acc[w][g][lane];
                v1 += s_acc[w][g][lane + 64];
            }
            if constexpr (Q8) {
                v0 *= 1.0f / ash;
                v1 *= 1.0f / ash;
            } else {
                fwht128_lanes(v0, v1, lane);
                v0 *= a.tab->signs[lane] * sc;
                v1 *= a.tab->signs[lane + 64] * sc;
            }
            float *o = a.out + io_row(a, b, kvh, g) * 128;
            __hip_atomic_fetch_add(o + lane, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(o + lane + 64, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------------------------ launch
template <int G, int KK, int KB, int VK, int VB>
static int launch_passes(const AttnArgs &as, hipStream_t s) {
    dim3 grid(unsigned(as.n_chunks), unsigned(as.B * as.Hkv));
    if constexpr (KK == TQ_KIND_PROD) {
        if (as.append) {
            // the chunks of every row, then the rows' extra blocks (the last
            // chunk column of the statistics) in grid rows of their own
            const unsigned nc = unsigned(as.n_chunks - 1), rows = unsigned(as.B * as.Hkv);
            const dim3 sgrid(nc, rows + (rows + nc - 1) / nc);
            hipLaunchKernelGGL((attn_scores_kernel<G, KK, KB, true>), sgrid, dim3(256), 0, s, as, as.kidx, as.ksign,
                               as.knorm, as.scores);
        } else
            hipLaunchKernelGGL((attn_scores_kernel<G, KK, KB>), grid, dim3(256), 0, s, as, as.kidx, as.ksign,
                               as.knorm, as.scores);
    } else {
        hipLaunchKernelGGL((attn_scores_kernel<G, KK, KB>), grid, dim3(256), 0, s, as, as.kidx, as.ksign, as.knorm,
                           as.scores);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return int(e);
    // with an append the values pass sees the new token too (in the chunk
    // that holds its position; the statistics have one column more)
    AttnArgs a = as;
    if (a.append) {
        a.len_add = 1;
        grid.x = unsigned(a.n_chunks - 1);
    }
    if constexpr (G == 8 && ((VK == TQ_KIND_MSE && VB >= 2) || VK == TQ_KIND_Q8)) {
        // 8 query heads: the kept rows of all heads together are most of the
        // tokens unless attention is very peaked, and the per-row cost of the
        // compacting pass grows with the head count, so the whole range goes
        // through the matrix cores.  Blocks of vsub tokens, ~512 blocks in all.
        const int64_t rows = int64_t(a.B) * a.Hkv;
        const int64_t per = (int64_t(a.T) * rows + 511) / 512;
        AttnArgs v = a;
        v.vsub = int(std::min<int64_t>(std::max<int64_t>((per + 255) / 256 * 256, 256), (int64_t(a.T) + 31) / 32 * 32));
        const dim3 vgrid(unsigned((a.T + v.vsub - 1) / v.vsub), unsigned(rows));
        hipLaunchKernelGGL((attn_values_mfma_kernel<G, VK, VB>), vgrid, dim3(kMThreads), 0, s, v);
    } else {
        hipLaunchKernelGGL((attn_values_kernel<G, VK, VB>), grid, dim3(kVThreads), 0, s, a);
    }
    return int(hipGetLastError());
}

template <int G, int KK, int KB>
static int dispatch_v(const AttnArgs &a, tq_format vf, hipStream_t s) {
    if (vf.kind == TQ_KIND_Q8) return launch_passes<G, KK, KB, TQ_KIND_Q8, 8>(a, s);
    switch (vf.bits) {
        case 1: return launch_passes<G, KK, KB, TQ_KIND_MSE, 1>(a, s);
        case 2: return launch_passes<G, KK, KB, TQ_KIND_MSE, 2>(a, s);
        case 3: return launch_passes<G, KK, KB, TQ_KIND_MSE, 3>(a, s);
        case 4: return launch_passes<G, KK, KB, TQ_KIND_MSE, 4>(a, s);
    }
    return int(hipErrorInvalidValue);
}

template <int G>
static int dispatch_k(const AttnArgs &a, tq_format kf, tq_format vf, hipStream_t s) {
    if (kf.kind == TQ_KIND_Q8) return dispatch_v<G, TQ_KIND_Q8, 8>(a, vf, s);
    if (kf.kind == TQ_KIND_PROD) {
        switch (kf.bits) {
            case 1: return dispatch_v<G, TQ_KIND_PROD, 1>(a, vf, s);
            case 2: return dispatch_v<G, TQ_KIND_PROD, 2>(a, vf, s);
            case 3: return dispatch_v<G, TQ_KIND_PROD, 3>(a, vf, s);
        }
    } else {
        switch (kf.bits) {
            case 1: return dispatch_v<G, TQ_KIND_MSE, 1>(a, vf, s);
            case 2: return dispatch_v<G, TQ_KIND_MSE, 2>(a, vf, s);
            case 3: return dispatch_v<G, TQ_KIND_MSE, 3>(a, vf, s);
            case 4: return dispatch_v<G, TQ_KIND_MSE, 4>(a, vf, s);
        }
    }
    return int(hipErrorInvalidValue);
}

int launch_attn(const DevTables *tab, const void *q, const void *kp, const void *vp, tq_format kf,
                tq_format vf, const tq_planes_desc &klay, const tq_planes_desc &vlay, int B, int Hq,
                int Hkv, int T, int tq, const int32_t *seq_lens, float tau, float *out, void *ws,
                const AttnPlan &plan, int len_add, const AttnAppend *app, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *w = static_cast<uint8_t *>(ws);
    const uint8_t *kb = static_cast<const uint8_t *>(kp), *vb = static_cast<const uint8_t *>(vp);
    AttnArgs a{};
    a.tab = tab;
    a.q = static_cast<const uint16_t *>(q);
    a.kidx = kb + klay.idx_offset;
    a.ksign = kb + klay.sign_offset;
    a.knorm = kb + klay.norm_offset;
    a.vidx = vb + vlay.idx_offset;
    a.vnorm = vb + vlay.norm_offset;
    a.seq_lens = seq_lens;
    a.scores = reinterpret_cast<float *>(w + plan.off_scores);
    a.stats = reinterpret_cast<float *>(w + plan.off_stats);
    a.out = out;
    a.tau = tau;
    const int qp = prefill_group(Hq / Hkv, tq);
    a.B = B * (tq / qp);  // virtual sequences of qp queries each
    a.tq = tq;
    a.qp = qp;
    a.qg = Hq / Hkv;
    a.hq_io = Hq;
    a.Hq = Hq * qp;
    a.Hkv = Hkv;
    a.T = T;
    a.chunk = plan.chunk;
    a.n_chunks = plan.n_chunks;
    a.ld_scores = plan.ld_scores;
    a.k_rotated = kf.kind != TQ_KIND_Q8;
    a.v_rotated = vf.kind != TQ_KIND_Q8;
    a.len_add = len_add;
    if (app) {
        // the new token of each row goes to position seq_lens[b]: the
        // single-launch kernel encodes it in the block that owns that
        // position; the two-pass scores kernel in an extra chunk column
        uint8_t *kw = static_cast<uint8_t *>(app->k_packed), *vw = static_cast<uint8_t *>(app->v_packed);
        a.k_new = static_cast<const uint16_t *>(app->k_new);
        a.v_new = static_cast<const uint16_t *>(app->v_new);
        a.kw = EncodePlanes{kw + klay.idx_offset, kw + klay.sign_offset, kw + klay.norm_offset, nullptr};
        a.vw = EncodePlanes{vw + vlay.idx_offset, nullptr, vw + vlay.norm_offset, nullptr};
        a.vbits = vf.bits;
        a.append = plan.fused ? 2 : 1;
        if (plan.fused) a.len_add = 1;
        else a.n_chunks = plan.n_chunks + 1;
    }
    if (plan.tiled) {
        // prompt-scale prefill: real sequences and heads, token ranges
        a.B = B;
        a.Hq = Hq;
        a.chunk = plan.chunk;
        a.n_chunks = plan.n_chunks;
        return launch_attn_prefill(a, kf, vf, stream);
    }
    if (block32_format(kf) || block32_format(vf)) return launch_attn_generic(a, kf, vf, stream);
    if (plan.fused) {
        a.sync = reinterpret_cast<uint32_t *>(w + plan.off_sync);
        a.nblk = plan.nblk;
        a.tb = plan.tb;
        return launch_attn_fused(a, kf, vf, stream);
    }
    if (plan.fused4 && !app) {
        // the barrier region at the start of the workspace (counters, then
        // the (max, sum) slots), as for the 8-head kernel
        a.sync = reinterpret_cast<uint32_t *>(w);
        a.stats = reinterpret_cast<float *>(w + kSyncCounterBytes);
        a.nblk = plan.nblk;
        a.tb = plan.tb;
        return launch_attn_fused4(a, kf, vf, stream);
    }
    switch (a.Hq / Hkv) {
        case 1: return dispatch_k<1>(a, kf, vf, s);
        case 2: return dispatch_k<2>(a, kf, vf, s);
        case 4: return dispatch_k<4>(a, kf, vf, s);
        case 8: return dispatch_k<8>(a, kf, vf, s);
    }
    return int(hipErrorInvalidValue);
}

}  // namespace tq
