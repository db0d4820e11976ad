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
//   1. prologue   one wave per (batch, q head): q_rot, q_proj, their sums;
//                 zeroes the per-(batch, kv head) completion counters.
//   2. scores     grid (chunk, batch*kv head); one token per lane, the g query
//                 heads of the kv head share one unpack; scores go to the
//                 workspace with per-chunk (max, sum exp) per head.
//   3. values     same grid; combines the chunk statistics into the exact
//                 softmax normaliser, keeps tokens with some weight >= tau,
//                 compacts them, accumulates weight * level over 8 coordinates
//                 per lane, writes the chunk's partial sum; the last block of
//                 each (batch, kv head) sums the partials and applies R^T.
#include <type_traits>

#include "device_common.h"

namespace tq {

constexpr float kRsqrtD = 0.08838834764831845f;            // 1/sqrt(128)
constexpr float kQjlOverSqrtD = 1.2533141373155003f / 128.0f * 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQc = 8;  // query coordinates per scalar-load chunk

// Read-only data in the constant address space: uniform loads from it become
// scalar (s_load) loads into SGPRs.
typedef const __attribute__((address_space(4))) float *const_fp;
__device__ __forceinline__ const_fp as_const(const float *p) { return (const_fp)p; }

struct AttnArgs {
    const DevTables *tab;
    const uint16_t *q;
    const uint8_t *kidx, *ksign, *knorm;  // K planes
    const uint8_t *vidx, *vnorm;          // V planes
    const int32_t *seq_lens;
    float *qr, *qp, *qsum, *scores, *stats, *part;
    uint32_t *cnt;
    float *out;
    float tau;
    int B, Hq, Hkv, T, chunk, n_chunks;
    int k_rotated;  // K codec works in the rotated domain
    int v_rotated;  // V codec works in the rotated domain
};

__device__ __forceinline__ int seq_len_of(const AttnArgs &a, int b) {
    if (!a.seq_lens) return a.T;
    int L = a.seq_lens[b];
    return L < 0 ? 0 : (L > a.T ? a.T : L);
}

// ---------------------------------------------------------------- prologue
__global__ __launch_bounds__(64) void attn_prologue_kernel(AttnArgs a, int want_proj) {
    __shared__ float s_q[128];
    const int head = blockIdx.x;  // b * Hq + h
    const int lane = threadIdx.x;
    const int g = a.Hq / a.Hkv;
    const uint16_t *q = a.q + int64_t(head) * 128;
    float v0 = h2f(q[lane]), v1 = h2f(q[lane + 64]);
    if (a.k_rotated) {
        v0 *= a.tab->signs[lane];
        v1 *= a.tab->signs[lane + 64];
        // H over coordinate bit 6 in-lane, bits 0..5 across lanes
        const float s0 = v0 + v1, s1 = v0 - v1;
        v0 = s0;
        v1 = s1;
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
            const float sg = (lane & s) ? -1.0f : 1.0f;
            const float p0 = __shfl_xor(v0, s), p1 = __shfl_xor(v1, s);
            v0 = fmaf(sg, v0, p0);
            v1 = fmaf(sg, v1, p1);
        }
        v0 *= kRsqrtD;  // q_rot = H D q / sqrt(d)
        v1 *= kRsqrtD;
    }
    // rotated keys: s = (1/sqrt d)(n/sqrt d) <q_rot, c> = n <q_rot/d, c>;
    // q8 keys: s = <q/sqrt(d), k> on the unrotated query
    const float f = a.k_rotated ? (1.0f / 128.0f) : kRsqrtD;
    a.qr[int64_t(head) * 128 + lane] = v0 * f;
    a.qr[int64_t(head) * 128 + lane + 64] = v1 * f;
    if (want_proj) {
        s_q[lane] = v0;
        s_q[lane + 64] = v1;
        __syncthreads();
        const uint16_t *S = a.tab->S;
        float p0 = 0.0f, p1 = 0.0f;
        for (int i = 0; i < 128; ++i) {
            const float qi = s_q[i];
            p0 = fmaf(h2f(S[lane * 128 + i]), qi, p0);
            p1 = fmaf(h2f(S[(lane + 64) * 128 + i]), qi, p1);
        }
        p0 *= kQjlOverSqrtD;
        p1 *= kQjlOverSqrtD;
        a.qp[int64_t(head) * 128 + lane] = p0;
        a.qp[int64_t(head) * 128 + lane + 64] = p1;
        float sum = p0 + p1;
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) sum += __shfl_xor(sum, s);
        if (lane == 0) a.qsum[head] = sum;
    }
    if (lane == 0 && (head % a.Hq) % g == 0) a.cnt[(head / a.Hq) * a.Hkv + (head % a.Hq) / g] = 0u;
}

// ------------------------------------------------------------------ scores
template <int G, int KIND, int BITS>
__global__ __launch_bounds__(256) void attn_scores_kernel(AttnArgs a, const float *__restrict__ qr_all,
                                                          const float *__restrict__ qp_all,
                                                          const uint8_t *__restrict__ kidx,
                                                          float *__restrict__ scores) {
    __shared__ float s_levels[16];
    __shared__ float s_red[4][G][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk_id = blockIdx.x, row = blockIdx.y;  // row = b*Hkv + kvh
    const int b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int hq0 = kvh * G;
    if constexpr (KIND != TQ_KIND_Q8) {
        if (tid < 16) s_levels[tid] = a.tab->levels[BITS - 1][tid];
    }
    __syncthreads();
    const int L = seq_len_of(a, b);
    const int t0 = chunk_id * a.chunk;
    const int t1 = min(t0 + a.chunk, L);
    const int64_t head0 = int64_t(b) * a.Hq + hq0;
    const float *qr_base = qr_all + head0 * 128;
    const float *qp_base = qp_all + head0 * 128;
    float qsum[G];
    if constexpr (KIND == TQ_KIND_PROD) {
#pragma unroll
        for (int g = 0; g < G; ++g) qsum[g] = a.qsum[head0 + g];
    }
    float m[G], l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) { m[g] = -INFINITY; l[g] = 0.0f; }

    for (int t = t0 + tid; t < t1; t += 256) {
        const int64_t vec = int64_t(row) * a.T + t;
        float sc[G];
        if constexpr (KIND == TQ_KIND_Q8) {
            const uint4 *src = reinterpret_cast<const uint4 *>(kidx + vec * 128);
            const uint2 sc2 = *reinterpret_cast<const uint2 *>(a.knorm + vec * 8);
            const float bs[4] = {h2f(sc2.x & 0xFFFFu), h2f(sc2.x >> 16), h2f(sc2.y & 0xFFFFu), h2f(sc2.y >> 16)};
#pragma unroll
            for (int g = 0; g < G; ++g) sc[g] = 0.0f;
            Unroll<16>::run([&](auto K) {  // 16 chunks of 8 int8 values
                constexpr int k = decltype(K)::value;
                const_fp qk = as_const(qr_base + k * 8);
                asm volatile("" : "+s"(qk));
                const uint4 u = src[k >> 1];
                const uint32_t w0 = (k & 1) ? u.z : u.x, w1 = (k & 1) ? u.w : u.y;
                float part[G];
#pragma unroll
                for (int g = 0; g < G; ++g) part[g] = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t ww = i < 4 ? w0 : w1;
                    const float kv = float(int8_t((ww >> (8 * (i & 3))) & 0xFFu));
#pragma unroll
                    for (int g = 0; g < G; ++g) part[g] = fmaf(qk[g * 128 + i], kv, part[g]);
                }
#pragma unroll
                for (int g = 0; g < G; ++g) sc[g] = fmaf(bs[k >> 2], part[g], sc[g]);
            });
        } else {
            uint32_t w[4 * BITS];
            const uint4 *src = reinterpret_cast<const uint4 *>(kidx + vec * (16 * BITS));
#pragma unroll
            for (int c = 0; c < BITS; ++c) {
                const uint4 u = src[c];
                w[4 * c] = u.x; w[4 * c + 1] = u.y; w[4 * c + 2] = u.z; w[4 * c + 3] = u.w;
            }
            float acc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = 0.0f;
            // the query values are read from the scalar cache in chunks of
            // kQc coordinates; the empty asm re-derives the pointer per chunk so
            // the compiler cannot hoist all 128*G loads into registers at once
            Unroll<128 / kQc>::run([&](auto K) {
                constexpr int k = decltype(K)::value;
                const_fp qk = as_const(qr_base + k * kQc);
                asm volatile("" : "+s"(qk));
                Unroll<kQc>::run([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    const float lv = s_levels[code_at<BITS, k * kQc + i>(w)];
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g] = fmaf(qk[g * 128 + i], lv, acc[g]);
                });
            });
            if constexpr (KIND == TQ_KIND_PROD) {
                const uint32_t nn = reinterpret_cast<const uint32_t *>(a.knorm)[vec];
                const float n = h2f(nn & 0xFFFFu), gam = h2f(nn >> 16);
                const uint4 su = *reinterpret_cast<const uint4 *>(a.ksign + vec * 16);
                const uint32_t sw[4] = {su.x, su.y, su.z, su.w};
                float aj[G];
#pragma unroll
                for (int g = 0; g < G; ++g) aj[g] = 0.0f;
                Unroll<128 / kQc>::run([&](auto K) {
                    constexpr int k = decltype(K)::value;
                    const_fp qk = as_const(qp_base + k * kQc);
                    asm volatile("" : "+s"(qk));
#pragma unroll
                    for (int i = 0; i < kQc; ++i) {
                        const int p = k * kQc + i;
                        const float bf = float((sw[p >> 5] >> (p & 31)) & 1u);
#pragma unroll
                        for (int g = 0; g < G; ++g) aj[g] = fmaf(qk[g * 128 + i], bf, aj[g]);
                    }
                });
#pragma unroll
                for (int g = 0; g < G; ++g) sc[g] = fmaf(n, acc[g], gam * fmaf(2.0f, aj[g], -qsum[g]));
            } else {
                const float n = h2f(reinterpret_cast<const uint16_t *>(a.knorm)[vec]);
#pragma unroll
                for (int g = 0; g < G; ++g) sc[g] = n * acc[g];
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            scores[(head0 + g) * a.T + t] = sc[g];
            if (sc[g] > m[g]) {
                l[g] = l[g] * exp2f((m[g] - sc[g]) * kLog2e) + 1.0f;
                m[g] = sc[g];
            } else {
                l[g] += exp2f((sc[g] - m[g]) * kLog2e);
            }
        }
    }
    // (max, sum) per head over the block
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
            const float om = __shfl_xor(m[g], s), ol = __shfl_xor(l[g], s);
            const float nm = fmaxf(m[g], om);
            float nl = 0.0f;
            if (nm != -INFINITY) nl = l[g] * exp2f((m[g] - nm) * kLog2e) + ol * exp2f((om - nm) * kLog2e);
            m[g] = nm;
            l[g] = nl;
        }
        if (lane == 0) { s_red[wave][g][0] = m[g]; s_red[wave][g][1] = l[g]; }
    }
    __syncthreads();
    if (tid < G) {
        float mm = -INFINITY;
        for (int w = 0; w < 4; ++w) mm = fmaxf(mm, s_red[w][tid][0]);
        float ll = 0.0f;
        if (mm != -INFINITY)
            for (int w = 0; w < 4; ++w) ll += s_red[w][tid][1] * exp2f((s_red[w][tid][0] - mm) * kLog2e);
        float *st = a.stats + ((head0 + tid) * a.n_chunks + chunk_id) * 2;
        st[0] = mm;
        st[1] = ll;
    }
}

// ------------------------------------------------------------------ values
template <int G, int KIND, int BITS>
__global__ __launch_bounds__(256) void attn_values_kernel(AttnArgs a) {
    __shared__ float s_levels[16];
    __shared__ float s_M[G], s_invL[G];
    __shared__ float s_w[G][256];
    __shared__ int s_tok[256];
    __shared__ int s_wcount[4];
    __shared__ float s_acc[4][G][128];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk_id = blockIdx.x, row = blockIdx.y;
    const int b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int hq0 = kvh * G;
    const int64_t head0 = int64_t(b) * a.Hq + hq0;
    if constexpr (KIND != TQ_KIND_Q8) {
        if (tid < 16) s_levels[tid] = a.tab->levels[BITS - 1][tid];
    }
    // exact softmax statistics from all chunks of this (batch, kv head)
    for (int g = wave; g < G; g += 4) {
        const float *st = a.stats + (head0 + g) * a.n_chunks * 2;
        float mm = -INFINITY;
        for (int c = lane; c < a.n_chunks; c += 64) mm = fmaxf(mm, st[2 * c]);
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) mm = fmaxf(mm, __shfl_xor(mm, s));
        float ll = 0.0f;
        if (mm != -INFINITY)
            for (int c = lane; c < a.n_chunks; c += 64) ll += st[2 * c + 1] * exp2f((st[2 * c] - mm) * kLog2e);
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) ll += __shfl_xor(ll, s);
        if (lane == 0) {
            s_M[g] = mm;
            s_invL[g] = ll > 0.0f ? 1.0f / ll : 0.0f;
        }
    }
    __syncthreads();
    const int L = seq_len_of(a, b);
    const int t0 = chunk_id * a.chunk;
    const int t1 = min(t0 + a.chunk, L);
    const int tk = lane >> 4, cg = lane & 15;  // token slot within the wave, coordinate group
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[g][j] = 0.0f;

    for (int base = t0; base < t1; base += 256) {
        // 1) weights and the keep decision, one token per thread
        const int t = base + tid;
        float wgt[G];
        bool keep = false;
        if (t < t1) {
            float vscale = 1.0f;
            if constexpr (KIND != TQ_KIND_Q8)
                vscale = h2f(reinterpret_cast<const uint16_t *>(a.vnorm)[int64_t(row) * a.T + t]) * kRsqrtD;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float s = a.scores[(head0 + g) * a.T + t];
                const float p = exp2f((s - s_M[g]) * kLog2e) * s_invL[g];
                const bool k = p >= a.tau;
                keep |= k;
                wgt[g] = k ? p * vscale : 0.0f;
            }
        }
        // 2) compact the kept tokens of this 256-token slice
        const uint64_t bal = __ballot(keep);
        if (lane == 0) s_wcount[wave] = __popcll(bal);
        __syncthreads();
        int off = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int c = s_wcount[w];
            off += (w < wave) ? c : 0;
            total += c;
        }
        if (keep) {
            const int slot = off + __popcll(bal & ((uint64_t(1) << lane) - 1));
            s_tok[slot] = t;
#pragma unroll
            for (int g = 0; g < G; ++g) s_w[g][slot] = wgt[g];
        }
        __syncthreads();
        // 3) accumulate kept rows: 16 tokens per pass (4 per wave), 8 coordinates per lane
        for (int k0 = 0; k0 < total; k0 += 16) {
            const int slot = k0 + wave * 4 + tk;
            if (slot < total) {
                const int64_t vec = int64_t(row) * a.T + s_tok[slot];
                float val[8];
                if constexpr (KIND == TQ_KIND_Q8) {
                    const uint2 u = *reinterpret_cast<const uint2 *>(a.vidx + vec * 128 + 8 * cg);
                    const float bsc = h2f(reinterpret_cast<const uint16_t *>(a.vnorm)[vec * 4 + (cg >> 2)]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        val[j] = float(int8_t((u.x >> (8 * j)) & 0xFFu)) * bsc;
                        val[4 + j] = float(int8_t((u.y >> (8 * j)) & 0xFFu)) * bsc;
                    }
                } else {
                    const uint8_t *rowp = a.vidx + vec * (16 * BITS);
                    uint32_t bitsw;
                    if constexpr (BITS == 4) {
                        bitsw = reinterpret_cast<const uint32_t *>(rowp)[cg];
                    } else if constexpr (BITS == 2) {
                        bitsw = reinterpret_cast<const uint16_t *>(rowp)[cg];
                    } else if constexpr (BITS == 1) {
                        bitsw = rowp[cg];
                    } else {  // 3 bits: 24 bits starting at byte 3*cg
                        const uint32_t *wp = reinterpret_cast<const uint32_t *>(rowp);
                        const int byte = 3 * cg;
                        const uint32_t lo = wp[byte >> 2], hi = wp[(byte + 2) >> 2];
                        const uint64_t both = (uint64_t(hi) << 32) | lo;
                        bitsw = uint32_t(both >> (8 * (byte & 3)));
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) val[j] = s_levels[(bitsw >> (BITS * j)) & ((1u << BITS) - 1u)];
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float wg = s_w[g][slot];
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[g][j] = fmaf(wg, val[j], acc[g][j]);
                }
            }
        }
        __syncthreads();
    }
    // reduce over the 4 token slots of each wave, then over the 4 waves
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[g][j] = quad_sum(acc[g][j]);
    if (tk == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < 8; ++j) s_acc[wave][g][8 * cg + j] = acc[g][j];
    }
    __syncthreads();
    for (int i = tid; i < G * 128; i += 256) {
        const int g = i >> 7, c = i & 127;
        const float s = s_acc[0][g][c] + s_acc[1][g][c] + s_acc[2][g][c] + s_acc[3][g][c];
        a.part[((head0 + g) * a.n_chunks + chunk_id) * 128 + c] = s;
    }
    // the last block of this (batch, kv head) merges the chunk partials
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(a.cnt + row, 1u);
        s_last = (prev == uint32_t(a.n_chunks - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int g = wave; g < G; g += 4) {
        float v0 = 0.0f, v1 = 0.0f;
        const volatile float *pp = a.part + (head0 + g) * a.n_chunks * 128;
        for (int c = 0; c < a.n_chunks; ++c) {
            v0 += pp[c * 128 + lane];
            v1 += pp[c * 128 + lane + 64];
        }
        if (a.v_rotated) {
            // out = R^T acc = D H acc / sqrt(d)
            const float s0 = v0 + v1, s1 = v0 - v1;
            v0 = s0;
            v1 = s1;
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const float sg = (lane & s) ? -1.0f : 1.0f;
                const float p0 = __shfl_xor(v0, s), p1 = __shfl_xor(v1, s);
                v0 = fmaf(sg, v0, p0);
                v1 = fmaf(sg, v1, p1);
            }
            v0 *= a.tab->signs[lane] * kRsqrtD;
            v1 *= a.tab->signs[lane + 64] * kRsqrtD;
        }
        a.out[(head0 + g) * 128 + lane] = v0;
        a.out[(head0 + g) * 128 + lane + 64] = v1;
    }
    if (tid == 0) a.cnt[row] = 0u;
}

template <int G, int KK, int KB, int VK, int VB>
static int launch_pair(const AttnArgs &a, hipStream_t s) {
    dim3 grid(unsigned(a.n_chunks), unsigned(a.B * a.Hkv));
    hipLaunchKernelGGL((attn_scores_kernel<G, KK, KB>), grid, dim3(256), 0, s, a, a.qr, a.qp, a.kidx,
                       a.scores);
    if (hipGetLastError() != hipSuccess) return 1;
    hipLaunchKernelGGL((attn_values_kernel<G, VK, VB>), grid, dim3(256), 0, s, a);
    return int(hipGetLastError());
}

template <int G, int KK, int KB>
static int dispatch_v(const AttnArgs &a, tq_format vf, hipStream_t s) {
    if (vf.kind == TQ_KIND_Q8) return launch_pair<G, KK, KB, TQ_KIND_Q8, 8>(a, s);
    switch (vf.bits) {
        case 1: return launch_pair<G, KK, KB, TQ_KIND_MSE, 1>(a, s);
        case 2: return launch_pair<G, KK, KB, TQ_KIND_MSE, 2>(a, s);
        case 3: return launch_pair<G, KK, KB, TQ_KIND_MSE, 3>(a, s);
        case 4: return launch_pair<G, KK, KB, TQ_KIND_MSE, 4>(a, s);
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
                int Hkv, int T, const int32_t *seq_lens, float tau, float *out, void *ws,
                const AttnPlan &plan, void *stream) {
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
    a.qr = reinterpret_cast<float *>(w + plan.off_qr);
    a.qp = reinterpret_cast<float *>(w + plan.off_qp);
    a.qsum = reinterpret_cast<float *>(w + plan.off_qsum);
    a.scores = reinterpret_cast<float *>(w + plan.off_scores);
    a.stats = reinterpret_cast<float *>(w + plan.off_stats);
    a.part = reinterpret_cast<float *>(w + plan.off_part);
    a.cnt = reinterpret_cast<uint32_t *>(w + plan.off_cnt);
    a.out = out;
    a.tau = tau;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.T = T;
    a.chunk = plan.chunk;
    a.n_chunks = plan.n_chunks;
    a.k_rotated = kf.kind != TQ_KIND_Q8;
    a.v_rotated = vf.kind != TQ_KIND_Q8;
    hipLaunchKernelGGL(attn_prologue_kernel, dim3(unsigned(B * Hq)), dim3(64), 0, s, a,
                       kf.kind == TQ_KIND_PROD ? 1 : 0);
    if (hipGetLastError() != hipSuccess) return 1;
    switch (Hq / Hkv) {
        case 1: return dispatch_k<1>(a, kf, vf, s);
        case 2: return dispatch_k<2>(a, kf, vf, s);
        case 4: return dispatch_k<4>(a, kf, vf, s);
        case 8: return dispatch_k<8>(a, kf, vf, s);
    }
    return int(hipErrorInvalidValue);
}

}  // namespace tq
