// Decode attention over caches with block-32 norm storage (gfx950).
//
// yeyulingfeng.com, "TurboQuant+: 3.8x compression ...", technical
// highlights: block-32 storage, here one fp16 Stage-1 norm per block of 32
// rotated coordinates.  The attention it serves is the same as the other
// kernels' (chenxutan.com, "TurboQuant+ deep dive", 1.1 cached decode
// attention; quidproquo.cc, "TurboQuant+ KV cache compression", Stage 2: the
// QJL term of the K score; yeyulingfeng.com core item 4 and chenxutan.com
// 3.3: V rows below the weight threshold are skipped, kept weights are not
// renormalised).  With four scales per vector the per-token factor no longer
// comes out of the coordinate sum, so these two kernels read the packed
// planes directly, coordinate by coordinate, in plain fp32 arithmetic; any K
// format may meet any V format here.
//
//   scores: block (chunk, row), one thread per token: q_rot = H D q / sqrt(d)
//           and q_proj = S q_rot in LDS, each key coordinate decoded once and
//           applied to every head; scores to the workspace, the chunk's
//           (max, sum) per head to the statistics.  Chunk 0 zeroes the
//           output rows.
//   values: block (chunk, row), 32 threads per head, 4 rotated coordinates
//           per thread: the exact (M, L) from every chunk, the kept tokens'
//           weighted V values, one inverse rotation per head, fp32 atomics
//           into the output.
#include "attn_common.h"

namespace tq {

constexpr int kGenThreads = 256;
constexpr float kRsqrt32 = 0.17677669529663687f;      // 1/sqrt(32)
constexpr float kQjlM = 1.2533141373155003f / 128.0f;  // sqrt(pi/2)/m

__device__ __forceinline__ bool rotated_kind(int kind) { return kind != TQ_KIND_Q8; }
__device__ __forceinline__ bool block32_kind(int kind) { return kind == TQ_KIND_MSE32 || kind == TQ_KIND_PROD32; }

// Codes i .. i + 3 (i a multiple of 4) of width B from one packed row.
template <int B>
__device__ __forceinline__ uint32_t codes4(const uint8_t *row, int i) {
    const int bit = i * B;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(row) + (bit >> 5);
    const int sh = bit & 31;
    uint64_t v = w[0];
    if (sh + 4 * B > 32) v |= uint64_t(w[1]) << 32;
    return uint32_t(v >> sh) & ((1u << (4 * B)) - 1u);
}

// Scale of rotated block q4 (coordinates 32 q4 + [0, 32)) of vector v:
// n / sqrt(d) (one norm per vector) or n_q4 / sqrt(32) (block-32).
template <int KIND>
__device__ __forceinline__ float stage1_scale(const uint8_t *norm_plane, int64_t v, int q4) {
    if constexpr (KIND == TQ_KIND_PROD) return h2f(reinterpret_cast<const uint16_t *>(norm_plane)[2 * v]) * kRsqrtD;
    if constexpr (KIND == TQ_KIND_MSE) return h2f(reinterpret_cast<const uint16_t *>(norm_plane)[v]) * kRsqrtD;
    return h2f(reinterpret_cast<const uint16_t *>(norm_plane)[4 * v + q4]) * kRsqrt32;
}

// Residual norm of a K vector: the high half of its norm pair (PROD), or the
// block-32 residual norms that follow the n_vec x 4 block norms (PROD32).
template <int KIND>
__device__ __forceinline__ float residual_norm(const uint8_t *norm_plane, int64_t v, int64_t n_vec) {
    if constexpr (KIND == TQ_KIND_PROD) return h2f(reinterpret_cast<const uint16_t *>(norm_plane)[2 * v + 1]);
    return h2f(reinterpret_cast<const uint16_t *>(norm_plane + n_vec * 8)[v]);
}

template <int KK, int KB>
__global__ __launch_bounds__(kGenThreads) void attn_generic_scores_kernel(AttnArgs a) {
    constexpr bool PROJ = KK == TQ_KIND_PROD || KK == TQ_KIND_PROD32;
    __shared__ float s_q[8][128];
    __shared__ float s_p[PROJ ? 8 : 1][128];
    __shared__ float s_lv[16];
    __shared__ float s_red[8][kGenThreads / 64][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.Hq / a.Hkv;
    const int row = blockIdx.y, b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int c = blockIdx.x;
    const int L = seq_len_of(a, b);
    const int t0 = c * a.chunk, t1 = min(t0 + a.chunk, L);
    const int64_t head0 = int64_t(b) * a.Hq + int64_t(kvh) * G;
    const int64_t n_vec = int64_t(a.B) * a.Hkv * a.T;

    if (c == 0)
        for (int i = tid; i < G * 128; i += kGenThreads) a.out[head0 * 128 + i] = 0.0f;
    if constexpr (KK != TQ_KIND_Q8) {
        if (tid < (1 << KB)) s_lv[tid] = a.tab->levels[KB - 1][tid];
    }
    // q_rot = H D q / sqrt(d) of each head (q itself for q8 keys)
    for (int i = tid; i < G * 128; i += kGenThreads) {
        const int h = i >> 7, x = i & 127;
        float v = h2f(a.q[(head0 + h) * 128 + x]);
        if (rotated_kind(KK)) v *= a.tab->signs[x];
        s_q[h][x] = v;
    }
    __syncthreads();
    if (rotated_kind(KK)) {
        for (int len = 1; len < 128; len <<= 1) {
            for (int i = tid; i < G * 64; i += kGenThreads) {
                const int h = i >> 6, j = i & 63;
                const int x0 = (j / len) * 2 * len + (j % len), x1 = x0 + len;
                const float u = s_q[h][x0], w = s_q[h][x1];
                s_q[h][x0] = u + w;
                s_q[h][x1] = u - w;
            }
            __syncthreads();
        }
        for (int i = tid; i < G * 128; i += kGenThreads) s_q[i >> 7][i & 127] *= kRsqrtD;
        __syncthreads();
    }
    // q_proj = S q_rot
    if constexpr (PROJ) {
        for (int i = tid; i < G * 128; i += kGenThreads) {
            const int h = i >> 7, p = i & 127;
            const uint16_t *srow = a.tab->S + p * 128;
            float acc = 0.0f;
            for (int x = 0; x < 128; ++x) acc = fmaf(h2f(srow[x]), s_q[h][x], acc);
            s_p[h][p] = acc;
        }
        __syncthreads();
    }

    // scores of the chunk, one thread per token; running (max, sum) per head
    float m[8], l[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
    }
    for (int t = t0 + tid; t < t1; t += kGenThreads) {
        const int64_t v = int64_t(row) * a.T + t;
        float dot[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (KK == TQ_KIND_Q8) {
            const int8_t *qrow = reinterpret_cast<const int8_t *>(a.kidx) + v * 128;
            for (int q4 = 0; q4 < 4; ++q4) {
                const float sc = h2f(reinterpret_cast<const uint16_t *>(a.knorm)[4 * v + q4]);
                for (int j = 0; j < 32; ++j) {
                    const float val = sc * float(qrow[32 * q4 + j]);
#pragma unroll
                    for (int h = 0; h < 8; ++h)
                        if (h < G) dot[h] = fmaf(s_q[h][32 * q4 + j], val, dot[h]);
                }
            }
        } else {
            const uint8_t *crow = a.kidx + v * (16 * KB);
            for (int q4 = 0; q4 < 4; ++q4) {
                const float sc = stage1_scale<KK == TQ_KIND_PROD32 ? TQ_KIND_MSE32 : KK>(a.knorm, v, q4);
                for (int j4 = 0; j4 < 32; j4 += 4) {
                    const uint32_t cw = codes4<KB>(crow, 32 * q4 + j4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float val = sc * s_lv[(cw >> (KB * e)) & ((1u << KB) - 1u)];
#pragma unroll
                        for (int h = 0; h < 8; ++h)
                            if (h < G) dot[h] = fmaf(s_q[h][32 * q4 + j4 + e], val, dot[h]);
                    }
                }
            }
            if constexpr (PROJ) {
                // sqrt(pi/2)/m gamma sum_p q_proj,p (2 bit_p - 1)
                const float gq = kQjlM * residual_norm<KK>(a.knorm, v, n_vec);
                const uint32_t *sg = reinterpret_cast<const uint32_t *>(a.ksign + v * 16);
                for (int w4 = 0; w4 < 4; ++w4) {
                    const uint32_t bits = sg[w4];
                    for (int j = 0; j < 32; ++j) {
                        const float sv = ((bits >> j) & 1u) ? gq : -gq;
#pragma unroll
                        for (int h = 0; h < 8; ++h)
                            if (h < G) dot[h] = fmaf(s_p[h][32 * w4 + j], sv, dot[h]);
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            if (h < G) {
                const float s = dot[h] * kRsqrtD;
                a.scores[(head0 + h) * int64_t(a.ld_scores) + t] = s;
                const float nm = fmaxf(m[h], s);
                l[h] = l[h] * __expf(m[h] - nm) + __expf(s - nm);
                m[h] = nm;
            }
        }
    }
    // (max, sum) of the chunk per head: lanes, then waves
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        if (h >= G) break;
        float mm = m[h];
        for (int o = 32; o > 0; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
        float ll = m[h] == -INFINITY ? 0.0f : l[h] * __expf(m[h] - mm);
        for (int o = 32; o > 0; o >>= 1) ll += __shfl_xor(ll, o);
        if (lane == 0) {
            s_red[h][wave][0] = mm;
            s_red[h][wave][1] = ll;
        }
    }
    __syncthreads();
    if (tid < G) {
        float mm = -INFINITY, ll = 0.0f;
        for (int w = 0; w < kGenThreads / 64; ++w) mm = fmaxf(mm, s_red[tid][w][0]);
        if (mm != -INFINITY)
            for (int w = 0; w < kGenThreads / 64; ++w)
                ll += s_red[tid][w][0] == -INFINITY ? 0.0f : s_red[tid][w][1] * __expf(s_red[tid][w][0] - mm);
        float *st = a.stats + ((head0 + tid) * a.n_chunks + c) * 2;
        st[0] = mm;
        st[1] = ll;
    }
}

template <int VK, int VB>
__global__ __launch_bounds__(kGenThreads) void attn_generic_values_kernel(AttnArgs a) {
    __shared__ float s_o[8][128];
    __shared__ float s_lv[16];
    const int tid = threadIdx.x;
    const int G = a.Hq / a.Hkv;
    const int row = blockIdx.y, b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int c = blockIdx.x;
    const int L = seq_len_of(a, b);
    const int t0 = c * a.chunk, t1 = min(t0 + a.chunk, L);
    const int64_t head0 = int64_t(b) * a.Hq + int64_t(kvh) * G;
    if constexpr (VK != TQ_KIND_Q8) {
        if (tid < (1 << VB)) s_lv[tid] = a.tab->levels[VB - 1][tid];
    }
    for (int i = tid; i < 8 * 128; i += kGenThreads) s_o[i >> 7][i & 127] = 0.0f;
    __syncthreads();
    const int h = tid >> 5, x4 = 4 * (tid & 31), q4 = x4 >> 5;
    if (h < G) {
        // exact softmax statistics of head h from every chunk
        const float *st = a.stats + (head0 + h) * a.n_chunks * 2;
        float M = -INFINITY;
        for (int k = 0; k < a.n_chunks; ++k) M = fmaxf(M, st[2 * k]);
        float Ls = 0.0f;
        if (M != -INFINITY)
            for (int k = 0; k < a.n_chunks; ++k)
                Ls += st[2 * k] == -INFINITY ? 0.0f : st[2 * k + 1] * __expf(st[2 * k] - M);
        const float invL = Ls > 0.0f ? 1.0f / Ls : 0.0f;
        const float *srow = a.scores + (head0 + h) * int64_t(a.ld_scores);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int t = t0; t < t1; ++t) {
            const float p = __expf(srow[t] - M) * invL;
            if (!(p >= a.tau)) continue;  // skipped weights are not renormalised
            const int64_t v = int64_t(row) * a.T + t;
            if constexpr (VK == TQ_KIND_Q8) {
                const float sc = h2f(reinterpret_cast<const uint16_t *>(a.vnorm)[4 * v + q4]);
                const uint32_t w = *reinterpret_cast<const uint32_t *>(a.vidx + v * 128 + x4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(p, sc * float(int8_t((w >> (8 * e)) & 0xFFu)), acc[e]);
            } else {
                const float sc = stage1_scale<VK>(a.vnorm, v, q4);
                const uint32_t cw = codes4<VB>(a.vidx + v * (16 * VB), x4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[e] = fmaf(p, sc * s_lv[(cw >> (VB * e)) & ((1u << VB) - 1u)], acc[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) s_o[h][x4 + e] = acc[e];
    }
    __syncthreads();
    // rotated-domain V back to x: R^T y = D H y / sqrt(d)
    if constexpr (VK != TQ_KIND_Q8) {
        for (int len = 1; len < 128; len <<= 1) {
            for (int i = tid; i < G * 64; i += kGenThreads) {
                const int hh = i >> 6, j = i & 63;
                const int y0 = (j / len) * 2 * len + (j % len), y1 = y0 + len;
                const float u = s_o[hh][y0], w = s_o[hh][y1];
                s_o[hh][y0] = u + w;
                s_o[hh][y1] = u - w;
            }
            __syncthreads();
        }
    }
    if (t0 < t1) {
        for (int i = tid; i < G * 128; i += kGenThreads) {
            const int hh = i >> 7, x = i & 127;
            const float y = VK == TQ_KIND_Q8 ? s_o[hh][x] : s_o[hh][x] * a.tab->signs[x] * kRsqrtD;
            atomicAdd(a.out + (head0 + hh) * 128 + x, y);
        }
    }
}

template <int KK, int KB>
static int launch_generic_k(const AttnArgs &a, tq_format vf, hipStream_t s) {
    const dim3 grid(unsigned(a.n_chunks), unsigned(a.B * a.Hkv));
    hipLaunchKernelGGL((attn_generic_scores_kernel<KK, KB>), grid, dim3(kGenThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return int(hipErrorLaunchFailure);
    switch (vf.kind) {
        case TQ_KIND_Q8:
            hipLaunchKernelGGL((attn_generic_values_kernel<TQ_KIND_Q8, 8>), grid, dim3(kGenThreads), 0, s, a);
            break;
        case TQ_KIND_MSE:
        case TQ_KIND_MSE32: {
            const bool b32 = vf.kind == TQ_KIND_MSE32;
            switch (vf.bits) {
                case 1: hipLaunchKernelGGL((b32 ? attn_generic_values_kernel<TQ_KIND_MSE32, 1> : attn_generic_values_kernel<TQ_KIND_MSE, 1>), grid, dim3(kGenThreads), 0, s, a); break;
                case 2: hipLaunchKernelGGL((b32 ? attn_generic_values_kernel<TQ_KIND_MSE32, 2> : attn_generic_values_kernel<TQ_KIND_MSE, 2>), grid, dim3(kGenThreads), 0, s, a); break;
                case 3: hipLaunchKernelGGL((b32 ? attn_generic_values_kernel<TQ_KIND_MSE32, 3> : attn_generic_values_kernel<TQ_KIND_MSE, 3>), grid, dim3(kGenThreads), 0, s, a); break;
                case 4: hipLaunchKernelGGL((b32 ? attn_generic_values_kernel<TQ_KIND_MSE32, 4> : attn_generic_values_kernel<TQ_KIND_MSE, 4>), grid, dim3(kGenThreads), 0, s, a); break;
                default: return int(hipErrorInvalidValue);
            }
            break;
        }
        default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}

int launch_attn_generic(const AttnArgs &a, tq_format kf, tq_format vf, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kf.kind) {
        case TQ_KIND_Q8: return launch_generic_k<TQ_KIND_Q8, 8>(a, vf, s);
        case TQ_KIND_PROD:
            switch (kf.bits) {
                case 1: return launch_generic_k<TQ_KIND_PROD, 1>(a, vf, s);
                case 2: return launch_generic_k<TQ_KIND_PROD, 2>(a, vf, s);
                case 3: return launch_generic_k<TQ_KIND_PROD, 3>(a, vf, s);
            }
            break;
        case TQ_KIND_PROD32:
            switch (kf.bits) {
                case 1: return launch_generic_k<TQ_KIND_PROD32, 1>(a, vf, s);
                case 2: return launch_generic_k<TQ_KIND_PROD32, 2>(a, vf, s);
                case 3: return launch_generic_k<TQ_KIND_PROD32, 3>(a, vf, s);
            }
            break;
        case TQ_KIND_MSE:
        case TQ_KIND_MSE32: {
            const bool b32 = kf.kind == TQ_KIND_MSE32;
            switch (kf.bits) {
                case 1: return b32 ? launch_generic_k<TQ_KIND_MSE32, 1>(a, vf, s) : launch_generic_k<TQ_KIND_MSE, 1>(a, vf, s);
                case 2: return b32 ? launch_generic_k<TQ_KIND_MSE32, 2>(a, vf, s) : launch_generic_k<TQ_KIND_MSE, 2>(a, vf, s);
                case 3: return b32 ? launch_generic_k<TQ_KIND_MSE32, 3>(a, vf, s) : launch_generic_k<TQ_KIND_MSE, 3>(a, vf, s);
                case 4: return b32 ? launch_generic_k<TQ_KIND_MSE32, 4>(a, vf, s) : launch_generic_k<TQ_KIND_MSE, 4>(a, vf, s);
            }
            break;
        }
    }
    return int(hipErrorInvalidValue);
}

}  // namespace tq
