// Reconstruction of fp16 rows from packed tensors (gfx950).
//
// quidproquo.cc, "TurboQuant+ KV cache compression": Stage 1 reconstruction
// n R^T c[idx] / sqrt(d); for K the QJL estimate of the residual is added,
// sqrt(pi/2)/m * gamma * R^T S^T (2 bit - 1) (the estimator that makes
// <q, k_hat> unbiased for Gaussian S).  q8 blocks: int8 * fp16 block scale.
//
// Lane layout as in the encoder: 16 tokens per wavefront, lane l owns token
// l&15 and, in the rotated domain, coordinates 32*(l>>4)+[0,32); the inverse
// transform leaves it holding 8*(l>>4) + [0,8) + 32k of the output row.  The QJL term S^T (2b - 1) for the
// 16 tokens of a wave is one [128 x 128] x [128 x 16] fp16 MFMA product
// (entries of S and +-1 are exact in fp16; fp32 accumulation).
// Block-32 norm storage: lane group q holds rotated block q, whose scale is
// its own norm, n_q / sqrt(32).
#include <type_traits>

#include "device_common.h"

namespace tq {

constexpr float kRsqrtD = 0.08838834764831845f;        // 1/sqrt(128)
constexpr float kQjlScale = 1.2533141373155003f / 128;  // sqrt(pi/2)/m

template <int BITS, bool PROD, bool B32>
__global__ __launch_bounds__(256) void decode_tq_kernel(const DevTables *__restrict__ tab,
                                                        const uint8_t *__restrict__ idx_plane,
                                                        const uint8_t *__restrict__ sign_plane,
                                                        const uint8_t *__restrict__ norm_plane,
                                                        int64_t n_vec, uint16_t *__restrict__ out,
                                                        int64_t n_tiles) {
    __shared__ float s_levels[16];
    __shared__ half8 s_frag[PROD ? 32 * 64 : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < 16) s_levels[tid] = tab->levels[BITS - 1][tid];
    if constexpr (PROD) {
        const half8 *src = reinterpret_cast<const half8 *>(tab->St_dec);
        for (int i = tid; i < 32 * 64; i += 256) s_frag[i] = src[i];
    }
    __syncthreads();
    const int t = lane & 15, q = lane >> 4;
    // D/sqrt(d) for the coordinates this lane holds after the transform
    // (layout A: register r holds coordinate 8q + (r&7) + 32(r>>3))
    float dsg[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) dsg[r] = tab->signs[layoutA_coord(q, r)] * kRsqrtD;

    for (int64_t tile = int64_t(blockIdx.x) * 4 + wave; tile < n_tiles; tile += int64_t(gridDim.x) * 4) {
        const int64_t tok = tile * 16 + t;
        const bool valid = tok < n_vec;
        uint32_t w[BITS];
        float nrm = 0.0f, gam = 0.0f;
        uint32_t sbits = 0;
        if (valid) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(idx_plane + tok * (16 * BITS) + q * (4 * BITS));
#pragma unroll
            for (int i = 0; i < BITS; ++i) w[i] = src[i];
            if constexpr (B32) {
                // block norm q; K: the residual norms follow all block norms
                nrm = h2f(reinterpret_cast<const uint16_t *>(norm_plane)[tok * 4 + q]);
                if constexpr (PROD) {
                    gam = h2f(reinterpret_cast<const uint16_t *>(norm_plane + n_vec * 8)[tok]);
                    sbits = reinterpret_cast<const uint32_t *>(sign_plane + tok * 16)[q];
                }
            } else if constexpr (PROD) {
                const uint32_t nn = reinterpret_cast<const uint32_t *>(norm_plane)[tok];
                nrm = h2f(nn & 0xFFFFu);
                gam = h2f(nn >> 16);
                sbits = reinterpret_cast<const uint32_t *>(sign_plane + tok * 16)[q];
            } else {
                nrm = h2f(reinterpret_cast<const uint16_t *>(norm_plane)[tok]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < BITS; ++i) w[i] = 0;
        }
        float v[32];
        const float sc = nrm * (B32 ? 0.17677669529663687f : kRsqrtD);  // 1/sqrt(32) or 1/sqrt(d)
        Unroll<32>::run([&](auto I) {
            constexpr int j = decltype(I)::value;
            v[j] = sc * s_levels[code_at<BITS, j>(w)];
        });
        if constexpr (PROD) {
            // B operand: +-1 for projections 32q + 8s + j of this lane's token
            half8 b[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    b[s][j] = ((sbits >> (8 * s + j)) & 1u) ? _Float16(1.0f) : _Float16(-1.0f);
            const float gs = gam * kQjlScale;
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(s_frag[(cb * 4 + s) * 64 + lane], b[s], acc, 0, 0, 0);
                // lane (t, q) holds coordinates 32q + 4cb + j of token t
#pragma unroll
                for (int j = 0; j < 4; ++j) v[4 * cb + j] = fmaf(gs, acc[j], v[4 * cb + j]);
            }
        }
        // x_hat = R^T v = D H v / sqrt(d); the transform leaves layout A
        fwht128_swap(v);
        if (valid) {
            uint32_t o[16];
#pragma unroll
            for (int p = 0; p < 16; ++p) o[p] = f2h(v[2 * p] * dsg[2 * p]) | (f2h(v[2 * p + 1] * dsg[2 * p + 1]) << 16);
            uint16_t *row = out + tok * kHeadDim + 8 * q;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<uint4 *>(row + 32 * k) = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
        }
    }
}

__global__ __launch_bounds__(256) void decode_q8_kernel(const int8_t *__restrict__ qplane,
                                                        const uint16_t *__restrict__ scale_plane,
                                                        int64_t n_vec, uint16_t *__restrict__ out) {
    const int64_t gl = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t tok = gl >> 2;
    const int blk = int(gl & 3);
    if (tok >= n_vec) return;
    const float scale = h2f(scale_plane[tok * 4 + blk]);
    const uint4 *src = reinterpret_cast<const uint4 *>(qplane + tok * kHeadDim + 32 * blk);
    uint32_t o[16];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint4 u = src[c];
        const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t x = ww[p];
            const float a = float(int8_t(x & 0xFF)) * scale, b = float(int8_t((x >> 8) & 0xFF)) * scale;
            const float cc = float(int8_t((x >> 16) & 0xFF)) * scale, d = float(int8_t(x >> 24)) * scale;
            o[8 * c + 2 * p] = f2h(a) | (f2h(b) << 16);
            o[8 * c + 2 * p + 1] = f2h(cc) | (f2h(d) << 16);
        }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(out + tok * kHeadDim + 32 * blk);
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
}

template <int BITS, bool PROD, bool B32 = false>
static int launch_dec(const DevTables *tab, const uint8_t *base, int64_t n_vec, const tq_planes_desc &lay,
                      uint16_t *out, hipStream_t s) {
    const int64_t n_tiles = (n_vec + 15) / 16;
    int64_t blocks = (n_tiles + 3) / 4;
    if (PROD && blocks > 1024) blocks = 1024;
    if (blocks > (int64_t(1) << 30)) blocks = int64_t(1) << 30;
    hipLaunchKernelGGL((decode_tq_kernel<BITS, PROD, B32>), dim3(unsigned(blocks)), dim3(256), 0, s, tab,
                       base + lay.idx_offset, PROD ? base + lay.sign_offset : nullptr,
                       base + lay.norm_offset, n_vec, out, n_tiles);
    return int(hipGetLastError());
}

int launch_decode(const DevTables *tab, const void *packed, tq_format f, int64_t n_vec,
                  const tq_planes_desc &lay, void *outv, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *base = static_cast<const uint8_t *>(packed);
    uint16_t *out = static_cast<uint16_t *>(outv);
    if (f.kind == TQ_KIND_Q8) {
        const int64_t blocks = (n_vec * 4 + 255) / 256;
        hipLaunchKernelGGL(decode_q8_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                           reinterpret_cast<const int8_t *>(base + lay.idx_offset),
                           reinterpret_cast<const uint16_t *>(base + lay.norm_offset), n_vec, out);
        return int(hipGetLastError());
    }
    if (f.kind == TQ_KIND_PROD32) {
        switch (f.bits) {
            case 1: return launch_dec<1, true, true>(tab, base, n_vec, lay, out, s);
            case 2: return launch_dec<2, true, true>(tab, base, n_vec, lay, out, s);
            case 3: return launch_dec<3, true, true>(tab, base, n_vec, lay, out, s);
        }
        return int(hipErrorInvalidValue);
    }
    if (f.kind == TQ_KIND_MSE32) {
        switch (f.bits) {
            case 1: return launch_dec<1, false, true>(tab, base, n_vec, lay, out, s);
            case 2: return launch_dec<2, false, true>(tab, base, n_vec, lay, out, s);
            case 3: return launch_dec<3, false, true>(tab, base, n_vec, lay, out, s);
            case 4: return launch_dec<4, false, true>(tab, base, n_vec, lay, out, s);
        }
        return int(hipErrorInvalidValue);
    }
    if (f.kind == TQ_KIND_PROD) {
        switch (f.bits) {
            case 1: return launch_dec<1, true>(tab, base, n_vec, lay, out, s);
            case 2: return launch_dec<2, true>(tab, base, n_vec, lay, out, s);
            case 3: return launch_dec<3, true>(tab, base, n_vec, lay, out, s);
        }
    } else {
        switch (f.bits) {
            case 1: return launch_dec<1, false>(tab, base, n_vec, lay, out, s);
            case 2: return launch_dec<2, false>(tab, base, n_vec, lay, out, s);
            case 3: return launch_dec<3, false>(tab, base, n_vec, lay, out, s);
            case 4: return launch_dec<4, false>(tab, base, n_vec, lay, out, s);
        }
    }
    return int(hipErrorInvalidValue);
}

}  // namespace tq
