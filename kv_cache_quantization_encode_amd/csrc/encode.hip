// Per-token KV encode for gfx950: the bulk encode of a packed tensor, the
// in-place append of a decode step's new tokens, and the q8 boundary blocks.
//
// quidproquo.cc, "TurboQuant+ KV cache compression", Stage 1 and Stage 2: the
// per-tile arithmetic (encode_common.h).
// yeyulingfeng.com TurboQuant+ introduction, core item 3: boundary layers
// kept at q8_0 (symmetric absmax int8 per block of 32 here).
#include <type_traits>

#include "encode_common.h"

namespace tq {

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
    __shared__ EncodeTables s_tab;
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
    fill_encode_tables<BITS, PROD>(tab, &s_tab, tid, 256);
    if constexpr (PROD) {
        const half8 *src = reinterpret_cast<const half8 *>(tab->S_enc);
        for (int i = tid; i < 32 * 64; i += 256) s_frag[i] = src[i];
    }
    __syncthreads();
    EncodeLane el;
    encode_lane<BITS>(tab, lane, el);
    const EncodePlanes pl{idx_plane, sign_plane, norm_plane, rnorm_plane};

    for (int tile = int(blockIdx.x) * 4 + wave; tile < ntl; tile += stride) {
        const int tok = tile * 16 + t;
        bool valid = tok < nv;
        const int dst = dest_row<APPEND>(map, tok, valid);
        load_rows(min(tile + stride, ntl - 1), xn);
        encode_tile<BITS, PROD, B32>(
            xb, el, s_tab.levels, s_tab.lut, [&](int i) { return s_frag[i]; }, lane, valid, dst, pl, [&] {
                // the prefetched rows become the next tile's operands before
                // any store of this tile: waiting for them after a (possibly
                // skipped) store would wait for the stores as well
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    xb[s] = xn[s];
                    asm volatile("" : "+v"(xb[s]));
                }
            });
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
