// Single-launch decode attention for 4 query heads per kv head (gfx950).
//
// The same computation as the two passes of attn.hip (chenxutan.com,
// "TurboQuant+ deep dive", 1.1 cached decode attention; quidproquo.cc,
// "TurboQuant+ KV cache compression", Stage 2: the QJL term of the K score;
// yeyulingfeng.com TurboQuant+ introduction, core item 4, and chenxutan.com
// 3.3: V rows below the weight threshold are skipped, kept weights are not
// renormalised), in one kernel, for the few long rows of a single-sequence
// decode step (the 8-head analogue is attn_fused.hip):
//   phase 1  each block scores its token range [t0, t1) of one (sequence,
//            kv head) row with the scan of the two-pass scores kernel (query
//            rows on the matrix cores, 16-token tiles, 8 waves) and keeps the
//            scores in LDS; its (max, sum exp) per head go to the workspace.
//   barrier  the nblk blocks of a row wait for each other (one 64-bit slot
//            per block and head, bounded spin), as in attn_fused.hip: exact
//            sparse V needs the row's global statistics before any V row is
//            skipped.  Every block of the grid is resident at once.
//   phase 2  the exact (M, L); the compacting V pass of attn.hip over the
//            block's range (values_compact), reading the scores from LDS;
//            each block's share is rotated back and added into the output
//            with fp32 atomics (block 0 zeroes the output before the barrier).
// Compared with the two passes: no fp32 score round trip through HBM, no
// second launch and no second query setup.
#include "attn_common.h"

namespace tq {

constexpr int kQThreads = 512;  // 8 waves
constexpr int kQWaves = kQThreads / 64;
static_assert(kQThreads == kVThreads, "the values pass runs on the same block");
constexpr int kQSlice = 16 * kQWaves * kSliceTiles;  // tokens per slice (512)
static_assert(kQSlice == kFusedSlice, "slice size shared with the host plan");
constexpr int kQSuper = 1024;                       // tokens compacted at a time
constexpr uint64_t kQSpinTicks = 25000000;          // barrier spin budget: 0.25 s of the 100 MHz clock

template <int KK, int KB, int VK, int VB>
__global__ __launch_bounds__(kQThreads) void attn_fused4_kernel(AttnArgs a, const uint8_t *__restrict__ kidx,
                                                                const uint8_t *__restrict__ ksign,
                                                                const uint8_t *__restrict__ knorm) {
    constexpr int G = 4;
    constexpr bool PROJ = KK == TQ_KIND_PROD;
    static_assert(PROJ, "TurboQuant K");
    constexpr int kPairs = 1 << (2 * KB);
    // per-head score row stride: the most tokens of a block plus 16, so that
    // the heads' rows start 16 banks apart (the scan stores one token of
    // every head per lane group at once)
    constexpr int LD = kFusedMaxTokens + 16;
    constexpr int R = kQSuper / kVThreads;
    using VL = ValuesLds<G, VK, VB, kQSuper>;
    struct Lds {
        float sc[G * LD];  // head h, token t0 + i at sc[h * LD + i]
        float red[kQWaves][G][2];
        float M[G], invL[G];
        int okw[G], ok, last;
        union {
            struct {
                uint2 pair[kPairs];
                half8 sgn[256];
                __attribute__((aligned(16))) _Float16 a[16][128];
                __attribute__((aligned(16))) _Float16 ap[16][128];
            } s;
            VL v;  // after the scan
        } u;
    };
    __shared__ Lds lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = lane & 15, kq = lane >> 4;
    const int blk = blockIdx.x, row = blockIdx.y;  // row = b * Hkv + kvh
    const int b = row / a.Hkv, kvh = row - b * a.Hkv;
    const int L = seq_len_of(a, b);
    const int t0 = blk * a.tb;
    const int t1 = min(t0 + a.tb, L);
    const int n_tok = max(t1 - t0, 0);
    const int tmax = max(t1 - 1, 0);
    const int krow = kv_row(a, row);
    const uint8_t *kid = kidx + int64_t(krow) * a.T * (16 * KB);
    const uint8_t *ksg = ksign + int64_t(krow) * a.T * 16;
    const uint8_t *knm = knorm + int64_t(krow) * a.T * 4;

    // ---- global reads first: query, tables, the first K slices
    QueryLoads<G, PROJ, kQWaves> ql;
    load_query(ql, a, b, kvh);
    float lv[2] = {0.0f, 0.0f};
    if (tid < kPairs) {
        lv[0] = a.tab->levels[KB - 1][tid & ((1 << KB) - 1)];
        lv[1] = a.tab->levels[KB - 1][tid >> KB];
    }
    asm volatile("" ::: "memory");
    const bool whole = n_tok % kQSlice == 0;
    KTiles<PROJ ? TQ_KIND_PROD : TQ_KIND_MSE, KB> ta, tb, tc;
    load_ktiles<kQWaves>(ta, t0, tmax, wave, t, kq, kid, ksg, knm);
    if (t0 + kQSlice < t1) load_ktiles<kQWaves>(tb, t0 + kQSlice, tmax, wave, t, kq, kid, ksg, knm);
    // the V scale words of the block's first super-slice, needed right after
    // the barrier, travel with the first loads
    const int vrow = krow;
    const uint16_t *vn_base = reinterpret_cast<const uint16_t *>(a.vnorm) + int64_t(vrow) * a.T;
    uint32_t vraw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) vraw[r] = vn_base[min(t0 + kVThreads * r + tid, tmax)];

    // the row's output is summed with atomics: block 0 zeroes it before the
    // barrier
    if (blk == 0) {
        for (int i = tid; i < G * 128; i += kQThreads)
            __hip_atomic_store(a.out + io_row(a, b, kvh, i >> 7) * 128 + (i & 127), 0.0f, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    auto &ls = lds.u.s;
    for (int i = tid; i < (16 - 2 * G) * 32; i += kQThreads) {
        reinterpret_cast<uint2 *>(&ls.a[2 * G][0])[i] = uint2{0u, 0u};
        reinterpret_cast<uint2 *>(&ls.ap[2 * G][0])[i] = uint2{0u, 0u};
    }
    if (tid < 256) {
        half8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ((tid >> j) & 1) ? _Float16(1.0f) : _Float16(-1.0f);
        ls.sgn[tid] = v;
    }
    if (tid < kPairs) {
        uint32_t hp = 0, lp = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const _Float16 hi = _Float16(lv[u]);
            const _Float16 lo = _Float16(lv[u] - float(hi));
            hp |= uint32_t(__builtin_bit_cast(uint16_t, hi)) << (16 * u);
            lp |= uint32_t(__builtin_bit_cast(uint16_t, lo)) << (16 * u);
        }
        ls.pair[tid] = uint2{hp, lp};
    }
    build_query_rows<G>(ql, a, ls.a, ls.ap);  // ends with a barrier

    // A operands, as in the scores pass of attn.hip
    half8 aq[8], ap[4];
    {
        const _Float16 *ra = ls.a[lane & 15];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint2 v = *reinterpret_cast<const uint2 *>(ra + 32 * kq + 4 * u);
            aq[u] = __builtin_bit_cast(half8, make_uint4(v.x, v.x, v.y, v.y));
        }
        const _Float16 *rp = ls.ap[lane & 15];
#pragma unroll
        for (int s = 0; s < 4; ++s) ap[s] = *reinterpret_cast<const half8 *>(rp + 32 * kq + 8 * s);
    }

    // ---- phase 1: scores into LDS, running (max, sum) per own head
    float m[kOwn<G>], l[kOwn<G>];
    int lim[kOwn<G>];
#pragma unroll
    for (int j = 0; j < kOwn<G>; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
        lim[j] = L;
    }
    auto sink = [&](int h, int tok, float v) { lds.sc[h * LD + (tok - t0)] = v; };
    auto scan = [&](auto full_c) {
        constexpr bool F = decltype(full_c)::value;
        if (t0 >= t1) return;
        // slices are requested two ahead, and only inside the range: the
        // arrival below waits for every outstanding access of the block
        for (int base = t0;;) {
            if (base + 2 * kQSlice < t1) load_ktiles<kQWaves>(tc, base + 2 * kQSlice, tmax, wave, t, kq, kid, ksg, knm);
            score_ktiles<F, false, G, kQWaves>(ta, base, t1, wave, t, kq, ls.pair, ls.sgn, aq, ap, sink, lim, m, l);
            base += kQSlice;
            if (base >= t1) break;
            if (base + 2 * kQSlice < t1) load_ktiles<kQWaves>(ta, base + 2 * kQSlice, tmax, wave, t, kq, kid, ksg, knm);
            score_ktiles<F, false, G, kQWaves>(tb, base, t1, wave, t, kq, ls.pair, ls.sgn, aq, ap, sink, lim, m, l);
            base += kQSlice;
            if (base >= t1) break;
            if (base + 2 * kQSlice < t1) load_ktiles<kQWaves>(tb, base + 2 * kQSlice, tmax, wave, t, kq, kid, ksg, knm);
            score_ktiles<F, false, G, kQWaves>(tc, base, t1, wave, t, kq, ls.pair, ls.sgn, aq, ap, sink, lim, m, l);
            base += kQSlice;
            if (base >= t1) break;
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
            lds.red[wave][own_head<G>(kq, j)][0] = m[j];
            lds.red[wave][own_head<G>(kq, j)][1] = l[j];
        }
    }
    __syncthreads();  // scores and partial statistics complete; the scan's tables are free
    if (blk == 0) {
        // the zeroed output is visible before this block's statistics are
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    }
    // block statistics per head, in natural-log units
    uint64_t *slots = reinterpret_cast<uint64_t *>(a.stats) + int64_t(row) * a.nblk * G;  // [nblk][G]
    if (tid < G) {
        float bm = -INFINITY, bl = 0.0f;
        for (int w = 0; w < kQWaves; ++w) bm = fmaxf(bm, lds.red[w][tid][0]);
        if (bm != -INFINITY)
            for (int w = 0; w < kQWaves; ++w) bl += lds.red[w][tid][1] * fast_exp2(lds.red[w][tid][0] - bm);
        bm = bm == -INFINITY ? bm : bm / kLog2e;
        if (a.nblk > 1) {
            // one 64-bit slot carries both values and marks them written: a
            // written slot is never zero (an empty block stores -inf, 0)
            const uint64_t v = uint64_t(__float_as_uint(bm)) | (uint64_t(__float_as_uint(bl)) << 32);
            __hip_atomic_store(slots + int64_t(blk) * G + tid, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            lds.M[tid] = bm;
            lds.invL[tid] = bl > 0.0f ? 1.0f / bl : 0.0f;
            lds.okw[tid] = 1;
        }
    }

    // ---- barrier of the row's blocks: wave h polls head h's slots (bounded
    // spin) and reduces them to the exact statistics; device-coherent atomic
    // accesses only, no cache-wide fences
    if (a.nblk > 1 && wave < G) {
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
            if (__builtin_amdgcn_s_memrealtime() - tstart > kQSpinTicks) {
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
            lds.M[wave] = mm;
            lds.invL[wave] = ll > 0.0f ? 1.0f / ll : 0.0f;
            lds.okw[wave] = ok;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int ok = 1;
        for (int h = 0; h < G; ++h) ok &= lds.okw[h];
        lds.ok = ok;
    }
    VL &vl = lds.u.v;
    if constexpr (VK != TQ_KIND_Q8) {
        if (tid < VL::kVPairs)
            vl.vpair[tid] = make_float2(a.tab->levels[VB - 1][tid & ((1 << VB) - 1)], a.tab->levels[VB - 1][tid >> VB]);
    }
    __syncthreads();

    // ---- phase 2: the compacting V pass over the block's range
    if (lds.ok && n_tok > 0) {  // uniform over the block
        float sv[R][G];
        auto load_super = [&](int base) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int tt = min(base + kVThreads * r + tid, tmax);
#pragma unroll
                for (int g = 0; g < G; ++g) sv[r][g] = lds.sc[g * LD + (tt - t0)];
                vraw[r] = vn_base[tt];
            }
        };
        // the first super-slice: scores from LDS, V scale words already here
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tt = min(t0 + kVThreads * r + tid, tmax);
#pragma unroll
            for (int g = 0; g < G; ++g) sv[r][g] = lds.sc[g * LD + (tt - t0)];
        }
        values_compact<G, VK, VB, kQSuper, true>(a, b, kvh, vrow, t0, t1, lds.M, lds.invL, sv, vraw, load_super, vl);
    } else if (!lds.ok && wave < G) {
        // a row whose blocks did not all arrive: NaN outputs instead of a hang
        float *o = a.out + io_row(a, b, kvh, wave) * 128;
        __hip_atomic_fetch_add(o + lane, __builtin_nanf(""), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(o + lane + 64, __builtin_nanf(""), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // departure: the last block of the row to leave clears the row's slots
    // and its counter for the next call (no block reads them any more)
    if (a.nblk > 1) {
        uint32_t *depart = a.sync + row;
        __syncthreads();
        if (tid == 0)
            lds.last = __hip_atomic_fetch_add(depart, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       uint32_t(a.nblk) - 1;
        __syncthreads();
        if (lds.last) {
            for (int i = tid; i < a.nblk * G; i += kQThreads)
                __hip_atomic_store(slots + i, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0) __hip_atomic_store(depart, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------------------------ launch
template <int KB, int VB>
static int launch_fused4_t(const AttnArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((attn_fused4_kernel<TQ_KIND_PROD, KB, TQ_KIND_MSE, VB>), dim3(unsigned(a.nblk),
                       unsigned(a.B * a.Hkv)), dim3(kQThreads), 0, s, a, a.kidx, a.ksign, a.knorm);
    return int(hipGetLastError());
}

template <int KB>
static int fused4_dispatch_v(const AttnArgs &a, tq_format vf, hipStream_t s) {
    switch (vf.bits) {
        case 2: return launch_fused4_t<KB, 2>(a, s);
        case 3: return launch_fused4_t<KB, 3>(a, s);
        case 4: return launch_fused4_t<KB, 4>(a, s);
    }
    return int(hipErrorInvalidValue);
}

int launch_attn_fused4(const AttnArgs &a, tq_format kf, tq_format vf, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!fused4_formats(kf, vf) || a.Hq != 4 * a.Hkv) return int(hipErrorInvalidValue);
    switch (kf.bits) {  // codebook bits of the TurboQuant K (plus the QJL bit)
        case 1: return fused4_dispatch_v<1>(a, vf, s);
        case 2: return fused4_dispatch_v<2>(a, vf, s);
        case 3: return fused4_dispatch_v<3>(a, vf, s);
    }
    return int(hipErrorInvalidValue);
}

// Blocks of the 4-head kernel resident at once on the current device (as
// fused_capacity), cached per device; 0 when it cannot be resident.
int fused4_capacity() {
    static int cache[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    const int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v != 0) return v > 0 ? v : 0;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(attn_fused4_kernel<TQ_KIND_PROD, 3, TQ_KIND_MSE, 4>), kQThreads,
            0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        per_cu = cus = 0;
    const int cap = per_cu > 0 && cus > 0 ? per_cu * cus : 0;
    __atomic_store_n(&cache[dev], cap > 0 ? cap : -1, __ATOMIC_RELAXED);
    return cap;
}

}  // namespace tq
