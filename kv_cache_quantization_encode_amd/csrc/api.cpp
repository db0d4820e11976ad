// libturbokv C ABI: argument validation, plane layouts, table upload and
// dispatch to the HIP kernels.  Every check runs on the host before any HIP
// call, so all error paths can be exercised without a GPU.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <new>

#include "internal.h"

namespace tq {

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

static bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static bool format_ok(tq_format f) {
    switch (f.kind) {
        case TQ_KIND_MSE: return f.bits >= 1 && f.bits <= 4;
        case TQ_KIND_PROD: return f.bits >= 1 && f.bits <= 3;
        case TQ_KIND_Q8: return f.bits == 8;
        case TQ_KIND_MSE32: return f.bits >= 1 && f.bits <= 4;
        case TQ_KIND_PROD32: return f.bits >= 1 && f.bits <= 3;
        default: return false;
    }
}

bool plane_layout(tq_format f, int d, int64_t n_vec, tq_planes_desc *out) {
    if (!format_ok(f) || d != kHeadDim || n_vec < 0) return false;
    if (n_vec > (int64_t(1) << 40)) return false;
    tq_planes_desc p{};
    int64_t off = 0;
    if (f.kind == TQ_KIND_Q8) {
        p.idx_offset = 0;
        p.idx_bytes = n_vec * d;
        off = align256(p.idx_bytes);
        p.norm_offset = off;
        p.norm_bytes = n_vec * (d / 32) * 2;
        off = align256(off + p.norm_bytes);
    } else {
        p.idx_offset = 0;
        p.idx_bytes = n_vec * f.bits * d / 8;
        off = align256(p.idx_bytes);
        if (f.kind == TQ_KIND_PROD || f.kind == TQ_KIND_PROD32) {
            p.sign_offset = off;
            p.sign_bytes = n_vec * d / 8;
            off = align256(off + p.sign_bytes);
        }
        p.norm_offset = off;
        switch (f.kind) {
            case TQ_KIND_PROD: p.norm_bytes = n_vec * 4; break;
            case TQ_KIND_MSE32: p.norm_bytes = n_vec * (d / 32) * 2; break;
            case TQ_KIND_PROD32: p.norm_bytes = n_vec * ((d / 32) * 2 + 2); break;
            default: p.norm_bytes = n_vec * 2; break;
        }
        off = align256(off + p.norm_bytes);
    }
    p.total_bytes = off;
    *out = p;
    return true;
}

AttnPlan attn_plan(int B, int Hq, int Hkv, int T) {
    AttnPlan p{};
    const int64_t rows = int64_t(B) * Hkv;
    int64_t want = (512 + rows - 1) / rows;  // aim for ~512 blocks per pass
    int64_t maxc = (int64_t(T) + 255) / 256;
    int64_t nc = want < maxc ? want : maxc;
    if (nc < 1) nc = 1;
    // every block first forms its query rows (q_rot, q_proj); once the grid
    // has a block per CU (256), chunks of at least 1024 tokens amortise that
    // setup better than more, shorter chunks (measured on the 32-query /
    // 8-KV-head, 32768-token layer: 25.3 us at 256 blocks of 1024 tokens
    // against 27.8 us at 512 blocks of 512)
    const int64_t min_nc = (256 + rows - 1) / rows;
    if (nc * rows > 256 && int64_t(T) < nc * 1024) {
        const int64_t by_len = int64_t(T) / 1024;
        nc = by_len > min_nc ? by_len : min_nc;
    }
    int64_t chunk = (int64_t(T) + nc - 1) / nc;
    chunk = (chunk + 255) / 256 * 256;
    nc = (int64_t(T) + chunk - 1) / chunk;
    if (nc < 1) nc = 1;
    p.n_chunks = int(nc);
    p.chunk = int(chunk);
    const int64_t heads = int64_t(B) * Hq;
    int64_t off = int64_t(kSyncBytes);  // barrier counters of the single-launch path, never written here
    // score rows padded to 32 tokens, so that a 32-token group of a row can
    // be read whole (16-byte aligned) near the end of the sequence
    p.ld_scores = int((int64_t(T) + 31) / 32 * 32);
    p.off_scores = size_t(off); off = align256(off + heads * int64_t(p.ld_scores) * 4);
    // chunk statistics: one column more than chunks, for the new token of a
    // decode step that appends it (scored by an extra block)
    p.off_stats = size_t(off); off = align256(off + heads * (nc + 1) * 2 * 4);
    p.total = size_t(off);
    return p;
}

// Prompt-scale prefill: blocks of 64 (query, head) rows; enough token
// ranges that the grid has ~512 blocks (two per CU), ranges of at least 512
// tokens (multiples of 64).
static AttnPlan prefill_plan(int B, int Hq, int Hkv, int T, int Tq) {
    AttnPlan p{};
    p.tiled = 1;
    const int64_t qblocks = (int64_t(Tq) * (Hq / Hkv) + 63) / 64;
    const int64_t blocks = qblocks * B * Hkv;
    int64_t ns = (512 + blocks - 1) / blocks;
    const int64_t maxs = (int64_t(T) + 511) / 512;
    if (ns > maxs) ns = maxs;
    if (ns < 1) ns = 1;
    int64_t span = (int64_t(T) + ns - 1) / ns;
    span = (span + 63) / 64 * 64;
    ns = (int64_t(T) + span - 1) / span;
    p.n_chunks = int(ns);
    p.chunk = int(span);
    p.off_stats = kSyncBytes;
    p.total = align256(int64_t(kSyncBytes) + int64_t(B) * Tq * Hq * ns * 2 * 4);
    return p;
}

AttnPlan attn_call_plan(int B, int Hq, int Hkv, int T, int Tq, tq_format kf, tq_format vf, int capacity,
                        int capacity4) {
    // prompt-scale prefill kernels past the grouped path's grid limit (within
    // it the grouped decode kernels are faster: measured on the llama8b-like
    // layer, Tq 2048: 11.4 ms against 15.7 ms)
    if (prefill_tiled_call(B, Hkv, Tq, kf, vf)) return prefill_plan(B, Hq, Hkv, T, Tq);
    const int g = Hq / Hkv;
    const int qp = prefill_group(g, Tq);
    AttnPlan p = attn_plan(B * (Tq / qp), Hq * qp, Hkv, T);
    if (block32_format(kf) || block32_format(vf)) return p;  // scores + values passes
    // single launch with 4 query heads per kv head: decode, every block of a
    // row resident at once, a block's scores (tb tokens x 4 heads) in its LDS
    if (Tq == 1 && g == 4 && capacity4 > 0 && fused4_formats(kf, vf)) {
        const int64_t rows = int64_t(B) * Hkv;
        const int64_t slices = (int64_t(T) + kFusedSlice - 1) / kFusedSlice;
        int64_t nblk = capacity4 / rows;
        if (nblk < 1) nblk = 1;
        if (nblk > slices) nblk = slices;
        if (nblk > kFusedMaxBlocks) nblk = kFusedMaxBlocks;
        const int64_t tb = (slices + nblk - 1) / nblk * kFusedSlice;
        nblk = (int64_t(T) + tb - 1) / tb;
        if (tb <= kFusedMaxTokens && rows * nblk <= capacity4 && rows <= kSyncRows &&
            rows * nblk <= kFusedMaxGrid) {
            AttnPlan f = p;
            f.fused4 = 1;
            f.nblk = int(nblk);
            f.tb = int(tb);
            return f;
        }
        return p;
    }
    // single launch: decode with 8 query heads per kv head and a V codec the
    // fused kernel reads (2-bit codebook, q8); every block of a row is resident
    // at once, and a block's scores (tb tokens x 8 heads) fit its LDS
    if (Tq != 1 || g != 8 || capacity <= 0) return p;
    if (!(vf.kind == TQ_KIND_Q8 || (vf.kind == TQ_KIND_MSE && vf.bits == 2))) return p;
    const int64_t rows = int64_t(B) * Hkv;
    const int64_t slices = (int64_t(T) + kFusedSlice - 1) / kFusedSlice;
    int64_t nblk = capacity / rows;
    if (nblk < 1) nblk = 1;
    if (nblk > slices) nblk = slices;
    if (nblk > kFusedMaxBlocks) nblk = kFusedMaxBlocks;
    const int64_t tb = (slices + nblk - 1) / nblk * kFusedSlice;
    if (tb > kFusedMaxTokens) return p;
    nblk = (int64_t(T) + tb - 1) / tb;
    if (nblk > 1 && (rows > kSyncRows || rows * nblk > kFusedMaxGrid)) return p;
    AttnPlan f{};
    f.fused = 1;
    f.nblk = int(nblk);
    f.tb = int(tb);
    f.off_sync = 0;
    f.off_stats = kSyncCounterBytes;
    f.total = kSyncBytes;
    return f;
}

}  // namespace tq

using namespace tq;

extern "C" {

const char *tq_status_str(tq_status s) {
    switch (s) {
        case TQ_OK: return "ok";
        case TQ_ERR_INVALID_ARG: return "invalid argument";
        case TQ_ERR_UNSUPPORTED: return "unsupported by this build";
        case TQ_ERR_HIP: return "HIP runtime error";
        case TQ_ERR_ALLOC: return "allocation failed";
        case TQ_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

tq_status tq_host_tables(int head_dim, int qjl_dim, uint64_t seed, double *levels, double *bounds,
                         float *signs, uint16_t *S) {
    if (head_dim < 2 || head_dim > 256 || (head_dim & (head_dim - 1))) return TQ_ERR_INVALID_ARG;
    if (qjl_dim < 1 || qjl_dim > 4096 || (int64_t(qjl_dim) * head_dim) % 2) return TQ_ERR_INVALID_ARG;
    if (levels || bounds) {
        for (int b = 1; b <= 4; ++b) {
            double lv[16] = {0}, bd[16] = {0};
            lloyd_max_gaussian(b, lv, bd);
            if (levels) std::memcpy(levels + 16 * (b - 1), lv, sizeof lv);
            if (bounds) std::memcpy(bounds + 16 * (b - 1), bd, sizeof bd);
        }
    }
    if (signs || S) {
        float *sg = new (std::nothrow) float[head_dim];
        uint16_t *ss = new (std::nothrow) uint16_t[size_t(qjl_dim) * head_dim];
        if (!sg || !ss) { delete[] sg; delete[] ss; return TQ_ERR_ALLOC; }
        random_tables(head_dim, qjl_dim, seed, sg, ss);
        if (signs) std::memcpy(signs, sg, sizeof(float) * head_dim);
        if (S) std::memcpy(S, ss, sizeof(uint16_t) * size_t(qjl_dim) * head_dim);
        delete[] sg;
        delete[] ss;
    }
    return TQ_OK;
}

tq_status tq_packed_layout(tq_format f, int head_dim, int64_t n_vec, tq_planes_desc *out) {
    if (!out) return TQ_ERR_INVALID_ARG;
    if (!format_ok(f) || n_vec < 0) return TQ_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return TQ_ERR_UNSUPPORTED;
    return plane_layout(f, head_dim, n_vec, out) ? TQ_OK : TQ_ERR_INVALID_ARG;
}

tq_status tq_codebook_init(tq_ctx **ctx, int head_dim, int qjl_dim, uint64_t seed, void *stream) {
    if (!ctx) return TQ_ERR_INVALID_ARG;
    *ctx = nullptr;
    if (head_dim < 2 || head_dim > 256 || (head_dim & (head_dim - 1))) return TQ_ERR_INVALID_ARG;
    if (qjl_dim < 1) return TQ_ERR_INVALID_ARG;
    if (head_dim != kHeadDim || qjl_dim != kHeadDim) return TQ_ERR_UNSUPPORTED;
    DevTables *host = new (std::nothrow) DevTables;
    tq_ctx *c = new (std::nothrow) tq_ctx;
    if (!host || !c) { delete host; delete c; return TQ_ERR_ALLOC; }
    if (!build_device_tables(head_dim, qjl_dim, seed, host)) { delete host; delete c; return TQ_ERR_UNSUPPORTED; }
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        delete host; delete c; return TQ_ERR_HIP;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) { delete host; delete c; return TQ_ERR_UNSUPPORTED; }
    // this device's copy of the library-owned attention workspace
    if (scratch_prepare(dev) != 0) { delete host; delete c; return TQ_ERR_HIP; }
    void *d = nullptr;
    if (hipMalloc(&d, sizeof(DevTables)) != hipSuccess) { delete host; delete c; return TQ_ERR_ALLOC; }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(d, host, sizeof(DevTables), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        (void)hipFree(d); delete host; delete c; return TQ_ERR_HIP;
    }
    delete host;
    c->head_dim = head_dim;
    c->qjl_dim = qjl_dim;
    c->seed = seed;
    c->device = dev;
    c->dev = static_cast<DevTables *>(d);
    *ctx = c;
    return TQ_OK;
}

tq_status tq_ctx_destroy(tq_ctx *ctx) {
    if (!ctx) return TQ_ERR_INVALID_ARG;
    hipError_t e = hipFree(ctx->dev);
    delete ctx;
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

tq_status tq_encode_kv(const tq_ctx *ctx, const void *k_f16, const void *v_f16, int64_t n_vec,
                       tq_format kf, tq_format vf, void *k_packed, void *v_packed, void *stream) {
    if (!ctx || n_vec < 0) return TQ_ERR_INVALID_ARG;
    if (n_vec > kMaxRows) return TQ_ERR_UNSUPPORTED;
    if (!k_f16 && !v_f16) return TQ_ERR_INVALID_ARG;
    tq_planes_desc kl{}, vl{};
    if (k_f16) {
        if (!k_packed || !aligned(k_f16, 16) || !aligned(k_packed, 256)) return TQ_ERR_INVALID_ARG;
        if (!plane_layout(kf, ctx->head_dim, n_vec, &kl)) return TQ_ERR_INVALID_ARG;
    }
    if (v_f16) {
        if (!v_packed || !aligned(v_f16, 16) || !aligned(v_packed, 256)) return TQ_ERR_INVALID_ARG;
        if (!plane_layout(vf, ctx->head_dim, n_vec, &vl)) return TQ_ERR_INVALID_ARG;
    }
    if (n_vec == 0) return TQ_OK;
    if (k_f16 && v_f16) {
        const int r = launch_encode_pair(ctx->dev, k_f16, v_f16, n_vec, kf, vf, k_packed, v_packed, kl, vl, stream);
        if (r != kPairDeclined) return r == 0 ? TQ_OK : TQ_ERR_HIP;
    }
    if (k_f16 && launch_encode(ctx->dev, k_f16, n_vec, kf, k_packed, kl, stream) != 0) return TQ_ERR_HIP;
    if (v_f16 && launch_encode(ctx->dev, v_f16, n_vec, vf, v_packed, vl, stream) != 0) return TQ_ERR_HIP;
    return TQ_OK;
}

tq_status tq_append_kv(const tq_ctx *ctx, const void *k_new_f16, const void *v_new_f16, int B, int Hkv,
                       int T_cap, const int32_t *pos, tq_format kf, tq_format vf, void *k_packed,
                       void *v_packed, void *stream) {
    if (!ctx || !pos || B < 1 || Hkv < 1 || T_cap < 1) return TQ_ERR_INVALID_ARG;
    if (!k_new_f16 && !v_new_f16) return TQ_ERR_INVALID_ARG;
    if (!aligned(pos, 4)) return TQ_ERR_INVALID_ARG;
    const int64_t n_cache = int64_t(B) * Hkv * T_cap;
    if (n_cache > kMaxRows) return TQ_ERR_UNSUPPORTED;
    tq_planes_desc kl{}, vl{};
    if (k_new_f16) {
        if (!k_packed || !aligned(k_new_f16, 16) || !aligned(k_packed, 256)) return TQ_ERR_INVALID_ARG;
        if (!plane_layout(kf, ctx->head_dim, n_cache, &kl)) return TQ_ERR_INVALID_ARG;
    }
    if (v_new_f16) {
        if (!v_packed || !aligned(v_new_f16, 16) || !aligned(v_packed, 256)) return TQ_ERR_INVALID_ARG;
        if (!plane_layout(vf, ctx->head_dim, n_cache, &vl)) return TQ_ERR_INVALID_ARG;
    }
    if (k_new_f16 && v_new_f16) {
        const int r = launch_append_kv(ctx->dev, k_new_f16, v_new_f16, B, Hkv, T_cap, pos, kf, vf, k_packed,
                                       v_packed, kl, vl, stream);
        if (r != kPairDeclined) return r == 0 ? TQ_OK : TQ_ERR_HIP;
    }
    if (k_new_f16 && launch_append(ctx->dev, k_new_f16, B, Hkv, T_cap, pos, kf, k_packed, kl, stream) != 0)
        return TQ_ERR_HIP;
    if (v_new_f16 && launch_append(ctx->dev, v_new_f16, B, Hkv, T_cap, pos, vf, v_packed, vl, stream) != 0)
        return TQ_ERR_HIP;
    return TQ_OK;
}

tq_status tq_decode_kv(const tq_ctx *ctx, const void *packed, tq_format f, int64_t n_vec,
                       void *out_f16, void *stream) {
    if (!ctx || !packed || !out_f16 || n_vec < 0) return TQ_ERR_INVALID_ARG;
    if (n_vec > kMaxRows) return TQ_ERR_UNSUPPORTED;
    if (!aligned(packed, 256) || !aligned(out_f16, 16)) return TQ_ERR_INVALID_ARG;
    tq_planes_desc l{};
    if (!plane_layout(f, ctx->head_dim, n_vec, &l)) return TQ_ERR_INVALID_ARG;
    if (n_vec == 0) return TQ_OK;
    return launch_decode(ctx->dev, packed, f, n_vec, l, out_f16, stream) == 0 ? TQ_OK : TQ_ERR_HIP;
}

size_t tq_attn_workspace_bytes(int B, int Hq, int Hkv, int T, tq_format kf, tq_format vf) {
    return tq_attn_prefill_workspace_bytes(B, Hq, Hkv, T, 1, kf, vf);
}

size_t tq_attn_prefill_workspace_bytes(int B, int Hq, int Hkv, int T, int Tq, tq_format kf, tq_format vf) {
    (void)kf;
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || Tq < 1 || Hq % Hkv) return 0;
    if (int64_t(B) * Hkv > kMaxGridY) return 0;
    // the grouped prefill path puts (sequence, query group, kv head) on grid y
    if (!prefill_tiled_call(B, Hkv, Tq, kf, vf) && int64_t(B) * Tq * Hkv > kMaxGridY) return 0;
    return attn_call_plan(B, Hq, Hkv, T, Tq, kf, vf, fused_capacity(), fused4_capacity()).total;
}

// Decode (Tq = 1) and causal prefill (Tq queries per sequence) share one path:
// query i of sequence b becomes virtual sequence b * Tq + i over b's cache.
// Every argument check, nothing launched.
static tq_status attn_check(const tq_ctx *ctx, const void *q_f16, const void *k_packed, const void *v_packed,
                            tq_format kf, tq_format vf, int B, int Hq, int Hkv, int T, int Tq,
                            const int32_t *seq_lens, float sparse_v_tau, float *out_f32, void *workspace,
                            size_t ws_bytes, tq_planes_desc *kl, tq_planes_desc *vl, AttnPlan *plan) {
    if (!ctx || !q_f16 || !k_packed || !v_packed || !out_f32) return TQ_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || Tq < 1 || Hq % Hkv) return TQ_ERR_INVALID_ARG;
    if (!(sparse_v_tau >= 0.0f) || !std::isfinite(sparse_v_tau)) return TQ_ERR_INVALID_ARG;
    if (!aligned(q_f16, 16) || !aligned(k_packed, 256) || !aligned(v_packed, 256) ||
        !aligned(out_f32, 16) || (seq_lens && !aligned(seq_lens, 4)))
        return TQ_ERR_INVALID_ARG;
    if (!format_ok(kf) || !format_ok(vf)) return TQ_ERR_INVALID_ARG;
    if (vf.kind == TQ_KIND_PROD || vf.kind == TQ_KIND_PROD32) return TQ_ERR_UNSUPPORTED;
    if ((block32_format(kf) || block32_format(vf)) && Tq != 1) return TQ_ERR_UNSUPPORTED;
    const int g = Hq / Hkv;
    if (g != 1 && g != 2 && g != 4 && g != 8) return TQ_ERR_UNSUPPORTED;
    if (int64_t(B) * Hkv * T > kMaxRows || int64_t(T) * 128 >= (int64_t(1) << 31)) return TQ_ERR_UNSUPPORTED;
    if (int64_t(B) * Hkv > kMaxGridY) return TQ_ERR_UNSUPPORTED;
    if (!prefill_tiled_call(B, Hkv, Tq, kf, vf) && int64_t(B) * Tq * Hkv > kMaxGridY) return TQ_ERR_UNSUPPORTED;
    const int64_t n_vec = int64_t(B) * Hkv * T;
    if (!plane_layout(kf, ctx->head_dim, n_vec, kl) || !plane_layout(vf, ctx->head_dim, n_vec, vl))
        return TQ_ERR_INVALID_ARG;
    *plan = attn_call_plan(B, Hq, Hkv, T, Tq, kf, vf, fused_capacity(), fused4_capacity());
    if (!workspace || !aligned(workspace, 256) || ws_bytes < plan->total) return TQ_ERR_WORKSPACE;
    return TQ_OK;
}

static tq_status attn_call(const tq_ctx *ctx, const void *q_f16, const void *k_packed, const void *v_packed,
                           tq_format kf, tq_format vf, int B, int Hq, int Hkv, int T, int Tq,
                           const int32_t *seq_lens, float sparse_v_tau, float *out_f32, void *workspace,
                           size_t ws_bytes, void *stream) {
    tq_planes_desc kl{}, vl{};
    AttnPlan plan{};
    const tq_status st = attn_check(ctx, q_f16, k_packed, v_packed, kf, vf, B, Hq, Hkv, T, Tq, seq_lens,
                                    sparse_v_tau, out_f32, workspace, ws_bytes, &kl, &vl, &plan);
    if (st != TQ_OK) return st;
    return launch_attn(ctx->dev, q_f16, k_packed, v_packed, kf, vf, kl, vl, B, Hq, Hkv, T, Tq, seq_lens,
                       sparse_v_tau, out_f32, workspace, plan, 0, nullptr, stream) == 0
               ? TQ_OK
               : TQ_ERR_HIP;
}

tq_status tq_attn_decode_append(const tq_ctx *ctx, const void *q_f16, const void *k_new_f16,
                                const void *v_new_f16, const int32_t *pos, void *k_packed, void *v_packed,
                                tq_format kf, tq_format vf, int B, int Hq, int Hkv, int T_cap,
                                float sparse_v_tau, float *out_f32, void *workspace, size_t ws_bytes,
                                void *stream) {
    if (!ctx || !k_new_f16 || !v_new_f16 || !pos) return TQ_ERR_INVALID_ARG;
    if (!aligned(k_new_f16, 16) || !aligned(v_new_f16, 16)) return TQ_ERR_INVALID_ARG;
    tq_planes_desc kl{}, vl{};
    AttnPlan plan{};
    const tq_status st = attn_check(ctx, q_f16, k_packed, v_packed, kf, vf, B, Hq, Hkv, T_cap, 1, pos,
                                    sparse_v_tau, out_f32, workspace, ws_bytes, &kl, &vl, &plan);
    if (st != TQ_OK) return st;
    // the 4-head single launch has no append: the two-pass plan of the same
    // call (its fields are kept in the plan) appends in its scores pass
    plan.fused4 = 0;
    // (the two-pass kernels put the rows' extra blocks in grid rows of their
    // own: at most twice B * Hkv grid rows)
    if (append_in_attention(kf, vf) && (plan.fused || 2 * int64_t(B) * Hkv <= kMaxGridY)) {
        const AttnAppend app{k_new_f16, v_new_f16, k_packed, v_packed};
        return launch_attn(ctx->dev, q_f16, k_packed, v_packed, kf, vf, kl, vl, B, Hq, Hkv, T_cap, 1, pos,
                           sparse_v_tau, out_f32, workspace, plan, 0, &app, stream) == 0
                   ? TQ_OK
                   : TQ_ERR_HIP;
    }
    // other formats: the append launch first, then attention over pos + 1
    int r = launch_append_kv(ctx->dev, k_new_f16, v_new_f16, B, Hkv, T_cap, pos, kf, vf, k_packed, v_packed, kl,
                             vl, stream);
    if (r == kPairDeclined) {
        r = launch_append(ctx->dev, k_new_f16, B, Hkv, T_cap, pos, kf, k_packed, kl, stream);
        if (r == 0) r = launch_append(ctx->dev, v_new_f16, B, Hkv, T_cap, pos, vf, v_packed, vl, stream);
    }
    if (r != 0) return TQ_ERR_HIP;
    return launch_attn(ctx->dev, q_f16, k_packed, v_packed, kf, vf, kl, vl, B, Hq, Hkv, T_cap, 1, pos,
                       sparse_v_tau, out_f32, workspace, plan, 1, nullptr, stream) == 0
               ? TQ_OK
               : TQ_ERR_HIP;
}

tq_status tq_attn_decode_noalloc(const tq_ctx *ctx, const void *q_f16, const void *k_packed,
                                 const void *v_packed, tq_format kf, tq_format vf, int B, int Hq, int Hkv,
                                 int T, const int32_t *seq_lens, float sparse_v_tau, float *out_f32,
                                 void *stream) {
    if (!ctx) return TQ_ERR_INVALID_ARG;
    // the library-owned workspace lives on the ctx's device: it must be current
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TQ_ERR_HIP;
    if (dev != ctx->device) return TQ_ERR_INVALID_ARG;
    void *ws = scratch_device_ptr(dev);
    if (!ws) return TQ_ERR_HIP;
    return attn_call(ctx, q_f16, k_packed, v_packed, kf, vf, B, Hq, Hkv, T, 1, seq_lens, sparse_v_tau, out_f32, ws,
                     kScratchBytes, stream);
}

tq_status tq_attn_decode(const tq_ctx *ctx, const void *q_f16, const void *k_packed,
                         const void *v_packed, tq_format kf, tq_format vf, int B, int Hq, int Hkv,
                         int T, const int32_t *seq_lens, float sparse_v_tau, float *out_f32,
                         void *workspace, size_t ws_bytes, void *stream) {
    return attn_call(ctx, q_f16, k_packed, v_packed, kf, vf, B, Hq, Hkv, T, 1, seq_lens, sparse_v_tau, out_f32,
                     workspace, ws_bytes, stream);
}

tq_status tq_attn_prefill(const tq_ctx *ctx, const void *q_f16, const void *k_packed,
                          const void *v_packed, tq_format kf, tq_format vf, int B, int Hq, int Hkv,
                          int T, int Tq, const int32_t *seq_lens, float sparse_v_tau, float *out_f32,
                          void *workspace, size_t ws_bytes, void *stream) {
    return attn_call(ctx, q_f16, k_packed, v_packed, kf, vf, B, Hq, Hkv, T, Tq, seq_lens, sparse_v_tau, out_f32,
                     workspace, ws_bytes, stream);
}

tq_status tq_minmax_quant(const void *x_f16, int64_t n, int group_size, int bits, void *codes,
                          void *scale_f16, void *zero_f16, void *stream) {
    if (!x_f16 || !codes || !scale_f16 || !zero_f16 || n < 0) return TQ_ERR_INVALID_ARG;
    if (bits < 1 || bits > 8 || group_size < 1) return TQ_ERR_INVALID_ARG;
    if (group_size != 64 || bits < 2 || bits > 4) return TQ_ERR_UNSUPPORTED;
    if (n % group_size) return TQ_ERR_INVALID_ARG;
    if (!aligned(x_f16, 16) || !aligned(codes, 4) || !aligned(scale_f16, 2) || !aligned(zero_f16, 2))
        return TQ_ERR_INVALID_ARG;
    if (n == 0) return TQ_OK;
    return launch_minmax_quant(x_f16, n, bits, codes, scale_f16, zero_f16, stream) == 0 ? TQ_OK
                                                                                       : TQ_ERR_HIP;
}

tq_status tq_minmax_dequant(const void *codes, const void *scale_f16, const void *zero_f16,
                            int64_t n, int group_size, int bits, void *out_f16, void *stream) {
    if (!codes || !scale_f16 || !zero_f16 || !out_f16 || n < 0) return TQ_ERR_INVALID_ARG;
    if (bits < 1 || bits > 8 || group_size < 1) return TQ_ERR_INVALID_ARG;
    if (group_size != 64 || bits < 2 || bits > 4) return TQ_ERR_UNSUPPORTED;
    if (n % group_size) return TQ_ERR_INVALID_ARG;
    if (!aligned(codes, 4) || !aligned(scale_f16, 2) || !aligned(zero_f16, 2) || !aligned(out_f16, 16))
        return TQ_ERR_INVALID_ARG;
    if (n == 0) return TQ_OK;
    return launch_minmax_dequant(codes, scale_f16, zero_f16, n, bits, out_f16, stream) == 0
               ? TQ_OK
               : TQ_ERR_HIP;
}

}  // extern "C"
