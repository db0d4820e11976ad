// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/turbokv.h"

namespace tq {

constexpr int kHeadDim = 128;  // head_dim (= QJL dimension m) of this build
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 16;  // rows per packed tensor (32-bit row indices)
constexpr int64_t kMaxGridY = 65535;  // attention grids put (sequence, kv head) pairs on y

// One bucket of the quantiser lookup: z in bucket j gets index
// base + (z >= thr) and level (z >= thr ? c_hi : c_lo).
struct QBucket {
    float thr;
    uint32_t base;
    float c_lo, c_hi;
};
// Bucket j = floor(4 z + 48.5) for j = 0..96 covers |z| <= 12.125, more than
// the largest standardised coordinate sqrt(128) (|(Rx)_i| <= ||x||).
constexpr int kBuckets = 97;

// Tables uploaded once per ctx.  Plain data, identical on host and device.
struct DevTables {
    float levels[4][16];             // row b-1: 2^b ascending N(0,1) Lloyd-Max levels
    float bounds[4][16];             // row b-1: 2^b-1 midpoints, then +inf padding
    uint32_t sign_pair_xor[4][16];   // fp16-pair sign flips of D per lane quarter (load layout A)
    QBucket qlut[4][kBuckets];       // row b-1: quantiser buckets of the b-bit codebook
    float signs[kHeadDim];           // D
    uint16_t S[kHeadDim * kHeadDim]; // QJL matrix, fp16 bits, row-major [m][d]
    uint16_t ST[kHeadDim * kHeadDim];// its transpose [d][m]
    uint16_t S_enc[32 * 64 * 8];     // S as encode MFMA A-fragments
    uint16_t St_dec[32 * 64 * 8];    // S^T as dequant MFMA A-fragments
};

// tables.cpp (host only)
uint16_t double_to_half_rne(double v);
double half_to_double(uint16_t h);
void lloyd_max_gaussian(int bits, double *levels, double *bounds);
void random_tables(int d, int m, uint64_t seed, float *signs, uint16_t *S);
bool build_device_tables(int d, int m, uint64_t seed, DevTables *t);

// Plane layout (api.cpp); returns false for an invalid format/size.
bool plane_layout(tq_format f, int d, int64_t n_vec, tq_planes_desc *out);

// Attention partitioning shared by the host (workspace size) and launchers.
struct AttnPlan {
    int n_chunks;    // token chunks per (batch, kv head)
    int chunk;       // tokens per chunk (multiple of 256)
    int ld_scores;   // score row stride in floats: T rounded up to 32
    size_t off_scores, off_stats, total;
    // single-launch path (decode, 8 query heads per kv head, 2-bit codebook or
    // q8 V): nblk blocks of tb tokens per row; departure counters at
    // off_sync, (max, sum) slots at off_stats
    int fused, nblk, tb;
    size_t off_sync;
    // prompt-scale prefill (attn_prefill.hip): n_chunks token ranges of
    // chunk tokens, (max, sum) statistics per row and range at off_stats
    int tiled;
    // single launch with 4 query heads per kv head (attn_fused4.hip): nblk
    // blocks of tb tokens per row, departure counters at the start of the
    // workspace and (max, sum) slots after them; the other fields keep the
    // two-pass plan of the same call (same workspace size), which a decode
    // step that appends takes instead
    int fused4;
};
AttnPlan attn_plan(int B, int Hq, int Hkv, int T);
// The plan of one attention call: the single-launch path when its shape and
// the device allow it, else the two-pass plan.  capacity = blocks of the
// single-launch kernel resident at once on the current device (0: unknown).
AttnPlan attn_call_plan(int B, int Hq, int Hkv, int T, int Tq, tq_format kf, tq_format vf, int capacity,
                        int capacity4 = 0);
inline bool block32_format(tq_format f) { return f.kind == TQ_KIND_MSE32 || f.kind == TQ_KIND_PROD32; }
// Tokens per block and block size limits of the single-launch kernel.
constexpr int kFusedSlice = 512;
constexpr int kFusedMaxTokens = 4096;
constexpr int kFusedMaxBlocks = 256;  // blocks per row (statistics read in one pass)
// Every attention workspace plan starts with kSyncBytes for the barrier of
// the single-launch path: a departure counter per row (rows < kSyncRows),
// then a 64-bit (max, sum) slot per block and head (grids of up to
// kFusedMaxGrid blocks).  Nothing else is ever stored there and every call
// leaves it zero, so a workspace zero-filled once stays valid for calls of
// any shape and path.
constexpr int kSyncRows = 1024;
constexpr int kFusedMaxGrid = 1024;
constexpr size_t kSyncCounterBytes = size_t(kSyncRows) * 4;
constexpr size_t kSyncBytes = kSyncCounterBytes + size_t(kFusedMaxGrid) * 8 * 8;
// Prefill queries of one sequence that share a scores pass: the largest of
// 8/g, ..., 2, 1 (g = query heads per kv head) dividing Tq, so that the
// group's g * qp rows fill at most the 8 query rows of one pass.
inline int prefill_group(int g, int tq) {
    for (int qp = 8 / g; qp > 1; qp /= 2)
        if (tq % qp == 0) return qp;
    return 1;
}

// Kernel launchers (HIP translation units).  All return a hipError_t as int.
int launch_encode(const DevTables *tab, const void *x, int64_t n_vec, tq_format f, void *packed,
                  const tq_planes_desc &lay, void *stream);
int launch_append(const DevTables *tab, const void *x, int B, int hkv, int tcap, const int32_t *pos,
                  tq_format f, void *packed, const tq_planes_desc &lay, void *stream);
// K (PROD) and V (MSE) of a small encode, or of one decode step's append,
// in one launch.  kPairDeclined: nothing launched (formats or size), the
// caller encodes K and V separately.
constexpr int kPairDeclined = -1;
int launch_encode_pair(const DevTables *tab, const void *k, const void *v, int64_t n_vec, tq_format kf,
                       tq_format vf, void *kp, void *vp, const tq_planes_desc &kl, const tq_planes_desc &vl,
                       void *stream);
int launch_append_kv(const DevTables *tab, const void *k, const void *v, int B, int hkv, int tcap,
                     const int32_t *pos, tq_format kf, tq_format vf, void *kp, void *vp,
                     const tq_planes_desc &kl, const tq_planes_desc &vl, void *stream);
int launch_decode(const DevTables *tab, const void *packed, tq_format f, int64_t n_vec,
                  const tq_planes_desc &lay, void *out, void *stream);
// Causal prefill with many queries per block (attn_prefill.hip): K PROD or
// MSE, V MSE; a.chunk / a.n_chunks = token range length / count.
inline bool prefill_tiled_formats(tq_format kf, tq_format vf) {
    return (kf.kind == TQ_KIND_PROD || kf.kind == TQ_KIND_MSE) && vf.kind == TQ_KIND_MSE;
}
// The prefill calls that take those kernels: the ones past the grouped
// path's grid limit (B * Tq * Hkv grid rows).
inline bool prefill_tiled_call(int B, int Hkv, int Tq, tq_format kf, tq_format vf) {
    return Tq > 1 && prefill_tiled_formats(kf, vf) && int64_t(B) * Tq * Hkv > kMaxGridY;
}
int launch_attn_prefill(const struct AttnArgs &a, tq_format kf, tq_format vf, void *stream);
// Decode attention when K or V uses block-32 norms (attn_generic.hip): a
// scores and a values pass over the two-pass workspace.
int launch_attn_generic(const struct AttnArgs &a, tq_format kf, tq_format vf, void *stream);
// A decode step's new tokens ([B * Hkv][128] fp16 each), encoded by the
// attention launch into the caches it reads (writable aliases of kp, vp).
struct AttnAppend {
    const void *k_new, *v_new;
    void *k_packed, *v_packed;
};
// True when the attention kernels can encode the new token themselves
// (TurboQuant K and codebook V with 128-element norms); other formats take a
// separate append launch first.
inline bool append_in_attention(tq_format kf, tq_format vf) {
    return kf.kind == TQ_KIND_PROD && vf.kind == TQ_KIND_MSE;
}
// len_add: each seq_lens[b] counts len_add more tokens (clamped to [0, T]);
// app: the append of a decode step (nullptr: none).
int launch_attn(const DevTables *tab, const void *q, const void *kp, const void *vp, tq_format kf,
                tq_format vf, const tq_planes_desc &klay, const tq_planes_desc &vlay, int B, int Hq,
                int Hkv, int T, int tq, const int32_t *seq_lens, float tau, float *out, void *ws,
                const AttnPlan &plan, int len_add, const AttnAppend *app, void *stream);
// Single-launch decode attention (attn_fused.hip); capacity of the current
// device for it (0 when it cannot run).
int launch_attn_fused(const struct AttnArgs &a, tq_format kf, tq_format vf, void *stream);
int fused_capacity();
// Single-launch decode attention with 4 query heads per kv head
// (attn_fused4.hip): TurboQuant K, 2/3/4-bit codebook V; capacity as above.
inline bool fused4_formats(tq_format kf, tq_format vf) {
    return kf.kind == TQ_KIND_PROD && kf.bits >= 1 && kf.bits <= 3 && vf.kind == TQ_KIND_MSE && vf.bits >= 2 &&
           vf.bits <= 4;
}
int launch_attn_fused4(const struct AttnArgs &a, tq_format kf, tq_format vf, void *stream);
int fused4_capacity();
// Library-owned attention workspace (scratch.hip): kScratchBytes on every
// GPU the library runs on.  scratch_prepare looks up this device's copy (the
// device must be current); scratch_device_ptr returns it (nullptr if not
// prepared).
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxScratchDevices = 64;
int scratch_prepare(int device);
void *scratch_device_ptr(int device);
int launch_minmax_quant(const void *x, int64_t n, int bits, void *codes, void *scale, void *zero,
                        void *stream);
int launch_minmax_dequant(const void *codes, const void *scale, const void *zero, int64_t n,
                          int bits, void *out, void *stream);

}  // namespace tq

struct tq_ctx {
    int head_dim;
    int qjl_dim;
    uint64_t seed;
    int device;
    tq::DevTables *dev;  // device copy
};
