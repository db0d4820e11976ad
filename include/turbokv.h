/*
 * libturbokv: TurboQuant / TurboQuant+ KV-cache codec and decode attention
 * for AMD Instinct MI355X (gfx950).  C ABI: plain pointers, sizes and a HIP
 * stream passed as void*.  No C++ exceptions cross this boundary.
 *
 * Method sources (web pages, cited by title and section):
 *   [QPQ] quidproquo.cc, "TurboQuant+ KV cache compression": Stage 1
 *         (PolarQuant: L2 norm, random Walsh-Hadamard rotation, Lloyd-Max
 *         Gaussian codebook, per-coordinate indices), Stage 2 (QJL: residual,
 *         residual norm, 1-bit sign of a random projection), format table
 *         (turbo2/3/4), K/V asymmetric strategy (K = both stages, V = Stage 1).
 *   [CXT] chenxutan.com, "TurboQuant+ deep dive": 1.1 cached decode attention,
 *         1.2 KV-cache size, 2.3 QJL (one fixed-seed matrix at both ends,
 *         bit = projection > 0), 3.3 sparse V (no renormalisation), 3.4
 *         backend matrix (each step's new K/V rows written into the cache).
 *   [YYL] yeyulingfeng.com, TurboQuant+ introduction: core item 3 (Boundary V:
 *         first 2 + last 2 layers at q8_0), item 4 (Sparse V below 1e-6).
 *   [MAC] mac-code GitHub issue #1, technical analysis, section 2.1
 *         (per-group asymmetric min-max quantisation, group 64).
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer (inputs, packed planes, outputs,
 *     workspace).  The library allocates device memory only inside
 *     tq_codebook_init and frees it in tq_ctx_destroy.  A ctx is immutable
 *     after init and may be shared by calls on different streams.
 *   - Memory: "device" pointers must be HIP device (or managed) memory on the
 *     current device; "host" pointers are ordinary CPU memory.
 *   - Layout: a K or V tensor of one layer is [n_vec, head_dim] fp16 row-major
 *     (row = one token of one KV head; for attention n_vec = B*Hkv*T in
 *     [B, Hkv, T] order).  Packed tensors are described by tq_packed_layout.
 *   - Errors: every call validates all arguments on the host before any HIP
 *     call and returns a negative tq_status on failure without launching.
 *     Launch failures return TQ_ERR_HIP.  Faults inside a kernel surface at
 *     the caller's next synchronisation of the stream.
 *   - Async: all compute calls are stream-ordered and return immediately.
 */
#ifndef TURBOKV_H
#define TURBOKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
    TQ_OK = 0,
    TQ_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or format */
    TQ_ERR_UNSUPPORTED = -2,  /* valid request this build does not implement */
    TQ_ERR_HIP = -3,          /* a HIP runtime call or launch failed */
    TQ_ERR_ALLOC = -4,        /* device or host allocation failed */
    TQ_ERR_WORKSPACE = -5     /* workspace pointer null or too small */
} tq_status;

/* Codec of one packed tensor.
 *   TQ_KIND_MSE : Stage 1 only ("TurboQuantMSE", the V codec of [QPQ]):
 *                 b-bit codebook indices + fp16 norm.          bits = 1..4
 *   TQ_KIND_PROD: Stage 1 + QJL (the K codec of [QPQ]): b-bit indices,
 *                 1 sign bit per projection, fp16 norm, fp16 residual norm.
 *                 turboN K = {TQ_KIND_PROD, N-1}.              bits = 1..3
 *   TQ_KIND_Q8  : boundary-layer blocks ([YYL] item 3): int8 per element,
 *                 fp16 absmax/127 scale per block of 32.       bits = 8
 *   TQ_KIND_MSE32, TQ_KIND_PROD32: block-32 norm storage ([YYL] technical
 *                 highlights, "block-32 storage"; the [QPQ] format-table
 *                 ratios 16/(2+0.5) = 6.4 and 16/(3+0.5) = 4.57): as MSE and
 *                 PROD, but the Stage-1 norm is kept per block of 32 rotated
 *                 coordinates, n_b = ||(R x)_b||, and each block is
 *                 standardised by its own norm, z = sqrt(32) (R x)_b / n_b.
 *                 PROD32 keeps one residual norm per vector.
 *                                           bits: MSE32 1..4, PROD32 1..3   */
typedef enum tq_kind {
    TQ_KIND_MSE = 0,
    TQ_KIND_PROD = 1,
    TQ_KIND_Q8 = 2,
    TQ_KIND_MSE32 = 3,
    TQ_KIND_PROD32 = 4
} tq_kind;

typedef struct tq_format {
    int32_t kind; /* tq_kind */
    int32_t bits;
} tq_format;

typedef struct tq_ctx tq_ctx;

/* Byte offsets (from the start of one packed buffer) and sizes of its planes.
 * Every plane starts on a 256-byte boundary.
 *   MSE : idx plane   n_vec * bits*d/8 bytes, LSB-first bitstream per row
 *                     (bit j of the code of coordinate i is row bit i*bits+j);
 *         norm plane  n_vec * 2 bytes (fp16 ||x||).
 *   PROD: idx plane as MSE; sign plane n_vec * m/8 bytes (bit p = [(S e)_p > 0]);
 *         norm plane  n_vec * 4 bytes (fp16 ||x|| then fp16 residual norm).
 *   Q8  : idx plane   n_vec * d int8 values; norm plane n_vec * d/32 fp16
 *         block scales; no sign plane.
 *   MSE32: idx plane as MSE; norm plane n_vec * 8 bytes (the d/32 = 4 fp16
 *         block norms of each vector, block order).
 *   PROD32: idx and sign planes as PROD; norm plane n_vec * 10 bytes: the
 *         four fp16 block norms of every vector (n_vec * 8 bytes), then the
 *         fp16 residual norm of every vector (n_vec * 2 bytes).              */
typedef struct tq_planes_desc {
    int64_t idx_offset, idx_bytes;
    int64_t sign_offset, sign_bytes;
    int64_t norm_offset, norm_bytes;
    int64_t total_bytes;
} tq_planes_desc;

/* Build the codec tables for head_dim d and QJL dimension m from a seed
 * ([QPQ] Stage 1 "precomputed Lloyd-Max codebook"; [CXT] 2.3 fixed-seed
 * matrix): Lloyd-Max levels and boundaries of N(0,1) for 1..4 bits (float64
 * on the host, stored as float32), the random sign diagonal D and the
 * m x d Gaussian matrix S (fp16), both drawn from a splitmix64 counter stream
 * (counter i = 1..d -> signs, d+1.. -> Box-Muller pairs, row-major S).
 * Uploads them to the current device and synchronises `stream`.
 * This build supports d = m = 128.  *ctx receives an owning handle. */
tq_status tq_codebook_init(tq_ctx **ctx, int head_dim, int qjl_dim, uint64_t seed, void *stream);
tq_status tq_ctx_destroy(tq_ctx *ctx);

/* Host-only copy of the tables tq_codebook_init would build (no GPU needed).
 * levels: 4*16 doubles (row b-1 holds the 2^b ascending levels of b bits);
 * bounds: 4*16 doubles (row b-1 holds the 2^b - 1 midpoints);
 * signs:  head_dim floats (+1/-1);  S: qjl_dim*head_dim fp16 bit patterns.
 * Any output pointer may be NULL. */
tq_status tq_host_tables(int head_dim, int qjl_dim, uint64_t seed, double *levels, double *bounds,
                         float *signs, uint16_t *S);

/* Plane layout of n_vec packed vectors in format f (host only). */
tq_status tq_packed_layout(tq_format f, int head_dim, int64_t n_vec, tq_planes_desc *out);

/* Encode per-token K and V rows ([QPQ] Stage 1 and Stage 2; K/V asymmetric).
 * k_f16, v_f16: device, [n_vec, d] fp16 (either may be NULL to skip it);
 * k_packed, v_packed: device, tq_packed_layout(kf|vf, d, n_vec).total_bytes
 * each, 256-byte aligned.  Formats: MSE, PROD or Q8 for either tensor. */
tq_status tq_encode_kv(const tq_ctx *ctx, const void *k_f16, const void *v_f16, int64_t n_vec,
                       tq_format kf, tq_format vf, void *k_packed, void *v_packed, void *stream);

/* Append the new token of each sequence to a packed cache during decode: the
 * per-token encode of [QPQ] Stage 1 and Stage 2 applied to one row per
 * (sequence, KV head), written in place into a cache laid out for
 * n_cache = B*Hkv*T_cap rows in [B, Hkv, T_cap] order (the layout that
 * tq_attn_decode reads with T = T_cap).
 * k_new_f16, v_new_f16: device [B, Hkv, d] fp16 (either may be NULL to skip
 * it); pos: device int32 [B], the cache position of sequence b's new token;
 * k_packed, v_packed: device, tq_packed_layout(kf|vf, d, n_cache) each,
 * 256-byte aligned.  Row (b, h) is encoded exactly as tq_encode_kv encodes
 * it and lands in cache row (b*Hkv + h)*T_cap + pos[b]; a sequence whose pos
 * is outside [0, T_cap) gets nothing written, and every other row of the
 * cache is left untouched.  Order this call before a tq_attn_decode that
 * should see the new token (same stream, seq_lens[b] = pos[b] + 1). */
tq_status tq_append_kv(const tq_ctx *ctx, const void *k_new_f16, const void *v_new_f16, int B, int Hkv,
                       int T_cap, const int32_t *pos, tq_format kf, tq_format vf, void *k_packed,
                       void *v_packed, void *stream);

/* Reconstruct fp16 rows from one packed tensor: MSE -> n R^T c[idx]/sqrt(d);
 * PROD -> R^T (n c[idx]/sqrt(d) + sqrt(pi/2)/m * gamma * S^T (2 bit - 1));
 * Q8 -> int8 * block scale.  packed: device; out_f16: device [n_vec, d]. */
tq_status tq_decode_kv(const tq_ctx *ctx, const void *packed, tq_format f, int64_t n_vec,
                       void *out_f16, void *stream);

/* Single-token decode attention over a packed cache ([CXT] 1.1, [YYL] item 4,
 * [CXT] 3.3).  q_f16: device [B, Hq, d]; k_packed / v_packed: device, one
 * packed tensor each over n_vec = B*Hkv*T rows in [B, Hkv, T] order.
 * seq_lens: device int32 [B] (values clamped to [0, T]) or NULL (= T).
 * Scores <q, k_hat>/sqrt(d) with q head h reading kv head h/(Hq/Hkv); full
 * softmax over each sequence; V rows whose normalised weight is below tau
 * are skipped and not renormalised (tau = 0 keeps every row).
 * out_f32: device [B, Hq, d].  workspace: device, at least
 * tq_attn_workspace_bytes(...) bytes, 256-byte aligned, zero-filled once
 * before its first use.  Its first 68 KiB hold barrier counters and flags
 * that every call leaves at zero; the rest is clobbered.  So one workspace serves calls
 * of any shape, format and Tq in turn without clearing it again (sized for
 * the largest).  K: MSE, PROD or Q8; V: MSE or Q8.
 * out_f32 is written as a sum of per-chunk shares added with fp32 atomics,
 * so repeated calls may differ in the last bits.  Calls that share one
 * workspace or one output must be ordered on one stream. */
tq_status tq_attn_decode(const tq_ctx *ctx, const void *q_f16, const void *k_packed,
                         const void *v_packed, tq_format kf, tq_format vf, int B, int Hq, int Hkv,
                         int T, const int32_t *seq_lens, float sparse_v_tau, float *out_f32,
                         void *workspace, size_t ws_bytes, void *stream);
/* tq_attn_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and conventions as
 * tq_attn_decode; the workspace is a library-owned device array of 8 MiB per
 * GPU (held until the process ends), and this call allocates nothing.  The
 * ctx's device must be current (TQ_ERR_INVALID_ARG otherwise).  A shape whose
 * workspace (tq_attn_workspace_bytes) exceeds 8 MiB returns
 * TQ_ERR_WORKSPACE without launching.  Calls on one GPU share the array:
 * calls that overlap in time on that GPU (different streams, no ordering)
 * race and must not be issued; calls ordered on one stream are safe. */
tq_status tq_attn_decode_noalloc(const tq_ctx *ctx, const void *q_f16, const void *k_packed,
                                 const void *v_packed, tq_format kf, tq_format vf, int B, int Hq, int Hkv,
                                 int T, const int32_t *seq_lens, float sparse_v_tau, float *out_f32,
                                 void *stream);
/* One decode step with the append of its new token ([CXT] 3.4: every step
 * writes the new K/V rows into the quantised cache; [CXT] 1.1, [YYL] item 4,
 * [CXT] 3.3 as tq_attn_decode): the new K and V of every (sequence, kv head)
 * are encoded into the caches at position pos[b], then every query head of
 * sequence b attends over its first pos[b] + 1 cached tokens, the new one
 * included.  Same result as tq_append_kv(k_new, v_new, pos) followed by
 * tq_attn_decode with seq_lens[b] = pos[b] + 1 and T = T_cap: identical cache
 * bytes, outputs equal up to the last bits.  A sequence whose pos[b] lies
 * outside [0, T_cap) gets nothing written and attends over its first
 * clamp(pos[b] + 1, 0, T_cap) tokens.
 * q_f16: device [B, Hq, d]; k_new_f16, v_new_f16: device [B, Hkv, d] fp16,
 * 16-byte aligned; pos: device int32 [B]; k_packed, v_packed: device, the
 * [B, Hkv, T_cap] caches (tq_packed_layout over B*Hkv*T_cap rows), read and
 * written; out_f32, workspace (tq_attn_workspace_bytes(B, Hq, Hkv, T_cap,
 * kf, vf)), tau and ordering as tq_attn_decode.  TurboQuant K (PROD) with
 * codebook V (MSE) is encoded inside the attention launch, by one block of
 * each row; other formats take one append launch ahead of it. */
tq_status tq_attn_decode_append(const tq_ctx *ctx, const void *q_f16, const void *k_new_f16,
                                const void *v_new_f16, const int32_t *pos, void *k_packed, void *v_packed,
                                tq_format kf, tq_format vf, int B, int Hq, int Hkv, int T_cap,
                                float sparse_v_tau, float *out_f32, void *workspace, size_t ws_bytes,
                                void *stream);
/* Workspace of tq_attn_decode (0 for an invalid shape, or when B*Hkv > 65535). */
size_t tq_attn_workspace_bytes(int B, int Hq, int Hkv, int T, tq_format kf, tq_format vf);

/* Causal prefill attention over a packed cache: the last Tq positions of each
 * sequence attend to the cache, each exactly as the decode step above does
 * with its own prefix ([CXT] 1.1 scores and softmax, [YYL] item 4 and
 * [CXT] 3.3 sparse V, per query and head).  The Tq new tokens must already be
 * in the cache (tq_encode_kv or tq_append_kv).
 * q_f16: device [B, Tq, Hq, d]; out_f32: device [B, Tq, Hq, d].  With
 * L_b = seq_lens[b] clamped to [0, T] (or T when seq_lens is NULL), query i
 * of sequence b sits at position L_b - Tq + i and sees the first
 * L_b - Tq + i + 1 tokens; a query that sees none gets a zero row.
 * Other arguments, formats, ownership and the last-bit nondeterminism of
 * the fp32 atomics as for tq_attn_decode; workspace:
 * tq_attn_prefill_workspace_bytes(...) bytes, 256-byte aligned.  Tq = 1 is
 * exactly tq_attn_decode.  Up to B*Tq*Hkv = 65535, queries are taken in
 * groups of up to 8 / (Hq / Hkv) per kv head; the queries of a group are
 * stacked as extra MFMA rows and share every K and V load of their scores
 * and values passes, while separate groups each read the prefix again.
 * Past that, calls with TurboQuant or codebook K and codebook V run the
 * prompt-scale kernels (64 (query, head) rows per block share each K tile;
 * any B*Hkv <= 65535); other formats return TQ_ERR_UNSUPPORTED there. */
tq_status tq_attn_prefill(const tq_ctx *ctx, const void *q_f16, const void *k_packed,
                          const void *v_packed, tq_format kf, tq_format vf, int B, int Hq, int Hkv,
                          int T, int Tq, const int32_t *seq_lens, float sparse_v_tau, float *out_f32,
                          void *workspace, size_t ws_bytes, void *stream);
size_t tq_attn_prefill_workspace_bytes(int B, int Hq, int Hkv, int T, int Tq, tq_format kf, tq_format vf);

/* Per-group asymmetric min-max quantisation ([MAC] 2.1): for each group of
 * group_size consecutive elements, fp16 scale = (max-min)/(2^bits-1) (from the
 * exact fp16 extremes, rounded once), fp16 zero = min, code =
 * clamp(rint((x - zero)/scale), 0, 2^bits-1) in float32 (0 when scale = 0).
 * x_f16: device [n]; codes: device, n*bits/8 bytes, one LSB-first bitstream;
 * scale_f16, zero_f16: device [n/group_size].  This build: group_size 64,
 * bits 2..4, n a multiple of group_size. */
tq_status tq_minmax_quant(const void *x_f16, int64_t n, int group_size, int bits, void *codes,
                          void *scale_f16, void *zero_f16, void *stream);
/* x_hat = code*scale + zero (float32, rounded to fp16). */
tq_status tq_minmax_dequant(const void *codes, const void *scale_f16, const void *zero_f16,
                            int64_t n, int group_size, int bits, void *out_f16, void *stream);

const char *tq_status_str(tq_status s);

#ifdef __cplusplus
}
#endif
#endif /* TURBOKV_H */
