// CPU-only exercise of libturbokv's host code under AddressSanitizer and
// UBSan: table generation for several sizes and seeds, the device-table
// builder, plane layouts over all formats and sizes, and the argument checks
// of every entry point with fake (never dereferenced) addresses.  Exits 0
// when every expectation holds; the sanitizers abort on any memory error or
// undefined behaviour.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../kv_cache_quantization_encode_amd/csrc/internal.h"

static int failures = 0;
#define EXPECT(c)                                                        \
    do {                                                                 \
        if (!(c)) {                                                      \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

int main() {
    using namespace tq;
    // tables: several head sizes, projection sizes and seeds
    const int dims[][2] = {{2, 1}, {8, 8}, {64, 32}, {128, 128}, {256, 256}, {128, 4096}};
    for (auto &dm : dims)
        for (uint64_t seed : {0ull, 42ull, ~0ull}) {
            std::vector<double> lv(64), bd(64);
            std::vector<float> sg(dm[0]);
            std::vector<uint16_t> S(size_t(dm[0]) * dm[1]);
            EXPECT(tq_host_tables(dm[0], dm[1], seed, lv.data(), bd.data(), sg.data(), S.data()) == TQ_OK);
            for (int b = 1; b <= 4; ++b) {
                const int L = 1 << b;
                for (int k = 0; k + 1 < L; ++k) {
                    EXPECT(lv[16 * (b - 1) + k] < lv[16 * (b - 1) + k + 1]);
                    EXPECT(std::fabs(bd[16 * (b - 1) + k] -
                                     0.5 * (lv[16 * (b - 1) + k] + lv[16 * (b - 1) + k + 1])) < 1e-12);
                }
            }
            for (float x : sg) EXPECT(x == 1.0f || x == -1.0f);
        }
    EXPECT(tq_host_tables(100, 8, 1, nullptr, nullptr, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_host_tables(128, 0, 1, nullptr, nullptr, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
    // the device-table builder on the host
    DevTables *t = new DevTables;
    EXPECT(build_device_tables(128, 128, 42, t));
    for (int b = 1; b <= 4; ++b)
        for (int j = 0; j < kBuckets; ++j) EXPECT(t->qlut[b - 1][j].base < (1u << b));
    delete t;
    // plane layouts
    const tq_format fmts[] = {{TQ_KIND_MSE, 1}, {TQ_KIND_MSE, 2}, {TQ_KIND_MSE, 3}, {TQ_KIND_MSE, 4},
                              {TQ_KIND_PROD, 1}, {TQ_KIND_PROD, 2}, {TQ_KIND_PROD, 3}, {TQ_KIND_Q8, 8}};
    for (const tq_format &f : fmts)
        for (int64_t n : {int64_t(0), int64_t(1), int64_t(17), int64_t(262144), kMaxRows}) {
            tq_planes_desc d{};
            EXPECT(tq_packed_layout(f, 128, n, &d) == TQ_OK);
            EXPECT(d.total_bytes >= d.idx_bytes + d.sign_bytes + d.norm_bytes);
            EXPECT(d.idx_offset % 256 == 0 && d.sign_offset % 256 == 0 && d.norm_offset % 256 == 0);
        }
    tq_planes_desc d{};
    EXPECT(tq_packed_layout({TQ_KIND_PROD, 4}, 128, 8, &d) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_packed_layout({7, 3}, 128, 8, &d) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_packed_layout({TQ_KIND_MSE, 2}, 128, 8, nullptr) == TQ_ERR_INVALID_ARG);
    // entry points: every call is decided on the host (the stub launchers
    // would report TQ_ERR_HIP if a launch were attempted)
    tq_ctx fake{128, 128, 42, 0, nullptr};
    void *A = reinterpret_cast<void *>(uintptr_t(1) << 20);
    const tq_format k3{TQ_KIND_PROD, 3}, v2{TQ_KIND_MSE, 2}, bad{9, 9};
    EXPECT(tq_encode_kv(&fake, A, A, 0, k3, v2, A, A, nullptr) == TQ_OK);
    EXPECT(tq_encode_kv(&fake, A, A, -1, k3, v2, A, A, nullptr) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_encode_kv(&fake, A, A, kMaxRows + 1, k3, v2, A, A, nullptr) == TQ_ERR_UNSUPPORTED);
    EXPECT(tq_encode_kv(&fake, A, A, 16, bad, v2, A, A, nullptr) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_encode_kv(&fake, A, A, 16, k3, v2, A, A, nullptr) == TQ_ERR_HIP);  // reached the launcher
    EXPECT(tq_append_kv(&fake, A, A, 2, 8, 64, nullptr, k3, v2, A, A, nullptr) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_append_kv(&fake, A, A, 1 << 20, 8, 1 << 20, static_cast<const int32_t *>(A), k3, v2, A, A,
                        nullptr) == TQ_ERR_UNSUPPORTED);
    EXPECT(tq_decode_kv(&fake, A, k3, 0, A, nullptr) == TQ_OK);
    EXPECT(tq_decode_kv(&fake, A, bad, 4, A, nullptr) == TQ_ERR_INVALID_ARG);
    const size_t ws = tq_attn_workspace_bytes(1, 32, 8, 32768, k3, v2);
    EXPECT(ws > 0);
    EXPECT(tq_attn_workspace_bytes(1, 30, 8, 64, k3, v2) == 0);
    EXPECT(tq_attn_workspace_bytes(65536, 8, 8, 64, k3, v2) == 0);
    float *o = static_cast<float *>(A);
    EXPECT(tq_attn_decode(&fake, A, A, A, k3, v2, 1, 32, 8, 32768, nullptr, 1e-6f, o, A, ws - 1, nullptr) ==
           TQ_ERR_WORKSPACE);
    EXPECT(tq_attn_decode(&fake, A, A, A, k3, v2, 1, 32, 8, 32768, nullptr, NAN, o, A, ws, nullptr) ==
           TQ_ERR_INVALID_ARG);
    EXPECT(tq_attn_decode(&fake, A, A, A, k3, v2, 1, 24, 8, 32768, nullptr, 1e-6f, o, A, ws, nullptr) ==
           TQ_ERR_UNSUPPORTED);
    EXPECT(tq_attn_decode(&fake, A, A, A, k3, v2, 1, 32, 8, 32768, nullptr, 1e-6f, o, A, ws, nullptr) ==
           TQ_ERR_HIP);
    const int32_t *P = static_cast<const int32_t *>(A);
    EXPECT(tq_attn_decode_append(&fake, A, A, A, P, A, A, k3, v2, 1, 32, 8, 32768, 1e-6f, o, A, ws, nullptr) ==
           TQ_ERR_HIP);
    EXPECT(tq_attn_decode_append(&fake, A, A, A, nullptr, A, A, k3, v2, 1, 32, 8, 32768, 1e-6f, o, A, ws,
                                 nullptr) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_attn_decode_append(&fake, A, nullptr, A, P, A, A, k3, v2, 1, 32, 8, 32768, 1e-6f, o, A, ws,
                                 nullptr) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_attn_decode_append(&fake, A, A, A, P, A, A, k3, v2, 1, 32, 8, 32768, 1e-6f, o, A, 1024,
                                 nullptr) == TQ_ERR_WORKSPACE);
    EXPECT(tq_attn_decode_append(&fake, A, A, A, P, A, A, k3, {TQ_KIND_PROD, 2}, 1, 32, 8, 32768, 1e-6f, o, A, ws,
                                 nullptr) == TQ_ERR_UNSUPPORTED);
    // q8 caches take the separate append launch (the stub fails it first)
    const tq_format q8{TQ_KIND_Q8, 8};
    const size_t qws = tq_attn_workspace_bytes(1, 32, 8, 4096, q8, q8);
    EXPECT(tq_attn_decode_append(&fake, A, A, A, P, A, A, q8, q8, 1, 32, 8, 4096, 1e-6f, o, A, qws, nullptr) ==
           TQ_ERR_HIP);
    const size_t pws = tq_attn_prefill_workspace_bytes(2, 32, 8, 4096, 16, k3, v2);
    EXPECT(pws > 0);
    EXPECT(tq_attn_prefill(&fake, A, A, A, k3, v2, 2, 32, 8, 4096, 16, nullptr, 1e-6f, o, A, pws, nullptr) ==
           TQ_ERR_HIP);
    EXPECT(tq_attn_prefill(&fake, A, A, A, k3, v2, 2, 32, 8, 4096, 0, nullptr, 1e-6f, o, A, pws, nullptr) ==
           TQ_ERR_INVALID_ARG);
    EXPECT(tq_minmax_quant(A, 0, 64, 3, A, A, A, nullptr) == TQ_OK);
    EXPECT(tq_minmax_quant(A, 65, 64, 3, A, A, A, nullptr) == TQ_ERR_INVALID_ARG);
    EXPECT(tq_minmax_dequant(A, A, A, 64, 64, 3, A, nullptr) == TQ_ERR_HIP);
    for (int s = -6; s <= 0; ++s) EXPECT(tq_status_str(tq_status(s)) != nullptr);
    std::printf("host checks: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
