// Stand-ins for the HIP kernel launchers, so that the host half of libturbokv
// (argument checks, plane layouts, table generation) links into a CPU-only
// program built with AddressSanitizer and UBSan.  Every stub reports a
// failure: the host checks must decide each call before any launch.
#include "../../kv_cache_quantization_encode_amd/csrc/internal.h"

namespace tq {
int launch_encode(const DevTables *, const void *, int64_t, tq_format, void *, const tq_planes_desc &, void *) {
    return 1;
}
int launch_encode_pair(const DevTables *, const void *, const void *, int64_t, tq_format, tq_format, void *, void *,
                       const tq_planes_desc &, const tq_planes_desc &, void *) {
    return 1;
}
int launch_append(const DevTables *, const void *, int, int, int, const int32_t *, tq_format, void *,
                  const tq_planes_desc &, void *) {
    return 1;
}
int launch_append_kv(const DevTables *, const void *, const void *, int, int, int, const int32_t *, tq_format,
                     tq_format, void *, void *, const tq_planes_desc &, const tq_planes_desc &, void *) {
    return 1;
}
int launch_decode(const DevTables *, const void *, tq_format, int64_t, const tq_planes_desc &, void *, void *) {
    return 1;
}
int launch_attn(const DevTables *, const void *, const void *, const void *, tq_format, tq_format,
                const tq_planes_desc &, const tq_planes_desc &, int, int, int, int, int, const int32_t *, float,
                float *, void *, const AttnPlan &, int, const AttnAppend *, void *) {
    return 1;
}
int launch_attn_fused(const AttnArgs &, tq_format, tq_format, void *) { return 1; }
int launch_attn_generic(const AttnArgs &, tq_format, tq_format, void *) { return 1; }
int launch_attn_prefill(const AttnArgs &, tq_format, tq_format, void *) { return 1; }
int launch_attn_fused4(const AttnArgs &, tq_format, tq_format, void *) { return 1; }
// no device: the single-launch attention paths are never planned
int fused_capacity() { return 0; }
int fused4_capacity() { return 0; }
int scratch_prepare(int) { return 1; }
void *scratch_device_ptr(int) { return nullptr; }
int launch_minmax_quant(const void *, int64_t, int, void *, void *, void *, void *) { return 1; }
int launch_minmax_dequant(const void *, const void *, const void *, int64_t, int, void *, void *) { return 1; }
}  // namespace tq
