// Prefill GEMM (M > 8): placeholder until the MFMA tile kernel lands; larger
// M is served by repeated decode passes.
#include "common.h"

namespace nvfp4 {

int make_prefill_config(int max_M, int K, int N, PrefillConfig* out) {
    (void)max_M; (void)K; (void)N;
    out->enabled = 0;
    out->ws_bytes = 0;
    return NVFP4_OK;
}

int launch_prefill(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                   float ts, const uint16_t* act, void* out, void* ws, hipStream_t s) {
    (void)p; (void)M; (void)codes; (void)scales; (void)ts; (void)act; (void)out; (void)ws; (void)s;
    return set_error(NVFP4_EUNSUPPORTED, "prefill kernel not built");
}

}  // namespace nvfp4
