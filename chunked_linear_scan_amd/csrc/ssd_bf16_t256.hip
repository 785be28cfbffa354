// Instantiations of the bf16 SSD kernels for 256-token tiles.
#include "ssd_bf16.hpp"

namespace cls {

template <int P, int S>
static int run(const SsdBf16Params& prm, hipStream_t stream) {
    if constexpr (ssd_bf16_lds_fits(256, P, S)) {
        return launch_ssd_bf16_tpl<256, P, S>(prm, stream);
    } else {
        return -8;
    }
}

int ssd_bf16_launch_t256(int P, int S, const SsdBf16Params& prm, hipStream_t stream) {
#define CLS_CASE(PP, SS) \
    if (P == PP && S == SS) return run<PP, SS>(prm, stream);
    CLS_CASE(16, 32) CLS_CASE(16, 64) CLS_CASE(16, 128) CLS_CASE(16, 256)
    CLS_CASE(32, 32) CLS_CASE(32, 64) CLS_CASE(32, 128) CLS_CASE(32, 256)
    CLS_CASE(64, 32) CLS_CASE(64, 64) CLS_CASE(64, 128) CLS_CASE(64, 256)
    CLS_CASE(128, 32) CLS_CASE(128, 64) CLS_CASE(128, 128) CLS_CASE(128, 256)
#undef CLS_CASE
    return -8;
}

}  // namespace cls
