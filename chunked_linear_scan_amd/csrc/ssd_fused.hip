// Launchers of the fused head-dim-64 SSD kernel (see ssd_fused.hpp) and of
// the CB pass that precedes it.
#include "ssd_bf16.hpp"
#include "ssd_fused.hpp"

namespace cls {

template <int TT, int S>
static int launch_fused_tpl(const SsdBf16Params& cbp, const SsdFusedParams& fp, int ntiles,
                            hipStream_t stream, hipEvent_t* ev) {
    using Lay = FuLayout<TT, S>;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_fused_kernel<TT, S>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, Lay::BYTES) != hipSuccess)
            return -7;
        attr_set = true;
    }
    const dim3 gcb{cb_grid<TT>(cbp), 1u, 1u};
    const dim3 bcb{uint32_t(kBfThreads), 1u, 1u};
    if (ev) hipEventRecord(ev[0], stream);
    hipLaunchKernelGGL((ssd_cb_kernel<TT, S>), gcb, bcb, 0, stream, cbp);
    if (ev) hipEventRecord(ev[1], stream);
    const dim3 gmain{uint32_t(ntiles), 1u, 1u};
    const dim3 bmain{uint32_t(kFuThreads), 1u, 1u};
    hipLaunchKernelGGL((ssd_fused_kernel<TT, S>), gmain, bmain, Lay::BYTES, stream, fp);
    if (ev) hipEventRecord(ev[2], stream);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

size_t ssd_fused_lds_bytes(int TT, int S) {
    switch (TT * 1000 + S) {
        case 32064: return FuLayout<32, 64>::BYTES;
        case 32128: return FuLayout<32, 128>::BYTES;
        case 64064: return FuLayout<64, 64>::BYTES;
        case 64128: return FuLayout<64, 128>::BYTES;
        case 128064: return FuLayout<128, 64>::BYTES;
        case 128128: return FuLayout<128, 128>::BYTES;
        default: return 0;
    }
}

int ssd_fused_state_floats(int S) { return kFuP * S; }

int ssd_fused_launch(int TT, int S, const SsdBf16Params& cbp, const SsdFusedParams& fp, int ntiles,
                     hipStream_t stream, hipEvent_t* ev) {
    switch (TT * 1000 + S) {
        case 32064: return launch_fused_tpl<32, 64>(cbp, fp, ntiles, stream, ev);
        case 32128: return launch_fused_tpl<32, 128>(cbp, fp, ntiles, stream, ev);
        case 64064: return launch_fused_tpl<64, 64>(cbp, fp, ntiles, stream, ev);
        case 64128: return launch_fused_tpl<64, 128>(cbp, fp, ntiles, stream, ev);
        case 128064: return launch_fused_tpl<128, 64>(cbp, fp, ntiles, stream, ev);
        case 128128: return launch_fused_tpl<128, 128>(cbp, fp, ntiles, stream, ev);
        default: return -8;
    }
}

}  // namespace cls
