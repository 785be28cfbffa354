// SSD validation, workspace sizing and dispatch to the fp32 or bf16 path.
#include "../../include/chunked_linear_scan.h"
#include "launch.hpp"
#include "ssd_kernels.hpp"

namespace cls {

int ssd_bf16_launch_t32(int P, int S, const SsdBf16Params& prm, hipStream_t stream);
int ssd_bf16_launch_t64(int P, int S, const SsdBf16Params& prm, hipStream_t stream);
int ssd_bf16_launch_t128(int P, int S, const SsdBf16Params& prm, hipStream_t stream);
int ssd_bf16_launch_t256(int P, int S, const SsdBf16Params& prm, hipStream_t stream);

bool ssd_bf16_supported(int TT, int P, int S) {
    const bool p_ok = P == 16 || P == 32 || P == 64 || P == 128;
    const bool s_ok = S == 32 || S == 64 || S == 128 || S == 256;
    return p_ok && s_ok && ssd_bf16_lds_fits(TT, P, S);
}

int ssd_bf16_launch(int TT, int P, int S, const SsdBf16Params& prm, hipStream_t stream) {
    switch (TT) {
        case 32: return ssd_bf16_launch_t32(P, S, prm, stream);
        case 64: return ssd_bf16_launch_t64(P, S, prm, stream);
        case 128: return ssd_bf16_launch_t128(P, S, prm, stream);
        case 256: return ssd_bf16_launch_t256(P, S, prm, stream);
        default: return SSD_ERR_CHUNK;
    }
}

}  // namespace cls

namespace {

bool valid_chunk(int64_t c) { return c == 16 || c == 32 || c == 64 || c == 128 || c == 256; }

int64_t nchunks(const SsdShape& s) { return (s.seqlen + s.chunk - 1) / s.chunk; }

}  // namespace

extern "C" int cls_ssd_check(const SsdShape& s) {
    if (s.batch <= 0 || s.seqlen <= 0 || s.nheads <= 0 || s.headdim <= 0 || s.dstate <= 0 ||
        s.ngroups <= 0)
        return SSD_ERR_SHAPE;
    if (s.nheads % s.ngroups != 0) return SSD_ERR_SHAPE;
    if (s.dtype != SSD_F32 && s.dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (!valid_chunk(s.chunk)) return SSD_ERR_CHUNK;
    // index arithmetic stays in 64 bits; grids are bounded by 2^31 workgroups
    if (s.batch * s.nheads > (int64_t(1) << 31) || s.seqlen > (int64_t(1) << 40)) return SSD_ERR_SHAPE;
    if (s.nheads > (int64_t(1) << 30) || s.headdim > 4096 || s.dstate > 4096) return SSD_ERR_SHAPE;
    if (s.dtype == SSD_F32) {
        if (s.headdim * s.dstate > 16384 || s.headdim % 4 != 0 || s.dstate % 4 != 0) return SSD_ERR_UNSUPPORTED;
        if (cls::ssd_f32_lds_bytes(int(s.headdim), int(s.dstate)) > 160 * 1024) return SSD_ERR_UNSUPPORTED;
    } else {
        const int TT = cls::bf16_tile_tokens(int(s.chunk));
        if (!cls::ssd_bf16_supported(TT, int(s.headdim), int(s.dstate))) return SSD_ERR_UNSUPPORTED;
        if (s.batch * nchunks(s) * s.ngroups > (int64_t(1) << 31)) return SSD_ERR_SHAPE;
    }
    return SSD_OK;
}

extern "C" size_t cls_ssd_workspace_bytes(const SsdShape& s) {
    if (s.dtype == SSD_F32) return 0;
    const int64_t TT = cls::bf16_tile_tokens(int(s.chunk));
    return size_t(s.batch) * size_t(nchunks(s)) * size_t(s.ngroups) * size_t(TT * TT) * 2 + 256;
}

extern "C" int cls_ssd_launch(const SsdShape& s, const SsdArgs& a, hipStream_t stream) {
    if (s.dtype == SSD_F32) {
        cls::SsdF32Params p{a.x, a.dt, a.A, a.B, a.C, a.D, a.h0, a.y, a.h_final, s.batch, s.seqlen,
                            int(s.nheads), int(s.headdim), int(s.dstate), int(s.ngroups), int(s.chunk)};
        return cls::ssd_f32_launch(p, stream) == 0 ? SSD_OK : SSD_ERR_HIP;
    }
    cls::SsdBf16Params p{};
    p.x = static_cast<const uint16_t*>(a.x);
    p.dt = a.dt;
    p.A = a.A;
    p.B = static_cast<const uint16_t*>(a.B);
    p.C = static_cast<const uint16_t*>(a.C);
    p.D = a.D;
    p.h0 = a.h0;
    p.y = static_cast<uint16_t*>(a.y);
    p.h_final = a.h_final;
    p.cb = reinterpret_cast<uint16_t*>(static_cast<char*>(a.workspace) + 256);
    p.batch = s.batch;
    p.L = s.seqlen;
    p.H = int(s.nheads);
    p.G = int(s.ngroups);
    p.chunk = int(s.chunk);
    p.nchunks = int(nchunks(s));
    const int TT = cls::bf16_tile_tokens(int(s.chunk));
    const int st = cls::ssd_bf16_launch(TT, int(s.headdim), int(s.dstate), p, stream);
    if (st == -8) return SSD_ERR_UNSUPPORTED;
    return st == 0 ? SSD_OK : SSD_ERR_HIP;
}
