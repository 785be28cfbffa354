// Launchers of the fused head-dim-64 SSD kernel (see ssd_fused.hpp) and of
// the CB pass that precedes it.
#include "ssd_bf16.hpp"
#include "ssd_fused.hpp"

namespace cls {

// S2a for the fused kernel: one workgroup (4 waves) per (batch, chunk, group).
// Writes CB[i][j] = sum_s C[i][s] B[j][s] for the 32-token blocks with
// block(j) <= block(i) (the only ones the fused kernel reads) and the
// token-contiguous copy B^T[s][t].  C and B rows are read through buffer loads
// whose range ends at the chunk's last real token, so padded rows read as
// zeros.  Wave w takes the 16-row tiles k and NIT-1-k (k = w, w + 4, ..), which
// gives every wave the same number of tiles of the triangle.
template <int TT, int S>
__global__ __launch_bounds__(kBfThreads) void ssd_cbt_kernel(SsdBf16Params p) {
    constexpr int KS = S / 32;
    constexpr int NIT = TT / 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int64_t bcg = blockIdx.x;
    const int g = int(bcg % p.G);
    const int64_t c = (bcg / p.G) % p.nchunks;
    const int64_t b = bcg / (int64_t(p.G) * p.nchunks);
    const int64_t tok0 = c * p.chunk;
    const int n = int((p.L - tok0 < p.chunk) ? (p.L - tok0) : p.chunk);
    const uint32_t rowb = uint32_t(p.G * S * 2);  // bytes between consecutive tokens
    const int64_t base = ((b * p.L + tok0) * p.G + g) * S;
    const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.C + base), 0, int(uint32_t(n) * rowb),
                                                      0x00020000);
    const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.B + base), 0, int(uint32_t(n) * rowb),
                                                      0x00020000);
    uint16_t* out = p.cb + bcg * (TT * TT);
    auto load_rows = [&](const __amdgpu_buffer_rsrc_t& r, int row, u32x4 (&dst)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            dst[ks] = __builtin_amdgcn_raw_buffer_load_b128(r, int(uint32_t(row) * rowb + 64 * ks + 16 * kg), 0, 0);
    };
    for (int k = wave; k < NIT / 2; k += 4) {
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int it = side ? NIT - 1 - k : k;
            const int jmax = 2 * (it >> 1) + 1;  // last 16-column tile of the blocks <= block(it)
            u32x4 cf[KS], bcur[KS], bnxt[KS];
            load_rows(rc, 16 * it + l16, cf);
            load_rows(rb, l16, bcur);
            for (int jt = 0; jt <= jmax; ++jt) {
                if (jt < jmax) load_rows(rb, 16 * (jt + 1) + l16, bnxt);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(bcur[ks], cf[ks], acc);
                // lane holds CB[i][16 jt + 4 kg + r], r = 0..3
                u32x2 v;
                v[0] = pack_bf16x2(acc[0], acc[1]);
                v[1] = pack_bf16x2(acc[2], acc[3]);
                *reinterpret_cast<u32x2*>(out + (16 * it + l16) * TT + 16 * jt + 4 * kg) = v;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) bcur[ks] = bnxt[ks];
            }
        }
    }
    // B^T: item u covers tokens 8 tg .. 8 tg + 7 and states 8 sg .. 8 sg + 7,
    // moved as eight 16-byte rows and transposed in registers
    uint16_t* bt = p.bt + bcg * (int64_t(S) * TT);
    for (int u = tid; u < (TT / 8) * (S / 8); u += kBfThreads) {
        const int tg = u / (S / 8), sg = u % (S / 8);
        u32x4 rows[8], cols[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            rows[r] = __builtin_amdgcn_raw_buffer_load_b128(rb, int(uint32_t(8 * tg + r) * rowb + 16 * sg), 0, 0);
        transpose8x8_b16(rows, cols);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<u32x4*>(bt + (8 * sg + cc) * TT + 8 * tg) = cols[cc];
    }
}

template <int TT, int S>
static int launch_fused_tpl(const SsdBf16Params& cbp, const SsdFusedParams& fp, hipStream_t stream,
                            hipEvent_t* ev) {
    using Lay = FuLayout<TT, S>;
    using LayA = FuLayout<TT, S, true>;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_fused_kernel<TT, S>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, Lay::BYTES) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_fused_agg_kernel<TT, S>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LayA::BYTES) != hipSuccess)
            return -7;
        attr_set = true;
    }
    const int nst = fp.nsegs * (fp.nchains - fp.nwhole);              // segments
    const int npieces = (fp.nchains - fp.nwhole) * (fp.nsegs - 1) * fp.agg_d;  // aggregate pieces
    const dim3 gcb{uint32_t(cbp.batch * cbp.nchunks * cbp.G), 1u, 1u};
    const dim3 bcb{uint32_t(kBfThreads), 1u, 1u};
    const dim3 bmain{uint32_t(kFuThreads), 1u, 1u};
    if (ev) (void)hipEventRecord(ev[0], stream);
    hipLaunchKernelGGL((ssd_cbt_kernel<TT, S>), gcb, bcb, 0, stream, cbp);
    if (ev) (void)hipEventRecord(ev[1], stream);
    if (npieces > 0) {
        const dim3 gagg{uint32_t(npieces), 1u, 1u};
        hipLaunchKernelGGL((ssd_fused_agg_kernel<TT, S>), gagg, bmain, LayA::BYTES, stream, fp);
    }
    if (ev) (void)hipEventRecord(ev[2], stream);
    const dim3 gout{uint32_t(fp.nwhole + nst), 1u, 1u};
    hipLaunchKernelGGL((ssd_fused_kernel<TT, S>), gout, bmain, Lay::BYTES, stream, fp);
    if (ev) (void)hipEventRecord(ev[3], stream);
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

int ssd_fused_launch(int TT, int S, const SsdBf16Params& cbp, const SsdFusedParams& fp, hipStream_t stream,
                     hipEvent_t* ev) {
    switch (TT * 1000 + S) {
        case 32064: return launch_fused_tpl<32, 64>(cbp, fp, stream, ev);
        case 32128: return launch_fused_tpl<32, 128>(cbp, fp, stream, ev);
        case 64064: return launch_fused_tpl<64, 64>(cbp, fp, stream, ev);
        case 64128: return launch_fused_tpl<64, 128>(cbp, fp, stream, ev);
        case 128064: return launch_fused_tpl<128, 64>(cbp, fp, stream, ev);
        case 128128: return launch_fused_tpl<128, 128>(cbp, fp, stream, ev);
        default: return -8;
    }
}

}  // namespace cls
