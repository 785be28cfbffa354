// Launchers of the fused SSD kernels (see ssd_fused.hpp) and of
// the CB pass that precedes it.
#include "device_once.hpp"
#include "ssd_bf16.hpp"
#include "ssd_fused.hpp"

namespace cls {

// S2a for the fused kernel: one workgroup (4 waves) per (batch, chunk, group),
// then one per (batch, chunk) that rewrites dt head-major (cbt_dt_transpose).
// Writes CB[i][j] = sum_s C[i][s] B[j][s] for the 32-token blocks with
// block(j) <= block(i) (the only ones the fused kernel reads), B^T[s][t], and
// (unless p.cf is null) a copy of the chunk's C rows, all three fragment-major: the MFMA operand
// fragment (16-row tile m, 32-column block k) holds row 16 m + l of the
// operand, columns 32 k + 8 g .. + 7, in lane l + 16 g, and is stored as 64
// lanes x 16 bytes at fragment index m * (columns / 32) + k.  A wave of the
// fused kernel then loads a fragment as 1 KB in lane order (its cache
// accesses are a quarter of what a row-major tile needs).  The chunk's B rows are staged in LDS once
// (every load issued at once, so the workgroup waits out one memory latency);
// each wave loads the C rows of its two 16-row tiles k and NIT-1-k straight
// into registers, which gives every wave the same share of the triangle.  C
// and B rows are read through buffer loads whose range ends at the chunk's
// last real token, so padded rows read as zeros.
template <int TT, int S>
struct CbtLayout {
    static constexpr int BP = S + 8;                 // bf16 pitch of the staged B rows
    static constexpr int DP = 65;                    // float pitch of a staged dt row (64 heads)
    static constexpr int BYTES = TT * BP * 2 > TT * DP * 4 ? TT * BP * 2 : TT * DP * 4;
};

// The dt workgroups of the CB pass: dt of chunk c of batch row b, token-major
// [t][h] in the input, rewritten head-major and token-contiguous [h][t] (zero
// past the chunk's last real row), 64 heads at a time through LDS: the loads
// read token rows and the stores whole per-head runs, both coalesced.
template <int TT, int S>
__device__ __forceinline__ void cbt_dt_transpose(const SsdBf16Params& p, int64_t bc, unsigned char* smem) {
    using Lay = CbtLayout<TT, S>;
    constexpr int DP = Lay::DP;
    const int tid = threadIdx.x;
    const int64_t c = bc % p.nchunks, b = bc / p.nchunks;
    const int64_t tok0 = c * p.chunk;
    const int n = int((p.L - tok0 < p.chunk) ? (p.L - tok0) : p.chunk);
    float* st = reinterpret_cast<float*>(smem);
    for (int h0 = 0; h0 < p.H; h0 += 64) {
        constexpr int NL = TT * 64 / kBfThreads;
        float v[NL];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int idx = tid + kBfThreads * k, t = idx >> 6, hh = idx & 63;
            v[k] = (t < n && h0 + hh < p.H) ? p.dt[(b * p.L + tok0 + t) * p.H + h0 + hh] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int idx = tid + kBfThreads * k;
            st[(idx >> 6) * DP + (idx & 63)] = v[k];
        }
        __syncthreads();
        constexpr int NS = 64 * (TT / 4) / kBfThreads;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int idx = tid + kBfThreads * k, hh = idx / (TT / 4), t4 = 4 * (idx % (TT / 4));
            if (h0 + hh < p.H) {
                const f32x4 o = {st[t4 * DP + hh], st[(t4 + 1) * DP + hh], st[(t4 + 2) * DP + hh],
                                 st[(t4 + 3) * DP + hh]};
                *reinterpret_cast<f32x4*>(p.dtt + ((b * p.nchunks + c) * p.H + h0 + hh) * TT + t4) = o;
            }
        }
        __syncthreads();
    }
}

template <int TT, int S>
__global__ __launch_bounds__(kBfThreads) void ssd_cbt_kernel(SsdBf16Params p) {
    using Lay = CbtLayout<TT, S>;
    constexpr int KS = S / 32;
    constexpr int NIT = TT / 16;
    constexpr int CPR = S / 8;  // 16-byte pieces per row
    extern __shared__ __attribute__((aligned(16))) unsigned char cbt_sm[];
    // workgroups past the (batch, chunk, group) tiles rewrite dt, one per (batch, chunk)
    const int64_t ncbg = p.batch * p.nchunks * p.G;
    if (int64_t(blockIdx.x) >= ncbg) {
        cbt_dt_transpose<TT, S>(p, int64_t(blockIdx.x) - ncbg, cbt_sm);
        return;
    }
    uint16_t* sB = reinterpret_cast<uint16_t*>(cbt_sm);
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
    constexpr int NB = TT / 32;
    // B rows into LDS: piece q of the tile is row q / CPR, 16 bytes (q % CPR)
    constexpr int NBQ = TT * CPR / kBfThreads;
    u32x4 bq[NBQ];
#pragma unroll
    for (int k = 0; k < NBQ; ++k) {
        const int q = tid + kBfThreads * k;
        bq[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, int(uint32_t(q / CPR) * rowb + 16 * (q % CPR)), 0, 0);
    }
    // the C rows of this wave's tiles (MFMA B operand: row 16 it + l16, states 32 ks + 8 kg ..)
    const bool has_tiles = wave < NIT / 2;
    u32x4 cf[2][KS];
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        const int it = side ? NIT - 1 - wave : wave;
        const uint32_t row = has_tiles ? uint32_t(16 * it + l16) * rowb + 16 * kg : 0x7ffffff0u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            cf[side][ks] = __builtin_amdgcn_raw_buffer_load_b128(rc, int(row + (has_tiles ? 64 * ks : 0)), 0, 0);
    }
#pragma unroll
    for (int k = 0; k < NBQ; ++k) {
        const int q = tid + kBfThreads * k;
        *reinterpret_cast<u32x4*>(sB + (q / CPR) * Lay::BP + 8 * (q % CPR)) = bq[k];
    }
    // the C fragments, as loaded (rows past the chunk's end are zeros)
    if (has_tiles && p.cf) {
        uint16_t* cfo = p.cf + bcg * (int64_t(TT) * S);
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int it = side ? NIT - 1 - wave : wave;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                *reinterpret_cast<u32x4*>(cfo + ((it * KS + ks) * 64 + tid % 64) * 8) = cf[side][ks];
        }
    }
    __syncthreads();

    uint16_t* out = p.cb + bcg * (TT * TT);
    if (has_tiles) {
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int it = side ? NIT - 1 - wave : wave;
            const int ntj = 2 * (it >> 1) + 2;  // 16-column tiles of the blocks <= block(it), even
            const int i = 16 * it + l16;
            for (int jt = 0; jt < ntj; jt += 2) {
                // lane holds CB[i][16 jt' + 4 kg + r], r = 0..3, for jt' = jt, jt + 1
                f32x4 acc[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    acc[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const uint16_t* brow = sB + (16 * (jt + h2) + l16) * Lay::BP + 8 * kg;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        acc[h2] = mfma16x16x32(*reinterpret_cast<const u32x4*>(brow + 32 * ks), cf[side][ks], acc[h2]);
                }
                // lanes kg, kg ^ 1 trade halves: each lane then holds 8 consecutive
                // columns of row i, for one tile of the pair
                const uint32_t e0 = pack_bf16x2(acc[0][0], acc[0][1]), e1 = pack_bf16x2(acc[0][2], acc[0][3]);
                const uint32_t o0 = pack_bf16x2(acc[1][0], acc[1][1]), o1 = pack_bf16x2(acc[1][2], acc[1][3]);
                const auto s0 = __builtin_amdgcn_permlane16_swap(e0, o0, false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(e1, o1, false, false);
                const int j0 = 16 * (jt + (kg & 1)) + 8 * (kg >> 1);  // first of the lane's 8 columns
                *reinterpret_cast<u32x4*>(out + ((it * NB + (j0 >> 5)) * 64 + l16 + 16 * ((j0 >> 3) & 3)) * 8) =
                    u32x4{s0[0], s1[0], s0[1], s1[1]};
            }
        }
    }
    // B^T from the staged rows, one whole fragment per wave and store (1 KB in
    // lane order): fragment (16-state tile m, 32-token block k) gives lane
    // l16 + 16 kg state 16 m + l16 of tokens 32 k + 8 kg .. + 7, gathered by two
    // transposed LDS reads of 4 tokens each (lane l16 addresses token row
    // l16 / 4, states 4 (l16 % 4) .. + 3 of the 4 x 16 block)
    uint16_t* bt = p.bt + bcg * (int64_t(S) * TT);
    const unsigned char* sBb = reinterpret_cast<const unsigned char*>(sB);
    for (int f = wave; f < (S / 16) * NB; f += kBfThreads / 64) {
        const int m = f / NB, k = f % NB;
        const uint32_t o1 = uint32_t(((32 * k + 8 * kg + (l16 >> 2)) * Lay::BP + 16 * m + 4 * (l16 & 3)) * 2);
        *reinterpret_cast<u32x4*>(bt + (int64_t(f) * 64 + lane) * 8) = lds_tr_pair(sBb, o1, o1 + 8 * Lay::BP);
    }
}

// NT: the kernel instances with non-temporal x loads and y stores
template <int TT, int S, bool NT>
static int launch_fused_tpl(const SsdBf16Params& cbp, const SsdFusedParams& fp, hipStream_t stream,
                            hipEvent_t* ev) {
    using Lay = FuLayout<TT, S>;
    using LayA = FuLayout<TT, S, true>;
    static DeviceOnce attrs;
    const int ast = run_once_per_device(attrs, [] {
        return (hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_cbt_kernel<TT, S>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, CbtLayout<TT, S>::BYTES) != hipSuccess ||
                hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_fused_kernel<TT, S, NT>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, Lay::BYTES) != hipSuccess ||
                hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_fused_lb_kernel<TT, S, NT>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, Lay::BYTES) != hipSuccess ||
                hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_fused_agg_kernel<TT, S, NT>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, LayA::BYTES) != hipSuccess)
                   ? -7
                   : 0;
    });
    if (ast != 0) return ast;
    const int nst = fp.nsegs * (fp.nchains - fp.nwhole);              // segments
    // aggregate pieces (none when split chains pass state by look-back)
    const int npieces = fp.lookback ? 0 : (fp.nchains - fp.nwhole) * (fp.nsegs - 1) * fp.agg_d;
    const dim3 gcb{uint32_t(cbp.batch * cbp.nchunks * (cbp.G + 1)), 1u, 1u};  // + the dt workgroups
    const dim3 bcb{uint32_t(kBfThreads), 1u, 1u};
    const dim3 bmain{uint32_t(kFuThreads), 1u, 1u};
    if (ev) (void)hipEventRecord(ev[0], stream);
    constexpr unsigned cbt_lds = CbtLayout<TT, S>::BYTES;
    hipLaunchKernelGGL((ssd_cbt_kernel<TT, S>), gcb, bcb, cbt_lds, stream, cbp);
    if (ev) (void)hipEventRecord(ev[1], stream);
    if (npieces > 0) {
        const dim3 gagg{uint32_t(npieces), 1u, 1u};
        hipLaunchKernelGGL((ssd_fused_agg_kernel<TT, S, NT>), gagg, bmain, LayA::BYTES, stream, fp);
    }
    if (ev) (void)hipEventRecord(ev[2], stream);
    const dim3 gout{uint32_t(fp.nwhole + nst), 1u, 1u};
    const dim3 bout{uint32_t(kFuThreadsOut), 1u, 1u};
    if (fp.lookback)
        hipLaunchKernelGGL((ssd_fused_lb_kernel<TT, S, NT>), gout, bout, Lay::BYTES, stream, fp);
    else
        hipLaunchKernelGGL((ssd_fused_kernel<TT, S, NT>), gout, bout, Lay::BYTES, stream, fp);
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
                     hipEvent_t* ev, bool nt) {
    // non-temporal instances exist for 128-token sub-chunks only (the plan
    // asks for them nowhere else)
    switch (TT * 1000 + S) {
        case 32064: return launch_fused_tpl<32, 64, false>(cbp, fp, stream, ev);
        case 32128: return launch_fused_tpl<32, 128, false>(cbp, fp, stream, ev);
        case 64064: return launch_fused_tpl<64, 64, false>(cbp, fp, stream, ev);
        case 64128: return launch_fused_tpl<64, 128, false>(cbp, fp, stream, ev);
        case 128064:
            return nt ? launch_fused_tpl<128, 64, true>(cbp, fp, stream, ev)
                      : launch_fused_tpl<128, 64, false>(cbp, fp, stream, ev);
        case 128128:
            return nt ? launch_fused_tpl<128, 128, true>(cbp, fp, stream, ev)
                      : launch_fused_tpl<128, 128, false>(cbp, fp, stream, ev);
        default: return -8;
    }
}

}  // namespace cls
