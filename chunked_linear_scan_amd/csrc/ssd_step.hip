// One decode token of the Mamba-2 SSD recurrence on gfx950.
//
// Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
// NVIDIA cuTile", section "Mamba-2 architecture": the recurrent form, which
// that section names as the one for sequential inference.  With a = A dt and
// b = dt B_t the state becomes exp(a) h + b x^T, and the output is c^T of the
// new state plus D x (the token's own update is seen by its output, as in the
// chunked pass).
//
// The step reads and rewrites the state, P x S fp32 per (batch, head), and
// touches little else, so it is bound by HBM.  One 512-thread workgroup per
// (batch, head).  A row of the state (one head-dim channel, S states) is held
// by S/4 lanes as float4s, so one wave instruction reads or writes 1 KB of
// consecutive state (64 / (S/4) rows).  Each thread loads kStU row steps
// before it computes, so a workgroup keeps 16 KB of loads in flight: the
// whole 64 x 128 state in one pass.  Measured on a 64-sequence, 80-head
// token: 512 threads x 2 steps 55.6-56.0 us; 256 x 4 57.1; 512 x 1 56.7-56.9;
// 1024 x 1 or 2 58.5-59.2; 256 x 2 58.9; 128 x 4 61.5.  The state is read and written with non-temporal
// accesses: each byte is touched once per token, and keeping it out of the
// caches measured 14 % faster on a 64-sequence batch of 80 heads.  The
// output's sum over the states is an xor-shuffle tree inside each row's lanes
// (a fixed order: the result is the same from run to run).
#include "common.hpp"
#include "launch.hpp"

namespace cls {
namespace {

constexpr int kStThreads = 512;
constexpr int kStWaves = kStThreads / 64;
constexpr int kStU = 2;  // row steps a thread loads at once

struct StepParams {
    float* h;
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    void* y;
    int H, P, S, G;
};

template <bool BF16>
__device__ __forceinline__ float load_e(const void* p, int64_t i) {
    if constexpr (BF16) return __builtin_bit_cast(float, uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
    else return static_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_e(void* p, int64_t i, float v) {
    if constexpr (BF16) static_cast<uint16_t*>(p)[i] = uint16_t(pack_bf16x2(v, 0.0f) & 0xffffu);
    else static_cast<float*>(p)[i] = v;
}

// LS: lanes per state row (S / 4)
template <bool BF16, int LS>
__global__ __launch_bounds__(kStThreads) void ssd_step_kernel(StepParams p) {
    constexpr int R = 64 / LS;  // rows per wave instruction
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H;
    const int hd = int(bh % p.H);
    const int g = hd / (p.H / p.G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane / LS, l = lane % LS;
    const float dtv = p.dt[bh];
    const float decay = fexp2(p.A[hd] * dtv * kLog2e);
    const float Dh = p.D ? p.D[hd] : 0.0f;
    // b = dt B and c for this lane's four states (one group row of B and C)
    const int64_t bc = (b * p.G + g) * p.S + 4 * l;
    f32x4 bv, cv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bv[e] = dtv * load_e<BF16>(p.B, bc + e);
        cv[e] = load_e<BF16>(p.C, bc + e);
    }
    float* hb = p.h + bh * int64_t(p.P) * p.S;
    const int64_t xb = bh * p.P;
    for (int p0 = 0; p0 < p.P; p0 += kStWaves * R * kStU) {
        f32x4 hv[kStU];
        float xv[kStU];
        int row[kStU];
#pragma unroll
        for (int u = 0; u < kStU; ++u) {
            row[u] = p0 + (u * kStWaves + wave) * R + sub;
            const bool ok = row[u] < p.P;
            const f32x4* src = reinterpret_cast<const f32x4*>(hb + int64_t(row[u]) * p.S + 4 * l);
            hv[u] = ok ? __builtin_nontemporal_load(src) : f32x4{0.f, 0.f, 0.f, 0.f};
            xv[u] = ok ? load_e<BF16>(p.x, xb + row[u]) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kStU; ++u) {
            const bool ok = row[u] < p.P;
            f32x4 hn;
#pragma unroll
            for (int e = 0; e < 4; ++e) hn[e] = fmaf(decay, hv[u][e], xv[u] * bv[e]);
            if (ok) __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(hb + int64_t(row[u]) * p.S + 4 * l));
            float part = hn[0] * cv[0] + hn[1] * cv[1] + hn[2] * cv[2] + hn[3] * cv[3];
#pragma unroll
            for (int o = LS / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
            if (l == 0 && ok) store_e<BF16>(p.y, xb + row[u], part + Dh * xv[u]);
        }
    }
}

template <bool BF16>
int launch_step(const StepParams& p, int64_t nbh, hipStream_t stream) {
    const dim3 grid{uint32_t(nbh), 1u, 1u}, block{uint32_t(kStThreads), 1u, 1u};
    switch (p.S) {
        case 4: hipLaunchKernelGGL((ssd_step_kernel<BF16, 1>), grid, block, 0, stream, p); break;
        case 8: hipLaunchKernelGGL((ssd_step_kernel<BF16, 2>), grid, block, 0, stream, p); break;
        case 16: hipLaunchKernelGGL((ssd_step_kernel<BF16, 4>), grid, block, 0, stream, p); break;
        case 32: hipLaunchKernelGGL((ssd_step_kernel<BF16, 8>), grid, block, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((ssd_step_kernel<BF16, 16>), grid, block, 0, stream, p); break;
        case 128: hipLaunchKernelGGL((ssd_step_kernel<BF16, 32>), grid, block, 0, stream, p); break;
        case 256: hipLaunchKernelGGL((ssd_step_kernel<BF16, 64>), grid, block, 0, stream, p); break;
        default: return -8;
    }
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace
}  // namespace cls

extern "C" int cls_ssd_step_launch(float* h, const void* x, const float* dt, const float* A, const void* B,
                                   const void* C, const float* D, void* y, int64_t batch, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups, int dtype,
                                   hipStream_t stream) {
    cls::StepParams p{h, x, dt, A, B, C, D, y, int(nheads), int(headdim), int(dstate), int(ngroups)};
    return dtype == 1 ? cls::launch_step<true>(p, batch * nheads, stream)
                      : cls::launch_step<false>(p, batch * nheads, stream);
}
