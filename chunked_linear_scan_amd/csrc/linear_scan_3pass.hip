// Three-pass (block scan, spine scan, apply) form of the scalar linear
// recurrence h[t] = a[t] h[t-1] + b[t] on gfx950.
//
// Follows "Selective-scan CUDA kernels", section "The five kernels" (level 2:
// block scan, spine scan and prefix application as three launches) with the
// affine combine of its section "The problem": (a1, b1) then (a2, b2) is
// (a1 a2, a2 b1 + b2).  It moves seven arrays' worth of traffic (a and b read;
// the tile-local scan and the tile-local product of a written, then read back;
// h written) where the single-pass look-back kernel moves three, and it
// shares no code with that kernel: it serves as an independent check of it
// and as a measurement of the traffic model on this GPU.
//
//   * block scan: one 256-thread workgroup per 8192-element tile of a row.
//     Each wave owns a 2048-element run, read in steps of 64 lanes x V
//     elements (V = 4: 16-byte vectors, lanes 16 bytes apart; V = 1 when the
//     row length is not a multiple of 4, so rows start unaligned).  A lane
//     scans its V items serially, the wave scans the lane totals with an
//     ordered shuffle ladder, the step carry stays wave-uniform, and the four
//     wave totals are combined through LDS.  The tile's local scan (the h it
//     would have from a zero state) goes to h, the local product of a to the
//     workspace, the tile aggregate to the workspace.
//   * spine: one thread per row walks the row's tile aggregates and writes
//     each tile's incoming state.
//   * apply: h[t] = prod_a[t] h_in(tile) + h[t].
#include "common.hpp"
#include "launch.hpp"

namespace cls {
namespace {

constexpr int kL3Threads = 256;
constexpr int kL3Tile = 8192;             // elements per tile
constexpr int kL3WaveRun = kL3Tile / 4;   // elements per wave

struct Aff {
    float a, b;
};

// (first, then second): h -> s.a (f.a h + f.b) + s.b
__device__ __forceinline__ Aff cmb(Aff f, Aff s) { return Aff{f.a * s.a, fmaf(s.a, f.b, s.b)}; }

__device__ __forceinline__ Aff shfl_up_aff(Aff v, int d) {
    return Aff{__shfl_up(v.a, d, 64), __shfl_up(v.b, d, 64)};
}

template <int V>
__global__ __launch_bounds__(kL3Threads) void ls3_block_scan(const float* __restrict__ a, const float* __restrict__ b,
                                                             float* __restrict__ hloc, float* __restrict__ aprod,
                                                             float* __restrict__ agg, int64_t L, int ntiles) {
    constexpr int STEP = 64 * V;
    constexpr int NSTEP = kL3WaveRun / STEP;
    __shared__ Aff wtot[4];
    const int64_t row = blockIdx.x / ntiles;
    const int tile = int(blockIdx.x % ntiles);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rbase = row * L;
    const int64_t run0 = int64_t(tile) * kL3Tile + int64_t(wave) * kL3WaveRun;
    Aff v[NSTEP][V];
    Aff carry{1.0f, 0.0f};  // the wave's run before the current step (wave-uniform)
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        const int64_t t = run0 + s * STEP + V * lane;
        float av[V], bv[V];
        if constexpr (V == 4) {
            if (t + 4 <= L) {
                const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + rbase + t));
                const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + rbase + t));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    av[e] = x[e];
                    bv[e] = y[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    av[e] = t + e < L ? a[rbase + t + e] : 1.0f;
                    bv[e] = t + e < L ? b[rbase + t + e] : 0.0f;
                }
            }
        } else {
            av[0] = t < L ? a[rbase + t] : 1.0f;
            bv[0] = t < L ? b[rbase + t] : 0.0f;
        }
        Aff acc{1.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < V; ++e) {
            acc = cmb(acc, Aff{av[e], bv[e]});
            v[s][e] = acc;
        }
        // inclusive scan of the lane totals over the wave, in lane order
        Aff x = acc;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const Aff y = shfl_up_aff(x, d);
            if (lane >= d) x = cmb(y, x);
        }
        Aff ex = shfl_up_aff(x, 1);
        if (lane == 0) ex = Aff{1.0f, 0.0f};
        const Aff pre = cmb(carry, ex);
#pragma unroll
        for (int e = 0; e < V; ++e) v[s][e] = cmb(pre, v[s][e]);
        carry = cmb(carry, Aff{__shfl(x.a, 63, 64), __shfl(x.b, 63, 64)});
    }
    if (lane == 0) wtot[wave] = carry;
    __syncthreads();
    Aff wpre{1.0f, 0.0f};
    for (int k = 0; k < wave; ++k) wpre = cmb(wpre, wtot[k]);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        const int64_t t = run0 + s * STEP + V * lane;
        Aff o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = cmb(wpre, v[s][e]);
        if constexpr (V == 4) {
            if (t + 4 <= L) {
                *reinterpret_cast<f32x4*>(hloc + rbase + t) = f32x4{o[0].b, o[1].b, o[2].b, o[3].b};
                *reinterpret_cast<f32x4*>(aprod + rbase + t) = f32x4{o[0].a, o[1].a, o[2].a, o[3].a};
                continue;
            }
        }
#pragma unroll
        for (int e = 0; e < V; ++e) {
            if (t + e < L) {
                hloc[rbase + t + e] = o[e].b;
                aprod[rbase + t + e] = o[e].a;
            }
        }
    }
    if (threadIdx.x == 0) {
        Aff tot{1.0f, 0.0f};
        for (int k = 0; k < 4; ++k) tot = cmb(tot, wtot[k]);
        agg[2 * (row * ntiles + tile)] = tot.a;
        agg[2 * (row * ntiles + tile) + 1] = tot.b;
    }
}

__global__ __launch_bounds__(kL3Threads) void ls3_spine(const float* __restrict__ agg, float* __restrict__ hin,
                                                        int64_t rows, int ntiles) {
    const int64_t row = int64_t(blockIdx.x) * kL3Threads + threadIdx.x;
    if (row >= rows) return;
    float h = 0.0f;
    for (int k = 0; k < ntiles; ++k) {
        hin[row * ntiles + k] = h;
        h = fmaf(agg[2 * (row * ntiles + k)], h, agg[2 * (row * ntiles + k) + 1]);
    }
}

template <int V>
__global__ __launch_bounds__(kL3Threads) void ls3_apply(float* __restrict__ h, const float* __restrict__ aprod,
                                                        const float* __restrict__ hin, int64_t L, int ntiles) {
    constexpr int STEP = kL3Threads * V;
    const int64_t row = blockIdx.x / ntiles;
    const int tile = int(blockIdx.x % ntiles);
    const float hi = hin[row * ntiles + tile];
    const int64_t rbase = row * L;
#pragma unroll 4
    for (int s = 0; s < kL3Tile / STEP; ++s) {
        const int64_t t = int64_t(tile) * kL3Tile + s * STEP + V * threadIdx.x;
        if constexpr (V == 4) {
            if (t + 4 <= L) {
                const f32x4 p = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(aprod + rbase + t));
                const f32x4 q = *reinterpret_cast<const f32x4*>(h + rbase + t);
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = fmaf(p[e], hi, q[e]);
                __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(h + rbase + t));
                continue;
            }
        }
#pragma unroll
        for (int e = 0; e < V; ++e)
            if (t + e < L) h[rbase + t + e] = fmaf(aprod[rbase + t + e], hi, h[rbase + t + e]);
    }
}

template <int V>
int launch3(const float* a, const float* b, float* h, int64_t rows, int64_t L, float* aprod, float* agg,
            float* hin, hipStream_t stream) {
    const int ntiles = int((L + kL3Tile - 1) / kL3Tile);
    const dim3 block{uint32_t(kL3Threads), 1u, 1u};
    const dim3 gt{uint32_t(rows * ntiles), 1u, 1u};
    hipLaunchKernelGGL((ls3_block_scan<V>), gt, block, 0, stream, a, b, h, aprod, agg, L, ntiles);
    hipLaunchKernelGGL(ls3_spine, dim3(uint32_t((rows + kL3Threads - 1) / kL3Threads)), block, 0, stream, agg, hin,
                       rows, ntiles);
    hipLaunchKernelGGL((ls3_apply<V>), gt, block, 0, stream, h, aprod, hin, L, ntiles);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace
}  // namespace cls

extern "C" size_t cls_ls3_workspace_bytes(int64_t rows, int64_t L) {
    const int64_t ntiles = (L + cls::kL3Tile - 1) / cls::kL3Tile;
    const size_t prod = (size_t(rows) * size_t(L) * 4 + 255) / 256 * 256;
    const size_t aggb = (size_t(rows) * size_t(ntiles) * 8 + 255) / 256 * 256;
    return prod + aggb + size_t(rows) * size_t(ntiles) * 4;
}

extern "C" int cls_ls3_launch(const float* a, const float* b, float* h, int64_t rows, int64_t L, void* ws,
                              hipStream_t stream) {
    const int64_t ntiles = (L + cls::kL3Tile - 1) / cls::kL3Tile;
    char* w = static_cast<char*>(ws);
    float* aprod = reinterpret_cast<float*>(w);
    float* agg = reinterpret_cast<float*>(w + (size_t(rows) * size_t(L) * 4 + 255) / 256 * 256);
    float* hin = reinterpret_cast<float*>(reinterpret_cast<char*>(agg) +
                                          (size_t(rows) * size_t(ntiles) * 8 + 255) / 256 * 256);
    return (L % 4 == 0) ? cls::launch3<4>(a, b, h, rows, L, aprod, agg, hin, stream)
                        : cls::launch3<1>(a, b, h, rows, L, aprod, agg, hin, stream);
}
