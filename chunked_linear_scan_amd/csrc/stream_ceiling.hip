// A plain streaming kernel with the linear scan's HBM traffic (read two fp32
// arrays, write one: h[i] = a[i] b[i]), used to measure what a three-stream
// kernel reaches on this device.  It is no part of the scan; it is the
// ceiling the scan's bandwidth is read against.
//
// Each thread moves VEC 16-byte vectors of each array per iteration, spaced
// one workgroup-width apart, so every wave-wide access covers 1 KB of
// consecutive memory.  grid_blocks = 0 gives one pass with one workgroup per
// 256 * VEC vectors; otherwise a grid-stride loop over that many workgroups.
// nt: non-temporal loads and stores (the scan's policy) or the default one.
#include "common.hpp"

namespace cls {

template <int VEC, bool NT>
__global__ __launch_bounds__(256) void stream_mul_kernel(const f32x4* __restrict__ a, const f32x4* __restrict__ b,
                                                         f32x4* __restrict__ h, int64_t n4) {
    const int64_t step = int64_t(gridDim.x) * 256 * VEC;
    for (int64_t base = int64_t(blockIdx.x) * 256 * VEC + threadIdx.x; base < n4; base += step) {
        f32x4 x[VEC], y[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const int64_t i = base + int64_t(v) * 256;
            if (i < n4) {
                x[v] = NT ? __builtin_nontemporal_load(a + i) : a[i];
                y[v] = NT ? __builtin_nontemporal_load(b + i) : b[i];
            }
        }
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const int64_t i = base + int64_t(v) * 256;
            if (i < n4) {
                const f32x4 r = x[v] * y[v];
                if (NT)
                    __builtin_nontemporal_store(r, h + i);
                else
                    h[i] = r;
            }
        }
    }
}

template <int VEC, bool NT>
int launch_stream(const float* a, const float* b, float* h, int64_t n4, int64_t grid_blocks, hipStream_t s) {
    const int64_t per = int64_t(256) * VEC;
    const int64_t blocks = grid_blocks > 0 ? grid_blocks : (n4 + per - 1) / per;
    const dim3 grid{uint32_t(blocks), 1u, 1u};
    const dim3 block{256u, 1u, 1u};
    hipLaunchKernelGGL((stream_mul_kernel<VEC, NT>), grid, block, 0, s, reinterpret_cast<const f32x4*>(a),
                       reinterpret_cast<const f32x4*>(b), reinterpret_cast<f32x4*>(h), n4);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace cls

// n: a multiple of 4; vec in {1, 2, 4, 8}; the caller has checked pointers,
// alignment and sizes.
extern "C" int cls_launch_stream_mul(const float* a, const float* b, float* h, int64_t n, int vec, int nt,
                                     int64_t grid_blocks, hipStream_t s) {
    using namespace cls;
    const int64_t n4 = n / 4;
    switch (vec * 2 + (nt ? 1 : 0)) {
        case 2: return launch_stream<1, false>(a, b, h, n4, grid_blocks, s);
        case 3: return launch_stream<1, true>(a, b, h, n4, grid_blocks, s);
        case 4: return launch_stream<2, false>(a, b, h, n4, grid_blocks, s);
        case 5: return launch_stream<2, true>(a, b, h, n4, grid_blocks, s);
        case 8: return launch_stream<4, false>(a, b, h, n4, grid_blocks, s);
        case 9: return launch_stream<4, true>(a, b, h, n4, grid_blocks, s);
        case 16: return launch_stream<8, false>(a, b, h, n4, grid_blocks, s);
        case 17: return launch_stream<8, true>(a, b, h, n4, grid_blocks, s);
        default: return -2;
    }
}
