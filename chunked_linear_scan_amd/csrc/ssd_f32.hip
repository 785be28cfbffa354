// fp32 SSD chunked forward pass on gfx950 (VALU, fp32 end to end).
//
// Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
// NVIDIA cuTile": per chunk, the inclusive cumulative sum G of a_t = A dt_t
// (section "Kernel 1"), the output from the chunk-start state plus the
// decay-masked intra-chunk product (section "Kernel 3" and the decayed output
// formula of section "Mamba-2 architecture"), and the state jump to the next
// chunk start (section "Kernel 2").  The output keeps the diagonal of the
// causal mask (y_t sees h_t).
//
// This path exists for fp32 inputs, where bf16 operands would exceed the fp32
// error budget.  One workgroup owns one (batch, head) and walks its chunks in
// order with the state in LDS; it is correct for any head dim / state size
// whose state fits in LDS, and is not the throughput path.
#include "common.hpp"
#include "device_once.hpp"
#include "ssd_kernels.hpp"

namespace cls {

constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads) void ssd_f32_kernel(SsdF32Params p) {
    extern __shared__ float smem[];
    const int P = p.P, S = p.S, T = p.chunk;
    const int HP = S + 1;  // padded state row pitch
    float* Hs = smem;                        // [P][S+1]
    float* Gs = Hs + P * HP;                 // [T]
    float* dts = Gs + 256;                   // [T]
    float* ws = dts + 256;                   // [T]
    float* Cb = ws + 256;                    // [16][S]
    float* Wb = Cb + 16 * S;                 // [16][T]
    float* Xs = Wb + 16 * 256;               // [32][P]
    float* Bs = Xs + 32 * P;                 // [32][S]
    float* scratch = Bs + 32 * S;            // [4]

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H;
    const int h = int(bh % p.H);
    const int g = h / (p.H / p.G);
    const float Ah = p.A[h];
    const float Dh = p.D ? p.D[h] : 0.0f;

    for (int q = tid; q < P * S; q += kF32Threads) {
        const int pp = q / S, ss = q % S;
        Hs[pp * HP + ss] = p.h0 ? p.h0[(bh * P + pp) * S + ss] : 0.0f;
    }
    __syncthreads();

    const int64_t L = p.L;
    const float* x = static_cast<const float*>(p.x);
    const float* Bm = static_cast<const float*>(p.B);
    const float* Cm = static_cast<const float*>(p.C);
    float* y = static_cast<float*>(p.y);

    for (int64_t tok0 = 0; tok0 < L; tok0 += T) {
        const int n = int((L - tok0 < T) ? (L - tok0) : T);
        // cumulative sum of a_t inside the chunk (natural-log units)
        float dtv = 0.0f;
        if (tid < n) dtv = p.dt[((b * L) + tok0 + tid) * p.H + h];
        const float G = block_inclusive_sum_256(Ah * dtv, scratch);
        if (tid < T) {
            Gs[tid] = G;
            dts[tid] = dtv;
        }
        __syncthreads();
        const float Glast = Gs[n - 1];
        if (tid < n) ws[tid] = dts[tid] * expf(Glast - Gs[tid]);

        // outputs, 16 rows at a time
        for (int i0 = 0; i0 < n; i0 += 16) {
            const int nr = (n - i0 < 16) ? (n - i0) : 16;
#pragma unroll 4
            for (int q = tid; q < 16 * S; q += kF32Threads) {
                const int r = q / S, ss = q % S;
                Cb[q] = (r < nr) ? Cm[((b * L + tok0 + i0 + r) * p.G + g) * S + ss] : 0.0f;
            }
            __syncthreads();
            const int jmax = i0 + nr;
            for (int j = tid; j < jmax; j += kF32Threads) {
                float acc[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
                const float* brow = Bm + ((b * L + tok0 + j) * p.G + g) * S;
                // eight loads in flight at a time: one at a time, each waited for
                // before the next, the chunk cost a global-memory latency per item
                int ss = 0;
                for (; ss + 8 <= S; ss += 8) {
                    float bv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) bv[e] = brow[ss + e];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[r] = fmaf(Cb[r * S + ss + e], bv[e], acc[r]);
                }
                for (; ss < S; ++ss) {
                    const float bv = brow[ss];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[r] = fmaf(Cb[r * S + ss], bv, acc[r]);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = i0 + r;
                    float w = 0.0f;
                    if (r < nr && j <= i) w = acc[r] * expf(Gs[i] - Gs[j]) * dts[j];
                    if (j == i) w += Dh;
                    Wb[r * 256 + j] = w;
                }
            }
            __syncthreads();
            for (int q = tid; q < nr * P; q += kF32Threads) {
                const int r = q / P, pp = q % P;
                const int i = i0 + r;
                float s1 = 0.0f;
                for (int ss = 0; ss < S; ++ss) s1 = fmaf(Cb[r * S + ss], Hs[pp * HP + ss], s1);
                float out = expf(Gs[i]) * s1;
                const float* xc = x + ((b * L + tok0) * p.H + h) * P + pp;  // token j at j * H * P
                const int64_t xs = int64_t(p.H) * P;
                int j = 0;
                for (; j + 8 <= i + 1; j += 8) {  // eight loads in flight, as above
                    float xv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) xv[e] = xc[(j + e) * xs];
#pragma unroll
                    for (int e = 0; e < 8; ++e) out = fmaf(Wb[r * 256 + j + e], xv[e], out);
                }
                for (; j <= i; ++j) out = fmaf(Wb[r * 256 + j], xc[j * xs], out);
                y[((b * L + tok0 + i) * p.H + h) * P + pp] = out;
            }
            __syncthreads();
        }

        // state jump to the next chunk start
        const float alpha = expf(Glast);
        for (int j0 = 0; j0 < n; j0 += 32) {
            const int nj = (n - j0 < 32) ? (n - j0) : 32;
#pragma unroll 4
            for (int q = tid; q < 32 * P; q += kF32Threads) {
                const int jj = q / P, pp = q % P;
                Xs[q] = (jj < nj) ? ws[j0 + jj] * x[((b * L + tok0 + j0 + jj) * p.H + h) * P + pp] : 0.0f;
            }
#pragma unroll 4
            for (int q = tid; q < 32 * S; q += kF32Threads) {
                const int jj = q / S, ss = q % S;
                Bs[q] = (jj < nj) ? Bm[((b * L + tok0 + j0 + jj) * p.G + g) * S + ss] : 0.0f;
            }
            __syncthreads();
            for (int q = tid; q < P * S; q += kF32Threads) {
                const int pp = q / S, ss = q % S;
                float v = Hs[pp * HP + ss];
                if (j0 == 0) v *= alpha;
                for (int jj = 0; jj < nj; ++jj) v = fmaf(Xs[jj * P + pp], Bs[jj * S + ss], v);
                Hs[pp * HP + ss] = v;
            }
            __syncthreads();
        }
    }

    if (p.h_final) {
        for (int q = tid; q < P * S; q += kF32Threads) {
            const int pp = q / S, ss = q % S;
            p.h_final[(bh * P + pp) * S + ss] = Hs[pp * HP + ss];
        }
    }
}

size_t ssd_f32_lds_bytes(int P, int S) {
    return sizeof(float) * (size_t(P) * (S + 1) + 3 * 256 + 16 * S + 16 * 256 + 32 * P + 32 * S + 4);
}

int ssd_f32_launch(const SsdF32Params& prm, hipStream_t stream) {
    const size_t lds = ssd_f32_lds_bytes(prm.P, prm.S);
    static DeviceOnce attrs;
    if (run_once_per_device(attrs, [] {
            return hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_f32_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess
                       ? 0
                       : -7;
        }) != 0)
        return -7;
    const dim3 grid{uint32_t(prm.batch * prm.H), 1u, 1u};
    const dim3 block{uint32_t(kF32Threads), 1u, 1u};
    hipLaunchKernelGGL(ssd_f32_kernel, grid, block, lds, stream, prm);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace cls
