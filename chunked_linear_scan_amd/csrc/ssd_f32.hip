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
// whose state fits in LDS, and is not the throughput path.  Where two chunks'
// operands fit in LDS (small head dims, state sizes and chunks), the next
// chunk's are loaded while the current one is computed.
#include "common.hpp"
#include "device_once.hpp"
#include "ssd_kernels.hpp"

namespace cls {

constexpr int kF32Threads = 256;
constexpr int kF32Prefetch = 32;  // most floats of a staged chunk one thread holds in flight

// A staged chunk: x [T][P], B [T][S], C [T][S] and dt [T], zero past the last
// real token.
__host__ __device__ constexpr int f32_stage_floats(int P, int S, int T) { return T * (P + 2 * S + 1); }

size_t ssd_f32_lds_bytes(int P, int S) {
    return sizeof(float) * (size_t(P) * (S + 1) + 3 * 256 + 16 * S + 16 * 256 + 32 * P + 32 * S + 4);
}

// Chunks are staged when two of them fit in LDS beside the working tiles and a
// thread's share fits its prefetch registers: then a chunk's operands arrive in
// one load round trip, issued while the previous chunk is computed, instead of
// one round trip per phase of the chunk (the shapes where the walk over the
// chunks is latency-bound).
static bool f32_staged(int P, int S, int T) {
    const int sf = f32_stage_floats(P, S, T);
    return sf <= kF32Threads * kF32Prefetch && ssd_f32_lds_bytes(P, S) + 2 * sizeof(float) * sf <= 160 * 1024;
}

template <bool STAGED, bool AGG>
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
    float* Stg = scratch + 4;                // STAGED: [2][stage floats], chunk c in half c & 1

    const int tid = threadIdx.x;
    // workgroup = (chain, segment), segments of a chain adjacent
    const int nsegs = p.nsegs > 1 ? p.nsegs : 1;
    const int per_chain = AGG ? nsegs - 1 : nsegs;
    const int64_t bh = int64_t(blockIdx.x) / per_chain;
    const int seg = int(int64_t(blockIdx.x) % per_chain);
    const int64_t tok_begin = nsegs > 1 ? int64_t(seg) * p.seg_chunks * T : 0;
    const int64_t tok_end =
        (nsegs > 1 && tok_begin + int64_t(p.seg_chunks) * T < p.L) ? tok_begin + int64_t(p.seg_chunks) * T : p.L;
    const int64_t b = bh / p.H;
    const int h = int(bh % p.H);
    const int g = h / (p.H / p.G);
    const float Ah = p.A[h];
    const float Dh = p.D ? p.D[h] : 0.0f;

    const int64_t L = p.L;
    const float* x = static_cast<const float*>(p.x);
    const float* Bm = static_cast<const float*>(p.B);
    const float* Cm = static_cast<const float*>(p.C);
    float* y = static_cast<float*>(p.y);
    const int SF = f32_stage_floats(P, S, T);
    const int OFF_B = T * P, OFF_C = T * (P + S), OFF_DT = T * (P + 2 * S);

    // this thread's share of the chunk starting at t0, loaded into registers:
    // 16-byte piece q = tid + 256 k of the staged x, B and C rows, and (tid < T)
    // dt of token tid
    const int P4 = P / 4, S4 = S / 4, NX4 = T * P4, NB4 = T * S4;
    f32x4 pf[kF32Prefetch / 4];
    float pdt = 0.0f;
    auto fetch = [&](int64_t t0) {
        const int n = int((L - t0 < T) ? (L - t0) : T);
#pragma unroll
        for (int k = 0; k < kF32Prefetch / 4; ++k) {
            const int q = tid + kF32Threads * k;
            const bool isx = q < NX4;
            const bool isc = !isx && q - NX4 >= NB4;
            const int idx = isx ? q : q - NX4 - (isc ? NB4 : 0);
            const int w4 = isx ? P4 : S4;
            const int row = idx / w4, col = 4 * (idx - row * w4);
            // the source address, chosen with masks (a select between three
            // pointers is otherwise compiled as a table in scratch memory)
            const uint64_t ax = reinterpret_cast<uint64_t>(x + ((b * L + t0 + row) * p.H + h) * P + col);
            const uint64_t bo = uint64_t(((b * L + t0 + row) * p.G + g) * S + col) * sizeof(float);
            const uint64_t ab = reinterpret_cast<uint64_t>(Bm) + bo, ac = reinterpret_cast<uint64_t>(Cm) + bo;
            const uint64_t mx = 0 - uint64_t(isx), mc = 0 - uint64_t(isc), mb = ~(mx | mc);
            const float* src = reinterpret_cast<const float*>((ax & mx) | (ab & mb) | (ac & mc));
            pf[k] = (q < NX4 + 2 * NB4 && row < n) ? *reinterpret_cast<const f32x4*>(src) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        pdt = tid < n ? p.dt[(b * L + t0 + tid) * p.H + h] : 0.0f;
    };
    auto stash = [&](int half) {
        f32x4* dst = reinterpret_cast<f32x4*>(Stg + half * SF);
#pragma unroll
        for (int k = 0; k < kF32Prefetch / 4; ++k) {
            const int q = tid + kF32Threads * k;
            if (q < NX4 + 2 * NB4) dst[q] = pf[k];
        }
        if (tid < T) Stg[half * SF + OFF_DT + tid] = pdt;
    };

    // start state: zero (aggregate launch), else h0 folded with the earlier
    // segments' aggregates in order (segment by segment, each thread over its
    // own elements, so a segment's loads are in flight together)
    for (int q = tid; q < P * S; q += kF32Threads) {
        const int pp = q / S, ss = q % S;
        Hs[pp * HP + ss] = (!AGG && p.h0) ? p.h0[(bh * P + pp) * S + ss] : 0.0f;
    }
    if constexpr (!AGG) {
        for (int k = 0; k < seg; ++k) {
            const int64_t slot = bh * (nsegs - 1) + k;
            const float a = expf(p.seg_decay[slot]);
            const float* sv = p.seg_state + slot * P * S;
#pragma unroll 4
            for (int q = tid; q < P * S; q += kF32Threads) {
                float& hq = Hs[(q / S) * HP + q % S];
                hq = hq * a + sv[q];
            }
        }
    }
    if constexpr (STAGED) {
        fetch(tok_begin);
        stash(0);
    }
    __syncthreads();

    int ci = 0;
    float sumG = 0.0f;  // natural-log decay of the chunks so far (aggregate launch)
    for (int64_t tok0 = tok_begin; tok0 < tok_end; tok0 += T, ++ci) {
        const int n = int((tok_end - tok0 < T) ? (tok_end - tok0) : T);
        const bool more = tok0 + T < tok_end;
        if constexpr (STAGED) {
            if (more) fetch(tok0 + T);  // in flight while this chunk is computed
        }
        const float* St = Stg + (ci & 1) * SF;  // STAGED: this chunk
        // cumulative sum of a_t inside the chunk (natural-log units)
        float dtv = 0.0f;
        if (tid < n) dtv = STAGED ? St[OFF_DT + tid] : p.dt[((b * L) + tok0 + tid) * p.H + h];
        const float G = block_inclusive_sum_256(Ah * dtv, scratch);
        if (tid < T) {
            Gs[tid] = G;
            dts[tid] = dtv;
        }
        __syncthreads();
        const float Glast = Gs[n - 1];
        sumG += Glast;
        if (tid < n) ws[tid] = dts[tid] * expf(Glast - Gs[tid]);

        // outputs, 16 rows at a time (none in the aggregate launch)
        for (int i0 = 0; !AGG && i0 < n; i0 += 16) {
            const int nr = (n - i0 < 16) ? (n - i0) : 16;
            // the 16 C rows (a staged chunk holds zeros past its last real row)
            const float* Cr = STAGED ? St + OFF_C + i0 * S : Cb;
            if constexpr (!STAGED) {
#pragma unroll 4
                for (int q = tid; q < 16 * S; q += kF32Threads) {
                    const int r = q / S, ss = q % S;
                    Cb[q] = (r < nr) ? Cm[((b * L + tok0 + i0 + r) * p.G + g) * S + ss] : 0.0f;
                }
            }
            __syncthreads();
            const int jmax = i0 + nr;
            for (int j = tid; j < jmax; j += kF32Threads) {
                float acc[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
                const float* brow = STAGED ? St + OFF_B + j * S : Bm + ((b * L + tok0 + j) * p.G + g) * S;
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
                        for (int r = 0; r < 16; ++r) acc[r] = fmaf(Cr[r * S + ss + e], bv[e], acc[r]);
                }
                for (; ss < S; ++ss) {
                    const float bv = brow[ss];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[r] = fmaf(Cr[r * S + ss], bv, acc[r]);
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
                for (int ss = 0; ss < S; ++ss) s1 = fmaf(Cr[r * S + ss], Hs[pp * HP + ss], s1);
                float out = expf(Gs[i]) * s1;
                // token j of this channel at xc[j * xs]
                const float* xc = STAGED ? St + pp : x + ((b * L + tok0) * p.H + h) * P + pp;
                const int64_t xs = STAGED ? int64_t(P) : int64_t(p.H) * P;
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
        // the next chunk into the other half (its last reader was the previous
        // chunk, before this chunk's first barrier); the state jump's barriers
        // order these writes before the next chunk's reads
        if constexpr (STAGED) {
            if (more) stash((ci + 1) & 1);
        }

        // state jump to the next chunk start
        const float alpha = expf(Glast);
        for (int j0 = 0; j0 < n; j0 += 32) {
            const int nj = (n - j0 < 32) ? (n - j0) : 32;
#pragma unroll 4
            for (int q = tid; q < 32 * P; q += kF32Threads) {
                const int jj = q / P, pp = q % P;
                const float xv = (jj < nj) ? (STAGED ? St[(j0 + jj) * P + pp]
                                                     : x[((b * L + tok0 + j0 + jj) * p.H + h) * P + pp])
                                           : 0.0f;
                Xs[q] = (jj < nj) ? ws[j0 + jj] * xv : 0.0f;
            }
#pragma unroll 4
            for (int q = tid; q < 32 * S; q += kF32Threads) {
                const int jj = q / S, ss = q % S;
                Bs[q] = (jj < nj) ? (STAGED ? St[OFF_B + (j0 + jj) * S + ss]
                                            : Bm[((b * L + tok0 + j0 + jj) * p.G + g) * S + ss])
                                  : 0.0f;
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

    if constexpr (AGG) {
        const int64_t slot = bh * (nsegs - 1) + seg;
        for (int q = tid; q < P * S; q += kF32Threads) p.seg_state[slot * P * S + q] = Hs[(q / S) * HP + q % S];
        if (tid == 0) p.seg_decay[slot] = sumG;
    } else if (p.h_final && seg == nsegs - 1) {
        for (int q = tid; q < P * S; q += kF32Threads) {
            const int pp = q / S, ss = q % S;
            p.h_final[(bh * P + pp) * S + ss] = Hs[pp * HP + ss];
        }
    }
}

size_t ssd_f32_launch_lds(int P, int S, int T) {
    return ssd_f32_lds_bytes(P, S) + (f32_staged(P, S, T) ? 2 * sizeof(float) * f32_stage_floats(P, S, T) : 0);
}

int ssd_f32_launch(const SsdF32Params& prm, hipStream_t stream) {
    const bool staged = f32_staged(prm.P, prm.S, prm.chunk);
    const size_t lds = ssd_f32_launch_lds(prm.P, prm.S, prm.chunk);
    static DeviceOnce attrs;
    if (run_once_per_device(attrs, [] {
            const void* fns[] = {reinterpret_cast<const void*>(ssd_f32_kernel<false, false>),
                                 reinterpret_cast<const void*>(ssd_f32_kernel<true, false>),
                                 reinterpret_cast<const void*>(ssd_f32_kernel<false, true>),
                                 reinterpret_cast<const void*>(ssd_f32_kernel<true, true>)};
            for (const void* f : fns)
                if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
                    return -7;
            return 0;
        }) != 0)
        return -7;
    const int64_t nsegs = prm.nsegs > 1 ? prm.nsegs : 1;
    const dim3 block{uint32_t(kF32Threads), 1u, 1u};
    if (nsegs > 1) {
        const dim3 gagg{uint32_t(prm.batch * prm.H * (nsegs - 1)), 1u, 1u};
        if (staged)
            hipLaunchKernelGGL((ssd_f32_kernel<true, true>), gagg, block, lds, stream, prm);
        else
            hipLaunchKernelGGL((ssd_f32_kernel<false, true>), gagg, block, lds, stream, prm);
    }
    const dim3 grid{uint32_t(prm.batch * prm.H * nsegs), 1u, 1u};
    if (staged)
        hipLaunchKernelGGL((ssd_f32_kernel<true, false>), grid, block, lds, stream, prm);
    else
        hipLaunchKernelGGL((ssd_f32_kernel<false, false>), grid, block, lds, stream, prm);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace cls
