// bf16 SSD chunked forward pass on gfx950: MFMA contractions with fp32
// accumulation and an fp32 state.
//
// Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
// NVIDIA cuTile".  Per chunk of T tokens and per (batch, head):
//   S1  G = inclusive cumulative sum of A dt (kept in log2 units so every
//       exponential is one exp2), section "Kernel 1";
//   S2a CB = C B^T for the chunk, computed once per (batch, chunk, group) by
//       ssd_cb_kernel and shared by all heads of the group (the page's output
//       kernel recomputes it per head);
//   S2b the decay-masked product (CB . exp(G_i - G_j) . dt_j . [i >= j]) X, with
//       the skip term D x folded into the diagonal;
//   S2c/S3 the state jump h <- exp(G_last) h + X^T (dt exp(G_last - G) . B),
//       section "Kernel 2", with h carried in registers across chunks;
//   S4  y = exp(G_i) (C_i h^T) + intra term, section "Kernel 3".
// Positive exponents (j > i) are never kept: the masked entries are selected
// away, not multiplied by zero.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16] and D[4(l/16)..+3][l%16].  Every product is arranged
// so its output columns are tokens or head-dim channels that a lane can store
// or reuse without a register transpose:
//   y^T[p][i]   = H[p][s] C[i][s]^T  +  X^T[p][j] W[i][j]^T     (k = s, then j)
//   h^T[s][p]  += (B^T[s][t] w_t) X[t][p]                        (k = t)
//   CB^T[j][i]  = B[j][s] C[i][s]^T                              (k = s)
// The token-major operands (X and B for k = t) are transposed once per chunk
// into LDS with an in-register 8x8 transpose.
#pragma once

#include "common.hpp"
#include "device_once.hpp"
#include "ssd_kernels.hpp"

namespace cls {

constexpr int kBfThreads = 256;

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// ---------------------------------------------------------------------------
// S2a: CB[b, c, g][i][j] = sum_s C[i][s] B[j][s] for the 32-token blocks with
// block(j) <= block(i), row-major [TT][TT] bf16.  Padded rows and columns
// (token >= chunk length) are written as zeros.  One workgroup (four waves)
// per (batch, chunk, group): the chunk's B rows are staged in LDS once, and
// wave w takes the 16-row tiles in pairs (w + 4 k, NIT - 1 - w - 4 k), so every
// wave has the same share of the triangle (with fewer tiles than 8, one tile
// per wave).  A tile's C rows stay in registers.
// ---------------------------------------------------------------------------
template <int TT>
inline uint32_t cb_grid(const SsdBf16Params& prm) {
    return uint32_t(prm.batch * prm.nchunks * prm.G);
}

// LDS of the CB pass: the chunk's B rows at a pitch of S + 8 bf16
constexpr size_t ssd_cb_lds_bytes(int TT, int S) { return size_t(TT) * (S + 8) * 2; }

template <int TT, int S>
__global__ __launch_bounds__(kBfThreads) void ssd_cb_kernel(SsdBf16Params p) {
    constexpr int KS = S / 32;
    constexpr int NIT = TT / 16;
    constexpr int BP = S + 8;
    constexpr int CPR = S / 8;  // 16-byte pieces per row
    extern __shared__ __attribute__((aligned(16))) unsigned char cb_sm[];
    uint16_t* sB = reinterpret_cast<uint16_t*>(cb_sm);  // [TT][BP]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int64_t bcg = blockIdx.x;
    const int g = int(bcg % p.G);
    const int64_t c = (bcg / p.G) % p.nchunks;
    const int64_t b = bcg / (int64_t(p.G) * p.nchunks);
    const int64_t tok0 = c * p.chunk;
    const int n = int((p.L - tok0 < p.chunk) ? (p.L - tok0) : p.chunk);
    uint16_t* out = p.cb + bcg * (TT * TT);
    const int64_t rowstride = int64_t(p.G) * S;
    const uint16_t* Cbase = p.C + ((b * p.L + tok0) * p.G + g) * S;
    const uint16_t* Bbase = p.B + ((b * p.L + tok0) * p.G + g) * S;

    for (int q = tid; q < TT * CPR; q += kBfThreads) {
        const int r = q / CPR, c8 = q % CPR;
        const u32x4 v = r < n ? ldg16(Bbase + r * rowstride + 8 * c8) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(sB + r * BP + 8 * c8) = v;
    }
    __syncthreads();

    constexpr int NTW = NIT >= 8 ? NIT / 4 : 1;  // row tiles per wave
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
        const int w4 = wave + 4 * (k >> 1);
        const int it = NIT < 8 ? wave : ((k & 1) ? NIT - 1 - w4 : w4);
        if (it >= NIT) continue;
        const int i = 16 * it + l16;
        u32x4 cf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            cf[ks] = (i < n) ? ldg16(Cbase + i * rowstride + 32 * ks + 8 * kg) : u32x4{0, 0, 0, 0};
        const int ntj = 2 * (it >> 1) + 2;  // the column tiles of the blocks <= block(it)
        for (int jt = 0; jt < ntj; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = mfma16x16x32(*reinterpret_cast<const u32x4*>(sB + (16 * jt + l16) * BP + 32 * ks + 8 * kg),
                                   cf[ks], acc);
            // lane holds CB[i][16 jt + 4 kg + r], r = 0..3
            u32x2 v;
            v[0] = pack_bf16x2(acc[0], acc[1]);
            v[1] = pack_bf16x2(acc[2], acc[3]);
            *reinterpret_cast<u32x2*>(out + i * TT + 16 * jt + 4 * kg) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// S1, S2b, S2c, S3, S4 for one (batch, head): chunks in order, state in
// registers (fp32) and in LDS as the bf16 MFMA operand.
//
// One workgroup of four waves per (batch, head), or per (batch, column block
// of a head) where heads are split (SsdBf16Params.hshift); chunks over 128
// tokens run as 128-token sub-chunks (or shorter, until the tiles fit LDS).  Where LDS
// allows few workgroups per CU, each output tile issues all of its C and
// C B^T loads before its first product and chunk c + 1's dt, X and B rows
// are loaded while chunk c computes.  The barriers order LDS only
// (s_waitcnt lgkmcnt(0); s_barrier), so loads stay in flight across them.
// Eight waves per workgroup measured slower on three of four shapes.
//
// Where the chains are too few to fill the CUs they are cut into segments
// (SsdBf16Params.nsegs): an aggregate launch (AGG) runs every segment but a
// chain's last from a zero state without outputs and writes its state and
// log2 decay; the output launch runs one workgroup per segment, which starts
// from h0 folded with its predecessors' aggregates in segment order
// (h <- exp2(decay) h + state).
// ---------------------------------------------------------------------------
constexpr int kChunkWaves = 4;
constexpr int kChunkThreads = 64 * kChunkWaves;

__device__ __forceinline__ void chunk_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive sum over the workgroup's threads in order (one value each);
// `scratch` holds kChunkWaves floats of LDS.  Ends with a barrier.
__device__ __forceinline__ float chunk_inclusive_sum(float v, float* scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    if (lane == 63) scratch[wave] = v;
    chunk_lds_barrier();
    float add = 0.0f;
#pragma unroll
    for (int q = 0; q < kChunkWaves - 1; ++q)
        if (q < wave) add += scratch[q];
    chunk_lds_barrier();
    return v + add;
}

template <int TT, int P, int S, bool AGG>
__global__ __launch_bounds__(kChunkThreads) void ssd_chunk_kernel(SsdBf16Params p) {
    constexpr int NW = kChunkWaves, NT = kChunkThreads;
    constexpr int XP = TT + 8;            // LDS pitch (elements) of X^T and B^T rows
    constexpr int HP = S + 8;             // LDS pitch of the bf16 state rows
    constexpr int NPT = P / 16;           // head-dim tiles
    constexpr int NST = S / 16;           // state tiles
    constexpr int KS = (NST + NW - 1) / NW;  // state tiles per wave
    constexpr int NJB = TT / 32;          // 32-token blocks of a chunk
    // 8-token x 8-channel items of the X and B transposes, and per thread
    constexpr int NXQ = (TT / 8) * (P / 8), NBQ = (TT / 8) * (S / 8);
    constexpr int NXI = (NXQ + NT - 1) / NT, NBI = (NBQ + NT - 1) / NT;
    // Loads ahead of use.  Where LDS already keeps a CU to at most three of
    // these workgroups, the registers are better spent holding loads early:
    // a tile issues all of its loads at once and, with room to spare, the
    // next chunk's rows are held through this chunk's products (VGPRs per
    // lane estimated from the state, a tile's loads and accumulators, and the
    // held rows; spill-free per instance at these bounds).  Where more
    // workgroups fit, fewer registers per wave (more workgroups per CU) hide
    // latency better: measured 706 against 1228 us on a head-dim-32 layer.
    constexpr int kLdsWorkgroups = int((size_t(160) * 1024) / ssd_bf16_lds_bytes(TT, P, S));
    constexpr int kTileRegs = (KS * NPT + S / 32 + NJB + NPT) * 4;
    constexpr bool kTileAhead = kLdsWorkgroups <= 3 && kTileRegs <= 192;
    constexpr bool kAhead = kTileAhead && kTileRegs + 32 * (NXI + NBI) <= 160;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    uint16_t* Xt = reinterpret_cast<uint16_t*>(smem_raw);   // [P][XP]
    uint16_t* Bt = Xt + P * XP;                              // [S][XP]
    uint16_t* Hs = Bt + S * XP;                              // [P][HP]
    float* Gs = reinterpret_cast<float*>(Hs + P * HP);       // [TT]
    float* dts = Gs + TT;                                    // [TT]
    float* ws = dts + TT;                                    // [TT]
    float* scratch = ws + TT;                                // [NW]

    static_assert(size_t(KS) * NPT * NT * 4 == chunk_state_floats(P, S), "segment state layout");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    // workgroup = (chain, segment), segments of a chain adjacent
    const int nsegs = p.nsegs > 1 ? p.nsegs : 1;
    const int per_chain = AGG ? nsegs - 1 : nsegs;
    const int64_t bh = int64_t(blockIdx.x) / per_chain;
    const int seg = int(int64_t(blockIdx.x) % per_chain);
    const int c_begin = nsegs > 1 ? seg * p.seg_chunks : 0;
    const int c_end = (nsegs > 1 && c_begin + p.seg_chunks < p.nchunks) ? c_begin + p.seg_chunks : p.nchunks;
    const int64_t b = bh / p.H;
    const int h = int(bh % p.H);
    const int g = h / (p.H / p.G);
    const int hin = h >> p.hshift;  // the input head (dt, A, D)
    const int Hin = p.H >> p.hshift;
    const float A2 = p.A[hin] * kLog2e;
    const float Dh = p.D ? p.D[hin] : 0.0f;
    const int64_t L = p.L;

    // state h^T tiles owned by this wave: s-tiles st = wave + NW k, all p-tiles.
    // Segment state fragment (k, pt) of this thread at f32x4 index
    // ((slot * KS + k) * NPT + pt) * NT + tid, slot = chain * (nsegs - 1) + segment.
    const f32x4* seg_state = reinterpret_cast<const f32x4*>(p.seg_state);
    f32x4 hacc[KS][NPT];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int st = wave + NW * k;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (!AGG && st < NST && p.h0) {
                const float* src = p.h0 + (bh * P + 16 * pt + l16) * S + 16 * st + 4 * kg;
                v = *reinterpret_cast<const f32x4*>(src);
            }
            hacc[k][pt] = v;
        }
    }
    // the earlier segments' aggregates, in order; each segment's fragments are
    // loaded together, so a segment costs one memory latency, not one per fragment
    if constexpr (!AGG) {
        for (int k2 = 0; k2 < seg; ++k2) {
            const int64_t slot = bh * (nsegs - 1) + k2;
            const float a = fexp2(p.seg_decay[slot]);
            f32x4 sv[KS][NPT];
#pragma unroll
            for (int k = 0; k < KS; ++k)
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt)
                    sv[k][pt] = wave + NW * k < NST ? seg_state[((slot * KS + k) * NPT + pt) * NT + tid]
                                                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; ++k)
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) hacc[k][pt] = hacc[k][pt] * a + sv[k][pt];
        }
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int st = wave + NW * k;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
            const f32x4 v = hacc[k][pt];
            if (st < NST) {
                u32x2 w;
                w[0] = pack_bf16x2(v[0], v[1]);
                w[1] = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<u32x2*>(Hs + (16 * pt + l16) * HP + 16 * st + 4 * kg) = w;
            }
        }
    }

    // dt of a chunk (one token per thread); X and B rows of transpose item q
    // (8 tokens x 8 channels, 8 rows of 16 bytes)
    auto load_dt = [&](int64_t tok0, int n) { return tid < n ? p.dt[(b * L + tok0 + tid) * Hin + hin] : 0.0f; };
    auto x_row = [&](int64_t tok0, int n, int q, int e) {
        const int t = 8 * (q / (P / 8)) + e;
        return (q < NXQ && t < n) ? ldg16(p.x + ((b * L + tok0 + t) * p.H + h) * P + 8 * (q % (P / 8)))
                                  : u32x4{0, 0, 0, 0};
    };
    auto b_row = [&](int64_t tok0, int n, int q, int e) {
        const int t = 8 * (q / (S / 8)) + e;
        return (q < NBQ && t < n) ? ldg16(p.B + ((b * L + tok0 + t) * p.G + g) * S + 8 * (q % (S / 8)))
                                  : u32x4{0, 0, 0, 0};
    };
    // X^T [p][t] and B^T [s][t] (bf16) into LDS through an 8x8 register transpose
    auto store_x = [&](int q, const u32x4 (&r)[8]) {
        const int tb = q / (P / 8), pb = q % (P / 8);
        u32x4 o[8];
        transpose8x8_b16(r, o);
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(Xt + (8 * pb + e) * XP + 8 * tb) = o[e];
    };
    auto store_b = [&](int q, const u32x4 (&r)[8]) {
        const int tb = q / (S / 8), sb = q % (S / 8);
        u32x4 o[8];
        transpose8x8_b16(r, o);
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(Bt + (8 * sb + e) * XP + 8 * tb) = o[e];
    };
    // kAhead: the next chunk's dt and rows, loaded during this chunk's products
    float dt_nx = 0.0f;
    u32x4 xr[kAhead ? NXI : 1][8], br[kAhead ? NBI : 1][8];
    auto fetch = [&](int c) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = int((L - tok0 < p.chunk) ? (L - tok0) : p.chunk);
        dt_nx = load_dt(tok0, n);
#pragma unroll
        for (int k = 0; k < NXI; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[k][e] = x_row(tok0, n, tid + NT * k, e);
#pragma unroll
        for (int k = 0; k < NBI; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) br[k][e] = b_row(tok0, n, tid + NT * k, e);
    };
    if constexpr (kAhead) fetch(c_begin);

    float sumG = 0.0f;  // log2 decay of the chunks so far (AGG)
    for (int c = c_begin; c < c_end; ++c) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = int((L - tok0 < p.chunk) ? (L - tok0) : p.chunk);

        // S1: cumulative sum of a_t (log2 units) inside the chunk (threads
        // past the chunk add 0)
        const float dtv = kAhead ? dt_nx : load_dt(tok0, n);
        const float G = chunk_inclusive_sum(A2 * dtv, scratch);
        if (tid < TT) {
            Gs[tid] = G;
            dts[tid] = dtv;
        }

        if constexpr (kAhead) {
#pragma unroll
            for (int k = 0; k < NXI; ++k)
                if (tid + NT * k < NXQ) store_x(tid + NT * k, xr[k]);
#pragma unroll
            for (int k = 0; k < NBI; ++k)
                if (tid + NT * k < NBQ) store_b(tid + NT * k, br[k]);
        } else {
            // one item at a time: the state holds most of the registers
            for (int q = tid; q < NXQ; q += NT) {
                u32x4 r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = x_row(tok0, n, q, e);
                store_x(q, r);
            }
            for (int q = tid; q < NBQ; q += NT) {
                u32x4 r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = b_row(tok0, n, q, e);
                store_b(q, r);
            }
        }
        chunk_lds_barrier();
        if constexpr (kAhead)
            if (c + 1 < c_end) fetch(c + 1);  // in flight through this chunk's products
        const float Glast = Gs[TT - 1];  // padded positions add 0: G at the last real token
        sumG += Glast;
        if (tid < TT) ws[tid] = dts[tid] * fexp2(Glast - Gs[tid]);

        // S2b + S4: y^T tiles, 16 tokens per tile, tiles spread over the waves
        const uint16_t* cbase = p.cb + ((b * p.nchunks + c) * p.G + g) * (TT * TT);
        const uint16_t* Cbase = p.C + ((b * L + tok0) * p.G + g) * S;
        const int ntile = AGG ? 0 : (n + 15) / 16;  // the aggregate launch has no outputs
        for (int it = wave; it < ntile; it += NW) {
            const int i = 16 * it + l16;
            const bool vi = i < n;
            const int jb_end = (16 * it + 15) / 32;
            // C row i and the C B^T row pieces: all issued first (kTileAhead),
            // else each right before its product
            auto load_c = [&](int ks) {
                return vi ? ldg16(Cbase + int64_t(i) * p.G * S + 32 * ks + 8 * kg) : u32x4{0, 0, 0, 0};
            };
            auto load_cb = [&](int jb) {
                return jb <= jb_end ? ldg16(cbase + i * TT + 32 * jb + 8 * kg) : u32x4{0, 0, 0, 0};
            };
            u32x4 cf[S / 32], cbw[NJB];
            if constexpr (kTileAhead) {
#pragma unroll
                for (int ks = 0; ks < S / 32; ++ks) cf[ks] = load_c(ks);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) cbw[jb] = load_cb(jb);
            }
            const float gi = Gs[i];
            f32x4 acc[NPT];
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < S / 32; ++ks) {
                const u32x4 cfk = kTileAhead ? cf[ks] : load_c(ks);
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) {
                    const u32x4 hf = *reinterpret_cast<const u32x4*>(Hs + (16 * pt + l16) * HP + 32 * ks + 8 * kg);
                    acc[pt] = mfma16x16x32(hf, cfk, acc[pt]);
                }
            }
            const float sc = fexp2(gi);
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) acc[pt] *= sc;
            // diagonal-and-below block jb: W = CB . exp2(G_i - G_j) . dt_j on j <= i, D on j = i
            auto block = [&](int jb, const u32x4& cbj) {
                const int j0 = 32 * jb + 8 * kg;
                float wv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t word = cbj[e >> 1];
                    const float cbv = (e & 1) ? bf16_hi(word) : bf16_lo(word);
                    const int j = j0 + e;
                    float w = cbv * fexp2(gi - Gs[j]) * dts[j];
                    w = (j <= i) ? w : 0.0f;
                    w += (j == i) ? Dh : 0.0f;
                    wv[e] = w;
                }
                u32x4 wf;
#pragma unroll
                for (int e = 0; e < 4; ++e) wf[e] = pack_bf16x2(wv[2 * e], wv[2 * e + 1]);
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) {
                    const u32x4 xf = *reinterpret_cast<const u32x4*>(Xt + (16 * pt + l16) * XP + 32 * jb + 8 * kg);
                    acc[pt] = mfma16x16x32(xf, wf, acc[pt]);
                }
            };
            if constexpr (kTileAhead) {
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
                    if (jb <= jb_end) block(jb, cbw[jb]);
            } else {
                for (int jb = 0; jb <= jb_end; ++jb) block(jb, load_cb(jb));
            }
            if (vi) {
                uint16_t* dst = p.y + ((b * L + tok0 + i) * p.H + h) * P + 4 * kg;
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) {
                    u32x2 v;
                    v[0] = pack_bf16x2(acc[pt][0], acc[pt][1]);
                    v[1] = pack_bf16x2(acc[pt][2], acc[pt][3]);
                    *reinterpret_cast<u32x2*>(dst + 16 * pt) = v;
                }
            }
        }
        chunk_lds_barrier();

        // S2c + S3: h^T <- exp(G_last) h^T + (B^T w) X
        const float alpha = fexp2(Glast);
        const int ntb = (n + 31) / 32;
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) hacc[k][pt] *= alpha;
        for (int tb = 0; tb < ntb; ++tb) {
            const int t0 = 32 * tb + 8 * kg;
            float wt[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) wt[e] = ws[t0 + e];
            u32x4 xf[NPT];
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt)
                xf[pt] = *reinterpret_cast<const u32x4*>(Xt + (16 * pt + l16) * XP + t0);
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int st = wave + NW * k;
                if (st >= NST) continue;
                const u32x4 braw = *reinterpret_cast<const u32x4*>(Bt + (16 * st + l16) * XP + t0);
                u32x4 af;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    af[e] = pack_bf16x2(bf16_lo(braw[e]) * wt[2 * e], bf16_hi(braw[e]) * wt[2 * e + 1]);
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) hacc[k][pt] = mfma16x16x32(af, xf[pt], hacc[k][pt]);
            }
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int st = wave + NW * k;
            if (st >= NST) continue;
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                u32x2 w;
                w[0] = pack_bf16x2(hacc[k][pt][0], hacc[k][pt][1]);
                w[1] = pack_bf16x2(hacc[k][pt][2], hacc[k][pt][3]);
                *reinterpret_cast<u32x2*>(Hs + (16 * pt + l16) * HP + 16 * st + 4 * kg) = w;
            }
        }
        chunk_lds_barrier();
    }

    if constexpr (AGG) {
        const int64_t slot = bh * (nsegs - 1) + seg;
        f32x4* out = reinterpret_cast<f32x4*>(p.seg_state);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            if (wave + NW * k >= NST) continue;
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) out[((slot * KS + k) * NPT + pt) * NT + tid] = hacc[k][pt];
        }
        if (tid == 0) p.seg_decay[slot] = sumG;
    } else if (p.h_final && seg == nsegs - 1) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int st = wave + NW * k;
            if (st >= NST) continue;
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                float* dst = p.h_final + (bh * P + 16 * pt + l16) * S + 16 * st + 4 * kg;
                *reinterpret_cast<f32x4*>(dst) = hacc[k][pt];
            }
        }
    }
}

template <int TT, int P, int S>
int launch_ssd_bf16_tpl(const SsdBf16Params& prm, hipStream_t stream) {
    const size_t lds = ssd_bf16_lds_bytes(TT, P, S);
    constexpr size_t cb_lds = ssd_cb_lds_bytes(TT, S);
    static DeviceOnce attrs;
    if (run_once_per_device(attrs, [lds] {
            return hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_chunk_kernel<TT, P, S, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) == hipSuccess &&
                           hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_chunk_kernel<TT, P, S, true>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) == hipSuccess &&
                           hipFuncSetAttribute(reinterpret_cast<const void*>(ssd_cb_kernel<TT, S>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(cb_lds)) == hipSuccess
                       ? 0
                       : -7;
        }) != 0)
        return -7;
    const int64_t nsegs = prm.nsegs > 1 ? prm.nsegs : 1;
    const dim3 gcb{cb_grid<TT>(prm), 1u, 1u}, bcb{uint32_t(kBfThreads), 1u, 1u};
    hipLaunchKernelGGL((ssd_cb_kernel<TT, S>), gcb, bcb, cb_lds, stream, prm);
    const dim3 bmain{uint32_t(kChunkThreads), 1u, 1u};
    if (nsegs > 1) {
        const dim3 gagg{uint32_t(prm.batch * prm.H * (nsegs - 1)), 1u, 1u};
        hipLaunchKernelGGL((ssd_chunk_kernel<TT, P, S, true>), gagg, bmain, lds, stream, prm);
    }
    const dim3 gmain{uint32_t(prm.batch * prm.H * nsegs), 1u, 1u};
    hipLaunchKernelGGL((ssd_chunk_kernel<TT, P, S, false>), gmain, bmain, lds, stream, prm);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace cls
