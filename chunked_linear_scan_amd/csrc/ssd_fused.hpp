// Fused bf16 SSD forward pass on gfx950 for head dim 64: one kernel walks a
// segment of chunks of one (batch, head) with the state on chip, and the
// segments of a sequence are chained by a decoupled look-back over their
// state aggregates.
//
// Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
// NVIDIA cuTile" (sections "Mamba-2 architecture", "Kernel 1/2/3"): per chunk
// the cumulative sum G of a_t = A dt_t, the decayed intra-chunk product, the
// output from the chunk-start state and the state jump
// h <- exp(G_last) h + X^T (dt exp(G_last - G) . B).  The state recurrence
// across chunks is the affine scan (a1, S1) then (a2, S2) = (a1 a2, a2 S1 + S2)
// of "Selective-scan CUDA kernels" (section "The problem") lifted to a
// matrix-valued state, run as a single-pass decoupled look-back (section "The
// five kernels") over segments of chunks.
//
// Work unit (one workgroup, 4 waves): segment `seg` of chain (b, h), i.e.
// chunks [seg K, seg K + K).  A sequence split into more than one segment runs
//   phase 1: the segment's own state aggregate S_seg (zero initial state) and
//            its decay alpha_seg = exp2(sum of the chunks' G_last);
//   publish: aggregate (flag 1) or, for segment 0, the inclusive state
//            alpha h0 + S_seg (flag 2);
//   look-back: fold the predecessors' aggregates back to the nearest
//            inclusive state -> the segment's initial state h_in;
//   publish: inclusive state alpha h_in + S_seg (flag 2);
//   phase 2: outputs and states chunk by chunk from h_in.
// A sequence with one segment runs phase 2 only.  Segments are claimed from
// a counter in segment-major order, so a waiting segment's predecessors are
// always claimed already.
//
// Per chunk (TT tokens, the chunk padded to a multiple of 32):
//   * X is staged row-major in LDS with a 32-byte-pair XOR swizzle; MFMA
//     operands whose contraction index is the token (X as A of the intra
//     product, X as B of the state product, B^T as A of the state product) are
//     read with ds_read_b64_tr_b16, which transposes 4x16 blocks of 16-bit
//     values across each 16-lane group;
//   * each wave stages only the B columns of its own state tiles, in 64-token
//     blocks, so the state product needs no workgroup barrier for B;
//   * off-diagonal 32-token blocks of the intra product use CB scaled by a
//     per-token factor dt_j exp2(G_blockend - G_j) (<= dt_j) and a running
//     rescale of the accumulator by exp2(G_blockend' - G_blockend) (<= 1), so
//     the per-element exponentials are needed only on the diagonal block; every
//     exponent formed is <= 0 under a_t <= 0;
//   * the next chunk's X and dt are prefetched into registers while the
//     current chunk computes.
#pragma once

#include "common.hpp"
#include "ssd_kernels.hpp"

namespace cls {

constexpr int kFuThreads = 256;
constexpr int kFuP = 64;  // head dim of this kernel
constexpr uint32_t kFuSpinLimit = 1u << 24;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 fu_mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two transposed 4x16 reads = one MFMA operand with k = 8(l/16) .. +7.
__device__ __forceinline__ u32x4 lds_tr_pair(const unsigned char* base, uint32_t off1, uint32_t off2) {
    typedef __attribute__((address_space(3))) s16x4* lp;
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(base + off1));
    const s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(base + off2));
    const u32x2 w1 = __builtin_bit_cast(u32x2, v1);
    const u32x2 w2 = __builtin_bit_cast(u32x2, v2);
    return u32x4{w1[0], w1[1], w2[0], w2[1]};
}

template <int TT, int S>
struct FuLayout {
    static constexpr int NSTW = S / 64;                   // state tiles per wave
    static constexpr int TB = TT < 64 ? TT : 64;          // tokens per B block
    static constexpr int NBLK = TT / TB;                  // B blocks per chunk
    static constexpr int BROW = 32 * NSTW;                // bytes per private B row
    static constexpr int HP = S + 8;                      // bf16 pitch of the state rows
    static constexpr int NACC = NSTW * 4 * 4;             // state floats per lane
    static constexpr int X_OFF = 0;                       // [TT][64] bf16, swizzled
    static constexpr int B_OFF = X_OFF + TT * 128;        // 4 x [TB][BROW]
    static constexpr int H_OFF = B_OFF + 4 * TB * BROW;   // [64][HP] bf16
    static constexpr int G_OFF = H_OFF + kFuP * HP * 2;   // G  [TT] f32
    static constexpr int DT_OFF = G_OFF + TT * 4;         // dt [TT]
    static constexpr int CF_OFF = DT_OFF + TT * 4;        // off-diagonal factor [TT]
    static constexpr int W_OFF = CF_OFF + TT * 4;         // state weight [TT]
    static constexpr int Q_OFF = W_OFF + TT * 4;          // block rescale [TT/32]
    static constexpr int MISC_OFF = Q_OFF + 64;           // scan scratch [4], ints [4]
    static constexpr int ALPHA_OFF = MISC_OFF + 32;       // look-back decays [64]
    static constexpr int BYTES = ALPHA_OFF + 64 * 4;
};

// byte offset of (row t, 32-byte pair `pair`, byte `within` < 32) in X
__device__ __forceinline__ uint32_t x_off(int t, int pair, int within) {
    return uint32_t(t * 128 + ((pair ^ (t & 3)) << 5) + within);
}

template <int NSTW>
__device__ __forceinline__ uint32_t b_off(int t, int pair, int within) {
    const int swz = (NSTW == 2) ? ((t >> 1) & 1) : 0;
    return uint32_t(t * (32 * NSTW) + ((pair ^ swz) << 5) + within);
}

template <int TT, int S>
struct FuChunk {
    using Lay = FuLayout<TT, S>;
    static constexpr int NX = TT * 8 / kFuThreads;   // 16-byte pieces of X per thread
    static constexpr int NB = Lay::TB * 2 * Lay::NSTW / 64;  // 16-byte B pieces per lane per block
};

template <bool OUT>
struct FuPhase {
    static constexpr bool value = OUT;
};

// ---------------------------------------------------------------------------
template <int TT, int S>
__global__ __launch_bounds__(kFuThreads) void ssd_fused_kernel(SsdFusedParams p) {
    using Lay = FuLayout<TT, S>;
    constexpr int NSTW = Lay::NSTW;
    constexpr int NX = FuChunk<TT, S>::NX > 0 ? FuChunk<TT, S>::NX : 1;
    constexpr int NB = FuChunk<TT, S>::NB;
    constexpr int NPT = kFuP / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    unsigned char* Xs = sm + Lay::X_OFF;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    unsigned char* Bw = sm + Lay::B_OFF + wave * (Lay::TB * Lay::BROW);
    uint16_t* Hs = reinterpret_cast<uint16_t*>(sm + Lay::H_OFF);
    float* Gt = reinterpret_cast<float*>(sm + Lay::G_OFF);
    float* Dtt = reinterpret_cast<float*>(sm + Lay::DT_OFF);
    float* Cf = reinterpret_cast<float*>(sm + Lay::CF_OFF);
    float* Wt = reinterpret_cast<float*>(sm + Lay::W_OFF);
    float* Qt = reinterpret_cast<float*>(sm + Lay::Q_OFF);
    float* scratch = reinterpret_cast<float*>(sm + Lay::MISC_OFF);
    int* lb_int = reinterpret_cast<int*>(sm + Lay::MISC_OFF + 16);
    float* lb_alpha = reinterpret_cast<float*>(sm + Lay::ALPHA_OFF);

    // ---- claim a segment (segment-major order) ----
    if (tid == 0) lb_int[0] = int(atomic_add_u32(p.claim, 1u));
    __syncthreads();
    const int tile = lb_int[0];
    if (tile < 0 || tile >= p.nchains * p.nsegs) return;  // only a corrupted workspace gets here
    const int seg = tile / p.nchains;
    const int chain = tile % p.nchains;
    const int64_t b = chain / p.H;
    const int h = chain % p.H;
    const int g = h / (p.H / p.G);
    const int c_begin = seg * p.seg_chunks;
    const int c_end = (c_begin + p.seg_chunks < p.nchunks) ? c_begin + p.seg_chunks : p.nchunks;
    const float A2 = p.A[h] * kLog2e;
    const float Dh = p.D ? p.D[h] : 0.0f;
    const int64_t L = p.L;
    const int64_t bh = b * p.H + h;

    f32x4 hacc[NSTW][NPT];
    auto zero_state = [&]() {
#pragma unroll
        for (int k = 0; k < NSTW; ++k)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) hacc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // lane's state tile k covers s-tile st = wave + 4k: rows s = 16 st + 4 kg + r, column p = 16 pt + l16
    auto load_h0 = [&](f32x4 (&dst)[NSTW][NPT]) {
#pragma unroll
        for (int k = 0; k < NSTW; ++k)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (p.h0) v = *reinterpret_cast<const f32x4*>(
                              p.h0 + (bh * kFuP + 16 * pt + l16) * S + 16 * (wave + 4 * k) + 4 * kg);
                dst[k][pt] = v;
            }
    };
    auto store_hs = [&]() {
#pragma unroll
        for (int k = 0; k < NSTW; ++k)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                u32x2 w;
                w[0] = pack_bf16x2(hacc[k][pt][0], hacc[k][pt][1]);
                w[1] = pack_bf16x2(hacc[k][pt][2], hacc[k][pt][3]);
                *reinterpret_cast<u32x2*>(Hs + (16 * pt + l16) * Lay::HP + 16 * (wave + 4 * k) + 4 * kg) = w;
            }
    };

    // ---- chunk loop (phase 1 when OUT == false, phase 2 when OUT == true) ----
    u32x4 xreg[NX];
    float dtv = 0.0f;
    auto prefetch_chunk = [&](int c) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = int((L - tok0 < p.chunk) ? (L - tok0) : p.chunk);
#pragma unroll
        for (int m = 0; m < NX; ++m) {
            const int u = tid + kFuThreads * m;  // piece index: row u / 8, 16-byte chunk u % 8
            const int t = u >> 3, cc = u & 7;
            xreg[m] = (t < n && u < TT * 8)
                          ? ldg_b128(p.x + ((b * L + tok0 + t) * p.H + h) * kFuP + 8 * cc)
                          : u32x4{0u, 0u, 0u, 0u};
        }
        dtv = (tid < n) ? p.dt[(b * L + tok0 + tid) * p.H + h] : 0.0f;
    };
    float sumG = 0.0f;

    auto run_chunks = [&](auto out_tag) {
        constexpr bool OUT = decltype(out_tag)::value;
        if (c_begin < c_end) prefetch_chunk(c_begin);
        for (int c = c_begin; c < c_end; ++c) {
            const int64_t tok0 = int64_t(c) * p.chunk;
            const int n = int((L - tok0 < p.chunk) ? (L - tok0) : p.chunk);
            // X -> LDS (swizzled rows of 128 bytes)
#pragma unroll
            for (int m = 0; m < NX; ++m) {
                const int u = tid + kFuThreads * m;
                if (u < TT * 8) {
                    const int t = u >> 3, cc = u & 7;
                    *reinterpret_cast<u32x4*>(Xs + x_off(t, cc >> 1, (cc & 1) * 16)) = xreg[m];
                }
            }
            const float dt_c = dtv;
            // S1: cumulative sum of a_t inside the chunk (log2 units)
            const float G = block_inclusive_sum_256(A2 * dt_c, scratch);
            if (tid < TT) {
                Gt[tid] = G;
                Dtt[tid] = dt_c;
            }
            if (c + 1 < c_end) prefetch_chunk(c + 1);
            // the first B block of this chunk, into registers
            u32x4 breg[NB];
            auto load_bblock = [&](int blk) {
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    const int u = lane + 64 * m;           // piece: row u/(2 NSTW), state tile (u/2)%NSTW, half u%2
                    const int row = u / (2 * NSTW);
                    const int kk = (u >> 1) % NSTW;
                    const int half = u & 1;
                    const int t = blk * Lay::TB + row;
                    breg[m] = (t < n) ? ldg_b128(p.B + ((b * L + tok0 + t) * p.G + g) * S +
                                                 16 * (wave + 4 * kk) + 8 * half)
                                      : u32x4{0u, 0u, 0u, 0u};
                }
            };
            load_bblock(0);
            __syncthreads();
            // decay tables
            const float Glast = Gt[TT - 1];
            if (tid < TT) {
                const int be = (tid | 31);
                Cf[tid] = Dtt[tid] * fexp2(Gt[be] - Gt[tid]);
                Wt[tid] = Dtt[tid] * fexp2(Glast - Gt[tid]);
            }
            if (tid < TT / 32) {
                const float prev = tid == 0 ? 0.0f : Gt[32 * tid - 1];
                Qt[tid] = fexp2(Gt[32 * tid + 31] - prev);
            }
            sumG += Glast;
            __syncthreads();

            if constexpr (OUT) {
                // S2b + S4: y^T tiles of 16 tokens, balanced over the waves
                constexpr int NIT = TT / 16;
                const uint16_t* cbase = p.cb + ((b * p.nchunks + c) * p.G + g) * (int64_t(TT) * TT);
                const uint16_t* Crow = p.C + ((b * L + tok0) * p.G + g) * S;
                for (int q = 0; q < (NIT + 3) / 4; ++q) {
                    // pairing keeps the causal work per wave even
                    const int it = (q & 1) ? (4 * (q + 1) - 1 - wave) : (4 * q + wave);
                    if (it >= NIT) continue;
                    const int i = 16 * it + l16;
                    const bool vi = i < n;
                    const int jd = it >> 1;
                    u32x4 cfr[S / 32];
#pragma unroll
                    for (int ks = 0; ks < S / 32; ++ks)
                        cfr[ks] = vi ? ldg_b128(Crow + int64_t(i) * p.G * S + 32 * ks + 8 * kg) : u32x4{0u, 0u, 0u, 0u};
                    u32x4 cbr[TT / 32];
#pragma unroll
                    for (int jb = 0; jb < TT / 32; ++jb)
                        cbr[jb] = (jb <= jd) ? ldg_b128(cbase + i * TT + 32 * jb + 8 * kg) : u32x4{0u, 0u, 0u, 0u};
                    f32x4 acc[NPT];
#pragma unroll
                    for (int pt = 0; pt < NPT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    // state term C h^T (k = s)
#pragma unroll
                    for (int ks = 0; ks < S / 32; ++ks) {
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) {
                            const u32x4 hf = *reinterpret_cast<const u32x4*>(
                                Hs + (16 * pt + l16) * Lay::HP + 32 * ks + 8 * kg);
                            acc[pt] = fu_mfma(hf, cfr[ks], acc[pt]);
                        }
                    }
                    // off-diagonal 32-token blocks with a running rescale
#pragma unroll
                    for (int jb = 0; jb < TT / 32; ++jb) {
                        if (jb >= jd) break;
                        const float qv = Qt[jb];
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) acc[pt] *= qv;
                        const int j0 = 32 * jb + 8 * kg;
                        const f32x4 c0 = *reinterpret_cast<const f32x4*>(Cf + j0);
                        const f32x4 c1 = *reinterpret_cast<const f32x4*>(Cf + j0 + 4);
                        const u32x4 cw = cbr[jb];
                        u32x4 wf;
                        wf[0] = pack_bf16x2(bf16_lo(cw[0]) * c0[0], bf16_hi(cw[0]) * c0[1]);
                        wf[1] = pack_bf16x2(bf16_lo(cw[1]) * c0[2], bf16_hi(cw[1]) * c0[3]);
                        wf[2] = pack_bf16x2(bf16_lo(cw[2]) * c1[0], bf16_hi(cw[2]) * c1[1]);
                        wf[3] = pack_bf16x2(bf16_lo(cw[3]) * c1[2], bf16_hi(cw[3]) * c1[3]);
                        const int tr = 32 * jb + 8 * kg + (l16 >> 2);
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) {
                            const uint32_t o1 = x_off(tr, pt, 8 * (l16 & 3));
                            const u32x4 xf = lds_tr_pair(Xs, o1, o1 + 512);
                            acc[pt] = fu_mfma(xf, wf, acc[pt]);
                        }
                    }
                    // bring the accumulator from the last block end to row i
                    {
                        const float gref = jd == 0 ? 0.0f : Gt[32 * jd - 1];
                        const float ri = fexp2(Gt[i] - gref);
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) acc[pt] *= ri;
                    }
                    // diagonal block: element-wise decay, mask and skip term
                    {
                        const float gi = Gt[i];
                        const int j0 = 32 * jd + 8 * kg;
                        const u32x4 cw = cbr[jd];
                        float wv[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint32_t word = cw[e >> 1];
                            const float cbv = (e & 1) ? bf16_hi(word) : bf16_lo(word);
                            const int j = j0 + e;
                            float w = cbv * fexp2(gi - Gt[j]) * Dtt[j];
                            w = (j <= i) ? w : 0.0f;
                            w += (j == i) ? Dh : 0.0f;
                            wv[e] = w;
                        }
                        u32x4 wf;
#pragma unroll
                        for (int e = 0; e < 4; ++e) wf[e] = pack_bf16x2(wv[2 * e], wv[2 * e + 1]);
                        const int tr = 32 * jd + 8 * kg + (l16 >> 2);
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) {
                            const uint32_t o1 = x_off(tr, pt, 8 * (l16 & 3));
                            const u32x4 xf = lds_tr_pair(Xs, o1, o1 + 512);
                            acc[pt] = fu_mfma(xf, wf, acc[pt]);
                        }
                    }
                    if (vi) {
                        uint16_t* dst = p.y + ((b * L + tok0 + i) * p.H + h) * kFuP + 4 * kg;
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) {
                            u32x2 v;
                            v[0] = pack_bf16x2(acc[pt][0], acc[pt][1]);
                            v[1] = pack_bf16x2(acc[pt][2], acc[pt][3]);
                            *reinterpret_cast<u32x2*>(dst + 16 * pt) = v;
                        }
                    }
                }
                __syncthreads();  // every wave is done reading the chunk-start state
            }

            // S2c + S3: h^T <- exp(G_last) h^T + (B^T w) X, wave-private B blocks
            const float alpha = fexp2(Glast);
#pragma unroll
            for (int k = 0; k < NSTW; ++k)
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) hacc[k][pt] *= alpha;
            for (int blk = 0; blk < Lay::NBLK; ++blk) {
                if (blk * Lay::TB >= n) break;
                // this wave's previous block reads are complete (wave-local order)
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    const int u = lane + 64 * m;
                    const int row = u / (2 * NSTW);
                    const int kk = (u >> 1) % NSTW;
                    const int half = u & 1;
                    *reinterpret_cast<u32x4*>(Bw + b_off<NSTW>(row, kk, 16 * half)) = breg[m];
                }
                if (blk + 1 < Lay::NBLK) load_bblock(blk + 1);
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes landed
#pragma unroll
                for (int kt = 0; kt < Lay::TB / 32; ++kt) {
                    const int tl = 32 * kt;                       // token offset in the block
                    const int tc = blk * Lay::TB + tl;            // token offset in the chunk
                    if (tc >= n) break;
                    u32x4 xf[NPT];
                    const int trx = tc + 8 * kg + (l16 >> 2);
#pragma unroll
                    for (int pt = 0; pt < NPT; ++pt) {
                        const uint32_t o1 = x_off(trx, pt, 8 * (l16 & 3));
                        xf[pt] = lds_tr_pair(Xs, o1, o1 + 512);
                    }
                    const f32x4 w0 = *reinterpret_cast<const f32x4*>(Wt + tc + 8 * kg);
                    const f32x4 w1 = *reinterpret_cast<const f32x4*>(Wt + tc + 8 * kg + 4);
                    const int trb = tl + 8 * kg + (l16 >> 2);
#pragma unroll
                    for (int k = 0; k < NSTW; ++k) {
                        const uint32_t o1 = b_off<NSTW>(trb, k, 8 * (l16 & 3));
                        const u32x4 braw = lds_tr_pair(Bw, o1, o1 + 4 * Lay::BROW);
                        u32x4 af;
                        af[0] = pack_bf16x2(bf16_lo(braw[0]) * w0[0], bf16_hi(braw[0]) * w0[1]);
                        af[1] = pack_bf16x2(bf16_lo(braw[1]) * w0[2], bf16_hi(braw[1]) * w0[3]);
                        af[2] = pack_bf16x2(bf16_lo(braw[2]) * w1[0], bf16_hi(braw[2]) * w1[1]);
                        af[3] = pack_bf16x2(bf16_lo(braw[3]) * w1[2], bf16_hi(braw[3]) * w1[3]);
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) hacc[k][pt] = fu_mfma(af, xf[pt], hacc[k][pt]);
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
            if constexpr (OUT) store_hs();
            __syncthreads();  // X, tables and the state rows are free for the next chunk
        }
    };

    if (p.nsegs > 1) {
        // phase 1: this segment's own aggregate
        zero_state();
        run_chunks(FuPhase<false>{});
        const float alpha_seg = fexp2(sumG);
        float* pay = p.payload + int64_t(tile) * 2 * (kFuThreads * Lay::NACC);
        float* pay_agg = pay + tid * Lay::NACC;
        float* pay_inc = pay + kFuThreads * Lay::NACC + tid * Lay::NACC;
        f32x4 hin[NSTW][NPT];
        if (seg == 0) {
            load_h0(hin);
        } else {
            // publish the aggregate
#pragma unroll
            for (int k = 0; k < NSTW; ++k)
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt)
                    store_payload(pay_agg + 4 * (k * NPT + pt), hacc[k][pt]);
            wait_vmem();
            __syncthreads();
            if (tid == 0) store_coherent_b128(p.status + tile, u32x4{1u, as_uint(alpha_seg), 0u, 0u});
            // look back: wave 0 inspects up to 64 predecessors
            if (wave == 0) {
                const int pred = seg - 1 - lane;
                uint32_t spins = 0;
                int kp = 64;
                float al = 1.0f;
                while (true) {
                    int kind = 2;
                    if (pred >= 0) {
                        const u32x4 st = load_coherent_b128(p.status + int64_t(pred) * p.nchains + chain);
                        kind = int(st[0]);
                        al = as_float(st[1]);
                    }
                    const uint64_t incm = __ballot(kind == 2);
                    const uint64_t notready = __ballot(kind == 0);
                    kp = incm ? int(__builtin_ctzll(incm)) : 64;
                    const uint64_t below = (kp >= 64) ? ~0ull : ((1ull << kp) - 1ull);
                    if (!(notready & below) && kp < 64) break;
                    if (++spins > kFuSpinLimit) {
                        if (lane == 0) atomic_add_u32(p.err, 1u);
                        kp = -1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (lane == 0) lb_int[1] = kp;
                if (lane < kp) lb_alpha[lane] = al;
            }
            __syncthreads();
            const int kp = lb_int[1];
#pragma unroll
            for (int k = 0; k < NSTW; ++k)
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) hin[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (kp >= 0) {
                const int base_seg = seg - 1 - kp;
                if (base_seg >= 0) {
                    const float* src = p.payload + (int64_t(base_seg) * p.nchains + chain) * 2 * (kFuThreads * Lay::NACC) +
                                       kFuThreads * Lay::NACC + tid * Lay::NACC;
#pragma unroll
                    for (int k = 0; k < NSTW; ++k)
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt)
                            hin[k][pt] = load_payload(src + 4 * (k * NPT + pt));
                } else {
                    load_h0(hin);  // every predecessor was an aggregate: start from h0
                }
                for (int kk = kp - 1; kk >= 0; --kk) {
                    const float al = lb_alpha[kk];
                    const int sp = seg - 1 - kk;
                    const float* src = p.payload + (int64_t(sp) * p.nchains + chain) * 2 * (kFuThreads * Lay::NACC) +
                                       tid * Lay::NACC;
#pragma unroll
                    for (int k = 0; k < NSTW; ++k)
#pragma unroll
                        for (int pt = 0; pt < NPT; ++pt) {
                            const f32x4 s = load_payload(src + 4 * (k * NPT + pt));
                            hin[k][pt] = hin[k][pt] * al + s;
                        }
                }
            }
        }
        // publish the inclusive state at the segment end
#pragma unroll
        for (int k = 0; k < NSTW; ++k)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                const f32x4 v = hin[k][pt] * alpha_seg + hacc[k][pt];
                store_payload(pay_inc + 4 * (k * NPT + pt), v);
                hacc[k][pt] = hin[k][pt];
            }
        wait_vmem();
        __syncthreads();
        if (tid == 0) store_coherent_b128(p.status + tile, u32x4{2u, as_uint(alpha_seg), 0u, 0u});
    } else {
        load_h0(hacc);
    }
    store_hs();
    __syncthreads();
    run_chunks(FuPhase<true>{});
    if (p.h_final && seg == p.nsegs - 1) {
#pragma unroll
        for (int k = 0; k < NSTW; ++k)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt)
                *reinterpret_cast<f32x4*>(p.h_final + (bh * kFuP + 16 * pt + l16) * S + 16 * (wave + 4 * k) + 4 * kg) =
                    hacc[k][pt];
    }
}

}  // namespace cls
