// Fused bf16 SSD forward pass on gfx950 for head dim 64: one workgroup walks
// a segment of chunks of one (batch, head) with the state on chip, and the
// segments of a sequence are chained by a decoupled look-back over their
// state aggregates.
//
// Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
// NVIDIA cuTile" (sections "Mamba-2 architecture", "Kernel 1/2/3"): per chunk
// the cumulative sum G of a_t = A dt_t, the output from the chunk-start state,
// the decayed intra-chunk product and the state jump
// h <- exp(G_last) h + X^T (dt exp(G_last - G) . B).  The state recurrence
// across chunks is the affine scan (a1, S1) then (a2, S2) = (a1 a2, a2 S1 + S2)
// of "Selective-scan CUDA kernels" (section "The problem") lifted to a
// matrix-valued state and run as a single-pass decoupled look-back (section
// "The five kernels") over segments of chunks.
//
// Work unit (one workgroup, 8 waves): segment `seg` of chain (b, h), i.e.
// chunks [seg K, seg K + K).  A sequence split into several segments runs
//   phase 1: the segment's own aggregate S_seg (zero initial state) and its
//            decay alpha_seg = exp2(sum of the chunks' G_last);
//   publish: the aggregate (flag 1), or for segment 0 the inclusive state
//            alpha h0 + S_seg (flag 2);
//   look-back: fold the predecessors' aggregates back to the nearest
//            inclusive state -> the segment's initial state h_in;
//   publish: the inclusive state alpha h_in + S_seg (flag 2);
//   phase 2: outputs and states chunk by chunk from h_in.
// A sequence with one segment runs phase 2 only.  Segments are claimed from a
// counter in segment-major order, so a waiting segment's predecessors are
// always claimed already.
//
// Per chunk (TT tokens, the chunk padded to a multiple of 32), one pass over
// 32-token blocks does three products at once: the state jump (wave = state
// tile), and the intra product of two 16-token output tiles per wave, paired
// (i, NIT-1-i) so every wave has the same causal work.  The X fragments of a
// block (read from LDS with ds_read_b64_tr_b16, which transposes 4x16 blocks
// of 16-bit values across a 16-lane group) serve as the B operand of the state
// product and the A operand of the intra product.  B^T comes ready-made from
// the CB pass, so its fragments are plain 16-byte loads.  C, CB and B^T
// fragments are fetched a little ahead into small register rings (the next
// chunk's first ones while the current chunk ends), and the next chunk's X goes
// straight from global memory into the other half of a double LDS buffer while
// the current one computes.  Off-diagonal blocks of the intra product use CB scaled by a
// per-token factor dt_j exp2(G_blockend - G_j) (<= dt_j) and a running rescale
// of the accumulator by exp2(G_blockend' - G_blockend) (<= 1), so
// per-element exponentials are needed only on the diagonal block; every
// exponent formed is <= 0 under a_t <= 0.
#pragma once

#include "common.hpp"
#include "ssd_kernels.hpp"

namespace cls {

constexpr int kFuThreads = 512;
constexpr int kFuWaves = kFuThreads / 64;
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

// Workgroup barrier for LDS traffic only: the wave's LDS operations are
// complete, then all waves meet.  Global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int TT, int S>
struct FuLayout {
    static_assert(S == 64 || S == 128, "state size of the fused kernel");
    static_assert(TT >= 32 && TT <= 256 && TT % 32 == 0, "tile tokens");
    static constexpr int NST = S / 16;                    // state tiles (16 wide)
    static constexpr int NPW = (4 * NST) / kFuWaves;      // state head-dim tiles per wave
    static constexpr int NACC = NPW * 4;                  // state floats per lane
    static constexpr int NIT = TT / 16;                   // 16-token output tiles
    static constexpr int NPAIR = NIT / 2;                 // output tile pairs
    static constexpr int WPP = kFuWaves / NPAIR;          // waves per pair
    static constexpr int NPTW = WPP >= 4 ? 1 : 4 / WPP;   // output head-dim tiles per wave
    static constexpr int NB = TT / 32;                    // 32-token blocks
    static constexpr int XBYTES = TT * 128;               // one X buffer [TT][64] bf16
    static constexpr int NXP = XBYTES / 1024;             // 1 KB pieces of X (8 rows)
    static constexpr int NXI = (NXP + kFuWaves - 1) / kFuWaves;  // X pieces per wave
    static constexpr int HP = S + 8;                      // bf16 pitch of the state rows
    static constexpr int X_OFF = 0;                       // 2 x [TT][64] bf16, swizzled
    static constexpr int H_OFF = X_OFF + 2 * XBYTES;      // [64][HP] bf16
    static constexpr int G_OFF = H_OFF + kFuP * HP * 2;   // G  [TT] f32
    static constexpr int DT_OFF = G_OFF + TT * 4;         // dt [TT]
    static constexpr int CF_OFF = DT_OFF + TT * 4;        // off-diagonal factor [TT]
    static constexpr int W_OFF = CF_OFF + TT * 4;         // state weight [TT]
    static constexpr int Q_OFF = W_OFF + TT * 4;          // block rescale [TT/32]
    static constexpr int MISC_OFF = Q_OFF + 64;           // scan scratch [8], ints [4]
    static constexpr int ALPHA_OFF = MISC_OFF + 64;       // look-back decays [64]
    static constexpr int BYTES = ALPHA_OFF + 64 * 4;
};

// byte offset of (row t, 32-byte pair `pair`, byte `within` < 32) in X
__device__ __forceinline__ uint32_t x_off(int t, int pair, int within) {
    return uint32_t(t * 128 + ((pair ^ (t & 3)) << 5) + within);
}

// 16 bytes per lane from global memory straight into LDS at lds_wave + 16 lane
// (global_load_lds_dwordx4; the LDS base must be wave-uniform).  The compiler
// counts it as a vector memory load but does not order later LDS reads after
// it: readers wait with wait_vmcnt and a barrier.
__device__ __forceinline__ void load_to_lds(const void* src, unsigned char* lds_wave) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave, 16, 0, 0);
}

// s_waitcnt vmcnt(N): at most N vector memory operations of this wave are
// still outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <bool OUT>
struct FuPhase {
    static constexpr bool value = OUT;
};

// Inclusive sum over the workgroup (threads past the chunk add 0).
__device__ __forceinline__ float fu_inclusive_sum(float v, float* scratch) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    if (lane == 63) scratch[wave] = v;
    lds_barrier();
    float add = 0.0f;
#pragma unroll
    for (int q = 0; q < kFuWaves - 1; ++q)
        if (q < wave) add += scratch[q];
    lds_barrier();
    return v + add;
}

// ---------------------------------------------------------------------------
template <int TT, int S>
__global__ __launch_bounds__(kFuThreads) void ssd_fused_kernel(SsdFusedParams p) {
    using Lay = FuLayout<TT, S>;
    constexpr int NPW = Lay::NPW;
    constexpr int NPTW = Lay::NPTW;
    constexpr int NB = Lay::NB;
    constexpr int NXI = Lay::NXI;
    constexpr int KS = S / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches and bases
    const int l16 = lane & 15, kg = lane >> 4;
    uint16_t* Hs = reinterpret_cast<uint16_t*>(sm + Lay::H_OFF);
    float* Gt = reinterpret_cast<float*>(sm + Lay::G_OFF);
    float* Dtt = reinterpret_cast<float*>(sm + Lay::DT_OFF);
    float* Cf = reinterpret_cast<float*>(sm + Lay::CF_OFF);
    float* Wt = reinterpret_cast<float*>(sm + Lay::W_OFF);
    float* Qt = reinterpret_cast<float*>(sm + Lay::Q_OFF);
    float* scratch = reinterpret_cast<float*>(sm + Lay::MISC_OFF);
    int* lb_int = reinterpret_cast<int*>(sm + Lay::MISC_OFF + 32);
    float* lb_alpha = reinterpret_cast<float*>(sm + Lay::ALPHA_OFF);

    // state tile of this wave: s-tile st, head-dim tiles pt0 .. pt0 + NPW - 1
    const int st = wave % Lay::NST;
    const int pt0 = (wave / Lay::NST) * NPW;
    // output tiles of this wave: 16-token tiles itA, itB, head-dim tiles ptb ..
    const int pair = wave % Lay::NPAIR;
    const int ptb = (wave / Lay::NPAIR) * NPTW;
    const bool has_out = ptb < 4;
    const int itA = pair, itB = Lay::NIT - 1 - pair;
    const int jdA = itA >> 1, jdB = itB >> 1;

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

    // state: lane holds h^T[s][p] for s = 16 st + 4 kg + r, p = 16 (pt0 + j) + l16
    f32x4 hacc[NPW];
    auto load_h0 = [&](f32x4 (&dst)[NPW]) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (p.h0) v = *reinterpret_cast<const f32x4*>(p.h0 + (bh * kFuP + 16 * (pt0 + j) + l16) * S +
                                                          16 * st + 4 * kg);
            dst[j] = v;
        }
    };
    auto store_hs = [&]() {
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            u32x2 w;
            w[0] = pack_bf16x2(hacc[j][0], hacc[j][1]);
            w[1] = pack_bf16x2(hacc[j][2], hacc[j][3]);
            *reinterpret_cast<u32x2*>(Hs + (16 * (pt0 + j) + l16) * Lay::HP + 16 * st + 4 * kg) = w;
        }
    };

    // ---- per-chunk operand fetches ----
    auto chunk_rows = [&](int c) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        return int((L - tok0 < p.chunk) ? (L - tok0) : p.chunk);
    };
    // X of chunk c into buffer `buf`: every wave issues NXI pieces of 8 rows; lane
    // i of a piece fills LDS bytes 16 i .. 16 i + 15, so it loads the 16 bytes of
    // the logical row and column that the swizzle places there.  Rows past the
    // chunk load a real row of it (finite values; their weights are zero).
    auto issue_x = [&](int c, int buf) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = chunk_rows(c);
        const char* base = reinterpret_cast<const char*>(p.x + ((b * L + tok0) * p.H + h) * kFuP);
        unsigned char* xb = sm + Lay::X_OFF + buf * Lay::XBYTES;
#pragma unroll
        for (int m = 0; m < NXI; ++m) {
            const int piece = (wave + kFuWaves * m) % Lay::NXP;  // small tiles: duplicates, same data
            const int t = 8 * piece + (lane >> 3);
            const int pc = lane & 7;                                    // 16-byte slot in the row
            const int cc = (((pc >> 1) ^ (t & 3)) << 1) | (pc & 1);     // logical 16-byte column
            const int tr = t < n ? t : n - 1;
            load_to_lds(base + uint32_t(tr) * uint32_t(p.H * kFuP * 2) + uint32_t(cc * 16), xb + piece * 1024);
        }
    };
    auto fetch_dt = [&](int c) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = chunk_rows(c);
        return tid < n ? p.dt[(b * L + tok0 + tid) * p.H + h] : 0.0f;
    };
    // operands shared by the heads of a group live per (b, chunk, g); lane offsets are 32-bit
    const int64_t bcg0 = b * p.nchunks * p.G + g;  // (b, chunk 0, g)
    auto cb_base = [&](int c) {
        return reinterpret_cast<const char*>(p.cb + (bcg0 + int64_t(c) * p.G) * (int64_t(TT) * TT));
    };
    auto bt_base = [&](int c) {
        return reinterpret_cast<const char*>(p.bt + (bcg0 + int64_t(c) * p.G) * (int64_t(S) * TT));
    };
    const uint32_t bt_lane = uint32_t(((16 * st + l16) * TT + 8 * kg) * 2);
    const uint32_t cbA_lane = uint32_t(((16 * itA + l16) * TT + 8 * kg) * 2);
    const uint32_t cbB_lane = uint32_t(((16 * itB + l16) * TT + 8 * kg) * 2);
    auto fetch_c = [&](int c, int it, u32x4 (&dst)[KS]) {
        const int n = chunk_rows(c);
        const int i = 16 * it + l16;
        const int ir = i < n ? i : n - 1;  // rows past the sequence: any finite row (outputs not stored)
        const char* base = reinterpret_cast<const char*>(p.C + ((b * L + int64_t(c) * p.chunk) * p.G + g) * S);
        const uint32_t off = uint32_t(ir) * uint32_t(p.G * S * 2) + uint32_t(16 * kg);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dst[ks] = ldg_b128(base + off + 64 * ks);
    };

    // Rings of kRing fragments: block k of a chunk sits in slot k % kRing.  When
    // block k is consumed its slot is refilled with block k + kRing of the same
    // chunk or, past the tile's last block jd, with block k % kRing of the next.
    constexpr int kRing = 2;
    u32x4 btr[kRing];              // B^T fragments (state product)
    u32x4 rA[kRing], rB[kRing];    // CB fragments of the two output tiles
    u32x4 cA[KS], cB[KS];          // C fragments of the two output tiles
    float sumG = 0.0f;

    auto run_chunks = [&](auto out_tag) {
        constexpr bool OUT = decltype(out_tag)::value;
        if (c_begin >= c_end) return;
        // prologue: operands of the first chunk (X first: the waits below count on it)
        issue_x(c_begin, c_begin & 1);
        float dtv = fetch_dt(c_begin);
#pragma unroll
        for (int k = 0; k < kRing; ++k)
            if (k < NB) btr[k] = ldg_b128(bt_base(c_begin) + bt_lane + 64 * k);
        if (OUT && has_out) {
            fetch_c(c_begin, itA, cA);
            fetch_c(c_begin, itB, cB);
#pragma unroll
            for (int k = 0; k < kRing; ++k) {
                if (k <= jdA) rA[k] = ldg_b128(cb_base(c_begin) + cbA_lane + 64 * k);
                if (k <= jdB) rB[k] = ldg_b128(cb_base(c_begin) + cbB_lane + 64 * k);
            }
        }

        for (int c = c_begin; c < c_end; ++c) {
            const int64_t tok0 = int64_t(c) * p.chunk;
            const int n = chunk_rows(c);
            const bool more = c + 1 < c_end;
            const int cn = c + 1;
            const char* cbc = cb_base(c);
            const char* cbn = cb_base(cn);
            const char* btc = bt_base(c);
            const char* btn = bt_base(cn);
            const unsigned char* Xs = sm + Lay::X_OFF + (c & 1) * Lay::XBYTES;
            const float dt_c = dtv;
            // the other X buffer was last read in the previous chunk: every wave is past it
            if (more) {
                issue_x(cn, cn & 1);
                dtv = fetch_dt(cn);
            }
            // S1: cumulative sum of a_t inside the chunk (log2 units)
            const float G = fu_inclusive_sum(A2 * dt_c, scratch);
            if (tid < TT) {
                Gt[tid] = G;
                Dtt[tid] = dt_c;
            }
            // This chunk's X pieces of this wave have landed.  Issued after them: the
            // B^T ring refills (min(kRing, NB) in the prologue, NB in a full chunk)
            // and, when there is a next chunk, its NXI X pieces.
            if (c == c_begin) {
                if (more) wait_vmcnt<(kRing < NB ? kRing : NB) + NXI>();
                else wait_vmcnt<(kRing < NB ? kRing : NB)>();
            } else {
                if (more) wait_vmcnt<NB + NXI>();
                else wait_vmcnt<NB>();
            }
            lds_barrier();
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
            lds_barrier();

            const float alpha = fexp2(Glast);
#pragma unroll
            for (int j = 0; j < NPW; ++j) hacc[j] *= alpha;

            // S4 state term y^T += H C^T from the chunk-start state (bf16 in LDS)
            f32x4 accA[NPTW], accB[NPTW];
            if constexpr (OUT) {
#pragma unroll
                for (int q = 0; q < NPTW; ++q) {
                    accA[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                    accB[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                if (has_out) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                        for (int q = 0; q < NPTW; ++q) {
                            const u32x4 hf = *reinterpret_cast<const u32x4*>(
                                Hs + (16 * (ptb + q) + l16) * Lay::HP + 32 * ks + 8 * kg);
                            accA[q] = fu_mfma(hf, cA[ks], accA[q]);
                            accB[q] = fu_mfma(hf, cB[ks], accB[q]);
                        }
                    }
                    if (more) {
                        fetch_c(cn, itA, cA);
                        fetch_c(cn, itB, cB);
                    }
                }
            }

            // one pass over the 32-token blocks: S2c/S3 state jump, S2b intra product
#pragma unroll 1
            for (int jb0 = 0; jb0 < NB; jb0 += kRing)
#pragma unroll
            for (int slot = 0; slot < kRing; ++slot) {
                const int jb = jb0 + slot;
                if (kRing > NB && jb >= NB) break;
                const int trx = 32 * jb + 8 * kg + (l16 >> 2);
                u32x4 xf[4];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const uint32_t o1 = x_off(trx, pt, 8 * (l16 & 3));
                    xf[pt] = lds_tr_pair(Xs, o1, o1 + 512);
                }
                {
                    const int t0 = 32 * jb + 8 * kg;
                    const f32x4 w0 = *reinterpret_cast<const f32x4*>(Wt + t0);
                    const f32x4 w1 = *reinterpret_cast<const f32x4*>(Wt + t0 + 4);
                    const u32x4 braw = btr[slot];
                    u32x4 af;
                    af[0] = pack_bf16x2(bf16_lo(braw[0]) * w0[0], bf16_hi(braw[0]) * w0[1]);
                    af[1] = pack_bf16x2(bf16_lo(braw[1]) * w0[2], bf16_hi(braw[1]) * w0[3]);
                    af[2] = pack_bf16x2(bf16_lo(braw[2]) * w1[0], bf16_hi(braw[2]) * w1[1]);
                    af[3] = pack_bf16x2(bf16_lo(braw[3]) * w1[2], bf16_hi(braw[3]) * w1[3]);
                    if (jb + kRing < NB)
                        btr[slot] = ldg_b128(btc + bt_lane + 64 * (jb + kRing));
                    else if (more)
                        btr[slot] = ldg_b128(btn + bt_lane + 64 * slot);
#pragma unroll
                    for (int j = 0; j < NPW; ++j) hacc[j] = fu_mfma(af, xf[pt0 + j], hacc[j]);
                }
                if constexpr (OUT) {
                    if (has_out) {
                        auto tile_block = [&](f32x4 (&acc)[NPTW], const u32x4 cw, int it, int jd) {
                            if (jb < jd) {
                                const float qv = Qt[jb];
                                const int j0 = 32 * jb + 8 * kg;
                                const f32x4 c0 = *reinterpret_cast<const f32x4*>(Cf + j0);
                                const f32x4 c1 = *reinterpret_cast<const f32x4*>(Cf + j0 + 4);
                                u32x4 wf;
                                wf[0] = pack_bf16x2(bf16_lo(cw[0]) * c0[0], bf16_hi(cw[0]) * c0[1]);
                                wf[1] = pack_bf16x2(bf16_lo(cw[1]) * c0[2], bf16_hi(cw[1]) * c0[3]);
                                wf[2] = pack_bf16x2(bf16_lo(cw[2]) * c1[0], bf16_hi(cw[2]) * c1[1]);
                                wf[3] = pack_bf16x2(bf16_lo(cw[3]) * c1[2], bf16_hi(cw[3]) * c1[3]);
#pragma unroll
                                for (int q = 0; q < NPTW; ++q) acc[q] = fu_mfma(xf[ptb + q], wf, acc[q] * qv);
                            } else {
                                // jb == jd: bring the accumulator from the last block end to
                                // row i, then the diagonal block: element-wise decay, mask
                                // and skip term
                                const int i = 16 * it + l16;
                                const float gi = Gt[i];
                                const float gref = jd == 0 ? 0.0f : Gt[32 * jd - 1];
                                const float ri = fexp2(gi - gref);
                                const int j0 = 32 * jd + 8 * kg;
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
#pragma unroll
                                for (int q = 0; q < NPTW; ++q) acc[q] = fu_mfma(xf[ptb + q], wf, acc[q] * ri);
                            }
                        };
                        if (jb <= jdA) {
                            const u32x4 cw = rA[slot];
                            if (jb + kRing <= jdA)
                                rA[slot] = ldg_b128(cbc + cbA_lane + 64 * (jb + kRing));
                            else if (more)
                                rA[slot] = ldg_b128(cbn + cbA_lane + 64 * slot);
                            tile_block(accA, cw, itA, jdA);
                        }
                        if (jb <= jdB) {
                            const u32x4 cw = rB[slot];
                            if (jb + kRing <= jdB)
                                rB[slot] = ldg_b128(cbc + cbB_lane + 64 * (jb + kRing));
                            else if (more)
                                rB[slot] = ldg_b128(cbn + cbB_lane + 64 * slot);
                            tile_block(accB, cw, itB, jdB);
                        }
                    }
                }
            }

            if constexpr (OUT) {
                if (has_out) {
                    auto store_y = [&](const f32x4 (&acc)[NPTW], int it) {
                        const int i = 16 * it + l16;
                        if (i < n) {
                            uint16_t* dst = p.y + ((b * L + tok0 + i) * p.H + h) * kFuP + 16 * ptb + 4 * kg;
#pragma unroll
                            for (int q = 0; q < NPTW; ++q) {
                                u32x2 v;
                                v[0] = pack_bf16x2(acc[q][0], acc[q][1]);
                                v[1] = pack_bf16x2(acc[q][2], acc[q][3]);
                                *reinterpret_cast<u32x2*>(dst + 16 * q) = v;
                            }
                        }
                    };
                    store_y(accA, itA);
                    store_y(accB, itB);
                }
            }
            lds_barrier();  // X, tables and the state rows are free
            if constexpr (OUT) store_hs();
        }
    };

    if (p.nsegs > 1) {
        // phase 1: this segment's own aggregate
#pragma unroll
        for (int j = 0; j < NPW; ++j) hacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        run_chunks(FuPhase<false>{});
        const float alpha_seg = fexp2(sumG);
        float* pay = p.payload + int64_t(tile) * 2 * (kFuThreads * Lay::NACC);
        float* pay_agg = pay + tid * Lay::NACC;
        float* pay_inc = pay + kFuThreads * Lay::NACC + tid * Lay::NACC;
        f32x4 hin[NPW];
        if (seg == 0) {
            load_h0(hin);
        } else {
            // publish the aggregate
#pragma unroll
            for (int j = 0; j < NPW; ++j) store_payload(pay_agg + 4 * j, hacc[j]);
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
                        const u32x4 stw = load_coherent_b128(p.status + int64_t(pred) * p.nchains + chain);
                        kind = int(stw[0]);
                        al = as_float(stw[1]);
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
            for (int j = 0; j < NPW; ++j) hin[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (kp >= 0) {
                const int base_seg = seg - 1 - kp;
                const int64_t tile_floats = 2 * (kFuThreads * Lay::NACC);
                if (base_seg >= 0) {
                    const float* src = p.payload + (int64_t(base_seg) * p.nchains + chain) * tile_floats +
                                       kFuThreads * Lay::NACC + tid * Lay::NACC;
#pragma unroll
                    for (int j = 0; j < NPW; ++j) hin[j] = load_payload(src + 4 * j);
                } else {
                    load_h0(hin);  // every predecessor was an aggregate: start from h0
                }
                for (int kk = kp - 1; kk >= 0; --kk) {
                    const float al = lb_alpha[kk];
                    const int sp = seg - 1 - kk;
                    const float* src = p.payload + (int64_t(sp) * p.nchains + chain) * tile_floats + tid * Lay::NACC;
#pragma unroll
                    for (int j = 0; j < NPW; ++j) hin[j] = hin[j] * al + load_payload(src + 4 * j);
                }
            }
        }
        // publish the inclusive state at the segment end
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            store_payload(pay_inc + 4 * j, hin[j] * alpha_seg + hacc[j]);
            hacc[j] = hin[j];
        }
        wait_vmem();
        __syncthreads();
        if (tid == 0) store_coherent_b128(p.status + tile, u32x4{2u, as_uint(alpha_seg), 0u, 0u});
    } else {
        load_h0(hacc);
    }
    store_hs();
    lds_barrier();
    run_chunks(FuPhase<true>{});
    if (p.h_final && seg == p.nsegs - 1) {
#pragma unroll
        for (int j = 0; j < NPW; ++j)
            *reinterpret_cast<f32x4*>(p.h_final + (bh * kFuP + 16 * (pt0 + j) + l16) * S + 16 * st + 4 * kg) = hacc[j];
    }
}

}  // namespace cls
