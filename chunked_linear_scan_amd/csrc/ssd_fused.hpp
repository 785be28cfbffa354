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
// A chunk (TT tokens, padded to a multiple of 32) is handled as 32-token
// blocks; wave b prepares block b of the NEXT chunk at the end of the current
// one, so no wave waits on another while a chunk computes except at two
// barriers (after the state term, at the end).  With GL the cumulative sum of
// a_t inside its block (log2 units, <= 0) and every exponent formed <= 0
// unless guarded:
//   * prep: the block's X arrives straight from global memory into a double
//     LDS buffer (global_load_lds_dwordx4), the wave scans GL, stores the
//     per-token tables and the block decay Q = exp2(GL_end), and writes
//     X~[t] = dt_t exp2(GL_end - GL_t) X[t] (a factor <= dt_t) to a second
//     double buffer;
//   * one pass over the blocks does the state jump (wave = state tile) and the
//     intra product of two 16-token output tiles per wave, paired (i, NIT-1-i)
//     so every wave has the same causal work.  Both use the X~ fragments of
//     the block (ds_read_b64_tr_b16, which transposes 4x16 blocks of 16-bit
//     values across a 16-lane group) and raw B^T or CB fragments; the decay
//     between blocks is a running rescale of the fp32 accumulators by Q, which
//     for the state also supplies exp2(G_last) h;
//   * the diagonal block of a tile uses raw X with weights CB dt exp2(GL_i -
//     GL_j) for j <= i and the skip term D on j = i.  When the block decays by
//     at most 2^100 they are split as exp2(GL_i) [CB dt_j exp2(-GL_j)], so only
//     per-token factors and one per-row scale are needed; stronger decay takes
//     the element-wise form.
//   * B^T comes ready-made from the CB pass; B^T, CB and C fragments are fetched
//     a little ahead into small register rings; y leaves as 16-byte pieces
//     assembled across lane rows with v_permlane16_swap.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "ssd_kernels.hpp"

namespace cls {

constexpr int kFuThreads = 512;
constexpr int kFuWaves = kFuThreads / 64;
constexpr int kFuP = 64;  // head dim of this kernel
constexpr uint32_t kFuSpinLimit = 1u << 24;
constexpr float kFuSplitMin = 7.8886091e-31f;  // 2^-100: weakest block decay of the split diagonal form

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

// 16 bytes per lane from global memory straight into LDS at lds_wave + 16 lane
// (global_load_lds_dwordx4 with the wave-uniform LDS base in M0, which is
// restored afterwards).  Issued from inline assembly so the compiler does not
// make every later LDS read wait for it: readers wait with wait_vmcnt.  The
// compiler's own waits for loads issued before or after it stay correct, as
// vector memory operations complete in issue order (an unseen one only makes
// them wait longer).
__device__ __forceinline__ void load_to_lds(const void* src, unsigned char* lds_wave) {
    const uint32_t la = uint32_t(uintptr_t((__attribute__((address_space(3))) unsigned char*)lds_wave));
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(la)
        : "memory");
}

// s_waitcnt vmcnt(N): at most N vector memory operations of this wave are
// still outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// f(std::integral_constant<int, v>) for a wave-uniform v in [K, N).
template <int K, int N, typename F>
__device__ __forceinline__ void fu_static_switch(int v, F& f) {
    if constexpr (K < N) {
        if (v == K)
            f(std::integral_constant<int, K>{});
        else
            fu_static_switch<K + 1, N>(v, f);
    }
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
    static constexpr int NB = TT / 32;                    // 32-token blocks (wave b prepares block b)
    static constexpr int XBYTES = TT * 128;               // one X buffer [TT][64] bf16
    static constexpr int HP = S + 8;                      // bf16 pitch of the state rows
    // per-chunk tables (floats): block-local cumulative decay GL, dt, the split
    // factors U = dt exp2(-GL) and VD = D exp2(-GL), and the block decays Q
    static constexpr int T_GL = 0, T_DT = TT, T_U = 2 * TT, T_VD = 3 * TT, T_Q = 4 * TT;
    static constexpr int TFLOATS = 4 * TT + 16;
    static constexpr int X_OFF = 0;                       // 2 x raw X [TT][64] bf16, swizzled
    static constexpr int XT_OFF = X_OFF + 2 * XBYTES;     // 2 x X~, same layout
    static constexpr int H_OFF = XT_OFF + 2 * XBYTES;     // [64][HP] bf16
    static constexpr int TB_OFF = H_OFF + kFuP * HP * 2;  // 2 x tables
    static constexpr int MISC_OFF = TB_OFF + 2 * TFLOATS * 4;  // ints [4]
    static constexpr int ALPHA_OFF = MISC_OFF + 64;            // look-back decays [64]
    static constexpr int BYTES = ALPHA_OFF + 64 * 4;
};

// byte offset of (row t, 32-byte pair `pair`, byte `within` < 32) in X or X~
__device__ __forceinline__ uint32_t x_off(int t, int pair, int within) {
    return uint32_t(t * 128 + ((pair ^ (t & 3)) << 5) + within);
}

// X~ fragment of head-dim tile PT for this wave, when the state (tiles PT0 ..)
// or the outputs (tiles PTB ..) use it.
template <int PT, int PT0, int NPW, int PTB, int NPTW, bool OUT>
__device__ __forceinline__ void fu_load_xf(u32x4 (&xf)[4], const unsigned char* base, int trx, int l16) {
    if constexpr ((PT >= PT0 && PT < PT0 + NPW) || (OUT && PT >= PTB && PT < PTB + NPTW)) {
        const uint32_t o1 = x_off(trx, PT, 8 * (l16 & 3));
        xf[PT] = lds_tr_pair(base, o1, o1 + 512);
    }
}

template <bool OUT>
struct FuPhase {
    static constexpr bool value = OUT;
};

// ---------------------------------------------------------------------------
template <int TT, int S>
__global__ __launch_bounds__(kFuThreads) void ssd_fused_kernel(SsdFusedParams p) {
    using Lay = FuLayout<TT, S>;
    constexpr int NPW = Lay::NPW;
    constexpr int NPTW = Lay::NPTW;
    constexpr int NB = Lay::NB;
    constexpr int KS = S / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches and bases
    const int l16 = lane & 15, kg = lane >> 4;
    uint16_t* Hs = reinterpret_cast<uint16_t*>(sm + Lay::H_OFF);
    int* lb_int = reinterpret_cast<int*>(sm + Lay::MISC_OFF);
    float* lb_alpha = reinterpret_cast<float*>(sm + Lay::ALPHA_OFF);
    auto tables = [&](int buf) { return reinterpret_cast<float*>(sm + Lay::TB_OFF) + buf * Lay::TFLOATS; };

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
    const int tile = __builtin_amdgcn_readfirstlane(lb_int[0]);  // uniform: everything derived is scalar
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
    // X rows of this wave's block of chunk c into raw buffer `buf` (waves < NB):
    // 4 pieces of 8 rows; lane i of a piece fills LDS bytes 16 i .. 16 i + 15,
    // so it loads the 16 bytes of the logical row and column that the swizzle
    // places there.  Rows past the chunk load a real row of it (finite values;
    // their weights are zero).
    auto issue_x = [&](int c, int buf) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = chunk_rows(c);
        const char* base = reinterpret_cast<const char*>(p.x + ((b * L + tok0) * p.H + h) * kFuP);
        unsigned char* xb = sm + Lay::X_OFF + buf * Lay::XBYTES;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int piece = 4 * wave + m;
            const int t = 8 * piece + (lane >> 3);
            const int pc = lane & 7;                                    // 16-byte slot in the row
            const int cc = (((pc >> 1) ^ (t & 3)) << 1) | (pc & 1);     // logical 16-byte column
            const int tr = t < n ? t : n - 1;
            load_to_lds(base + uint32_t(tr) * uint32_t(p.H * kFuP * 2) + uint32_t(cc * 16), xb + piece * 1024);
        }
    };
    // dt of this wave's block of chunk c: lane l holds row 32 wave + l / 2
    auto fetch_dt = [&](int c) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = chunk_rows(c);
        const int t = 32 * wave + (lane >> 1);
        return t < n ? p.dt[(b * L + tok0 + t) * p.H + h] : 0.0f;
    };
    // Block preparation (wave b < NB, block b of chunk c): GL scan, tables, X~.
    auto prep = [&](float dtv, int buf) {
        const int r = lane >> 1;                       // row in the block
        const int t = 32 * wave + r;                   // row in the chunk
        float v = A2 * dtv;
#pragma unroll
        for (int d = 2; d < 64; d <<= 1) {             // inclusive scan over rows (lane pairs)
            const float o = __shfl_up(v, d, 64);
            if (lane >= d) v += o;
        }
        const float gl = v;                            // GL_t <= 0
        const float ge = __shfl(v, 63, 64);            // GL at the block end
        const float cf = dtv * fexp2(ge - gl);         // X~ factor, <= dt
        float* T = tables(buf);
        if ((lane & 1) == 0) {
            const float e = fexp2(fminf(-gl, 126.0f));  // used only when the block decay is <= 2^100
            T[Lay::T_GL + t] = gl;
            T[Lay::T_DT + t] = dtv;
            T[Lay::T_U + t] = dtv * e;
            T[Lay::T_VD + t] = Dh * e;
        }
        if (lane == 0) T[Lay::T_Q + wave] = fexp2(ge);
        const unsigned char* xr = sm + Lay::X_OFF + buf * Lay::XBYTES;
        unsigned char* xt = sm + Lay::XT_OFF + buf * Lay::XBYTES;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int cc = 4 * (lane & 1) + m;
            const uint32_t off = x_off(t, cc >> 1, (cc & 1) * 16);
            const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + off);
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(bf16_lo(xv[e]) * cf, bf16_hi(xv[e]) * cf);
            *reinterpret_cast<u32x4*>(xt + off) = w;
        }
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

    // Rings of kRing fragments (the block loop is unrolled, so slots are static
    // registers): block k of a chunk sits in slot k % kRing.  When
    // block k is consumed its slot is refilled with block k + kRing of the same
    // chunk or, past the tile's last block jd, with block k % kRing of the next.
    constexpr int kRing = 3;
    u32x4 btr[kRing];              // B^T fragments (state product)
    u32x4 rA[kRing], rB[kRing];    // CB fragments of the two output tiles
    u32x4 cA[KS], cB[KS];          // C fragments of the two output tiles
    float sumG = 0.0f;

    auto run_chunks = [&](auto out_tag, auto pt0_c, auto ptb_c) {
        constexpr bool OUT = decltype(out_tag)::value;
        constexpr int PT0 = decltype(pt0_c)::value * NPW;
        constexpr int PTB = decltype(ptb_c)::value * NPTW;
        if (c_begin >= c_end) return;
        // prologue: the first chunk's blocks, then the operand rings
        float dtn = 0.0f;
        if (wave < NB) {
            issue_x(c_begin, c_begin & 1);
            dtn = fetch_dt(c_begin);
        }
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
        if (wave < NB) {
            wait_vmcnt<0>();
            prep(dtn, c_begin & 1);
        }
        lds_barrier();

        for (int c = c_begin; c < c_end; ++c) {
            const int64_t tok0 = int64_t(c) * p.chunk;
            const int n = chunk_rows(c);
            const bool more = c + 1 < c_end;
            const int cn = c + 1;
            const int cur = c & 1, nxt = cur ^ 1;
            const char* cbc = cb_base(c);
            const char* cbn = cb_base(cn);
            const char* btc = bt_base(c);
            const char* btn = bt_base(cn);
            const unsigned char* Xr = sm + Lay::X_OFF + cur * Lay::XBYTES;
            const unsigned char* Xt = sm + Lay::XT_OFF + cur * Lay::XBYTES;
            const float* T = tables(cur);
            // next chunk's blocks: X straight into the other raw buffer (last read in
            // the previous chunk), dt into a register
            if (more && wave < NB) {
                issue_x(cn, nxt);
                dtn = fetch_dt(cn);
            }
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) sumG += T[Lay::T_GL + 32 * bb + 31];  // log2 decay of the chunk

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
                                Hs + (16 * (PTB + q) + l16) * Lay::HP + 32 * ks + 8 * kg);
                            accA[q] = fu_mfma(hf, cA[ks], accA[q]);
                            accB[q] = fu_mfma(hf, cB[ks], accB[q]);
                        }
                    }
                    if (more) {
                        fetch_c(cn, itA, cA);
                        fetch_c(cn, itB, cB);
                    }
                }
                lds_barrier();  // every wave has read the chunk-start state
            }

            // one pass over the 32-token blocks: S2c/S3 state jump, S2b intra product
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                const int slot = jb % kRing;
                const int trx = 32 * jb + 8 * kg + (l16 >> 2);
                u32x4 xf[4];
                fu_load_xf<0, PT0, NPW, PTB, NPTW, OUT>(xf, Xt, trx, l16);
                fu_load_xf<1, PT0, NPW, PTB, NPTW, OUT>(xf, Xt, trx, l16);
                fu_load_xf<2, PT0, NPW, PTB, NPTW, OUT>(xf, Xt, trx, l16);
                fu_load_xf<3, PT0, NPW, PTB, NPTW, OUT>(xf, Xt, trx, l16);
                const float qv = T[Lay::T_Q + jb];
                {
                    const u32x4 braw = btr[slot];
                    if (jb + kRing < NB)
                        btr[slot] = ldg_b128(btc + bt_lane + 64 * (jb + kRing));
                    else if (more)
                        btr[slot] = ldg_b128(btn + bt_lane + 64 * slot);
#pragma unroll
                    for (int j = 0; j < NPW; ++j) hacc[j] = fu_mfma(braw, xf[PT0 + j], hacc[j] * qv);
                }
                if constexpr (OUT) {
                    if (has_out) {
                        auto tile_block = [&](f32x4 (&acc)[NPTW], const u32x4 cw, int it, int jd) {
                            if (jb < jd) {
#pragma unroll
                                for (int q = 0; q < NPTW; ++q) acc[q] = fu_mfma(xf[PTB + q], cw, acc[q] * qv);
                                return;
                            }
                            // jb == jd: diagonal block on raw X.  The accumulator holds the
                            // contributions up to the previous block end; row i is exp2(GL_i)
                            // further on.
                            const int i = 16 * it + l16;
                            const int il = i & 31;                 // row in the block
                            const float gi = T[Lay::T_GL + i];
                            const float ri = fexp2(gi);
                            const int j0 = 32 * jd + 8 * kg;
                            // causal position of the lane's first column: element e is kept
                            // when e <= kd and is the diagonal when e == kd (kept opaque so
                            // the per-element lane masks are not held across chunks)
                            int kd = il - 8 * kg;
                            asm volatile("" : "+v"(kd));
                            u32x4 wf;
                            if (qv >= kFuSplitMin) {
                                // split form: CB dt_j exp2(-GL_j) (+ D exp2(-GL_i) on j = i), then ri
                                const f32x4 u0 = *reinterpret_cast<const f32x4*>(T + Lay::T_U + j0);
                                const f32x4 u1 = *reinterpret_cast<const f32x4*>(T + Lay::T_U + j0 + 4);
                                const float vd = T[Lay::T_VD + i];
                                float wv[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const uint32_t word = cw[e >> 1];
                                    const float cbv = (e & 1) ? bf16_hi(word) : bf16_lo(word);
                                    const float u = e < 4 ? u0[e] : u1[e - 4];
                                    float w = (e <= kd) ? cbv * u : 0.0f;
                                    wv[e] = (e == kd) ? w + vd : w;
                                }
#pragma unroll
                                for (int e = 0; e < 4; ++e) wf[e] = pack_bf16x2(wv[2 * e], wv[2 * e + 1]);
#pragma unroll
                                for (int q = 0; q < NPTW; ++q) {
                                    const uint32_t o1 = x_off(trx, PTB + q, 8 * (l16 & 3));
                                    acc[q] = fu_mfma(lds_tr_pair(Xr, o1, o1 + 512), wf, acc[q]) * ri;
                                }
                            } else {
                                // element-wise form
                                float wv[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const uint32_t word = cw[e >> 1];
                                    const float cbv = (e & 1) ? bf16_hi(word) : bf16_lo(word);
                                    const int j = j0 + e;
                                    float w = cbv * fexp2(gi - T[Lay::T_GL + j]) * T[Lay::T_DT + j];
                                    w = (e <= kd) ? w : 0.0f;
                                    wv[e] = (e == kd) ? w + Dh : w;
                                }
#pragma unroll
                                for (int e = 0; e < 4; ++e) wf[e] = pack_bf16x2(wv[2 * e], wv[2 * e + 1]);
#pragma unroll
                                for (int q = 0; q < NPTW; ++q) {
                                    const uint32_t o1 = x_off(trx, PTB + q, 8 * (l16 & 3));
                                    acc[q] = fu_mfma(lds_tr_pair(Xr, o1, o1 + 512), wf, acc[q] * ri);
                                }
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
                        uint16_t* row = p.y + ((b * L + tok0 + i) * p.H + h) * kFuP;
                        u32x2 d[NPTW];
#pragma unroll
                        for (int q = 0; q < NPTW; ++q) {
                            d[q][0] = pack_bf16x2(acc[q][0], acc[q][1]);
                            d[q][1] = pack_bf16x2(acc[q][2], acc[q][3]);
                        }
                        if constexpr (NPTW >= 2) {
                            // lane rows kg, kg ^ 1 trade halves: each lane then holds 8
                            // consecutive head-dim values of row i for one tile of each pair
#pragma unroll
                            for (int q = 0; q < NPTW; q += 2) {
                                const auto s0 = __builtin_amdgcn_permlane16_swap(d[q][0], d[q + 1][0], false, false);
                                const auto s1 = __builtin_amdgcn_permlane16_swap(d[q][1], d[q + 1][1], false, false);
                                const int pt = PTB + ((kg & 1) ? q + 1 : q);
                                if (i < n)
                                    *reinterpret_cast<u32x4*>(row + 16 * pt + 8 * (kg >> 1)) =
                                        u32x4{s0[0], s1[0], s0[1], s1[1]};
                            }
                        } else {
                            if (i < n) *reinterpret_cast<u32x2*>(row + 16 * PTB + 4 * kg) = d[0];
                        }
                    };
                    store_y(accA, itA);
                    store_y(accB, itB);
                }
                store_hs();  // every wave is past the state term (barrier above)
            }
            if (more && wave < NB) {
                wait_vmcnt<NB>();  // this wave's X pieces of the next chunk: the B^T refills came after them
                prep(dtn, nxt);
            }
            lds_barrier();  // next chunk's X~ and tables are complete; this chunk's buffers are free
        }
    };
    // the wave's head-dim offsets become compile-time constants (static register indices)
    auto run_phase = [&](auto out_tag) {
        auto with_pt0 = [&](auto pt0_c) {
            if constexpr (decltype(out_tag)::value) {
                auto with_ptb = [&](auto ptb_c) { run_chunks(out_tag, pt0_c, ptb_c); };
                fu_static_switch<0, 4 / NPTW>(has_out ? ptb / NPTW : 0, with_ptb);
            } else {
                run_chunks(out_tag, pt0_c, std::integral_constant<int, 0>{});
            }
        };
        fu_static_switch<0, 4 / NPW>(pt0 / NPW, with_pt0);
    };

    if (p.nsegs > 1) {
        // phase 1: this segment's own aggregate
#pragma unroll
        for (int j = 0; j < NPW; ++j) hacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        run_phase(FuPhase<false>{});
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
            const int kp = __builtin_amdgcn_readfirstlane(lb_int[1]);
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
    run_phase(FuPhase<true>{});
    if (p.h_final && seg == p.nsegs - 1) {
#pragma unroll
        for (int j = 0; j < NPW; ++j)
            *reinterpret_cast<f32x4*>(p.h_final + (bh * kFuP + 16 * (pt0 + j) + l16) * S + 16 * st + 4 * kg) = hacc[j];
    }
}

}  // namespace cls
