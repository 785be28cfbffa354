// Fused bf16 SSD forward pass on gfx950 for head dim 64: one workgroup walks
// a run of chunks of one (batch, head) with the state on chip.  A head of dim
// 128 runs as two heads of dim 64 (the recurrence is per channel), which share
// its dt, A and D.
//
// Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
// NVIDIA cuTile" (sections "Mamba-2 architecture", "Kernel 1/2/3"): per chunk
// the cumulative sum G of a_t = A dt_t, the output from the chunk-start state,
// the decayed intra-chunk product and the state jump
// h <- exp(G_last) h + X^T (dt exp(G_last - G) . B).  Across chunks the state
// follows the affine recurrence (a1, S1) then (a2, S2) = (a1 a2, a2 S1 + S2)
// of "Selective-scan CUDA kernels" (section "The problem") with a
// matrix-valued state, evaluated here as reduce-then-fold over segments.
//
// Work units.  A (batch, head) chain runs whole in one workgroup or, so that
// the last round of workgroups fills the CUs, as segments of chunks.  The
// aggregate launch computes, for pieces of every segment but a chain's last,
// the piece's state from zero S and its decay alpha = exp2(sum of the chunks'
// G_last).  The output launch runs the whole chains and the segments; a
// segment starts from h0 folded through the pieces before it, h <- alpha h + S.
//
// Wave roles.  Eight compute waves run the chunk's MFMA work.  Loader waves do
// the rest, one 32-token block each:
//   * prep loaders fetch the next chunk's X and dt, scan GL, and write the
//     per-token tables, the raw X tile, X~ and the diagonal-block weights;
//   * state loaders (output launch only) compute the chunk's state term C h^T
//     from the chunk-start state, and store the previous chunk's outputs.
// The output launch has 16 waves (8 + 4 + 4), the aggregate launch 12.
// Vector memory operations of a wave complete in issue order, so a wave that
// fetched X from HBM would wait out that latency before any later L2 operand;
// the compute waves only load L2-resident operands.  All waves meet at one
// barrier per chunk; inside a chunk the compute waves wait only for the state
// loaders' count.
//
// A chunk (TT tokens, padded to a multiple of 32) is handled as 32-token
// blocks.  With GL the cumulative sum of a_t inside its block (log2 units,
// <= 0) and every exponent formed <= 0 unless guarded:
//   * prep (loader waves, block by block): the wave scans GL, stores the
//     per-token tables and the block decay Q = exp2(GL_end), and writes the
//     raw X tile and X~[t] = dt_t exp2(GL_end - GL_t) X[t] (a factor <= dt_t)
//     to double LDS buffers;
//   * one pass over the blocks does the state jump (wave = state tile) and the
//     intra product of two 16-token output tiles per wave, paired (i, NIT-1-i)
//     so every wave has the same causal work.  Both use the X~ fragments of
//     the block (ds_read_b64_tr_b16, which transposes 4x16 blocks of 16-bit
//     values across a 16-lane group) and B^T or CB fragments; the decay
//     between blocks is a running rescale of the fp32 accumulators by Q, which
//     for the state also supplies exp2(G_last) h;
//   * the diagonal block of a tile uses raw X with weights CB dt exp2(GL_i -
//     GL_j) for j <= i and the skip term D on j = i.  When the block decays by
//     at most 2^100 they are split as exp2(GL_i) [CB dt_j exp2(-GL_j)], so only
//     per-token factors and one per-row scale are needed; stronger decay takes
//     the element-wise form.
//   * B^T, CB and (unless C is read from its rows) a copy of C come
//     fragment-major from the CB pass (a wave's operand fragment is 1 KB in
//     lane order); the compute waves fetch B^T and
//     CB fragments a chunk ahead into register rings.  Every ring slot is
//     refilled at every block (the address, not the load, depends on the
//     wave's causal extent), so no ring register is merged across branches,
//     which would force the load to complete on the spot.  y goes to LDS as
//     16-byte pieces assembled across lane rows with v_permlane16_swap, and
//     leaves for HBM as whole 128-byte rows from the state loaders.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "ssd_kernels.hpp"

namespace cls {

constexpr int kFuCompute = 512;                              // compute threads (8 waves)
constexpr int kFuWaves = kFuCompute / 64;                    // compute waves
constexpr int kFuLoaders = 4;                                // loader waves of one role
constexpr int kFuThreads = kFuCompute + 64 * kFuLoaders;     // workgroup size (aggregate launch)
constexpr int kFuThreadsOut = kFuThreads + 64 * kFuLoaders;  // output launch: + state-term loaders
constexpr int kFuP = 64;  // head dim of this kernel
constexpr uint32_t kFuSpinLimit = 1u << 24;  // bound of the compute waves' wait for the state term
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
// make every later LDS read wait for it; only loader waves issue it, and they
// wait for it with wait_vmcnt before touching the data.
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

// f(std::integral_constant<int, k>) for k = K .. N - 1, in order.
template <int K, int N, typename F>
__device__ __forceinline__ void fu_static_for(F&& f) {
    if constexpr (K < N) {
        f(std::integral_constant<int, K>{});
        fu_static_for<K + 1, N>(f);
    }
}

// v from the lane N below inside its 16-lane row, 0 for the first N lanes of
// the row (DPP row_shr).
template <int N>
__device__ __forceinline__ float fu_dpp_shr(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + N, 0xf, 0xf,
                                                                 false));
}

// lane 15 of each even row into every lane of the following row, 0 elsewhere
// (DPP row_bcast:15 on rows 1 and 3).
__device__ __forceinline__ float fu_dpp_bcast15(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf,
                                                                 false));
}

// LDS layout.  The aggregate launch (AGG) keeps only X~ and the tables, so two
// of its workgroups fit a CU.
template <int TT, int S, bool AGG = false>
struct FuLayout {
    static_assert(S == 64 || S == 128, "state size of the fused kernel");
    static_assert(TT >= 32 && TT <= 128 && TT % 32 == 0, "tile tokens");
    static constexpr int NST = S / 16;                    // state tiles (16 wide)
    static constexpr int NPW = (4 * NST) / kFuWaves;      // state head-dim tiles per wave
    static constexpr int NACC = NPW * 4;                  // state floats per lane
    static constexpr int NIT = TT / 16;                   // 16-token output tiles
    static constexpr int NPAIR = NIT / 2;                 // output tile pairs
    static constexpr int WPP = kFuWaves / NPAIR;          // waves per pair
    static constexpr int NPTW = WPP >= 4 ? 1 : 4 / WPP;   // output head-dim tiles per wave
    static constexpr int NB = TT / 32;                    // 32-token blocks
    static constexpr int NBL = (NB + kFuLoaders - 1) / kFuLoaders;  // blocks per loader wave (<= 2)
    static_assert(NBL <= 2, "a loader wave scans at most two blocks at once");
    static constexpr int XBYTES = TT * 128;               // X buffer [TT][64] bf16
    static constexpr int HP = S + 8;                      // bf16 pitch of the state rows
    static constexpr int HBYTES = kFuP * HP * 2;          // one state copy
    // per-chunk tables (floats): block-local cumulative decay GL, dt, the split
    // factor U = dt exp2(-GL), the row factor R = exp2(GL), and the block decays Q
    static constexpr int T_GL = 0, T_DT = TT, T_U = 2 * TT, T_R = 3 * TT, T_Q = 4 * TT;
    static constexpr int TFLOATS = 4 * TT + 16;
    // decay-weighted causal weights of the diagonal 32 x 32 blocks, as the MFMA
    // B fragments of the output tiles (1 KB per 16-token tile, lane-major)
    static constexpr int WBYTES = NIT * 1024;             // one chunk's weights
    static constexpr int RA = (NPAIR - 1) >> 1;           // off-diagonal blocks tile A can reach
    static constexpr int RB = NB - 1;                     // off-diagonal blocks tile B can reach
    static constexpr int X_OFF = 0;                                // 2 x raw X [TT][64] bf16, swizzled
    static constexpr int XT_OFF = AGG ? 0 : X_OFF + 2 * XBYTES;    // 2 x X~, same layout
    static constexpr int H_OFF = XT_OFF + 2 * XBYTES;              // [64][HP] bf16 chunk-start state
    // the state term of the chunk, fp32, one 1 KB block per (16-token tile, head-dim
    // tile) in the MFMA result layout
    static constexpr int YBYTES = NIT * 4 * 1024;
    static constexpr int Y_OFF = H_OFF + (AGG ? 0 : HBYTES);
    // the chunk's bf16 outputs [TT][64], staged for the loaders' stores; 16-byte piece
    // k of row r sits at k ^ (r & 7), so 8 rows written or read at once use every bank
    static constexpr int YO_OFF = Y_OFF + (AGG ? 0 : YBYTES);
    static constexpr int TB_OFF = YO_OFF + (AGG ? 0 : TT * 128);   // 2 x tables
    static constexpr int W_OFF = TB_OFF + 2 * TFLOATS * 4;         // 2 x diagonal weights
    static constexpr int MISC_OFF = W_OFF + (AGG ? 0 : 2 * WBYTES);  // ints [16]
    static constexpr int BYTES = MISC_OFF + 64;
    static_assert(BYTES <= 160 * 1024, "LDS of one workgroup");
};

// byte offset of (row t, 32-byte pair `pair`, byte `within` < 32) in X or X~.
// The pair is swizzled by rows t & 3 and t >> 3 & 3, so the 16 rows a
// transposed read touches (t = 8 kg + 0..3) fall on distinct 32-byte bank
// groups of the two row halves.
__device__ __forceinline__ uint32_t x_off(int t, int pair, int within) {
    return uint32_t(t * 128 + ((pair ^ (t & 3) ^ ((t >> 3) & 3)) << 5) + within);
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
// Tile of workgroup i among `n` work items that occupy workgroups
// [base, base + n).  Workgroups are dispatched to the XCDs round robin (XCD
// i % nx); the items are dealt so every XCD gets a contiguous range, i.e.
// neighbouring (batch, head) chains that share B and C stay in one L2.
__device__ __forceinline__ int fu_xcd_item(int i, int base, int n, int nx) {
    // the range's workgroups on XCD k are base + r_k + m nx, r_k = (k - base) mod nx
    const int x = i % nx;
    int start = 0;
    for (int k = 0; k < x; ++k) {
        const int r = ((k - base) % nx + nx) % nx;
        start += r < n ? (n - 1 - r) / nx + 1 : 0;
    }
    const int r = ((x - base) % nx + nx) % nx;
    return start + (i - base - r) / nx;
}

// Tagged status word of segment `item` of a look-back call: the call's epoch,
// the segment's index and its kind (1: its aggregate is published, 2: its
// inclusive prefix is).  A word left by another call, another shape or other
// data in the workspace never matches both the epoch and the index.
__device__ __forceinline__ uint64_t fu_seg_tag(uint32_t epoch, int item, uint32_t kind) {
    return (uint64_t(epoch) << 32) | (uint64_t(uint32_t(item)) << 2) | kind;
}

// Look-back over the earlier segments of a chain, on one 64-lane wave: lane l
// inspects segment seg - 1 - l (item - 1 - l).  It is anchored at the chain's
// first segment: it waits until segment 0 holds its inclusive prefix (which
// that segment publishes directly, from h0) and every segment in between holds
// its aggregate.  The fold over them then has one order whatever the timing
// (the page's tiles fold up to the nearest inclusive prefix they find, and the
// fp32 grouping follows the timing).  A chain has at most 64 segments, so one
// window reaches segment 0.  The wait is bounded; giving up raises the error
// word.
__device__ __forceinline__ void fu_segment_lookback(const SsdFusedParams& p, int item, int seg, uint32_t epoch,
                                                    int lane) {
    const int pred = seg - 1 - lane;
    const int it = item - 1 - lane;
    uint32_t spins = 0;
    while (true) {
        bool ready = true;
        if (pred >= 0) {
            const uint64_t w = __hip_atomic_load(p.seg_status + it, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t kind = (w & ~uint64_t(3)) == fu_seg_tag(epoch, it, 0) ? uint32_t(w & 3u) : 0u;
            ready = kind == (pred == 0 ? 2u : 1u);
        }
        if (__ballot(!ready) == 0) return;
        if (++spins > kFuSpinLimit) {
            if (lane == 0) atomic_add_u32(p.err, 1u);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Look-back stress (tests only): with a nonzero seed, about one segment in
// four sleeps a pseudo-random 0 .. 31 x 8K clocks before it publishes, so
// segments publish out of order.  Seed 0: no delay.
__device__ __forceinline__ void fu_stress_delay(uint32_t seed, int item) {
    if (seed == 0) return;
    uint32_t x = seed ^ (uint32_t(item) * 0x9E3779B1u);
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 12;
    x *= 0x297A2D39u;
    x ^= x >> 15;
    if ((x & 3u) != 0u) return;
    for (uint32_t k = (x >> 2) & 31u; k > 0; --k) __builtin_amdgcn_s_sleep(127);
}

// The inter-chunk state pass of a split chain's segment as a single-pass
// decoupled look-back ("Selective-scan CUDA kernels", section "The five
// kernels", levels 3 and 3b; the combine of section "The problem" with the
// matrix state of "Accelerating Mamba-2 ...", section "Kernel 2:
// fwd_pass_state"):
//   * every segment but a chain's last runs its chunks once without outputs
//     (the aggregate phase) and publishes its aggregate (alpha_k, S_k); the
//     first segment starts that phase from h0, so it publishes its inclusive
//     prefix P_0 directly;
//   * wave 0 looks back, anchored at the first segment (fu_segment_lookback);
//     all compute waves fold h <- alpha_i h + S_i over the aggregates after
//     P_0, which gives the state at the segment's start, in the same order on
//     every run.
// Payloads are written with agent-scope 64-bit stores, completed (vmcnt
// wait) and joined at a workgroup barrier before one thread writes the
// status word; readers take payloads only after they have seen the word.
// Each payload is written once per call (the first segment's inclusive prefix
// and the other segments' aggregates have separate slots), so a reader never
// races a rewrite.  On return the compute waves hold the state at the
// segment's start in hacc.
template <int TT, int S, typename HArr, typename LoadH0, typename RunPhase>
__device__ __forceinline__ void ssd_lookback_segment(const SsdFusedParams& p, int item, int seg, int nst, int wave,
                                                     int lane, int tid, bool loader, HArr& hacc, float& sumG,
                                                     int* lb_int, LoadH0& load_h0, RunPhase& run_phase) {
    using Lay = FuLayout<TT, S>;
    constexpr int NPW = Lay::NPW;
    constexpr int NACC = Lay::NACC;
    const uint32_t epoch = uint32_t(__builtin_amdgcn_readfirstlane(lb_int[5]));
    const bool last = seg == p.nsegs - 1;
    const int64_t slot = int64_t(kFuCompute) * NACC;
    float* payA = p.seg_pay;
    float* payP = p.seg_pay + int64_t(nst) * slot;
    uint32_t* alpha = reinterpret_cast<uint32_t*>(p.seg_alpha);
    if (!last) {
        if (!loader) {
            if (seg == 0) {
                load_h0(hacc);
            } else {
#pragma unroll
                for (int j = 0; j < NPW; ++j) hacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        run_phase(FuPhase<false>{});
        if (!loader) {
            float* dst = (seg == 0 ? payP : payA) + int64_t(item) * slot + tid * NACC;
#pragma unroll
            for (int j = 0; j < NPW; ++j) store_payload(dst + 4 * j, hacc[j]);
            if (tid == 0 && seg > 0) store_coherent_u32(alpha + item, as_uint(fexp2(sumG)));
            wait_vmem();
        }
        fu_stress_delay(p.stress, item);
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(p.seg_status + item, fu_seg_tag(epoch, item, seg == 0 ? 2u : 1u), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (seg == 0) {
        if (!loader) load_h0(hacc);  // the output pass starts from h0
        return;
    }
    if (wave == 0) fu_segment_lookback(p, item, seg, epoch, lane);
    __syncthreads();
    if (!loader) {
        const int base = item - seg;  // this chain's first segment
        const float* src = payP + int64_t(base) * slot + tid * NACC;
#pragma unroll
        for (int j = 0; j < NPW; ++j) hacc[j] = load_payload(src + 4 * j);
        for (int k = 1; k < seg; ++k) {
            const float al = as_float(load_coherent_u32(alpha + base + k));
            const float* a = payA + int64_t(base + k) * slot + tid * NACC;
#pragma unroll
            for (int j = 0; j < NPW; ++j) hacc[j] = hacc[j] * al + load_payload(a + 4 * j);
        }
    }
}

// AGG: the aggregate launch (one workgroup per segment of a split chain: its
// state from zero and its decay); otherwise the output launch (whole chains,
// then the segments of split chains from the folded aggregates).  NT: x is
// loaded and y stored non-temporally (each is touched once per launch), the
// plan's choice for long chains, where it measured 1-4 % faster; on short
// chains the default policy measured 4 % faster.
template <int TT, int S, bool AGG, bool LB = false, bool NT = false>
__device__ __forceinline__ void ssd_fused_body(const SsdFusedParams& p) {
    constexpr int kXyPolicy = NT ? 2 : 0;  // buffer-op cache policy of the x loads and y stores
    using Lay = FuLayout<TT, S, AGG>;
    constexpr int NPW = Lay::NPW;
    constexpr int NPTW = Lay::NPTW;
    constexpr int NB = Lay::NB;
    constexpr int KS = S / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches and bases
    const bool loader = wave >= kFuWaves;
    const bool sloader = !AGG && wave >= kFuWaves + kFuLoaders;    // state-term loader (output launch)
    const int lw = sloader ? wave - kFuWaves - kFuLoaders : wave - kFuWaves;  // loader's block
    const int l16 = lane & 15, kg = lane >> 4;
    // bf16 copy of the chunk-start state (one copy: the compute waves write the
    // next chunk's only after every loader has read this chunk's, see below)
    auto hs_buf = [&](int) { return reinterpret_cast<uint16_t*>(sm + Lay::H_OFF); };
    float* Ys = reinterpret_cast<float*>(sm + Lay::Y_OFF);
    // lb_int[2]: loader waves done with the state term (running count over the
    // output phase)
    int* lb_int = reinterpret_cast<int*>(sm + Lay::MISC_OFF);

    // state tile of this wave: s-tile st, head-dim tiles pt0 .. pt0 + NPW - 1
    const int st = wave % Lay::NST;
    const int pt0 = ((wave % kFuWaves) / Lay::NST) * NPW;
    // output tiles of this wave: 16-token tiles itA, itB, head-dim tiles ptb ..
    const int pair = wave % Lay::NPAIR;
    const int ptb = ((wave % kFuWaves) / Lay::NPAIR) * NPTW;
    const bool has_out = ptb < 4;
    const int itA = pair, itB = Lay::NIT - 1 - pair;
    const int jdA_w = itA >> 1, jdB_w = itB >> 1;

    // ---- the work item (workgroup-uniform: everything derived is scalar) ----
    // Output launch: workgroups [0, nwhole) run whole chains, the rest the
    // segments of the split chains; as workgroups start in index order, the
    // long whole chains go first.  Items are chain-major within each list.
    // Aggregate launch: piece m of segment seg (every segment but a chain's
    // last), chain-major, so a chain's pieces are consecutive payload slots.
    const int nsplit = p.nchains - p.nwhole;  // chains run as segments
    const int nst = p.nsegs * nsplit;         // segments
    const int npc = (p.nsegs - 1) * p.agg_d;  // aggregate pieces per split chain
    const int wg = blockIdx.x;
    bool split;
    int item, seg, chain, c_begin, c_end;
    if constexpr (AGG) {
        if (wg >= nsplit * npc) return;
        split = true;
        item = fu_xcd_item(wg, 0, nsplit * npc, p.nxcd);  // payload slot
        chain = p.nwhole + item / npc;
        seg = (item % npc) / p.agg_d;
        c_begin = seg * p.seg_chunks + (item % p.agg_d) * p.agg_chunks;
        const int seg_end = (seg + 1) * p.seg_chunks;
        c_end = c_begin + p.agg_chunks < seg_end ? c_begin + p.agg_chunks : seg_end;
    } else {
        if (wg >= p.nwhole + nst) return;
        split = wg >= p.nwhole;
        item = split ? fu_xcd_item(wg, p.nwhole, nst, p.nxcd) : fu_xcd_item(wg, 0, p.nwhole, p.nxcd);
        if (LB && split) {
            // The segment is claimed, not assigned: range r holds whole split
            // chains, its segments in chain order, so a segment's predecessors
            // hold smaller claims of the same counter and are already running
            // (or done) when it waits for them.  A workgroup starts at the range
            // of its XCD and moves on when that range is used up.
            if (tid == 0) {
                const int r0 = (wg % p.nxcd) % p.nranges;
                int got = -1;
                for (int k = 0; k < p.nranges && got < 0; ++k) {
                    const int r = (r0 + k) % p.nranges;
                    const int cb = int(int64_t(nsplit) * r / p.nranges);
                    const int ce = int(int64_t(nsplit) * (r + 1) / p.nranges);
                    const uint32_t t = atomic_add_u32(p.seg_ctl + 16 + r, 1u);
                    if (t < uint32_t((ce - cb) * p.nsegs)) got = cb * p.nsegs + int(t);
                }
                lb_int[4] = got;
                lb_int[5] = int(load_coherent_u32(p.seg_ctl));  // this call's epoch
            }
            __syncthreads();
            item = __builtin_amdgcn_readfirstlane(lb_int[4]);
            if (item < 0) item = 0;  // unreachable: the grid has one workgroup per segment
        }
        seg = split ? item % p.nsegs : 0;
        chain = split ? p.nwhole + item / p.nsegs : item;
        c_begin = split ? seg * p.seg_chunks : 0;
        c_end = (split && c_begin + p.seg_chunks < p.nchunks) ? c_begin + p.seg_chunks : p.nchunks;
    }
    if (tid == 0) lb_int[2] = 0;
    const int64_t b = chain / p.H;
    const int h = chain % p.H;
    const int g = h / (p.H / p.G);
    const int hin = h >> p.hshift;  // the input head (dt, A, D)
    const float A2 = p.A[hin] * kLog2e;
    const float Dh = p.D ? p.D[hin] : 0.0f;
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
    auto store_hs = [&](int c, int l16, int kg) {
        uint16_t* Hs = hs_buf(c);
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            u32x2 w;
            w[0] = pack_bf16x2(hacc[j][0], hacc[j][1]);
            w[1] = pack_bf16x2(hacc[j][2], hacc[j][3]);
            *reinterpret_cast<u32x2*>(Hs + (16 * (pt0 + j) + l16) * Lay::HP + 16 * st + 4 * kg) = w;
        }
    };

    auto chunk_rows = [&](int c) {
        const int64_t tok0 = int64_t(c) * p.chunk;
        return int((L - tok0 < p.chunk) ? (L - tok0) : p.chunk);
    };

    // =======================================================================
    // Loader waves.  Loader lw owns the 32-token block lw of every chunk (scan
    // lane = row of the block); its X lanes hold 8-row pieces of the block.
    // All loader loads are buffer loads whose range ends at the chunk's last
    // real row, so rows past a ragged end read as zeros.  They prepare chunk
    // c + 1 into the other half of the double-buffered X, X~ and tables while
    // the compute waves work on chunk c.
    // =======================================================================
    static_assert(Lay::NBL == 1, "one block per loader wave");
    const int64_t bcg0 = b * p.nchunks * p.G + g;    // (b, chunk 0, g) of the operands shared by a group
    auto cb_base = [&](int c) {
        return reinterpret_cast<const char*>(p.cb + (bcg0 + int64_t(c) * p.G) * (int64_t(TT) * TT));
    };

    const bool lblk = lw < NB;                       // this loader has a block
    const int lrow = 32 * lw + 8 * 0 + (lane >> 3);  // row of X piece m = 0 (+ 8 m)
    const uint32_t xrow_bytes = uint32_t(p.H * kFuP * 2);
    const uint32_t kNoRow = 0x7ffffff0u;             // offset past any range: reads zeros
    // diagonal C B^T block of the loader's block: the fragments (tile 2 lw + h,
    // block lw), h = 0, 1 (C B^T is stored fragment-major, see the CB pass)
    const uint32_t cboff = lblk ? uint32_t(((2 * lw * NB + lw) * 64 + lane) * 16) : kNoRow;
    uint32_t xoff[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        xoff[m] = lblk ? uint32_t(lrow + 8 * m) * xrow_bytes + uint32_t((lane & 7) * 16) : kNoRow;
    const uint32_t dtoff = (lblk && lane < 32) ? uint32_t(32 * lw + lane) * 4u : kNoRow;  // token-contiguous dt
    u32x4 cfr[2][KS];  // C^T fragments (MFMA B operand) of the loader's two 16-token tiles
    // X and dt of chunk c into the register set (xreg, dtv) (and, for the
    // output phase, the diagonal C B^T block of the loader's block)
    auto issue_x = [&](int c, auto out_tag, u32x4 (&xreg)[4], float& dtv, u32x4 (&dreg)[2]) {
        constexpr bool OUT = decltype(out_tag)::value;
        const int64_t tok0 = int64_t(c) * p.chunk;
        const int n = chunk_rows(c);
        const auto rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(p.x + ((b * L + tok0) * p.H + h) * kFuP), 0, int(uint32_t(n) * xrow_bytes), 0x00020000);
#pragma unroll
        for (int m = 0; m < 4; ++m) xreg[m] = __builtin_amdgcn_raw_buffer_load_b128(rx, int(xoff[m]), 0, kXyPolicy);
        // dt from the CB pass's token-contiguous copy (zeros past the last real row)
        const auto rd = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(p.dtt + ((b * p.nchunks + c) * (p.H >> p.hshift) + hin) * TT), 0, TT * 4, 0x00020000);
        dtv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, int(dtoff), 0, 0));
        if constexpr (OUT) {
            const auto rcb = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(cb_base(c)), 0, TT * TT * 2,
                                                               0x00020000);
            dreg[0] = __builtin_amdgcn_raw_buffer_load_b128(rcb, int(cboff), 0, 0);
            dreg[1] = __builtin_amdgcn_raw_buffer_load_b128(rcb, int(cboff + (lblk ? NB * 1024 : 0)), 0, 0);
        }
    };
    // GL scan, tables, raw X and X~ of the loader's block into buffers `buf`
    // (the aggregate phase needs only GL, the block decays and X~)
    float lgl = 0.0f, lge = 0.0f;  // the scan's GL (lanes < 32) and block-end GL, for the weights
    auto prep = [&](int buf, auto out_tag, const u32x4 (&xreg)[4], const float dtv) {
        constexpr bool OUT = decltype(out_tag)::value;
        float* T = reinterpret_cast<float*>(sm + Lay::TB_OFF) + buf * Lay::TFLOATS;
        unsigned char* Xr = sm + Lay::X_OFF + buf * Lay::XBYTES;
        unsigned char* Xt = sm + Lay::XT_OFF + buf * Lay::XBYTES;
        const int t = 32 * lw + (lane & 31);
        // inclusive scan over the 32 rows (lanes 0-31; lanes 32-63 carry zeros):
        // row shifts inside 16-lane rows, then lane 15 of row 0 into row 1
        float v = A2 * dtv;
        v += fu_dpp_shr<1>(v);
        v += fu_dpp_shr<2>(v);
        v += fu_dpp_shr<4>(v);
        v += fu_dpp_shr<8>(v);
        v += fu_dpp_bcast15(v);
        const float gl = v;                                  // GL_t <= 0
        const float ge = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
        lgl = gl;
        lge = ge;
        const float cf = dtv * fexp2(ge - gl);               // X~ factor, <= dt
        if (lblk && lane < 32) {
            T[Lay::T_GL + t] = gl;
            if constexpr (OUT) {
                const float e = fexp2(fminf(-gl, 126.0f));  // used only when the block decay is <= 2^100
                T[Lay::T_DT + t] = dtv;
                T[Lay::T_U + t] = dtv * e;
                T[Lay::T_R + t] = fexp2(gl);
            }
            if (lane == 0) T[Lay::T_Q + lw] = fexp2(ge);
        }
        float f[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) f[m] = __shfl(cf, 8 * m + (lane >> 3), 64);
        if (lblk) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int tr = lrow + 8 * m;
                const int cc = lane & 7;
                const uint32_t off = x_off(tr, cc >> 1, (cc & 1) * 16);
                const u32x4 xv = xreg[m];
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t word = xv[e];
                    w[e] = pack_bf16x2(bf16_lo(word) * f[m], bf16_hi(word) * f[m]);
                }
                if constexpr (OUT) *reinterpret_cast<u32x4*>(Xr + off) = xv;
                *reinterpret_cast<u32x4*>(Xt + off) = w;
            }
        }
    };
    auto prep_w = [&](int buf, const u32x4 (&dreg)[2]) {
        const float* T = reinterpret_cast<const float*>(sm + Lay::TB_OFF) + buf * Lay::TFLOATS;
        const float gl = lgl, ge = lge;
        // Diagonal-block weights W[r][j] = CB[r][j] dt_j exp2(GL_r - GL_j) for j <= r,
        // plus D on j = r (the skip term), rounded to bf16, as the MFMA B fragments of
        // the block's two 16-token tiles: for tile h the lane holds row r = 16 h + l16,
        // columns 8 kg + e.  Split as CB U_j R_r (bounded factors) unless the block
        // decays by more than 2^-100, where the exponent is formed per element.
        if (lblk) {
            unsigned char* Wb = sm + Lay::W_OFF + buf * Lay::WBYTES + 2 * lw * 1024;
            const int l16 = lane & 15, kg = lane >> 4, c0 = 8 * kg;
            const float* Tb = T + 32 * lw + c0;
            const bool split = fexp2(ge) >= kFuSplitMin;
            float a[8], gj[8];  // U_j (split) or dt_j, and GL_j
#pragma unroll
            for (int e4 = 0; e4 < 2; ++e4) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(Tb + (split ? Lay::T_U : Lay::T_DT) + 4 * e4);
                const f32x4 gv = *reinterpret_cast<const f32x4*>(Tb + Lay::T_GL + 4 * e4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[4 * e4 + e] = av[e];
                    gj[4 * e4 + e] = gv[e];
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int r = 16 * hh + l16;
                const float gr = __shfl(gl, r, 64);
                const float rr = fexp2(gr);
                float w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float cbv = (e & 1) ? bf16_hi(dreg[hh][e >> 1]) : bf16_lo(dreg[hh][e >> 1]);
                    const float v = split ? cbv * a[e] * rr : cbv * a[e] * fexp2(fminf(gr - gj[e], 0.0f));
                    const int jj = c0 + e;
                    w[e] = (jj < r) ? v : (jj == r ? v + Dh : 0.0f);
                }
                const u32x4 o = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                                 pack_bf16x2(w[6], w[7])};
                *reinterpret_cast<u32x4*>(Wb + hh * 1024 + lane * 16) = o;
            }
        }
    };
    // S4 state term y^T = H C^T of the loader's block (16-token tiles 2 lw and
    // 2 lw + 1, every head-dim tile) from the chunk-start state in LDS and C
    // fragments loaded straight from global memory.  The loaders compute it
    // while the compute waves run the chunk's block loop; the compute waves add
    // it, decayed to each row, once their block loop is done.
    // C fragments (fragment (tile, 32-state step): lane l16 + 16 kg holds row
    // l16 of the tile, states 32 step + 8 kg ..), from the CB pass's
    // fragment-major copy of the chunk's C rows (1 KB in lane order), or, when
    // there is no copy (p.cf null), from the C rows themselves (16 rows of 64
    // bytes) through a range that ends at the chunk's last real row.  Rows
    // past a ragged end are zeros either way.  Byte offset of fragment (it2,
    // ks): cf_lane + it2 * cf_it + ks * cf_ks.
    const bool c_copy = p.cf != nullptr;
    const uint32_t crow = uint32_t(p.G * S * 2);  // bytes between consecutive tokens of C
    const uint32_t cf_lane = !lblk ? kNoRow
                             : c_copy ? uint32_t((2 * lw * KS * 64 + lane) * 16)
                                      : uint32_t(32 * lw + (lane & 15)) * crow + uint32_t((lane >> 4) * 16);
    const uint32_t cf_it = c_copy ? uint32_t(KS * 1024) : 16 * crow;
    const uint32_t cf_ks = c_copy ? 1024u : 64u;
    auto issue_cf = [&](int c) {
        const auto rc =
            c_copy ? __builtin_amdgcn_make_buffer_rsrc(
                         const_cast<uint16_t*>(p.cf + (bcg0 + int64_t(c) * p.G) * (int64_t(TT) * S)), 0, TT * S * 2,
                         0x00020000)
                   : __builtin_amdgcn_make_buffer_rsrc(
                         const_cast<uint16_t*>(p.C + ((b * L + int64_t(c) * p.chunk) * p.G + g) * S), 0,
                         int(uint32_t(chunk_rows(c)) * crow), 0x00020000);
#pragma unroll
        for (int it2 = 0; it2 < 2; ++it2)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                cfr[it2][ks] = __builtin_amdgcn_raw_buffer_load_b128(rc, int(cf_lane + it2 * cf_it + ks * cf_ks), 0, 0);
    };
    // The outputs of a chunk, staged in LDS by the compute waves, are stored by
    // the loader waves during the next chunk, as whole 128-byte rows: 16-byte
    // pieces m = 0..3 of the loader's block (rows lrow + 8 m, the X piece layout),
    // through a buffer range that ends at the chunk's last real row.
    auto read_yo = [&](u32x4 (&yo)[4]) {
        const unsigned char* Yo = sm + Lay::YO_OFF;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = lrow + 8 * m, cc = lane & 7;
            yo[m] = *reinterpret_cast<const u32x4*>(Yo + r * 128 + ((cc ^ (r & 7)) << 4));
        }
    };
    auto y_rsrc = [&](int cy, int rows) {
        return __builtin_amdgcn_make_buffer_rsrc(p.y + ((b * L + int64_t(cy) * p.chunk) * p.H + h) * kFuP, 0,
                                                 int(uint32_t(rows) * xrow_bytes), 0x00020000);
    };
    // the state term of chunk c; the previous chunk's staged outputs are read
    // first (before the count that lets the compute waves overwrite them) and
    // stored one piece per 32-state step of the product, so the stores leave
    // under its LDS waits instead of in one burst that holds up the loads
    // issued after them
    auto ystate = [&](int c) {
        if (lblk) {
            u32x4 yo[4];
            read_yo(yo);
            const auto ry = y_rsrc(c > c_begin ? c - 1 : c, c > c_begin ? chunk_rows(c - 1) : 0);
            const int l16 = lane & 15, kg = lane >> 4;
            const uint16_t* Hs = hs_buf(c);
            f32x4 y[2][4];
#pragma unroll
            for (int it2 = 0; it2 < 2; ++it2)
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) y[it2][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const u32x4 hf =
                        *reinterpret_cast<const u32x4*>(Hs + (16 * pt + l16) * Lay::HP + 32 * ks + 8 * kg);
                    y[0][pt] = fu_mfma(hf, cfr[0][ks], y[0][pt]);
                    y[1][pt] = fu_mfma(hf, cfr[1][ks], y[1][pt]);
                }
#pragma unroll
                for (int m = ks * 4 / KS; m < (ks + 1) * 4 / KS; ++m)
                    __builtin_amdgcn_raw_buffer_store_b128(yo[m], ry, int(xoff[m]), 0, kXyPolicy);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int it2 = 0; it2 < 2; ++it2)
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    *reinterpret_cast<f32x4*>(Ys + (((2 * lw + it2) * 4 + pt) * 64 + lane) * 4) = y[it2][pt];
            // written (LDS operations of a wave complete in order): publish
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0) __hip_atomic_fetch_add(lb_int + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    };
    // The prep loaders' share of a phase, with the same barriers as the compute
    // waves (one per chunk).  X, dt and (output phase) the diagonal C B^T
    // fragments are fetched D = 2 chunks ahead into a ring of two register
    // sets: a load issued at the end of a chunk's preparation is consumed two
    // barriers later.  With one set it would be consumed right after the next
    // barrier, and its HBM latency would sit on the loaders' path.  Each
    // register set is consumed before it is refilled, with the scheduler kept
    // from hoisting the refill: a load issued while the old value is live
    // would land in other registers and be copied back at the loop edge, which
    // waits for the load to complete.  Loads are issued unconditionally (past
    // the last chunk the last one is reloaded and prepared into the free buffer
    // half) so no register is merged across branches.
    auto run_loader = [&](auto out_tag) {
        constexpr bool OUT = decltype(out_tag)::value;
        constexpr int D = 2;
        if (c_begin >= c_end) return;
        const int last = c_end - 1;
        auto clampc = [&](int c) { return c <= last ? c : last; };
        u32x4 xreg[D][4];  // chunk j in set (j - c_begin) % D
        float dtv[D];
        u32x4 dreg[D][2];  // (output phase) its diagonal C B^T fragments
        fu_static_for<0, D>([&](auto sc) {
            constexpr int sl = decltype(sc)::value;
            issue_x(clampc(c_begin + sl), out_tag, xreg[sl], dtv[sl], dreg[sl]);
        });
        prep(c_begin & 1, out_tag, xreg[0], dtv[0]);
        if constexpr (OUT) prep_w(c_begin & 1, dreg[0]);
        __builtin_amdgcn_sched_barrier(0);
        issue_x(clampc(c_begin + D), out_tag, xreg[0], dtv[0], dreg[0]);
        lds_barrier();
        // chunk c + 1 into the half chunk c - 1 used (free since the last barrier)
        auto step = [&](auto kc, int c) {
            constexpr int sl = (decltype(kc)::value + 1) % D;  // set of chunk c + 1
            prep((c + 1) & 1, out_tag, xreg[sl], dtv[sl]);
            if constexpr (OUT) prep_w((c + 1) & 1, dreg[sl]);
            __builtin_amdgcn_sched_barrier(0);
            issue_x(clampc(c + 1 + D), out_tag, xreg[sl], dtv[sl], dreg[sl]);
            lds_barrier();  // chunk c + 1 ready; chunk c's half free
            __builtin_amdgcn_sched_barrier(0);  // the next step's waits stay after the barrier
        };
        // unrolled by D so the sets are static registers, with the loop's only
        // exit at its end and the remainder after it: the loop head then sees
        // the loads in one issue order on every path
        static_assert(D == 1 || D == 2, "register sets");
        const int nrounds = (c_end - c_begin) / D;
        int c = c_begin;
        for (int i = 0; i < nrounds; ++i) {
            step(std::integral_constant<int, 0>{}, c);
            if constexpr (D == 2) step(std::integral_constant<int, 1>{}, c + 1);
            c += D;
        }
        if constexpr (D == 2) {
            if (c < c_end) step(std::integral_constant<int, 0>{}, c);
        }
    };

    // The state loaders' share of the output phase: the state term of chunk c
    // (which also stores chunk c - 1's outputs), then the C fragments of chunk
    // c + 1, with the same barriers as every other wave (one per chunk).
    auto run_state_loader = [&]() {
        if (c_begin >= c_end) return;
        const int last = c_end - 1;
        issue_cf(c_begin);
        lds_barrier();
        for (int c = c_begin; c < c_end; ++c) {
            ystate(c);
            __builtin_amdgcn_sched_barrier(0);
            issue_cf(c + 1 <= last ? c + 1 : last);
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        constexpr bool OUT = true;
        if constexpr (OUT) {
            if (lblk) {  // the last chunk's outputs
                u32x4 yo[4];
                read_yo(yo);
                const auto ry = y_rsrc(last, chunk_rows(last));
#pragma unroll
                for (int m = 0; m < 4; ++m) __builtin_amdgcn_raw_buffer_store_b128(yo[m], ry, int(xoff[m]), 0, kXyPolicy);
            }
        }
    };

    // =======================================================================
    // Compute waves: operands shared by the heads of a group live per
    // (b, chunk, g); lane offsets are 32-bit.
    // =======================================================================
    auto bt_base = [&](int c) {
        return reinterpret_cast<const char*>(p.bt + (bcg0 + int64_t(c) * p.G) * (int64_t(S) * TT));
    };
    // B^T and C B^T are stored fragment-major (the CB pass): fragment (tile, block)
    // is 64 lanes x 16 bytes, so a wave's fragment load reads 1 KB in lane order
    const uint32_t bt_lane = uint32_t((st * NB * 64 + lane) * 16);
    const uint32_t cbA_lane = uint32_t((itA * NB * 64 + lane) * 16);
    const uint32_t cbB_lane = uint32_t((itB * NB * 64 + lane) * 16);

    // Operand rings (the block loop is unrolled, so slots are static registers):
    // slot k holds block k of the current chunk.  When block k is consumed its
    // slot is refilled, always, with block k of the next chunk (of the same
    // chunk after the last one: a harmless reload), so every fragment is
    // fetched a whole chunk ahead.  A slot beyond the wave's causal extent is
    // reloaded every chunk and never read.
    constexpr int RA = Lay::RA, RB = Lay::RB;
    // CB fragment of chunk c at byte offset off (kNoRow: a slot past the wave's
    // causal extent, read as zeros without touching memory)
    auto cb_load = [&](int c, uint32_t off) {
        const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(cb_base(c)), 0, TT * TT * 2, 0x00020000);
        return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
    };
    u32x4 btr[NB];                                  // B^T fragments (state product)
    u32x4 rA[RA > 0 ? RA : 1], rB[RB > 0 ? RB : 1];  // off-diagonal CB fragments of the output tiles
    float sumG = 0.0f;

    // The compute waves wait for the loaders' state term of a chunk (a running
    // count of the loader waves that have written theirs).  The wait is
    // bounded; running out of it is reported in the error word.
    auto wait_ystate = [&](int target) {
        uint32_t spins = 0;
        while (__hip_atomic_load(lb_int + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
            if (++spins > kFuSpinLimit) {
                if (lane == 0) atomic_add_u32(p.err, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    };
    auto run_chunks = [&](auto out_tag, auto pt0_c, auto ptb_c) {
        constexpr bool OUT = decltype(out_tag)::value;
        constexpr int PT0 = decltype(pt0_c)::value * NPW;
        constexpr int PTB = decltype(ptb_c)::value * NPTW;
        if (c_begin >= c_end) return;
        // prologue: the first chunk's operand rings (the loaders prepare its X and C)
#pragma unroll
        for (int k = 0; k < NB; ++k) btr[k] = ldg_b128(bt_base(c_begin) + bt_lane + 1024 * k);
        if (OUT && has_out) {
#pragma unroll
            for (int k = 0; k < RA; ++k) rA[k] = cb_load(c_begin, k < jdA_w ? cbA_lane + 1024 * k : kNoRow);
#pragma unroll
            for (int k = 0; k < RB; ++k) rB[k] = cb_load(c_begin, k < jdB_w ? cbB_lane + 1024 * k : kNoRow);
        }
        lds_barrier();  // the loaders have prepared the first chunk

        for (int c = c_begin; c < c_end; ++c) {
            // Lane-dependent offsets are rebuilt every chunk from an opaque copy of
            // the lane id: hoisted out of the chunk loop they would each hold a
            // register for the whole loop.
            int lane_c = lane;
            asm volatile("" : "+v"(lane_c));
            const int l16 = lane_c & 15, kg = lane_c >> 4;
            // likewise the wave's causal extents, so the per-block branch
            // conditions are formed where they are used
            int jdA = jdA_w, jdB = jdB_w;
            asm volatile("" : "+s"(jdA), "+s"(jdB));
            const uint32_t bt_lane = uint32_t((st * NB * 64 + lane_c) * 16);
            const uint32_t cbA_lane = uint32_t((itA * NB * 64 + lane_c) * 16);
            const uint32_t cbB_lane = uint32_t((itB * NB * 64 + lane_c) * 16);
            const int64_t tok0 = int64_t(c) * p.chunk;
            const int n = chunk_rows(c);
            const int cx = c + 1 < c_end ? c + 1 : c;  // operand source of the refills for the next chunk
            // this chunk's half of the double-buffered X, X~ and tables
            const unsigned char* Xr = sm + Lay::X_OFF + (c & 1) * Lay::XBYTES;
            const unsigned char* Xt = sm + Lay::XT_OFF + (c & 1) * Lay::XBYTES;
            const float* T = reinterpret_cast<const float*>(sm + Lay::TB_OFF) + (c & 1) * Lay::TFLOATS;
            const unsigned char* Wb = sm + Lay::W_OFF + (c & 1) * Lay::WBYTES;
            const char* cbx = cb_base(cx);
            const char* btx = bt_base(cx);

            // intra-chunk outputs from zero; the state term is added after the
            // block loop
            f32x4 accA[NPTW], accB[NPTW];
            if constexpr (OUT) {
#pragma unroll
                for (int q = 0; q < NPTW; ++q) {
                    accA[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                    accB[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else {
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) sumG += T[Lay::T_GL + 32 * bb + 31];  // log2 decay of the chunk
            }

            // one pass over the 32-token blocks: S2c/S3 state jump, S2b intra product
            // X~ fragments are read one block ahead, so their LDS latency overlaps
            // the previous block's products
            auto load_xf = [&](u32x4 (&dst)[4], int trx) {
                fu_load_xf<0, PT0, NPW, PTB, NPTW, OUT>(dst, Xt, trx, l16);
                fu_load_xf<1, PT0, NPW, PTB, NPTW, OUT>(dst, Xt, trx, l16);
                fu_load_xf<2, PT0, NPW, PTB, NPTW, OUT>(dst, Xt, trx, l16);
                fu_load_xf<3, PT0, NPW, PTB, NPTW, OUT>(dst, Xt, trx, l16);
            };
            // X~ fragments XD blocks ahead (a ring of XD + 1 sets; the block loop is
            // unrolled, so the set indices are static) and all block decays at once.
            // Two blocks ahead measured no faster than one.  The output launch reads
            // them in the block itself: at 16 waves a wave has 128 registers, and the
            // prefetch set does not fit beside the operand rings.
            constexpr int XD = (OUT || LB) ? 0 : 1;
            u32x4 xs[XD + 1][4];
            fu_static_for<0, XD>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if constexpr (k < NB) load_xf(xs[k], 32 * k + 8 * kg + (l16 >> 2));
            });
            const f32x4 qall = *reinterpret_cast<const f32x4*>(T + Lay::T_Q);
            fu_static_for<0, NB>([&](auto jbc) {
                constexpr int jb = decltype(jbc)::value;
                const int trx = 32 * jb + 8 * kg + (l16 >> 2);
                if constexpr (jb + XD < NB) load_xf(xs[(jb + XD) % (XD + 1)], trx + 32 * XD);
                u32x4 (&xf)[4] = xs[jb % (XD + 1)];
                const float qv = qall[jb];
#pragma unroll
                for (int j = 0; j < NPW; ++j) hacc[j] = fu_mfma(btr[jb], xf[PT0 + j], hacc[j] * qv);
                if constexpr (OUT) {
                    if (has_out) {
                        // off-diagonal block: the accumulator moves to this block's end
                        auto tile_off = [&](f32x4 (&acc)[NPTW], const u32x4 cw) {
#pragma unroll
                            for (int q = 0; q < NPTW; ++q) acc[q] = fu_mfma(xf[PTB + q], cw, acc[q] * qv);
                        };
                        // diagonal block on raw X with the loaders' weights: the accumulator
                        // holds the contributions up to the block start, row i is exp2(GL_i)
                        // further on
                        auto tile_diag = [&](f32x4 (&acc)[NPTW], int it) {
                            const int i = 16 * it + l16;
                            const float ri = T[Lay::T_R + i];
                            const u32x4 wf = *reinterpret_cast<const u32x4*>(Wb + it * 1024 + lane_c * 16);
#pragma unroll
                            for (int q = 0; q < NPTW; ++q) {
                                const uint32_t o1 = x_off(trx, PTB + q, 8 * (l16 & 3));
                                acc[q] = fu_mfma(lds_tr_pair(Xr, o1, o1 + 512), wf, acc[q] * ri);
                            }
                        };
                        if constexpr (jb < RA) {
                            if (jb < jdA) tile_off(accA, rA[jb]);
                        }
                        if (jb == jdA) tile_diag(accA, itA);
                        if constexpr (jb < RB) {
                            if (jb < jdB) tile_off(accB, rB[jb]);
                        }
                        if (jb == jdB) tile_diag(accB, itB);
                    }
                }
                // refill the block's ring slots for the next chunk, after their last
                // use in this one (see the loader loop for why the order matters)
                __builtin_amdgcn_sched_barrier(0);
                btr[jb] = ldg_b128(btx + bt_lane + 1024 * jb);
                if constexpr (OUT) {
                    if (has_out) {
                        if constexpr (jb < RA) rA[jb] = cb_load(cx, jb < jdA ? cbA_lane + 1024 * jb : kNoRow);
                        if constexpr (jb < RB) rB[jb] = cb_load(cx, jb < jdB ? cbB_lane + 1024 * jb : kNoRow);
                    }
                }
            });

            if constexpr (OUT) {
                // every loader is done with this chunk's state copy and with the
                // previous chunk's staged outputs once it has published its state
                // term: the waves without outputs wait too, as they rewrite the copy
                wait_ystate(NB * (c - c_begin + 1));
                if (has_out) {
                    // S4: add the loaders' state term C_i h^T, decayed from the chunk
                    // start to row i: exp2 of the row's cumulative log decay, as the
                    // block decays before its block times exp2(GL_i)
                    auto add_state = [&](f32x4 (&acc)[NPTW], int it) {
                        const int i = 16 * it + l16;
                        float f = T[Lay::T_R + i];
                        for (int bb = 0; bb < (it >> 1); ++bb) f *= T[Lay::T_Q + bb];
#pragma unroll
                        for (int q = 0; q < NPTW; ++q)
                            acc[q] += *reinterpret_cast<const f32x4*>(Ys + ((it * 4 + PTB + q) * 64 + lane_c) * 4) * f;
                    };
                    add_state(accA, itA);
                    add_state(accB, itB);
                    // the bf16 outputs into the LDS stage the loaders store from
                    auto store_y = [&](const f32x4 (&acc)[NPTW], int it) {
                        const int i = 16 * it + l16;
                        unsigned char* yrow = sm + Lay::YO_OFF + i * 128;
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
                                const int e = 16 * (PTB + ((kg & 1) ? q + 1 : q)) + 8 * (kg >> 1);
                                *reinterpret_cast<u32x4*>(yrow + (((e >> 3) ^ (i & 7)) << 4)) =
                                    u32x4{s0[0], s1[0], s0[1], s1[1]};
                            }
                        } else {
                            const int e = 16 * PTB + 4 * kg;
                            *reinterpret_cast<u32x2*>(yrow + (((e >> 3) ^ (i & 7)) << 4) + (e & 7) * 2) = d[0];
                        }
                    };
                    store_y(accA, itA);
                    store_y(accB, itB);
                }
                store_hs(c + 1, l16, kg);
            }
            lds_barrier();  // the next chunk's state copy, X, X~ and tables are complete
        }
    };
    // the wave's head-dim offsets become compile-time constants (static register indices)
    auto run_phase = [&](auto out_tag) {
        if (loader) {
            // In the aggregate pass the loaders' work is on the path of every
            // (short) chunk: without a higher issue priority the compute waves
            // sharing their SIMD win every arbitration.  In the output pass a
            // raised priority only took issue slots from the compute waves
            // (measured 3 % slower).
            if constexpr (!decltype(out_tag)::value) __builtin_amdgcn_s_setprio(3);
            if constexpr (decltype(out_tag)::value) {
                if (sloader) {
                    run_state_loader();
                    return;
                }
            } else if constexpr (!AGG && LB) {
                // a segment's own aggregate inside the output launch: the state
                // loaders have nothing to do but meet the other waves' barriers
                // (one before the first chunk and one per chunk)
                if (sloader) {
                    for (int c = c_begin; c <= c_end && c_begin < c_end; ++c) lds_barrier();
                    __builtin_amdgcn_s_setprio(0);
                    return;
                }
            }
            run_loader(out_tag);
            if constexpr (!decltype(out_tag)::value) __builtin_amdgcn_s_setprio(0);
            return;
        }
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

    float* pay_alpha = p.payload + int64_t(nsplit) * npc * (kFuCompute * Lay::NACC);  // piece decays
    if constexpr (AGG) {
        // the piece's aggregate: its state from zero, and its decay
#pragma unroll
        for (int j = 0; j < NPW; ++j) hacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        run_phase(FuPhase<false>{});
        if (!loader) {
            float* pay = p.payload + int64_t(item) * (kFuCompute * Lay::NACC) + tid * Lay::NACC;
#pragma unroll
            for (int j = 0; j < NPW; ++j) *reinterpret_cast<f32x4*>(pay + 4 * j) = hacc[j];
        }
        if (tid == 0) pay_alpha[item] = fexp2(sumG);  // wave 0's (a compute wave)
        return;
    } else {
        if (LB && split) {
            // the state at the segment's start by look-back over the chain's
            // earlier segments (this segment's own aggregate published first)
            ssd_lookback_segment<TT, S>(p, item, seg, nst, wave, lane, tid, loader, hacc, sumG, lb_int,
                                        load_h0, run_phase);
        } else if (!loader) {
            load_h0(hacc);
            // a segment starts from h0 folded through the aggregates of the
            // pieces before it: h <- alpha_k h + S_k (the aggregate launch has
            // finished)
            for (int k = 0; k < seg * p.agg_d; ++k) {
                const int t = (chain - p.nwhole) * npc + k;
                const float al = pay_alpha[t];
                const float* src = p.payload + int64_t(t) * (kFuCompute * Lay::NACC) + tid * Lay::NACC;
#pragma unroll
                for (int j = 0; j < NPW; ++j) hacc[j] = hacc[j] * al + *reinterpret_cast<const f32x4*>(src + 4 * j);
            }
        }
        if (!loader) store_hs(c_begin, l16, kg);
        lds_barrier();
        run_phase(FuPhase<true>{});
        if (p.h_final && (!split || seg == p.nsegs - 1) && !loader) {
#pragma unroll
            for (int j = 0; j < NPW; ++j)
                *reinterpret_cast<f32x4*>(p.h_final + (bh * kFuP + 16 * (pt0 + j) + l16) * S + 16 * st + 4 * kg) =
                    hacc[j];
        }
        if (LB && split) {
            // The last segment to finish resets the claim counters and the
            // finish count and moves the epoch on, so the next call starts
            // clean without any clearing launch (every segment has done its
            // look-back reads before it counts itself finished).
            __syncthreads();
            if (tid == 0 && atomic_add_u32(p.seg_ctl + 1, 1u) == uint32_t(nst - 1)) {
                for (int r = 0; r < p.nranges; ++r) store_coherent_u32(p.seg_ctl + 16 + r, 0u);
                store_coherent_u32(p.seg_ctl + 1, 0u);
                store_coherent_u32(p.seg_ctl, uint32_t(lb_int[5]) + 1u);
            }
        }
    }
}

// The two launches: outputs (one workgroup per CU), and the aggregate pass
// of split chains (two workgroups per CU: it needs little LDS and few
// registers).
template <int TT, int S, bool NT = false>
__global__ __launch_bounds__(kFuThreadsOut) void ssd_fused_kernel(SsdFusedParams p) {
    ssd_fused_body<TT, S, false, false, NT>(p);
}

// The output launch of plans whose split chains pass state by look-back: the
// segments claim their work, run their own aggregate and look back (see
// ssd_lookback_segment); whole chains run as in ssd_fused_kernel.
template <int TT, int S, bool NT = false>
__global__ __launch_bounds__(kFuThreadsOut) void ssd_fused_lb_kernel(SsdFusedParams p) {
    ssd_fused_body<TT, S, false, true, NT>(p);
}

template <int TT, int S, bool NT = false>
__global__ __launch_bounds__(kFuThreads) __attribute__((amdgpu_waves_per_eu(6, 6))) void ssd_fused_agg_kernel(
    SsdFusedParams p) {
    ssd_fused_body<TT, S, true, false, NT>(p);
}

}  // namespace cls
