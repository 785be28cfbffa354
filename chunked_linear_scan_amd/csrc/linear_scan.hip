// Scalar linear recurrence h[t] = a[t] h[t-1] + b[t] on gfx950.
//
// The recurrence and its affine combine follow "Selective-scan CUDA kernels",
// section "The problem"; the single-pass scheme (tiles claimed in order from a
// counter, local aggregate published under flag A, look-back over a window of
// predecessors to an inclusive prefix P, items scanned serially in registers)
// follows its section "The five kernels" (levels 3b and 3c).  The look-back
// is anchored: only every 64th tile publishes an inclusive prefix, and a tile
// always folds from its anchor, so the combine order (and every bit of the
// result) does not depend on which predecessors happened to have published.
//
// MI355X choices:
//   * a tile is 4 waves x 2048 elements (the built-in choice; fp32 scans may
//     also run 1024 or 4096 per wave); each wave owns a contiguous run and
//     loads it as 16-byte vectors (4 fp32 or 8 bf16 items per lane) with
//     lanes 16 bytes apart, so every wave-wide load covers 1 KB of
//     consecutive memory; a 16-byte aligned
//     window makes rows that start misaligned (ragged lengths) use the same
//     vector loads; positions outside the row are the identity (a = 1, b = 0);
//   * the in-tile scan is a serial scan over each lane's items of a step, a
//     64-lane DPP wave scan per step (256 fp32 or 512 bf16 items) with the
//     step carry kept wave-uniform, and a 4-wave combine through LDS;
//   * one 64-lane wave inspects the tile's predecessors back to its anchor
//     (at most 63) in one step and folds the anchor's inclusive prefix and
//     the aggregates after it with a 6-step order-preserving tree reduction;
//   * rows are independent chains: tiles are claimed from one counter per row,
//     so claims never contend across rows and a row's chain never waits on
//     another row;
//   * the last tile of a row to finish (a per-row done counter, bumped after
//     the tile's stores) clears the row's status words and counters, so the
//     workspace is all-zero after every call and any later call, whatever its
//     shape and workspace layout, starts clean;
//   * a claimed index outside the row is treated as an empty tile, so even a
//     corrupted workspace can only produce wrong values and bounded waits,
//     never an out-of-range address;
//   * inputs are read with non-temporal loads (each is read once); fp32
//     outputs are stored with the default policy, 1-3 % faster than
//     non-temporal stores (measured), 16-bit outputs non-temporally;
//   * rows no longer than a tile are packed whole into tiles and scanned with a
//     row-start reset flag, with no look-back at all;
//   * a, b and h may each be fp32 or bf16: bf16 items are widened to fp32 at
//     the load and rounded to nearest even once at the store; the scan
//     itself is fp32 either way.
#include <type_traits>

#include "common.hpp"
#include "device_once.hpp"
#include "launch.hpp"

namespace cls {

constexpr int kLsThreads = 256;
constexpr int kLsWaves = kLsThreads / 64;
// Elements per wave (RUN) and per tile (4 RUN): 2048 / 8192 is the built-in
// choice for every element type; fp32 scans also have 1024 / 4096 and
// 4096 / 16384 instances, which the autotuner may pick per shape.
// Each look-back poll sleeps ~64 clocks; 2^24 polls is several seconds, far
// beyond any legitimate wait, so a corrupted workspace ends the kernel instead
// of hanging it (the error word is raised and the tile treats the missing
// predecessors as the identity).
constexpr uint32_t kLsSpinLimit = 1u << 24;

// An affine step h -> a h + b.  In segmented (packed-rows) mode `f` marks a
// run that contains a row start: such a run ignores whatever precedes it, so
// a NaN/Inf at the end of one row cannot leak into the next.
struct Pair {
    float a, b;
    int f;
};

// (first, then second): h -> s.a (f.a h + f.b) + s.b
__device__ __forceinline__ Pair combine(Pair f, Pair s) {
    if (s.f) return s;
    return Pair{f.a * s.a, fmaf(s.a, f.b, s.b), f.f};
}

// 16-bit element formats: raw bits, two to a 32-bit word (the earlier item in
// the low half).  Items are widened to fp32 exactly and results rounded to
// nearest even once.
struct bf16_t {
    uint16_t v;
};
struct f16_t {
    uint16_t v;
};
template <typename T>
struct Fmt16;
template <>
struct Fmt16<bf16_t> {
    static constexpr uint32_t one = 0x3f80u;  // 1.0
    __device__ static float lo(uint32_t w) { return bf16_lo(w); }
    __device__ static float hi(uint32_t w) { return bf16_hi(w); }
    __device__ static uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};
template <>
struct Fmt16<f16_t> {
    static constexpr uint32_t one = 0x3c00u;  // 1.0
    __device__ static float lo(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xffffu))); }
    __device__ static float hi(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16))); }
    // The fp32 values are pinned in registers first: otherwise the compiler
    // fuses the producing fma with the conversion (v_fma_mixlo_f16), which
    // rounds the exact product-sum to fp16 once instead of rounding the fp32
    // result, and differs from it at fp32 values that are exact fp16 ties.
    __device__ static uint32_t pack(float a, float b) {
        asm volatile("" : "+v"(a), "+v"(b));
        return uint32_t(__builtin_bit_cast(uint16_t, _Float16(a))) |
               (uint32_t(__builtin_bit_cast(uint16_t, _Float16(b))) << 16);
    }
};

// Items per lane and step: 4 fp32 (one 16-byte load) or 8 16-bit items (one
// 16-byte load), so every wave-wide load covers 1 KB of consecutive memory.
template <typename T>
struct ItemsPerLane {
    static constexpr int value = sizeof(T) == 2 ? 8 : 4;
};

// 16-byte vectors at 8-byte aligned addresses (bf16 rows start on a 4-item
// boundary).
typedef uint32_t u32x4a8 __attribute__((ext_vector_type(4), aligned(8)));
typedef uint32_t u32x2a8 __attribute__((ext_vector_type(2), aligned(8)));

// Items i .. i+N-1 of p; positions outside [lo, hi) read as `ident`.
__device__ __forceinline__ void load_items(const float* __restrict__ p, int64_t i, int64_t lo, int64_t hi,
                                           float ident, float (&v)[4]) {
    if (i >= lo && i + 4 <= hi) {
        const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i));
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = w[k];
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t e = i + k;
        v[k] = (e >= lo && e < hi) ? p[e] : ident;
    }
}

// Items i .. i+7 of p as raw 16-bit words, two per word (item 2k in the low
// half of word k); positions outside [lo, hi) hold `ident` (raw bits).
template <typename T>
__device__ __forceinline__ u32x4a8 load_raw8(const T* __restrict__ pt, int64_t i, int64_t lo, int64_t hi,
                                            uint32_t ident) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(pt);
    if (i >= lo && i + 8 <= hi) return __builtin_nontemporal_load(reinterpret_cast<const u32x4a8*>(p + i));
    u32x4a8 w{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t e = i + k;
        const uint32_t v = (e >= lo && e < hi) ? uint32_t(p[e]) : ident;
        w[k / 2] |= v << (16 * (k & 1));
    }
    return w;
}

template <typename T>
__device__ __forceinline__ float raw_item(const u32x4a8& w, int k) {
    return (k & 1) ? Fmt16<T>::hi(w[k / 2]) : Fmt16<T>::lo(w[k / 2]);
}

// Unchecked forms for tiles that lie wholly inside [lo, hi).
__device__ __forceinline__ void load_items_full(const float* __restrict__ p, int64_t i, float (&v)[4]) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i));
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = w[k];
}

// Stores items i .. i+N-1 that lie in [lo, hi).
template <int N>
__device__ __forceinline__ void store_items(float* __restrict__ p, int64_t i, int64_t lo, int64_t hi,
                                            const float (&v)[N], bool full = false) {
    if (full || (i >= lo && i + N <= hi)) {
#pragma unroll
        for (int c = 0; c < N; c += 4)
            *reinterpret_cast<f32x4*>(p + i + c) = f32x4{v[c], v[c + 1], v[c + 2], v[c + 3]};
        return;
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int64_t e = i + k;
        if (e >= lo && e < hi) p[e] = v[k];
    }
}

template <int N, typename T>
__device__ __forceinline__ void store_items(T* __restrict__ pt, int64_t i, int64_t lo, int64_t hi,
                                            const float (&v)[N], bool full = false) {
    uint16_t* p = reinterpret_cast<uint16_t*>(pt);
    uint32_t w[N / 2];
#pragma unroll
    for (int k = 0; k < N / 2; ++k) w[k] = Fmt16<T>::pack(v[2 * k], v[2 * k + 1]);
    if (full || (i >= lo && i + N <= hi)) {
        if constexpr (N == 8)
            __builtin_nontemporal_store(u32x4a8{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4a8*>(p + i));
        else
            __builtin_nontemporal_store(u32x2a8{w[0], w[1]}, reinterpret_cast<u32x2a8*>(p + i));
        return;
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int64_t e = i + k;
        if (e >= lo && e < hi) p[e] = uint16_t((w[k / 2] >> (16 * (k & 1))) & 0xffffu);
    }
}

// Status word of a tile: two 64-bit halves {kind, alpha} and {kind, beta},
// kind 1 for the tile's own aggregate and 2 for its inclusive prefix, which
// later overwrites the aggregate in place; 0 means not yet published.  Each
// half is stored and loaded as one aligned 64-bit access (single-copy atomic
// on this device), but the two halves are separate accesses: a reader may see
// one half of the aggregate and the other of the prefix, or one published
// half beside an unpublished one.  It takes the word only when both halves
// carry the same nonzero kind, and polls again otherwise.
struct Status {
    uint32_t kind;
    Pair v;
};

__device__ __forceinline__ void store_status(uint64_t* w, uint32_t kind, Pair v) {
    __hip_atomic_store(w, uint64_t(kind) | (uint64_t(as_uint(v.a)) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(w + 1, uint64_t(kind) | (uint64_t(as_uint(v.b)) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ Status load_status(const uint64_t* w) {
    const uint64_t lo = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t k0 = uint32_t(lo), k1 = uint32_t(hi);
    return Status{k0 == k1 ? k0 : 0u, Pair{as_float(uint32_t(lo >> 32)), as_float(uint32_t(hi >> 32)), 0}};
}

// DPP move of a float / int: lanes whose source lies outside the pattern (or
// whose row is not in ROWMASK) keep `old`.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xf,
                                                                 false));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWMASK, 0xf, false);
}

// One step of the 64-lane inclusive scan: combine with the value a DPP pattern
// brings from a lower lane (the identity where there is none).
template <int CTRL, int ROWMASK, bool SEG>
__device__ __forceinline__ Pair scan_step(Pair w) {
    const Pair o{dpp_f<CTRL, ROWMASK>(1.0f, w.a), dpp_f<CTRL, ROWMASK>(0.0f, w.b),
                 SEG ? dpp_i<CTRL, ROWMASK>(0, w.f) : 0};
    return combine(o, w);
}

// Inclusive scan over the 64 lanes of a wave in lane order: row shifts by 1, 2,
// 4, 8 inside each 16-lane row, then lane 15 of rows 0 and 2 into rows 1 and 3,
// then lane 31 into rows 2 and 3 (the gfx9 DPP row broadcasts).
template <bool SEG>
__device__ __forceinline__ Pair wave_inclusive_scan(Pair w) {
    w = scan_step<0x111, 0xf, SEG>(w);
    w = scan_step<0x112, 0xf, SEG>(w);
    w = scan_step<0x114, 0xf, SEG>(w);
    w = scan_step<0x118, 0xf, SEG>(w);
    w = scan_step<0x142, 0xa, SEG>(w);
    w = scan_step<0x143, 0xc, SEG>(w);
    return w;
}

// Tiles whose index in the row is a multiple of kLsAnchor are anchors: they
// publish only their inclusive prefix, every other tile only its aggregate.
constexpr int kLsAnchor = 64;

// Exclusive prefix of tile j > 0 of a row: the inclusive prefix of its anchor
// a = 64 floor((j - 1) / 64) followed by the aggregates of tiles a + 1 .. j - 1
// ("anchored" look-back).  The page's tiles take the nearest inclusive prefix
// they find, so the grouping of the combines, and the fp32 rounding, follows
// the timing; here the grouping depends on j alone, so every run gives the
// same bits.  The anchor is at most 63 tiles back: one 64-lane window (lane l
// reads tile j - 1 - l) always reaches it.  Runs on one full wave; every lane
// returns the same value.  status_row holds one status word (two 64-bit
// halves) per tile.
__device__ Pair lookback(const uint64_t* status_row, int j, uint32_t* err) {
    const int lane = lane_id();
    const int kp = (j - 1) % kLsAnchor;  // the anchor's lane
    const int p = j - 1 - lane;
    Pair v{1.0f, 0.0f, 0};
    uint32_t spins = 0;
    while (true) {
        bool ready = true;
        if (lane <= kp) {
            const Status w = load_status(status_row + 2 * int64_t(p));
            ready = w.kind == (lane == kp ? 2u : 1u);
            v = Pair{w.v.a, w.v.b, 0};
        }
        if (__ballot(!ready) == 0) break;
        if (++spins > kLsSpinLimit) {
            if (lane == 0) atomic_add_u32(err, 1u);
            return Pair{1.0f, 0.0f, 0};
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (lane > kp) v = Pair{1.0f, 0.0f, 0};
    // Ordered tree reduction: lane k ends up holding lanes [k, k+2d) with the
    // higher lane (the earlier tile) applied first.
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        Pair o{shfl_down(v.a, d), shfl_down(v.b, d), 0};
        if (lane + d >= 64) o = Pair{1.0f, 0.0f, 0};
        v = combine(o, v);
    }
    return Pair{bcast_lane0(v.a), bcast_lane0(v.b), 0};
}

// Look-back stress (tests only): with a nonzero seed, wave 0 of about one tile
// in four sleeps a pseudo-random 0 .. 31 x 8K clocks before it publishes and
// looks back, so tiles publish out of order.  Seed 0: no delay.
__device__ __forceinline__ void stress_delay(uint32_t seed, int64_t row, int j) {
    if (seed == 0) return;
    uint32_t x = seed ^ (uint32_t(row) * 0x9E3779B1u) ^ (uint32_t(j) * 0x85EBCA77u);
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 12;
    x *= 0x297A2D39u;
    x ^= x >> 15;
    if ((x & 3u) != 0u) return;
    for (uint32_t k = (x >> 2) & 31u; k > 0; --k) __builtin_amdgcn_s_sleep(127);
}

// One tile per workgroup.  SEGMENTED: tiles hold whole rows and reset at each
// row start (rows no longer than a tile); otherwise each tile belongs to one
// row and the row's tiles chain through the look-back.  TIn / TOut: float
// (fp32) or uint16_t (bf16 bits).
// Register-resident Hillis-Steele scan of one step's 64 x 4 items (item k of
// lane l is element 4 l + k): at distance d = 1, 2, 4, ..., 128 every element
// combines with the one d places before it, all at once (double-buffered),
// so after log2(256) = 8 rounds element i holds the inclusive prefix of
// elements 0..i.  O(n log n) combines, against the O(n) of the serial-items
// plus wave-scan form; items come from other lanes by shuffles.  x_f marks a
// row start (packed rows), carried by the combine.
template <bool SEGMENTED>
__device__ __forceinline__ void hillis_steele_step(float (&x_a)[4], float (&x_b)[4], int (&x_f)[4], int lane) {
#pragma unroll
    for (int d = 1; d < 256; d <<= 1) {
        float na[4], nb[4];
        int nf[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int off = d < 4 ? (k >= d ? 0 : 1) : d / 4;  // lanes back
            const int sk = d < 4 ? (k - d + 4) % 4 : k;        // item there
            Pair prev{x_a[sk], x_b[sk], SEGMENTED ? x_f[sk] : 0};
            bool valid = true;
            if (off > 0) {
                prev.a = shfl_up(prev.a, off);
                prev.b = shfl_up(prev.b, off);
                if (SEGMENTED) prev.f = shfl_up_i(prev.f, off);
                valid = lane >= off;
            }
            const Pair cur{x_a[k], x_b[k], SEGMENTED ? x_f[k] : 0};
            const Pair r = valid ? combine(prev, cur) : cur;
            na[k] = r.a;
            nb[k] = r.b;
            nf[k] = r.f;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x_a[k] = na[k];
            x_b[k] = nb[k];
            x_f[k] = nf[k];
        }
    }
}

// HS: the in-tile scan by Hillis-Steele rounds (fp32 items only) instead of
// serial items plus the wave scan; tiles, look-back and stores are shared.
template <bool SEGMENTED, typename TIn, typename TOut, bool HS = false, int RUN = 2048>
__global__ __launch_bounds__(kLsThreads) void linear_scan_kernel(
    const TIn* __restrict__ a, const TIn* __restrict__ b, TOut* __restrict__ h,
    int64_t rows, int64_t L, int tiles_per_row, int rows_per_tile,
    uint32_t* __restrict__ claim, uint32_t* __restrict__ done, uint64_t* __restrict__ status,
    uint32_t* __restrict__ err, uint32_t stress) {
    __shared__ uint32_t s_claim;
    __shared__ float s_wa[kLsWaves], s_wb[kLsWaves];
    __shared__ int s_wf[kLsWaves];
    __shared__ float s_pa, s_pb;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    int64_t lo, hi, row = 0;
    uint32_t cnt = 0;
    if (SEGMENTED) {
        const int64_t r0 = int64_t(blockIdx.x) * rows_per_tile;
        const int64_t r1 = (r0 + rows_per_tile < rows) ? r0 + rows_per_tile : rows;
        lo = r0 * L;
        hi = r1 * L;
    } else {
        row = blockIdx.x / tiles_per_row;
        if (tid == 0) s_claim = atomic_add_u32(&claim[row], 1u);
        __syncthreads();
        cnt = s_claim;
        lo = row * L;
        hi = lo + L;
    }
    const bool in_range = SEGMENTED || cnt < uint32_t(tiles_per_row);
    const int j = in_range ? int(cnt) : 0;
    constexpr int TILE = kLsWaves * RUN;
    const int64_t abase = (lo & ~int64_t(3)) + int64_t(j) * TILE;
    const bool empty_tile = !SEGMENTED && (!in_range || abase >= hi);
    constexpr int IPL = ItemsPerLane<TIn>::value;  // items per lane and step
    // An fp32 tile wholly inside its row (every tile but a row's first and
    // last, unless the row is tile-aligned) loads and stores without bounds
    // checks: 1-2 % faster for fp32, slower for bf16 items (measured), which
    // keep the checked form.
    const bool full = IPL == 4 && !empty_tile && abase >= lo && abase + TILE <= hi;
    constexpr int NS = RUN / (64 * IPL);             // steps per wave
    constexpr int STEP = 64 * IPL;                   // elements per wave step
    const int64_t wbase = abase + int64_t(wave) * RUN + IPL * lane;  // + STEP q

    // LS1: load every step's items; scan the items of each step serially.
    // fp32 items keep their running prefix (a-product, state) per item.  bf16
    // items stay packed as loaded (half the registers, so more workgroups fit
    // a CU): only each step's lane aggregate is kept, and the output reruns
    // the recurrence over the items from the state in front of them.
    constexpr bool PACKED = IPL == 8;
    float av[PACKED ? 1 : NS][IPL], bv[PACKED ? 1 : NS][IPL];
    u32x4a8 ra[PACKED ? NS : 1], rb[PACKED ? NS : 1];
    float la[NS], lb[NS];  // lane aggregate of each step's items
    // one bit per item of the lane (NS IPL of them)
    using Mask = std::conditional_t<(NS * IPL > 32), uint64_t, uint32_t>;
    Mask rmask = 0;  // bit IPL q + k: the run up to item k of step q holds a row start
    Mask smask = 0;  // bit IPL q + k: item k of step q starts a row (packed items)
    if constexpr (PACKED) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            constexpr uint32_t one = Fmt16<TIn>::one, one2 = one | (one << 16);
            ra[q] = empty_tile ? u32x4a8{one2, one2, one2, one2} : load_raw8(a, wbase + STEP * q, lo, hi, one);
            rb[q] = empty_tile ? u32x4a8{0u, 0u, 0u, 0u} : load_raw8(b, wbase + STEP * q, lo, hi, 0u);
        }
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int64_t t0 = wbase + STEP * q;
            int64_t ns = 0;
            if (SEGMENTED) ns = ((t0 + L - 1) / L) * L;  // first row start >= t0
            float A = 1.0f, Bs = 0.0f;
            int f = 0;
#pragma unroll
            for (int k = 0; k < IPL; ++k) {
                const float x = raw_item<TIn>(ra[q], k), y = raw_item<TIn>(rb[q], k);
                bool reset = false;
                if (SEGMENTED && t0 + k == ns && ns < hi) {
                    reset = true;
                    ns += L;
                }
                if (reset) {
                    A = x;
                    Bs = y;
                    f = 1;
                    smask |= Mask(1) << (IPL * q + k);
                } else {
                    Bs = fmaf(x, Bs, y);
                    A = A * x;
                }
            }
            la[q] = A;
            lb[q] = Bs;
            rmask |= Mask(f) << (IPL * q + IPL - 1);
        }
    } else {
        if (!empty_tile) {
            if (full) {
#pragma unroll
                for (int q = 0; q < NS; ++q) {
                    load_items_full(a, wbase + STEP * q, av[q]);
                    load_items_full(b, wbase + STEP * q, bv[q]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < NS; ++q) {
                    load_items(a, wbase + STEP * q, lo, hi, 1.0f, av[q]);
                    load_items(b, wbase + STEP * q, lo, hi, 0.0f, bv[q]);
                }
            }
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const int64_t t0 = wbase + STEP * q;
                int64_t ns = 0;
                if (SEGMENTED) ns = ((t0 + L - 1) / L) * L;  // first row start >= t0
                int f = 0;
                int hf[IPL];  // row start at this item (Hillis-Steele form)
#pragma unroll
                for (int k = 0; k < IPL; ++k) {
                    bool reset = false;
                    if (SEGMENTED && t0 + k == ns && ns < hi) {
                        reset = true;
                        ns += L;
                    }
                    hf[k] = reset ? 1 : 0;
                    if constexpr (!HS) {
                        if (k > 0 && !reset) {
                            bv[q][k] = fmaf(av[q][k], bv[q][k - 1], bv[q][k]);
                            av[q][k] = av[q][k - 1] * av[q][k];
                        }
                        f |= reset ? 1 : 0;
                        rmask |= Mask(f) << (IPL * q + k);
                    }
                }
                if constexpr (HS) {
                    // the step's inclusive prefixes; a prefix whose run holds a
                    // row start does not see what precedes the step
                    hillis_steele_step<SEGMENTED>(av[q], bv[q], hf, lane);
#pragma unroll
                    for (int k = 0; k < IPL; ++k) rmask |= Mask(hf[k] & 1) << (IPL * q + k);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < NS; ++q)
#pragma unroll
                for (int k = 0; k < IPL; ++k) {
                    av[q][k] = 1.0f;
                    bv[q][k] = 0.0f;
                }
        }
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            la[q] = av[q][IPL - 1];
            lb[q] = bv[q][IPL - 1];
        }
    }

    // LS2: per step, a 64-lane scan of the lane aggregates; the steps chain
    // through a wave-uniform carry.  pre[q] is the wave-local prefix in front
    // of this lane's items of step q.
    Pair pre[NS];
    Pair carry{1.0f, 0.0f, 0};
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        if constexpr (HS) {
            // items already hold the step's inclusive prefixes: only the carry
            // from earlier steps is in front of them; the step's total is the
            // last item of lane 63
            pre[q] = carry;
            const Pair tot{__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, la[q]), 63)),
                           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lb[q]), 63)),
                           SEGMENTED ? int(__builtin_amdgcn_readlane(int((rmask >> (IPL * q + IPL - 1)) & 1u), 63)) : 0};
            carry = combine(carry, tot);
            continue;
        }
        Pair w{la[q], lb[q], int((rmask >> (IPL * q + IPL - 1)) & 1u)};
        w = wave_inclusive_scan<SEGMENTED>(w);
        Pair ex{shfl_up(w.a, 1), shfl_up(w.b, 1), SEGMENTED ? shfl_up_i(w.f, 1) : 0};
        if (lane == 0) ex = Pair{1.0f, 0.0f, 0};
        pre[q] = combine(carry, ex);
        const Pair tot{__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w.a), 63)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w.b), 63)),
                       SEGMENTED ? __builtin_amdgcn_readlane(w.f, 63) : 0};
        carry = combine(carry, tot);
    }
    if (lane == 0) {
        s_wa[wave] = carry.a;
        s_wb[wave] = carry.b;
        s_wf[wave] = carry.f;
    }
    __syncthreads();
    Pair wave_excl{1.0f, 0.0f, 0};
    Pair tile_agg{1.0f, 0.0f, 0};
#pragma unroll
    for (int q = 0; q < kLsWaves; ++q) {
        const Pair s{s_wa[q], s_wb[q], s_wf[q]};
        if (q < wave) wave_excl = combine(wave_excl, s);
        tile_agg = combine(tile_agg, s);
    }

    // LS3: publish the aggregate (anchors: nothing yet), look back, and
    // (anchors only) publish the inclusive prefix.
    uint64_t* srow = status + 2 * row * int64_t(tiles_per_row);
    if (!SEGMENTED) {
        if (wave == 0) {
            Pair prefix{1.0f, 0.0f, 0};
            if (!empty_tile) {
                stress_delay(stress, row, j);
                const bool anchor = j % kLsAnchor == 0;
                if (j > 0) {
                    if (!anchor && lane == 0) store_status(srow + 2 * j, 1u, tile_agg);
                    prefix = lookback(srow, j, err);
                }
                if (anchor && lane == 0) store_status(srow + 2 * j, 2u, combine(prefix, tile_agg));
            }
            if (lane == 0) {
                s_pa = prefix.a;
                s_pb = prefix.b;
            }
        }
        __syncthreads();
    }

    // LS4: apply the prefix and store.  The state in front of a lane's items
    // is the b-part of the full prefix (the state before a row is 0); items
    // whose run already holds a row start do not see it.
    if (!empty_tile) {
        Pair tp = wave_excl;
        if (!SEGMENTED) tp = combine(Pair{s_pa, s_pb, 0}, tp);
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const float hin = combine(tp, pre[q]).b;
            float out[IPL];
            if constexpr (PACKED) {
                // An empty asm that claims to change the packed words keeps the
                // compiler from holding the items unpacked since the scan above
                // (which would cost the registers packing saves).
                u32x4a8 wa = ra[q], wb = rb[q];
                asm volatile("" : "+v"(wa), "+v"(wb));
                float st = hin;
#pragma unroll
                for (int k = 0; k < IPL; ++k) {
                    const float x = raw_item<TIn>(wa, k), y = raw_item<TIn>(wb, k);
                    const bool start = SEGMENTED && ((smask >> (IPL * q + k)) & 1u);
                    st = start ? y : fmaf(x, st, y);
                    out[k] = st;
                }
            } else {
#pragma unroll
                for (int k = 0; k < IPL; ++k) {
                    const bool own = SEGMENTED && ((rmask >> (IPL * q + k)) & 1u);
                    out[k] = own ? bv[q][k] : fmaf(av[q][k], hin, bv[q][k]);
                }
            }
            store_items(h, wbase + STEP * q, lo, hi, out, full);
        }
    }

    // The row's last finisher clears its status words and counters; every
    // tile of the row has finished its look-back before it counts itself done.
    if (!SEGMENTED && wave == 0) {
        uint32_t last = 0;
        if (lane == 0) last = (atomic_add_u32(&done[row], 1u) == uint32_t(tiles_per_row - 1)) ? 1u : 0u;
        last = __builtin_amdgcn_readfirstlane(last);
        if (last) {
            for (int q = lane; q < 2 * tiles_per_row; q += 64)
                __hip_atomic_store(srow + q, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane == 0) {
                store_coherent_u32(&claim[row], 0u);
                store_coherent_u32(&done[row], 0u);
            }
        }
    }
}

// Zero n16 16-byte words at p (a plain store kernel, so that a caller may
// capture it in a graph; memset nodes are avoided there).
__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* __restrict__ p, uint64_t n16) {
    for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += uint64_t(gridDim.x) * 256)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace cls

// The workspace of linear_scan_noalloc: a fixed array in device memory that
// each GPU holds for the life of the process (its address comes from
// hipGetSymbolAddress; in host code this name is not a device address).
static __device__ __align__(256) unsigned char scratch[CLS_NOALLOC_SCAN_SCRATCH_BYTES];

// Device address of this device's scratch array, looked up once per device.
extern "C" int cls_noalloc_scratch(void** ptr) {
    static cls::DeviceOnce once;
    static void* addr[cls::kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= cls::kMaxDevices) return -7;
    const int st = cls::run_once_per_device(once, [&] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -7;
        addr[dev] = p;
        return 0;
    });
    if (st != 0) return st;
    *ptr = addr[dev];
    return 0;
}

// Zero `bytes` (a multiple of 16) at p on `stream`.
extern "C" int cls_zero_fill(void* p, size_t bytes, hipStream_t stream) {
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    const uint64_t blocks = (n16 + 255) / 256;
    const dim3 grid{uint32_t(blocks < 1024 ? blocks : 1024), 1u, 1u};
    const dim3 block{256u, 1u, 1u};
    hipLaunchKernelGGL(cls::zero_fill_kernel, grid, block, 0, stream, static_cast<cls::u32x4*>(p), n16);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

namespace {

template <typename TIn, typename TOut, bool HS = false, int RUN = 2048>
void launch_typed(const void* a, const void* b, void* h, int64_t rows, int64_t L, int segmented, int tiles_per_row,
                  int rows_per_tile, int64_t ntiles, uint32_t* claim, uint32_t* done, void* status, uint32_t* err,
                  hipStream_t stream, uint32_t stress = 0) {
    using namespace cls;
    const dim3 grid{uint32_t(ntiles), 1u, 1u};
    const dim3 block{uint32_t(kLsThreads), 1u, 1u};
    const TIn* ta = static_cast<const TIn*>(a);
    const TIn* tb = static_cast<const TIn*>(b);
    TOut* th = static_cast<TOut*>(h);
    uint64_t* st = reinterpret_cast<uint64_t*>(status);
    if (segmented) {
        hipLaunchKernelGGL((linear_scan_kernel<true, TIn, TOut, HS, RUN>), grid, block, 0, stream, ta, tb, th, rows,
                           L, tiles_per_row, rows_per_tile, claim, done, st, err, stress);
    } else {
        hipLaunchKernelGGL((linear_scan_kernel<false, TIn, TOut, HS, RUN>), grid, block, 0, stream, ta, tb, th, rows,
                           L, tiles_per_row, rows_per_tile, claim, done, st, err, stress);
    }
}

template <typename TIn>
void launch_in(const void* a, const void* b, void* h, int64_t rows, int64_t L, int out_fmt, int segmented,
               int tiles_per_row, int rows_per_tile, int64_t ntiles, uint32_t* claim, uint32_t* done, void* status,
               uint32_t* err, hipStream_t stream) {
    using namespace cls;
    switch (out_fmt) {
        case 1:
            launch_typed<TIn, bf16_t>(a, b, h, rows, L, segmented, tiles_per_row, rows_per_tile, ntiles, claim, done,
                                      status, err, stream);
            break;
        case 2:
            launch_typed<TIn, f16_t>(a, b, h, rows, L, segmented, tiles_per_row, rows_per_tile, ntiles, claim, done,
                                     status, err, stream);
            break;
        default:
            launch_typed<TIn, float>(a, b, h, rows, L, segmented, tiles_per_row, rows_per_tile, ntiles, claim, done,
                                     status, err, stream);
    }
}

}  // namespace

// in_fmt / out_fmt: 0 fp32, 1 bf16, 2 fp16; hs: the Hillis-Steele in-tile
// scan (fp32 in and out only); tile: elements per tile, 8192, or 4096 or
// 16384 for fp32 in and out without hs (else -2); stress: look-back stress
// seed (fp32 in and out without hs only, else -2; 0: none).
extern "C" int cls_launch_linear_scan(const void* a, const void* b, void* h, int64_t rows, int64_t L,
                                      int in_fmt, int out_fmt, int segmented, int tiles_per_row, int rows_per_tile,
                                      int64_t ntiles, uint32_t* claim, uint32_t* done, void* status,
                                      uint32_t* err, hipStream_t stream, int hs, int tile, uint32_t stress) {
    using namespace cls;
    const bool f32 = in_fmt == 0 && out_fmt == 0;
    if (tile != 8192 && (!f32 || hs || (tile != 4096 && tile != 16384))) return -2;
    if (stress != 0 && (!f32 || hs)) return -2;
    if (hs) {
        launch_typed<float, float, true>(a, b, h, rows, L, segmented, tiles_per_row, rows_per_tile, ntiles, claim,
                                         done, status, err, stream);
        return hipGetLastError() == hipSuccess ? 0 : -7;
    }
    if (tile == 4096) {
        launch_typed<float, float, false, 1024>(a, b, h, rows, L, segmented, tiles_per_row, rows_per_tile, ntiles,
                                                claim, done, status, err, stream, stress);
        return hipGetLastError() == hipSuccess ? 0 : -7;
    }
    if (tile == 16384) {
        launch_typed<float, float, false, 4096>(a, b, h, rows, L, segmented, tiles_per_row, rows_per_tile, ntiles,
                                                claim, done, status, err, stream, stress);
        return hipGetLastError() == hipSuccess ? 0 : -7;
    }
    if (f32) {
        launch_typed<float, float>(a, b, h, rows, L, segmented, tiles_per_row, rows_per_tile, ntiles, claim, done,
                                   status, err, stream, stress);
        return hipGetLastError() == hipSuccess ? 0 : -7;
    }
    switch (in_fmt) {
        case 1:
            launch_in<bf16_t>(a, b, h, rows, L, out_fmt, segmented, tiles_per_row, rows_per_tile, ntiles, claim, done,
                              status, err, stream);
            break;
        case 2:
            launch_in<f16_t>(a, b, h, rows, L, out_fmt, segmented, tiles_per_row, rows_per_tile, ntiles, claim, done,
                             status, err, stream);
            break;
        default:
            launch_in<float>(a, b, h, rows, L, out_fmt, segmented, tiles_per_row, rows_per_tile, ntiles, claim, done,
                             status, err, stream);
    }
    return hipGetLastError() == hipSuccess ? 0 : -7;
}
