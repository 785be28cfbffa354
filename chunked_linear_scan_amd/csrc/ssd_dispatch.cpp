// SSD validation, workspace sizing and dispatch to the fp32 or bf16 path.
#include <algorithm>
#include <cmath>
#include <array>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/chunked_linear_scan.h"
#include "launch.hpp"
#include "ssd_kernels.hpp"
#include "tune.hpp"

namespace cls {

int ssd_bf16_launch_t32(int P, int S, const SsdBf16Params& prm, hipStream_t stream);
int ssd_bf16_launch_t64(int P, int S, const SsdBf16Params& prm, hipStream_t stream);
int ssd_bf16_launch_t128(int P, int S, const SsdBf16Params& prm, hipStream_t stream);
int ssd_bf16_launch_t256(int P, int S, const SsdBf16Params& prm, hipStream_t stream);

bool ssd_bf16_supported(int TT, int P, int S) {
    const bool p_ok = P == 16 || P == 32 || P == 64 || P == 128;
    const bool s_ok = S == 32 || S == 64 || S == 128 || S == 256;
    return p_ok && s_ok && ssd_bf16_lds_fits(TT, P, S);
}

// The per-(batch, head) kernel's head split: a head of dim P runs as
// 1 << split heads of dim P >> split (bit-identical results; every split
// head recomputes the head's diagonal weights).  Head dim 128 halves (the
// weights are shared by many columns; measured 2156 against 2425 us on a
// 4 x 8192, 40-head, state-256 layer).  Few chains are cut into segments
// instead of narrower heads (chunk_kernel_segs): 32 heads of a 65536-token
// sequence at state size 256 took 5731 us split into 128 heads of dim 16 and
// 1601 us as 32 heads in 8 segments.
int chunk_kernel_split(int64_t batch, int64_t H, int64_t P) {
    int split = P == 128 ? 1 : 0;
    // the grid (batch * H << split workgroups) and the head count stay in 31 bits
    while (split > 0 && (batch * H << split) >= (int64_t(1) << 31)) --split;
    return split;
}

// The per-(batch, head) kernel's tile: the chunk (at least 32 tokens), run as
// sub-chunks of at most kChunkMaxTile tokens and halved until its LDS fits.
// Sub-chunks change the result only by rounding: the chunked form equals the
// recurrence for every chunk length.  0: no tile fits (head dim or state size
// outside the kernel's set).
int chunk_kernel_tile(int64_t chunk, int P, int S) {
    int tt = bf16_tile_tokens(int(chunk));
    if (tt > kChunkMaxTile) tt = kChunkMaxTile;
    while (tt > 32 && !ssd_bf16_lds_fits(tt, P, S)) tt /= 2;
    return ssd_bf16_supported(tt, P, S) ? tt : 0;
}

int ssd_bf16_launch(int TT, int P, int S, const SsdBf16Params& prm, hipStream_t stream) {
    switch (TT) {
        case 32: return ssd_bf16_launch_t32(P, S, prm, stream);
        case 64: return ssd_bf16_launch_t64(P, S, prm, stream);
        case 128: return ssd_bf16_launch_t128(P, S, prm, stream);
        case 256: return ssd_bf16_launch_t256(P, S, prm, stream);
        default: return SSD_ERR_CHUNK;
    }
}

// concurrent workgroups of the fused kernel: one per CU
int64_t fused_slots() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        return n;
    return 256;
}

// Segment plans chosen by the autotuner, per (device, shape).
using TuneKey = std::array<int64_t, 9>;
std::mutex g_tune_mu;
std::map<TuneKey, SegChoice> g_tuned;

TuneKey tune_key(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t S, int64_t G, int64_t chunk, int dtype) {
    chunk = chunk > kFusedMaxChunk ? kFusedMaxChunk : chunk;  // the sub-chunk the kernel runs
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    return TuneKey{dev, batch, L, H, P, S, G, chunk, dtype};
}

bool tuned_choice(const TuneKey& k, SegChoice* out) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    const auto it = g_tuned.find(k);
    if (it == g_tuned.end()) return false;
    *out = it->second;
    return true;
}

// The autotuner's search space: no split; the chains left over after whole
// rounds of the CUs cut into 2..32 segments; every chain cut into 2..32
// segments.  Plans of more than four rounds of workgroups are left out.
SsdFusedPlan ssd_fused_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t S, int64_t G,
                            int64_t chunk, int dtype, const SegChoice* force, int path, int s3, int xcds,
                            int policy = 0, int csrc = 0);

// Passed as `force`: the built-in heuristic, ignoring any tuned plan (the
// autotuner's incumbent).
const SegChoice kUseHeuristic{-1, 0};

std::vector<SegChoice> seg_candidates(int64_t nchains, int64_t nc, int64_t slots) {
    std::vector<SegChoice> v{{1, 0}};
    const int64_t r = nchains % slots;
    auto add = [&](int64_t g, int64_t ns) {
        // the aggregate launch's pieces per segment: the heuristic's count
        // (about two workgroups per CU, rounded down), and 2x and 4x finer
        const int64_t h = std::max<int64_t>(1, (2 * slots) / (ns * (g - 1)));
        for (int64_t m : {1, 2, 4}) v.push_back({g, ns, m == 1 ? 0 : h * m});
    };
    for (int64_t g : {2, 3, 4, 6, 8, 12, 16, 24, 32}) {
        if (g > nc) break;
        if (r > 0 && (nchains - r) + r * g <= 4 * slots) add(g, r);
        if (r != nchains && nchains * g <= 4 * slots) add(g, nchains);
    }
    return v;
}

// force: null (a tuned choice for this shape, else the heuristic), or the
// segment plan to use.  path: SSD_PATH_* of the call (SSD_PATH_CHUNK keeps
// the fused path out).  policy: the call's x/y cache policy (0: the plan's).
// csrc: where the state term reads C (0: the heuristic's choice, 1: the CB
// pass's copy, 2: the C rows).
SsdFusedPlan ssd_fused_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t S, int64_t G,
                            int64_t chunk, int dtype, const SegChoice* force, int path, int s3, int xcds,
                            int policy, int csrc) {
    SsdFusedPlan pl{};
    // The kernel's quadratic block is at most 128 tokens: a longer chunk is run
    // as sub-chunks of 128 with the state passed between them, which changes the
    // result only by rounding (the chunked form equals the recurrence for every
    // chunk length).  A plan may ask for shorter sub-chunks (64 or 32 tokens).
    chunk = chunk > kFusedMaxChunk ? kFusedMaxChunk : chunk;
    // a head of dim 128 runs as two chains of head dim 64
    const int64_t nchains = (batch * H) << fused_head_shift(P);
    // the segment plan: forced, else tuned for this shape, else the heuristic
    SegChoice ch{1, 0};
    bool heuristic = true;
    if (force && force != &kUseHeuristic) {
        ch = *force;
        heuristic = false;
    } else if (!force && dtype == 1 && tuned_choice(tune_key(batch, L, H, P, S, G, chunk, dtype), &ch)) {
        heuristic = false;
    }
    if (!heuristic && ch.sub >= 32 && ch.sub < chunk && chunk % ch.sub == 0) chunk = ch.sub;
    const int TT = bf16_tile_tokens(int(chunk));
    pl.use = dtype == 1 && (P == 64 || P == 128) && (S == 64 || S == 128) && ssd_fused_lds_bytes(TT, int(S)) > 0 &&
             ssd_fused_lds_bytes(TT, int(S)) <= 160 * 1024 && path != 1;
    // the kernel's per-chunk buffer ranges and lane offsets are 32-bit
    if (H * P * 2 * TT >= (int64_t(1) << 31) || G * S * 2 * TT >= (int64_t(1) << 31)) pl.use = false;
    if (!pl.use) return pl;
    const int64_t nc = (L + chunk - 1) / chunk;
    // Each workgroup runs one chain (or segment) at a time, one per CU.  The
    // chains that fill whole rounds of the CUs run whole; the remainder would
    // leave most CUs idle in a last round, so it is split into segments that
    // fill them.  A segment costs its output pass plus its share of the
    // aggregate launch (about half its length), which the split must beat.
    int64_t nsegs = 1, nsplit = 0, want_agg_d = 0;
    int want_s3 = 0;
    if (!heuristic) {
        nsegs = ch.nsegs;
        nsplit = (ch.nsplit > 0 && ch.nsplit < nchains) ? ch.nsplit : nchains;
        want_agg_d = ch.agg_d;
        want_s3 = ch.s3;
    } else {
        const int64_t slots = fused_slots();
        const int64_t r = nchains % slots;
        const int64_t sg = r > 0 ? slots / r : 0;
        if (sg >= 2 && ((nc + sg - 1) / sg) * 3 < nc * 2) {
            nsegs = sg;
            nsplit = r;
        }
    }
    if (nsegs > 64) nsegs = 64;
    if (nsegs > nc) nsegs = nc;
    if (nsegs < 1) nsegs = 1;
    const int64_t k = (nc + nsegs - 1) / nsegs;
    nsegs = (nc + k - 1) / k;
    if (nsegs == 1) nsplit = 0;
    const int64_t nsplit_tiles = nsegs * nsplit;
    const int64_t ntiles = (nchains - nsplit) + nsplit_tiles;
    // Aggregate pieces: the segments but the last of each split chain, cut so
    // the aggregate launch has about two workgroups per CU (it fits two).
    int64_t agg_d = 1, agg_k = k;
    if (nsplit > 0) {
        agg_d = want_agg_d > 0 ? want_agg_d : (2 * fused_slots()) / (nsplit * (nsegs - 1));
        if (agg_d < 1) agg_d = 1;
        if (agg_d > k) agg_d = k;
        agg_k = (k + agg_d - 1) / agg_d;
        agg_d = (k + agg_k - 1) / agg_k;
    }
    // the inter-segment scheme: the call's request, else the plan's, else
    // reduce-then-fold
    const int scheme = s3 > 0 ? s3 : (want_s3 > 0 ? want_s3 : 1);
    pl.lookback = nsplit > 0 && scheme == 2;
    // x/y cache policy: the call's request, else the plan's, else non-temporal
    // when a workgroup walks at least 32 sub-chunks (long chains: measured
    // 1-4 % faster; on chains of 16 sub-chunks the default policy is 4 %
    // faster).  Non-temporal instances exist for 128-token sub-chunks only.
    const int64_t run = (nchains - nsplit) > 0 ? nc : k;  // longest walk of a workgroup
    const int want_nt = policy > 0 ? policy : (!heuristic && ch.nt > 0 ? ch.nt : (run >= 32 ? 2 : 1));
    pl.nt = want_nt == 2 && TT == 128;
    // The state term's C operand: the CB pass's fragment-major copy (one write
    // and one read of C per group), or the C rows read by every head's state
    // loaders (16 rows of 64 bytes per load instead of 1 KB in lane order, more
    // work for the texture path).  Measured on one MI355X: with 8 chains per
    // group the rows are 1.4 % faster per call, with 24 the two are even, with
    // 80 the copy is 4 % faster.
    pl.cdirect = csrc > 0 ? csrc == 2 : nchains <= 8 * batch * G;
    const int64_t npieces = pl.lookback ? 0 : nsplit * (nsegs - 1) * agg_d;
    if (ntiles >= (int64_t(1) << 24)) {
        pl.use = false;
        return pl;
    }
    pl.TT = TT;
    pl.chunk = int(chunk);
    pl.nsegs = int(nsegs);
    pl.seg_chunks = int(k);
    pl.nchains = int(nchains);
    pl.nwhole = int(nchains - nsplit);
    pl.agg_d = int(agg_d);
    pl.agg_chunks = int(agg_k);
    pl.npieces = int(npieces);
    const int nx = xcds > 0 ? xcds : kXcds;
    pl.nranges = int(nsplit < nx ? nsplit : nx);
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    pl.payload_off = kSsdWsHeader;
    // reduce-then-fold, per aggregate piece: its state (fp32) and its decay
    const size_t pay = size_t(npieces) * (size_t(ssd_fused_state_floats(int(S))) + 1) * 4;
    // look-back, per segment: a status word, an aggregate and a prefix state, a decay
    const size_t nseg = pl.lookback ? size_t(nsegs * nsplit) : 0;
    pl.status_off = pl.payload_off + up(pay);
    pl.segpay_off = pl.status_off + up(nseg * 8);
    pl.alpha_off = pl.segpay_off + up(nseg * 2 * size_t(ssd_fused_state_floats(int(S))) * 4);
    pl.cb_off = pl.alpha_off + up(nseg * 4);
    pl.bt_off = pl.cb_off + up(size_t(batch) * size_t(nc) * size_t(G) * size_t(TT) * TT * 2);
    pl.cf_off = pl.bt_off + up(size_t(batch) * size_t(nc) * size_t(G) * size_t(S) * TT * 2);
    pl.dtt_off = pl.cf_off + (pl.cdirect ? 0 : up(size_t(batch) * size_t(nc) * size_t(G) * size_t(S) * TT * 2));
    pl.bytes = pl.dtt_off + size_t(batch) * size_t(nc) * size_t(H) * TT * 4;
    return pl;
}

SsdFusedPlan ssd_fused_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t S, int64_t G,
                            int64_t chunk, int dtype) {
    return ssd_fused_plan(batch, L, H, P, S, G, chunk, dtype, nullptr, 0, 0, 0);
}

}  // namespace cls

namespace {

bool valid_chunk(int64_t c) { return c == 16 || c == 32 || c == 64 || c == 128 || c == 256; }

int64_t nchunks(const SsdShape& s) { return (s.seqlen + s.chunk - 1) / s.chunk; }

// Segments of the per-(batch, head) kernel's chains.  Where the chains fill
// at most half of the workgroup slots (256 CUs times the workgroups that fit
// a CU's LDS, at most 4), each is cut so that about one workgroup per slot
// runs, in segments of at least 8 sub-chunks (shorter ones would spend more on
// the aggregate launch and the fold than the parallelism buys).  Counting the
// slots rather than the CUs measured 35-47 % faster on state sizes 32 and 64
// (e.g. 2 x 8192 tokens x 80 heads, P = 32, S = 64: 448 -> 239 us).
// want > 0: that many segments (a plan request), at most one per sub-chunk.
int64_t chunk_kernel_segs(int64_t chains, int64_t nc, int64_t want, int64_t per_cu) {
    const int64_t slots = 256 * per_cu;
    int64_t n = want > 0 ? want : (2 * chains <= slots ? slots / chains : 1);
    if (want <= 0 && n > nc / 8) n = nc / 8;
    if (n > 64) n = 64;
    if (n > nc) n = nc;
    if (n < 1 || chains * n >= (int64_t(1) << 31)) n = 1;  // the grid stays in 31 bits
    const int64_t k = (nc + n - 1) / n;
    return (nc + k - 1) / k;  // every segment holds at least one sub-chunk
}

// The per-(batch, head) kernel's plan: sub-chunk (tile TT, tokens per
// sub-chunk), head split, segments, and its workspace: C B^T per (batch,
// sub-chunk, group), then (segments) the aggregate states and decays.  TT = 0
// when it has no tile.
struct ChunkTile {
    int TT, chunk;
    int64_t nchunks;
    int split, nsegs, seg_chunks;
    size_t state_off, decay_off, bytes;
};

ChunkTile chunk_kernel_plan(const SsdShape& s, int64_t want_segs = 0) {
    ChunkTile t{};
    t.TT = cls::chunk_kernel_tile(s.chunk, int(s.headdim), int(s.dstate));
    if (t.TT == 0) return t;
    t.chunk = t.TT < s.chunk ? t.TT : int(s.chunk);
    t.nchunks = (s.seqlen + t.chunk - 1) / t.chunk;
    t.split = cls::chunk_kernel_split(s.batch, s.nheads, s.headdim);
    const int64_t chains = (s.batch * s.nheads) << t.split;
    int64_t per_cu = int64_t(160 * 1024) / int64_t(cls::ssd_bf16_lds_bytes(t.TT, int(s.headdim >> t.split), int(s.dstate)));
    per_cu = per_cu < 1 ? 1 : (per_cu > 4 ? 4 : per_cu);
    t.nsegs = int(chunk_kernel_segs(chains, t.nchunks, want_segs, per_cu));
    t.seg_chunks = int((t.nchunks + t.nsegs - 1) / t.nsegs);
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t cb = size_t(s.batch) * size_t(t.nchunks) * size_t(s.ngroups) * size_t(t.TT) * size_t(t.TT) * 2;
    const size_t nagg = size_t(chains) * size_t(t.nsegs - 1);
    t.state_off = cls::kSsdWsHeader + up(cb);
    t.decay_off = t.state_off + up(nagg * cls::chunk_state_floats(int(s.headdim >> t.split), int(s.dstate)) * 4);
    t.bytes = t.nsegs > 1 ? t.decay_off + nagg * 4 : cls::kSsdWsHeader + cb;
    return t;
}

// the segment count a plan request asks for (0: the heuristic's)
int64_t chunk_kernel_want(const cls::SegChoice* force) {
    return (force && force != &cls::kUseHeuristic) ? force->nsegs : 0;
}

// The fp32 kernel's segments (the same rule; at most two workgroups per CU,
// which is what its registers allow) and their workspace: per chain and
// segment but the last, the [P][S] state and the decay.
struct F32Plan {
    int nsegs, seg_chunks;
    size_t state_off, decay_off, bytes;
};

F32Plan f32_plan(const SsdShape& s, int64_t want_segs = 0) {
    F32Plan f{};
    const int64_t chains = s.batch * s.nheads;
    const int64_t nc = (s.seqlen + s.chunk - 1) / s.chunk;
    int64_t per_cu = int64_t(160 * 1024) / int64_t(cls::ssd_f32_launch_lds(int(s.headdim), int(s.dstate), int(s.chunk)));
    per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
    f.nsegs = int(chunk_kernel_segs(chains, nc, want_segs, per_cu));
    f.seg_chunks = int((nc + f.nsegs - 1) / f.nsegs);
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t nagg = size_t(chains) * size_t(f.nsegs - 1);
    f.state_off = cls::kSsdWsHeader;
    f.decay_off = f.state_off + up(nagg * size_t(s.headdim) * size_t(s.dstate) * 4);
    f.bytes = f.nsegs > 1 ? f.decay_off + nagg * 4 : 0;
    return f;
}

size_t chunk_kernel_ws_bytes(const SsdShape& s, int64_t want_segs = 0) {
    const ChunkTile t = chunk_kernel_plan(s, want_segs);
    return t.TT == 0 ? 0 : t.bytes;
}

}  // namespace

extern "C" int cls_ssd_check(const SsdShape& s) {
    if (s.batch <= 0 || s.seqlen <= 0 || s.nheads <= 0 || s.headdim <= 0 || s.dstate <= 0 ||
        s.ngroups <= 0)
        return SSD_ERR_SHAPE;
    if (s.nheads % s.ngroups != 0) return SSD_ERR_SHAPE;
    if (s.dtype != SSD_F32 && s.dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (!valid_chunk(s.chunk)) return SSD_ERR_CHUNK;
    // index arithmetic stays in 64 bits; grids are bounded by 2^31 workgroups
    if (s.batch * s.nheads > (int64_t(1) << 31) || s.seqlen > (int64_t(1) << 40)) return SSD_ERR_SHAPE;
    if (s.nheads > (int64_t(1) << 30) || s.headdim > 4096 || s.dstate > 4096) return SSD_ERR_SHAPE;
    if (s.dtype == SSD_F32) {
        if (s.headdim * s.dstate > 16384 || s.headdim % 4 != 0 || s.dstate % 4 != 0) return SSD_ERR_UNSUPPORTED;
        if (cls::ssd_f32_lds_bytes(int(s.headdim), int(s.dstate)) > 160 * 1024) return SSD_ERR_UNSUPPORTED;
    } else {
        if (cls::chunk_kernel_tile(s.chunk, int(s.headdim), int(s.dstate)) == 0 &&
            !cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk, s.dtype)
                 .use)
            return SSD_ERR_UNSUPPORTED;
        // (batch, sub-chunk, group) blocks of either path, sub-chunks of at least
        // 16 tokens: their count and the sub-chunk count stay below 2^31
        if (s.batch * ((s.seqlen + 15) / 16) * s.ngroups >= (int64_t(1) << 31)) return SSD_ERR_SHAPE;
    }
    return SSD_OK;
}

namespace {

// The candidate plans of a fused-path shape (empty when the fused path is not
// used): the segment plans of seg_candidates, each with reduce-then-fold and,
// when it splits chains, with the look-back; for every sub-chunk the kernel
// may run (the chunk up to 128 tokens, and 64 when the chunk is longer); each
// with the default and the non-temporal x/y cache policy.
std::vector<cls::SegChoice> fused_candidates(const SsdShape& s) {
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype);
    if (!pl.use) return {};
    const int64_t base = s.chunk > cls::kFusedMaxChunk ? cls::kFusedMaxChunk : s.chunk;
    std::vector<cls::SegChoice> out;
    for (int64_t sub : {base, int64_t(64)}) {
        if (sub != base && !(sub < base && base % sub == 0)) continue;
        const int64_t nc = (s.seqlen + sub - 1) / sub;
        for (cls::SegChoice c : cls::seg_candidates(pl.nchains, nc, cls::fused_slots())) {
            c.sub = sub == base ? 0 : sub;
            for (int nt : {1, 2}) {
                c.nt = nt;
                c.s3 = 1;
                out.push_back(c);
                if (c.nsegs > 1 && c.agg_d == 0) {
                    c.s3 = 2;
                    out.push_back(c);
                }
            }
        }
    }
    return out;
}

}  // namespace

// The workspace fits every plan the autotuner may choose, so a buffer sized
// before tuning stays large enough after it.
extern "C" size_t cls_ssd_workspace_bytes(const SsdShape& s) {
    if (s.dtype == SSD_F32) return f32_plan(s).bytes;
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype);
    if (pl.use) {
        size_t bytes = pl.bytes;
        for (const cls::SegChoice& c : fused_candidates(s)) {
            const cls::SsdFusedPlan q = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                            s.ngroups, s.chunk, s.dtype, &c, 0, 0, 0);
            if (q.use && q.bytes > bytes) bytes = q.bytes;
        }
        return bytes;
    }
    return chunk_kernel_ws_bytes(s);
}

extern "C" size_t cls_ssd_plan_bytes(const SsdShape& s, const SsdLaunchOpts& o) {
    if (s.dtype == SSD_F32) return f32_plan(s, chunk_kernel_want(o.force)).bytes;
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype, o.force, o.path, o.s3, o.xcds,
                                                     o.policy, o.csrc);
    if (pl.use) return pl.bytes;
    // 0: the plan keeps the fused path out and the per-(batch, head) kernel
    // has no tile for the shape
    return chunk_kernel_ws_bytes(s, chunk_kernel_want(o.force));
}

static int ssd_launch_plan(const SsdShape& s, const SsdArgs& a, const SsdLaunchOpts& o, hipStream_t stream) {
    const cls::SegChoice* force = o.force;
    hipEvent_t* ev = o.ev;
    // single-launch paths record the call's four events around their launch
    auto ev_pre = [&]() {
        if (ev)
            for (int k = 0; k < 3; ++k) (void)hipEventRecord(ev[k], stream);
    };
    auto ev_post = [&]() {
        if (ev) (void)hipEventRecord(ev[3], stream);
    };
    if (s.dtype == SSD_F32) {
        cls::SsdF32Params p{a.x, a.dt, a.A, a.B, a.C, a.D, a.h0, a.y, a.h_final, s.batch, s.seqlen,
                            int(s.nheads), int(s.headdim), int(s.dstate), int(s.ngroups), int(s.chunk)};
        const F32Plan fp = f32_plan(s, chunk_kernel_want(force));
        p.nsegs = fp.nsegs;
        p.seg_chunks = fp.seg_chunks;
        if (fp.nsegs > 1) {
            p.seg_state = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + fp.state_off);
            p.seg_decay = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + fp.decay_off);
        }
        ev_pre();
        const int st = cls::ssd_f32_launch(p, stream);
        ev_post();
        return st == 0 ? SSD_OK : SSD_ERR_HIP;
    }
    cls::SsdBf16Params p{};
    p.x = static_cast<const uint16_t*>(a.x);
    p.dt = a.dt;
    p.A = a.A;
    p.B = static_cast<const uint16_t*>(a.B);
    p.C = static_cast<const uint16_t*>(a.C);
    p.D = a.D;
    p.h0 = a.h0;
    p.y = static_cast<uint16_t*>(a.y);
    p.h_final = a.h_final;
    p.cb = reinterpret_cast<uint16_t*>(static_cast<char*>(a.workspace) + cls::kSsdWsHeader);
    p.batch = s.batch;
    p.L = s.seqlen;
    p.H = int(s.nheads);
    p.G = int(s.ngroups);
    p.chunk = int(s.chunk);
    p.nchunks = int(nchunks(s));
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype, force, o.path, o.s3, o.xcds,
                                                     o.policy, o.csrc);
    if (pl.use) {
        p.chunk = pl.chunk;
        p.nchunks = int((s.seqlen + pl.chunk - 1) / pl.chunk);
        char* ws = static_cast<char*>(a.workspace);
        p.cb = reinterpret_cast<uint16_t*>(ws + pl.cb_off);
        p.bt = reinterpret_cast<uint16_t*>(ws + pl.bt_off);
        p.cf = pl.cdirect ? nullptr : reinterpret_cast<uint16_t*>(ws + pl.cf_off);
        p.dtt = reinterpret_cast<float*>(ws + pl.dtt_off);
        cls::SsdFusedParams f{};
        f.x = p.x;
        f.dt = p.dt;
        f.A = p.A;
        f.B = p.B;
        f.C = p.C;
        f.D = p.D;
        f.h0 = p.h0;
        f.y = p.y;
        f.h_final = p.h_final;
        f.cb = p.cb;
        f.bt = p.bt;
        f.cf = p.cf;
        f.dtt = p.dtt;
        f.payload = reinterpret_cast<float*>(ws + pl.payload_off);
        f.err = reinterpret_cast<uint32_t*>(ws);
        f.batch = s.batch;
        f.L = s.seqlen;
        f.hshift = cls::fused_head_shift(s.headdim);
        f.H = int(s.nheads) << f.hshift;
        f.G = int(s.ngroups);
        f.chunk = p.chunk;
        f.nchunks = p.nchunks;
        f.seg_chunks = pl.seg_chunks;
        f.nsegs = pl.nsegs;
        f.nchains = pl.nchains;
        f.nwhole = pl.nwhole;
        f.agg_d = pl.agg_d;
        f.agg_chunks = pl.agg_chunks;
        f.nxcd = o.xcds > 0 ? o.xcds : cls::kXcds;
        f.stress = o.stress;
        f.lookback = pl.lookback ? 1 : 0;
        f.nranges = pl.nranges > 0 ? pl.nranges : 1;
        f.seg_ctl = reinterpret_cast<uint32_t*>(ws + cls::kSsdCtlOff);
        f.seg_status = reinterpret_cast<uint64_t*>(ws + pl.status_off);
        f.seg_pay = reinterpret_cast<float*>(ws + pl.segpay_off);
        f.seg_alpha = reinterpret_cast<float*>(ws + pl.alpha_off);
        const int st = cls::ssd_fused_launch(pl.TT, int(s.dstate), p, f, stream, ev, pl.nt);
        if (st == -8) return SSD_ERR_UNSUPPORTED;
        return st == 0 ? SSD_OK : SSD_ERR_HIP;
    }
    const ChunkTile t = chunk_kernel_plan(s, chunk_kernel_want(force));
    if (t.TT == 0) return SSD_ERR_UNSUPPORTED;
    p.chunk = t.chunk;
    p.nchunks = int(t.nchunks);
    p.hshift = t.split;
    p.H = int(s.nheads) << p.hshift;
    p.nsegs = t.nsegs;
    p.seg_chunks = t.seg_chunks;
    if (t.nsegs > 1) {
        p.seg_state = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + t.state_off);
        p.seg_decay = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + t.decay_off);
    }
    ev_pre();
    const int st = cls::ssd_bf16_launch(t.TT, int(s.headdim) >> p.hshift, int(s.dstate), p, stream);
    ev_post();
    if (st == -8) return SSD_ERR_UNSUPPORTED;
    return st == 0 ? SSD_OK : SSD_ERR_HIP;
}

extern "C" int cls_ssd_launch(const SsdShape& s, const SsdArgs& a, const SsdLaunchOpts& o, hipStream_t stream) {
    return ssd_launch_plan(s, a, o, stream);
}

// Autotuner of the fused path's plan (segment plan, inter-segment scheme,
// sub-chunk): the built-in heuristic's plan is the incumbent, the timing loop
// is tune_candidates (tune.hpp), so the tuned plan never loses to the
// heuristic by more than the noise.  The winner is kept for the shape on the
// current device.  The call ends with one more pass on the chosen plan, so y
// and h_final hold exactly what a later ssd_fwd call returns.
namespace {

struct PlanId {
    int64_t nsegs, nsplit, agg_d, sub;
    int s3, nt;
    bool operator==(const PlanId& o) const {
        return nsegs == o.nsegs && nsplit == o.nsplit && agg_d == o.agg_d && sub == o.sub && s3 == o.s3 &&
               nt == o.nt;
    }
};

// The plan a choice realises (segment counts are capped and rounded, pieces
// apply to reduce-then-fold only), as the choice to store.
cls::SegChoice realised(const SsdShape& s, const cls::SegChoice* c, PlanId* id) {
    const cls::SsdFusedPlan q = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups,
                                                    s.chunk, s.dtype, c, 0, 0, 0);
    const int64_t base = s.chunk > cls::kFusedMaxChunk ? cls::kFusedMaxChunk : s.chunk;
    const bool split = q.nsegs > 1;
    *id = PlanId{q.nsegs, split ? int64_t(q.nchains - q.nwhole) : 0, split && !q.lookback ? int64_t(q.agg_d) : 0,
                 q.chunk == base ? 0 : int64_t(q.chunk), split ? (q.lookback ? 2 : 1) : 0, q.nt ? 2 : 1};
    cls::SegChoice out{id->nsegs, id->nsplit, id->agg_d};
    out.s3 = id->s3;
    out.sub = id->sub;
    out.nt = id->nt;
    return out;
}

}  // namespace

extern "C" int cls_ssd_autotune(const SsdShape& s, const SsdArgs& a, hipStream_t stream, int reps, int64_t* nsegs,
                                int64_t* nsplit, int64_t* agg_pieces, int64_t* sub_chunk, int* s3, int* policy,
                                float* ms) {
    *nsegs = 0;
    *nsplit = 0;
    *agg_pieces = 0;
    *sub_chunk = 0;
    *s3 = 0;
    *policy = 0;
    *ms = 0.0f;
    const std::vector<cls::SegChoice> cands = fused_candidates(s);
    if (cands.empty()) return ssd_launch_plan(s, a, SsdLaunchOpts{}, stream);
    auto with = [](const cls::SegChoice* c) {
        SsdLaunchOpts o{};
        o.force = c;
        return o;
    };
    // distinct plans, the incumbent (the heuristic's) first
    std::vector<cls::SegChoice> plans;
    std::vector<PlanId> ids;
    auto add = [&](const cls::SegChoice* c) {
        PlanId id{};
        const cls::SegChoice r = realised(s, c, &id);
        for (const PlanId& e : ids)
            if (e == id) return;
        ids.push_back(id);
        plans.push_back(r);
    };
    add(&cls::kUseHeuristic);
    for (const cls::SegChoice& c : cands) add(&c);

    size_t chosen = 0;  // the incumbent
    float chosen_ms = 0.0f;
    const int st = cls::tune_candidates(
        plans.size(), [&](size_t i) { return ssd_launch_plan(s, a, with(&plans[i]), stream); }, stream, reps,
        SSD_ERR_HIP, &chosen, &chosen_ms);
    if (st != SSD_OK) return st;
    const cls::SegChoice best = plans[chosen];
    {
        std::lock_guard<std::mutex> lock(cls::g_tune_mu);
        cls::g_tuned[cls::tune_key(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk,
                                   s.dtype)] = best;
    }
    const cls::SsdFusedPlan qb = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups,
                                                     s.chunk, s.dtype, &best, 0, 0, 0);
    *nsegs = best.nsegs;
    *nsplit = best.nsplit;
    *agg_pieces = best.agg_d;
    *sub_chunk = qb.chunk;
    *s3 = best.s3;
    *policy = qb.nt ? 2 : 1;
    *ms = chosen_ms;
    return ssd_launch_plan(s, a, with(&best), stream);
}

extern "C" int cls_ssd_plan_query(const SsdShape& s, int64_t* nsegs, int64_t* nsplit, int64_t* agg_pieces,
                                  int64_t* sub_chunk, int* s3, int* policy) {
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype);
    *nsegs = 0;
    *nsplit = 0;
    *agg_pieces = 0;
    *sub_chunk = 0;
    *s3 = 0;
    *policy = 0;
    if (s.dtype == SSD_F32 || !pl.use) return 2;
    PlanId id{};
    (void)realised(s, nullptr, &id);
    *nsegs = id.nsegs;
    *nsplit = id.nsplit;
    *agg_pieces = id.agg_d;
    *sub_chunk = pl.chunk;
    *s3 = id.s3;
    *policy = id.nt;
    cls::SegChoice t{};
    const bool tuned = cls::tuned_choice(cls::tune_key(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                       s.ngroups, s.chunk, s.dtype), &t);
    return tuned ? 1 : 0;
}

extern "C" void cls_ssd_autotune_reset() {
    std::lock_guard<std::mutex> lock(cls::g_tune_mu);
    cls::g_tuned.clear();
}
