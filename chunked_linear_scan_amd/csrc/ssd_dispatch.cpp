// SSD validation, workspace sizing and dispatch to the fp32 or bf16 path.
#include <algorithm>
#include <array>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/chunked_linear_scan.h"
#include "launch.hpp"
#include "ssd_kernels.hpp"

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
                            int64_t chunk, int dtype, const SegChoice* force, int path, int s3, int xcds);

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
// the fused path out).
SsdFusedPlan ssd_fused_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t S, int64_t G,
                            int64_t chunk, int dtype, const SegChoice* force, int path, int s3, int xcds) {
    SsdFusedPlan pl{};
    // The kernel's quadratic block is at most 128 tokens: a longer chunk is run
    // as sub-chunks of 128 with the state passed between them, which changes the
    // result only by rounding (the chunked form equals the recurrence for every
    // chunk length).
    chunk = chunk > kFusedMaxChunk ? kFusedMaxChunk : chunk;
    const int TT = bf16_tile_tokens(int(chunk));
    pl.use = dtype == 1 && P == 64 && (S == 64 || S == 128) && ssd_fused_lds_bytes(TT, int(S)) > 0 &&
             ssd_fused_lds_bytes(TT, int(S)) <= 160 * 1024 && path != 1;
    // the kernel's per-chunk buffer ranges and lane offsets are 32-bit
    if (H * 64 * 2 * TT >= (int64_t(1) << 31) || G * S * 2 * TT >= (int64_t(1) << 31)) pl.use = false;
    if (!pl.use) return pl;
    const int64_t nc = (L + chunk - 1) / chunk;
    const int64_t nchains = batch * H;
    // Each workgroup runs one chain (or segment) at a time, one per CU.  The
    // chains that fill whole rounds of the CUs run whole; the remainder would
    // leave most CUs idle in a last round, so it is split into segments that
    // fill them.  A segment costs its output pass plus its share of the
    // aggregate launch (about half its length), which the split must beat.
    int64_t nsegs = 1, nsplit = 0, want_agg_d = 0;
    int want_s3 = 0;
    SegChoice tuned{};
    if (force) {
        nsegs = force->nsegs;
        nsplit = (force->nsplit > 0 && force->nsplit < nchains) ? force->nsplit : nchains;
        want_agg_d = force->agg_d;
        want_s3 = force->s3;
    } else if (tuned_choice(tune_key(batch, L, H, P, S, G, chunk, dtype), &tuned)) {
        nsegs = tuned.nsegs;
        nsplit = tuned.nsplit;
        want_agg_d = tuned.agg_d;
        want_s3 = tuned.s3;
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
    pl.dtt_off = pl.cf_off + up(size_t(batch) * size_t(nc) * size_t(G) * size_t(S) * TT * 2);
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
        const int TT = cls::bf16_tile_tokens(int(s.chunk));
        if (!cls::ssd_bf16_supported(TT, int(s.headdim), int(s.dstate))) return SSD_ERR_UNSUPPORTED;
        if (s.batch * nchunks(s) * s.ngroups > (int64_t(1) << 31)) return SSD_ERR_SHAPE;
    }
    return SSD_OK;
}

namespace {

// The candidate plans of a fused-path shape (empty when the fused path is not used).
std::vector<cls::SegChoice> fused_candidates(const SsdShape& s) {
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype);
    if (!pl.use) return {};
    const int64_t nc = (s.seqlen + pl.chunk - 1) / pl.chunk;
    return cls::seg_candidates(s.batch * s.nheads, nc, cls::fused_slots());
}

}  // namespace

// The workspace fits every plan the autotuner may choose, so a buffer sized
// before tuning stays large enough after it.
extern "C" size_t cls_ssd_workspace_bytes(const SsdShape& s) {
    if (s.dtype == SSD_F32) return 0;
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
    const int64_t TT = cls::bf16_tile_tokens(int(s.chunk));
    return size_t(s.batch) * size_t(nchunks(s)) * size_t(s.ngroups) * size_t(TT * TT) * 2 + cls::kSsdWsHeader;
}

extern "C" size_t cls_ssd_plan_bytes(const SsdShape& s, const SsdLaunchOpts& o) {
    if (s.dtype == SSD_F32) return 0;
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype, o.force, o.path, o.s3, o.xcds);
    if (pl.use) return pl.bytes;
    const int64_t TT = cls::bf16_tile_tokens(int(s.chunk));
    return size_t(s.batch) * size_t(nchunks(s)) * size_t(s.ngroups) * size_t(TT * TT) * 2 + cls::kSsdWsHeader;
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
                                                     s.ngroups, s.chunk, s.dtype, force, o.path, o.s3, o.xcds);
    if (pl.use) {
        p.chunk = pl.chunk;
        p.nchunks = int((s.seqlen + pl.chunk - 1) / pl.chunk);
        char* ws = static_cast<char*>(a.workspace);
        p.cb = reinterpret_cast<uint16_t*>(ws + pl.cb_off);
        p.bt = reinterpret_cast<uint16_t*>(ws + pl.bt_off);
        p.cf = reinterpret_cast<uint16_t*>(ws + pl.cf_off);
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
        f.H = int(s.nheads);
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
        f.lookback = pl.lookback ? 1 : 0;
        f.nranges = pl.nranges > 0 ? pl.nranges : 1;
        f.seg_ctl = reinterpret_cast<uint32_t*>(ws + cls::kSsdCtlOff);
        f.seg_status = reinterpret_cast<uint64_t*>(ws + pl.status_off);
        f.seg_pay = reinterpret_cast<float*>(ws + pl.segpay_off);
        f.seg_alpha = reinterpret_cast<float*>(ws + pl.alpha_off);
        const int st = cls::ssd_fused_launch(pl.TT, int(s.dstate), p, f, stream, ev);
        if (st == -8) return SSD_ERR_UNSUPPORTED;
        return st == 0 ? SSD_OK : SSD_ERR_HIP;
    }
    const int TT = cls::bf16_tile_tokens(int(s.chunk));
    ev_pre();
    const int st = cls::ssd_bf16_launch(TT, int(s.headdim), int(s.dstate), p, stream);
    ev_post();
    if (st == -8) return SSD_ERR_UNSUPPORTED;
    return st == 0 ? SSD_OK : SSD_ERR_HIP;
}

extern "C" int cls_ssd_launch(const SsdShape& s, const SsdArgs& a, const SsdLaunchOpts& o, hipStream_t stream) {
    return ssd_launch_plan(s, a, o, stream);
}

// Autotuner of the fused path's segment plan (the one run-time choice of its
// launches): after one untimed pass over every candidate, each runs `reps`
// times between two events on the caller's stream, in two rounds; the lowest
// mean of its better round wins and is kept for the shape on the current
// device.  Candidates that reduce to the same plan are timed once.  The call ends with one more pass on the chosen plan, so y and
// h_final hold exactly what a later ssd_fwd call returns.
extern "C" int cls_ssd_autotune(const SsdShape& s, const SsdArgs& a, hipStream_t stream, int reps, int64_t* nsegs,
                                int64_t* nsplit, int64_t* agg_pieces, float* ms) {
    *nsegs = 0;
    *nsplit = 0;
    *agg_pieces = 0;
    *ms = 0.0f;
    const std::vector<cls::SegChoice> cands = fused_candidates(s);
    if (cands.empty()) return ssd_launch_plan(s, a, SsdLaunchOpts{}, stream);
    auto with = [](const cls::SegChoice* c) {
        SsdLaunchOpts o{};
        o.force = c;
        return o;
    };
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return SSD_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return SSD_ERR_HIP;
    }
    // distinct plans only
    std::vector<cls::SegChoice> plans;
    for (const cls::SegChoice& c : cands) {
        const cls::SsdFusedPlan q = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                        s.ngroups, s.chunk, s.dtype, &c, 0, 0, 0);
        const cls::SegChoice ce{q.nsegs, q.nsegs > 1 ? int64_t(q.nchains - q.nwhole) : 0,
                                q.nsegs > 1 ? int64_t(q.agg_d) : 0};
        bool dup = false;
        for (const auto& e : plans)
            dup = dup || (e.nsegs == ce.nsegs && e.nsplit == ce.nsplit && e.agg_d == ce.agg_d);
        if (!dup) plans.push_back(ce);
    }
    // One untimed pass over every plan first (clocks and caches settle), then
    // two timed rounds over all plans; each plan keeps its better round, so a
    // plan is not favoured by where it falls in the sequence.
    int st = SSD_OK;
    std::vector<float> t_best(plans.size(), -1.0f);
    for (size_t i = 0; i < plans.size() && st == SSD_OK; ++i) st = ssd_launch_plan(s, a, with(&plans[i]), stream);
    for (int round = 0; round < 2 && st == SSD_OK; ++round) {
        for (size_t i = 0; i < plans.size() && st == SSD_OK; ++i) {
            st = ssd_launch_plan(s, a, with(&plans[i]), stream);
            if (st != SSD_OK) break;
            if (hipEventRecord(e0, stream) != hipSuccess) {
                st = SSD_ERR_HIP;
                break;
            }
            for (int r = 0; r < reps && st == SSD_OK; ++r) st = ssd_launch_plan(s, a, with(&plans[i]), stream);
            if (st != SSD_OK) break;
            float t = 0.0f;
            if (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&t, e0, e1) != hipSuccess) {
                st = SSD_ERR_HIP;
                break;
            }
            t /= float(reps);
            if (t_best[i] < 0.0f || t < t_best[i]) t_best[i] = t;
        }
    }
    float best_ms = 0.0f;
    cls::SegChoice best{0, 0, 0};
    for (size_t i = 0; i < plans.size(); ++i)
        if (t_best[i] >= 0.0f && (best.nsegs == 0 || t_best[i] < best_ms)) {
            best_ms = t_best[i];
            best = plans[i];
        }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != SSD_OK) return st;
    {
        std::lock_guard<std::mutex> lock(cls::g_tune_mu);
        cls::g_tuned[cls::tune_key(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk,
                                   s.dtype)] = best;
    }
    *nsegs = best.nsegs;
    *nsplit = best.nsplit;
    *agg_pieces = best.agg_d;
    *ms = best_ms;
    return ssd_launch_plan(s, a, with(&best), stream);
}

extern "C" int cls_ssd_plan_query(const SsdShape& s, int64_t* nsegs, int64_t* nsplit, int64_t* agg_pieces) {
    const cls::SsdFusedPlan pl = cls::ssd_fused_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                     s.ngroups, s.chunk, s.dtype);
    if (s.dtype == SSD_F32 || !pl.use) {
        *nsegs = 0;
        *nsplit = 0;
        *agg_pieces = 0;
        return 2;
    }
    *nsegs = pl.nsegs;
    *nsplit = pl.nsegs > 1 ? int64_t(pl.nchains - pl.nwhole) : 0;
    *agg_pieces = pl.nsegs > 1 ? int64_t(pl.agg_d) : 0;
    cls::SegChoice t{};
    const bool tuned = cls::tuned_choice(cls::tune_key(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate,
                                                       s.ngroups, s.chunk, s.dtype), &t);
    return tuned ? 1 : 0;
}

extern "C" void cls_ssd_autotune_reset() {
    std::lock_guard<std::mutex> lock(cls::g_tune_mu);
    cls::g_tuned.clear();
}
