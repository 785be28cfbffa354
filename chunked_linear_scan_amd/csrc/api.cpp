// C ABI of the library: host-side validation, workspace sizing and dispatch.
// Every argument is checked before anything is enqueued; kernels are
// launched on the caller's stream and nothing here synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <array>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/chunked_linear_scan.h"
#include "../../include/chunked_linear_scan_testing.h"
#include "launch.hpp"
#include "tune.hpp"


namespace {

constexpr int64_t kLsTile = 8192;  // elements per linear-scan tile: the built-in choice
// fp32 tiles the scan autotuner may choose (the built-in one first)
constexpr int64_t kLsTileCandidates[] = {8192, 4096, 16384};
constexpr size_t kHeader = 256;    // bytes: error word and padding

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct ScanPlan {
    bool segmented;
    int64_t tile;
    int64_t tiles_per_row;
    int64_t rows_per_tile;
    int64_t ntiles;
    size_t claim_off, done_off, status_off, bytes;
};

ScanPlan plan_scan(int64_t rows, int64_t L, int64_t tile = kLsTile) {
    ScanPlan p{};
    p.tile = tile;
    p.segmented = L <= tile - 6;
    if (p.segmented) {
        // A packed tile covers its rows from the 16-byte boundary at or before
        // the first row's start, up to 3 elements early, so its rows may hold
        // tile - 3 elements.  When L is a multiple of 4 every row starts on
        // such a boundary (the base is 16-byte aligned), so whole rows fill
        // the tile exactly.
        p.rows_per_tile = (L % 4 == 0) ? tile / L : (tile - 3) / L;
        p.tiles_per_row = 1;
        p.ntiles = (rows + p.rows_per_tile - 1) / p.rows_per_tile;
        p.claim_off = p.done_off = p.status_off = kHeader;
        p.bytes = kHeader;
    } else {
        p.rows_per_tile = 1;
        p.tiles_per_row = (L + 3 + tile - 1) / tile;
        p.ntiles = rows * p.tiles_per_row;
        p.claim_off = kHeader;
        p.done_off = p.claim_off + round_up(size_t(rows) * 4, 256);
        p.status_off = p.done_off + round_up(size_t(rows) * 4, 256);
        p.bytes = p.status_off + size_t(rows) * size_t(p.tiles_per_row) * 16;
    }
    return p;
}

// grid x times 256 work-items must stay below 2^32
bool plan_fits(const ScanPlan& p) { return p.ntiles <= (int64_t(1) << 23) && p.tiles_per_row < (int64_t(1) << 30); }

bool scan_sizes_ok(int64_t rows, int64_t L) {
    if (rows <= 0 || L <= 0) return false;
    if (L > (int64_t(1) << 40) || rows > (int64_t(1) << 40)) return false;
    return plan_fits(plan_scan(rows, L));
}

// Workspace that every candidate tile of a valid shape fits.
size_t scan_ws_bytes(int64_t rows, int64_t L) {
    size_t b = 0;
    for (int64_t t : kLsTileCandidates) {
        const ScanPlan p = plan_scan(rows, L, t);
        if (plan_fits(p)) b = p.bytes > b ? p.bytes : b;
    }
    return b;
}

// fp32 tiles chosen by linear_scan_autotune, per (device, rows, length).
std::mutex g_scan_mu;
std::map<std::array<int64_t, 3>, int64_t> g_scan_tuned;

std::array<int64_t, 3> scan_key(int64_t rows, int64_t L) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    return {dev, rows, L};
}

// The tile an fp32 linear_scan of this shape runs, and whether it is tuned.
int64_t scan_tile(int64_t rows, int64_t L, bool* tuned = nullptr) {
    std::lock_guard<std::mutex> lock(g_scan_mu);
    const auto it = g_scan_tuned.find(scan_key(rows, L));
    if (tuned) *tuned = it != g_scan_tuned.end();
    return it != g_scan_tuned.end() ? it->second : kLsTile;
}

}  // namespace

extern "C" {

const char* ssd_strerror(int status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "invalid shape (a size <= 0, too large, or heads % groups != 0)";
        case SSD_ERR_DTYPE: return "dtype must be SSD_F32 or SSD_BF16";
        case SSD_ERR_CHUNK: return "chunk must be 16, 32, 64, 128 or 256";
        case SSD_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case SSD_ERR_WORKSPACE: return "workspace is NULL or smaller than required";
        case SSD_ERR_HIP: return "a HIP kernel launch failed";
        case SSD_ERR_UNSUPPORTED: return "head dim / state size not supported by this dtype's kernels";
        default: return "unknown status";
    }
}

size_t linear_scan_workspace_size(int64_t rows, int64_t length) {
    if (!scan_sizes_ok(rows, length)) return 0;
    return scan_ws_bytes(rows, length);
}

// in_fmt / out_fmt: 0 fp32, 1 bf16, 2 fp16; hs: the Hillis-Steele in-tile
// scan; tile: elements per tile (0: the tuned fp32 tile of the shape, else the
// built-in one).
static int linear_scan_launch(const void* a, const void* b, void* h, int64_t rows, int64_t length, int in_fmt,
                              int out_fmt, void* workspace, size_t workspace_bytes, void* stream, int hs = 0,
                              int64_t tile = 0, uint32_t stress = 0) {
    if (!a || !b || !h || !workspace) return SSD_ERR_NULL;
    if (!scan_sizes_ok(rows, length)) return SSD_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(h) || !aligned16(workspace)) return SSD_ERR_ALIGN;
    if (tile == 0) tile = (in_fmt == 0 && out_fmt == 0 && !hs) ? scan_tile(rows, length) : kLsTile;
    const ScanPlan p = plan_scan(rows, length, tile);
    if (!plan_fits(p)) return SSD_ERR_SHAPE;
    if (workspace_bytes < p.bytes) return SSD_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    const int st = cls_launch_linear_scan(a, b, h, rows, length, in_fmt, out_fmt, p.segmented ? 1 : 0,
                                          int(p.tiles_per_row), int(p.rows_per_tile), p.ntiles,
                                          reinterpret_cast<uint32_t*>(ws + p.claim_off),
                                          reinterpret_cast<uint32_t*>(ws + p.done_off), ws + p.status_off,
                                          reinterpret_cast<uint32_t*>(ws), static_cast<hipStream_t>(stream), hs,
                                          int(tile), stress);
    return st == 0 ? SSD_OK : st == -2 ? SSD_ERR_SHAPE : SSD_ERR_HIP;
}

int linear_scan(const float* a, const float* b, float* h, int64_t rows, int64_t length,
                void* workspace, size_t workspace_bytes, void* stream) {
    return linear_scan_launch(a, b, h, rows, length, 0, 0, workspace, workspace_bytes, stream);
}

int linear_scan_noalloc(const float* a, const float* b, float* h, int64_t rows, int64_t length, void* stream) {
    if (!a || !b || !h) return SSD_ERR_NULL;
    if (!scan_sizes_ok(rows, length)) return SSD_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(h)) return SSD_ERR_ALIGN;
    if (scan_ws_bytes(rows, length) > CLS_NOALLOC_SCAN_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
    // the tile linear_scan runs for this shape (tuned or built-in), fixed here
    // so the cleared range and the launch agree
    const int64_t tile = scan_tile(rows, length);
    const ScanPlan p = plan_scan(rows, length, tile);
    void* ws = nullptr;
    if (cls_noalloc_scratch(&ws) != 0) return SSD_ERR_HIP;
    // the array keeps whatever the last call left: clear the counters, the
    // status words and the error word this call uses
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (cls_zero_fill(ws, round_up(p.bytes, 16), s) != 0) return SSD_ERR_HIP;
    return linear_scan_launch(a, b, h, rows, length, 0, 0, ws, CLS_NOALLOC_SCAN_SCRATCH_BYTES, stream, 0, tile);
}

int linear_scan_typed(const void* a, const void* b, void* h, int64_t rows, int64_t length, int in_dtype,
                      int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    auto fmt = [](int d) { return d == SSD_F32 ? 0 : d == SSD_BF16 ? 1 : d == SSD_F16 ? 2 : -1; };
    if (fmt(in_dtype) < 0 || fmt(out_dtype) < 0) return SSD_ERR_DTYPE;
    return linear_scan_launch(a, b, h, rows, length, fmt(in_dtype), fmt(out_dtype), workspace, workspace_bytes,
                              stream);
}

int linear_scan_planned(const float* a, const float* b, float* h, int64_t rows, int64_t length, int64_t tile,
                        uint32_t stress_seed, void* workspace, size_t workspace_bytes, void* stream) {
    if (tile != 0 && tile != 4096 && tile != 8192 && tile != 16384) return SSD_ERR_SHAPE;
    return linear_scan_launch(a, b, h, rows, length, 0, 0, workspace, workspace_bytes, stream, 0, tile,
                              stress_seed);
}

int linear_scan_autotune(const float* a, const float* b, float* h, int64_t rows, int64_t length, void* workspace,
                         size_t workspace_bytes, void* stream, int reps, int64_t* tile, float* ms_per_call) {
    if (!tile || !ms_per_call) return SSD_ERR_NULL;
    *tile = 0;
    *ms_per_call = 0.0f;
    if (!a || !b || !h || !workspace) return SSD_ERR_NULL;
    if (!scan_sizes_ok(rows, length)) return SSD_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(h) || !aligned16(workspace)) return SSD_ERR_ALIGN;
    if (workspace_bytes < scan_ws_bytes(rows, length)) return SSD_ERR_WORKSPACE;
    if (reps < 1 || reps > 10000) return SSD_ERR_SHAPE;
    std::vector<int64_t> cands;  // valid tiles, the built-in one first
    for (int64_t t : kLsTileCandidates)
        if (plan_fits(plan_scan(rows, length, t))) cands.push_back(t);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    size_t chosen = 0;
    float ms = 0.0f;
    const int st = cls::tune_candidates(
        cands.size(),
        [&](size_t i) {
            return linear_scan_launch(a, b, h, rows, length, 0, 0, workspace, workspace_bytes, stream, 0, cands[i]);
        },
        s, reps, SSD_ERR_HIP, &chosen, &ms);
    if (st != SSD_OK) return st;
    {
        std::lock_guard<std::mutex> lock(g_scan_mu);
        g_scan_tuned[scan_key(rows, length)] = cands[chosen];
    }
    *tile = cands[chosen];
    *ms_per_call = ms;
    // h ends as a later linear_scan of this shape returns it
    return linear_scan_launch(a, b, h, rows, length, 0, 0, workspace, workspace_bytes, stream, 0, cands[chosen]);
}

int linear_scan_plan(int64_t rows, int64_t length, int64_t* tile) {
    if (!tile) return SSD_ERR_NULL;
    *tile = 0;
    if (!scan_sizes_ok(rows, length)) return SSD_ERR_SHAPE;
    bool tuned = false;
    *tile = scan_tile(rows, length, &tuned);
    return tuned ? 1 : 0;
}

void linear_scan_autotune_reset(void) {
    std::lock_guard<std::mutex> lock(g_scan_mu);
    g_scan_tuned.clear();
}

int linear_scan_hillis_steele(const float* a, const float* b, float* h, int64_t rows, int64_t length,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return linear_scan_launch(a, b, h, rows, length, 0, 0, workspace, workspace_bytes, stream, 1);
}

int stream_mul_f32(const float* a, const float* b, float* h, int64_t n, int vec, int nt, int64_t grid_blocks,
                   void* stream) {
    if (!a || !b || !h) return SSD_ERR_NULL;
    if (!aligned16(a) || !aligned16(b) || !aligned16(h)) return SSD_ERR_ALIGN;
    if (n <= 0 || n % 4 != 0 || n > (int64_t(1) << 40)) return SSD_ERR_SHAPE;
    if (!(vec == 1 || vec == 2 || vec == 4 || vec == 8) || (nt != 0 && nt != 1)) return SSD_ERR_SHAPE;
    if (grid_blocks < 0 || grid_blocks > (int64_t(1) << 23)) return SSD_ERR_SHAPE;
    if (grid_blocks == 0 && (n / 4 + 256 * vec - 1) / (256 * vec) > (int64_t(1) << 23)) return SSD_ERR_SHAPE;
    return cls_launch_stream_mul(a, b, h, n, vec, nt, grid_blocks, static_cast<hipStream_t>(stream)) == 0
               ? SSD_OK
               : SSD_ERR_HIP;
}

size_t ssd_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t ngroups, int64_t chunk, int dtype) {
    SsdShape s{batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype};
    if (cls_ssd_check(s) != SSD_OK) return 0;
    return cls_ssd_workspace_bytes(s);
}

// The checks ssd_fwd and ssd_fwd_autotune make before any launch.
static int ssd_fwd_validate(const SsdShape& s, const SsdArgs& a, size_t workspace_bytes) {
    if (!a.x || !a.dt || !a.A || !a.B || !a.C || !a.y) return SSD_ERR_NULL;
    const int st = cls_ssd_check(s);
    if (st != SSD_OK) return st;
    const size_t need = cls_ssd_workspace_bytes(s);
    if (need > 0 && !a.workspace) return SSD_ERR_NULL;
    if (workspace_bytes < need) return SSD_ERR_WORKSPACE;
    const void* ptrs[] = {a.x, a.dt, a.A, a.B, a.C, a.D, a.h0, a.y, a.h_final, a.workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    return SSD_OK;
}

int ssd_fwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
            const float* D, const float* h0, int64_t batch, int64_t seqlen, int64_t nheads,
            int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk, int dtype, void* y,
            float* h_final, void* workspace, size_t workspace_bytes, void* stream) {
    const SsdShape s{batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype};
    const SsdArgs args{x, dt, A, B, C, D, h0, y, h_final, workspace};
    const int st = ssd_fwd_validate(s, args, workspace_bytes);
    if (st != SSD_OK) return st;
    return cls_ssd_launch(s, args, SsdLaunchOpts{}, static_cast<hipStream_t>(stream));
}

// The launch options an ssd_plan_request asks for (false: a field is out of range).
static bool plan_options(const ssd_plan_request* plan, cls::SegChoice* seg, SsdLaunchOpts* o) {
    *o = SsdLaunchOpts{};
    if (!plan) return true;
    if (plan->path < SSD_PATH_AUTO || plan->path > SSD_PATH_FUSED) return false;
    if (plan->s3 < SSD_S3_AUTO || plan->s3 > SSD_S3_LOOKBACK) return false;
    if (plan->nsegs < 0 || plan->nsegs > 64 || plan->nsplit < 0 || plan->agg_pieces < 0) return false;
    if (plan->agg_pieces > (int64_t(1) << 20) || plan->nsplit > (int64_t(1) << 31)) return false;
    if (plan->xcds < 0 || plan->xcds > 64) return false;
    if (plan->sub_chunk != 0 && plan->sub_chunk != 32 && plan->sub_chunk != 64) return false;
    if (plan->cache_policy < 0 || plan->cache_policy > 2) return false;
    if (plan->c_source < SSD_CSRC_AUTO || plan->c_source > SSD_CSRC_ROWS) return false;
    o->path = plan->path;
    o->s3 = plan->s3;
    o->xcds = plan->xcds;
    o->stress = plan->stress_seed;
    o->policy = plan->cache_policy;
    o->csrc = plan->c_source;
    if (plan->nsegs > 0) {
        *seg = cls::SegChoice{plan->nsegs, plan->nsplit, plan->agg_pieces};
        seg->s3 = plan->s3;
        seg->sub = plan->sub_chunk;
        seg->nt = plan->cache_policy;
        o->force = seg;
    }
    return true;
}

size_t ssd_fwd_planned_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                      int64_t dstate, int64_t ngroups, int64_t chunk, int dtype,
                                      const ssd_plan_request* plan) {
    const SsdShape s{batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype};
    cls::SegChoice seg{};
    SsdLaunchOpts o{};
    if (cls_ssd_check(s) != SSD_OK || !plan_options(plan, &seg, &o)) return 0;
    const size_t need = cls_ssd_plan_bytes(s, o);
    if (dtype == SSD_BF16 && need == 0) return 0;  // this plan cannot run the shape
    const size_t base = cls_ssd_workspace_bytes(s);
    return need > base ? need : base;
}

int ssd_fwd_planned(const void* x, const float* dt, const float* A, const void* B, const void* C,
                    const float* D, const float* h0, int64_t batch, int64_t seqlen, int64_t nheads,
                    int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk, int dtype, void* y,
                    float* h_final, void* workspace, size_t workspace_bytes, void* stream,
                    const ssd_plan_request* plan, void* const* events) {
    const SsdShape s{batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype};
    const SsdArgs args{x, dt, A, B, C, D, h0, y, h_final, workspace};
    cls::SegChoice seg{};
    SsdLaunchOpts o{};
    if (!plan_options(plan, &seg, &o)) return SSD_ERR_SHAPE;
    // pointers, shape and alignment first, then whether this plan can run the
    // shape, then the workspace size
    int st = ssd_fwd_validate(s, args, SIZE_MAX);
    if (st != SSD_OK) return st;
    const size_t need = cls_ssd_plan_bytes(s, o);
    if (dtype == SSD_BF16 && need == 0) return SSD_ERR_UNSUPPORTED;
    st = ssd_fwd_validate(s, args, workspace_bytes);
    if (st != SSD_OK) return st;
    if (workspace_bytes < need) return SSD_ERR_WORKSPACE;
    hipEvent_t ev[4];
    if (events) {
        for (int k = 0; k < 4; ++k) {
            if (!events[k]) return SSD_ERR_NULL;
            ev[k] = static_cast<hipEvent_t>(events[k]);
        }
        o.ev = ev;
    }
    return cls_ssd_launch(s, args, o, static_cast<hipStream_t>(stream));
}

int ssd_fwd_autotune(const void* x, const float* dt, const float* A, const void* B, const void* C,
                     const float* D, const float* h0, int64_t batch, int64_t seqlen, int64_t nheads,
                     int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk, int dtype, void* y,
                     float* h_final, void* workspace, size_t workspace_bytes, void* stream, int reps,
                     int64_t* nsegs, int64_t* nsplit, int64_t* agg_pieces, int64_t* sub_chunk, int* s3,
                     int* cache_policy, float* ms_per_call) {
    if (!nsegs || !nsplit || !agg_pieces || !sub_chunk || !s3 || !cache_policy || !ms_per_call) return SSD_ERR_NULL;
    if (reps < 1 || reps > 1000) return SSD_ERR_SHAPE;
    const SsdShape s{batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype};
    const SsdArgs args{x, dt, A, B, C, D, h0, y, h_final, workspace};
    const int st = ssd_fwd_validate(s, args, workspace_bytes);
    if (st != SSD_OK) return st;
    return cls_ssd_autotune(s, args, static_cast<hipStream_t>(stream), reps, nsegs, nsplit, agg_pieces, sub_chunk,
                            s3, cache_policy, ms_per_call);
}

int ssd_fwd_plan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                 int64_t chunk, int dtype, int64_t* nsegs, int64_t* nsplit, int64_t* agg_pieces, int64_t* sub_chunk,
                 int* s3, int* cache_policy) {
    if (!nsegs || !nsplit || !agg_pieces || !sub_chunk || !s3 || !cache_policy) return SSD_ERR_NULL;
    const SsdShape s{batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype};
    const int st = cls_ssd_check(s);
    if (st != SSD_OK) return st;
    return cls_ssd_plan_query(s, nsegs, nsplit, agg_pieces, sub_chunk, s3, cache_policy);
}

void ssd_fwd_autotune_reset(void) { cls_ssd_autotune_reset(); }

static bool ls3_sizes_ok(int64_t rows, int64_t L) {
    if (rows <= 0 || L <= 0 || L > (int64_t(1) << 40) || rows > (int64_t(1) << 40)) return false;
    const int64_t ntiles = (L + 8191) / 8192;
    return rows * ntiles < (int64_t(1) << 31) && rows * L < (int64_t(1) << 46);
}

size_t linear_scan_three_pass_workspace_size(int64_t rows, int64_t length) {
    return ls3_sizes_ok(rows, length) ? cls_ls3_workspace_bytes(rows, length) : 0;
}

int linear_scan_three_pass(const float* a, const float* b, float* h, int64_t rows, int64_t length,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (!a || !b || !h || !workspace) return SSD_ERR_NULL;
    if (!ls3_sizes_ok(rows, length)) return SSD_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(h) || !aligned16(workspace)) return SSD_ERR_ALIGN;
    if (workspace_bytes < cls_ls3_workspace_bytes(rows, length)) return SSD_ERR_WORKSPACE;
    return cls_ls3_launch(a, b, h, rows, length, workspace, static_cast<hipStream_t>(stream)) == 0 ? SSD_OK
                                                                                                 : SSD_ERR_HIP;
}

int ssd_step(float* h, const void* x, const float* dt, const float* A, const void* B, const void* C,
             const float* D, int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
             int dtype, void* y, void* stream) {
    if (!h || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    if (dtype != SSD_F32 && dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 || nheads % ngroups != 0)
        return SSD_ERR_SHAPE;
    if (nheads > (int64_t(1) << 20) || headdim > (int64_t(1) << 20) || batch * nheads >= (int64_t(1) << 31) ||
        batch * nheads * headdim * dstate >= (int64_t(1) << 46))
        return SSD_ERR_SHAPE;
    if (dstate < 4 || dstate > 256 || (dstate & (dstate - 1)) != 0) return SSD_ERR_UNSUPPORTED;
    // the state is read and written as 16-byte vectors; the others element by element
    const uintptr_t esz = dtype == SSD_BF16 ? 2 : 4;
    if (!aligned16(h)) return SSD_ERR_ALIGN;
    const void* ep[] = {x, B, C, y};
    for (const void* p : ep)
        if (reinterpret_cast<uintptr_t>(p) % esz) return SSD_ERR_ALIGN;
    const void* fp[] = {dt, A, D};
    for (const void* p : fp)
        if (p && reinterpret_cast<uintptr_t>(p) % 4) return SSD_ERR_ALIGN;
    const int st = cls_ssd_step_launch(h, x, dt, A, B, C, D, y, batch, nheads, headdim, dstate, ngroups, dtype,
                                       static_cast<hipStream_t>(stream));
    return st == 0 ? SSD_OK : (st == -8 ? SSD_ERR_UNSUPPORTED : SSD_ERR_HIP);
}

}  // extern "C"
