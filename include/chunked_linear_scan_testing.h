/*
 * chunked_linear_scan — entry point for tests and measurement.
 *
 * ssd_fwd chooses its kernels and, on the fused bf16 path, its
 * segment plan by itself (a tuned plan from ssd_fwd_autotune, else a built-in
 * heuristic).  ssd_fwd_planned is ssd_fwd with that choice made explicitly by
 * the caller, per call: parity tests use it to force every plan shape (whole
 * chains, split chains, one-chunk segments, the per-(batch, head) kernel, each
 * inter-chunk state scheme), and the benchmark uses it to time the launches of
 * one call separately.  Nothing it sets outlives the call: the library keeps
 * no override state between calls.
 */
#ifndef CHUNKED_LINEAR_SCAN_TESTING_H
#define CHUNKED_LINEAR_SCAN_TESTING_H

#include <stdint.h>

#include "chunked_linear_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel choice of one call. */
enum {
    SSD_PATH_AUTO = 0,   /* what ssd_fwd would run                                 */
    SSD_PATH_CHUNK = 1,  /* the per-(batch, head) chunk kernel (any bf16 shape)    */
    SSD_PATH_FUSED = 2   /* the fused kernels, head dim 64 or 128 (falls back to
                            AUTO where they do not apply)                          */
};

/* Where the fused path's state term y = C h^T reads C ("Accelerating Mamba-2
 * with high-performance forward pass kernels in NVIDIA cuTile", section
 * "Kernel 3: compute_out").  The values are the same either way, and so is
 * every bit of y and h_final. */
enum {
    SSD_CSRC_AUTO = 0,  /* the plan's choice: the C rows when a group has at most
                           8 chains of head dim 64, else the copy              */
    SSD_CSRC_COPY = 1,  /* a fragment-major copy of C that the CB pass writes
                           into the workspace                                 */
    SSD_CSRC_ROWS = 2   /* the C rows of the input (no copy in the workspace)  */
};

/* The inter-segment schemes (SSD_S3_AUTO, SSD_S3_REDUCE, SSD_S3_LOOKBACK) are
 * declared in chunked_linear_scan.h ("Selective-scan CUDA kernels", section
 * "The five kernels", levels 2 and 3). */

typedef struct {
    int32_t path;        /* SSD_PATH_*                                               */
    int32_t s3;          /* SSD_S3_*                                                 */
    int64_t nsegs;       /* segments per split chain, 1..64; 0: tuned or heuristic
                            (the per-(batch, head) and fp32 kernels cut every
                            chain into nsegs segments, at most one per sub-chunk;
                            nsplit and agg_pieces do not apply to them)            */
    int64_t nsplit;      /* with nsegs: split only the last nsplit (batch, head)
                            chains, the others run whole; 0: split every chain
                            (a head of dim 128 is two chains of dim 64)            */
    int64_t agg_pieces;  /* with nsegs and SSD_S3_REDUCE: aggregate pieces per
                            segment; 0: the heuristic's count                      */
    int32_t xcds;        /* XCDs the workgroups are dealt across (chain mapping
                            only); 0: the device's 8; 1: plain index order          */
    int32_t sub_chunk;   /* with nsegs: the sub-chunk the kernels run (32 or 64, a
                            divisor of the chunk capped at 128); 0: that cap      */
    uint32_t stress_seed; /* look-back stress (SSD_S3_LOOKBACK plans): 0, or a seed
                            by which about one segment in four waits a pseudo-
                            random 0 to 31 sleeps of ~8K clocks before it
                            publishes, so segments publish out of order; the
                            results must not change ("Selective-scan CUDA
                            kernels", section "Correctness")                      */
    int32_t cache_policy; /* SSD_CACHE_*: the x/y cache policy (128-token sub-chunks
                            only); 0: the plan's choice                            */
    int32_t c_source;     /* SSD_CSRC_*: where the fused path's state term reads C */
} ssd_plan_request;

/*
 * ssd_fwd with an explicit plan.  All of ssd_fwd's arguments, layouts,
 * checks, workspace rules and status codes apply.  `plan` may be NULL (then
 * this is ssd_fwd).  Fields outside their ranges return SSD_ERR_SHAPE before
 * anything is launched.  A forced segment plan may need more workspace than
 * ssd_fwd_workspace_size reports (which covers the plans ssd_fwd itself may
 * run): size it with ssd_fwd_planned_workspace_size; a smaller workspace
 * returns SSD_ERR_WORKSPACE.
 *
 * events: NULL, or four hipEvent_t handles (created by the caller, owned by
 * the caller) that are recorded on `stream`: before the call's first launch,
 * after the CB pass, after the aggregate launch (recorded also when there is
 * none) and after the output launch.  On paths with a single launch events
 * 1 and 2 are recorded right after event 0.
 */
int ssd_fwd_planned(const void* x, const float* dt, const float* A, const void* B,
                    const void* C, const float* D, const float* h0,
                    int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                    int64_t dstate, int64_t ngroups, int64_t chunk, int dtype,
                    void* y, float* h_final, void* workspace, size_t workspace_bytes,
                    void* stream, const ssd_plan_request* plan, void* const* events);

/* Workspace bytes ssd_fwd_planned needs for this shape and plan (at least
 * ssd_fwd_workspace_size); 0 for an invalid shape or plan. */
size_t ssd_fwd_planned_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                      int64_t headdim, int64_t dstate, int64_t ngroups,
                                      int64_t chunk, int dtype, const ssd_plan_request* plan);

/*
 * linear_scan with the tile size chosen by the caller: tile 4096, 8192 or
 * 16384 elements (0: what linear_scan would run for the shape), else
 * SSD_ERR_SHAPE.  Parity tests use it to run every tile instance; nothing it
 * sets outlives the call.  All of linear_scan's arguments, checks, workspace
 * rule (linear_scan_workspace_size covers every tile) and status codes
 * apply.
 *
 * stress_seed: 0, or a look-back stress run ("Selective-scan CUDA kernels",
 * section "Correctness": look-back races show up only under other
 * schedules).  About one tile in four, chosen by a hash of the seed, the row
 * and the tile, then waits a pseudo-random 0 to 31 sleeps of about 8K clocks
 * each before it publishes and looks back, so tiles publish out of order.
 * The results must equal those of the unperturbed call bit for bit (the
 * look-back's combine order does not depend on timing).
 */
int linear_scan_planned(const float* a, const float* b, float* h, int64_t rows, int64_t length,
                        int64_t tile, uint32_t stress_seed, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * A plain streaming kernel with linear_scan's HBM traffic: h[i] = a[i] * b[i]
 * for 0 <= i < n (read two fp32 arrays, write one).  It is no part of the
 * scan: it measures what a kernel that only streams those bytes reaches on
 * the device, the ceiling the scan's bandwidth is read against.
 *
 * a, b, h: n fp32 each, 16-byte aligned; h must not alias a or b.  n: a
 * positive multiple of 4, at most 2^40.  vec: 16-byte vectors of each array a
 * thread moves per iteration, 1, 2, 4 or 8.  nt: 1 for non-temporal loads and
 * stores (the scan's policy), 0 for the default policy.  grid_blocks: 0 for
 * one pass (one 256-thread workgroup per 256 * vec vectors), else 1 .. 2^23
 * workgroups in a grid-stride loop.  Returns SSD_OK, SSD_ERR_NULL,
 * SSD_ERR_ALIGN, SSD_ERR_SHAPE (n, vec, nt or grid_blocks out of range, or a
 * one-pass grid above 2^23 workgroups) or SSD_ERR_HIP.  Asynchronous on
 * `stream`.
 */
int stream_mul_f32(const float* a, const float* b, float* h, int64_t n, int vec, int nt,
                   int64_t grid_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKED_LINEAR_SCAN_TESTING_H */
