// Internal launch interface between the C ABI (api.cpp) and the kernel
// translation units.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct SsdShape {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int dtype;
};

namespace cls {
// Segment plan of the fused SSD path: each split chain is cut into nsegs
// segments, and the last nsplit (batch, head) chains are split (the others run
// whole).
struct SegChoice {
    int64_t nsegs, nsplit;
    int64_t agg_d = 0;  // aggregate pieces per segment (0: the heuristic's)
    int s3 = 0;         // inter-segment scheme (SSD_S3_*; 0: the built-in choice)
    int64_t sub = 0;    // sub-chunk the kernel runs (0: the chunk, at most 128)
    int nt = 0;         // cache policy of x loads and y stores: 0 the heuristic's, 1 default, 2 non-temporal
};
}  // namespace cls

// Per-call choices of ssd_fwd_planned (ssd_fwd passes the defaults).
struct SsdLaunchOpts {
    int path = 0;                          // SSD_PATH_*
    int s3 = 0;                            // SSD_S3_*
    const cls::SegChoice* force = nullptr;  // segment plan, or null: tuned or heuristic
    int xcds = 0;                          // XCDs of the chain mapping (0: the device's)
    hipEvent_t* ev = nullptr;              // four events to record, or null
    uint32_t stress = 0;                   // look-back stress seed of the segment look-back (0: none)
    int policy = 0;                        // x/y cache policy: 0 the plan's, 1 default, 2 non-temporal
    int csrc = 0;                          // C source of the state term: 0 the plan's, 1 copy, 2 C rows
};

struct SsdArgs {
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* h0;
    void* y;
    float* h_final;
    void* workspace;
};

// Size of the fixed device array behind linear_scan_noalloc.
#define CLS_NOALLOC_SCAN_SCRATCH_BYTES (1u << 20)

extern "C" {
// Device address of the current device's fixed scratch array (looked up
// once per device); 0 or -7.
int cls_noalloc_scratch(void** ptr);
// Zero `bytes` (a multiple of 16) at p with a store kernel on `stream`.
int cls_zero_fill(void* p, size_t bytes, hipStream_t stream);
// a, b and h: fp32 (format 0), bf16 (1) or fp16 (2); hs = 1: the
// Hillis-Steele in-tile scan (fp32 only); tile: elements per tile, 8192, or
// 4096 or 16384 for fp32 without hs (else -2); stress: look-back stress seed
// (fp32 without hs; 0: none).
int cls_launch_linear_scan(const void* a, const void* b, void* h, int64_t rows, int64_t L, int in_fmt, int out_fmt,
                           int segmented, int tiles_per_row, int rows_per_tile, int64_t ntiles,
                           uint32_t* claim, uint32_t* done, void* status, uint32_t* err,
                           hipStream_t stream, int hs, int tile, uint32_t stress);

// Shape/dtype/chunk validation shared by sizing and launching (SSD_OK or a
// negative status).
int cls_ssd_check(const SsdShape& s);
size_t cls_ssd_workspace_bytes(const SsdShape& s);
int cls_ssd_launch(const SsdShape& s, const SsdArgs& a, const SsdLaunchOpts& o, hipStream_t stream);
// Workspace bytes of the plan a call with these options runs (0 for paths
// without a workspace, and for a bf16 plan that cannot run the shape).
size_t cls_ssd_plan_bytes(const SsdShape& s, const SsdLaunchOpts& o);
// Times the fused path's candidate segment plans on these arguments, keeps the
// fastest for the shape and leaves its result in y / h_final (blocking).
int cls_ssd_autotune(const SsdShape& s, const SsdArgs& a, hipStream_t stream, int reps, int64_t* nsegs,
                     int64_t* nsplit, int64_t* agg_pieces, int64_t* sub_chunk, int* s3, int* policy, float* ms);
// The segment plan ssd_fwd uses for a shape: 1 tuned, 0 heuristic, 2 no plan
// (not the fused path); negative status on error.
int cls_ssd_plan_query(const SsdShape& s, int64_t* nsegs, int64_t* nsplit, int64_t* agg_pieces, int64_t* sub_chunk,
                       int* s3, int* policy);
void cls_ssd_autotune_reset();
// h[i] = a[i] b[i] for i < n (stream_ceiling.hip): n a multiple of 4, vec 1,
// 2, 4 or 8 (else -2), nt 0 or 1, grid_blocks 0 (one pass) or the grid of a
// grid-stride loop; arguments already validated.
int cls_launch_stream_mul(const float* a, const float* b, float* h, int64_t n, int vec, int nt,
                          int64_t grid_blocks, hipStream_t s);
// Three-pass linear scan (linear_scan_3pass.hip); shapes already validated.
size_t cls_ls3_workspace_bytes(int64_t rows, int64_t L);
int cls_ls3_launch(const float* a, const float* b, float* h, int64_t rows, int64_t L, void* ws, hipStream_t stream);
// One decode token (ssd_step.hip); shapes already validated.  0, or -7 when the
// launch fails, -8 for a state size without a kernel.
int cls_ssd_step_launch(float* h, const void* x, const float* dt, const float* A, const void* B,
                        const void* C, const float* D, void* y, int64_t batch, int64_t nheads,
                        int64_t headdim, int64_t dstate, int64_t ngroups, int dtype, hipStream_t stream);
}
