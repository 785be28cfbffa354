/*
 * chunked_linear_scan — MI355X (gfx950) Mamba-2 SSD chunked forward pass and
 * scalar linear scan behind a plain C ABI.
 *
 * Every entry point takes plain pointers and sizes.  Device pointers are HIP
 * device memory on the current device; `stream` is a hipStream_t passed as
 * void* (NULL = the default stream).  All work is enqueued on that stream and
 * nothing synchronises the host, except ssd_fwd_autotune, which waits for its
 * own timed runs.  The library never allocates or frees device
 * memory: the caller owns every buffer, including the workspace.
 *
 * Errors: arguments are validated on the host before anything is launched.
 * A negative status means nothing was enqueued (except SSD_ERR_HIP, which is
 * returned when a launch itself fails).  No exceptions cross this boundary.
 *
 * Workspace contract: size it with the matching *_workspace_size call, fill it
 * with zero bytes once before its first use, and keep it for later calls of
 * any shape that fits it: the kernels keep it consistent from call to call
 * (per-call epochs and counters the kernels themselves advance or reset), so
 * it is never cleared again.  Calls that share a workspace must be ordered on
 * one stream.  After a call that returned an error from a launch, zero the
 * workspace again.
 */
#ifndef CHUNKED_LINEAR_SCAN_H
#define CHUNKED_LINEAR_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,        /* a required pointer is NULL                      */
    SSD_ERR_SHAPE = -2,       /* a size is <= 0, or heads % groups != 0          */
    SSD_ERR_DTYPE = -3,       /* dtype is not SSD_F32 or SSD_BF16                */
    SSD_ERR_CHUNK = -4,       /* chunk is not one of 16, 32, 64, 128, 256        */
    SSD_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                */
    SSD_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required         */
    SSD_ERR_HIP = -7,         /* a HIP launch failed                             */
    SSD_ERR_UNSUPPORTED = -8  /* head dim / state size outside the kernel's set  */
};

/* Element types of x, B, C and y (SSD_F32, SSD_BF16); dt, A, D and both
 * states are always fp32.  The scan's elements may also be SSD_F16. */
enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_F16 = 2 };

/*
 * Mamba-2 SSD (state-space duality) chunked forward pass.
 *
 * Computes, per batch b and head h, the recurrence of "Accelerating Mamba-2
 * with high-performance forward pass kernels in NVIDIA cuTile", section
 * "Mamba-2 architecture":
 *     h_t = exp(A[h] dt_t) h_{t-1} + dt_t B_t x_t^T,   y_t = c_t^T h_t + D[h] x_t
 * with h_{-1} = h0, evaluated chunk by chunk as in that page's three kernel
 * sections (cumulative sum of A dt inside each chunk, the state at each chunk
 * start, the per-chunk output).  The output uses the token's own updated
 * state (causal mask that keeps the diagonal).  Head h reads B/C group
 * h / (nheads / ngroups).
 *
 * Layouts (row-major, contiguous, 16-byte aligned):
 *   x, y      [batch, seqlen, nheads, headdim]   dtype
 *   dt        [batch, seqlen, nheads]            fp32
 *   A, D      [nheads]                           fp32  (D may be NULL = 0)
 *   B, C      [batch, seqlen, ngroups, dstate]   dtype
 *   h0        [batch, nheads, headdim, dstate]   fp32  (may be NULL = zeros)
 *   h_final   [batch, nheads, headdim, dstate]   fp32  (may be NULL = not written)
 *
 * chunk: 16, 32, 64, 128 or 256 tokens; seqlen need not be a multiple of it.
 * The decay exponents A[h] dt_t are expected to be <= 0 (decays in (0, 1]);
 * the kernels rely on that to never keep a positive exponent.
 *
 * SSD_BF16 runs the MFMA path (bf16 operands, fp32 accumulation and fp32
 * state) for headdim in {16, 32, 64, 128} and dstate in {32, 64, 128, 256},
 * at every chunk length (SSD_ERR_UNSUPPORTED otherwise;
 * ssd_fwd_workspace_size returns 0 then).  Head dim 64 or 128 with dstate 64
 * or 128 runs the fused kernels (a head of dim 128 as two heads of dim 64,
 * whose channels are independent); the other shapes run the per-(batch,
 * head) kernel.  Both run a chunk longer than their tiles (128 tokens, or
 * less where the per-(batch, head) kernel's tiles would overflow LDS) as
 * sub-chunks, which changes the result only by rounding.
 * SSD_F32 runs an fp32 path for any shape with headdim * dstate <= 16384 and
 * headdim, dstate multiples of 4.
 *
 * Outputs must not alias inputs.  Returns SSD_OK or a negative status.
 */
size_t ssd_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                              int64_t headdim, int64_t dstate, int64_t ngroups,
                              int64_t chunk, int dtype);

int ssd_fwd(const void* x, const float* dt, const float* A, const void* B,
            const void* C, const float* D, const float* h0,
            int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
            int64_t dstate, int64_t ngroups, int64_t chunk, int dtype,
            void* y, float* h_final, void* workspace, size_t workspace_bytes,
            void* stream);

/*
 * Per-shape autotuning of ssd_fwd ("Accelerating Mamba-2 with high-performance
 * forward pass kernels in NVIDIA cuTile", section "Mamba-2 performance
 * optimization", its autotuner item: a search per input shape, since no one
 * setting suits every shape).  The run-time choices of the fused bf16
 * path form its plan:
 *   - the segment plan: how many segments a long (batch, head) chain is cut
 *     into, which chains are cut, and, for reduce-then-fold, how many pieces
 *     the aggregate launch cuts each segment into;
 *   - how a cut chain's segments get their start state: reduce-then-fold (an
 *     aggregate launch, then a fold) or the single-pass look-back
 *     ("Selective-scan CUDA kernels", section "The five kernels");
 *   - the sub-chunk the kernels run: the chunk up to 128 tokens, or 64 (a
 *     different instantiation of the kernels: its tiles, register and LDS
 *     budget; results differ only by rounding);
 *   - the cache policy of the x loads and y stores (128-token sub-chunks):
 *     default, or non-temporal (a separate instantiation; results are
 *     identical bit for bit).  The heuristic takes non-temporal when a
 *     workgroup walks at least 32 sub-chunks.
 * Tile shapes and occupancy within each instantiation are fixed at compile
 * time.
 *
 * ssd_fwd_autotune takes exactly ssd_fwd's arguments (same layouts, same
 * checks, same workspace) plus reps (1..1000).  The built-in heuristic's plan
 * is the incumbent.  Every distinct candidate runs once untimed, then in two
 * rounds reps times between two events on `stream`, keeping its better round.
 * The fastest challenger replaces the incumbent only if it is faster by more
 * than the incumbent's round-to-round spread (at least 1 %), and again by that
 * margin in a head-to-head of three alternating rounds.  The chosen plan is
 * kept for this shape on the current device; later ssd_fwd calls with the
 * same shape, dtype and chunk on that device use it.  It returns the chosen
 * plan (*nsegs segments, the last *nsplit chains cut, *agg_pieces aggregate
 * pieces per segment, each 0 when nothing is cut or not applicable;
 * *sub_chunk tokens per sub-chunk; *s3 = SSD_S3_REDUCE or SSD_S3_LOOKBACK
 * when chains are cut, else 0; *cache_policy = SSD_CACHE_DEFAULT or
 * SSD_CACHE_NONTEMPORAL) and its time per call in ms.  y and h_final
 * hold the result of the chosen plan, which is what ssd_fwd then returns.
 * Shapes outside the fused path have nothing to tune: one plain ssd_fwd pass,
 * all outputs 0.  The call blocks until its timed runs finish.  The table is
 * process-wide and guarded by a lock; tuning while other calls of the same
 * shape run changes their plan only between calls.  ssd_fwd_workspace_size
 * already covers every candidate plan, so a workspace sized before tuning
 * stays large enough.  Every plan computes the same recurrence; results
 * differ only by fp32 rounding.
 *
 * ssd_fwd_plan reports the plan ssd_fwd would use for a shape without
 * launching anything (same outputs as ssd_fwd_autotune; *sub_chunk 0 and all
 * others 0 for shapes outside the fused path): returns 1 (a tuned plan), 0
 * (the built-in heuristic), 2 (the shape does not take the fused path) or a
 * negative status.  ssd_fwd_autotune_reset forgets every tuned plan.
 */
/* Cache policy of the x loads and y stores of the fused path. */
enum {
    SSD_CACHE_AUTO = 0,        /* the plan's choice (in a plan request)                 */
    SSD_CACHE_DEFAULT = 1,     /* the default policy                                    */
    SSD_CACHE_NONTEMPORAL = 2  /* non-temporal: x and y are touched once per launch     */
};

/* How a cut chain's segments get their start state. */
enum {
    SSD_S3_AUTO = 0,      /* the library's choice (in a plan request)                */
    SSD_S3_REDUCE = 1,    /* reduce-then-fold: an aggregate launch computes every
                             piece's (decay, state), the output launch folds them   */
    SSD_S3_LOOKBACK = 2   /* single pass: segments claimed from a counter publish
                             their aggregate and look back over their predecessors  */
};

int ssd_fwd_autotune(const void* x, const float* dt, const float* A, const void* B,
                     const void* C, const float* D, const float* h0,
                     int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                     int64_t dstate, int64_t ngroups, int64_t chunk, int dtype,
                     void* y, float* h_final, void* workspace, size_t workspace_bytes,
                     void* stream, int reps, int64_t* nsegs, int64_t* nsplit,
                     int64_t* agg_pieces, int64_t* sub_chunk, int* s3, int* cache_policy,
                     float* ms_per_call);

int ssd_fwd_plan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                 int64_t dstate, int64_t ngroups, int64_t chunk, int dtype,
                 int64_t* nsegs, int64_t* nsplit, int64_t* agg_pieces,
                 int64_t* sub_chunk, int* s3, int* cache_policy);

void ssd_fwd_autotune_reset(void);

/*
 * Scalar linear recurrence of "Selective-scan CUDA kernels", section "The
 * problem":  h[r, t] = a[r, t] h[r, t-1] + b[r, t],  h[r, -1] = 0,
 * independently for each of `rows` rows of `length` elements.
 *
 * Layout: a, b, h are [rows, length] fp32, row-major, contiguous, 16-byte
 * aligned at the base (rows need not be aligned).  One single-pass kernel:
 * each row is split into tiles that look back over their predecessors in
 * one 64-wide window (decoupled look-back).  The look-back is anchored: every
 * 64th tile of a row publishes its inclusive prefix, the others only their
 * aggregate, and each tile folds from its anchor.  The combine order depends
 * on the tile index alone, so the result is bit-identical from run to run
 * whatever order tiles finish in.  h must not alias a or b.
 *
 * A tile is 8192 elements unless linear_scan_autotune has chosen another
 * size (4096 or 16384) for this shape on this device; the tile changes only
 * the fp32 rounding order.  linear_scan_workspace_size covers every tile
 * size: 256 bytes for rows of up to 4090 elements, else 256 + 8 bytes per row
 * (rounded up to 256 bytes twice) + 16 bytes per 4096-element tile of every
 * row.
 */
size_t linear_scan_workspace_size(int64_t rows, int64_t length);

int linear_scan(const float* a, const float* b, float* h, int64_t rows,
                int64_t length, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * linear_scan for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same scan, kernels and results as linear_scan (bit for bit), with the
 * workspace taken from a fixed 1 MiB array in device memory that the library
 * holds on each GPU it runs on until the process ends, instead of a caller's
 * buffer.  Nothing is allocated or freed.  Each call first clears the part of
 * the array it uses with a store kernel on `stream`, then runs the scan.
 * Shapes whose workspace (linear_scan_workspace_size) exceeds 1 MiB return
 * SSD_ERR_WORKSPACE with nothing enqueued: rows of up to 4090 elements need
 * none beyond a 256-byte header, longer rows need 16 bytes per 4096 elements
 * plus 8 bytes per row.  It runs the tile linear_scan runs for the shape
 * (tuned or built-in).  All calls on one GPU share its array: calls
 * that may overlap on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.  Same layouts, alignment and status codes
 * as linear_scan.
 */
int linear_scan_noalloc(const float* a, const float* b, float* h, int64_t rows,
                        int64_t length, void* stream);

/*
 * Autotuner of linear_scan's tile size ("Accelerating Mamba-2 ...", section
 * "Optimizations", which closes with an autotuner that picks kernel settings
 * per input shape).  The tile size is a compile-time setting of the kernel;
 * fp32 instances exist for 4096, 8192 (the built-in choice, the incumbent)
 * and 16384 elements per tile.  Each runs `reps` times (1..10000) in two
 * timed rounds on the caller's arguments; a challenger replaces the built-in
 * tile only when faster by more than the built-in tile's own round-to-round
 * spread (at least 1 %), and again by that margin in a head-to-head of three
 * alternating rounds.  The winner is kept per (device, rows, length) for the
 * life of the process: later fp32 linear_scan, linear_scan_typed (fp32 in
 * and out) and linear_scan_noalloc calls of that shape use it.  On return h
 * holds what such a later call returns, *tile the chosen size and
 * *ms_per_call its mean time.  Blocking (waits for the timed rounds).  Same
 * arguments, workspace (linear_scan_workspace_size) and status codes as
 * linear_scan, plus SSD_ERR_NULL for tile or ms_per_call and SSD_ERR_SHAPE
 * for reps out of range.
 */
int linear_scan_autotune(const float* a, const float* b, float* h, int64_t rows,
                         int64_t length, void* workspace, size_t workspace_bytes,
                         void* stream, int reps, int64_t* tile, float* ms_per_call);

/* The tile an fp32 linear_scan of this shape runs on the current device:
 * returns 1 (tuned), 0 (built-in), or SSD_ERR_SHAPE / SSD_ERR_NULL. */
int linear_scan_plan(int64_t rows, int64_t length, int64_t* tile);

/* Forgets every tuned scan tile (all devices). */
void linear_scan_autotune_reset(void);

/*
 * linear_scan with fp32, bf16 or fp16 elements.  The page's scan is fp32 only
 * ("Selective-scan CUDA kernels", section "Limitations"); this entry point
 * takes a and b as in_dtype and writes h as out_dtype, each SSD_F32, SSD_BF16
 * or SSD_F16 (SSD_ERR_DTYPE otherwise).  16-bit elements are raw bits
 * (uint16_t).  The recurrence is evaluated in fp32 either way, exactly as
 * linear_scan does: 16-bit inputs are widened exactly, and a 16-bit h is the
 * fp32 result rounded to nearest even once (fp16: values past its range
 * become infinities).  Same layouts, workspace (size from
 * linear_scan_workspace_size), alignment, aliasing rule and status codes as
 * linear_scan; with both dtypes SSD_F32 it is linear_scan.
 */
int linear_scan_typed(const void* a, const void* b, void* h, int64_t rows,
                      int64_t length, int in_dtype, int out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same scan with a register-resident Hillis-Steele scan inside each tile:
 * the work-inefficient, step-efficient scan that "Selective-scan CUDA
 * kernels" (sections "Findings" and "Limitations") measures only as a
 * PyTorch baseline of full-array passes and names as the fair comparison
 * still to build.  Within each 256-item step of a wave, log2(256) = 8 rounds
 * combine every item with the one 1, 2, 4, ..., 128 places before it, all at
 * once, with items exchanged between lanes by shuffles: O(n log n) combines
 * instead of linear_scan's serial items plus wave scan.  Tiles, claims, the
 * look-back, the workspace and every argument rule are linear_scan's (fp32
 * elements; size the workspace with linear_scan_workspace_size).  Results
 * agree with linear_scan to fp32 rounding (the combine order differs) and are
 * the same from run to run.
 */
int linear_scan_hillis_steele(const float* a, const float* b, float* h, int64_t rows,
                              int64_t length, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The same scalar recurrence as three launches: block scan, spine scan over
 * the tile aggregates, prefix application ("Selective-scan CUDA kernels",
 * section "The five kernels", level 2).  It moves seven arrays' worth of
 * traffic where linear_scan moves three, and shares no code with it: an
 * independent cross-check of the single-pass kernel.  Same layouts and
 * alignment as linear_scan; h is also used as scratch between the passes.
 * The workspace (size from linear_scan_three_pass_workspace_size, 16-byte
 * aligned) needs no initial contents.  Results agree with linear_scan to
 * fp32 rounding (the combine order inside a tile differs), and are the same
 * from run to run.
 */
size_t linear_scan_three_pass_workspace_size(int64_t rows, int64_t length);

int linear_scan_three_pass(const float* a, const float* b, float* h, int64_t rows,
                           int64_t length, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * One decode token of the same recurrence, for sequential inference: the
 * recurrent form of "Accelerating Mamba-2 with high-performance forward pass
 * kernels in NVIDIA cuTile", section "Mamba-2 architecture", which that
 * section names as the one for generation.  Per batch b and head h:
 *     h <- exp(A[h] dt) h + dt B x^T,   y = c^T h + D[h] x
 * (the output sees the token's own update, as ssd_fwd's does).  ssd_fwd's
 * h_final is the state to continue a sequence from.
 *
 * Layouts (row-major, contiguous):
 *   h         [batch, nheads, headdim, dstate]   fp32, device, read and
 *                                                overwritten in place;
 *                                                16-byte aligned
 *   x, y      [batch, nheads, headdim]           dtype (y written)
 *   dt        [batch, nheads]                    fp32
 *   A, D      [nheads]                           fp32  (D may be NULL = 0)
 *   B, C      [batch, ngroups, dstate]           dtype
 * Head h reads group h / (nheads / ngroups).  dstate must be a power of two
 * from 4 to 256 (SSD_ERR_UNSUPPORTED otherwise); any headdim.  No workspace.
 * y must not alias an input.  Returns SSD_OK or a negative status (nothing
 * is enqueued on a validation error).
 */
int ssd_step(float* h, const void* x, const float* dt, const float* A,
             const void* B, const void* C, const float* D,
             int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
             int64_t ngroups, int dtype, void* y, void* stream);

/* Human-readable text for a status code (static storage). */
const char* ssd_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKED_LINEAR_SCAN_H */
