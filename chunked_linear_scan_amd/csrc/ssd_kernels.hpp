// Internal declarations shared by the SSD kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cls {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct SsdF32Params {
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* h0;
    void* y;
    float* h_final;
    int64_t batch, L;
    int H, P, S, G, chunk;
    // chains cut into nsegs segments of seg_chunks chunks (nsegs <= 1: whole
    // chains), as for the per-(batch, head) bf16 kernel: the aggregate launch
    // writes every segment's state but a chain's last ([P][S], from a zero
    // start) and its natural-log decay; each segment folds its predecessors'.
    int nsegs, seg_chunks;
    float* seg_state;  // [chains][nsegs - 1][P][S]
    float* seg_decay;  // [chains][nsegs - 1]
};

size_t ssd_f32_lds_bytes(int P, int S);
size_t ssd_f32_launch_lds(int P, int S, int T);  // LDS of one workgroup as launched (staged chunks included)
int ssd_f32_launch(const SsdF32Params& prm, hipStream_t stream);

struct SsdBf16Params {
    const uint16_t* x;   // bf16 [Bt, L, H, P]
    const float* dt;     // [Bt, L, H]
    const float* A;      // [H]
    const uint16_t* B;   // bf16 [Bt, L, G, S]
    const uint16_t* C;   // bf16 [Bt, L, G, S]
    const float* D;      // [H] or null
    const float* h0;     // [Bt, H, P, S] or null
    uint16_t* y;         // bf16 [Bt, L, H, P]
    float* h_final;      // [Bt, H, P, S] or null
    uint16_t* cb;        // workspace: bf16 [Bt, Nc, G, TT, TT]
    uint16_t* bt;        // workspace: bf16 [Bt, Nc, G, S, TT] (B^T), or null when not needed
    uint16_t* cf;        // workspace of the fused path: bf16 C fragments [Bt, Nc, G, TT * S], or null
    float* dtt;          // workspace of the fused path: dt per head, token-contiguous [Bt, Nc, H, TT], zero
                         // past the sequence end, or null
    int64_t batch, L;
    int H, G, chunk, nchunks;
    // per-(batch, head) kernel: H counts heads of dim P >> hshift; a head of
    // dim P runs as 1 << hshift adjacent heads (its channels are independent,
    // and x, y, h0 and h_final hold them at the same addresses), and head h
    // reads dt, A and D of head h >> hshift
    int hshift;
    // per-(batch, head) kernel: each chain cut into nsegs segments of
    // seg_chunks sub-chunks (nsegs <= 1: whole chains).  The aggregate launch
    // writes the state of every segment but a chain's last, from a zero start,
    // and its log2 decay; a segment's workgroup folds its predecessors' into
    // its start state (reduce-then-fold).
    int nsegs, seg_chunks;
    float* seg_state;  // [chains][nsegs - 1][chunk_state_floats(P >> hshift, S)]
    float* seg_decay;  // [chains][nsegs - 1]
};

struct SsdFusedParams {
    const uint16_t* x;
    const float* dt;
    const float* A;
    const uint16_t* B;
    const uint16_t* C;
    const float* D;
    const float* h0;
    uint16_t* y;
    float* h_final;
    const uint16_t* cb;
    const uint16_t* bt;
    const uint16_t* cf;
    const float* dtt;
    float* payload;      // [pieces][threads][state floats per lane] aggregates, then [pieces] decays
    uint32_t* err;
    int64_t batch, L;
    // chains [0, nwhole) run whole; chains [nwhole, nchains) are split into
    // nsegs segments of seg_chunks chunks.  The aggregate launch covers the
    // segments but the last of every split chain, as agg_d pieces of at most
    // agg_chunks chunks per segment.
    int H, G, chunk, nchunks, seg_chunks, nsegs, nchains, nwhole;
    // H counts heads of dim 64.  A head of dim 64 << hshift runs as 1 << hshift
    // adjacent heads of dim 64 (its channels are independent, and x, y, h0 and
    // h_final hold them at the same addresses either way); head h reads dt, A
    // and D of head h >> hshift.
    int hshift;
    int agg_d, agg_chunks;
    int nxcd;  // XCDs the workgroups are dealt across (tile mapping only)
    // Single-pass look-back over the segments of split chains (no aggregate
    // launch).  The output launch's segment workgroups claim their segment
    // from one counter per range of split chains, run the segment's own
    // aggregate (all segments but a chain's last), publish it, look back over
    // the chain's earlier segments and then run the output pass.
    int lookback;        // 1: this scheme; 0: reduce-then-fold over the aggregate launch's pieces
    int nranges;         // claim ranges: contiguous runs of whole split chains
    uint32_t* seg_ctl;   // [0] epoch of the call, [1] finished segments, [16 + r] claims of range r
    uint64_t* seg_status;  // [segments] tagged status words
    float* seg_pay;      // [2][segments][compute threads][state floats per lane]: aggregates, prefixes
    float* seg_alpha;    // [segments] decays of the aggregates
    uint32_t stress;     // look-back stress seed (tests only; 0: none)
};

// A head of dim 64 << fused_head_shift(P) runs on the fused path as that
// many adjacent chains of head dim 64 (P = 64 or 128).
constexpr int fused_head_shift(int64_t P) { return P == 128 ? 1 : 0; }

// Plan of the fused path (head dim 64, or 128 as two heads of 64) for one
// shape (also sizes its workspace).
constexpr int64_t kFusedMaxChunk = 128;  // longest quadratic block of the fused kernel

// The first bytes of every bf16 SSD workspace: the error word at 0 and the
// look-back control words (epoch, finish count, claim counters) at
// [kSsdCtlOff, kSsdWsHeader).  No plan puts data there, so the control words
// stay valid whichever plans and shapes share a workspace.
constexpr size_t kSsdCtlOff = 256;
constexpr size_t kSsdWsHeader = 1024;

struct SsdFusedPlan {
    bool use;
    int TT, chunk, nsegs, seg_chunks, nchains, nwhole;  // chunk: the sub-chunk the kernel runs
    int agg_d, agg_chunks, npieces;                     // aggregate pieces (see SsdFusedParams)
    bool lookback;                                      // split chains: single-pass look-back
    bool nt;                                            // non-temporal x loads and y stores
    bool cdirect;                                       // state term reads the C rows (no C copy)
    int nranges;                                        // look-back claim ranges
    size_t payload_off, cb_off, bt_off, cf_off, dtt_off, bytes;
    size_t status_off, segpay_off, alpha_off;           // look-back status words and payloads
};

// Tile sizes of the bf16 path: the chunk is padded to a multiple of 32 tokens.
constexpr int bf16_tile_tokens(int chunk) { return chunk < 32 ? 32 : chunk; }

// LDS bytes of the bf16 chunk kernel for a tile of TT tokens.
constexpr size_t ssd_bf16_lds_bytes(int TT, int P, int S) {
    return size_t(P) * (TT + 8) * 2 + size_t(S) * (TT + 8) * 2 + size_t(P) * (S + 8) * 2 +
           3 * size_t(TT) * 4 + 64;
}

constexpr bool ssd_bf16_lds_fits(int TT, int P, int S) {
    return size_t(P) * (TT + 8) * 2 + size_t(S) * (TT + 8) * 2 + size_t(P) * (S + 8) * 2 +
               3 * size_t(TT) * 4 + 64 <= size_t(160) * 1024;
}

bool ssd_bf16_supported(int TT, int P, int S);
constexpr int kChunkMaxTile = 128;  // longest sub-chunk of the per-(batch, head) kernel
int chunk_kernel_tile(int64_t chunk, int P, int S);
// floats of one segment state of the per-(batch, head) kernel (head dim P):
// its four waves' fp32 state fragments, state tiles wave, wave + 4, ..
constexpr size_t chunk_state_floats(int P, int S) { return size_t((S / 16 + 3) / 4) * (P / 16) * 256 * 4; }

size_t ssd_fused_lds_bytes(int TT, int S);
int ssd_fused_state_floats(int S);  // floats of one [64, S] state
// ev: null, or three events recorded before the CB pass, between the passes
// and after the fused kernel (measurement hook)
// CB pass, then (with split chains) the aggregate launch, then the output
// launch; ev (optional): four events, before and between the launches.
int ssd_fused_launch(int TT, int S, const SsdBf16Params& cbp, const SsdFusedParams& fp, hipStream_t stream,
                     hipEvent_t* ev, bool nt);
SsdFusedPlan ssd_fused_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t S, int64_t G,
                            int64_t chunk, int dtype);
constexpr int kXcds = 8;  // MI355X: 8 XCDs of 32 CUs
int ssd_bf16_launch(int TT, int P, int S, const SsdBf16Params& prm, hipStream_t stream);

}  // namespace cls
