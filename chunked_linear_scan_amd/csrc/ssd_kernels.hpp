// Internal declarations shared by the SSD kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cls {

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
};

size_t ssd_f32_lds_bytes(int P, int S);
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
    int64_t batch, L;
    int H, G, chunk, nchunks;
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
int ssd_bf16_launch(int TT, int P, int S, const SsdBf16Params& prm, hipStream_t stream);

}  // namespace cls
