// Timing loop shared by the autotuners (the SSD fused path's plans and the
// linear scan's tile): candidate 0 is the built-in choice, the incumbent.
//
// After one untimed call of every candidate, each runs `reps` times between
// two events on the caller's stream, in two rounds, and keeps its better
// round.  The fastest challenger replaces the incumbent only when it is faster
// by more than the incumbent's own round-to-round spread (at least 1 %), and
// again by that margin in a head-to-head of three alternating rounds (medians
// compared); so a tuned choice never loses to the built-in one by more than
// the noise.  Blocking: waits for each timed round.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

namespace cls {

// run(i) enqueues candidate i once on `stream` and returns 0 or a negative
// status.  On success *chosen is the winner's index and *chosen_ms its
// mean time per call (ms); returns 0, the first negative status of run(), or
// hip_error when an event call fails.
template <typename Run>
int tune_candidates(size_t n, Run&& run, hipStream_t stream, int reps, int hip_error, size_t* chosen,
                    float* chosen_ms) {
    *chosen = 0;
    *chosen_ms = 0.0f;
    if (n == 0) return 0;
    if (reps < 1) reps = 1;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return hip_error;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return hip_error;
    }
    int st = 0;
    // mean ms per call of candidate i over `reps` calls (after one untimed call)
    auto time_one = [&](size_t i, float* out) {
        st = run(i);
        if (st != 0) return;
        if (hipEventRecord(e0, stream) != hipSuccess) {
            st = hip_error;
            return;
        }
        for (int r = 0; r < reps && st == 0; ++r) st = run(i);
        if (st != 0) return;
        float t = 0.0f;
        if (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&t, e0, e1) != hipSuccess) {
            st = hip_error;
            return;
        }
        *out = t / float(reps);
    };
    for (size_t i = 0; i < n && st == 0; ++i) st = run(i);
    std::vector<float> best(n, -1.0f);
    float inc_round[2] = {0.0f, 0.0f};  // the incumbent's two rounds
    for (int round = 0; round < 2 && st == 0; ++round)
        for (size_t i = 0; i < n && st == 0; ++i) {
            float t = 0.0f;
            time_one(i, &t);
            if (st != 0) break;
            if (i == 0) inc_round[round] = t;
            if (best[i] < 0.0f || t < best[i]) best[i] = t;
        }
    size_t pick = 0;
    float pick_ms = best[0];
    if (st == 0 && n > 1) {
        size_t ch = 1;
        for (size_t i = 2; i < n; ++i)
            if (best[i] < best[ch]) ch = i;
        const float lo = std::min(inc_round[0], inc_round[1]);
        const float spread = lo > 0.0f ? std::fabs(inc_round[0] - inc_round[1]) / lo : 0.0f;
        const float margin = std::max(spread, 0.01f);
        if (best[ch] < best[0] * (1.0f - margin)) {
            float ti[3], tc[3];
            for (int k = 0; k < 3 && st == 0; ++k) {
                time_one(0, &ti[k]);
                if (st == 0) time_one(ch, &tc[k]);
            }
            if (st == 0) {
                std::sort(ti, ti + 3);
                std::sort(tc, tc + 3);
                if (tc[1] < ti[1] * (1.0f - margin)) {
                    pick = ch;
                    pick_ms = tc[1];
                } else {
                    pick_ms = ti[1];
                }
            }
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != 0) return st;
    *chosen = pick;
    *chosen_ms = pick_ms;
    return 0;
}

}  // namespace cls
