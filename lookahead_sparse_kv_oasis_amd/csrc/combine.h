// Merge of split-K attention partials (running max, normaliser, sum), shared
// by the combine of the decode attention and of the verification attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oasis {

// Partials merged per round trip of the combine.
constexpr int kCombineRegs = 24;

// Merge n partials (partial i at row pidx(i)) for output dimension c into a
// running (M, L, a): chunks of kCombineRegs partials, every load of a chunk
// issued up front (one round trip per chunk).  A single chunk is the plain
// max-subtracted merge.
template <typename F>
__device__ __forceinline__ void merge_partials(const float *__restrict__ part_m,
                                               const float *__restrict__ part_l,
                                               const float *__restrict__ part_acc, int d, int c,
                                               int n, F pidx, float &M, float &L, float &a) {
    for (int i0 = 0; i0 < n; i0 += kCombineRegs) {
        float pm[kCombineRegs], pl[kCombineRegs], pa[kCombineRegs];
#pragma unroll
        for (int k = 0; k < kCombineRegs; ++k) {
            pm[k] = -INFINITY;
            pl[k] = 0.f;
            pa[k] = 0.f;
            if (i0 + k < n) {
                const int64_t pi = pidx(i0 + k);
                pm[k] = part_m[pi];
                pl[k] = part_l[pi];
                pa[k] = part_acc[pi * d + c];
            }
        }
        // a partial marked empty (m = -inf) contributes nothing; its sums may
        // be stale
        float cm = -INFINITY;
#pragma unroll
        for (int k = 0; k < kCombineRegs; ++k) {
            if (pm[k] == -INFINITY) {
                pl[k] = 0.f;
                pa[k] = 0.f;
            }
            cm = fmaxf(cm, pm[k]);
        }
        if (cm == -INFINITY) continue;
        const float nm = fmaxf(M, cm);
        const float r = exp2f(M - nm);  // 0 while nothing was merged
        L *= r;
        a *= r;
#pragma unroll
        for (int k = 0; k < kCombineRegs; ++k) {
            const float wgt = exp2f(pm[k] - nm);
            L += wgt * pl[k];
            a += wgt * pa[k];
        }
        M = nm;
    }
}

}  // namespace oasis
