// Merge of split-K attention partials (running max, normaliser, sum), shared
// by the combine of the decode attention and of the verification attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

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

// Partial sums loaded per round trip by merge_row_wave.
constexpr int kWaveMergeRegs = 16;

// One wave merges the n partials of one output row of 128 dimensions (partial
// i at row pidx(i); lane l owns dimensions 2 l and 2 l + 1) into a running
// (M, L, a).  Per group of 64 partials, lane s reads partial s's m and l; the
// weights and the normaliser follow by wave reductions, and then only the
// sums (512-byte rows) of the live partials (m > -inf) are read,
// kWaveMergeRegs per round trip: partials marked empty cost no sum read,
// which matters where a unit's fixed set of partial rows is mostly unused.
// With Spec, the sums of the first kWaveMergeRegs partials are read together
// with the first group's m and l, live or not, so that the common case takes
// one round trip at the price of the dead rows' bytes (a gain for the decode
// combine's 4 rows per unit, a loss for the verification's 20).
template <bool Spec = false, typename F>
__device__ __forceinline__ void merge_row_wave(const float *__restrict__ part_m,
                                               const float *__restrict__ part_l,
                                               const float *__restrict__ part_acc, int n, F pidx,
                                               float &M, float &L, float2 &a) {
    const int lane = threadIdx.x & 63;
    float2 v0[kWaveMergeRegs];  // sums of partials 0 .. kWaveMergeRegs - 1 (0 again past n)
    if constexpr (Spec) {
#pragma unroll
        for (int k = 0; k < kWaveMergeRegs; ++k)
            v0[k] =
                *reinterpret_cast<const float2 *>(part_acc + pidx(k < n ? k : 0) * 128 + 2 * lane);
    }
    for (int i0 = 0; i0 < n; i0 += 64) {
        // lanes past n read partial i0 again and count as empty
        const int64_t pi = pidx(i0 + lane < n ? i0 + lane : i0);
        float pm = part_m[pi], pl = part_l[pi];
        if (i0 + lane >= n) {
            pm = -INFINITY;
            pl = 0.f;
        }
        uint64_t live = __ballot(pm != -INFINITY);
        if (live == 0) continue;
        const float nm = fmaxf(M, wave_max(pm));
        const float r = exp2f(M - nm);  // 0 while nothing was merged
        const float w = pm != -INFINITY ? exp2f(pm - nm) : 0.f;
        // a partial marked empty adds nothing, whatever its l holds
        L = L * r + wave_sum(pm != -INFINITY ? w * pl : 0.f);
        a.x *= r;
        a.y *= r;
        M = nm;
        if (Spec && i0 == 0) {
#pragma unroll
            for (int k = 0; k < kWaveMergeRegs; ++k) {
                // an empty partial's sums may hold anything (NaN included):
                // selected away, not multiplied by 0
                const bool lk = (live >> k) & 1;
                const float wf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
                a.x += lk ? wf * v0[k].x : 0.f;
                a.y += lk ? wf * v0[k].y : 0.f;
            }
            live &= ~((1ull << kWaveMergeRegs) - 1);
        }
        const int s_first = live ? __builtin_ctzll(live) : 0;
        while (live) {
            // every load issued before any is used; past the last live
            // partial the first one is read again with weight 0
            float2 v[kWaveMergeRegs];
            int wk[kWaveMergeRegs];  // weight bits
#pragma unroll
            for (int k = 0; k < kWaveMergeRegs; ++k) {
                const int s = live ? __builtin_ctzll(live) : s_first;
                wk[k] = live ? __builtin_amdgcn_readlane(__float_as_int(w), s) : 0;
                live &= live - 1;
                v[k] = *reinterpret_cast<const float2 *>(part_acc + pidx(i0 + s) * 128 + 2 * lane);
            }
#pragma unroll
            for (int k = 0; k < kWaveMergeRegs; ++k) {
                const float wf = __int_as_float(wk[k]);
                a.x += wf * v[k].x;
                a.y += wf * v[k].y;
            }
        }
    }
}

}  // namespace oasis
