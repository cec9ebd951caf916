// Block scores against the current and draft queries.
//
// OasisKV explainer page, Fig. 7: the draft query scans the min/max pooled
// ("compressed") keys to predict the next top-K blocks.  For one query row x
// the score of block j is the largest value x.k can take over the block's
// per-dimension box, sum_c max(x_c * max_jc, x_c * min_jc); a block's score is
// the maximum over the rows of its KV head's group (G query heads, for the
// current query and every draft).
//
// Splitting x into x+ = max(x, 0) and x- = min(x, 0) turns each row's score
// into one dot product of length 2d, [x+ | x-] . [max_j | min_j], so all rows
// against all blocks of a unit is a (rows x 2d) * (2d x blocks) contraction.
// For bf16 that contraction runs on the matrix cores: x+ and x- are exact
// bf16 values, bf16 x bf16 products are exact in fp32, and the fp32
// accumulation is the only rounding.
#include <stdlib.h>
#include <string.h>

#include "kernels.h"
#include "score_tile.h"

namespace oasis {

// ---------------------------------------------------------------- VALU, any dtype

// One wave per 64 blocks of a unit; query rows in LDS as fp32.
template <typename T>
__global__ __launch_bounds__(64) void score_valu_kernel(const T *__restrict__ summ,
                                                        const T *__restrict__ q,
                                                        const T *__restrict__ drafts,
                                                        int n_drafts, int qskip,
                                                        float *__restrict__ scores,
                                                        int B, int Hq, int Hkv, int G, int d,
                                                        int64_t NBmax, int64_t NB) {
    constexpr int V = Elem<T>::kVec;
    extern __shared__ float xs[];  // [Q][d]
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t u = (int64_t)b * Hkv + h;
    const int Q = G * (1 - qskip + n_drafts);
    for (int i = threadIdx.x; i < Q * d; i += blockDim.x) {
        const int r = i / d, c = i % d, src = r / G + qskip, g = r % G;
        const T *row = src == 0 ? q + ((int64_t)b * Hq + h * G + g) * d
                                : drafts + (((int64_t)(src - 1) * B + b) * Hq + h * G + g) * d;
        xs[i] = Elem<T>::f(row[c]);
    }
    __syncthreads();
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= NB) return;
    const T *sm = summ + (u * NBmax + j) * 2 * (int64_t)d;
    float best = -INFINITY;
    for (int r0 = 0; r0 < Q; r0 += 8) {
        float acc[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) acc[rr] = 0.f;
        for (int c = 0; c < d; c += V) {
            const Vec16<T> mx = ld16(sm + c), mn = ld16(sm + d + c);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float a = Elem<T>::f(mx.v[e]), bb = Elem<T>::f(mn.v[e]);
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    if (r0 + rr < Q) {
                        const float x = xs[(r0 + rr) * d + c + e];
                        const float p1 = x * a, p2 = x * bb;
                        acc[rr] += p1 > p2 ? p1 : p2;
                    }
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr)
            if (r0 + rr < Q) best = fmaxf(best, acc[rr]);
    }
    scores[u * NBmax + j] = best;
}

// ---------------------------------------------------------------- MFMA, bf16
// (operand layout and sign split: score_tile.h)

// One workgroup (4 waves) per contiguous range of tiles_per_wg tiles of one
// unit; the waves take the range's tiles in turn, one tile (16 KB at d = 128)
// in flight per wave.  Each tile's 32 scores go to LDS and the range is
// written out in one coalesced pass at the end: scattered 128-byte score
// stores between the summary reads cost about a tenth of the HBM rate.
template <int D, int QT, bool XT>
__global__ __launch_bounds__(256) void score_tiled_kernel(const uint16_t *__restrict__ summ,
                                                          const uint16_t *__restrict__ q,
                                                          const uint16_t *__restrict__ drafts,
                                                          int n_drafts, int qskip,
                                                          float *__restrict__ scores, int B,
                                                          int Hq, int Hkv, int G,
                                                          int64_t unit_elems, int64_t NBmax,
                                                          int64_t NB, int per_unit,
                                                          int tiles_per_wg) {
    extern __shared__ float tile_best[];  // [tiles_per_wg][32]
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t u = blockIdx.x / per_unit;
    const int64_t chunk = blockIdx.x % per_unit;
    const int h = (int)(u % Hkv), b = (int)(u / Hkv);
    const int64_t ntiles = (NB + 31) / 32;
    const int64_t t_begin = chunk * tiles_per_wg;
    const int64_t t_end = t_begin + tiles_per_wg < ntiles ? t_begin + tiles_per_wg : ntiles;
    if (t_begin >= t_end) return;  // whole workgroup
    ScoreTiles<D, QT> st;
    st.setup(summ, u, unit_elems);
    int64_t t = t_begin + wave;
    // XT: a wave that owns one tile more than the fewest (65 tiles over 4
    // waves: 17, 16, 16, 16) loads that last tile now into a second buffer,
    // so it costs no extra round trip at the end, where every other wave
    // would wait for it.  The buffer takes 64 more registers per lane, which
    // leave no room beside the kernel for another kernel's waves, so it is
    // used where each CU holds one workgroup and nothing else runs there.
    const int64_t mine = t < t_end ? (t_end - t + 3) / 4 : 0;
    const bool extra = XT && mine >= 2 && mine > (t_end - t_begin) / 4;
    const int64_t t_stop = extra ? t + 4 * (mine - 1) : t_end;
    bf16x8 bx[XT ? ScoreTiles<D, QT>::NI : 1];
    if (t < t_end) st.load(t);  // in flight while the query rows are read
    if constexpr (XT) {
        if (extra) st.load_to(bx, t_stop);
    }
    st.rows(q, drafts, n_drafts, qskip, B, Hq, G, b, h);
    for (; t < t_stop; t += 4) {
        const float best = st.best();
        if (st.half == 0) tile_best[(t - t_begin) * 32 + st.m] = best;
        if (t + 4 < t_stop) st.load(t + 4);
    }
    if constexpr (XT) {
        if (extra) {
            const float best = st.best_of(bx);
            if (st.half == 0) tile_best[(t_stop - t_begin) * 32 + st.m] = best;
        }
    }
    __syncthreads();
    const int64_t j0 = t_begin * 32;
    const int64_t j1 = t_end * 32 < NB ? t_end * 32 : NB;
    float *out = scores + u * NBmax;
    for (int64_t j = j0 + threadIdx.x; j < j1; j += 256) out[j] = tile_best[j - j0];
}

template <int D>
static void launch_tiled(int QT, bool xt, dim3 grid, size_t lds, hipStream_t st,
                         const uint16_t *summ, const uint16_t *q, const uint16_t *dr, int nd,
                         int qskip, float *scores, const Dims &Dm, int64_t NB, int per_unit,
                         int tpw) {
#define OASIS_SCORE_T(QT_, XT_)                                                                 \
    OASIS_LAUNCH((score_tiled_kernel<D, QT_, XT_>), grid, dim3(256), lds, st, summ, q, dr, nd,    \
                 qskip, scores, Dm.B, Dm.Hq, Dm.Hkv, Dm.G, Dm.summ_unit_elems(), Dm.NBmax, NB,    \
                 per_unit, tpw)
    if (QT == 1 && xt) OASIS_SCORE_T(1, true);
    else if (QT == 1) OASIS_SCORE_T(1, false);
    else if (QT == 2) OASIS_SCORE_T(2, false);
    else if (QT == 3) OASIS_SCORE_T(3, false);
    else OASIS_SCORE_T(4, false);
#undef OASIS_SCORE_T
}

hipError_t launch_score(const Dims &D, const void *summ, const void *q, const void *drafts,
                        int n_drafts, int64_t NB, float *scores, hipStream_t st) {
    if (NB <= 0) return hipSuccess;
    const int qskip = q ? 0 : 1;  // no current query: the drafts alone
    const int Q = D.G * (1 - qskip + n_drafts);
    if (D.tiled) {
        const int QT = (Q + 31) / 32;
        const int64_t ntiles = (NB + 31) / 32;
        // at least one workgroup per CU, and at most 256 tiles (32 KB of
        // scores) per workgroup.  Where the workgroups do not spread evenly
        // over the CUs (a CU subset of 240 for 256 units), at least four per
        // unit, so that CUs that finish early take more: one per unit left
        // 16 CUs with two and took 56.7 us on the Qwen3-8B layer, four per
        // unit 45.9 us (42.1 us on all 256 CUs).
        const int cus = compute_units(D);
        int64_t want = (cus + D.units() - 1) / D.units();
        if ((D.units() * want) % cus != 0 && want < 4) want = 4;
        int64_t tpw = (ntiles + want - 1) / want;
        if (tpw > 256) tpw = 256;
        if (tpw < 1) tpw = 1;
        const int64_t per_unit = (ntiles + tpw - 1) / tpw;
        const dim3 grid((unsigned)(per_unit * D.units()));
        const size_t lds = sizeof(float) * 32 * (size_t)tpw;
        const uint16_t *s = (const uint16_t *)summ, *qq = (const uint16_t *)q,
                       *dr = (const uint16_t *)drafts;
        // the extra-tile buffer where each CU holds at most one workgroup
        const bool xt = (int64_t)grid.x <= cus;
        if (D.d == 64)
            launch_tiled<64>(QT, xt, grid, lds, st, s, qq, dr, n_drafts, qskip, scores, D, NB,
                             (int)per_unit, (int)tpw);
        else if (D.d == 128)
            launch_tiled<128>(QT, xt, grid, lds, st, s, qq, dr, n_drafts, qskip, scores, D, NB,
                              (int)per_unit, (int)tpw);
        else
            launch_tiled<256>(QT, xt, grid, lds, st, s, qq, dr, n_drafts, qskip, scores, D, NB,
                              (int)per_unit, (int)tpw);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((NB + 63) / 64), D.Hkv, D.B), block(64);
    const size_t lds = sizeof(float) * Q * D.d;
    if (D.dtype == kF32)
        OASIS_LAUNCH(score_valu_kernel<float>, grid, block, lds, st, (const float *)summ,
                     (const float *)q, (const float *)drafts, n_drafts, qskip, scores, D.B, D.Hq,
                     D.Hkv, D.G, D.d, D.NBmax, NB);
    else
        OASIS_LAUNCH(score_valu_kernel<uint16_t>, grid, block, lds, st, (const uint16_t *)summ,
                     (const uint16_t *)q, (const uint16_t *)drafts, n_drafts, qskip, scores, D.B,
                     D.Hq,
                     D.Hkv, D.G, D.d, D.NBmax, NB);
    return hipGetLastError();
}

}  // namespace oasis
