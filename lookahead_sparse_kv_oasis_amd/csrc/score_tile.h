// Matrix-core block scores of one unit's tiled summaries, shared by the score
// kernel and the fused score + top-K + select kernel.
//
// OasisKV explainer page, Fig. 7: block score = max over the query rows x of
// sum_c max(x_c * max_c, x_c * min_c).  With x split into x+ = max(x, 0) and
// x- = min(x, 0) a row's score is the dot product [x+ | x-] . [max | min], so
// one tile of 32 blocks against all query rows is one (rows x 2d) * (2d x 32)
// product on v_mfma_f32_32x32x16_bf16: lane l supplies row (A) / column (B)
// l % 32 and 8 consecutive k of each 16-k step, k-half l / 32; k-half 0
// carries x+ against the maxima, k-half 1 x- against the minima.  The tiled
// summary layout (Dims) stores each k-step of a tile in this lane order, so a
// wave reads a k-step with one coalesced 1 KB load straight into operand
// registers.  Query rows past Q repeat row 0, so the max over the 32
// accumulator rows needs no mask; lanes l and l ^ 32 hold the two halves of
// block l % 32's rows.
#pragma once
#include "kernels.h"

namespace oasis {

__device__ __forceinline__ uint4 keep_sign(uint4 w, bool negative) {
    auto one = [&](uint32_t x) -> uint32_t {
        const uint32_t s = (x >> 15) & 0x00010001u;  // sign bit of each bf16
        const uint32_t neg = s * 0xFFFFu;             // 0xFFFF per negative element
        return negative ? (x & neg) : (x & ~neg);
    };
    return make_uint4(one(w.x), one(w.y), one(w.z), one(w.w));
}

template <int D, int QT> struct ScoreTiles {
    static constexpr int NI = D / 8;  // k-steps: 16 k each, 8 from each half
    bf16x8 a[QT][NI];                 // query rows (A operand)
    bf16x8 bv[NI];                    // one tile (B operand)
    const uint16_t *ubase;
    int m, half;

    __device__ __forceinline__ void setup(const uint16_t *summ, int64_t u, int64_t unit_elems) {
        const int lane = threadIdx.x & 63;
        m = lane & 31;
        half = lane >> 5;
        ubase = summ + u * unit_elems + 8 * lane;
    }
    __device__ __forceinline__ void load_to(bf16x8 (&dst)[NI], int64_t tile) const {
        const uint16_t *src = ubase + tile * 64 * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) dst[i] = __builtin_bit_cast(bf16x8, gload16_nt(src + 512 * i));
    }
    __device__ __forceinline__ void load(int64_t tile) { load_to(bv, tile); }
    // Rows: G heads x {current query (unless qskip), drafts}, sign-split.
    __device__ __forceinline__ void rows(const uint16_t *q, const uint16_t *drafts, int n_drafts,
                                         int qskip, int B, int Hq, int G, int b, int h) {
        const int Q = G * (1 - qskip + n_drafts);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            int r = 32 * qt + m;
            if (r >= Q) r = 0;
            const int src = r / G + qskip, g = r % G;
            const uint16_t *x = src == 0
                                    ? q + ((int64_t)b * Hq + h * G + g) * D
                                    : drafts + (((int64_t)(src - 1) * B + b) * Hq + h * G + g) * D;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const uint4 w = *reinterpret_cast<const uint4 *>(x + 8 * i);
                a[qt][i] = __builtin_bit_cast(bf16x8, keep_sign(w, half != 0));
            }
        }
    }
    // Score of block m of tile `tl` (valid in lanes with half == 0).
    __device__ __forceinline__ float best_of(const bf16x8 (&tl)[NI]) const {
        float b = -INFINITY;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            f32x16 acc = {};
#pragma unroll
            for (int i = 0; i < NI; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[qt][i], tl[i], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) b = fmaxf(b, acc[r]);
        }
        return fmaxf(b, __shfl_xor(b, 32, 64));
    }
    __device__ __forceinline__ float best() const { return best_of(bv); }
};

}  // namespace oasis
