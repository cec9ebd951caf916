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

namespace oasis {

// ---------------------------------------------------------------- VALU, any dtype

// One wave per 64 blocks of a unit; query rows in LDS as fp32.
template <typename T>
__global__ __launch_bounds__(64) void score_valu_kernel(const T *__restrict__ summ,
                                                        const T *__restrict__ q,
                                                        const T *__restrict__ drafts,
                                                        int n_drafts, float *__restrict__ scores,
                                                        int B, int Hq, int Hkv, int G, int d,
                                                        int64_t NBmax, int64_t NB) {
    constexpr int V = Elem<T>::kVec;
    extern __shared__ float xs[];  // [Q][d]
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t u = (int64_t)b * Hkv + h;
    const int Q = G * (1 + n_drafts);
    for (int i = threadIdx.x; i < Q * d; i += blockDim.x) {
        const int r = i / d, c = i % d, src = r / G, g = r % G;
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

// v_mfma_f32_32x32x16_bf16 operand layout (wave64): lane l supplies row
// (A) / column (B) l % 32 and 8 consecutive k of the 16-k step, k-half
// l / 32.  The k order inside the contraction is free as long as A and B
// agree, so k-half 0 carries x+ against the block maxima and k-half 1 carries
// x- against the block minima: each lane then streams 16 contiguous bytes of
// one summary row per step.  Query rows past Q repeat row 0, so the max over
// all 32 accumulator rows needs no mask.  Output column of lane l is block
// l % 32; lanes l and l ^ 32 hold the two halves of its rows.
__device__ __forceinline__ uint4 keep_sign(uint4 w, bool negative) {
    auto one = [&](uint32_t x) -> uint32_t {
        const uint32_t s = (x >> 15) & 0x00010001u;  // sign bit of each bf16
        const uint32_t neg = s * 0xFFFFu;             // 0xFFFF per negative element
        return negative ? (x & neg) : (x & ~neg);
    };
    return make_uint4(one(w.x), one(w.y), one(w.z), one(w.w));
}

template <int D, int QT>
__global__ __launch_bounds__(256) void score_mfma_kernel(const uint16_t *__restrict__ summ,
                                                         const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ drafts,
                                                         int n_drafts, float *__restrict__ scores,
                                                         int B, int Hq, int Hkv, int G,
                                                         int64_t NBmax, int64_t NB) {
    constexpr int NI = D / 8;  // MFMA steps: 16 k each, 8 from each half
    // One tile of 32 summaries is 16 KB per wave.  With one query tile the
    // next tile is loaded while the current one is multiplied (two register
    // buffers); with more query tiles the registers hold a single buffer whose
    // loads are all issued before the first multiply.
    constexpr bool kDouble = QT == 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t u = (int64_t)b * Hkv + h;
    const int Q = G * (1 + n_drafts);
    const int m = lane & 31, half = lane >> 5;

    bf16x8 a[QT][NI];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        int r = 32 * t + m;
        if (r >= Q) r = 0;
        const int src = r / G, g = r % G;
        const uint16_t *x = src == 0
                                ? q + ((int64_t)b * Hq + h * G + g) * D
                                : drafts + (((int64_t)(src - 1) * B + b) * Hq + h * G + g) * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint4 w = *reinterpret_cast<const uint4 *>(x + 8 * i);
            a[t][i] = __builtin_bit_cast(bf16x8, keep_sign(w, half != 0));
        }
    }

    const int64_t ntiles = (NB + 31) / 32;
    const uint16_t *base = summ + u * NBmax * 2 * D + half * D;
    float *out = scores + u * NBmax;
    const int64_t stride = (int64_t)gridDim.x * 4;

    auto load = [&](bf16x8(&bv)[NI], int64_t tile) {
        const int64_t j = tile * 32 + m;
        const uint16_t *src = base + (j < NB ? j : NB - 1) * 2 * D;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            bv[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src + 8 * i));
    };
    auto compute = [&](const bf16x8(&bv)[NI], int64_t tile) {
        float best = -INFINITY;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            f32x16 acc = {};
#pragma unroll
            for (int i = 0; i < NI; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][i], bv[i], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) best = fmaxf(best, acc[r]);
        }
        best = fmaxf(best, __shfl_xor(best, 32, 64));
        const int64_t j = tile * 32 + m;
        if (half == 0 && j < NB) out[j] = best;
    };

    int64_t t0 = (int64_t)blockIdx.x * 4 + wave;
    if (t0 >= ntiles) return;
    if constexpr (kDouble) {
        bf16x8 ba[NI], bb[NI];
        load(ba, t0);
        while (true) {
            const int64_t t1 = t0 + stride;
            if (t1 < ntiles) load(bb, t1);
            __builtin_amdgcn_sched_barrier(0);
            compute(ba, t0);
            if (t1 >= ntiles) break;
            const int64_t t2 = t1 + stride;
            if (t2 < ntiles) load(ba, t2);
            __builtin_amdgcn_sched_barrier(0);
            compute(bb, t1);
            if (t2 >= ntiles) break;
            t0 = t2;
        }
    } else {
        bf16x8 bv[NI];
        for (; t0 < ntiles; t0 += stride) {
            load(bv, t0);
            __builtin_amdgcn_sched_barrier(0);
            compute(bv, t0);
        }
    }
}

// LDS-staged variant (D = 128, one query tile).  A wave's tile of 32 block
// summaries is 16 KB of contiguous HBM; it is read with fully coalesced
// 16-byte loads (1 KB per instruction) into registers, written to a
// wave-private LDS buffer whose 512-byte rows are padded to 528 bytes (so the
// operand reads below hit 16 distinct banks per 16 lanes), and read back in
// the MFMA operand layout.  The next tile's global loads are in flight while
// the current tile is multiplied.
constexpr int kScoreRowPad = 528;                  // bytes per padded summary row
constexpr int kScoreTileLds = 32 * kScoreRowPad;   // bytes per wave

__global__ __launch_bounds__(256) void score_mfma_lds_kernel(const uint16_t *__restrict__ summ,
                                                             const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ drafts,
                                                             int n_drafts,
                                                             float *__restrict__ scores, int B,
                                                             int Hq, int Hkv, int G,
                                                             int64_t NBmax, int64_t NB) {
    constexpr int D = 128, NI = D / 8;
    extern __shared__ __attribute__((aligned(16))) unsigned char score_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t u = (int64_t)b * Hkv + h;
    const int Q = G * (1 + n_drafts);
    const int m = lane & 31, half = lane >> 5;
    unsigned char *buf = score_lds + wave * kScoreTileLds;

    bf16x8 a[NI];
    {
        int r = m;
        if (r >= Q) r = 0;
        const int src = r / G, g = r % G;
        const uint16_t *x = src == 0
                                ? q + ((int64_t)b * Hq + h * G + g) * D
                                : drafts + (((int64_t)(src - 1) * B + b) * Hq + h * G + g) * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint4 w = *reinterpret_cast<const uint4 *>(x + 8 * i);
            a[i] = __builtin_bit_cast(bf16x8, keep_sign(w, half != 0));
        }
    }

    const int64_t ntiles = (NB + 31) / 32;
    const unsigned char *base = reinterpret_cast<const unsigned char *>(summ + u * NBmax * 2 * D);
    const int64_t ubytes = NB * 2 * D * 2;  // valid summary bytes of this unit
    float *out = scores + u * NBmax;
    const int64_t stride = (int64_t)gridDim.x * 4;

    // coalesced: instruction k, lane l -> tile byte 1024 k + 16 l
    auto gload = [&](uint4 (&r)[16], int64_t tile) {
        const int64_t t0 = tile * 32 * 512;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            int64_t off = t0 + 1024 * k + 16 * lane;
            if (off >= ubytes) off = ubytes - 16;  // ragged last tile: stay in bounds
            r[k] = gload16(base + off);
        }
    };
    auto lds_store = [&](const uint4 (&r)[16]) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int o = 1024 * k + 16 * lane;
            *reinterpret_cast<uint4 *>(buf + (o >> 9) * kScoreRowPad + (o & 511)) = r[k];
        }
    };
    auto compute = [&](int64_t tile) {
        f32x16 acc = {};
        const unsigned char *row = buf + m * kScoreRowPad + half * 256;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint4 w = *reinterpret_cast<const uint4 *>(row + 16 * i);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], __builtin_bit_cast(bf16x8, w), acc,
                                                          0, 0, 0);
        }
        float best = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) best = fmaxf(best, acc[r]);
        best = fmaxf(best, __shfl_xor(best, 32, 64));
        const int64_t j = tile * 32 + m;
        if (half == 0 && j < NB) out[j] = best;
    };
    auto wave_lds_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        __builtin_amdgcn_wave_barrier();
    };

    int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= ntiles) return;
    uint4 r[16];
    gload(r, t);
    while (true) {
        lds_store(r);
        wave_lds_sync();
        const int64_t nx = t + stride;
        if (nx < ntiles) gload(r, nx);
        __builtin_amdgcn_sched_barrier(0);
        compute(t);
        wave_lds_sync();  // all lanes done reading before the next store
        if (nx >= ntiles) break;
        t = nx;
    }
}

template <int D>
static void launch_mfma(int QT, dim3 grid, hipStream_t st, const uint16_t *summ,
                        const uint16_t *q, const uint16_t *dr, int nd, float *scores,
                        const Dims &Dm, int64_t NB) {
    if (QT == 1)
        OASIS_LAUNCH((score_mfma_kernel<D, 1>), grid, dim3(256), 0, st, summ, q, dr, nd,
                           scores, Dm.B, Dm.Hq, Dm.Hkv, Dm.G, Dm.NBmax, NB);
    else if (QT == 2)
        OASIS_LAUNCH((score_mfma_kernel<D, 2>), grid, dim3(256), 0, st, summ, q, dr, nd,
                           scores, Dm.B, Dm.Hq, Dm.Hkv, Dm.G, Dm.NBmax, NB);
    else if (QT == 3)
        OASIS_LAUNCH((score_mfma_kernel<D, 3>), grid, dim3(256), 0, st, summ, q, dr, nd,
                           scores, Dm.B, Dm.Hq, Dm.Hkv, Dm.G, Dm.NBmax, NB);
    else
        OASIS_LAUNCH((score_mfma_kernel<D, 4>), grid, dim3(256), 0, st, summ, q, dr, nd,
                           scores, Dm.B, Dm.Hq, Dm.Hkv, Dm.G, Dm.NBmax, NB);
}

hipError_t launch_score(const Dims &D, const void *summ, const void *q, const void *drafts,
                        int n_drafts, int64_t NB, float *scores, bool use_mfma, hipStream_t st) {
    if (NB <= 0) return hipSuccess;
    static const bool lds_staged = [] {
        const char *e = getenv("OASIS_SCORE_IMPL");
        return !(e && !strcmp(e, "mfma_direct"));
    }();
    const int Q = D.G * (1 + n_drafts);
    if (use_mfma) {
        const int QT = (Q + 31) / 32;
        const int64_t ntiles = (NB + 31) / 32;
        int64_t per_unit = (1024 + D.units() - 1) / D.units();
        const int64_t max_per_unit = (ntiles + 3) / 4;
        if (per_unit > max_per_unit) per_unit = max_per_unit;
        if (per_unit < 1) per_unit = 1;
        dim3 grid((unsigned)per_unit, D.Hkv, D.B);
        const uint16_t *s = (const uint16_t *)summ, *qq = (const uint16_t *)q,
                       *dr = (const uint16_t *)drafts;
        if (D.d == 128 && QT == 1 && lds_staged) {
            OASIS_LAUNCH(score_mfma_lds_kernel, grid, dim3(256), 4 * kScoreTileLds, st, s, qq,
                               dr, n_drafts, scores, D.B, D.Hq, D.Hkv, D.G, D.NBmax, NB);
            return hipGetLastError();
        }
        if (D.d == 64)
            launch_mfma<64>(QT, grid, st, s, qq, dr, n_drafts, scores, D, NB);
        else if (D.d == 128)
            launch_mfma<128>(QT, grid, st, s, qq, dr, n_drafts, scores, D, NB);
        else
            launch_mfma<256>(QT, grid, st, s, qq, dr, n_drafts, scores, D, NB);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((NB + 63) / 64), D.Hkv, D.B), block(64);
    const size_t lds = (size_t)Q * D.d * sizeof(float);
    if (D.dtype == kF32)
        OASIS_LAUNCH(score_valu_kernel<float>, grid, block, lds, st, (const float *)summ,
                           (const float *)q, (const float *)drafts, n_drafts, scores, D.B, D.Hq,
                           D.Hkv, D.G, D.d, D.NBmax, NB);
    else
        OASIS_LAUNCH(score_valu_kernel<uint16_t>, grid, block, lds, st,
                           (const uint16_t *)summ, (const uint16_t *)q,
                           (const uint16_t *)drafts, n_drafts, scores, D.B, D.Hq, D.Hkv, D.G,
                           D.d, D.NBmax, NB);
    return hipGetLastError();
}

}  // namespace oasis
