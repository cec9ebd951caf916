// Verification attention over the sparse KV (OasisKV explainer page, Fig. 7
// right: the attention kernel runs the current and the draft queries over the
// sparse KV together), as speculative decoding verifies drafts.
#include <math.h>

#include "combine.h"
#include "kernels.h"

namespace oasis {

constexpr float kLog2eV = 1.4426950408889634f;

// ---------------------------------------------------------------- verification attention

// OasisKV page, Fig. 7 (right): the attention kernel runs the normal and the
// draft queries over the sparse KV together.  Query set j (0: the current
// query, j >= 1: draft j) of every head of the group attends over the attended
// blocks and, causally, over draft tokens 1..j.  The M = G (1 + D) rows of a
// unit are split into chunks of 16, 8, 4, 2 or 1 rows; each chunk is one pass
// of the block attention kernel above with G = chunk rows (one pass reads the
// attended KV once for all of its rows), and the combine below merges a row's
// partials with its draft tokens.
struct VerifyChunks {
    int n;
    int r0[12];
    int rows[12];
    int ns[12];  // partial rows per (unit, row) of the chunk's pass
};

static VerifyChunks verify_chunks(int M) {
    VerifyChunks c{};
    int r = 0;
    while (r < M && c.n < 12) {
        int g = 16;
        while (g > M - r) g >>= 1;
        c.r0[c.n] = r;
        c.rows[c.n] = g;
        ++c.n;
        r += g;
    }
    return c;
}

__device__ __forceinline__ int verify_chunk_of(const VerifyChunks &c, int r) {
    int k = 0;
    while (k + 1 < c.n && c.r0[k + 1] <= r) ++k;
    return k;
}

// Row r of unit u -> chunk buffer [units][rows][D] of its chunk.
__global__ __launch_bounds__(64) void verify_pack_kernel(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ drafts,
                                                         uint16_t *__restrict__ qpack, int B,
                                                         int Hq, int Hkv, int G,
                                                         VerifyChunks ch, int64_t units) {
    constexpr int D = 128;
    const int r = blockIdx.x;
    const int64_t u = blockIdx.y;
    const int b = (int)(u / Hkv), h = (int)(u % Hkv);
    const int j = r / G, g = r % G;
    const int k = verify_chunk_of(ch, r);
    const uint16_t *src = j == 0 ? q + ((int64_t)b * Hq + h * G + g) * D
                                 : drafts + (((int64_t)(j - 1) * B + b) * Hq + h * G + g) * D;
    uint16_t *dst = qpack + units * ch.r0[k] * D + (u * ch.rows[k] + (r - ch.r0[k])) * D;
    const int c = threadIdx.x * 8;
    if (c < D) gstore16(dst + c, gload16(src + c));
}

// One workgroup (128 threads, thread c = output dim c) per (row, unit).
__global__ __launch_bounds__(128) void verify_combine_kernel(
    const float *__restrict__ vpart_m, const float *__restrict__ vpart_l,
    const float *__restrict__ vpart_acc, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ drafts, const uint16_t *__restrict__ kd,
    const uint16_t *__restrict__ vd, float *__restrict__ out, int B, int Hq, int Hkv, int G,
    int ns, VerifyChunks ch, int64_t units, float scale_log2) {
    constexpr int D = 128;
    __shared__ float red[2];
    const int r = blockIdx.x;
    const int64_t u = blockIdx.y;
    const int b = (int)(u / Hkv), h = (int)(u % Hkv);
    const int j = r / G, g = r % G;
    const int k = verify_chunk_of(ch, r);
    const int rows = ch.rows[k], rr = r - ch.r0[k];
    const int64_t base = units * ns * ch.r0[k];  // this chunk's partial rows
    const int nk = ch.ns[k];
    const int c = threadIdx.x;
    auto pidx = [&](int s) -> int64_t { return base + (u * nk + s) * rows + rr; };
    float M = -INFINITY, L = 0.f, a = 0.f;
    merge_partials(vpart_m, vpart_l, vpart_acc, D, c, nk, pidx, M, L, a);
    if (j > 0) {
        const uint16_t *qr = drafts + (((int64_t)(j - 1) * B + b) * Hq + h * G + g) * D;
        const float qv = __uint_as_float((uint32_t)qr[c] << 16);
        for (int i = 0; i < j; ++i) {  // draft tokens 1..j
            const int64_t kv = (((int64_t)i * B + b) * Hkv + h) * D + c;
            float dot = qv * __uint_as_float((uint32_t)kd[kv] << 16);
            dot = wave_sum(dot);
            if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dot;
            __syncthreads();
            const float x = (red[0] + red[1]) * scale_log2;
            __syncthreads();
            const float mn = fmaxf(M, x);
            const float alpha = exp2f(M - mn), p = exp2f(x - mn);
            L = L * alpha + p;
            a = a * alpha + p * __uint_as_float((uint32_t)vd[kv] << 16);
            M = mn;
        }
    }
    (void)q;
    out[(((int64_t)j * B + b) * Hq + h * G + g) * D + c] = L > 0.f ? a / L : 0.f;
}

int verify_rows(const Dims &D, int n_drafts) { return D.G * (1 + n_drafts); }

hipError_t launch_verify(const Dims &D, const AttnPlan &P, int n_drafts, const void *q,
                         const void *drafts, const void *kd, const void *vd, void *slots,
                         const int32_t *att_block, const int32_t *att_slot,
                         const int32_t *counts, int64_t T, void *qpack, float *vpart_m,
                         float *vpart_l, float *vpart_acc, float *out, hipStream_t st) {
    const int M = verify_rows(D, n_drafts);
    VerifyChunks ch = verify_chunks(M);
    const int64_t units = D.units();
    // one pass per chunk over the attended blocks, each with the plan of its
    // row count: the balanced kernel where it applies (its partial rows per
    // unit fit the verify buffers' stride P.vns), else the split kernel
    AttnPlan Pk[12];
    for (int k = 0; k < ch.n; ++k) {
        Dims Dc = D;
        Dc.G = ch.rows[k];
        Dc.Hq = D.Hkv * ch.rows[k];
        Pk[k] = plan_attention(Dc);
        Pk[k].nsf_max = 0;
        if (Pk[k].flat && Pk[k].flat_rows > P.vns) Pk[k].flat = false;
        Pk[k].nsa = Pk[k].flat ? 0 : Pk[k].ns1;
        ch.ns[k] = Pk[k].flat ? Pk[k].flat_rows : Pk[k].ns1;
    }
    OASIS_LAUNCH(verify_pack_kernel, dim3((unsigned)M, (unsigned)units), dim3(64), 0, st,
                 (const uint16_t *)q, (const uint16_t *)drafts, (uint16_t *)qpack, D.B, D.Hq,
                 D.Hkv, D.G, ch, units);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // every attended block from its slot; chunk k's partials start at row
    // units r0 vns
    for (int k = 0; k < ch.n; ++k) {
        Dims Dc = D;
        Dc.G = ch.rows[k];
        Dc.Hq = D.Hkv * ch.rows[k];
        const int64_t rows0 = units * (int64_t)ch.r0[k];
        e = launch_attention(Dc, Pk[k], 0, 0, (const uint16_t *)qpack + rows0 * 128, slots,
                             nullptr, att_block, att_slot, counts, T, vpart_m + rows0 * P.vns,
                             vpart_l + rows0 * P.vns, vpart_acc + rows0 * P.vns * 128, st);
        if (e != hipSuccess) return e;
    }
    const float scale_log2 = kLog2eV / sqrtf(128.f);
    OASIS_LAUNCH(verify_combine_kernel, dim3((unsigned)M, (unsigned)units), dim3(128), 0, st,
                 vpart_m, vpart_l, vpart_acc, (const uint16_t *)q, (const uint16_t *)drafts,
                 (const uint16_t *)kd, (const uint16_t *)vd, out, D.B, D.Hq, D.Hkv, D.G,
                 P.vns, ch, units, scale_log2);
    return hipGetLastError();
}

}  // namespace oasis
