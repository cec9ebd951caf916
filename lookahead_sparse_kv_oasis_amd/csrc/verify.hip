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
// unit are cut into chunks of 32 rows while 32 or more remain, then one chunk
// of the next power of two at or above the rest (its extra rows repeat the
// chunk's first row; their partials are not written).  Each chunk is one
// pass of the block attention kernel with G = chunk rows, reading its query
// rows in place from q and the drafts: one pass reads the attended KV once for
// all of its rows, so the Qwen3-8B layer's 20 rows per KV head (4 heads x 5
// query sets) take a single 32-row pass on the matrix cores.  The combine
// below merges a row's partials with its draft tokens.
constexpr int kMaxChunks = 12;
constexpr int kChunkRows = 32;

struct VerifyChunks {
    int n;
    int r0[kMaxChunks];    // first query row of chunk k
    int real[kMaxChunks];  // query rows of chunk k
    int rows[kMaxChunks];  // rows of its pass: real rows and padding
    int p0[kMaxChunks];    // first padded row of chunk k (its partials' offset)
    int ns[kMaxChunks];    // partial rows per (unit, row) of the chunk's pass
};

// Chunks of at most wmax rows; returns false when M rows need more than
// kMaxChunks of them.
static bool verify_chunks(int M, int wmax, VerifyChunks &c) {
    c = VerifyChunks{};
    int r = 0, p = 0;
    while (r < M) {
        if (c.n == kMaxChunks) return false;
        const int rest = M - r;
        int w = wmax;
        if (rest < wmax) {
            w = 1;
            while (w < rest) w <<= 1;
        }
        c.r0[c.n] = r;
        c.real[c.n] = rest < w ? rest : w;
        c.rows[c.n] = w;
        c.p0[c.n] = p;
        ++c.n;
        r += c.real[c.n - 1];
        p += w;
    }
    return true;
}

__device__ __forceinline__ int chunk_of_row(const VerifyChunks &c, int r) {
    int k = 0;
    while (k + 1 < c.n && c.r0[k + 1] <= r) ++k;
    return k;
}

constexpr int kDraftBatch = 8;  // draft tokens whose loads go out together

// One wave per (query row, unit), four rows per workgroup; lane l owns output
// dimensions 2 l and 2 l + 1.  The row's partials are merged by
// merge_row_wave; the first batch of draft-token K/V loads goes out before
// it, so both travel together, and each draft token's logit is one wave
// reduction.
__global__ __launch_bounds__(256) void verify_combine_kernel(
    const float *__restrict__ vpart_m, const float *__restrict__ vpart_l,
    const float *__restrict__ vpart_acc, const uint16_t *__restrict__ drafts,
    const uint16_t *__restrict__ kd, const uint16_t *__restrict__ vd, float *__restrict__ out,
    int B, int Hq, int Hkv, int G, int M_rows, int ns, VerifyChunks ch, int64_t units,
    float scale_log2) {
    constexpr int D = 128;
    const int r = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
    if (r >= M_rows) return;
    const int64_t u = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int b = (int)(u / Hkv), h = (int)(u % Hkv);
    const int j = r / G, g = r % G;
    const int k = chunk_of_row(ch, r);
    const int rows = ch.rows[k], rr = r - ch.r0[k];
    const int64_t base = units * ns * ch.p0[k];  // this chunk's partial rows
    const int nk = ch.ns[k];
    // two bf16 values (dimensions 2 lane, 2 lane + 1) as floats
    auto pair = [&](const uint16_t *p) -> float2 {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(p + 2 * lane);
        return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
    };
    auto kv_at = [&](int i) -> int64_t { return (((int64_t)i * B + b) * Hkv + h) * D; };
    float2 qv = make_float2(0.f, 0.f), kx[kDraftBatch], vx[kDraftBatch];
    auto load_batch = [&](int i0) {
#pragma unroll
        for (int i = 0; i < kDraftBatch; ++i) {
            const int t = i0 + i < j ? i0 + i : 0;  // past j: token 0 again, unused
            kx[i] = pair(kd + kv_at(t));
            vx[i] = pair(vd + kv_at(t));
        }
    };
    if (j > 0) {
        qv = pair(drafts + (((int64_t)(j - 1) * B + b) * Hq + h * G + g) * D);
        load_batch(0);
    }
    float M = -INFINITY, L = 0.f;
    float2 a = make_float2(0.f, 0.f);
    merge_row_wave(vpart_m, vpart_l, vpart_acc, nk,
                   [&](int s) -> int64_t { return base + (u * nk + s) * rows + rr; }, M, L, a);
    for (int i0 = 0; i0 < j; i0 += kDraftBatch) {  // draft tokens 1..j
        if (i0 > 0) load_batch(i0);
        const int ni = j - i0 < kDraftBatch ? j - i0 : kDraftBatch;
#pragma unroll
        for (int i = 0; i < kDraftBatch; ++i) {
            if (i >= ni) break;
            const float x = wave_sum(qv.x * kx[i].x + qv.y * kx[i].y) * scale_log2;
            const float mn = fmaxf(M, x);
            const float alpha = exp2f(M - mn), pr = exp2f(x - mn);
            L = L * alpha + pr;
            a.x = a.x * alpha + pr * vx[i].x;
            a.y = a.y * alpha + pr * vx[i].y;
            M = mn;
        }
    }
    const float2 o = L > 0.f ? make_float2(a.x / L, a.y / L) : make_float2(0.f, 0.f);
    *reinterpret_cast<float2 *>(out + (((int64_t)j * B + b) * Hq + h * G + g) * D + 2 * lane) = o;
}

// (32-row chunks pad at least as many rows as 16-row ones, so buffers sized
// for them hold either cut.)
int verify_rows(const Dims &D, int n_drafts) {
    VerifyChunks ch;
    if (!verify_chunks(D.G * (1 + n_drafts), kChunkRows, ch)) return -1;
    return ch.p0[ch.n - 1] + ch.rows[ch.n - 1];
}

hipError_t launch_verify(const Dims &D, const AttnPlan &P, int n_drafts, const void *q,
                         const void *drafts, const void *kd, const void *vd, void *slots,
                         const int32_t *att_block, const int32_t *att_slot,
                         const int32_t *counts, int64_t T, float *vpart_m, float *vpart_l,
                         float *vpart_acc, float *out, hipStream_t st) {
    const int M = D.G * (1 + n_drafts);
    // 32-row passes need the balanced kernel (the split kernel serves up to
    // 16 rows); its partial rows per unit must fit the stride P.vns
    Dims D32 = D;
    D32.G = 32;
    D32.Hq = D.Hkv * 32;
    const AttnPlan P32 = plan_attention(D32);
    const int wmax = P32.flat && P32.flat_rows <= P.vns ? kChunkRows : 16;
    VerifyChunks ch;
    if (!verify_chunks(M, wmax, ch)) return hipErrorInvalidValue;
    const int64_t units = D.units();
    // one pass per chunk over the attended blocks, each with the plan of its
    // row count: the balanced kernel where it applies (its partial rows per
    // unit fit the verify buffers' stride P.vns), else the split kernel
    AttnPlan Pk[kMaxChunks];
    for (int k = 0; k < ch.n; ++k) {
        Dims Dc = D;
        Dc.G = ch.rows[k];
        Dc.Hq = D.Hkv * ch.rows[k];
        Pk[k] = plan_attention(Dc);
        Pk[k].gt = ch.rows[k];  // partial rows of the chunk's own width
        Pk[k].nsf_max = 0;
        if (Pk[k].flat && Pk[k].flat_rows > P.vns) Pk[k].flat = false;
        if (!Pk[k].flat && ch.rows[k] > 16) return hipErrorInvalidValue;
        Pk[k].nsa = Pk[k].flat ? 0 : Pk[k].ns1;
        ch.ns[k] = Pk[k].flat ? Pk[k].flat_rows : Pk[k].ns1;
    }
    // every attended block from its slot; chunk k's partials start at row
    // units p0 vns
    for (int k = 0; k < ch.n; ++k) {
        Dims Dc = D;
        Dc.G = ch.rows[k];
        Dc.Hq = D.Hkv * ch.rows[k];
        const int64_t rows0 = units * (int64_t)ch.p0[k];
        const QRows qr{(const uint16_t *)q, (const uint16_t *)drafts, (int64_t)D.B * D.Hq * 128,
                       D.Hq, D.G, ch.r0[k], ch.real[k]};
        const hipError_t e =
            launch_attention(Dc, Pk[k], 0, 0, q, slots, nullptr, att_block, att_slot, counts, T,
                             vpart_m + rows0 * P.vns, vpart_l + rows0 * P.vns,
                             vpart_acc + rows0 * P.vns * 128, st, &qr);
        if (e != hipSuccess) return e;
    }
    const float scale_log2 = kLog2eV / sqrtf(128.f);
    OASIS_LAUNCH(verify_combine_kernel, dim3((unsigned)((M + 3) / 4), (unsigned)units), dim3(256),
                 0, st, vpart_m, vpart_l, vpart_acc, (const uint16_t *)drafts,
                 (const uint16_t *)kd, (const uint16_t *)vd, out, D.B, D.Hq, D.Hkv, D.G, M,
                 P.vns, ch, units, scale_log2);
    return hipGetLastError();
}

}  // namespace oasis
