// Sparse GQA decode attention over the attended blocks of each (b, KV head).
//
// OasisKV explainer page, Fig. 7: the attention kernel runs over the sparse
// KV working set held in HBM; "KV cache offloading, week 2", section 3: under
// GQA one KV head serves a group of G query heads, and the KV lives in
// fixed-size blocks addressed through a table.  For every query head,
//   out = sum_p softmax_p(q . k_p / sqrt(d)) v_p
// over the valid tokens p of the attended blocks (hits, then fetched blocks).
//
// Split-K: each workgroup reduces a contiguous range of the attended list to
// a partial (running max m, normaliser l, unnormalised sum acc), in the
// base-2 exponent domain (logits pre-multiplied by log2(e) / sqrt(d)); the
// combine kernel merges the partials of a unit.
#include <stdlib.h>

#include <algorithm>

#include "combine.h"
#include "kernels.h"

namespace oasis {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- any dtype

// One wave per (split, unit); each lane owns d elements c = lane + 64 e.
template <typename T, int EPL>
__global__ __launch_bounds__(64) void attn_generic_kernel(
    const T *__restrict__ q, const T *__restrict__ slots, const int32_t *__restrict__ att_block,
    const int32_t *__restrict__ att_slot, const int32_t *__restrict__ counts, int64_t T_, int Hq,
    int Hkv, int G, int d, int K, int S, int bs, int bps, int nsa, int split_off,
    float scale_log2, float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_acc) {
    const int lane = threadIdx.x;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int64_t u = (int64_t)b * Hkv + h;
    const int n_att = counts[u * 4];
    const int e0 = split * bps;
    const int e1 = (e0 + bps) < n_att ? (e0 + bps) : n_att;
    for (int g = 0; g < G; ++g) {
        const T *qr = q + ((int64_t)b * Hq + h * G + g) * d;
        float qv[EPL], acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int c = lane + 64 * e;
            qv[e] = c < d ? Elem<T>::f(qr[c]) : 0.f;
            acc[e] = 0.f;
        }
        float m = -INFINITY, l = 0.f;
        for (int i = e0; i < e1; ++i) {
            const int32_t blk = att_block[u * K + i], s = att_slot[u * K + i];
            const int64_t first = (int64_t)blk * bs;
            const int valid = (int)((T_ - first) < bs ? (T_ - first) : bs);
            const T *kp = slots + (u * S + s) * 2 * (int64_t)bs * d;
            const T *vp = kp + (int64_t)bs * d;
            for (int t = 0; t < valid; ++t) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int c = lane + 64 * e;
                    if (c < d) dot += qv[e] * Elem<T>::f(kp[(int64_t)t * d + c]);
                }
                const float x = wave_sum(dot) * scale_log2;
                const float mn = fmaxf(m, x);
                const float alpha = exp2f(m - mn);
                const float p = exp2f(x - mn);
                l = l * alpha + p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int c = lane + 64 * e;
                    const float vv = c < d ? Elem<T>::f(vp[(int64_t)t * d + c]) : 0.f;
                    acc[e] = acc[e] * alpha + p * vv;
                }
                m = mn;
            }
        }
        const int64_t pi = (u * nsa + split_off + split) * G + g;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int c = lane + 64 * e;
            if (c < d) part_acc[pi * d + c] = acc[e];
        }
        if (lane == 0) {
            part_m[pi] = m;
            part_l[pi] = l;
        }
    }
}

// ---------------------------------------------------------------- bf16, d = 128, bs = 16

// Broadcast lane g of each 16-lane row to the whole row (DPP row_newbcast).
template <int g> __device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + g, 0xF, 0xF,
                                           false));
}

// Row r of a pass over unit (b, h): its query row r0 + r (r0 past `real`),
// query row j G + g = head h G + g of set j.
__device__ __forceinline__ const uint16_t *query_row(const QRows &qr, int64_t b, int h, int r) {
    const int R = qr.r0 + (r < qr.real ? r : 0);
    const int j = R / qr.G, g = R - j * qr.G;
    const uint16_t *base = j == 0 ? qr.q : qr.drafts + (int64_t)(j - 1) * qr.set_stride;
    return base + (b * qr.Hq + (int64_t)h * qr.G + g) * 128;
}

// Per 16-token block of one unit, in one wave:
//   S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (tokens are the M rows, the G
//   heads of the group the N columns, zero-padded to 16).  Lane l supplies
//   token / head l % 16 and, at step c, the dimensions 32 c + 8 (l / 16) ...
//   (8 of them), so the four lanes of a key row read 64 contiguous bytes per
//   step.  The accumulator of lane l holds head l % 16 for tokens
//   4 (l / 16) + r, r < 4.
//   P V on the vector ALU in fp32: lane l owns tokens 4 (l / 16) + r and the
//   8 dimensions 8 (l % 16) ...; the probabilities of head g for its tokens
//   sit in lane 16 (l / 16) + g of the same 16-lane row, so a DPP row
//   broadcast delivers them.
template <int G> struct AttnWave {
    static constexpr int D = 128, BS = 16, BLK = 2 * BS * D;
    static constexpr int kStage = 8;  // LDS staging per wave (unused here)
    uint16_t *vst = nullptr;
    int col, kg, koff, voff;
    bf16x8 qb[4];
    float m, lsum;
    float acc[G][8];

    // Lane roles; must run before the first load.
    __device__ __forceinline__ void lanes() {
        const int lane = threadIdx.x & 63;
        col = lane & 15;
        kg = lane >> 4;
        koff = col * D + 8 * kg;
        voff = BS * D + 4 * kg * D + 8 * col;
    }
    int nreal = G;  // rows whose partials are written
    // Queries of unit (b, h) and a cleared softmax state.
    __device__ __forceinline__ void init(const QRows &qr, int64_t b, int h) {
        load_q(qb, qr, b, h);
        reset();
    }
    // The query rows of unit (b, h) in the B-operand order (rows past G zero).
    __device__ __forceinline__ void load_q(bf16x8 (&dst)[4], const QRows &qr, int64_t b,
                                           int h) const {
        const uint16_t *qp = query_row(qr, b, h, col < G ? col : 0) + 8 * kg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 w = *reinterpret_cast<const uint4 *>(qp + 32 * i);
            if (col >= G) w = make_uint4(0, 0, 0, 0);
            dst[i] = __builtin_bit_cast(bf16x8, w);
        }
    }
    __device__ __forceinline__ void reset() {
        m = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }
    __device__ __forceinline__ void load(uint4 (&kk)[4], uint4 (&vv)[4], const uint16_t *p) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) kk[i] = gload16(p + koff + 32 * i);
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = gload16(p + voff + r * D);
    }
    // The same from a resident slot in HBM, streamed (read once per step).
    __device__ __forceinline__ void load_nt(uint4 (&kk)[4], uint4 (&vv)[4],
                                            const uint16_t *p) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) kk[i] = gload16_nt(p + koff + 32 * i);
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = gload16_nt(p + voff + r * D);
    }
    __device__ __forceinline__ void store(uint16_t *p, const uint4 (&kk)[4],
                                          const uint4 (&vv)[4]) const {
#pragma unroll
        for (int c = 0; c < 4; ++c) gstore16(p + koff + 32 * c, kk[c]);
#pragma unroll
        for (int r = 0; r < 4; ++r) gstore16(p + voff + r * D, vv[r]);
    }
    // Online-softmax update with one block of `valid` tokens.
    __device__ __forceinline__ void block(const uint4 (&kk)[4], const uint4 (&vv)[4], int valid,
                                          float scale_log2) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk[c]), qb[c],
                                                         s4, 0, 0, 0);
        float sr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sr[r] = (4 * kg + r < valid) ? s4[r] * scale_log2 : -INFINITY;
        float bm = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
        bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
        bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
        const float mn = fmaxf(m, bm);
        const bool live = mn != -INFINITY;
        const float alpha = live ? exp2f(m - mn) : 1.f;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = live ? exp2f(sr[r] - mn) : 0.f;
        lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m = mn;
        // rescale, then add the block's four value rows one at a time (the
        // rows past T are zeroed: their probability is 0 but the bytes may be
        // anything)
        static_for<0, G>([&](auto gi) {
            constexpr int g = decltype(gi)::value;
            const float ag = row_bcast<g>(alpha);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] *= ag;
        });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t keep = (4 * kg + r < valid) ? 0xFFFFFFFFu : 0u;
            float vf[8];
            bf16x8_to_f32(make_uint4(vv[r].x & keep, vv[r].y & keep, vv[r].z & keep,
                                     vv[r].w & keep),
                          vf);
            static_for<0, G>([&](auto gi) {
                constexpr int g = decltype(gi)::value;
                const float pg = row_bcast<g>(p[r]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] += pg * vf[e];
            });
        }
    }
    // Sum the four token groups; lanes with kg == 0 then hold the wave's acc.
    __device__ __forceinline__ void reduce() {
        lsum += __shfl_xor(lsum, 16, 64);
        lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = acc[g][e];
                a += __shfl_xor(a, 16, 64);
                a += __shfl_xor(a, 32, 64);
                acc[g][e] = a;
            }
    }
    // Write this wave's (reduced) state as partial pi0 + g.
    __device__ __forceinline__ void write_partial(int64_t pi0, float *part_m, float *part_l,
                                                  float *part_acc) const {
        if (kg == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (g >= nreal) break;
                float4 *dst = reinterpret_cast<float4 *>(part_acc + (pi0 + g) * D + 8 * col);
                dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
                dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
            }
            if (col < nreal) {
                part_m[pi0 + col] = m;
                part_l[pi0 + col] = lsum;
            }
        }
    }
    // This wave's (reduced) state into LDS for the workgroup's merge.
    __device__ __forceinline__ void stash(float (*sacc)[D], float *sm, float *sl) const {
        if (kg == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) sacc[g][8 * col + e] = acc[g][e];
            sm[col] = m;
            sl[col] = lsum;
        }
    }
};

// 16 or 32 query rows per KV head (16 heads per KV head, and the 16- and
// 32-row chunks of the verification attention): P V on the matrix cores as
// well, v_mfma_f32_16x16x16_bf16 per 16 rows and 16 output dimensions.  The
// rows form NT = G / 16 tiles of 16; S^T of tile t is its own
// v_mfma_f32_16x16x32_bf16 chain.  The probabilities of S^T already sit in
// the A-operand order (lane l: row 16 t + l % 16, tokens 4 (l / 16) + r);
// each is split into a bf16 high part and the bf16 of the remainder, two
// products whose sum keeps the relative error near 2^-16.  The B operand
// (lane l: dimension 16 n + l % 16, tokens 4 (l / 16) + r) comes from the
// block's V rows staged in LDS once for all tiles, rows past the valid tokens
// zeroed.  The output O[row][dim] of tile t sits in 8 accumulators per lane
// (lane l: dimension 16 n + l % 16, rows 16 t + 4 (l / 16) + r): 32 registers
// per tile instead of the 128 the vector-ALU form needs for 16 rows.
template <int G> struct AttnWaveM {
    static_assert(G == 16 || G == 32, "whole 16-row tiles");
    static constexpr int NT = G / 16;
    static constexpr int D = 128, BS = 16, BLK = 2 * BS * D;
    static constexpr int kStage = BS * D;  // bf16 elements staged per wave
    int col, kg, koff, voff;
    bf16x8 qb[4 * NT];
    float m[NT], lsum[NT];
    f32x4 o[NT][8];
    uint16_t *vst = nullptr;  // this wave's staging area in LDS

    __device__ __forceinline__ void lanes() {
        const int lane = threadIdx.x & 63;
        col = lane & 15;
        kg = lane >> 4;
        koff = col * D + 8 * kg;
        voff = BS * D + 4 * kg * D + 8 * col;
    }
    int nreal = G;  // rows whose partials are written
    __device__ __forceinline__ void init(const QRows &qr, int64_t b, int h) {
        load_q(qb, qr, b, h);
        reset();
    }
    __device__ __forceinline__ void load_q(bf16x8 (&dst)[4 * NT], const QRows &qr, int64_t b,
                                           int h) const {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint16_t *qp = query_row(qr, b, h, 16 * t + col) + 8 * kg;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[4 * t + i] =
                    __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp + 32 * i));
        }
    }
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            m[t] = -INFINITY;
            lsum[t] = 0.f;
#pragma unroll
            for (int n = 0; n < 8; ++n) o[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __device__ __forceinline__ void load(uint4 (&kk)[4], uint4 (&vv)[4], const uint16_t *p) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) kk[i] = gload16(p + koff + 32 * i);
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = gload16(p + voff + r * D);
    }
    __device__ __forceinline__ void load_nt(uint4 (&kk)[4], uint4 (&vv)[4],
                                            const uint16_t *p) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) kk[i] = gload16_nt(p + koff + 32 * i);
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = gload16_nt(p + voff + r * D);
    }
    __device__ __forceinline__ void store(uint16_t *p, const uint4 (&kk)[4],
                                          const uint4 (&vv)[4]) const {
#pragma unroll
        for (int c = 0; c < 4; ++c) gstore16(p + koff + 32 * c, kk[c]);
#pragma unroll
        for (int r = 0; r < 4; ++r) gstore16(p + voff + r * D, vv[r]);
    }
    __device__ __forceinline__ void block(const uint4 (&kk)[4], const uint4 (&vv)[4], int valid,
                                          float scale_log2) {
        s16x4 ahi[NT], alo[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk[c]),
                                                             qb[4 * t + c], s4, 0, 0, 0);
            float sr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sr[r] = (4 * kg + r < valid) ? s4[r] * scale_log2 : -INFINITY;
            float bm = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
            bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float mn = fmaxf(m[t], bm);
            const bool live = mn != -INFINITY;
            const float alpha = live ? exp2f(m[t] - mn) : 1.f;
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = live ? exp2f(sr[r] - mn) : 0.f;
            lsum[t] = lsum[t] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
            m[t] = mn;
            // rescale the rows of O (rows 4 kg + r of the tile); row h's
            // factor is in lane h
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
                for (int n = 0; n < 8; ++n) o[t][n][r] *= ar;
            }
            // P as bf16 high part + bf16 of the remainder
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t hb = __float_as_uint(p[r]) & 0xFFFF0000u;
                const float rest = p[r] - __uint_as_float(hb);
                ahi[t][r] = (short)(hb >> 16);
                alo[t][r] = (short)(__float_as_uint(rest) >> 16);
            }
        }
        // stage V (rows past the valid tokens zeroed: probability 0, bytes
        // possibly anything); the previous block's reads are done first
        wave_sync();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint4 w = (4 * kg + r < valid) ? vv[r] : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(vst + (4 * kg + r) * D + 8 * col) = w;
        }
        wave_sync();
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            s16x4 bv;
#pragma unroll
            for (int r = 0; r < 4; ++r) bv[r] = (short)vst[(4 * kg + r) * D + 16 * n + col];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                o[t][n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi[t], bv, o[t][n], 0, 0, 0);
                o[t][n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo[t], bv, o[t][n], 0, 0, 0);
            }
        }
    }
    // Sum the four token groups of lsum; O already holds all the tokens.
    __device__ __forceinline__ void reduce() {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            lsum[t] += __shfl_xor(lsum[t], 16, 64);
            lsum[t] += __shfl_xor(lsum[t], 32, 64);
        }
    }
    __device__ __forceinline__ void write_partial(int64_t pi0, float *part_m, float *part_l,
                                                  float *part_acc) const {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (16 * t >= nreal) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (16 * t + 4 * kg + r >= nreal) continue;
#pragma unroll
                for (int n = 0; n < 8; ++n)
                    part_acc[(pi0 + 16 * t + 4 * kg + r) * D + 16 * n + col] = o[t][n][r];
            }
            if (kg == 0 && 16 * t + col < nreal) {
                part_m[pi0 + 16 * t + col] = m[t];
                part_l[pi0 + 16 * t + col] = lsum[t];
            }
        }
    }
    __device__ __forceinline__ void stash(float (*sacc)[D], float *sm, float *sl) const {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int n = 0; n < 8; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[16 * t + 4 * kg + r][16 * n + col] = o[t][n][r];
            if (kg == 0) {
                sm[16 * t + col] = m[t];
                sl[16 * t + col] = lsum[t];
            }
        }
    }
};

__device__ __forceinline__ int block_valid(int64_t T, int32_t blk) {
    const int64_t first = (int64_t)blk * 16;
    return (int)((T - first) < 16 ? (T - first) : 16);
}

// Fetch waves of a fused launch (mode 1): item i of unit u, i < cap, is the
// i-th block fetched for u this step (attended entry n_att - n_fetch + i: the
// fetched blocks end the list).  Wave f of the F = 4 n_fetch_wg fetch waves
// takes items f, f + F, ...: it reads the block from the pinned host KV over
// the host link, writes it into its slot (the copy later steps will hit),
// attends to it from registers and writes partial i of the unit; items past
// their unit's fetch count get an empty partial (m = -inf).  A wave first
// reads the list entries of up to 64 of its items at once, one per lane, and
// then streams the existing ones one after the other: with the entries in
// registers, no dependent list read sits between two host reads.  Keeping a
// second item's host loads in flight (two register buffers) measured slower
// on the host link here: the extra registers cost the resident waves of the
// same launch one wave per SIMD.  A few such waves keep the host link
// saturated while holding only a small share of the CU slots.
template <int G, bool FromSlots = false, typename W>
__device__ __forceinline__ void fetch_waves(
    W &st, int wave, const QRows &qr, uint16_t *__restrict__ slots,
    const uint16_t *__restrict__ host_kv, const int32_t *__restrict__ att_block,
    const int32_t *__restrict__ att_slot, const int32_t *__restrict__ counts, int64_t T_, int Hq,
    int Hkv, int K, int S, int64_t NBmax, int cap, int n_fetch_wg, int nsa, int64_t units,
    float scale_log2, float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_acc) {
    const int lane = threadIdx.x & 63;
    const int64_t F = 4LL * n_fetch_wg;
    const int64_t n_items = units * cap;
    const int64_t it0 = (int64_t)blockIdx.x * 4 + wave;
    if (it0 >= n_items) return;
    const int64_t n_my = (n_items - it0 + F - 1) / F;
    auto rl = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };
    for (int64_t c0 = 0; c0 < n_my; c0 += 64) {
        // lane l: item it0 + (c0 + l) F = (unit u, index i)
        const int64_t item = it0 + (c0 + lane) * F;
        const bool in = c0 + lane < n_my;
        const int u = in ? (int)(item / cap) : 0, i = in ? (int)(item % cap) : 0;
        bool ok = false;
        int blk = 0, slot = 0;
        if (in) {
            const int n_att = counts[(int64_t)u * 4 + 0], n_fetch = counts[(int64_t)u * 4 + 2];
            if (i < n_fetch) {
                const int e = n_att - n_fetch + i;
                blk = att_block[(int64_t)u * K + e];
                slot = att_slot[(int64_t)u * K + e];
                ok = true;
            } else {
                for (int g = 0; g < G; ++g) {
                    part_m[((int64_t)u * nsa + i) * G + g] = -INFINITY;
                    part_l[((int64_t)u * nsa + i) * G + g] = 0.f;
                }
            }
        }
        const uint64_t mask = __ballot(ok);
        if (mask == 0) continue;
        // (a compile-time choice: with the slots a possible source, the host
        // reads could no longer be scheduled across the slot stores)
        auto src = [&](int l) -> const uint16_t * {
            const int ul = rl(u, l);
            if constexpr (FromSlots)
                return slots + ((int64_t)ul * S + rl(slot, l)) * (int64_t)W::BLK;
            else
                return host_kv + ((int64_t)ul * NBmax + rl(blk, l)) * W::BLK;
        };
        // lane l's item: read it from the host, store it into its slot,
        // attend, write partial i of its unit (from_slots: the block is in
        // its slot already, copied there by a gather)
        for (uint64_t m = mask; m; m &= m - 1) {
            const int l = __builtin_ctzll(m);
            const int ul = rl(u, l);
            uint4 kk[4], vv[4];
            st.load_q(st.qb, qr, ul / Hkv, ul % Hkv);
            st.load(kk, vv, src(l));
            st.reset();
            st.block(kk, vv, block_valid(T_, rl(blk, l)), scale_log2);
            // the whole host block (rows past T hold the host KV's zeros);
            // storing only the held rows cost this kernel 3% (78 -> 81 us
            // on the Qwen3-8B layer)
            if constexpr (!FromSlots)
                st.store(slots + ((int64_t)ul * S + rl(slot, l)) * (int64_t)W::BLK, kk, vv);
            st.reduce();
            st.write_partial(((int64_t)ul * nsa + rl(i, l)) * G, part_m, part_l, part_acc);
        }
    }
}

// Grid (1-D, 256 threads = 4 waves per workgroup):
//   workgroups [0, n_fetch_wg): fetch waves (mode 1 only).  Item i of unit u,
//     i < cap, is the i-th block fetched for u this step (attended entry
//     n_att - n_fetch + i: the fetched blocks end the list).  Wave f takes items f, f + F, ... (F = 4 n_fetch_wg): it
//     reads the block from the pinned host KV over the host link, writes it
//     into its slot (the copy later steps will hit), attends to it from
//     registers and writes partial i of the unit; an item past the unit's
//     fetch count writes an empty partial.  A few such waves keep the host
//     link saturated while holding only a small share of the CU slots.
//   workgroups after that: hit workgroups, ns1 per unit; wave w of split s
//     takes entries 4 BPW s + w + 4 j, j < BPW, of [0, n_end) (n_end =
//     n_att - n_fetch in mode 1, n_att in mode 0) from their slots; the four waves are merged
//     in LDS into partial nsf_max + s.
template <int G, int BPW>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    const QRows qr, uint16_t *__restrict__ slots, const uint16_t *__restrict__ host_kv, const int32_t *__restrict__ att_block,
    const int32_t *__restrict__ att_slot, const int32_t *__restrict__ counts, int64_t T_, int Hq,
    int Hkv, int K, int S, int64_t NBmax, int mode, int cap, int n_fetch_wg, int nsf_max,
    int ns1, int nsa, int64_t units, float scale_log2, float *__restrict__ part_m,
    float *__restrict__ part_l, float *__restrict__ part_acc) {
    static_assert(G <= 16, "the split path serves up to 16 rows per KV head");
    using W = std::conditional_t<G == 16, AttnWaveM<G>, AttnWave<G>>;
    constexpr int D = W::D;
    __shared__ __attribute__((aligned(16))) uint16_t vstage[4][W::kStage];
    // wave-uniform, so per-wave metadata comes through scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    W st;
    st.lanes();
    st.vst = vstage[wave];
    st.nreal = qr.real;

    if ((int64_t)blockIdx.x < n_fetch_wg) {
        fetch_waves<G>(st, wave, qr, slots, host_kv, att_block, att_slot, counts, T_, Hq, Hkv, K,
                       S, NBmax, cap, n_fetch_wg, nsa, units, scale_log2, part_m, part_l,
                       part_acc);
        return;
    }

    __shared__ float sm_m[4][16], sm_l[4][16];
    __shared__ float sm_acc[4][G][D];
    const int64_t g = (int64_t)blockIdx.x - n_fetch_wg;
    const int64_t u = g / ns1;
    const int s = (int)(g % ns1);
    const int e_end = __builtin_amdgcn_readfirstlane(
        mode == 1 ? counts[u * 4 + 0] - counts[u * 4 + 2] : counts[u * 4 + 0]);
    const int e_first = 4 * BPW * s + wave;
    st.init(qr, u / Hkv, (int)(u % Hkv));
    const int ne = e_first >= e_end ? 0 : (e_end - e_first + 3) / 4 < BPW ? (e_end - e_first + 3) / 4 : BPW;

    uint4 kr[2][4], vr[2][4];
    int32_t blk_cur = 0;
    if (ne > 0) {
        blk_cur = __builtin_amdgcn_readfirstlane(att_block[u * K + e_first]);
        const int32_t sl = __builtin_amdgcn_readfirstlane(att_slot[u * K + e_first]);
        st.load_nt(kr[0], vr[0], slots + (u * S + sl) * (int64_t)W::BLK);
    }
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        if (j >= ne) break;
        int32_t blk_nx = 0;
        if (j + 1 < ne) {
            const int e = e_first + 4 * (j + 1);
            blk_nx = __builtin_amdgcn_readfirstlane(att_block[u * K + e]);
            const int32_t sl = __builtin_amdgcn_readfirstlane(att_slot[u * K + e]);
            st.load_nt(kr[(j + 1) & 1], vr[(j + 1) & 1], slots + (u * S + sl) * (int64_t)W::BLK);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
        st.block(kr[j & 1], vr[j & 1], block_valid(T_, blk_cur), scale_log2);
        blk_cur = blk_nx;
    }
    st.reduce();
    st.stash(sm_acc[wave], sm_m[wave], sm_l[wave]);
    __syncthreads();

    // merge the four waves into this workgroup's partial
    for (int idx = threadIdx.x; idx < qr.real * D; idx += 256) {
        const int gg = idx / D, c = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][gg]);
        float a = 0.f, L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float wt = exp2f(sm_m[w][gg] - M);
                a += wt * sm_acc[w][gg][c];
                L += wt * sm_l[w][gg];
            }
        }
        const int64_t pi = (u * nsa + nsf_max + s) * G + gg;
        part_acc[pi * D + c] = a;
        if (c == 0) {
            part_m[pi] = M;
            part_l[pi] = L;
        }
    }
}

// ---------------------------------------------------------------- balanced hit path

// Exclusive prefix sums of the hit entries of every unit into pre[0..units]
// (LDS), by the 256 threads of a workgroup: hit entries of unit u are its
// attended list minus, in mode 1, the fetched blocks at its end.
__device__ __forceinline__ void hit_prefix(const int32_t *__restrict__ counts, int units, int mode,
                                           int32_t *pre, int32_t *red) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int chunk = (units + 255) / 256;
    const int lo = t * chunk < units ? t * chunk : units;
    const int hi = lo + chunk < units ? lo + chunk : units;
    int sum = 0;
    for (int u = lo; u < hi; ++u) {
        const int e = counts[u * 4 + 0] - (mode != 0 ? counts[u * 4 + 2] : 0);
        pre[u + 1] = e;
        sum += e;
    }
    int x = sum;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[wv] = x;
    __syncthreads();
    int r = x - sum;
    for (int i = 0; i < wv; ++i) r += red[i];
    for (int u = lo; u < hi; ++u) {
        r += pre[u + 1];
        pre[u + 1] = r;
    }
    if (t == 0) pre[0] = 0;
    __syncthreads();
}

// Sparse attention over the hit entries, with the work balanced over waves
// rather than split per unit (a unit's hit entries range from about 40 to
// 115 on the Qwen3-8B layer).  The hit entries of all units, concatenated in
// unit order (E of them), are cut into runs of P = max(ceil(E / W), pmin)
// entries; wave w streams run w and may cross from one unit into the next.
// W is what the GPU holds at once, so the launch is one round with equal
// work per wave.  A wave issues one block, waits for it and attends to it:
// on this part scattered 8 KB reads ran fastest with one block per wave in
// flight (a timing probe of the same access: 37.4 us with none ahead, 40.0
// with one block ahead, 42.4 with two, for 210 MB), and a new unit's query
// rows then travel with its first block at no extra wait.  For each unit it
// touches, a wave writes its partial at row hp0 + u R + s, s = the wave's
// rank among the waves of u (at most R = ceil(K / pmin) + 1 of them); the
// unit's last wave marks rows s + 1 .. R - 1 empty (m = -inf), and units
// without hit entries are marked by workgroup u mod the grid, so the
// combine reads a fixed set of rows with no dependent load.  Modes: 0, the
// hit waves over every attended entry; 1, fetch workgroups first in the grid
// (host reads, as in the split kernel), hit waves over the entries before
// the fetched ones; 2, those hit waves alone (attn_fetched_kernel below then
// attends to the fetched blocks from their slots).  Dynamic LDS: units + 1
// ints.
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_flat_kernel(
    const QRows qr, uint16_t *__restrict__ slots, const uint16_t *__restrict__ host_kv, const int32_t *__restrict__ att_block,
    const int32_t *__restrict__ att_slot, const int32_t *__restrict__ counts, int64_t T_, int Hq,
    int Hkv, int K, int S, int64_t NBmax, int mode, int cap, int n_fetch_wg, int nsa, int units,
    int W, int R, int pmin, float scale_log2, float *__restrict__ part_m,
    float *__restrict__ part_l, float *__restrict__ part_acc, int64_t hp0) {
    using Wv = std::conditional_t<(G >= 16), AttnWaveM<G>, AttnWave<G>>;
    __shared__ __attribute__((aligned(16))) uint16_t vstage[4][Wv::kStage];
    __shared__ int32_t red[4];
    extern __shared__ int32_t pre[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    Wv st;
    st.lanes();
    st.vst = vstage[wave];
    st.nreal = qr.real;
    if ((int)blockIdx.x < n_fetch_wg) {
        fetch_waves<G>(st, wave, qr, slots, host_kv, att_block, att_slot, counts, T_, Hq, Hkv, K,
                       S, NBmax, cap, n_fetch_wg, nsa, (int64_t)units, scale_log2, part_m,
                       part_l, part_acc);
        return;
    }
    hit_prefix(counts, units, mode, pre, red);
    const int wg = (int)blockIdx.x - n_fetch_wg, nwg = (int)gridDim.x - n_fetch_wg;
    auto mark_empty = [&](int64_t row0, int nrows, int t0, int nt) {  // rows of G partials
        for (int i = t0; i < nrows * G; i += nt) {
            part_m[row0 * G + i] = -INFINITY;
            part_l[row0 * G + i] = 0.f;
        }
    };
    for (int u = wg; u < units; u += nwg)
        if (pre[u + 1] == pre[u]) mark_empty(hp0 + (int64_t)u * R, R, threadIdx.x, 256);
    const int E = pre[units];
    if (E == 0) return;
    const int P0 = (E + W - 1) / W;
    const int P = P0 > pmin ? P0 : pmin;  // <= 64 (W >= E_max / 64)
    const int w = __builtin_amdgcn_readfirstlane(wg * 4 + wave);
    const int f0 = w * P;
    if (f0 >= E) return;
    const int n = (E - f0) < P ? (E - f0) : P;

    // lane i < n: unit, block and slot of entry f0 + i
    int my_u = 0, my_blk = 0, my_slot = 0;
    if (lane < n) {
        const int f = f0 + lane;
        int lo = 0, hi = units - 1;  // largest u with pre[u] <= f
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= f) lo = mid;
            else hi = mid - 1;
        }
        my_u = lo;
        my_blk = att_block[(int64_t)lo * K + f - pre[lo]];
        my_slot = att_slot[(int64_t)lo * K + f - pre[lo]];
    }
    auto rl = [](int v, int j) { return __builtin_amdgcn_readlane(v, j); };
    // partial of unit u from this wave; the unit's last wave marks the rest
    auto finish = [&](int u) {
        st.reduce();
        const int s0 = pre[u] / P, s1 = (pre[u + 1] - 1) / P;
        st.write_partial((hp0 + (int64_t)u * R + (w - s0)) * G, part_m, part_l, part_acc);
        if (w == s1) mark_empty(hp0 + (int64_t)u * R + (w - s0) + 1, R - 1 - (w - s0), lane, 64);
    };
    int cur_u = -1;
    auto src = [&](int j) {
        return slots + ((int64_t)rl(my_u, j) * S + rl(my_slot, j)) * Wv::BLK;
    };
    auto enter = [&](int u) {  // a new unit: its query rows, waited for with its block
        if (u == cur_u) return;
        if (cur_u >= 0) finish(cur_u);
        st.load_q(st.qb, qr, u / Hkv, u % Hkv);
        st.reset();
        cur_u = u;
    };
    if constexpr (G < 32) {
        uint4 kk[4], vv[4];
        for (int j = 0; j < n; ++j) {
            enter(rl(my_u, j));
            st.load_nt(kk, vv, src(j));
            st.block(kk, vv, block_valid(T_, rl(my_blk, j)), scale_log2);
        }
    } else {
        // 32 rows: a block's matrix work (two query tiles, V through LDS) is
        // long enough to hide part of the next block's round trip, so the
        // next block's loads are issued before it (two register buffers,
        // alternating).  A new unit's query loads go out before them, so
        // the wait for the current block and its query leaves the next
        // block in flight.  Every load in the loop is unconditional (the
        // last one or two blocks are peeled off), so that wait is never a
        // wait for everything.
        uint4 ka[4], va[4], kb[4], vb[4];
        auto valid = [&](int j) { return block_valid(T_, rl(my_blk, j)); };
        st.load_nt(ka, va, src(0));
        int j = 0;
        for (; j + 2 < n; j += 2) {
            enter(rl(my_u, j));
            st.load_nt(kb, vb, src(j + 1));
            st.block(ka, va, valid(j), scale_log2);
            enter(rl(my_u, j + 1));
            st.load_nt(ka, va, src(j + 2));
            st.block(kb, vb, valid(j + 1), scale_log2);
        }
        enter(rl(my_u, j));  // block j is in (ka, va); one more may follow
        if (j + 1 < n) {
            st.load_nt(kb, vb, src(j + 1));
            st.block(ka, va, valid(j), scale_log2);
            enter(rl(my_u, j + 1));
            st.block(kb, vb, valid(j + 1), scale_log2);
        } else {
            st.block(ka, va, valid(j), scale_log2);
        }
    }
    finish(cur_u);
}

// The fetched entries of a mode-2 launch, from their slots once a gather on
// another stream has copied them: the fetch waves' item loop (one wave per
// item, partial i of the unit as mode 1 writes it) with the slots as the
// source and no store.  A kernel of its own, so that the host-reading fetch
// waves keep their code and schedule.
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_fetched_kernel(
    const QRows qr, uint16_t *__restrict__ slots, const int32_t *__restrict__ att_block,
    const int32_t *__restrict__ att_slot, const int32_t *__restrict__ counts, int64_t T_, int Hq,
    int Hkv, int K, int S, int cap, int nsa, int units, float scale_log2,
    float *__restrict__ part_m, float *__restrict__ part_l, float *__restrict__ part_acc) {
    using Wv = std::conditional_t<(G >= 16), AttnWaveM<G>, AttnWave<G>>;
    __shared__ __attribute__((aligned(16))) uint16_t vstage[4][Wv::kStage];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Wv st;
    st.lanes();
    st.vst = vstage[wave];
    st.nreal = qr.real;
    fetch_waves<G, true>(st, wave, qr, slots, nullptr, att_block, att_slot, counts, T_, Hq, Hkv,
                         K, S, 0, cap, (int)gridDim.x, nsa, (int64_t)units, scale_log2, part_m,
                         part_l, part_acc);
}

// ---------------------------------------------------------------- combine

// Output row (b, query head qh) from its n partials, partial i at row
// pidx(i); thread c owns output dimension c.
template <typename F>
__device__ __forceinline__ void combine_row(const float *__restrict__ part_m,
                                            const float *__restrict__ part_l,
                                            const float *__restrict__ part_acc,
                                            float *__restrict__ out, int Hq, int d, int b, int qh,
                                            int n, F pidx) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
        float M = -INFINITY, L = 0.f, a = 0.f;
        merge_partials(part_m, part_l, part_acc, d, c, n, pidx, M, L, a);
        out[((int64_t)b * Hq + qh) * d + c] = (L > 0.f) ? a / L : 0.f;
    }
}

// One workgroup per (b, query head).  The partials of a unit are splits
// [0, n_a) and [off_b, off_b + n_b) of nsa.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ part_m,
                                                      const float *__restrict__ part_l,
                                                      const float *__restrict__ part_acc,
                                                      float *__restrict__ out, int Hq, int Hkv,
                                                      int G, int d, int nsa, int n_a, int off_b,
                                                      int n_b) {
    const int qh = blockIdx.x, b = blockIdx.y;
    const int h = qh / G, g = qh % G;
    const int64_t u = (int64_t)b * Hkv + h;
    combine_row(part_m, part_l, part_acc, out, Hq, d, b, qh, n_a + n_b, [&](int i) -> int64_t {
        const int s = i < n_a ? i : off_b + (i - n_a);
        return (u * nsa + s) * G + g;
    });
}

// The same after the balanced hit path, d = 128: the unit's n_f fetch
// partials (splits [0, n_f) of nsa), then its R hit partial rows
// hp0 + u R + s, the unused ones marked empty; gt query rows per partial.
// One wave per output row (four per workgroup), merging with merge_row_wave:
// the m and l of every partial and the sums of the first 16 in one round
// trip, the sums of later live ones after (4.58 -> 4.46 us on the Qwen3-8B
// layer against reading the m and l first).
__global__ __launch_bounds__(256) void combine_flat_kernel(
    const float *__restrict__ part_m, const float *__restrict__ part_l,
    const float *__restrict__ part_acc, float *__restrict__ out, int Hq, int Hkv, int G,
    int gt, int nsa, int n_f, int R, int64_t hp0) {
    const int qh = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
    const int b = blockIdx.y;
    if (qh >= Hq) return;
    const int h = qh / G, g = qh % G;
    const int u = b * Hkv + h;
    float M = -INFINITY, L = 0.f;
    float2 a = make_float2(0.f, 0.f);
    merge_row_wave<true>(part_m, part_l, part_acc, n_f + R, [&](int i) -> int64_t {
        if (i < n_f) return ((int64_t)u * nsa + i) * gt + g;
        return (hp0 + (int64_t)u * R + (i - n_f)) * gt + g;
    }, M, L, a);
    const float2 o = L > 0.f ? make_float2(a.x / L, a.y / L) : make_float2(0.f, 0.f);
    *reinterpret_cast<float2 *>(out + ((int64_t)b * Hq + qh) * 128 + 2 * (threadIdx.x & 63)) = o;
}

// ---------------------------------------------------------------- host side

static bool mfma_ok(const Dims &D) {
    const bool g_ok = D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8 || D.G == 16;
    return D.dtype == kBF16 && D.d == 128 && D.bs == 16 && g_ok;
}

// Rows of the balanced kernel's tile for G query rows per KV head.  Eight
// rows run on the 16-row matrix-core tile (P V on the matrix cores, 142
// VGPRs against 206): with 64 accumulators per lane the vector-ALU form's P V
// arithmetic, not HBM, set that kernel's time.  Four rows stay on the
// vector ALU: the 16-row tile made the Qwen3-8B layer's fused attention
// slower (82 -> 89 us) for no gain over resident blocks.
static int tile_rows(int G) { return G == 8 ? 16 : G; }

// Query rows per unit of one balanced launch: a launch that also fetches
// (nsf > 0) keeps the vector-ALU form for G = 8, whose fetch waves kept the
// host link busier (51.5 against 50.9 GB/s on the Qwen3-32B layer); a
// launch over resident blocks only takes the plan's tile (Qwen3-32B layer:
// 26.3 -> 22.8 us).  The partial buffers hold the larger of the two.
static int flat_rows_of_call(const Dims &D, const AttnPlan &P, int nsf) {
    return nsf > 0 ? D.G : P.gt;
}

// 32 rows per KV head (32 heads per KV head, or a 32-row verification chunk)
// run on the balanced kernel only.
static bool mfma32_ok(const Dims &D) {
    return D.dtype == kBF16 && D.d == 128 && D.bs == 16 && D.G == 32;
}

// Units whose hit-entry prefix sums the balanced kernel keeps in LDS.
constexpr int kFlatMaxUnits = 4096;

template <int G> static int flat_wgs_per_cu(int units) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_flat_kernel<G>, 256,
                                                     sizeof(int32_t) * (units + 1)) != hipSuccess)
        n = 0;
    return n;
}

AttnPlan plan_attention(const Dims &D) {
    AttnPlan P{};
    P.mfma = mfma_ok(D) || mfma32_ok(D);
    const int64_t units = D.units();
    if (P.mfma) {
        // largest blocks-per-wave that still gives >= 1024 workgroups
        int bpw = 8;
        while (bpw > 1 && units * ((D.K + 4 * bpw - 1) / (4 * bpw)) < 1024) bpw /= 2;
        P.blocks_per_wave = bpw;
        P.ns1 = (D.K + 4 * bpw - 1) / (4 * bpw);
        P.nsf_max = D.K;
        // Balanced hit path: as many waves as the GPU holds at once, runs of
        // at most 64 entries (one list entry per lane).
        if (units <= kFlatMaxUnits && !getenv("OASIS_ATTN_SPLIT")) {
            const int cus = compute_units(D);
            int per_cu = 0;
            {
                const int u = (int)units;
                switch (tile_rows(D.G)) {
                case 1: per_cu = flat_wgs_per_cu<1>(u); break;
                case 2: per_cu = flat_wgs_per_cu<2>(u); break;
                case 4: per_cu = flat_wgs_per_cu<4>(u); break;
                case 8: per_cu = flat_wgs_per_cu<8>(u); break;
                case 16: per_cu = flat_wgs_per_cu<16>(u); break;
                default: per_cu = flat_wgs_per_cu<32>(u); break;
                }
            }
            const int64_t emax = units * D.K;
            // at most two workgroups (eight waves) per CU: more concurrent
            // block streams read slower (a timing probe of the access: 37.3
            // us with 8 waves per CU, 39.2 with 12, for 210 MB)
            int64_t w = (int64_t)cus * std::min(per_cu, 2) * 4;
            w = std::min<int64_t>(w, std::max<int64_t>(4, (emax + 1) / 2));
            w = (w + 3) / 4 * 4;
            if (per_cu > 0 && w * 64 >= emax && w <= (1 << 20)) {
                P.flat = true;
                P.flat_waves = (int)w;
                // runs of at least pmin entries, so that a unit's K entries
                // meet at most R waves (the combine reads R rows per unit):
                // 8 where full lists give each wave 8 or more entries, down to
                // 2 for small batches (64 units), which would otherwise leave
                // most waves idle
                const int64_t per = (emax * 2 + 3 * w - 1) / (3 * w);  // ~ emax / 1.5 W
                const int pm = (int)std::max<int64_t>(2, std::min<int64_t>(8, per));
                const int segs = (D.K + pm - 1) / pm;
                P.flat_pmin = (D.K + segs - 1) / segs;
                P.flat_rows = segs + 1;
            }
        }
        if (D.G == 32 && !P.flat) P = AttnPlan{};  // the generic kernel instead
        P.gt = P.flat ? tile_rows(D.G) : D.G;
    }
    if (!P.mfma) {
        int bps = 8;
        while (bps > 1 && units * ((D.K + bps - 1) / bps) < 1024) bps /= 2;
        P.blocks_per_wave = bps;
        P.ns1 = (D.K + bps - 1) / bps;
        P.nsf_max = 0;
    }
    if (!P.mfma) P.gt = D.G;
    P.nsa = P.nsf_max + (P.flat ? 0 : P.ns1);
    P.vns = P.ns1;
    return P;
}

int verify_stride(const Dims &D) {
    int v = plan_attention(D).ns1;
    if (!mfma_ok(D)) return v;
    for (int g : {1, 2, 4, 8, 16, 32}) {
        Dims Dc = D;
        Dc.G = g;
        Dc.Hq = D.Hkv * g;
        const AttnPlan Pc = plan_attention(Dc);
        v = std::max(v, Pc.flat ? Pc.flat_rows : Pc.ns1);
    }
    return v;
}

int64_t attn_partial_rows(const Dims &D, const AttnPlan &P) {
    int64_t rows = D.units() * P.nsa * P.gt;
    if (P.flat) rows += D.units() * P.flat_rows * P.gt;
    return rows;
}

int attention_fetch_splits(const Dims &D, const AttnPlan &P, int cap) {
    if (!P.mfma || cap <= 0) return 0;
    return cap > D.K ? D.K : cap;
}

// Fetch workgroups for a fused launch.  Host reads by shader loads reach
// their best rate (about 50 GB/s, against 58 GB/s for a pinned DMA copy) with
// about 64 waves each keeping two blocks in flight; more waves lower the rate
// (256 waves: -10%, 512: -30%), fewer cannot cover the link latency.  Small
// fetch lists get one wave per two items.
static int fetch_workgroups(int64_t items) {
    int64_t waves = (items + 1) / 2;
    if (waves > 64) waves = 64;
    if (waves < 4) waves = 4;
    return (int)((waves + 3) / 4);
}

template <int G>
static void launch_mfma_g(const AttnPlan &P, dim3 grid, hipStream_t st, const QRows &q,
                          uint16_t *slots, const uint16_t *host_kv, const int32_t *ab,
                          const int32_t *as, const int32_t *counts, int64_t T, const Dims &D,
                          int mode, int cap, int n_fetch_wg, float sc, float *pm, float *pl,
                          float *pa) {
#define OASIS_ATTN(BPW)                                                                        \
    OASIS_LAUNCH((attn_mfma_kernel<G, BPW>), grid, dim3(256), 0, st, q, slots, host_kv,  \
                       ab, as, counts, T, D.Hq, D.Hkv, D.K, D.S, D.NBmax, mode, cap,           \
                       n_fetch_wg, P.nsf_max, P.ns1, P.nsa, D.units(), sc, pm, pl, pa)
    switch (P.blocks_per_wave) {
    case 1: OASIS_ATTN(1); break;
    case 2: OASIS_ATTN(2); break;
    case 4: OASIS_ATTN(4); break;
    default: OASIS_ATTN(8); break;
    }
#undef OASIS_ATTN
}

template <int G>
static void launch_flat_g(const AttnPlan &P, dim3 grid, size_t lds, hipStream_t st,
                          const QRows &q, uint16_t *slots, const uint16_t *host_kv,
                          const int32_t *ab, const int32_t *as, const int32_t *counts, int64_t T,
                          const Dims &D, int mode, int cap, int n_fetch_wg, int hit_waves,
                          float sc, float *pm, float *pl, float *pa) {
    OASIS_LAUNCH((attn_flat_kernel<G>), grid, dim3(256), lds, st, q, slots, host_kv, ab, as,
                 counts, T, D.Hq, D.Hkv, D.K, D.S, D.NBmax, mode, cap, n_fetch_wg, P.nsa,
                 (int)D.units(), hit_waves, P.flat_rows, P.flat_pmin, sc, pm, pl, pa,
                 D.units() * P.nsa);
}

// Hit waves of a balanced launch.  Alone, all the GPU holds at once.  In a
// launch that also fetches, the hits only have to be done when the transfer
// is: fewer hit waves, each with a longer run, then press less on the host
// reads, and leave CUs free of hit waves for the fetch workgroups (a CU's
// vector-memory loads complete at the pace of its slowest outstanding load,
// so hit waves beside a fetch wave wait on the host round trip).  The count
// paces the largest hit list (K per unit, about 1.5 us per block for a wave
// at this concurrency) to the transfer of nsf blocks per unit at 50 GB/s;
// the units cancel.  Qwen3-8B layer at cap 2: 584 waves instead of 2,048,
// fused attention 82.5 -> 78.5 us (host link 50.8 -> 53.4 GB/s); a quarter
// of them on every CU (1,024 waves) was slower, 98 us.
static int flat_hit_waves(const Dims &D, const AttnPlan &P, int nsf) {
    if (nsf <= 0) return P.flat_waves;
    const double t_block = 1.5e-6, host_rate = 50e9, blk = 8192.0;
    const double w = (double)D.K * t_block * host_rate / ((double)nsf * blk);
    const int64_t lo = (D.units() * D.K + 63) / 64;  // runs of at most 64 entries
    int64_t hw = (int64_t)w / 4 * 4;
    if (hw < lo) hw = (lo + 3) / 4 * 4;
    if (hw > P.flat_waves) hw = P.flat_waves;
    return (int)hw;
}

hipError_t launch_attention(const Dims &D, const AttnPlan &P, int mode, int nsf, const void *q,
                            void *slots, const void *host_kv, const int32_t *att_block,
                            const int32_t *att_slot, const int32_t *counts, int64_t T,
                            float *part_m, float *part_l, float *part_acc, hipStream_t st,
                            const QRows *qrows) {
    const float sc = kLog2e / sqrtf((float)D.d);
    const QRows qq = qrows ? *qrows : QRows{(const uint16_t *)q, nullptr, 0, D.Hq, D.G, 0, D.G};
    if (P.mfma && P.flat && mode == 3) {
        // the fetched blocks from HBM: a wave per block, up to 8 per CU
        if (nsf <= 0) return hipSuccess;
        const int64_t waves = std::min<int64_t>(D.units() * nsf, 8LL * compute_units(D));
        const dim3 grid((unsigned)((waves + 3) / 4));
        uint16_t *sl = (uint16_t *)slots;
#define OASIS_FETCHED(GG)                                                                        \
    OASIS_LAUNCH((attn_fetched_kernel<GG>), grid, dim3(256), 0, st, qq, sl, att_block, att_slot, \
                 counts, T, D.Hq, D.Hkv, D.K, D.S, nsf, P.nsa, (int)D.units(), sc, part_m,       \
                 part_l, part_acc)
        switch (flat_rows_of_call(D, P, nsf)) {
        case 1: OASIS_FETCHED(1); break;
        case 2: OASIS_FETCHED(2); break;
        case 4: OASIS_FETCHED(4); break;
        case 8: OASIS_FETCHED(8); break;
        case 16: OASIS_FETCHED(16); break;
        default: OASIS_FETCHED(32); break;
        }
#undef OASIS_FETCHED
        return hipGetLastError();
    }
    if (P.mfma && P.flat) {
        if (mode == 0) nsf = 0;
        int n_fetch_wg = 0, hw = 0;
        if (mode == 2) {
            hw = P.flat_waves;
        } else {
            n_fetch_wg = nsf > 0 ? fetch_workgroups(D.units() * nsf) : 0;
            hw = flat_hit_waves(D, P, nsf);
        }
        const dim3 grid((unsigned)(n_fetch_wg + hw / 4));
        const size_t lds = sizeof(int32_t) * (D.units() + 1);
        const uint16_t *hk = (const uint16_t *)host_kv;
        uint16_t *sl = (uint16_t *)slots;
#define OASIS_FLAT(GG)                                                                          \
    launch_flat_g<GG>(P, grid, lds, st, qq, sl, hk, att_block, att_slot, counts, T, D, mode, nsf, \
                      n_fetch_wg, hw, sc, part_m, part_l, part_acc)
        switch (flat_rows_of_call(D, P, nsf)) {
        case 1: OASIS_FLAT(1); break;
        case 2: OASIS_FLAT(2); break;
        case 4: OASIS_FLAT(4); break;
        case 8: OASIS_FLAT(8); break;
        case 16: OASIS_FLAT(16); break;
        default: OASIS_FLAT(32); break;
        }
#undef OASIS_FLAT
        return hipGetLastError();
    }
    if (P.mfma) {
        if (D.G > 16) return hipErrorInvalidValue;  // planned on the balanced kernel only
        if (mode == 0) nsf = 0;
        const int n_fetch_wg = nsf > 0 ? fetch_workgroups(D.units() * nsf) : 0;
        dim3 grid((unsigned)(n_fetch_wg + D.units() * P.ns1));
        const uint16_t *hk = (const uint16_t *)host_kv;
        uint16_t *sl = (uint16_t *)slots;
        switch (D.G) {
        case 1: launch_mfma_g<1>(P, grid, st, qq, sl, hk, att_block, att_slot, counts, T, D, mode, nsf, n_fetch_wg, sc, part_m, part_l, part_acc); break;
        case 2: launch_mfma_g<2>(P, grid, st, qq, sl, hk, att_block, att_slot, counts, T, D, mode, nsf, n_fetch_wg, sc, part_m, part_l, part_acc); break;
        case 4: launch_mfma_g<4>(P, grid, st, qq, sl, hk, att_block, att_slot, counts, T, D, mode, nsf, n_fetch_wg, sc, part_m, part_l, part_acc); break;
        case 8: launch_mfma_g<8>(P, grid, st, qq, sl, hk, att_block, att_slot, counts, T, D, mode, nsf, n_fetch_wg, sc, part_m, part_l, part_acc); break;
        default: launch_mfma_g<16>(P, grid, st, qq, sl, hk, att_block, att_slot, counts, T, D, mode, nsf, n_fetch_wg, sc, part_m, part_l, part_acc); break;
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)P.ns1, D.Hkv, D.B);
    const int epl = (D.d + 63) / 64;
#define OASIS_GENERIC(TT, E)                                                                     \
    OASIS_LAUNCH((attn_generic_kernel<TT, E>), grid, dim3(64), 0, st, (const TT *)q,       \
                       (const TT *)slots, att_block, att_slot, counts, T, D.Hq, D.Hkv, D.G, D.d, \
                       D.K, D.S, D.bs, P.blocks_per_wave, P.nsa, P.nsf_max, sc, part_m, part_l,  \
                       part_acc)
    if (D.dtype == kF32) {
        if (epl == 1) OASIS_GENERIC(float, 1);
        else if (epl == 2) OASIS_GENERIC(float, 2);
        else OASIS_GENERIC(float, 4);
    } else {
        if (epl == 1) OASIS_GENERIC(uint16_t, 1);
        else if (epl == 2) OASIS_GENERIC(uint16_t, 2);
        else OASIS_GENERIC(uint16_t, 4);
    }
#undef OASIS_GENERIC
    return hipGetLastError();
}

hipError_t launch_combine(const Dims &D, const AttnPlan &P, int nsf, const float *part_m,
                          const float *part_l, const float *part_acc, float *out,
                          hipStream_t st) {
    if (P.flat) {  // d = 128
        OASIS_LAUNCH(combine_flat_kernel, dim3((D.Hq + 3) / 4, D.B), dim3(256), 0, st, part_m,
                     part_l, part_acc, out, D.Hq, D.Hkv, D.G, flat_rows_of_call(D, P, nsf), P.nsa,
                     nsf, P.flat_rows,
                     D.units() * P.nsa);
        return hipGetLastError();
    }
    OASIS_LAUNCH(combine_kernel, dim3(D.Hq, D.B), dim3(D.d <= 256 ? D.d : 256), 0, st,
                       part_m, part_l, part_acc, out, D.Hq, D.Hkv, D.G, D.d, P.nsa, nsf,
                       P.nsf_max, P.ns1);
    return hipGetLastError();
}

}  // namespace oasis
