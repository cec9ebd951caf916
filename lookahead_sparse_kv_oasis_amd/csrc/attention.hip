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
#include "kernels.h"

namespace oasis {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- any dtype

// One wave per (split, unit); each lane owns d elements c = lane + 64 e.
template <typename T, int EPL>
__global__ __launch_bounds__(64) void attn_generic_kernel(
    const T *__restrict__ q, const T *__restrict__ slots, const int32_t *__restrict__ att_block,
    const int32_t *__restrict__ att_slot, const int32_t *__restrict__ counts, int64_t T_, int Hq,
    int Hkv, int G, int d, int K, int S, int bs, int bps, int n_splits, float scale_log2,
    float *__restrict__ part_m, float *__restrict__ part_l, float *__restrict__ part_acc) {
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
        const int64_t pi = (u * n_splits + split) * G + g;
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

// Four waves per (split, unit); wave w takes attended entries
// split * 4 * BPW + w + 4 i.  Per 16-token block:
//   S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (tokens are the M rows, the G
//   heads of the group the N columns, zero-padded to 16).  Lane l supplies
//   token / head l % 16 and the 32 consecutive dimensions 32 (l / 16) ...,
//   8 per MFMA step, so every lane reads one contiguous 64-byte piece of its
//   key row.  The accumulator of lane l holds head l % 16 for tokens
//   4 (l / 16) + r, r < 4.
//   P V on the vector ALU in fp32: lane l owns tokens 4 (l / 16) + r and the
//   8 dimensions 8 (l % 16) ...; the probabilities of head g for its tokens
//   sit in lane 16 (l / 16) + g of the same 16-lane row, so a DPP row
//   broadcast delivers them.
template <int G, int BPW>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ slots,
    const int32_t *__restrict__ att_block, const int32_t *__restrict__ att_slot,
    const int32_t *__restrict__ counts, int64_t T_, int Hq, int Hkv, int K, int S, int n_splits,
    float scale_log2, float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_acc) {
    constexpr int D = 128, BS = 16;
    __shared__ float sm_m[4][16], sm_l[4][16];
    __shared__ float sm_acc[4][G][D];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int64_t u = (int64_t)b * Hkv + h;
    const int n_att = counts[u * 4];
    const int col = lane & 15, kg = lane >> 4;

    bf16x8 qb[4];
    {
        const uint16_t *qr = q + ((int64_t)b * Hq + h * G + (col < G ? col : 0)) * D + 32 * kg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 w = *reinterpret_cast<const uint4 *>(qr + 8 * i);
            if (col >= G) w = make_uint4(0, 0, 0, 0);
            qb[i] = __builtin_bit_cast(bf16x8, w);
        }
    }

    float m = -INFINITY, lsum = 0.f;
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

    const int e0 = split * 4 * BPW + wave;
#pragma unroll 1
    for (int bi = 0; bi < BPW; ++bi) {
        const int e = e0 + 4 * bi;
        if (e >= n_att) break;
        const int32_t blk = att_block[u * K + e], slot = att_slot[u * K + e];
        const int64_t first = (int64_t)blk * BS;
        const int valid = (int)((T_ - first) < BS ? (T_ - first) : BS);
        const uint16_t *kp = slots + (u * S + slot) * 2 * (int64_t)BS * D;
        const uint16_t *vp = kp + BS * D;

        bf16x8 ka[4];
        const uint16_t *kr = kp + col * D + 32 * kg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ka[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(kr + 8 * i));
        uint4 vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vr[r] = *reinterpret_cast<const uint4 *>(vp + (4 * kg + r) * D + 8 * col);
            if (4 * kg + r >= valid) vr[r] = make_uint4(0, 0, 0, 0);
        }

        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qb[i], s4, 0, 0, 0);

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

        float vf[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) bf16x8_to_f32(vr[r], vf[r]);

        static_for<0, G>([&](auto gi) {
            constexpr int g = decltype(gi)::value;
            const float ag = row_bcast<g>(alpha);
            float pg[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pg[r] = row_bcast<g>(p[r]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = acc[g][e] * ag;
#pragma unroll
                for (int r = 0; r < 4; ++r) a += pg[r] * vf[r][e];
                acc[g][e] = a;
            }
        });
    }

    // reduce over the four token groups of the wave
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
    if (kg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_acc[wave][g][8 * col + e] = acc[g][e];
        sm_m[wave][col] = m;
        sm_l[wave][col] = lsum;
    }
    __syncthreads();

    // merge the four waves into this split's partial
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int g = idx / D, c = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][g]);
        float a = 0.f, L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float wt = exp2f(sm_m[w][g] - M);
                a += wt * sm_acc[w][g][c];
                L += wt * sm_l[w][g];
            }
        }
        const int64_t pi = (u * n_splits + split) * G + g;
        part_acc[pi * D + c] = a;
        if (c == 0) {
            part_m[pi] = M;
            part_l[pi] = L;
        }
    }
}

// ---------------------------------------------------------------- combine

// One workgroup per (b, query head); thread c owns output dimension c.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ part_m,
                                                      const float *__restrict__ part_l,
                                                      const float *__restrict__ part_acc,
                                                      float *__restrict__ out, int Hq, int Hkv,
                                                      int G, int d, int n_splits) {
    const int qh = blockIdx.x, b = blockIdx.y;
    const int h = qh / G, g = qh % G;
    const int64_t u = (int64_t)b * Hkv + h;
    const int64_t base = u * n_splits * G + g;  // partial index of split s: base + s * G
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_m[base + (int64_t)s * G]);
    float L = 0.f;
    if (M != -INFINITY)
        for (int s = 0; s < n_splits; ++s) {
            const int64_t pi = base + (int64_t)s * G;
            L += exp2f(part_m[pi] - M) * part_l[pi];
        }
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
        float a = 0.f;
        if (M != -INFINITY)
            for (int s = 0; s < n_splits; ++s) {
                const int64_t pi = base + (int64_t)s * G;
                a += exp2f(part_m[pi] - M) * part_acc[pi * d + c];
            }
        out[((int64_t)b * Hq + qh) * d + c] = (L > 0.f) ? a / L : 0.f;
    }
}

// ---------------------------------------------------------------- host side

static bool mfma_ok(const Dims &D) {
    const bool g_ok = D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8 || D.G == 16;
    return D.dtype == kBF16 && D.d == 128 && D.bs == 16 && g_ok;
}

AttnPlan plan_attention(const Dims &D) {
    AttnPlan P;
    P.mfma = mfma_ok(D);
    const int64_t units = D.units();
    if (P.mfma) {
        // largest blocks-per-wave that still gives >= 1024 workgroups
        int bpw = 8;
        while (bpw > 1 && units * ((D.K + 4 * bpw - 1) / (4 * bpw)) < 1024) bpw /= 2;
        P.blocks_per_wave = bpw;
        P.n_splits = (D.K + 4 * bpw - 1) / (4 * bpw);
    } else {
        int bps = 8;
        while (bps > 1 && units * ((D.K + bps - 1) / bps) < 1024) bps /= 2;
        P.blocks_per_wave = bps;
        P.n_splits = (D.K + bps - 1) / bps;
    }
    return P;
}

template <int G>
static void launch_mfma_g(const AttnPlan &P, dim3 grid, hipStream_t st, const uint16_t *q,
                          const uint16_t *slots, const int32_t *ab, const int32_t *as,
                          const int32_t *counts, int64_t T, const Dims &D, float sc, float *pm,
                          float *pl, float *pa) {
    switch (P.blocks_per_wave) {
    case 1:
        hipLaunchKernelGGL((attn_mfma_kernel<G, 1>), grid, dim3(256), 0, st, q, slots, ab, as,
                           counts, T, D.Hq, D.Hkv, D.K, D.S, P.n_splits, sc, pm, pl, pa);
        break;
    case 2:
        hipLaunchKernelGGL((attn_mfma_kernel<G, 2>), grid, dim3(256), 0, st, q, slots, ab, as,
                           counts, T, D.Hq, D.Hkv, D.K, D.S, P.n_splits, sc, pm, pl, pa);
        break;
    case 4:
        hipLaunchKernelGGL((attn_mfma_kernel<G, 4>), grid, dim3(256), 0, st, q, slots, ab, as,
                           counts, T, D.Hq, D.Hkv, D.K, D.S, P.n_splits, sc, pm, pl, pa);
        break;
    default:
        hipLaunchKernelGGL((attn_mfma_kernel<G, 8>), grid, dim3(256), 0, st, q, slots, ab, as,
                           counts, T, D.Hq, D.Hkv, D.K, D.S, P.n_splits, sc, pm, pl, pa);
        break;
    }
}

hipError_t launch_attention(const Dims &D, const AttnPlan &P, const void *q, const void *slots,
                            const int32_t *att_block, const int32_t *att_slot,
                            const int32_t *counts, int64_t T, float *part_m, float *part_l,
                            float *part_acc, hipStream_t st) {
    const float sc = kLog2e / sqrtf((float)D.d);
    dim3 grid((unsigned)P.n_splits, D.Hkv, D.B);
    if (P.mfma) {
        const uint16_t *qq = (const uint16_t *)q, *sl = (const uint16_t *)slots;
        switch (D.G) {
        case 1: launch_mfma_g<1>(P, grid, st, qq, sl, att_block, att_slot, counts, T, D, sc, part_m, part_l, part_acc); break;
        case 2: launch_mfma_g<2>(P, grid, st, qq, sl, att_block, att_slot, counts, T, D, sc, part_m, part_l, part_acc); break;
        case 4: launch_mfma_g<4>(P, grid, st, qq, sl, att_block, att_slot, counts, T, D, sc, part_m, part_l, part_acc); break;
        case 8: launch_mfma_g<8>(P, grid, st, qq, sl, att_block, att_slot, counts, T, D, sc, part_m, part_l, part_acc); break;
        default: launch_mfma_g<16>(P, grid, st, qq, sl, att_block, att_slot, counts, T, D, sc, part_m, part_l, part_acc); break;
        }
        return hipGetLastError();
    }
    const int epl = (D.d + 63) / 64;
#define OASIS_GENERIC(TT, E)                                                                     \
    hipLaunchKernelGGL((attn_generic_kernel<TT, E>), grid, dim3(64), 0, st, (const TT *)q,       \
                       (const TT *)slots, att_block, att_slot, counts, T, D.Hq, D.Hkv, D.G, D.d, \
                       D.K, D.S, D.bs, P.blocks_per_wave, P.n_splits, sc, part_m, part_l,        \
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

hipError_t launch_combine(const Dims &D, const AttnPlan &P, const float *part_m,
                          const float *part_l, const float *part_acc, float *out,
                          hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3(D.Hq, D.B), dim3(D.d <= 256 ? D.d : 256), 0, st,
                       part_m, part_l, part_acc, out, D.Hq, D.Hkv, D.G, D.d, P.n_splits);
    return hipGetLastError();
}

}  // namespace oasis
