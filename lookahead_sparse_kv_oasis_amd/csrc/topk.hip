// Per-(b, KV head) top-K of the block scores under the token budget.
//
// OasisKV explainer page (explanatory diagram, Fig. 7): predict the K blocks
// of the next step from the scores; K = budget_tokens / block_size.  Order:
// higher score first, equal scores by lower block id; -0 equals +0.
//
// One workgroup per unit.  Scores become order-preserving 32-bit keys held in
// registers (each thread owns a contiguous id range).  The K'-th largest key
// (K' = min(K, NB)) is found bit by bit from the top with block-wide counts,
// stopping as soon as exactly K' keys reach the candidate.  Equal keys at the
// threshold are taken in id order through a block scan, which makes the
// choice among ties deterministic.  The K' winners are then placed by rank
// counting, which is an exact sort for distinct (key, id) pairs.
#include "kernels.h"

namespace oasis {

constexpr int kTopkMaxK = 1024;

__device__ __forceinline__ uint32_t order_key(float f, bool &bad) {
    uint32_t b = __float_as_uint(f);
    if (!isfinite(f)) {
        bad = true;
        return 0u;
    }
    if (b == 0x80000000u) b = 0u;  // -0 == +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int NT>
__device__ __forceinline__ int block_sum(int v, int *red) {
    constexpr int NW = NT / 64;
    v = wave_sum_i(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w];
    return s;
}

template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += sh[w];
    return base + x - v;
}

template <int NT, int CMAX>
__global__ __launch_bounds__(NT) void topk_kernel(const float *__restrict__ scores, int64_t NBmax,
                                                  int NB, int K, int32_t *__restrict__ ids,
                                                  int32_t *__restrict__ ids_copy,
                                                  uint32_t *__restrict__ err) {
    constexpr int NW = NT / 64;
    __shared__ int red[34][NW];
    __shared__ int scan_sh[NW];
    __shared__ uint32_t ckey[kTopkMaxK];
    __shared__ int32_t cid[kTopkMaxK];
    __shared__ int ccount;

    const int64_t u = blockIdx.x;
    const float *s = scores + u * NBmax;
    int32_t *out = ids + u * K;
    int32_t *out2 = ids_copy ? ids_copy + u * K : nullptr;
    const int tid = threadIdx.x;
    const int Kp = K < NB ? K : NB;
    if (tid == 0) ccount = 0;

    const int C = (NB + NT - 1) / NT;
    const int begin = tid * C;
    uint32_t key[CMAX];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
        const int id = begin + i;
        key[i] = (i < C && id < NB) ? order_key(s[id], bad) : 0u;
    }
    if (bad) atomicOr(err, kErrNonFinite);

    // largest tau with #{key >= tau} >= Kp, built from the top bit down
    uint32_t tau = 0;
    bool exact = false;
    int pass = 0;
    for (int bit = 31; bit >= 0 && Kp > 0; --bit, ++pass) {
        const uint32_t cand = tau | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) cnt += key[i] >= cand ? 1 : 0;
        cnt = block_sum<NT>(cnt, red[pass]);
        if (cnt >= Kp) {
            tau = cand;
            if (cnt == Kp) {
                exact = true;
                break;
            }
        }
    }

    int take_eq = 0, eq_before = 0;
    if (!exact && Kp > 0) {
        int gt = 0, eq = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            const bool valid = i < C && id < NB;
            gt += (valid && key[i] > tau) ? 1 : 0;
            eq += (valid && key[i] == tau) ? 1 : 0;
        }
        gt = block_sum<NT>(gt, red[32]);
        take_eq = Kp - gt;
        eq_before = block_excl_scan<NT>(eq, scan_sh);
    }
    __syncthreads();  // ccount initialised

    int eq_seen = 0;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
        const int id = begin + i;
        if (i < C && id < NB && Kp > 0) {
            bool take;
            if (exact) {
                take = key[i] >= tau;
            } else {
                take = key[i] > tau;
                if (key[i] == tau) {
                    take = eq_before + eq_seen < take_eq;
                    ++eq_seen;
                }
            }
            if (take) {
                const int p = atomicAdd(&ccount, 1);
                if (p < kTopkMaxK) {
                    ckey[p] = key[i];
                    cid[p] = id;
                }
            }
        }
    }
    __syncthreads();

    for (int i = tid; i < Kp; i += NT) {
        const uint32_t ki = ckey[i];
        const int32_t ii = cid[i];
        int rank = 0;
        for (int j = 0; j < Kp; ++j) {
            const uint32_t kj = ckey[j];
            rank += (kj > ki || (kj == ki && cid[j] < ii)) ? 1 : 0;
        }
        out[rank] = ii;
        if (out2) out2[rank] = ii;
    }
    for (int i = Kp + tid; i < K; i += NT) {
        out[i] = -1;
        if (out2) out2[i] = -1;
    }
}

template <int NT>
static void launch_nt(int C, dim3 grid, hipStream_t st, const float *scores, int64_t NBmax,
                      int NB, int K, int32_t *ids, int32_t *ids_copy, uint32_t *err) {
    if (C <= 4)
        hipLaunchKernelGGL((topk_kernel<NT, 4>), grid, dim3(NT), 0, st, scores, NBmax, NB, K,
                           ids, ids_copy, err);
    else if (C <= 8)
        hipLaunchKernelGGL((topk_kernel<NT, 8>), grid, dim3(NT), 0, st, scores, NBmax, NB, K,
                           ids, ids_copy, err);
    else if (C <= 16)
        hipLaunchKernelGGL((topk_kernel<NT, 16>), grid, dim3(NT), 0, st, scores, NBmax, NB, K,
                           ids, ids_copy, err);
    else if (C <= 32)
        hipLaunchKernelGGL((topk_kernel<NT, 32>), grid, dim3(NT), 0, st, scores, NBmax, NB, K,
                           ids, ids_copy, err);
    else
        hipLaunchKernelGGL((topk_kernel<NT, 64>), grid, dim3(NT), 0, st, scores, NBmax, NB, K,
                           ids, ids_copy, err);
}

hipError_t launch_topk(const Dims &D, const float *scores, int64_t NB, int32_t *ids,
                       int32_t *ids_copy, uint32_t *err, hipStream_t st) {
    dim3 grid((unsigned)D.units());
    if (NB <= 256 * 64) {
        const int C = (int)((NB + 255) / 256);
        launch_nt<256>(C, grid, st, scores, D.NBmax, (int)NB, D.K, ids, ids_copy, err);
    } else {
        const int C = (int)((NB + 1023) / 1024);
        launch_nt<1024>(C, grid, st, scores, D.NBmax, (int)NB, D.K, ids, ids_copy, err);
    }
    return hipGetLastError();
}

}  // namespace oasis
