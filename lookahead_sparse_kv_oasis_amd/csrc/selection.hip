// Per-(b, KV head) selection: top-K of the block scores, then the residency
// diff with a capped fetch and LRU slot assignment.
//
// Top-K -- OasisKV explainer page (explanatory diagram, Fig. 7): predict the
// K blocks of the next step from the scores; K = budget_tokens / block_size.
// Order: higher score first, equal scores by lower block id; -0 equals +0.
// One workgroup per unit.  Scores become order-preserving 32-bit keys held in
// registers (each thread owns a contiguous id range).  The K'-th largest key
// (K' = min(K, NB)) is built bit by bit below the common prefix of the
// largest and smallest key with block-wide counts, stopping as soon as
// exactly K' keys reach the candidate.  Equal keys at the threshold are taken
// in id order through a block scan, which makes the choice among ties
// deterministic.  The K' winners are placed by rank counting, an exact sort
// for distinct (key, id) pairs.
//
// Select -- the explanatory diagram compares the predicted blocks with the
// blocks already on the GPU and transfers only the missing ones, capping the
// per-step transfer; the capped-eviction glossary entry bounds the blocks
// newly loaded in one step; Table 2 sets that cap by a fetch ratio and evicts
// LRU; Fig. 9 keeps, per KV head, a table from each GPU block (slot) to its
// CPU block.  Integer work only, per unit:
//   hits   = selected blocks held by a slot, in top-K order;
//   misses = selected blocks not held, in top-K order; the first
//            n = min(cap, |misses|) are fetched;
//   slots  = empty slots in ascending index, then slots of held blocks that
//            are not selected, least recently used first, ties to the lower
//            block id;
//   every hit and every fetched block gets last_used = t.
// The attended list is the hits followed by the fetched blocks.  One wave
// does it: ordered compactions use ballots; victims are ranked by counting
// smaller (last_used, block) keys, exact because held block ids are distinct.
//
// The fused kernel runs both for a unit in one workgroup: the slot tables are
// copied into LDS while the top-K runs, and the winners go straight from LDS
// into the select.
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

// Top-K of one unit's scores s[0..NB) into out[0..K) (and out2, out_lds when
// not null), -1 padded.  Called by every thread of an NT-thread workgroup.
template <int NT, int CMAX>
__device__ void topk_unit(const float *__restrict__ s, int NB, int K, int32_t *__restrict__ out,
                          int32_t *__restrict__ out2, int32_t *out_lds,
                          uint32_t *__restrict__ err) {
    constexpr int NW = NT / 64;
    __shared__ uint32_t red[2][NW];
    __shared__ uint32_t red_mx[NW], red_mn[NW];
    __shared__ int scan_a[NW], scan_b[NW];
    __shared__ int gt_total;
    __shared__ uint32_t ckey[kTopkMaxK];
    __shared__ int32_t cid[kTopkMaxK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Kp = K < NB ? K : NB;
    if (Kp <= 0) {
        for (int i = tid; i < K; i += NT) {
            out[i] = -1;
            if (out2) out2[i] = -1;
            if (out_lds) out_lds[i] = -1;
        }
        return;
    }

    const int C = (NB + NT - 1) / NT;
    const int begin = tid * C;
    uint32_t key[CMAX];
    bool bad = false;
    uint32_t lmx = 0u, lmn = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
        const int id = begin + i;
        const bool valid = i < C && id < NB;
        key[i] = valid ? order_key(s[id], bad) : 0u;
        if (valid) {
            lmx = key[i] > lmx ? key[i] : lmx;
            lmn = key[i] < lmn ? key[i] : lmn;
        }
    }
    if (bad) atomicOr(err, kErrNonFinite);
    lmx = wave_max_u32(lmx);
    lmn = wave_min_u32(lmn);
    if (lane == 0) {
        red_mx[wave] = lmx;
        red_mn[wave] = lmn;
    }
    __syncthreads();
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        kmax = red_mx[w] > kmax ? red_mx[w] : kmax;
        kmin = red_mn[w] < kmin ? red_mn[w] : kmin;
    }

    // Every key lies in [kmin, kmax] and so shares their common high bits; the
    // K'-th largest key tau is built below that prefix, one bit at a time,
    // keeping #{key >= tau} >= K'.  Stop as soon as exactly K' keys qualify.
    const uint32_t diff = kmax ^ kmin;
    const int top = diff ? 31 - __builtin_clz(diff) : -1;
    uint32_t tau = top < 0 ? kmax : (top == 31 ? 0u : (kmax & ~((2u << top) - 1u)));
    bool exact = false;
    int pass = 0;
    for (int bit = top; bit >= 0; --bit, ++pass) {
        const uint32_t cand = tau | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) cnt += key[i] >= cand ? 1u : 0u;
        cnt = wave_add_u32(cnt);
        if (lane == 0) red[pass & 1][wave] = cnt;
        __syncthreads();
        cnt = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) cnt += red[pass & 1][w];
        if ((int)cnt >= Kp) {
            tau = cand;
            if ((int)cnt == Kp) {
                exact = true;
                break;
            }
        }
    }

    // Taken: keys above tau, plus the lowest-id keys equal to tau up to K'.
    int take_eq = 0, eq_before = 0;
    if (!exact) {
        int gt = 0, eq = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            const bool valid = i < C && id < NB;
            gt += (valid && key[i] > tau) ? 1 : 0;
            eq += (valid && key[i] == tau) ? 1 : 0;
        }
        eq_before = block_excl_scan<NT>(eq, scan_a);
        const int gt_before = block_excl_scan<NT>(gt, scan_b);
        // total of gt: last thread's exclusive prefix plus its own count
        if (tid == NT - 1) gt_total = gt_before + gt;
        __syncthreads();
        take_eq = Kp - gt_total;
    }
    int take_local = 0;
    {
        int eq_seen = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            if (i < C && id < NB) {
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
                take_local += take ? 1 : 0;
            }
        }
    }
    __syncthreads();  // scan_a is reused below
    int pos = block_excl_scan<NT>(take_local, scan_a);
    {
        int eq_seen = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            if (i < C && id < NB) {
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
                if (take && pos < kTopkMaxK) {
                    ckey[pos] = key[i];
                    cid[pos] = id;
                    ++pos;
                }
            }
        }
    }
    __syncthreads();

    // place each winner by counting the winners that order before it
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
        if (out_lds) out_lds[rank] = ii;
    }
    for (int i = Kp + tid; i < K; i += NT) {
        out[i] = -1;
        if (out2) out2[i] = -1;
        if (out_lds) out_lds[i] = -1;
    }
}

template <int NT, int CMAX>
__global__ __launch_bounds__(NT) void topk_kernel(const float *__restrict__ scores, int64_t NBmax,
                                                  int NB, int K, int32_t *__restrict__ ids,
                                                  int32_t *__restrict__ ids_copy,
                                                  uint32_t *__restrict__ err) {
    const int64_t u = blockIdx.x;
    topk_unit<NT, CMAX>(scores + u * NBmax, NB, K, ids + u * K, ids_copy ? ids_copy + u * K : nullptr,
                        nullptr, err);
}

// LDS ordering between lanes of one wave.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

// Bytes of LDS scratch select_unit needs.
__host__ __device__ constexpr size_t select_lds_bytes(int K, int S) {
    return sizeof(int32_t) * (3 * (size_t)K + 2 * (size_t)S + 2) +
           sizeof(unsigned long long) * ((size_t)S + 1);
}

// Diff / cap / LRU of unit u, run by the 64 lanes of one wave.  sel: the K
// selected ids (global or LDS); sb_in / lu_in: the slot tables to read (the
// global tables, or LDS copies of them); the global tables slot_block /
// last_used / block_slot (rows of unit u) are written.  sh: LDS scratch of
// select_lds_bytes(K, S).
__device__ void select_unit(int64_t u, const int32_t *sel, const int32_t *sb_in,
                            const int32_t *lu_in, int32_t *__restrict__ slot_block,
                            int32_t *__restrict__ last_used, int32_t *__restrict__ block_slot,
                            int K, int S, int64_t NBmax, int cap, int32_t t,
                            int32_t *__restrict__ fetch_block, int32_t *__restrict__ fetch_slot,
                            int32_t *__restrict__ att_block, int32_t *__restrict__ att_slot,
                            int32_t *__restrict__ counts, DevStats *stats, uint32_t *err,
                            int32_t *sh) {
    int32_t *hit_blk = sh;             // [K]
    int32_t *hit_slot = hit_blk + K;   // [K]
    int32_t *miss_blk = hit_slot + K;  // [K]
    int32_t *cand = miss_blk + K;      // [S] slots to fill, in order
    int32_t *selected = cand + S;      // [S] slot holds a selected block
    unsigned long long *vkey = reinterpret_cast<unsigned long long *>(selected + S + (K & 1));  // 8-byte aligned

    const int lane = threadIdx.x & 63;
    int32_t *sb = slot_block + u * S;
    int32_t *lu = last_used + u * S;
    int32_t *bs = block_slot + u * NBmax;

    for (int s = lane; s < S; s += 64) selected[s] = 0;
    wave_sync();

    // hits and misses, in top-K order
    int nh = 0, nm = 0;
    for (int base = 0; base < K; base += 64) {
        const int i = base + lane;
        const int32_t id = i < K ? sel[i] : -1;
        const int32_t s = id >= 0 ? bs[id] : -1;
        const bool hit = id >= 0 && s >= 0;
        const bool miss = id >= 0 && s < 0;
        const unsigned long long hb = __ballot(hit), mb = __ballot(miss);
        if (hit) {
            const int p = nh + lanes_below(hb);
            hit_blk[p] = id;
            hit_slot[p] = s;
            selected[s] = 1;
        }
        if (miss) miss_blk[nm + lanes_below(mb)] = id;
        nh += __popcll(hb);
        nm += __popcll(mb);
    }
    wave_sync();
    const int n = nm < cap ? nm : cap;

    // empty slots first, ascending; then LRU victims among held, non-selected
    int nfree = 0;
    for (int base = 0; base < S; base += 64) {
        const int s = base + lane;
        const bool fr = s < S && sb_in[s] < 0;
        const unsigned long long fb = __ballot(fr);
        if (fr) cand[nfree + lanes_below(fb)] = s;
        nfree += __popcll(fb);
    }
    for (int s = lane; s < S; s += 64) {
        const int32_t blk = sb_in[s];
        vkey[s] = (blk >= 0 && !selected[s])
                      ? ((unsigned long long)((uint32_t)lu_in[s] ^ 0x80000000u) << 32) |
                            (uint32_t)blk
                      : ~0ull;
    }
    wave_sync();
    const int need = n - nfree;
    if (need > 0) {
        for (int s = lane; s < S; s += 64) {
            const unsigned long long k = vkey[s];
            if (k == ~0ull) continue;
            int rank = 0;
            for (int r = 0; r < S; ++r) rank += vkey[r] < k ? 1 : 0;
            if (rank < need) cand[nfree + rank] = s;
        }
    }
    wave_sync();
    int nvict = 0;
    for (int s = lane; s < S; s += 64) nvict += vkey[s] != ~0ull ? 1 : 0;
    nvict = wave_sum_i(nvict);
    if (nfree + nvict < n) {  // cannot happen with S >= K
        if (lane == 0) atomicOr(err, kErrSlots);
        return;
    }

    // apply: evict, fill, refresh recency, emit lists
    int32_t *fb = fetch_block + u * K, *fs = fetch_slot + u * K;
    int32_t *ab = att_block + u * K, *as = att_slot + u * K;
    for (int i = lane; i < n; i += 64) {
        const int s = cand[i];
        const int32_t old = sb_in[s];
        if (old >= 0) bs[old] = -1;
    }
    wave_sync();
    for (int i = lane; i < n; i += 64) {
        const int s = cand[i];
        const int32_t blk = miss_blk[i];
        sb[s] = blk;
        bs[blk] = s;
        lu[s] = t;
        fb[i] = blk;
        fs[i] = s;
        ab[nh + i] = blk;
        as[nh + i] = s;
    }
    for (int i = lane; i < nh; i += 64) {
        lu[hit_slot[i]] = t;
        ab[i] = hit_blk[i];
        as[i] = hit_slot[i];
    }
    if (lane == 0) {
        counts[u * 4 + 0] = nh + n;
        counts[u * 4 + 1] = nh;
        counts[u * 4 + 2] = n;
        counts[u * 4 + 3] = nm;
        atomicAdd(&stats->hits, (unsigned long long)nh);
        atomicAdd(&stats->misses, (unsigned long long)nm);
        atomicAdd(&stats->fetched, (unsigned long long)n);
        atomicAdd(&stats->attended, (unsigned long long)(nh + n));
    }
}

__global__ __launch_bounds__(64) void select_kernel(
    const int32_t *__restrict__ ids, int32_t *__restrict__ slot_block,
    int32_t *__restrict__ last_used, int32_t *__restrict__ block_slot, int K, int S,
    int64_t NBmax, int cap, int32_t t, int32_t *__restrict__ fetch_block,
    int32_t *__restrict__ fetch_slot, int32_t *__restrict__ att_block,
    int32_t *__restrict__ att_slot, int32_t *__restrict__ counts, DevStats *stats,
    uint32_t *err) {
    extern __shared__ __attribute__((aligned(16))) int32_t sh[];
    const int64_t u = blockIdx.x;
    select_unit(u, ids + u * K, slot_block + u * S, last_used + u * S, slot_block, last_used,
                block_slot, K, S, NBmax, cap, t, fetch_block, fetch_slot, att_block, att_slot,
                counts, stats, err, sh);
}

// Top-K and select of one unit in one workgroup.
template <int NT, int CMAX>
__global__ __launch_bounds__(NT) void topk_select_kernel(
    const float *__restrict__ scores, int NB, int32_t *__restrict__ ids,
    int32_t *__restrict__ slot_block, int32_t *__restrict__ last_used,
    int32_t *__restrict__ block_slot, int K, int S, int64_t NBmax, int cap, int32_t t,
    int32_t *__restrict__ fetch_block, int32_t *__restrict__ fetch_slot,
    int32_t *__restrict__ att_block, int32_t *__restrict__ att_slot,
    int32_t *__restrict__ counts, DevStats *stats, uint32_t *err) {
    extern __shared__ __attribute__((aligned(16))) int32_t sh[];
    const int64_t u = blockIdx.x;
    int32_t *sel_lds = sh;                 // [K]
    int32_t *sb_lds = sel_lds + K;         // [S]
    int32_t *lu_lds = sb_lds + S;          // [S]
    int32_t *scratch = lu_lds + S + ((K + 2 * S) & 1);  // 8-byte aligned
    for (int s = threadIdx.x; s < S; s += NT) {
        sb_lds[s] = slot_block[u * S + s];
        lu_lds[s] = last_used[u * S + s];
    }
    topk_unit<NT, CMAX>(scores + u * NBmax, NB, K, ids + u * K, nullptr, sel_lds, err);
    __syncthreads();
    if (threadIdx.x < 64)
        select_unit(u, sel_lds, sb_lds, lu_lds, slot_block, last_used, block_slot, K, S, NBmax,
                    cap, t, fetch_block, fetch_slot, att_block, att_slot, counts, stats, err,
                    scratch);
}

__global__ __launch_bounds__(64) void evict_kernel(const int32_t *__restrict__ blocks,
                                                   const int32_t *__restrict__ counts,
                                                   int max_per_unit, int32_t *slot_block,
                                                   int32_t *block_slot, int S, int64_t NBmax) {
    const int64_t u = blockIdx.x;
    const int n = counts[u];
    for (int i = threadIdx.x; i < n && i < max_per_unit; i += 64) {
        const int32_t blk = blocks[u * max_per_unit + i];
        if (blk < 0 || blk >= NBmax) continue;
        const int32_t s = block_slot[u * NBmax + blk];
        if (s < 0) continue;
        slot_block[u * S + s] = -1;
        block_slot[u * NBmax + blk] = -1;
    }
}

__global__ __launch_bounds__(256) void rebuild_block_slot_kernel(
    const int32_t *__restrict__ slot_block, int32_t *__restrict__ block_slot, int S,
    int64_t NBmax) {
    const int64_t u = blockIdx.y;
    for (int64_t j = blockIdx.x * 256LL + threadIdx.x; j < NBmax; j += gridDim.x * 256LL)
        block_slot[u * NBmax + j] = -1;
    __syncthreads();
    if (blockIdx.x == 0)
        for (int s = threadIdx.x; s < S; s += 256) {
            const int32_t blk = slot_block[u * S + s];
            if (blk >= 0) block_slot[u * NBmax + blk] = s;
        }
}

#define OASIS_CMAX_DISPATCH(NT, C, LAUNCH)          \
    do {                                             \
        if ((C) <= 4) LAUNCH(NT, 4);                 \
        else if ((C) <= 8) LAUNCH(NT, 8);            \
        else if ((C) <= 16) LAUNCH(NT, 16);          \
        else if ((C) <= 32) LAUNCH(NT, 32);          \
        else LAUNCH(NT, 64);                         \
    } while (0)

hipError_t launch_topk(const Dims &D, const float *scores, int64_t NB, int32_t *ids,
                       int32_t *ids_copy, uint32_t *err, hipStream_t st) {
    dim3 grid((unsigned)D.units());
#define OASIS_TOPK(NT_, CM_)                                                                    \
    hipLaunchKernelGGL((topk_kernel<NT_, CM_>), grid, dim3(NT_), 0, st, scores, D.NBmax,      \
                       (int)NB, D.K, ids, ids_copy, err)
    if (NB <= 256 * 64) {
        OASIS_CMAX_DISPATCH(256, (NB + 255) / 256, OASIS_TOPK);
    } else {
        OASIS_CMAX_DISPATCH(1024, (NB + 1023) / 1024, OASIS_TOPK);
    }
#undef OASIS_TOPK
    return hipGetLastError();
}

hipError_t launch_select(const Dims &D, const int32_t *ids, int32_t *slot_block,
                         int32_t *last_used, int32_t *block_slot, int cap, int32_t t,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *att_block,
                         int32_t *att_slot, int32_t *counts, DevStats *stats, uint32_t *err,
                         hipStream_t st) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)D.units()), dim3(64),
                       select_lds_bytes(D.K, D.S), st, ids, slot_block, last_used, block_slot,
                       D.K, D.S, D.NBmax, cap, t, fetch_block, fetch_slot, att_block, att_slot,
                       counts, stats, err);
    return hipGetLastError();
}

hipError_t launch_topk_select(const Dims &D, const float *scores, int64_t NB, int32_t *ids,
                              int32_t *slot_block, int32_t *last_used, int32_t *block_slot,
                              int cap, int32_t t, int32_t *fetch_block, int32_t *fetch_slot,
                              int32_t *att_block, int32_t *att_slot, int32_t *counts,
                              DevStats *stats, uint32_t *err, hipStream_t st) {
    dim3 grid((unsigned)D.units());
    const size_t lds = sizeof(int32_t) * ((size_t)D.K + 2 * (size_t)D.S + 1) +
                       select_lds_bytes(D.K, D.S);
#define OASIS_TS(NT_, CM_)                                                                      \
    hipLaunchKernelGGL((topk_select_kernel<NT_, CM_>), grid, dim3(NT_), lds, st, scores,      \
                       (int)NB, ids, slot_block, last_used, block_slot, D.K, D.S, D.NBmax, cap, \
                       t, fetch_block, fetch_slot, att_block, att_slot, counts, stats, err)
    if (NB <= 256 * 64) {
        OASIS_CMAX_DISPATCH(256, (NB + 255) / 256, OASIS_TS);
    } else {
        OASIS_CMAX_DISPATCH(1024, (NB + 1023) / 1024, OASIS_TS);
    }
#undef OASIS_TS
    return hipGetLastError();
}

hipError_t launch_evict(const Dims &D, const int32_t *blocks, const int32_t *counts,
                        int max_per_unit, int32_t *slot_block, int32_t *block_slot,
                        hipStream_t st) {
    hipLaunchKernelGGL(evict_kernel, dim3((unsigned)D.units()), dim3(64), 0, st, blocks, counts,
                       max_per_unit, slot_block, block_slot, D.S, D.NBmax);
    return hipGetLastError();
}

hipError_t launch_rebuild_block_slot(const Dims &D, const int32_t *slot_block,
                                     int32_t *block_slot, hipStream_t st) {
    // one workgroup per unit so the clear is ordered before the fill
    hipLaunchKernelGGL(rebuild_block_slot_kernel, dim3(1, (unsigned)D.units()), dim3(256), 0, st,
                       slot_block, block_slot, D.S, D.NBmax);
    return hipGetLastError();
}

}  // namespace oasis
