// Residency diff, capped fetch and LRU slot assignment.
//
// OasisKV explainer page: the explanatory diagram compares the predicted
// blocks with the blocks already on the GPU and transfers only the missing
// ones, capping the per-step transfer; the capped-eviction glossary entry
// bounds the number of blocks newly loaded in one step; Table 2 sets that cap
// by a fetch ratio and evicts LRU; Fig. 9 keeps, per KV head, a table from
// each GPU block (slot) to its CPU block.
//
// Per (b, KV head), integer work only:
//   hits   = selected blocks held by a slot, in top-K order;
//   misses = selected blocks not held, in top-K order; the first
//            n = min(cap, |misses|) are fetched;
//   slots  = empty slots in ascending index, then slots of held blocks that
//            are not selected, least recently used first, ties to the lower
//            block id;
//   every hit and every fetched block gets last_used = t.
// The attended list is the hits followed by the fetched blocks.
//
// One wave per unit: ordered compactions use ballots; victims are ranked by
// counting smaller (last_used, block) keys, which is exact because held block
// ids are distinct.
#include "kernels.h"

namespace oasis {

__global__ __launch_bounds__(64) void select_kernel(
    const int32_t *__restrict__ ids, int32_t *__restrict__ slot_block,
    int32_t *__restrict__ last_used, int32_t *__restrict__ block_slot, int K, int S,
    int64_t NBmax, int cap, int32_t t, int32_t *__restrict__ fetch_block,
    int32_t *__restrict__ fetch_slot, int32_t *__restrict__ att_block,
    int32_t *__restrict__ att_slot, int32_t *__restrict__ counts, DevStats *stats,
    uint32_t *err) {
    extern __shared__ __attribute__((aligned(16))) int32_t sh[];
    int32_t *hit_blk = sh;             // [K]
    int32_t *hit_slot = hit_blk + K;   // [K]
    int32_t *miss_blk = hit_slot + K;  // [K]
    int32_t *cand = miss_blk + K;      // [S] slots to fill, in order
    int32_t *selected = cand + S;      // [S] slot holds a selected block
    unsigned long long *vkey = reinterpret_cast<unsigned long long *>(selected + S + (K & 1));  // 8-byte aligned

    const int64_t u = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t *sel = ids + u * K;
    int32_t *sb = slot_block + u * S;
    int32_t *lu = last_used + u * S;
    int32_t *bs = block_slot + u * NBmax;

    for (int s = lane; s < S; s += 64) selected[s] = 0;
    __syncthreads();

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
    __syncthreads();
    const int n = nm < cap ? nm : cap;

    // empty slots first, ascending; then LRU victims among held, non-selected
    int nfree = 0;
    for (int base = 0; base < S; base += 64) {
        const int s = base + lane;
        const bool fr = s < S && sb[s] < 0;
        const unsigned long long fb = __ballot(fr);
        if (fr) cand[nfree + lanes_below(fb)] = s;
        nfree += __popcll(fb);
    }
    for (int s = lane; s < S; s += 64) {
        const int32_t blk = sb[s];
        vkey[s] = (blk >= 0 && !selected[s])
                      ? ((unsigned long long)((uint32_t)lu[s] ^ 0x80000000u) << 32) |
                            (uint32_t)blk
                      : ~0ull;
    }
    __syncthreads();
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
    __syncthreads();
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
        const int32_t old = sb[s];
        if (old >= 0) bs[old] = -1;
    }
    __syncthreads();
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

hipError_t launch_select(const Dims &D, const int32_t *ids, int32_t *slot_block,
                         int32_t *last_used, int32_t *block_slot, int cap, int32_t t,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *att_block,
                         int32_t *att_slot, int32_t *counts, DevStats *stats, uint32_t *err,
                         hipStream_t st) {
    const size_t lds = sizeof(int32_t) * (3 * (size_t)D.K + 2 * (size_t)D.S + 1) +
                       sizeof(unsigned long long) * ((size_t)D.S + 1);
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)D.units()), dim3(64), lds, st, ids,
                       slot_block, last_used, block_slot, D.K, D.S, D.NBmax, cap, t,
                       fetch_block, fetch_slot, att_block, att_slot, counts, stats, err);
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
