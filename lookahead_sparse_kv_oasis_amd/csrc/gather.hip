// Host -> HBM block gather.
//
// OasisKV explainer page (explanatory diagram, Fig. 7, Fig. 8): the blocks
// selected for this step that are missing from the GPU working set are
// transferred from the CPU full KV cache in the background, within the
// per-step cap.  Here the copy is a kernel that reads the pinned, mapped host
// KV over the host link and writes the slot in HBM: the fetch list it consumes
// is produced on the device by the select kernel, so no host round trip is
// needed, and it runs on its own stream.
//
// A few waves stream the whole list: wave w copies items w, w + W, ... of the
// units x max_n (unit, i) pairs (item i of a unit exists when i < its count),
// in chunks of 8 16-byte loads per lane (8 KB).  A wave keeps two chunks in
// flight: the next chunk's list entries are read (scalar loads) and its host
// loads issued before the current chunk is stored, so neither the list reads
// nor the slot stores leave the host link idle.  Host reads by shader loads
// run best with about 64 waves in flight (about 55 GB/s alone); one workgroup
// per block (thousands of waves) lowers the link rate and takes CU slots from
// the kernels running beside the copy.  A variant reading the list entries of
// 64 items at once (one per lane) and keeping the next block's loads in
// flight without branches copied no faster alone and made the 36-layer
// lookahead step slower (10.5 -> 11.8 ms): its copies pressed harder on the
// HBM-bound kernels running beside them.
//
// Only the tokens the sequences hold when the list is copied (T) are copied:
// rows at or past T of the last, partial block stay as they are in the slot.
// An append running beside the copy (on another stream) writes token T into
// the host KV and, the block being resident by then, into its slot; the two
// never touch the same bytes, so the append need not wait for the copy.
#include "kernels.h"

namespace oasis {

namespace {

constexpr int kChunk = 64 * 8;  // 16-byte vectors per wave chunk

struct GatherCursor {
    const u32x4 *src;
    u32x4 *dst;
    int64_t item;
    int c0;
    int valid_vec;  // vectors of the K (and of the V) half that hold tokens < T
};

// Vector c of a block (K half, then V half of block_vec / 2 vectors each) is
// copied when it lies in a row of a token < T.
__device__ __forceinline__ bool vec_copied(int c, const GatherCursor &g, int block_vec) {
    const int half = block_vec >> 1;
    const int cc = c >= half ? c - half : c;
    return c < block_vec && cc < g.valid_vec;
}

__device__ __forceinline__ void load_chunk(u32x4 (&r)[8], const GatherCursor &g, int block_vec,
                                           int lane) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int c = g.c0 + k * 64 + lane;
        if (vec_copied(c, g, block_vec)) r[k] = __builtin_nontemporal_load(g.src + c);
    }
}

__device__ __forceinline__ void store_chunk(const u32x4 (&r)[8], const GatherCursor &g,
                                            int block_vec, int lane) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int c = g.c0 + k * 64 + lane;
        if (vec_copied(c, g, block_vec)) g.dst[c] = r[k];
    }
}

}  // namespace

__global__ __launch_bounds__(256) void gather_kernel(const u32x4 *__restrict__ host_kv,
                                                     u32x4 *__restrict__ slots,
                                                     const int32_t *__restrict__ blocks,
                                                     const int32_t *__restrict__ slot_ids,
                                                     int list_stride,
                                                     const int32_t *__restrict__ counts,
                                                     int count_stride, int count_index,
                                                     int64_t NBmax, int S, int block_vec,
                                                     int max_n, int64_t units, int64_t T,
                                                     int bs) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t W = (int64_t)gridDim.x * 4;
    const int64_t n_items = units * max_n;
    // The first existing item at or after `item` (stride W): fills g and
    // returns true, or returns false when the list is exhausted.
    auto seek = [&](int64_t item, GatherCursor &g) -> bool {
        for (; item < n_items; item += W) {
            const int64_t u = item / max_n;
            const int i = (int)(item % max_n);
            const int n = __builtin_amdgcn_readfirstlane(counts[u * count_stride + count_index]);
            if (i >= n) continue;
            const int32_t blk = __builtin_amdgcn_readfirstlane(blocks[u * list_stride + i]);
            const int32_t s = __builtin_amdgcn_readfirstlane(slot_ids[u * list_stride + i]);
            g.src = host_kv + (u * NBmax + blk) * (int64_t)block_vec;
            g.dst = slots + (u * S + s) * (int64_t)block_vec;
            g.item = item;
            g.c0 = 0;
            const int64_t rows = T - (int64_t)blk * bs;
            g.valid_vec = (int)(rows < bs ? rows : bs) * (block_vec / (2 * bs));
            return true;
        }
        return false;
    };
    // The chunk after g: the next chunk of the same block, else the next item.
    auto advance = [&](const GatherCursor &g, GatherCursor &nx) -> bool {
        if (g.c0 + kChunk < block_vec) {
            nx = g;
            nx.c0 = g.c0 + kChunk;
            return true;
        }
        return seek(g.item + W, nx);
    };
    GatherCursor cur, nx;
    if (!seek((int64_t)blockIdx.x * 4 + wave, cur)) return;
    u32x4 ra[8], rb[8];
    load_chunk(ra, cur, block_vec, lane);
    // two register buffers in turn, so a chunk in flight is never copied
    for (;;) {
        bool more = advance(cur, nx);
        if (more) load_chunk(rb, nx, block_vec, lane);
        __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads go out first
        store_chunk(ra, cur, block_vec, lane);
        if (!more) break;
        cur = nx;
        more = advance(cur, nx);
        if (more) load_chunk(ra, nx, block_vec, lane);
        __builtin_amdgcn_sched_barrier(0);
        store_chunk(rb, cur, block_vec, lane);
        if (!more) break;
        cur = nx;
    }
}

hipError_t launch_gather(const Dims &D, const void *host_kv, void *slots, const int32_t *blocks,
                         const int32_t *slot_ids, int list_stride, const int32_t *counts,
                         int count_stride, int count_index, int max_n, int64_t T,
                         hipStream_t st) {
    if (max_n <= 0) return hipSuccess;
    const int block_vec = (int)(D.block_elems() * D.esize() / 16);
    const int64_t items = D.units() * max_n;
    int64_t waves = items < 64 ? items : 64;
    if (waves < 4) waves = 4;
    const dim3 grid((unsigned)((waves + 3) / 4));
    OASIS_LAUNCH(gather_kernel, grid, dim3(256), 0, st, (const u32x4 *)host_kv, (u32x4 *)slots,
                 blocks, slot_ids, list_stride, counts, count_stride, count_index, D.NBmax, D.S,
                 block_vec, max_n, D.units(), T, D.bs);
    return hipGetLastError();
}

}  // namespace oasis
