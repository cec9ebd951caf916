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
// units x max_n (unit, i) pairs (item i of a unit exists when i < its count).
// A wave reads the list entries of up to 64 of its items at once, one per
// lane.  8 KB blocks (8 16-byte loads per lane) are then copied with the next
// block's host loads issued before the current one is stored; those loads go
// out unconditionally (after the last block, a discarded read of slot 0) and
// the loop's one branch is its exit after the stores: with a load under a
// branch, or a list entry read between blocks, the compiler's wait before each
// store covered the block in flight as well, and the copy ran one block per
// host round trip.  Blocks of any other size are copied one at a time.  Host
// reads by shader loads run best with about 64 waves in flight (about
// 55 GB/s alone); one workgroup per block (thousands of waves) lowers the
// link rate and takes CU slots from the kernels running beside the copy.
#include "kernels.h"

namespace oasis {

// Lane l's 64-bit value, read by the whole wave.
__device__ __forceinline__ int64_t lane_i64(int64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(256) void gather_kernel(const u32x4 *__restrict__ host_kv,
                                                     u32x4 *__restrict__ slots,
                                                     const int32_t *__restrict__ blocks,
                                                     const int32_t *__restrict__ slot_ids,
                                                     int list_stride,
                                                     const int32_t *__restrict__ counts,
                                                     int count_stride, int count_index,
                                                     int64_t NBmax, int S, int block_vec,
                                                     int max_n, int64_t units) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t W = (int64_t)gridDim.x * 4;
    const int64_t n_items = units * max_n;
    const int64_t it0 = (int64_t)blockIdx.x * 4 + wave;
    if (it0 >= n_items) return;
    const int64_t n_my = (n_items - it0 + W - 1) / W;  // this wave's items
    for (int64_t c0 = 0; c0 < n_my; c0 += 64) {
        // lane l: item it0 + (c0 + l) W, its source and destination blocks
        const int64_t item = it0 + (c0 + lane) * W;
        bool ok = false;
        int64_t src = 0, dst = 0;
        if (c0 + lane < n_my) {
            const int64_t u = item / max_n;
            const int i = (int)(item % max_n);
            if (i < counts[u * count_stride + count_index]) {
                src = (u * NBmax + blocks[u * list_stride + i]) * (int64_t)block_vec;
                dst = (u * S + slot_ids[u * list_stride + i]) * (int64_t)block_vec;
                ok = true;
            }
        }
        const uint64_t mask = __ballot(ok);
        if (mask == 0) continue;
        if (block_vec == 512) {
            // 8 KB blocks (16 tokens x 128 dims of bf16 K and V): the
            // pipelined copy, 8 vectors per lane; the discarded read stays
            // inside slot 0, which is a whole block
            int l_cur = __builtin_ctzll(mask);
            uint64_t rest = mask & (mask - 1);  // set lanes after the current one
            u32x4 ra[8], rb[8];
            {
                const u32x4 *sp = host_kv + lane_i64(src, l_cur);
#pragma unroll
                for (int k = 0; k < 8; ++k) ra[k] = __builtin_nontemporal_load(sp + k * 64 + lane);
            }
            for (;;) {
                // the current item is in ra; issue the next (or a discarded read)
                bool more = rest != 0;
                int l_nx = __builtin_ctzll(rest | (1ull << 63));
                const u32x4 *sp = more ? host_kv + lane_i64(src, l_nx) : (const u32x4 *)slots;
#pragma unroll
                for (int k = 0; k < 8; ++k) rb[k] = __builtin_nontemporal_load(sp + k * 64 + lane);
                __builtin_amdgcn_sched_barrier(0);  // the next item's loads go out first
                u32x4 *dp = slots + lane_i64(dst, l_cur);
#pragma unroll
                for (int k = 0; k < 8; ++k) dp[k * 64 + lane] = ra[k];
                if (!more) break;
                l_cur = l_nx;
                rest &= rest - 1;
                more = rest != 0;
                l_nx = __builtin_ctzll(rest | (1ull << 63));
                sp = more ? host_kv + lane_i64(src, l_nx) : (const u32x4 *)slots;
#pragma unroll
                for (int k = 0; k < 8; ++k) ra[k] = __builtin_nontemporal_load(sp + k * 64 + lane);
                __builtin_amdgcn_sched_barrier(0);
                dp = slots + lane_i64(dst, l_cur);
#pragma unroll
                for (int k = 0; k < 8; ++k) dp[k * 64 + lane] = rb[k];
                if (!more) break;
                l_cur = l_nx;
                rest &= rest - 1;
            }
        } else {
            // other block sizes: one block at a time, every vector guarded
            for (uint64_t m = mask; m; m &= m - 1) {
                const int l = __builtin_ctzll(m);
                const u32x4 *sp = host_kv + lane_i64(src, l);
                u32x4 *dp = slots + lane_i64(dst, l);
                for (int c = lane; c < block_vec; c += 64) dp[c] = __builtin_nontemporal_load(sp + c);
            }
        }
    }
}

hipError_t launch_gather(const Dims &D, const void *host_kv, void *slots, const int32_t *blocks,
                         const int32_t *slot_ids, int list_stride, const int32_t *counts,
                         int count_stride, int count_index, int max_n, hipStream_t st) {
    if (max_n <= 0) return hipSuccess;
    const int block_vec = (int)(D.block_elems() * D.esize() / 16);
    const int64_t items = D.units() * max_n;
    int64_t waves = items < 64 ? items : 64;
    if (waves < 4) waves = 4;
    const dim3 grid((unsigned)((waves + 3) / 4));
    OASIS_LAUNCH(gather_kernel, grid, dim3(256), 0, st, (const u32x4 *)host_kv, (u32x4 *)slots,
                 blocks, slot_ids, list_stride, counts, count_stride, count_index, D.NBmax, D.S,
                 block_vec, max_n, D.units());
    return hipGetLastError();
}

}  // namespace oasis
