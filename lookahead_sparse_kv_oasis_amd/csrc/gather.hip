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
// One workgroup per fetched (unit, block); a block (K and V rows of
// block_size tokens) is contiguous in both the host KV and the slot pool.
// Each thread issues all its 16-byte loads before its stores to keep enough
// host-link requests in flight.
#include "kernels.h"

namespace oasis {



template <int PER_THREAD>
__global__ __launch_bounds__(256) void gather_kernel(const u32x4 *__restrict__ host_kv,
                                                     u32x4 *__restrict__ slots,
                                                     const int32_t *__restrict__ blocks,
                                                     const int32_t *__restrict__ slot_ids,
                                                     int list_stride,
                                                     const int32_t *__restrict__ counts,
                                                     int count_stride, int count_index,
                                                     int64_t NBmax, int S, int block_vec) {
    const int i = blockIdx.x;
    const int64_t u = blockIdx.y;
    const int n = counts[u * count_stride + count_index];
    if (i >= n) return;
    const int32_t blk = blocks[u * list_stride + i];
    const int32_t s = slot_ids[u * list_stride + i];
    const u32x4 *src = host_kv + (u * NBmax + blk) * (int64_t)block_vec;
    u32x4 *dst = slots + (u * S + s) * (int64_t)block_vec;
    for (int c0 = 0; c0 < block_vec; c0 += 256 * PER_THREAD) {
        u32x4 r[PER_THREAD];
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int c = c0 + k * 256 + threadIdx.x;
            if (c < block_vec) r[k] = __builtin_nontemporal_load(src + c);
        }
#pragma unroll
        for (int k = 0; k < PER_THREAD; ++k) {
            const int c = c0 + k * 256 + threadIdx.x;
            if (c < block_vec) dst[c] = r[k];
        }
    }
}

hipError_t launch_gather(const Dims &D, const void *host_kv, void *slots, const int32_t *blocks,
                         const int32_t *slot_ids, int list_stride, const int32_t *counts,
                         int count_stride, int count_index, int max_n, hipStream_t st) {
    if (max_n <= 0) return hipSuccess;
    const int block_vec = (int)(D.block_elems() * D.esize() / 16);
    dim3 grid((unsigned)max_n, (unsigned)D.units());
    if (block_vec <= 256)
        OASIS_LAUNCH(gather_kernel<1>, grid, dim3(256), 0, st, (const u32x4 *)host_kv,
                           (u32x4 *)slots, blocks, slot_ids, list_stride, counts, count_stride,
                           count_index, D.NBmax, D.S, block_vec);
    else if (block_vec <= 512)
        OASIS_LAUNCH(gather_kernel<2>, grid, dim3(256), 0, st, (const u32x4 *)host_kv,
                           (u32x4 *)slots, blocks, slot_ids, list_stride, counts, count_stride,
                           count_index, D.NBmax, D.S, block_vec);
    else
        OASIS_LAUNCH(gather_kernel<4>, grid, dim3(256), 0, st, (const u32x4 *)host_kv,
                           (u32x4 *)slots, blocks, slot_ids, list_stride, counts, count_stride,
                           count_index, D.NBmax, D.S, block_vec);
    return hipGetLastError();
}

}  // namespace oasis
