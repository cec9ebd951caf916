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
// each block with 16-byte loads of 8 per lane issued before the stores.  Host
// reads by shader loads run best with about 64 waves in flight (about 55 GB/s);
// one workgroup per block (thousands of waves) lowers the link rate and takes
// CU slots from the kernels running beside the copy.
#include "kernels.h"

namespace oasis {

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
    const int64_t W = (int64_t)gridDim.x * 4;
    const int64_t n_items = units * max_n;
    for (int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); item < n_items;
         item += W) {
        const int64_t u = item / max_n;
        const int i = (int)(item % max_n);
        const int n = counts[u * count_stride + count_index];
        if (i >= n) continue;
        const int32_t blk = blocks[u * list_stride + i];
        const int32_t s = slot_ids[u * list_stride + i];
        const u32x4 *src = host_kv + (u * NBmax + blk) * (int64_t)block_vec;
        u32x4 *dst = slots + (u * S + s) * (int64_t)block_vec;
        for (int c0 = 0; c0 < block_vec; c0 += 64 * 8) {
            u32x4 r[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = c0 + k * 64 + lane;
                if (c < block_vec) r[k] = __builtin_nontemporal_load(src + c);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = c0 + k * 64 + lane;
                if (c < block_vec) dst[c] = r[k];
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
