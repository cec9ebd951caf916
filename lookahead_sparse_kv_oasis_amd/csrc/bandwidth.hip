// Streaming read of a device buffer: the box's own reference rate for the
// HBM-bound kernels (the summary scan and the attention over resident slots),
// beside the published peak.
//
// Workgroup w reads 16 KB pieces w, w + W, ... of the buffer (W workgroups):
// each wave 4 KB of a piece, four 16-byte nontemporal loads per lane issued
// together.  The words are folded with XOR, per workgroup, into sink[w], so
// the loads cannot be dropped and the result can be checked against the
// buffer's contents.
#include "bandwidth.h"
#include "kernels.h"

namespace oasis {

namespace {

constexpr int kVecPerPiece = 256 * 4;  // 16-byte vectors in a 16 KB piece

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ buf,
                                                          int64_t n_vec,
                                                          uint32_t *__restrict__ sink) {
    __shared__ uint32_t part[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t acc = 0;
    const int64_t W = gridDim.x;
    for (int64_t p = blockIdx.x; p * kVecPerPiece < n_vec; p += W) {
        const int64_t base = p * kVecPerPiece + wave * 256 + lane;
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = base + k * 64;
            v[k] = i < n_vec ? __builtin_nontemporal_load(buf + i) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int workgroups,
                              hipStream_t st) {
    OASIS_LAUNCH(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, st,
                 (const u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace oasis
