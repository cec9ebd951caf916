// Token append and per-block min/max key summaries.
//
// OasisKV explainer page, Fig. 7: the GPU keeps "compressed keys" made by
// per-block min/max pooling of the keys whose full copy lives in CPU memory.
// A block's summary is, per dimension, the largest and smallest key value over
// the block's valid tokens.  Both kernels keep the first of equal values
// (strict comparisons in token order), so a summary is a bit-exact copy of
// existing key elements.  The summary region of a unit is block-major or tiled
// (the matrix-core operand order), see Dims; summ_offset addresses both.
#include "kernels.h"

namespace oasis {

// One workgroup per (b, KV head) unit; each thread moves 16-byte chunks of
// the token's K and V row.
template <typename T>
__global__ __launch_bounds__(64) void append_kernel(const T *__restrict__ k,
                                                    const T *__restrict__ v, int64_t pos,
                                                    T *host_kv, T *summ,
                                                    const int32_t *__restrict__ block_slot,
                                                    T *slots, int d, int bs, int S,
                                                    int64_t NBmax, bool tiled,
                                                    int64_t unit_elems) {
    constexpr int V = Elem<T>::kVec;
    const int64_t u = blockIdx.x;
    const int64_t j = pos / bs;
    const int o = (int)(pos % bs);
    const int32_t s = block_slot[u * NBmax + j];
    T *hk = host_kv + ((u * NBmax + j) * 2 * bs + o) * (int64_t)d;
    T *su = summ + u * unit_elems;
    for (int c = threadIdx.x * V; c < d; c += blockDim.x * V) {
        T *smx = su + summ_offset(tiled, d, j, 0, c);
        T *smn = su + summ_offset(tiled, d, j, 1, c);
        const Vec16<T> kk = ld16(k + u * d + c);
        const Vec16<T> vv = ld16(v + u * d + c);
        st16(hk + c, kk);
        st16(hk + (int64_t)bs * d + c, vv);
        Vec16<T> mx = kk, mn = kk;
        if (o != 0) {
            mx = ld16(smx);
            mn = ld16(smn);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float x = Elem<T>::f(kk.v[e]);
                if (x > Elem<T>::f(mx.v[e])) mx.v[e] = kk.v[e];
                if (x < Elem<T>::f(mn.v[e])) mn.v[e] = kk.v[e];
            }
        }
        st16(smx, mx);
        st16(smn, mn);
        if (s >= 0) {  // write-through into the resident copy of the block
            T *sl = slots + ((u * S + s) * 2 * bs + o) * (int64_t)d;
            st16(sl + c, kk);
            st16(sl + (int64_t)bs * d + c, vv);
        }
    }
}

// Grid-stride over (unit, block, 16-byte chunk of the key row).
template <typename T>
__global__ __launch_bounds__(256) void summary_build_kernel(const T *host_kv, int64_t T_,
                                                            T *summ, int d, int bs,
                                                            int64_t NBmax, int64_t NB,
                                                            int64_t units, bool tiled,
                                                            int64_t unit_elems) {
    constexpr int V = Elem<T>::kVec;
    const int chunks = d / V;
    const int64_t total = units * NB * chunks;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(i % chunks) * V;
        const int64_t r = i / chunks;
        const int64_t j = r % NB;
        const int64_t u = r / NB;
        const int64_t p0 = j * bs;
        const int n = (int)((T_ - p0) < bs ? (T_ - p0) : bs);
        const T *src = host_kv + (u * NBmax + j) * 2 * bs * (int64_t)d + c;
        Vec16<T> mx = ld16(src), mn = mx;
        for (int t = 1; t < n; ++t) {
            const Vec16<T> x = ld16(src + (int64_t)t * d);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float f = Elem<T>::f(x.v[e]);
                if (f > Elem<T>::f(mx.v[e])) mx.v[e] = x.v[e];
                if (f < Elem<T>::f(mn.v[e])) mn.v[e] = x.v[e];
            }
        }
        T *su = summ + u * unit_elems;
        st16(su + summ_offset(tiled, d, j, 0, c), mx);
        st16(su + summ_offset(tiled, d, j, 1, c), mn);
    }
}

hipError_t launch_append(const Dims &D, const void *k, const void *v, int64_t pos, void *host_kv,
                         void *summ, const int32_t *block_slot, void *slots, hipStream_t st) {
    dim3 grid((unsigned)D.units()), block(64);
    if (D.dtype == kF32)
        OASIS_LAUNCH(append_kernel<float>, grid, block, 0, st, (const float *)k,
                           (const float *)v, pos, (float *)host_kv, (float *)summ, block_slot,
                           (float *)slots, D.d, D.bs, D.S, D.NBmax, D.tiled,
                           D.summ_unit_elems());
    else
        OASIS_LAUNCH(append_kernel<uint16_t>, grid, block, 0, st, (const uint16_t *)k,
                           (const uint16_t *)v, pos, (uint16_t *)host_kv, (uint16_t *)summ,
                           block_slot, (uint16_t *)slots, D.d, D.bs, D.S, D.NBmax, D.tiled,
                           D.summ_unit_elems());
    return hipGetLastError();
}

hipError_t launch_summary_build(const Dims &D, const void *host_kv, int64_t T, void *summ,
                                hipStream_t st) {
    const int64_t NB = (T + D.bs - 1) / D.bs;
    if (NB == 0) return hipSuccess;
    const int V = D.dtype == kF32 ? 4 : 8;
    const int64_t total = D.units() * NB * (D.d / V);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (D.dtype == kF32)
        OASIS_LAUNCH(summary_build_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const float *)host_kv, T, (float *)summ, D.d, D.bs, D.NBmax, NB,
                           D.units(), D.tiled, D.summ_unit_elems());
    else
        OASIS_LAUNCH(summary_build_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0,
                           st, (const uint16_t *)host_kv, T, (uint16_t *)summ, D.d, D.bs,
                           D.NBmax, NB, D.units(), D.tiled, D.summ_unit_elems());
    return hipGetLastError();
}

}  // namespace oasis
