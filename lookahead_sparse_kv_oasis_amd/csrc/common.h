// Device-side helpers shared by the liboasis kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace oasis {

enum : int { kF32 = 0, kBF16 = 1 };

// Bits of the device error word.
enum : uint32_t {
    kErrNonFinite = 1u,   // a NaN / Inf score reached the top-K
    kErrSelect = 2u,      // diff/cap found an inconsistent table
    kErrSlots = 4u,       // not enough slots for the fetch (S < K misuse)
};

// Counters kept on the device, one row per (b, KV head) unit, summed over the
// units by oasis_get_stats.
struct DevStats {
    unsigned long long hits, misses, fetched, attended;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));  // 4 bf16 bit patterns

// LDS ordering between lanes of one wave.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// Element traits: storage type and exact conversion to fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kVec = 4;  // elements per 16-byte access
    __device__ __forceinline__ static float f(float x) { return x; }
};
template <> struct Elem<uint16_t> {
    static constexpr int kVec = 8;
    __device__ __forceinline__ static float f(uint16_t x) { return bf16_bits_to_f32(x); }
};

// 16-byte vector of storage elements.
template <typename T> struct alignas(16) Vec16 {
    T v[16 / sizeof(T)];
};

template <typename T> __device__ __forceinline__ Vec16<T> ld16(const T *p) {
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    return __builtin_bit_cast(Vec16<T>, u);
}
template <typename T> __device__ __forceinline__ void st16(T *p, const Vec16<T> &x) {
    *reinterpret_cast<uint4 *>(p) = __builtin_bit_cast(uint4, x);
}

// 16-byte global-memory access through an explicit global address space, so
// pointers picked at run time (slot or pinned host block) still compile to
// global_load / global_store rather than flat accesses.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const void *p) {
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Streaming read of data used once per decode step (summary tiles, resident
// KV slots): the nontemporal hint keeps it from displacing cached lines; on
// the summary scan it lifts the HBM rate from 5.5 to 6.0 TB/s.
__device__ __forceinline__ uint4 gload16_nt(const void *p) {
    const u32x4 v =
        __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void gstore16(void *p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    *(__attribute__((address_space(1))) u32x4 *)p = w;
}

// Unpack 8 bf16 held in a uint4 into fp32.
__device__ __forceinline__ void bf16x8_to_f32(const uint4 u, float *o) {
    o[0] = __uint_as_float(u.x << 16);
    o[1] = __uint_as_float(u.x & 0xffff0000u);
    o[2] = __uint_as_float(u.y << 16);
    o[3] = __uint_as_float(u.y & 0xffff0000u);
    o[4] = __uint_as_float(u.z << 16);
    o[5] = __uint_as_float(u.z & 0xffff0000u);
    o[6] = __uint_as_float(u.w << 16);
    o[7] = __uint_as_float(u.w & 0xffff0000u);
}

template <int I, int N, typename F> __device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Wave64 reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Wave64 reductions of 32-bit integers through DPP: an inclusive scan inside
// each 16-lane row (row_shr 1, 2, 4, 8), then the four row totals are read
// from lanes 15, 31, 47, 63.  The result is wave-uniform.
template <typename Op> __device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t id, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xF, 0xF, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ uint32_t wave_add_u32(uint32_t v) {
    return wave_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce_u32(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

// Lanes below this one in the wave (for ordered compaction with ballots).
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace oasis
