// Allocation-free sparse attention: the decode attention over caller-owned
// paged KV and attended lists, with its split-K partials in a fixed array of
// device memory that the library holds for the life of the process, one per
// GPU.  For callers that cannot allocate (code under HIP graph capture,
// serving loops that forbid hipMalloc).
#include <mutex>

#include "../../include/oasis.h"
#include "kernels.h"

using namespace oasis;

namespace {

// Partial rows the array holds: each row is one (m, l) pair and d = 128
// accumulators, fp32.
constexpr int64_t kRows = 61440;
constexpr int64_t kFloats = kRows * (2 + 128);  // 31.9 MB

}  // namespace

static __device__ __align__(256) float scratch[kFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float *g_ptr[kMaxDevices] = {};  // device address of `scratch` on each GPU

// The array's device address on the current device, looked up once per device.
int scratch_ptr(float **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return OASIS_E_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return OASIS_E_HIP;
        g_ptr[dev] = (float *)p;
    }
    *out = g_ptr[dev];
    return OASIS_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int oasis_sparse_attn_noalloc(const oasis_attn_desc *desc, const void *q_dev,
                                         const void *slots_dev, const int32_t *att_block_dev,
                                         const int32_t *att_slot_dev, const int32_t *counts_dev,
                                         int64_t tokens, float *out_dev, hipStream_t stream) {
    if (!desc || !q_dev || !slots_dev || !att_block_dev || !att_slot_dev || !counts_dev ||
        !out_dev)
        return OASIS_E_INVAL;
    if (!aligned16(q_dev) || !aligned16(slots_dev) || !aligned16(out_dev)) return OASIS_E_INVAL;
    const oasis_attn_desc &A = *desc;
    if (A.batch < 1 || A.num_kv_heads < 1 || A.num_q_heads < 1 ||
        A.num_q_heads % A.num_kv_heads != 0 || A.head_dim != 128 || A.block_size != 16 ||
        A.list_stride < 1 || A.list_stride > 1024 || A.slots_per_head < 1 || tokens < 0)
        return OASIS_E_INVAL;
    Dims D{};
    D.B = A.batch;
    D.Hq = A.num_q_heads;
    D.Hkv = A.num_kv_heads;
    D.G = A.num_q_heads / A.num_kv_heads;
    D.d = 128;
    D.dtype = kBF16;
    D.bs = 16;
    D.K = A.list_stride;
    D.S = A.slots_per_head;
    D.NBmax = (tokens + 15) / 16;
    if (D.G != 1 && D.G != 2 && D.G != 4 && D.G != 8 && D.G != 16) return OASIS_E_INVAL;
    AttnPlan P = plan_attention(D);
    P.nsf_max = 0;  // every attended block is read from its slot: no fetch partials
    P.nsa = P.flat ? 0 : P.ns1;
    const int64_t rows = attn_partial_rows(D, P);
    if (rows > kRows) return OASIS_E_CAPACITY;
    float *base = nullptr;
    if (int rc = scratch_ptr(&base)) return rc;
    float *pm = base, *pl = base + rows, *pa = base + 2 * rows;
    if (launch_attention(D, P, 0, 0, q_dev, const_cast<void *>(slots_dev), nullptr, att_block_dev,
                         att_slot_dev, counts_dev, tokens, pm, pl, pa, stream) != hipSuccess)
        return OASIS_E_HIP;
    if (launch_combine(D, P, 0, pm, pl, pa, out_dev, stream) != hipSuccess) return OASIS_E_HIP;
    return OASIS_OK;
}
