// C-ABI of liboasis: handle, allocations, streams and kernel dispatch.
//
// One handle is one layer.  It owns
//   - the pinned, device-mapped host KV [B][Hkv][NBmax][K|V][bs][d] (the CPU
//     full KV cache of the OasisKV page's Fig. 7),
//   - in HBM: the min/max summaries [B][Hkv][NBmax][max|min][d], the slot pool
//     [B][Hkv][S][K|V][bs][d] (the sparse KV working set), the per-KV-head
//     tables slot_block / block_slot / last_used (Fig. 9), scores, top-K ids,
//     fetch and attended lists, attention partials,
//   - a copy stream (default priority) for the host -> HBM gather, and the
//     events that order it against the caller's stream.
//
// Handles of layers whose KV is identical may share one host KV buffer
// (oasis_create_shared); the buffer is reference counted.
//
// Ordering: select waits for the previous gather and attention; the gather
// waits for select; attention and the next select wait for the gather (an
// append does not: the gather copies the rows of the tokens held at its
// select, the append writes the next one); attention, append and evict wait
// for the select; attention and select wait for the last append; attention
// waits for the previous attention.  A select, an append or a new predict
// also waits for score / top-K kernels that a predict queued on another
// stream.  A wait is issued only when the producing call ran on another
// stream (one stream is in order by itself).  No call synchronises the host
// except the inspection calls.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <memory>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "../../include/oasis.h"
#include "bandwidth.h"
#include "kernels.h"

using namespace oasis;

thread_local LaunchEvents oasis::g_launch_events;

namespace {

enum { TM_APPEND, TM_SCORE, TM_TOPK, TM_SELECT, TM_GATHER, TM_ATTN, TM_COMBINE, TM_N };
constexpr size_t kTimerCap = 4096;

struct Timers {
    std::vector<hipEvent_t> start, stop;
    size_t used = 0;
    double ms = 0.0;
    int64_t n = 0;
    int64_t seq = 0;      // launches seen since timing was set
    bool active = false;  // the current launch carries events
};

// Pinned, device-mapped host KV; shared by the handles created from one owner.
struct HostKV {
    void *host = nullptr;
    void *dev = nullptr;
    size_t bytes = 0;
    int64_t loaded = -1;   // tokens per sequence written by the last prompt load
    int64_t high = 0;      // rows per sequence below which a load or an append wrote
    ~HostKV() {
        if (host) (void)hipHostFree(host);
    }
};

// An event with the stream its last record went to.
struct Mark {
    hipEvent_t ev = nullptr;
    hipStream_t st = nullptr;
    bool set = false;
};

}  // namespace

struct oasis_handle {
    Dims D{};
    AttnPlan plan{};
    oasis_layout L{};
    float fetch_ratio = 0.f;
    int device = 0;
    bool use_mfma_score = false;

    int64_t T = 0, T_prefix = 0;
    bool predicted = false, selected = false;
    // Fused mode: the blocks chosen by select are copied host -> HBM inside
    // the next sparse attention (which reads them anyway); a call that needs
    // the slots before that (evict, select, reads) runs the standalone gather
    // first.  An append does not: the later copy takes its token from the
    // host KV.
    bool fused = false;
    bool fetch_pending = false;
    // The top-K of the last scores has not run yet: select_and_fetch runs it
    // fused with the select (one workgroup per unit).
    bool topk_pending = false;
    int64_t topk_nb = 0;
    // Score + top-K + select fusion (opt-in): predict records its query rows
    // and the next select scores, ranks and selects in one kernel.
    bool fuse_score = false;
    bool score_pending = false;
    const void *score_q = nullptr, *score_drafts = nullptr;
    int score_nd = 0;
    int last_cap = 0;
    // The last select's blocks are being copied by a gather on another
    // stream (m_gather) that no attention has waited for yet; with
    // split_beside_copy the next attention attends to the other blocks
    // before it waits for that copy.
    bool copy_open = false;
    bool split_beside_copy = false;

    std::shared_ptr<HostKV> hkv;
    void *host_kv = nullptr;      // host pointer (pinned), hkv->host
    void *host_kv_dev = nullptr;  // device view of the same memory
    void *summ = nullptr, *slots = nullptr;
    float *scores = nullptr;
    int32_t *ids = nullptr, *slot_block = nullptr, *block_slot = nullptr, *last_used = nullptr;
    int32_t *fetch_block = nullptr, *fetch_slot = nullptr, *att_block = nullptr,
            *att_slot = nullptr, *counts = nullptr;
    float *part_m = nullptr, *part_l = nullptr, *part_acc = nullptr;
    uint32_t *err = nullptr;
    DevStats *stats = nullptr;
    int32_t *evict_buf = nullptr;
    size_t evict_cap = 0;
    // oasis_set_state's device copy of the held blocks: [units][S] blocks,
    // [units][S] slots, [units] counts (allocated with the handle)
    int32_t *set_buf = nullptr;
    // verification attention: packed query rows and per-row partials
    float *vpart_m = nullptr, *vpart_l = nullptr, *vpart_acc = nullptr;

    hipStream_t copy = nullptr;
    Mark m_append, m_select, m_gather, m_attn;
    // The last score / top-K kernels launched outside a select (predict,
    // topk_from_scores, a flushed deferred score) and not yet ordered by a
    // select on their stream: a call on another stream that reads or
    // rewrites their inputs or outputs waits for them (after_predict).  The
    // event is recorded only then, so a caller that keeps predict and select
    // on one stream pays for no record.
    bool pred_open = false, pred_marked = false;
    hipStream_t pred_st = nullptr;
    hipEvent_t ev_predict = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;   // oasis_decode_layers
    // The marks are recorded only once the handle's work has used two
    // streams; until then stream order is all the ordering there is.
    bool multi = false;
    bool have_last = false;
    hipStream_t last_st = nullptr;

    int64_t n_select = 0;
    int32_t timing = 0;  // mask of timed kernel classes
    int32_t timing_period = 1;  // time one launch in this many per class
    Timers tm[TM_N];
    std::string last_error;
};

namespace {

int fail(oasis_t *h, int code, const char *fmt, ...) __attribute__((format(printf, 3, 4)));
int fail(oasis_t *h, int code, const char *fmt, ...) {
    if (h) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        h->last_error = buf;
    }
    return code;
}

#define HIP_OK(h, call)                                                                       \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return fail((h), OASIS_E_HIP, "%s: %s (%s:%d)", #call, hipGetErrorString(e_),    \
                        __FILE__, __LINE__);                                                  \
    } while (0)

int64_t nb_of(const oasis_t *h) { return (h->T + h->D.bs - 1) / h->D.bs; }

// Add the elapsed time of every recorded pair; a pair whose launch carried no
// kernel (nothing to do) has unrecorded events and is skipped.
void fold_timer(Timers &t) {
    for (size_t i = 0; i < t.used; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, t.start[i], t.stop[i]) == hipSuccess) {
            t.ms += ms;
            ++t.n;
        }
    }
    (void)hipGetLastError();
    t.used = 0;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Record m on st.
int mark(oasis_t *h, Mark &m, hipStream_t st) {
    if (!h->multi) return OASIS_OK;  // one stream so far: nothing waits across streams
    HIP_OK(h, hipEventRecord(m.ev, st));
    m.st = st;
    m.set = true;
    return OASIS_OK;
}

// Note that the handle's next work goes to st.  The first time that differs
// from the stream used so far, every mark is recorded there (covering all the
// work queued until now) and from then on each step records its marks.  A
// record costs the GPU a few microseconds before the next kernel, so a caller
// that keeps a handle on one stream pays for none.  The synchronous internal
// uses of the copy stream (prompt load, state set, reads) follow a device
// synchronization and end with one, so they do not count.
int use_stream(oasis_t *h, hipStream_t st) {
    if (h->multi) return OASIS_OK;
    if (!h->have_last) {
        h->have_last = true;
        h->last_st = st;
        return OASIS_OK;
    }
    if (st == h->last_st) return OASIS_OK;
    h->multi = true;
    for (Mark *m : {&h->m_append, &h->m_select, &h->m_gather, &h->m_attn})
        if (int rc = mark(h, *m, h->last_st)) return rc;
    return OASIS_OK;
}

// Make st wait for the work behind m when it was recorded on another stream.
int after(oasis_t *h, hipStream_t st, const Mark &m) {
    if (!m.set || m.st == st) return OASIS_OK;
    HIP_OK(h, hipStreamWaitEvent(st, m.ev, 0));
    return OASIS_OK;
}

int tbegin(oasis_t *h, int cls, hipStream_t st) {
    (void)st;
    if (!(h->timing & (1 << cls))) return OASIS_OK;
    Timers &t = h->tm[cls];
    t.active = (t.seq++ % h->timing_period) == 0;
    if (!t.active) return OASIS_OK;
    if (t.used == kTimerCap) {  // fold finished pairs into the sum
        HIP_OK(h, hipEventSynchronize(t.stop[t.used - 1]));
        fold_timer(t);
    }
    if (t.used == t.start.size()) {
        // read by the host only, after the stop event completes: no system
        // fence (with one, the timed launches ran 2-5 us longer than the
        // others: the fence flushed the caches around them)
        hipEvent_t a, b;
        HIP_OK(h, hipEventCreateWithFlags(&a, hipEventDisableSystemFence));
        HIP_OK(h, hipEventCreateWithFlags(&b, hipEventDisableSystemFence));
        t.start.push_back(a);
        t.stop.push_back(b);
    }
    g_launch_events.start = t.start[t.used];
    g_launch_events.stop = t.stop[t.used];
    return OASIS_OK;
}

int tend(oasis_t *h, int cls, hipStream_t st) {
    (void)st;
    if (!(h->timing & (1 << cls))) return OASIS_OK;
    Timers &t = h->tm[cls];
    if (!t.active) return OASIS_OK;
    g_launch_events = LaunchEvents{};
    t.active = false;
    ++t.used;
    return OASIS_OK;
}

#define TRY(expr)                  \
    do {                           \
        int rc_ = (expr);          \
        if (rc_ != OASIS_OK) return rc_; \
    } while (0)

#define LAUNCH(h, cls, st, call)                                                              \
    do {                                                                                      \
        TRY(tbegin((h), (cls), (st)));                                                        \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return fail((h), OASIS_E_HIP, "launch %s: %s", #call, hipGetErrorString(e_));    \
        TRY(tend((h), (cls), (st)));                                                          \
    } while (0)

template <typename F> void parallel_for(int64_t n, F &&f) {
    unsigned nt = std::thread::hardware_concurrency();
    if (nt == 0) nt = 4;
    if (nt > 16) nt = 16;
    if (n < (int64_t)nt) nt = (unsigned)std::max<int64_t>(n, 1);
    std::vector<std::thread> th;
    for (unsigned w = 0; w < nt; ++w)
        th.emplace_back([&, w] {
            for (int64_t i = w; i < n; i += nt) f(i);
        });
    for (auto &t : th) t.join();
}

void free_all(oasis_t *h) {
    (void)hipFree(h->summ);
    (void)hipFree(h->slots);
    (void)hipFree(h->scores);
    (void)hipFree(h->ids);
    (void)hipFree(h->slot_block);
    (void)hipFree(h->block_slot);
    (void)hipFree(h->last_used);
    (void)hipFree(h->fetch_block);
    (void)hipFree(h->fetch_slot);
    (void)hipFree(h->att_block);
    (void)hipFree(h->att_slot);
    (void)hipFree(h->counts);
    (void)hipFree(h->part_m);
    (void)hipFree(h->part_l);
    (void)hipFree(h->part_acc);
    (void)hipFree(h->err);
    (void)hipFree(h->stats);
    (void)hipFree(h->evict_buf);
    (void)hipFree(h->set_buf);
    (void)hipFree(h->vpart_m);
    (void)hipFree(h->vpart_l);
    (void)hipFree(h->vpart_acc);
    h->hkv.reset();
    if (h->copy) (void)hipStreamDestroy(h->copy);
    for (hipEvent_t e : {h->m_append.ev, h->m_select.ev, h->m_gather.ev, h->m_attn.ev, h->ev_fork,
                         h->ev_join, h->ev_predict})
        if (e) (void)hipEventDestroy(e);
    for (auto &t : h->tm) {
        for (auto e : t.start) (void)hipEventDestroy(e);
        for (auto e : t.stop) (void)hipEventDestroy(e);
    }
}

int reset_tables(oasis_t *h) {
    const Dims &D = h->D;
    HIP_OK(h, hipMemset(h->slot_block, 0xFF, sizeof(int32_t) * D.units() * D.S));
    HIP_OK(h, hipMemset(h->last_used, 0xFF, sizeof(int32_t) * D.units() * D.S));
    HIP_OK(h, hipMemset(h->block_slot, 0xFF, sizeof(int32_t) * D.units() * D.NBmax));
    HIP_OK(h, hipMemset(h->counts, 0, sizeof(int32_t) * D.units() * 4));
    HIP_OK(h, hipMemset(h->fetch_block, 0xFF, sizeof(int32_t) * D.units() * D.K));
    HIP_OK(h, hipMemset(h->fetch_slot, 0xFF, sizeof(int32_t) * D.units() * D.K));
    HIP_OK(h, hipMemset(h->att_block, 0xFF, sizeof(int32_t) * D.units() * D.K));
    HIP_OK(h, hipMemset(h->att_slot, 0xFF, sizeof(int32_t) * D.units() * D.K));
    HIP_OK(h, hipMemset(h->ids, 0xFF, sizeof(int32_t) * D.units() * D.K));
    h->predicted = h->selected = false;
    h->fetch_pending = false;
    h->topk_pending = false;
    h->score_pending = false;
    h->copy_open = false;
    return OASIS_OK;
}

// Score / top-K kernels were just queued on st outside a select.
void open_predict(oasis_t *h, hipStream_t st) {
    h->pred_open = true;
    h->pred_marked = false;
    h->pred_st = st;
}

// Make st wait for the open score / top-K kernels when they were queued on
// another stream.  The event is recorded on their stream now: it covers them
// and whatever was queued there after them.
int after_predict(oasis_t *h, hipStream_t st) {
    if (!h->pred_open || h->pred_st == st) return OASIS_OK;
    if (!h->pred_marked) {
        HIP_OK(h, hipEventRecord(h->ev_predict, h->pred_st));
        h->pred_marked = true;
    }
    HIP_OK(h, hipStreamWaitEvent(st, h->ev_predict, 0));
    return OASIS_OK;
}

// Run a deferred score on its own (when the scores are needed before a select).
int flush_score(oasis_t *h, hipStream_t st) {
    if (!h->score_pending) return OASIS_OK;
    h->score_pending = false;
    TRY(after(h, st, h->m_append));
    TRY(after(h, st, h->m_select));
    TRY(after_predict(h, st));
    LAUNCH(h, TM_SCORE, st,
           launch_score(h->D, h->summ, h->score_q, h->score_drafts, h->score_nd, h->topk_nb,
                        h->scores, st));
    open_predict(h, st);
    return OASIS_OK;
}

// Run a deferred top-K on its own (when the ids are needed before a select).
int flush_topk(oasis_t *h, hipStream_t st) {
    TRY(flush_score(h, st));
    if (!h->topk_pending) return OASIS_OK;
    h->topk_pending = false;
    TRY(after_predict(h, st));
    LAUNCH(h, TM_TOPK, st, launch_topk(h->D, h->scores, h->topk_nb, h->ids, nullptr, h->err, st));
    open_predict(h, st);
    return OASIS_OK;
}

// Copy the pending fetch list host -> HBM now (fused mode only).
int flush_fetch(oasis_t *h, hipStream_t st) {
    if (!h->fetch_pending) return OASIS_OK;
    h->fetch_pending = false;
    LAUNCH(h, TM_GATHER, st,
           launch_gather(h->D, h->host_kv_dev, h->slots, h->fetch_block, h->fetch_slot, h->D.K,
                         h->counts, 4, 2, h->last_cap, h->T, st));
    return OASIS_OK;
}

}  // namespace

// ------------------------------------------------------------------ helpers

extern "C" uint64_t oasis_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                             int32_t dtype_bytes) {
    if (layers < 0 || kv_heads < 0 || head_dim < 0 || dtype_bytes < 0) return 0;
    return (uint64_t)layers * 2u * (uint64_t)kv_heads * (uint64_t)head_dim *
           (uint64_t)dtype_bytes;
}

extern "C" int oasis_stream_read(const void *buf_dev, int64_t bytes, uint32_t *sink_dev,
                                 int32_t workgroups, hipStream_t stream) {
    if (!buf_dev || !sink_dev || !aligned16(buf_dev) || bytes <= 0 || bytes % 16 != 0 ||
        workgroups < 1 || workgroups > 65536)
        return OASIS_E_INVAL;
    return launch_stream_read(buf_dev, bytes, sink_dev, workgroups, stream) == hipSuccess
               ? OASIS_OK
               : OASIS_E_HIP;
}

extern "C" int32_t oasis_cap_from_ratio(float ratio, int32_t k_blocks) {
    if (!(ratio > 0.f) || k_blocks <= 0) return 0;
    if (ratio >= 1.f) return k_blocks;
    const double c = std::floor((double)ratio * (double)k_blocks + 1e-9);
    const int32_t cap = (int32_t)c;
    return cap < 1 ? 1 : (cap > k_blocks ? k_blocks : cap);
}

extern "C" const char *oasis_strerror(int status) {
    switch (status) {
    case OASIS_OK: return "ok";
    case OASIS_E_INVAL: return "invalid argument";
    case OASIS_E_NOMEM: return "out of memory";
    case OASIS_E_HIP: return "HIP runtime error";
    case OASIS_E_CAPACITY: return "sequence capacity exceeded";
    case OASIS_E_STATE: return "call out of order";
    case OASIS_E_NONFINITE: return "non-finite score";
    case OASIS_E_DEVICE: return "device invariant failed";
    default: return "unknown status";
    }
}

extern "C" const char *oasis_last_error(const oasis_t *h) {
    return h ? h->last_error.c_str() : "null handle";
}

// ------------------------------------------------------------------ lifetime

namespace {

int create_handle(const oasis_layout *layout, int32_t block_size, int32_t budget_tokens,
                  float fetch_ratio, const oasis_t *owner, oasis_t **out) {
    if (!layout || !out) return OASIS_E_INVAL;
    *out = nullptr;
    const oasis_layout &L = *layout;
    if (L.batch < 1 || L.num_q_heads < 1 || L.num_kv_heads < 1 ||
        L.num_q_heads % L.num_kv_heads != 0)
        return OASIS_E_INVAL;
    if (L.head_dim < 8 || L.head_dim > 256 || L.head_dim % 8 != 0) return OASIS_E_INVAL;
    if (L.dtype != OASIS_F32 && L.dtype != OASIS_BF16) return OASIS_E_INVAL;
    if (L.max_drafts < 0 || L.max_tokens < 1) return OASIS_E_INVAL;
    if (block_size < 1 || block_size > 64 || budget_tokens < block_size) return OASIS_E_INVAL;
    if (!(fetch_ratio >= 0.f) || !std::isfinite(fetch_ratio)) return OASIS_E_INVAL;
    const int K = budget_tokens / block_size;
    const int S = L.slots_per_head > 0 ? L.slots_per_head : K;
    const int G = L.num_q_heads / L.num_kv_heads;
    const int64_t NBmax = (L.max_tokens + block_size - 1) / block_size;
    if (K > 1024 || S < K || S > 2048 || NBmax > 65536) return OASIS_E_INVAL;
    Dims probe{};
    const int dev_cus = compute_units(probe);  // the current device's CUs
    if (L.compute_units < 0 || L.compute_units > dev_cus) return OASIS_E_INVAL;
    const int Q = G * (1 + L.max_drafts);
    if ((int64_t)Q * L.head_dim * 4 > 64 * 1024) return OASIS_E_INVAL;

    oasis_t *h = new (std::nothrow) oasis_t;
    if (!h) return OASIS_E_NOMEM;
    h->L = L;
    h->fetch_ratio = fetch_ratio;
    Dims &D = h->D;
    D.B = L.batch;
    D.Hq = L.num_q_heads;
    D.Hkv = L.num_kv_heads;
    D.G = G;
    D.d = L.head_dim;
    D.dtype = L.dtype;
    D.bs = block_size;
    D.K = K;
    D.S = S;
    D.NBmax = NBmax;
    D.cus = L.compute_units > 0 ? L.compute_units : dev_cus;
    h->plan = plan_attention(D);
    h->plan.vns = verify_stride(D);
    h->use_mfma_score = D.dtype == kBF16 && (D.d == 64 || D.d == 128 || D.d == 256) && Q <= 128;
    if (const char *e = getenv("OASIS_SCORE_IMPL"))
        if (!strcmp(e, "valu")) h->use_mfma_score = false;
    D.tiled = h->use_mfma_score;  // the matrix-core score reads the tiled summary layout
    h->fused = h->plan.mfma;
    if (const char *e = getenv("OASIS_GATHER"))
        if (!strcmp(e, "stream")) h->fused = false;

    auto bail = [&](int code) {
        free_all(h);
        delete h;
        return code;
    };
    if (hipGetDevice(&h->device) != hipSuccess) return bail(OASIS_E_HIP);

    const int64_t units = D.units();
    const size_t e = D.esize();
    const size_t host_bytes = (size_t)units * NBmax * D.block_elems() * e;
    if (owner) {
        const oasis_layout &O = owner->L;
        if (O.batch != L.batch || O.num_kv_heads != L.num_kv_heads || O.head_dim != L.head_dim ||
            O.dtype != L.dtype || owner->D.bs != block_size || owner->D.NBmax != NBmax ||
            owner->device != h->device || !owner->hkv || owner->hkv->bytes != host_bytes)
            return bail(OASIS_E_INVAL);
        h->hkv = owner->hkv;
    } else {
        auto hk = std::make_shared<HostKV>();
        if (hipHostMalloc(&hk->host, host_bytes, hipHostMallocMapped) != hipSuccess)
            return bail(OASIS_E_NOMEM);
        hk->bytes = host_bytes;
        if (hipHostGetDevicePointer(&hk->dev, hk->host, 0) != hipSuccess) return bail(OASIS_E_HIP);
        char *p = (char *)hk->host;
        const size_t chunk = 64u << 20;
        const int64_t nchunks = (int64_t)((host_bytes + chunk - 1) / chunk);
        parallel_for(nchunks, [&](int64_t i) {
            const size_t off = (size_t)i * chunk;
            memset(p + off, 0, std::min(chunk, host_bytes - off));
        });
        h->hkv = std::move(hk);
    }
    h->host_kv = h->hkv->host;
    h->host_kv_dev = h->hkv->dev;

    auto dmal = [&](void **p, size_t bytes) { return hipMalloc(p, bytes ? bytes : 16) == hipSuccess; };
    const int64_t PR = attn_partial_rows(D, h->plan);
    const size_t summ_bytes = (size_t)units * D.summ_unit_elems() * e;
    bool ok = dmal(&h->summ, summ_bytes) &&
              dmal(&h->slots, (size_t)units * S * D.block_elems() * e) &&
              dmal((void **)&h->scores, sizeof(float) * units * NBmax) &&
              dmal((void **)&h->ids, sizeof(int32_t) * units * K) &&
              dmal((void **)&h->slot_block, sizeof(int32_t) * units * S) &&
              dmal((void **)&h->block_slot, sizeof(int32_t) * units * NBmax) &&
              dmal((void **)&h->last_used, sizeof(int32_t) * units * S) &&
              dmal((void **)&h->fetch_block, sizeof(int32_t) * units * K) &&
              dmal((void **)&h->fetch_slot, sizeof(int32_t) * units * K) &&
              dmal((void **)&h->att_block, sizeof(int32_t) * units * K) &&
              dmal((void **)&h->att_slot, sizeof(int32_t) * units * K) &&
              dmal((void **)&h->counts, sizeof(int32_t) * units * 4) &&
              dmal((void **)&h->part_m, sizeof(float) * PR) &&
              dmal((void **)&h->part_l, sizeof(float) * PR) &&
              dmal((void **)&h->part_acc, sizeof(float) * PR * D.d) &&
              dmal((void **)&h->err, sizeof(uint32_t)) &&
              dmal((void **)&h->stats, sizeof(DevStats) * units) &&
              dmal((void **)&h->set_buf, sizeof(int32_t) * units * (2 * (size_t)S + 1)) &&
              dmal((void **)&h->evict_buf, sizeof(int32_t) * units * ((size_t)K + 1));
    h->evict_cap = (size_t)units * (K + 1);
    const int vrows = verify_rows(D, L.max_drafts);  // padded rows per unit, -1: too many
    if (ok && h->plan.mfma && vrows > 0) {
        // verification attention scratch, sized for max_drafts
        const size_t rows = (size_t)units * vrows;
        ok = dmal((void **)&h->vpart_m, rows * h->plan.vns * sizeof(float)) &&
             dmal((void **)&h->vpart_l, rows * h->plan.vns * sizeof(float)) &&
             dmal((void **)&h->vpart_acc, rows * h->plan.vns * 128 * sizeof(float));
    }
    if (!ok) return bail(OASIS_E_NOMEM);
    if (hipMemset(h->summ, 0, summ_bytes) != hipSuccess ||
        hipMemset(h->slots, 0, (size_t)units * S * D.block_elems() * e) != hipSuccess ||
        hipMemset(h->scores, 0, sizeof(float) * units * NBmax) != hipSuccess ||
        hipMemset(h->err, 0, sizeof(uint32_t)) != hipSuccess ||
        hipMemset(h->stats, 0, sizeof(DevStats) * units) != hipSuccess)
        return bail(OASIS_E_HIP);
    if (reset_tables(h) != OASIS_OK) return bail(OASIS_E_HIP);
    // The ordering events are only waited on by other streams of this GPU,
    // never by the host, and every kernel already ends with a device-wide
    // release of its writes.  Without the flag each record performed a
    // system-scope cache writeback and invalidate that left the GPU idle for
    // about 5.7 us before the next kernel (three records per decode step).
    constexpr unsigned kMarkFlags = hipEventDisableTiming | hipEventDisableSystemFence;
    if (hipStreamCreateWithFlags(&h->copy, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&h->m_append.ev, kMarkFlags) != hipSuccess ||
        hipEventCreateWithFlags(&h->m_select.ev, kMarkFlags) != hipSuccess ||
        hipEventCreateWithFlags(&h->m_gather.ev, kMarkFlags) != hipSuccess ||
        hipEventCreateWithFlags(&h->m_attn.ev, kMarkFlags) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_fork, kMarkFlags) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_join, kMarkFlags) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_predict, kMarkFlags) != hipSuccess)
        return bail(OASIS_E_HIP);
    if (hipDeviceSynchronize() != hipSuccess) return bail(OASIS_E_HIP);
    *out = h;
    return OASIS_OK;
}

}  // namespace

extern "C" int oasis_create(const oasis_layout *layout, int32_t block_size, int32_t budget_tokens,
                            float fetch_ratio, oasis_t **out) {
    return create_handle(layout, block_size, budget_tokens, fetch_ratio, nullptr, out);
}

extern "C" int oasis_create_shared(const oasis_layout *layout, int32_t block_size,
                                   int32_t budget_tokens, float fetch_ratio, const oasis_t *owner,
                                   oasis_t **out) {
    if (!owner) {
        if (out) *out = nullptr;
        return OASIS_E_INVAL;
    }
    return create_handle(layout, block_size, budget_tokens, fetch_ratio, owner, out);
}

extern "C" int oasis_destroy(oasis_t *h) {
    if (!h) return OASIS_E_INVAL;
    (void)hipDeviceSynchronize();
    free_all(h);
    delete h;
    return OASIS_OK;
}

// ------------------------------------------------------------------ setup

extern "C" int oasis_load_prefix(oasis_t *h, const void *k_host, const void *v_host,
                                 int64_t len, hipStream_t stream) {
    if (!h) return OASIS_E_INVAL;
    if (len < 0 || len > h->L.max_tokens)
        return fail(h, OASIS_E_CAPACITY, "prefix of %lld tokens exceeds max_tokens %lld",
                    (long long)len, (long long)h->L.max_tokens);
    const bool reuse = !k_host && !v_host;
    HostKV &hkv = *h->hkv;
    if (reuse && hkv.loaded != len)
        return fail(h, OASIS_E_STATE,
                    "prefix reuse: the host KV holds a prompt of %lld tokens, not %lld",
                    (long long)hkv.loaded, (long long)len);
    if (!reuse && len > 0 && (!k_host || !v_host)) return fail(h, OASIS_E_INVAL, "null prefix");
    const Dims &D = h->D;
    HIP_OK(h, hipDeviceSynchronize());
    const size_t e = D.esize();
    const size_t row = (size_t)D.d * e;
    const int64_t NB = (len + D.bs - 1) / D.bs;
    // Rows past the prompt are cleared up to the end of its next block and up
    // to the highest row any append wrote, so slots never carry stale tokens.
    const int64_t clear_to = std::min<int64_t>(std::max<int64_t>((NB + 1) * D.bs, hkv.high),
                                               D.NBmax * D.bs);
    char *hk = (char *)h->host_kv;
    parallel_for(D.units(), [&](int64_t u) {
        const char *ks = reuse ? nullptr : (const char *)k_host + (size_t)u * len * row;
        const char *vs = reuse ? nullptr : (const char *)v_host + (size_t)u * len * row;
        for (int64_t j = 0; j * D.bs < clear_to; ++j) {
            char *blk = hk + ((size_t)u * D.NBmax + j) * D.block_elems() * e;
            const int64_t p0 = j * D.bs;
            const int64_t n = j < NB ? std::min<int64_t>(D.bs, len - p0) : 0;
            if (n > 0 && !reuse) {
                memcpy(blk, ks + p0 * row, n * row);
                memcpy(blk + D.bs * row, vs + p0 * row, n * row);
            }
            if (n < D.bs) {
                memset(blk + n * row, 0, (D.bs - n) * row);
                memset(blk + D.bs * row + n * row, 0, (D.bs - n) * row);
            }
        }
    });
    hkv.loaded = len;
    hkv.high = len;
    h->T = h->T_prefix = len;
    HIP_OK(h, launch_summary_build(D, h->host_kv_dev, len, h->summ, stream));
    HIP_OK(h, hipStreamSynchronize(stream));
    TRY(reset_tables(h));
    HIP_OK(h, hipDeviceSynchronize());
    return OASIS_OK;
}

extern "C" int oasis_set_state(oasis_t *h, const int32_t *slot_block_host,
                               const int32_t *last_used_host) {
    if (!h || !slot_block_host || !last_used_host) return OASIS_E_INVAL;
    const Dims &D = h->D;
    const int64_t units = D.units(), NB = nb_of(h);
    std::vector<int32_t> lb((size_t)units * D.S), ls((size_t)units * D.S), cnt((size_t)units);
    std::vector<char> seen((size_t)NB > 0 ? (size_t)NB : 1);
    int maxn = 0;
    for (int64_t u = 0; u < units; ++u) {
        std::fill(seen.begin(), seen.end(), 0);
        int n = 0;
        for (int s = 0; s < D.S; ++s) {
            const int32_t b = slot_block_host[u * D.S + s];
            if (b < -1 || b >= NB)
                return fail(h, OASIS_E_INVAL, "unit %lld slot %d holds block %d (NB %lld)",
                            (long long)u, s, b, (long long)NB);
            if (b < 0) continue;
            if (seen[b]) return fail(h, OASIS_E_INVAL, "block %d held twice in unit %lld", b, (long long)u);
            seen[b] = 1;
            lb[u * D.S + n] = b;
            ls[u * D.S + n] = s;
            ++n;
        }
        cnt[u] = n;
        maxn = std::max(maxn, n);
    }
    h->fetch_pending = false;   // the tables are replaced wholesale
    h->copy_open = false;
    HIP_OK(h, hipDeviceSynchronize());
    HIP_OK(h, hipMemcpy(h->slot_block, slot_block_host, sizeof(int32_t) * units * D.S,
                        hipMemcpyHostToDevice));
    HIP_OK(h, hipMemcpy(h->last_used, last_used_host, sizeof(int32_t) * units * D.S,
                        hipMemcpyHostToDevice));
    HIP_OK(h, launch_rebuild_block_slot(D, h->slot_block, h->block_slot, h->copy));
    int32_t *dlb = h->set_buf, *dls = dlb + lb.size(), *dcnt = dls + ls.size();
    int rc = OASIS_OK;
    if (hipMemcpy(dlb, lb.data(), sizeof(int32_t) * lb.size(), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dls, ls.data(), sizeof(int32_t) * ls.size(), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dcnt, cnt.data(), sizeof(int32_t) * cnt.size(), hipMemcpyHostToDevice) != hipSuccess ||
        launch_gather(D, h->host_kv_dev, h->slots, dlb, dls, D.S, dcnt, 1, 0, maxn, h->T,
                      h->copy) !=
            hipSuccess ||
        hipStreamSynchronize(h->copy) != hipSuccess)
        rc = fail(h, OASIS_E_HIP, "set_state upload or payload copy failed");
    h->selected = false;
    return rc;
}

// ------------------------------------------------------------------ decode step

extern "C" int oasis_append_kv(oasis_t *h, const void *k_dev, const void *v_dev,
                               hipStream_t stream) {
    if (!h || !k_dev || !v_dev || !aligned16(k_dev) || !aligned16(v_dev))
        return h ? fail(h, OASIS_E_INVAL, "append: null or misaligned pointer") : OASIS_E_INVAL;
    if (h->T >= h->L.max_tokens)
        return fail(h, OASIS_E_CAPACITY, "append: sequence already holds max_tokens = %lld",
                    (long long)h->L.max_tokens);
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_attn));
    TRY(after(h, stream, h->m_select));  // and the score the select ranked
    // No wait for a gather still copying the last select's blocks on another
    // stream: it copies the rows of the tokens held at that select only, and
    // this token's row is written here (into the host KV, and into the slot,
    // the block being resident since the select), so the two touch disjoint
    // bytes.  A fetch left pending by the last select stays pending: it
    // copies the host blocks later on this stream, after this token is in
    // the host KV, so a fetched block's slot ends up with the token whether
    // or not the write-through below reaches it first.  In the lookahead
    // order (append, attend, predict, select) the next attention thus
    // streams its hits from HBM while its fetch waves read the host link.
    TRY(flush_score(h, stream));  // a deferred predict scores the summaries before this token
    TRY(after_predict(h, stream));  // a score on another stream may still read the summaries
    LAUNCH(h, TM_APPEND, stream,
           launch_append(h->D, k_dev, v_dev, h->T, h->host_kv_dev, h->summ, h->block_slot,
                         h->slots, stream));
    ++h->T;
    h->hkv->high = std::max(h->hkv->high, h->T);
    TRY(mark(h, h->m_append, stream));
    return OASIS_OK;
}

extern "C" int oasis_predict(oasis_t *h, const void *q_dev, const void *drafts_dev,
                             int32_t n_drafts, int32_t *block_ids_dev, float *scores_dev,
                             hipStream_t stream) {
    if (!h) return OASIS_E_INVAL;
    if ((q_dev && !aligned16(q_dev)) || (!q_dev && n_drafts < 1))
        return fail(h, OASIS_E_INVAL, "predict: bad q (null q needs at least one draft)");
    if (n_drafts < 0 || n_drafts > h->L.max_drafts)
        return fail(h, OASIS_E_INVAL, "predict: n_drafts %d outside [0, %d]", n_drafts,
                    h->L.max_drafts);
    if (n_drafts > 0 && (!drafts_dev || !aligned16(drafts_dev)))
        return fail(h, OASIS_E_INVAL, "predict: bad drafts pointer");
    const int64_t NB = nb_of(h);
    if (NB == 0) return fail(h, OASIS_E_STATE, "predict: no tokens loaded");
    const Dims &D = h->D;
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_append));
    TRY(after(h, stream, h->m_select));  // the previous select reads the scores
    TRY(after_predict(h, stream));       // an earlier score writes the same buffers
    h->score_pending = false;
    if (h->fuse_score && !block_ids_dev && !scores_dev &&
        score_topk_fusable(D, NB, D.G * ((q_dev ? 1 : 0) + n_drafts))) {
        h->score_pending = true;  // scored by the next select's fused kernel
        h->score_q = q_dev;
        h->score_drafts = drafts_dev;
        h->score_nd = n_drafts;
        h->topk_nb = NB;
        h->topk_pending = true;
        h->predicted = true;
        return OASIS_OK;
    }
    LAUNCH(h, TM_SCORE, stream,
           launch_score(D, h->summ, q_dev, drafts_dev, n_drafts, NB, h->scores,
                        stream));
    if (scores_dev)
        HIP_OK(h, hipMemcpyAsync(scores_dev, h->scores, sizeof(float) * D.units() * D.NBmax,
                                 hipMemcpyDeviceToDevice, stream));
    h->topk_nb = NB;
    if (block_ids_dev) {
        LAUNCH(h, TM_TOPK, stream,
               launch_topk(D, h->scores, NB, h->ids, block_ids_dev, h->err, stream));
        h->topk_pending = false;
    } else {
        h->topk_pending = true;
    }
    open_predict(h, stream);
    h->predicted = true;
    return OASIS_OK;
}

extern "C" int oasis_topk_from_scores(oasis_t *h, const float *scores_dev,
                                      int32_t *block_ids_dev, hipStream_t stream) {
    if (!h || !scores_dev) return h ? fail(h, OASIS_E_INVAL, "topk: null scores") : OASIS_E_INVAL;
    const int64_t NB = nb_of(h);
    if (NB == 0) return fail(h, OASIS_E_STATE, "topk: no tokens loaded");
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_select));  // the previous select reads the ids
    TRY(after_predict(h, stream));
    LAUNCH(h, TM_TOPK, stream,
           launch_topk(h->D, scores_dev, NB, h->ids, block_ids_dev, h->err, stream));
    open_predict(h, stream);
    h->topk_pending = false;
    h->score_pending = false;
    h->predicted = true;
    return OASIS_OK;
}

namespace {

// Select, then copy the fetched blocks: inside the next attention when the
// handle fuses the fetch and `gst` is null, else eagerly on `gst` (the copy
// stream when null).
int select_impl(oasis_t *h, int32_t cap, hipStream_t stream, bool eager, hipStream_t gst) {
    if (!h) return OASIS_E_INVAL;
    if (!h->predicted) return fail(h, OASIS_E_STATE, "select before predict");
    const Dims &D = h->D;
    if (cap < 0) cap = oasis_cap_from_ratio(h->fetch_ratio, D.K);
    if (cap > D.K) cap = D.K;
    const int64_t t64 = h->T - h->T_prefix;
    if (t64 > INT32_MAX - 1) return fail(h, OASIS_E_CAPACITY, "step index overflow");
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_gather));
    TRY(after(h, stream, h->m_attn));
    TRY(after(h, stream, h->m_append));  // it reads the block -> slot table the select rewrites
    TRY(after_predict(h, stream));  // the scores / ids it ranks and reads
    TRY(flush_fetch(h, stream));
    if (h->score_pending) {
        // the deferred predict's orderings, on this stream
        TRY(after(h, stream, h->m_append));
        TRY(after(h, stream, h->m_select));
        h->score_pending = false;
        h->topk_pending = false;
        LAUNCH(h, TM_SCORE, stream,
               launch_score_topk_select(D, h->summ, h->score_q, h->score_drafts, h->score_nd,
                                        h->topk_nb, h->scores, h->ids, h->slot_block,
                                        h->last_used, h->block_slot, cap, (int32_t)t64,
                                        h->fetch_block, h->fetch_slot, h->att_block,
                                        h->att_slot, h->counts, h->stats, h->err, stream));
    } else if (h->topk_pending) {
        h->topk_pending = false;
        LAUNCH(h, TM_SELECT, stream,
               launch_topk_select(D, h->scores, h->topk_nb, h->ids, h->slot_block, h->last_used,
                                  h->block_slot, cap, (int32_t)t64, h->fetch_block,
                                  h->fetch_slot, h->att_block, h->att_slot, h->counts, h->stats,
                                  h->err, stream));
    } else {
        LAUNCH(h, TM_SELECT, stream,
               launch_select(D, h->ids, h->slot_block, h->last_used, h->block_slot, cap,
                             (int32_t)t64, h->fetch_block, h->fetch_slot, h->att_block,
                             h->att_slot, h->counts, h->stats, h->err, stream));
    }
    h->last_cap = cap;
    // From here stream order after the select (and its mark) covers the
    // predict's kernels.
    h->pred_open = false;
    TRY(mark(h, h->m_select, stream));
    h->copy_open = false;
    if (h->fused && !eager) {
        h->fetch_pending = cap > 0;
    } else if (cap > 0) {
        hipStream_t g = gst ? gst : h->copy;
        TRY(use_stream(h, g));
        TRY(after(h, g, h->m_select));
        LAUNCH(h, TM_GATHER, g,
               launch_gather(D, h->host_kv_dev, h->slots, h->fetch_block, h->fetch_slot, D.K,
                             h->counts, 4, 2, cap, h->T, g));
        TRY(mark(h, h->m_gather, g));
        h->copy_open = true;
    }
    ++h->n_select;
    h->selected = true;
    return OASIS_OK;
}

}  // namespace

extern "C" int oasis_select_and_fetch(oasis_t *h, int32_t cap, hipStream_t stream,
                                      hipStream_t copy) {
    if (copy == OASIS_COPY_DEFAULT) return select_impl(h, cap, stream, false, nullptr);
    return select_impl(h, cap, stream, true, copy);
}

extern "C" int oasis_evict_attended(oasis_t *h, const double *draws_dev, double fraction,
                                    hipStream_t stream) {
    if (!h || !draws_dev || !(fraction >= 0.0) || !(fraction <= 1.0))
        return h ? fail(h, OASIS_E_INVAL, "evict_attended: bad arguments") : OASIS_E_INVAL;
    if (((uintptr_t)draws_dev & 7u) != 0)
        return fail(h, OASIS_E_INVAL, "evict_attended: draws not 8-byte aligned");
    if (!h->selected) return fail(h, OASIS_E_STATE, "evict_attended before select");
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_select));  // the attended list and the tables it rewrites
    TRY(after(h, stream, h->m_gather));
    TRY(after(h, stream, h->m_attn));
    TRY(after(h, stream, h->m_append));  // an append reads block_slot for its write-through
    TRY(flush_fetch(h, stream));  // a pending copy lands before its slot is emptied
    HIP_OK(h, launch_evict_attended(h->D, draws_dev, fraction, h->att_block, h->counts,
                                    h->slot_block, h->block_slot, stream));
    // later appends, selects and attentions on other streams wait for the tables
    TRY(mark(h, h->m_select, stream));
    return OASIS_OK;
}

extern "C" int oasis_evict(oasis_t *h, const int32_t *blocks_host, const int32_t *counts_host,
                           int32_t max_per_unit, hipStream_t stream) {
    if (!h || !blocks_host || !counts_host || max_per_unit < 1)
        return h ? fail(h, OASIS_E_INVAL, "evict: bad arguments") : OASIS_E_INVAL;
    const Dims &D = h->D;
    const size_t n = (size_t)D.units() * (max_per_unit + 1);
    if (n > h->evict_cap) {
        HIP_OK(h, hipDeviceSynchronize());
        (void)hipFree(h->evict_buf);
        h->evict_buf = nullptr;
        HIP_OK(h, hipMalloc(&h->evict_buf, sizeof(int32_t) * n));
        h->evict_cap = n;
    }
    int32_t *dblocks = h->evict_buf, *dcounts = h->evict_buf + (size_t)D.units() * max_per_unit;
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_gather));
    TRY(after(h, stream, h->m_attn));
    TRY(after(h, stream, h->m_select));  // a select on another stream rewrites the same tables
    TRY(flush_fetch(h, stream));
    HIP_OK(h, hipMemcpyAsync(dblocks, blocks_host, sizeof(int32_t) * D.units() * max_per_unit,
                             hipMemcpyHostToDevice, stream));
    HIP_OK(h, hipMemcpyAsync(dcounts, counts_host, sizeof(int32_t) * D.units(),
                             hipMemcpyHostToDevice, stream));
    HIP_OK(h, launch_evict(D, dblocks, dcounts, max_per_unit, h->slot_block, h->block_slot, stream));
    HIP_OK(h, hipStreamSynchronize(stream));
    return OASIS_OK;
}

extern "C" int oasis_sparse_attn(oasis_t *h, const void *q_dev, float *out_dev,
                                 hipStream_t stream) {
    if (!h || !q_dev || !out_dev || !aligned16(q_dev) || !aligned16(out_dev))
        return h ? fail(h, OASIS_E_INVAL, "attn: null or misaligned pointer") : OASIS_E_INVAL;
    if (!h->selected) return fail(h, OASIS_E_STATE, "attention before select");
    const Dims &D = h->D;
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_select));
    // the last append: its write-through into resident slots, and the host
    // token a pending fetch copies
    TRY(after(h, stream, h->m_append));
    // the previous attention: the same partials, and the slots its fetch wrote
    TRY(after(h, stream, h->m_attn));
    const bool split = h->split_beside_copy && h->copy_open && h->m_gather.set &&
                       h->m_gather.st != stream && h->plan.mfma && h->plan.flat &&
                       h->last_cap > 0 && !h->fetch_pending;
    h->copy_open = false;
    if (split) {
        // the blocks held before the select while the copy runs, the fetched
        // ones from their slots once it has landed (their partials in the
        // fetch splits, as the fused form writes them)
        const int nsf = attention_fetch_splits(D, h->plan, h->last_cap);
        LAUNCH(h, TM_ATTN, stream,
               launch_attention(D, h->plan, 2, nsf, q_dev, h->slots, h->host_kv_dev,
                                h->att_block, h->att_slot, h->counts, h->T, h->part_m,
                                h->part_l, h->part_acc, stream));
        TRY(after(h, stream, h->m_gather));
        HIP_OK(h, launch_attention(D, h->plan, 3, nsf, q_dev, h->slots, h->host_kv_dev,
                                   h->att_block, h->att_slot, h->counts, h->T, h->part_m,
                                   h->part_l, h->part_acc, stream));
        LAUNCH(h, TM_COMBINE, stream,
               launch_combine(D, h->plan, nsf, h->part_m, h->part_l, h->part_acc, out_dev,
                              stream));
        TRY(mark(h, h->m_attn, stream));
        return OASIS_OK;
    }
    TRY(after(h, stream, h->m_gather));
    int mode = 0, nsf = 0;
    if (h->fetch_pending) {
        if (h->plan.mfma) {
            mode = 1;
            nsf = attention_fetch_splits(D, h->plan, h->last_cap);
            h->fetch_pending = false;
        } else {
            TRY(flush_fetch(h, stream));
        }
    }
    LAUNCH(h, TM_ATTN, stream,
           launch_attention(D, h->plan, mode, nsf, q_dev, h->slots, h->host_kv_dev, h->att_block,
                            h->att_slot, h->counts, h->T, h->part_m, h->part_l, h->part_acc,
                            stream));
    LAUNCH(h, TM_COMBINE, stream,
           launch_combine(D, h->plan, nsf, h->part_m, h->part_l, h->part_acc, out_dev, stream));
    TRY(mark(h, h->m_attn, stream));
    return OASIS_OK;
}

extern "C" int oasis_sparse_attn_verify(oasis_t *h, const void *q_dev, const void *drafts_dev,
                                        int32_t n_drafts, const void *k_drafts_dev,
                                        const void *v_drafts_dev, float *out_dev,
                                        hipStream_t stream) {
    if (!h) return OASIS_E_INVAL;
    if (!q_dev || !out_dev || !aligned16(q_dev) || !aligned16(out_dev))
        return fail(h, OASIS_E_INVAL, "verify: null or misaligned q / out");
    if (n_drafts < 0 || n_drafts > h->L.max_drafts)
        return fail(h, OASIS_E_INVAL, "verify: n_drafts %d outside [0, %d]", n_drafts,
                    h->L.max_drafts);
    if (n_drafts > 0 && (!drafts_dev || !k_drafts_dev || !v_drafts_dev || !aligned16(drafts_dev) ||
                         !aligned16(k_drafts_dev) || !aligned16(v_drafts_dev)))
        return fail(h, OASIS_E_INVAL, "verify: null or misaligned drafts or draft K/V");
    if (!h->plan.mfma)
        return fail(h, OASIS_E_INVAL, "verify: needs the bf16, d = 128, block 16 layout");
    if (!h->vpart_m || verify_rows(h->D, n_drafts) < 0)
        return fail(h, OASIS_E_INVAL, "verify: %d query rows per KV head exceed the verify passes",
                    h->D.G * (1 + n_drafts));
    if (!h->selected) return fail(h, OASIS_E_STATE, "verify attention before select");
    const Dims &D = h->D;
    TRY(use_stream(h, stream));
    TRY(after(h, stream, h->m_select));
    TRY(after(h, stream, h->m_gather));
    TRY(after(h, stream, h->m_append));  // the last token, written through into its slot
    // the previous attention: its fetch waves write the slots read here, and
    // an earlier verify on another stream uses the same scratch
    TRY(after(h, stream, h->m_attn));
    TRY(flush_fetch(h, stream));  // every attended block resident before the passes
    // several launches: not a class of the per-kernel timers
    HIP_OK(h, launch_verify(D, h->plan, n_drafts, q_dev, drafts_dev, k_drafts_dev, v_drafts_dev,
                            h->slots, h->att_block, h->att_slot, h->counts, h->T,
                            h->vpart_m, h->vpart_l, h->vpart_acc, out_dev, stream));
    TRY(mark(h, h->m_attn, stream));
    return OASIS_OK;
}

// ------------------------------------------------------------------ layer pipeline

// One decode step over the layers of a model.  With side != stream, the
// append / predict / select of every layer go to `side` in layer order and
// each layer's attention goes to `stream` once that layer's select is done,
// so prediction and selection of later layers run under the attention (and
// its fused host fetch) of earlier ones (OasisKV page, Fig. 8: predict,
// select and transfer per layer overlapped with compute).  Per-layer
// ordering across steps comes from the handles' own marks.
extern "C" int oasis_decode_layers(oasis_t *const *layers, const oasis_layer_io *io,
                                   int32_t n_layers, int32_t n_drafts, int32_t cap,
                                   hipStream_t stream, hipStream_t side) {
    if (!layers || !io || n_layers < 1) return OASIS_E_INVAL;
    for (int32_t l = 0; l < n_layers; ++l) {
        if (!layers[l]) return OASIS_E_INVAL;
        for (int32_t m = 0; m < l; ++m)
            if (layers[m] == layers[l])
                return fail(layers[l], OASIS_E_INVAL, "decode_layers: handle %d repeats %d", l, m);
        if ((io[l].k_new == nullptr) != (io[l].v_new == nullptr))
            return fail(layers[l], OASIS_E_INVAL, "decode_layers: layer %d has k without v", l);
    }
    oasis_t *h0 = layers[0];
    const bool overlap = side != stream;
    if (overlap) {
        HIP_OK(h0, hipEventRecord(h0->ev_fork, stream));
        HIP_OK(h0, hipStreamWaitEvent(side, h0->ev_fork, 0));
    }
    hipStream_t pre = overlap ? side : stream;
    int rc = OASIS_OK, bad = -1;
    // All pre-attention work is queued first: the side stream runs ahead of
    // the attention stream by as many layers as it can.
    for (int32_t l = 0; l < n_layers && rc == OASIS_OK; ++l) {
        oasis_t *h = layers[l];
        if (io[l].k_new) rc = oasis_append_kv(h, io[l].k_new, io[l].v_new, pre);
        if (rc == OASIS_OK)
            rc = oasis_predict(h, io[l].q, io[l].drafts, n_drafts, nullptr, nullptr, pre);
        if (rc == OASIS_OK) rc = oasis_select_and_fetch(h, cap, pre, OASIS_COPY_DEFAULT);
        if (rc == OASIS_OK && !overlap) rc = oasis_sparse_attn(h, io[l].q, io[l].out, stream);
        if (rc != OASIS_OK) bad = l;
    }
    if (overlap) {
        for (int32_t l = 0; l < n_layers && rc == OASIS_OK; ++l) {
            rc = oasis_sparse_attn(layers[l], io[l].q, io[l].out, stream);
            if (rc != OASIS_OK) bad = l;
        }
        // Join: the caller's stream sees the side stream's work even where a
        // call failed half way.
        if (hipEventRecord(h0->ev_join, side) != hipSuccess ||
            hipStreamWaitEvent(stream, h0->ev_join, 0) != hipSuccess)
            return rc != OASIS_OK ? rc : fail(h0, OASIS_E_HIP, "decode_layers: join failed");
    }
    if (bad > 0) {
        const std::string msg = layers[bad]->last_error;
        fail(h0, rc, "decode_layers: layer %d: %s", bad, msg.c_str());
    }
    return rc;
}

// One decode step over the layers in the lookahead order (OasisKV page,
// Fig. 8): per layer, the new token is appended and the current query attends
// over the set the previous call selected (on `stream`); then the drafts alone
// predict the next step's set, which is selected (on `side`) and copied host
// -> HBM (on `xfer`).  Nothing waits for the copies until that layer's next
// attention, so each transfer has the rest of the step to land.
extern "C" int oasis_decode_layers_ahead(oasis_t *const *layers, const oasis_layer_io *io,
                                         int32_t n_layers, int32_t n_drafts, int32_t cap,
                                         int32_t cap_correct, hipStream_t stream,
                                         hipStream_t side, hipStream_t xfer) {
    if (!layers || !io || n_layers < 1) return OASIS_E_INVAL;
    if (n_drafts < 1) return fail(layers[0], OASIS_E_INVAL, "decode_layers_ahead: no drafts");
    for (int32_t l = 0; l < n_layers; ++l) {
        if (!layers[l]) return OASIS_E_INVAL;
        for (int32_t m = 0; m < l; ++m)
            if (layers[m] == layers[l])
                return fail(layers[l], OASIS_E_INVAL, "decode_layers_ahead: handle %d repeats %d",
                            l, m);
        if ((io[l].k_new == nullptr) != (io[l].v_new == nullptr))
            return fail(layers[l], OASIS_E_INVAL, "decode_layers_ahead: layer %d has k without v",
                        l);
        if (!io[l].drafts)
            return fail(layers[l], OASIS_E_INVAL, "decode_layers_ahead: layer %d has no drafts", l);
    }
    oasis_t *h0 = layers[0];
    // side and xfer see the caller's earlier work
    if (side != stream || xfer != stream) {
        HIP_OK(h0, hipEventRecord(h0->ev_fork, stream));
        if (side != stream) HIP_OK(h0, hipStreamWaitEvent(side, h0->ev_fork, 0));
        if (xfer != stream) HIP_OK(h0, hipStreamWaitEvent(xfer, h0->ev_fork, 0));
    }
    int rc = OASIS_OK, bad = -1;
    for (int32_t l = 0; l < n_layers && rc == OASIS_OK; ++l) {
        oasis_t *h = layers[l];
        if (io[l].k_new) rc = oasis_append_kv(h, io[l].k_new, io[l].v_new, stream);
        const bool attend = h->selected && io[l].q && io[l].out;
        if (rc == OASIS_OK && attend && cap_correct > 0) {
            // decode-time miss correction: the current query's own top-K, its
            // missing blocks fetched now (inside the attention when fused)
            rc = oasis_predict(h, io[l].q, nullptr, 0, nullptr, nullptr, stream);
            if (rc == OASIS_OK) rc = select_impl(h, cap_correct, stream, !h->fused, stream);
        }
        if (rc == OASIS_OK && attend) rc = oasis_sparse_attn(h, io[l].q, io[l].out, stream);
        if (rc == OASIS_OK)
            rc = oasis_predict(h, nullptr, io[l].drafts, n_drafts, nullptr, nullptr, side);
        if (rc == OASIS_OK) rc = select_impl(h, cap, side, true, xfer);
        if (rc != OASIS_OK) bad = l;
    }
    if (bad > 0) {
        const std::string msg = layers[bad]->last_error;
        fail(h0, rc, "decode_layers_ahead: layer %d: %s", bad, msg.c_str());
    }
    return rc;
}

// ------------------------------------------------------------------ inspection

extern "C" int64_t oasis_buffer_bytes(const oasis_t *h, int32_t which) {
    if (!h) return OASIS_E_INVAL;
    const Dims &D = h->D;
    const int64_t u = D.units(), e = D.esize();
    switch (which) {
    case OASIS_BUF_SUMMARY: return u * D.NBmax * 2 * D.d * e;
    case OASIS_BUF_SLOTS: return u * D.S * D.block_elems() * e;
    case OASIS_BUF_HOST_KV: return u * D.NBmax * D.block_elems() * e;
    case OASIS_BUF_SCORES: return u * D.NBmax * 4;
    case OASIS_BUF_IDS: return u * D.K * 4;
    case OASIS_BUF_SLOT_BLOCK: return u * D.S * 4;
    case OASIS_BUF_BLOCK_SLOT: return u * D.NBmax * 4;
    case OASIS_BUF_LAST_USED: return u * D.S * 4;
    case OASIS_BUF_FETCH_BLOCK:
    case OASIS_BUF_FETCH_SLOT:
    case OASIS_BUF_ATT_BLOCK:
    case OASIS_BUF_ATT_SLOT: return u * D.K * 4;
    case OASIS_BUF_COUNTS: return u * 4 * 4;
    default: return OASIS_E_INVAL;
    }
}

namespace {

// Block-major bytes [offset, offset + nbytes) of a tiled summary: the units the
// range touches are copied whole and reordered on the host.
int read_tiled_summary(oasis_t *h, int64_t offset, int64_t nbytes, char *dst) {
    const Dims &D = h->D;
    const size_t e = D.esize();
    const int64_t logical_unit = D.NBmax * 2 * D.d * (int64_t)e;
    if (nbytes == 0) return OASIS_OK;
    std::vector<uint16_t> tiled((size_t)D.summ_unit_elems());
    std::vector<uint16_t> plain((size_t)(D.NBmax * 2 * D.d));
    for (int64_t u = offset / logical_unit; u <= (offset + nbytes - 1) / logical_unit; ++u) {
        HIP_OK(h, hipMemcpy(tiled.data(), (const uint16_t *)h->summ + u * D.summ_unit_elems(),
                            tiled.size() * sizeof(uint16_t), hipMemcpyDeviceToHost));
        for (int64_t j = 0; j < D.NBmax; ++j)
            for (int half = 0; half < 2; ++half)
                for (int c = 0; c < D.d; c += 8)
                    memcpy(&plain[(size_t)(j * 2 * D.d + half * D.d + c)],
                           &tiled[(size_t)summ_offset(true, D.d, j, half, c)], 16);
        const int64_t lo = std::max(offset, u * logical_unit);
        const int64_t hi = std::min(offset + nbytes, (u + 1) * logical_unit);
        memcpy(dst + (lo - offset), (const char *)plain.data() + (lo - u * logical_unit),
               (size_t)(hi - lo));
    }
    return OASIS_OK;
}

}  // namespace

extern "C" int oasis_read(oasis_t *h, int32_t which, int64_t offset, int64_t nbytes,
                          void *dst_host) {
    if (!h || !dst_host) return OASIS_E_INVAL;
    const int64_t size = oasis_buffer_bytes(h, which);
    if (size < 0) return fail(h, OASIS_E_INVAL, "read: unknown buffer %d", which);
    if (offset < 0 || nbytes < 0 || offset + nbytes > size)
        return fail(h, OASIS_E_INVAL, "read: range [%lld, +%lld) outside %lld bytes",
                    (long long)offset, (long long)nbytes, (long long)size);
    HIP_OK(h, hipDeviceSynchronize());
    if (h->fetch_pending || (h->topk_pending && which == OASIS_BUF_IDS) ||
        (h->score_pending && which == OASIS_BUF_SCORES)) {
        TRY(flush_fetch(h, h->copy));
        if (which == OASIS_BUF_IDS) TRY(flush_topk(h, h->copy));
        if (which == OASIS_BUF_SCORES) TRY(flush_score(h, h->copy));
        HIP_OK(h, hipStreamSynchronize(h->copy));
    }
    const void *src = nullptr;
    switch (which) {
    case OASIS_BUF_SUMMARY:
        if (h->D.tiled) return read_tiled_summary(h, offset, nbytes, (char *)dst_host);
        src = h->summ;
        break;
    case OASIS_BUF_SLOTS: src = h->slots; break;
    case OASIS_BUF_HOST_KV:
        memcpy(dst_host, (const char *)h->host_kv + offset, (size_t)nbytes);
        return OASIS_OK;
    case OASIS_BUF_SCORES: src = h->scores; break;
    case OASIS_BUF_IDS: src = h->ids; break;
    case OASIS_BUF_SLOT_BLOCK: src = h->slot_block; break;
    case OASIS_BUF_BLOCK_SLOT: src = h->block_slot; break;
    case OASIS_BUF_LAST_USED: src = h->last_used; break;
    case OASIS_BUF_FETCH_BLOCK: src = h->fetch_block; break;
    case OASIS_BUF_FETCH_SLOT: src = h->fetch_slot; break;
    case OASIS_BUF_ATT_BLOCK: src = h->att_block; break;
    case OASIS_BUF_ATT_SLOT: src = h->att_slot; break;
    case OASIS_BUF_COUNTS: src = h->counts; break;
    }
    HIP_OK(h, hipMemcpy(dst_host, (const char *)src + offset, (size_t)nbytes,
                        hipMemcpyDeviceToHost));
    return OASIS_OK;
}

extern "C" int oasis_get_state(oasis_t *h, int32_t *slot_block, int32_t *last_used,
                               int32_t *fetch_list, int32_t *fetch_n, int32_t *attended) {
    if (!h) return OASIS_E_INVAL;
    const Dims &D = h->D;
    const int64_t units = D.units();
    HIP_OK(h, hipDeviceSynchronize());
    if (slot_block)
        HIP_OK(h, hipMemcpy(slot_block, h->slot_block, sizeof(int32_t) * units * D.S,
                            hipMemcpyDeviceToHost));
    if (last_used)
        HIP_OK(h, hipMemcpy(last_used, h->last_used, sizeof(int32_t) * units * D.S,
                            hipMemcpyDeviceToHost));
    if (!fetch_list && !fetch_n && !attended) return OASIS_OK;
    std::vector<int32_t> cnt((size_t)units * 4, 0);
    if (h->selected)
        HIP_OK(h, hipMemcpy(cnt.data(), h->counts, sizeof(int32_t) * cnt.size(),
                            hipMemcpyDeviceToHost));
    std::vector<int32_t> a((size_t)units * D.K), b((size_t)units * D.K);
    if (fetch_list) {
        HIP_OK(h, hipMemcpy(a.data(), h->fetch_block, sizeof(int32_t) * a.size(),
                            hipMemcpyDeviceToHost));
        HIP_OK(h, hipMemcpy(b.data(), h->fetch_slot, sizeof(int32_t) * b.size(),
                            hipMemcpyDeviceToHost));
        for (int64_t u = 0; u < units; ++u)
            for (int i = 0; i < D.K; ++i) {
                const bool v = i < cnt[u * 4 + 2];
                fetch_list[(u * D.K + i) * 2 + 0] = v ? a[u * D.K + i] : -1;
                fetch_list[(u * D.K + i) * 2 + 1] = v ? b[u * D.K + i] : -1;
            }
    }
    if (fetch_n)
        for (int64_t u = 0; u < units; ++u) fetch_n[u] = cnt[u * 4 + 2];
    if (attended) {
        HIP_OK(h, hipMemcpy(a.data(), h->att_block, sizeof(int32_t) * a.size(),
                            hipMemcpyDeviceToHost));
        for (int64_t u = 0; u < units; ++u)
            for (int i = 0; i < D.K; ++i)
                attended[u * D.K + i] = i < cnt[u * 4 + 0] ? a[u * D.K + i] : -1;
    }
    return OASIS_OK;
}

extern "C" int oasis_get_stats(oasis_t *h, oasis_stats *out) {
    if (!h || !out) return OASIS_E_INVAL;
    HIP_OK(h, hipDeviceSynchronize());
    std::vector<DevStats> rows((size_t)h->D.units());
    HIP_OK(h, hipMemcpy(rows.data(), h->stats, sizeof(DevStats) * rows.size(),
                        hipMemcpyDeviceToHost));
    DevStats s{};
    for (const DevStats &r : rows) {
        s.hits += r.hits;
        s.misses += r.misses;
        s.fetched += r.fetched;
        s.attended += r.attended;
    }
    out->steps = h->n_select;
    out->hits = (int64_t)s.hits;
    out->misses = (int64_t)s.misses;
    out->fetched = (int64_t)s.fetched;
    out->attended = (int64_t)s.attended;
    out->bytes_fetched = (int64_t)s.fetched * h->D.block_elems() * h->D.esize();
    out->tokens = h->T;
    out->fetch_fused = h->fused ? 1 : 0;
    return OASIS_OK;
}

extern "C" int oasis_check(oasis_t *h) {
    if (!h) return OASIS_E_INVAL;
    HIP_OK(h, hipDeviceSynchronize());
    uint32_t e = 0;
    HIP_OK(h, hipMemcpy(&e, h->err, sizeof e, hipMemcpyDeviceToHost));
    HIP_OK(h, hipMemset(h->err, 0, sizeof e));
    if (e & kErrNonFinite) return fail(h, OASIS_E_NONFINITE, "a NaN or infinite score reached the top-K");
    if (e) return fail(h, OASIS_E_DEVICE, "device invariant word 0x%x", e);
    return OASIS_OK;
}

extern "C" int oasis_set_timing(oasis_t *h, int32_t mask) {
    if (!h) return OASIS_E_INVAL;
    HIP_OK(h, hipDeviceSynchronize());
    h->timing = mask & OASIS_TIME_ALL;
    for (auto &t : h->tm) {
        t.used = 0;
        t.ms = 0.0;
        t.n = 0;
        t.seq = 0;
        t.active = false;
    }
    return OASIS_OK;
}

extern "C" int oasis_set_attend_all_resident(oasis_t *h, int32_t on) {
    if (!h) return OASIS_E_INVAL;
    if (on && h->D.S > h->D.K)
        return fail(h, OASIS_E_INVAL,
                    "attend_all_resident: %d slots per KV head exceed the %d-entry attended list",
                    h->D.S, h->D.K);
    h->D.attend_all = on != 0;
    return OASIS_OK;
}

extern "C" int oasis_set_score_topk_fusion(oasis_t *h, int32_t on) {
    if (!h) return OASIS_E_INVAL;
    h->fuse_score = on != 0;
    if (!h->fuse_score && h->score_pending) {
        HIP_OK(h, hipDeviceSynchronize());  // the work the deferred score follows
        TRY(flush_score(h, h->copy));
        HIP_OK(h, hipStreamSynchronize(h->copy));
    }
    return OASIS_OK;
}

extern "C" int oasis_set_fetch_in_attention(oasis_t *h, int32_t on) {
    if (!h) return OASIS_E_INVAL;
    if (on && !h->plan.mfma)
        return fail(h, OASIS_E_INVAL,
                    "fetch in attention: needs the bf16, d = 128, block 16 layout");
    if (h->fetch_pending) {
        HIP_OK(h, hipDeviceSynchronize());  // the select the copy follows
        TRY(flush_fetch(h, h->copy));
        HIP_OK(h, hipStreamSynchronize(h->copy));
    }
    h->fused = on != 0;
    return OASIS_OK;
}

extern "C" int oasis_set_attention_beside_copy(oasis_t *h, int32_t on) {
    if (!h) return OASIS_E_INVAL;
    h->split_beside_copy = on != 0;
    return OASIS_OK;
}

extern "C" int oasis_set_timing_period(oasis_t *h, int32_t period) {
    if (!h || period < 1) return h ? fail(h, OASIS_E_INVAL, "timing period %d < 1", period) : OASIS_E_INVAL;
    h->timing_period = period;
    return OASIS_OK;
}

extern "C" int oasis_get_timing(oasis_t *h, oasis_timing *out) {
    if (!h || !out) return OASIS_E_INVAL;
    HIP_OK(h, hipDeviceSynchronize());
    double ms[TM_N];
    int64_t n[TM_N];
    for (int c = 0; c < TM_N; ++c) {
        Timers &t = h->tm[c];
        fold_timer(t);
        ms[c] = t.ms;
        n[c] = t.n;
    }
    out->ms_append = ms[TM_APPEND];
    out->ms_score = ms[TM_SCORE];
    out->ms_topk = ms[TM_TOPK];
    out->ms_select = ms[TM_SELECT];
    out->ms_gather = ms[TM_GATHER];
    out->ms_attn = ms[TM_ATTN];
    out->ms_combine = ms[TM_COMBINE];
    out->n_append = n[TM_APPEND];
    out->n_score = n[TM_SCORE];
    out->n_topk = n[TM_TOPK];
    out->n_select = n[TM_SELECT];
    out->n_gather = n[TM_GATHER];
    out->n_attn = n[TM_ATTN];
    out->n_combine = n[TM_COMBINE];
    return OASIS_OK;
}

extern "C" int oasis_get_dims(const oasis_t *h, int32_t *k_blocks, int32_t *slots,
                              int64_t *nb_max, int32_t *block_size) {
    if (!h) return OASIS_E_INVAL;
    if (k_blocks) *k_blocks = h->D.K;
    if (slots) *slots = h->D.S;
    if (nb_max) *nb_max = h->D.NBmax;
    if (block_size) *block_size = h->D.bs;
    return OASIS_OK;
}

extern "C" int64_t oasis_tokens(const oasis_t *h) { return h ? h->T : OASIS_E_INVAL; }

extern "C" hipStream_t oasis_copy_stream(const oasis_t *h) { return h ? h->copy : nullptr; }

extern "C" int oasis_stream_create_cus(int32_t first_cu, int32_t n_cus, hipStream_t *out) {
    if (!out) return OASIS_E_INVAL;
    *out = nullptr;
    Dims probe{};
    const int ncu = compute_units(probe);
    if (first_cu < 0 || n_cus < 1 || (int64_t)first_cu + n_cus > ncu) return OASIS_E_INVAL;
    std::vector<uint32_t> mask((size_t)(ncu + 31) / 32, 0u);
    for (int i = first_cu; i < first_cu + n_cus; ++i) mask[(size_t)i / 32] |= 1u << (i % 32);
    if (hipExtStreamCreateWithCUMask(out, (uint32_t)mask.size(), mask.data()) != hipSuccess) {
        *out = nullptr;
        return OASIS_E_HIP;
    }
    return OASIS_OK;
}

extern "C" int oasis_stream_destroy(hipStream_t stream) {
    if (!stream) return OASIS_E_INVAL;
    return hipStreamDestroy(stream) == hipSuccess ? OASIS_OK : OASIS_E_HIP;
}
