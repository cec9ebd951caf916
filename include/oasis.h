/*
 * liboasis -- OasisKV per-layer decode hot path on MI355X (gfx950).
 *
 * The full KV cache of a layer lives in pinned host memory; HBM holds, per
 * (batch row, KV head): a min/max key summary of every KV block and a bounded
 * pool of block slots (the sparse KV working set).  One decode step is
 *
 *   oasis_append_kv        write the new token (host KV, summary, resident slot)
 *   oasis_predict          score every block against the current and draft
 *                          queries, take the per-KV-head top-K
 *   oasis_select_and_fetch diff the top-K against the resident slots, cap the
 *                          fetch, pick LRU victims, gather the missing blocks
 *                          from pinned host memory on a side stream
 *   oasis_sparse_attn      GQA decode attention over the selected resident
 *                          blocks
 *
 * Sources: the OasisKV explainer page ("OasisKV: Scaling In-Decode KV Cache
 * Beyond HBM with Lookahead Sparse Prefetching"), Fig. 7 (CPU full KV, GPU
 * min/max-pooled compressed keys, sparse KV working set; drafts score the
 * pooled keys to pick the next top-K), Fig. 8 (predict -> select ->
 * transfer per layer on streams), Fig. 9 (per-KV-head GPU block -> CPU block
 * table), Table 2 (fetch cap by fetch ratio, LRU eviction), the explanatory
 * diagram (diff against the GPU-resident blocks, cap the per-step transfer)
 * and the capped-eviction glossary entry; the "KV cache offloading, week 2"
 * study notes, section 2 (KV bytes per token) and section 3 (GQA,
 * PagedAttention blocks).
 *
 * Conventions
 *   - Every call returns an int status (OASIS_OK = 0, negative on error) and
 *     never throws or aborts.  oasis_last_error() gives the message of the
 *     last failing call on a handle.
 *   - Calls that take a hipStream_t are asynchronous on that stream, like HIP
 *     calls.  The calls of one handle may use different streams: each waits
 *     for the handle's earlier work it depends on (HIP events, recorded only
 *     once a handle has used two streams).  Pointers named *_dev are device
 *     memory owned by the caller, 16-byte aligned, contiguous, and must stay
 *     valid until the stream has run the work.  Pointers named *_host are host memory read or written
 *     before the call returns.
 *   - Element type of K, V, queries and drafts is the layout's dtype
 *     (OASIS_F32, or OASIS_BF16 as raw 16-bit patterns).  Scores and the
 *     attention output are fp32.
 *   - A handle is one layer.  It is not thread-safe.
 *   - All sequences of the batch have the same length T; each append adds one
 *     token to every sequence.
 */
#ifndef OASIS_H
#define OASIS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    OASIS_OK = 0,
    OASIS_E_INVAL = -1,     /* bad argument, shape or pointer */
    OASIS_E_NOMEM = -2,     /* host or device allocation failed */
    OASIS_E_HIP = -3,       /* a HIP runtime call failed (message in oasis_last_error) */
    OASIS_E_CAPACITY = -4,  /* append past max_tokens */
    OASIS_E_STATE = -5,     /* call out of order (select before predict, ...) */
    OASIS_E_NONFINITE = -6, /* a NaN or infinite score reached the top-K */
    OASIS_E_DEVICE = -7     /* a device-side invariant failed (see oasis_check) */
};

enum { OASIS_F32 = 0, OASIS_BF16 = 1 };

typedef struct {
    int32_t batch;          /* B */
    int32_t num_q_heads;    /* Hq */
    int32_t num_kv_heads;   /* Hkv; Hq % Hkv == 0, q head g uses KV head g / (Hq/Hkv) */
    int32_t head_dim;       /* d; multiple of 8, at most 256 */
    int32_t dtype;          /* OASIS_F32 or OASIS_BF16 */
    int32_t max_drafts;     /* largest n_drafts passed to oasis_predict */
    int32_t slots_per_head; /* HBM block slots per (b, KV head); 0 -> budget blocks;
                               budget blocks <= slots <= 2048 */
    int32_t compute_units;  /* CUs the handle's launches are sized to fill; 0 -> all
                               of the device's.  Set it to n_cus when the handle's
                               compute work runs on a stream from
                               oasis_stream_create_cus (0 or 1..device CUs) */
    int64_t max_tokens;     /* capacity of the host KV per sequence */
} oasis_layout;

typedef struct oasis_handle oasis_t;

/* Create a handle for one layer.  block_size: tokens per KV block (the
 * paging unit, 1..64).  budget_tokens: the KV budget per (b, KV head); the
 * top-K takes K = budget_tokens / block_size blocks (1..1024).  At most
 * 65536 blocks per sequence.  fetch_ratio: default
 * cap per (b, KV head) and step = max(1, floor(ratio * K)) (see
 * oasis_cap_from_ratio), used when oasis_select_and_fetch gets cap < 0.
 * Allocates the pinned host KV [B][Hkv][NBmax][K|V][block_size][d], the HBM
 * summaries [B][Hkv][NBmax][max|min][d] and slot pool
 * [B][Hkv][S][K|V][block_size][d], tables and work buffers, and one copy
 * stream at default priority.  On success *out owns all of it.
 * Environment, read here: OASIS_SCORE_IMPL=valu keeps bf16 summaries
 * block-major and scores them on the vector ALU instead of the matrix cores;
 * OASIS_GATHER=stream starts the handle with the fetch outside the attention
 * (as oasis_set_fetch_in_attention(h, 0)); OASIS_ATTN_SPLIT=1 runs the
 * attention over the resident blocks as fixed splits per (b, KV head)
 * instead of runs balanced over all of them (for comparisons). */
int oasis_create(const oasis_layout *layout, int32_t block_size, int32_t budget_tokens,
                 float fetch_ratio, oasis_t **out);

/* Create a handle for a layer whose KV data is identical to owner's, using
 * owner's pinned host KV instead of allocating its own (the host buffer is
 * reference counted and lives until the last handle using it is destroyed).
 * For models whose full host KV exceeds host memory, layers can be aliased
 * onto a few distinct host buffers.  batch, num_kv_heads, head_dim, dtype,
 * block_size and the block capacity (max_tokens rounded up to blocks) must
 * equal owner's, else OASIS_E_INVAL; everything in HBM (summaries, slots,
 * tables) is the new handle's own.  Every handle of a buffer must be given
 * the same appended tokens, since they all write them into the buffer. */
int oasis_create_shared(const oasis_layout *layout, int32_t block_size, int32_t budget_tokens,
                        float fetch_ratio, const oasis_t *owner, oasis_t **out);

/* Wait for all work of the handle, then free everything it owns. */
int oasis_destroy(oasis_t *h);

/* Load a prompt of len tokens per sequence.  k_host, v_host:
 * [B][Hkv][len][d] in the layout's dtype.  Copies them into the pinned host
 * KV, builds every block summary on the GPU (on `stream`) and empties the
 * slot pool; returns once all of it is done (synchronous: the host arrays
 * may be reused at once).
 * len <= max_tokens.  With k_host == v_host == NULL the host KV keeps the
 * prompt the last load wrote into it (OASIS_E_STATE unless that prompt had
 * len tokens) and the handle starts over from it; this is how a handle
 * sharing a buffer gets its prompt.  Either form clears every host row past
 * len that a load or an append wrote, so all handles of a shared buffer must
 * be reloaded before their next step. */
int oasis_load_prefix(oasis_t *h, const void *k_host, const void *v_host, int64_t len,
                      hipStream_t stream);

/* Set the residency tables (synchronous): slot_block_host[B][Hkv][S] (the
 * block each slot holds, -1 = empty) and last_used_host[B][Hkv][S] (the step
 * its block was last used).  The payload of every listed block is copied
 * from the host KV into its slot.  A block held twice, or a block id not
 * below the current block count, is OASIS_E_INVAL. */
int oasis_set_state(oasis_t *h, const int32_t *slot_block_host, const int32_t *last_used_host);

/* Append one token to every sequence: k_dev, v_dev [B][Hkv][d].  Writes it
 * into the host KV, updates its block's max/min summary (a new block starts
 * from this token, non-resident) and, if the block is resident, its slot.
 * OASIS_E_CAPACITY when T == max_tokens. */
int oasis_append_kv(oasis_t *h, const void *k_dev, const void *v_dev, hipStream_t stream);

/* Predict the blocks of this step (OasisKV Fig. 7: the draft queries scan
 * the min/max compressed keys).  q_dev [B][Hq][d] current query, or NULL to
 * predict from the drafts alone (the lookahead ordering of Fig. 8; needs
 * n_drafts >= 1); drafts_dev [n_drafts][B][Hq][d] (may be NULL when n_drafts
 * == 0).  Block score = max over the G query heads of the KV head's group and
 * over {q} + drafts of sum_c max(x_c * max_c, x_c * min_c).  Then per (b, KV head) the top
 * min(K, NB) blocks by (score desc, block id asc), -1 padded, become the
 * selection.  block_ids_dev [B][Hkv][K] and scores_dev [B][Hkv][NBmax]
 * (NBmax = ceil(max_tokens / block_size)) receive copies when non-NULL. */
int oasis_predict(oasis_t *h, const void *q_dev, const void *drafts_dev, int32_t n_drafts,
                  int32_t *block_ids_dev, float *scores_dev, hipStream_t stream);

/* Replace the selection with the top-K of the given fp32 scores
 * [B][Hkv][NBmax] (entries past the current block count are ignored).  A
 * NaN or infinite score sets OASIS_E_NONFINITE in the device error word
 * (oasis_check). */
int oasis_topk_from_scores(oasis_t *h, const float *scores_dev, int32_t *block_ids_dev,
                           hipStream_t stream);

/* Value of oasis_select_and_fetch's `copy` that leaves the host -> HBM copy
 * where the handle puts it (see oasis_set_fetch_in_attention). */
#define OASIS_COPY_DEFAULT ((hipStream_t)(intptr_t)-1)

/* Diff the selection against the resident slots and fetch (OasisKV
 * explanatory diagram, capped-eviction glossary, Table 2).  Per (b, KV head):
 * hits keep their slot; the first min(cap, misses) misses in top-K order are
 * fetched, into empty slots in ascending order first, then into the slots of
 * held non-selected blocks, least recently used first (ties: lower block id);
 * every hit and fetched block gets last_used = this step.  cap < 0 uses the
 * handle's fetch ratio; cap is clamped to K.  The table update runs on
 * `stream` (the compute stream).
 * copy: the stream of the host -> HBM block copies (OasisKV Fig. 8: the
 * transfer on a stream of its own).  A stream: the gather kernel copies the
 * fetched blocks there right after the table update (it waits for `stream`),
 * and the next call that reads the slots (attention, select, evict, verify)
 * waits for it; the copy takes the rows of the tokens held now, so an append
 * (which writes the next token's row) runs beside it.  OASIS_COPY_DEFAULT:
 * the handle's own placement, by default inside the next oasis_sparse_attn's
 * kernel (bf16, d = 128, block 16:
 * fetch waves read the host blocks while the other workgroups attend to the
 * hits, which measured faster than a separate copy the attention waits for),
 * else the handle's copy stream.  A copy left for the attention is made
 * earlier by any call that needs the slots first (evict, select, reading
 * SLOTS, verify); an append in between leaves it pending, and the copy then
 * takes the host block with the appended token. */
int oasis_select_and_fetch(oasis_t *h, int32_t cap, hipStream_t stream, hipStream_t copy);

/* Force blocks out of HBM (synchronous on `stream`): blocks_host
 * [B][Hkv][max_per_unit] block ids, counts_host[B][Hkv] how many of each row
 * to evict.  A listed block that is not resident is ignored.  Slots become
 * empty; last_used is left as it is. */
int oasis_evict(oasis_t *h, const int32_t *blocks_host, const int32_t *counts_host,
                int32_t max_per_unit, hipStream_t stream);

/* Forced non-residency from seeded draws, on the device (asynchronous on
 * `stream`): per (b, KV head), floor(fraction * n) entries of the attended
 * list of the last select (n entries) leave HBM, the entries i whose
 * draws_dev[b][Hkv][i] are smallest (ties: lower i); their slots become
 * empty, last_used is left as it is.  draws_dev [B][Hkv][K] fp64 device
 * memory, 8-byte aligned, i < n read; fraction in [0, 1].  The count is
 * floor(fraction * n + 1e-9) with the product and the sum each rounded.
 * This is the stress of decode-time misses (the OasisKV page lists
 * mispredicted, non-resident blocks among its limits) as a timed-step
 * operation: no host synchronisation, later calls on other streams wait
 * for it.  OASIS_E_STATE before the first select. */
int oasis_evict_attended(oasis_t *h, const double *draws_dev, double fraction,
                         hipStream_t stream);

/* Sparse GQA decode attention over the attended blocks of the last
 * select (the selected blocks that are now resident), for the current query
 * q_dev [B][Hq][d]: out_dev[B][Hq][d] (fp32) = softmax(q.k / sqrt(d)) v over
 * the valid tokens of those blocks; 0 when none is attended. */
int oasis_sparse_attn(oasis_t *h, const void *q_dev, float *out_dev, hipStream_t stream);

/* Verification attention (OasisKV page, Fig. 7 right): the current query
 * and every draft query attend over the sparse KV in one pass, as
 * speculative decoding verifies drafts.  q_dev [B][Hq][d] is
 * the current query (position T-1); drafts_dev [n_drafts][B][Hq][d] the draft
 * queries, draft j at position T-1+j; k_drafts_dev / v_drafts_dev
 * [n_drafts][B][Hkv][d] the draft tokens' keys and values (not appended to
 * the cache).  out_dev [1+n_drafts][B][Hq][d] fp32: set 0 = oasis_sparse_attn
 * of q; set j attends over the attended blocks of the last select (tokens
 * < T) and draft tokens 1..j (causal).  The G (1 + n_drafts) query rows per
 * KV head go through the KV in passes of 32 rows, the last one padded to a
 * power of two (20 rows: one pass); more than 12 passes is OASIS_E_INVAL.
 * Fetches pending from the last select are copied first.  bf16 layouts with
 * d = 128 and block_size 16 only, all pointers 16-byte aligned (OASIS_E_INVAL
 * otherwise); its scratch is allocated with the handle, for max_drafts
 * drafts, and shared by the handle's verify calls, which run in the order
 * they were issued (a call on another stream waits for the last attention or
 * verify). */
int oasis_sparse_attn_verify(oasis_t *h, const void *q_dev, const void *drafts_dev,
                             int32_t n_drafts, const void *k_drafts_dev,
                             const void *v_drafts_dev, float *out_dev, hipStream_t stream);

/* Shape of oasis_sparse_attn_noalloc's inputs. */
typedef struct {
    int32_t batch;           /* B */
    int32_t num_q_heads;     /* Hq, a multiple of Hkv with Hq / Hkv in {1, 2, 4, 8, 16} */
    int32_t num_kv_heads;    /* Hkv */
    int32_t head_dim;        /* 128 */
    int32_t block_size;      /* 16 */
    int32_t list_stride;     /* K: entries per (b, KV head) row of the lists, 1..1024 */
    int32_t slots_per_head;  /* S: block slots per (b, KV head) in the slot pool */
    int32_t reserved;
} oasis_attn_desc;

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid hipMalloc): oasis_sparse_attn over
 * caller-owned buffers, with no handle and no allocation.  Its split-K
 * partials live in an array of device memory that the library holds, one
 * per GPU, for the life of the process: 61,440 partial rows of 130 fp32
 * (31.9 MB).  A call needs G rows for each (b, KV head) and each of its run
 * segments, B * Hkv * G * (K / 8 + 1) rows at full lists of the Qwen3-8B
 * layer shape (17,408 at B = 32, K = 128; up to B * Hkv * G * (K / 2 + 1)
 * for small batches); a shape needing more than the array holds returns
 * OASIS_E_CAPACITY and launches nothing.  Every call on a GPU uses that GPU's one array: calls that overlap
 * in time on one GPU (different streams, no ordering) race and give wrong
 * results; calls ordered on a stream do not (each call writes every row it
 * reads).  Inputs, all bf16 bit patterns or int32, device memory, 16-byte
 * aligned:
 *   q_dev [B][Hq][128]; slots_dev [B][Hkv][S][K|V][16][128] (the slot pool
 *   layout of a handle); att_block_dev / att_slot_dev [B][Hkv][list_stride]:
 *   the attended blocks and the slots holding them; counts_dev [B][Hkv][4]:
 *   element 0 = number of attended entries of the row (the COUNTS layout of a
 *   handle); tokens: the sequence length T (a block's tokens at or past T are
 *   masked).  out_dev [B][Hq][128] fp32 = softmax(q.k / sqrt(128)) v over the
 *   valid tokens of the attended blocks, 0 for an empty list.  Asynchronous on
 *   `stream`; OASIS_E_INVAL for other shapes or null / misaligned pointers. */
int oasis_sparse_attn_noalloc(const oasis_attn_desc *desc, const void *q_dev,
                              const void *slots_dev, const int32_t *att_block_dev,
                              const int32_t *att_slot_dev, const int32_t *counts_dev,
                              int64_t tokens, float *out_dev, hipStream_t stream);

/* ---------------------------------------------------------------- layer pipeline */

typedef struct {
    const void *k_new;   /* [B][Hkv][d] token to append, or NULL: no append */
    const void *v_new;   /* [B][Hkv][d], NULL exactly when k_new is */
    const void *q;       /* [B][Hq][d] current query */
    const void *drafts;  /* [n_drafts][B][Hq][d], or NULL when n_drafts == 0 */
    float *out;          /* [B][Hq][d] fp32 attention output */
} oasis_layer_io;

/* One decode step over the n_layers layers of a model (OasisKV page,
 * Fig. 8: predict, select and transfer per layer, overlapped with compute):
 * per layer, in order, append (when io[l].k_new), predict with the deferred
 * top-K, select_and_fetch(cap) and sparse_attn, with the same semantics as
 * those calls.  With side != stream, append/predict/select of every layer
 * run on `side` and each layer's attention on `stream` after that layer's
 * select, so later layers' prediction and selection overlap earlier layers'
 * attention and host fetch; `stream` then waits for `side` before the call
 * returns.  side == stream runs everything on `stream` one layer after the
 * other.  Both give bit-identical results.  The handles must be distinct.
 * On error no further call is issued (work already queued still runs and
 * `stream` still joins `side`), and oasis_last_error(layers[0]) names the
 * failing layer. */
int oasis_decode_layers(oasis_t *const *layers, const oasis_layer_io *io, int32_t n_layers,
                        int32_t n_drafts, int32_t cap, hipStream_t stream, hipStream_t side);

/* One decode step over the layers in the lookahead order (OasisKV page,
 * Fig. 8: what step t's drafts predict is selected and moved to HBM before
 * that layer attends at step t+1).  Per layer l, in
 * order: on `stream`, append io[l].k_new/v_new (when not NULL) and, when the
 * layer has selected before and io[l].q and io[l].out are not NULL, attend
 * with io[l].q over the set the previous call selected; then on `side`,
 * predict from io[l].drafts alone (n_drafts >= 1) and select_and_fetch(cap);
 * the selected misses are copied host -> HBM on `xfer`.  The next call's
 * attention and select of that layer wait for the copy (its append runs
 * beside it); the call itself does not: `stream` does not wait for `side`
 * or `xfer`, so transfers run under the attention of the following layers
 * (provided the three streams sit on different hardware queues: the HIP
 * runtime spreads a process's streams over a few queues in creation order,
 * and streams sharing one run in order).  Synchronize all three streams (or
 * the device) before reusing the call's inputs.  Call it with every q = NULL
 * and cap = K for the admission step (predict and fetch only).
 * cap_correct > 0 adds decode-time miss correction (the corrective transfers
 * the OasisKV page lists among its limits): before attending, each layer
 * scores its current query alone, selects that top-K with cap_correct (the
 * blocks the earlier prediction missed are fetched synchronously, on
 * `stream`), and attends over it; the drafts' prefetch for the next step
 * follows as above.  cap_correct = 0: attention over the prefetched set.
 * The handles must be distinct; on error no further call is issued and
 * oasis_last_error(layers[0]) names the failing layer. */
int oasis_decode_layers_ahead(oasis_t *const *layers, const oasis_layer_io *io,
                              int32_t n_layers, int32_t n_drafts, int32_t cap,
                              int32_t cap_correct, hipStream_t stream, hipStream_t side,
                              hipStream_t xfer);

/* ---------------------------------------------------------------- inspection */

enum {
    OASIS_BUF_SUMMARY = 0,    /* dtype [B][Hkv][NBmax][2][d] (max, min) */
    OASIS_BUF_SLOTS = 1,      /* dtype [B][Hkv][S][2][bs][d] (K, V) */
    OASIS_BUF_HOST_KV = 2,    /* dtype [B][Hkv][NBmax][2][bs][d] */
    OASIS_BUF_SCORES = 3,     /* f32 [B][Hkv][NBmax] (last oasis_predict) */
    OASIS_BUF_IDS = 4,        /* i32 [B][Hkv][K] selection */
    OASIS_BUF_SLOT_BLOCK = 5, /* i32 [B][Hkv][S] */
    OASIS_BUF_BLOCK_SLOT = 6, /* i32 [B][Hkv][NBmax] */
    OASIS_BUF_LAST_USED = 7,  /* i32 [B][Hkv][S] */
    OASIS_BUF_FETCH_BLOCK = 8,/* i32 [B][Hkv][K] */
    OASIS_BUF_FETCH_SLOT = 9, /* i32 [B][Hkv][K] */
    OASIS_BUF_ATT_BLOCK = 10, /* i32 [B][Hkv][K]: hits (top-K order), then fetched */
    OASIS_BUF_ATT_SLOT = 11,  /* i32 [B][Hkv][K] */
    OASIS_BUF_COUNTS = 12,    /* i32 [B][Hkv][4]: attended, hits, fetched, misses */
    OASIS_BUF_COUNT_
};

/* Size in bytes of an inspection buffer, or a negative status. */
int64_t oasis_buffer_bytes(const oasis_t *h, int32_t which);

/* Copy nbytes at byte offset of an inspection buffer to dst_host, after
 * waiting for all work of the handle (synchronous). */
int oasis_read(oasis_t *h, int32_t which, int64_t offset, int64_t nbytes, void *dst_host);

typedef struct {
    int64_t steps;            /* oasis_select_and_fetch calls */
    int64_t hits;             /* selected blocks found resident */
    int64_t misses;           /* selected blocks not resident */
    int64_t fetched;          /* blocks copied host -> HBM */
    int64_t attended;         /* blocks attended */
    int64_t bytes_fetched;    /* fetched * 2 * block_size * d * elem bytes */
    int64_t tokens;           /* current sequence length T */
    int64_t fetch_fused;      /* 1: blocks are copied host -> HBM inside oasis_sparse_attn's
                                 kernel; 0: by a copy kernel on the handle's copy stream */
} oasis_stats;

/* Residency state after the last call (synchronous; waits for the device).
 * Each pointer may be NULL to skip it; all are host memory owned by the
 * caller.  slot_block [B][Hkv][S]: block held by each slot, -1 empty;
 * last_used [B][Hkv][S]: step its block was last selected or fetched;
 * fetch_list [B][Hkv][K][2]: (block, slot) pairs fetched by the last select,
 * -1 past fetch_n; fetch_n [B][Hkv]; attended [B][Hkv][K]: the attended
 * blocks of the last select (hits in top-K order, then fetched), -1 past
 * their number.  Before any select the lists are all -1 and fetch_n 0. */
int oasis_get_state(oasis_t *h, int32_t *slot_block, int32_t *last_used, int32_t *fetch_list,
                    int32_t *fetch_n, int32_t *attended);

/* Cumulative counters (synchronous). */
int oasis_get_stats(oasis_t *h, oasis_stats *out);

/* Wait for the handle's work and test the device error word: OASIS_OK,
 * OASIS_E_NONFINITE, or OASIS_E_DEVICE (an invariant of the selection
 * failed).  Clears the word. */
int oasis_check(oasis_t *h);

/* Per-kernel GPU time, summed over calls since timing was enabled. */
typedef struct {
    double ms_append, ms_score, ms_topk, ms_select, ms_gather, ms_attn, ms_combine;
    int64_t n_append, n_score, n_topk, n_select, n_gather, n_attn, n_combine;
} oasis_timing;

/* Kernel classes for oasis_set_timing. */
enum {
    OASIS_TIME_APPEND = 1, OASIS_TIME_SCORE = 2, OASIS_TIME_TOPK = 4, OASIS_TIME_SELECT = 8,
    OASIS_TIME_GATHER = 16, OASIS_TIME_ATTN = 32, OASIS_TIME_COMBINE = 64, OASIS_TIME_ALL = 127
};
/* mask != 0: bracket every launch of the kernel classes in mask with HIP
 * events on the stream it runs on; 0 turns timing off.  Resets the sums. */
int oasis_set_timing(oasis_t *h, int32_t mask);
/* Synchronous: read the sums. */
int oasis_get_timing(oasis_t *h, oasis_timing *out);
/* Bracket only one launch in `period` of each timed class with events (the
 * first, then every period-th); the others run as untimed launches.  Events
 * attached to a dispatch cost a few microseconds of the following work, so a
 * period above 1 measures average kernel times with less disturbance of the
 * stream.  Default 1; OASIS_E_INVAL for period < 1.  Does not reset the sums;
 * oasis_set_timing restarts the count. */
int oasis_set_timing_period(oasis_t *h, int32_t period);

/* Attended set (OasisKV page, Fig. 7: attention over the sparse KV working
 * set).  Off (default): the selected blocks held after the step, listed as
 * the hits in top-K order, then the fetched blocks.  On: every block held
 * after the step, listed as the hits, then the held blocks that were neither
 * selected nor evicted (slot order), then the fetched blocks; the two agree
 * when every selected block is held and S = K.  Residency, recency and the
 * fetch are the same either way.  The ATT_BLOCK / ATT_SLOT lists hold K
 * entries per KV head, so on needs S <= K (OASIS_E_INVAL otherwise).  Takes
 * effect at the next oasis_select_and_fetch. */
int oasis_set_attend_all_resident(oasis_t *h, int32_t on);

/* Score + top-K + select fusion (on != 0; off by default).  While on, an
 * oasis_predict that asks for neither ids nor scores is deferred: the next
 * oasis_select_and_fetch scores every block, takes the top-K and selects in
 * one kernel, one workgroup per (b, KV head), the scores staying in LDS (a
 * copy still lands in the SCORES buffer).  Applies to tiled bf16 layouts with
 * d = 128, at least 256 (b, KV head) units and at most 8192 blocks; other
 * shapes run the separate kernels.  While a predict is deferred its q and
 * drafts must stay valid until the select; an oasis_append_kv, or a read of
 * the IDS or SCORES buffer, in between runs the deferred score on its own
 * first.  The results are the same as without fusion. */
int oasis_set_score_topk_fusion(oasis_t *h, int32_t on);

/* Where the blocks chosen by oasis_select_and_fetch are copied host -> HBM
 * (OasisKV explanatory diagram: only the missing blocks are transferred).
 * on != 0: inside the next oasis_sparse_attn's kernel, whose fetch waves read
 * the host link while its other workgroups attend to the resident blocks;
 * the default where the attention runs on the matrix cores (bf16, d = 128,
 * block 16).  on == 0: by the gather kernel on the handle's copy stream right
 * after the select; the attention then waits for the copy.  Selections,
 * tables and slot payloads are the same either way; the attention output
 * differs only by the order of its fp32 split-K merge (inside the attention
 * each fetched block is a partial of its own).  A copy still pending is made
 * before the switch (synchronous).  OASIS_E_INVAL when on is asked for
 * another layout. */
int oasis_set_fetch_in_attention(oasis_t *h, int32_t on);

/* on != 0: when the last oasis_select_and_fetch copied its blocks on a copy
 * stream other than the stream of the next oasis_sparse_attn (and the
 * layout is bf16, d = 128, block 16), that attention starts on the blocks
 * held before the select while the copy runs and waits for the copy only
 * before the fetched blocks (two launches, then the combine), so the copy
 * overlaps the attention instead of preceding it (OasisKV Fig. 8: the
 * transfer beside the compute).  The output equals the one-launch form's up
 * to the order of the floating-point sums.  Default off. */
int oasis_set_attention_beside_copy(oasis_t *h, int32_t on);

/* Shape of a handle: K (top-K blocks), S (slots), NBmax, block size. */
int oasis_get_dims(const oasis_t *h, int32_t *k_blocks, int32_t *slots, int64_t *nb_max,
                   int32_t *block_size);

/* Current number of tokens per sequence. */
int64_t oasis_tokens(const oasis_t *h);

/* The handle's copy stream (gather); for callers that order their own work
 * after it. */
hipStream_t oasis_copy_stream(const oasis_t *h);

/* A stream of the current device (default priority) whose kernels run only
 * on compute units [first_cu, first_cu + n_cus) of the runtime's CU mask
 * (hipExtStreamCreateWithCUMask).  Streams made from disjoint ranges never
 * share a CU.  The OasisKV page puts the host -> HBM transfer on a stream of
 * its own beside the attention (Fig. 8); on this GPU a CU's vector loads
 * return at the pace of its slowest outstanding load, so HBM reads on a CU
 * that also runs host reads wait for the host link's round trip.  Giving the
 * copy stream a few CUs of its own and the compute streams the rest keeps
 * both at full rate.  Like a stream from hipStreamCreate it synchronizes
 * with the null stream, so the other streams of such a schedule should be
 * created streams too.  OASIS_E_INVAL when the range is empty or past the
 * device's CUs, OASIS_E_HIP when the runtime refuses.  Release with
 * oasis_stream_destroy. */
int oasis_stream_create_cus(int32_t first_cu, int32_t n_cus, hipStream_t *out);
int oasis_stream_destroy(hipStream_t stream);

/* ------------------------------------------------------------------ helpers */

/* "KV cache offloading, week 2", section 2: KV bytes per token =
 * layers * 2 * KV heads * head_dim * dtype bytes. */
uint64_t oasis_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                  int32_t dtype_bytes);

/* Measurement helper: read `bytes` of device memory at buf_dev (16-byte
 * aligned, bytes a positive multiple of 16) once, with `workgroups`
 * workgroups (1..65536) of 256 threads streaming 16 KB pieces in turn, on
 * `stream`.  sink_dev [workgroups] receives, per workgroup, the XOR of the
 * 32-bit words it read, so the XOR over sink equals the XOR of the buffer's
 * words.  Timed over a buffer larger than the last-level cache it gives the
 * box's streaming-read rate of HBM, the practical ceiling of the summary
 * scan and of the attention over resident slots.  OASIS_E_INVAL on bad
 * arguments; no handle needed. */
int oasis_stream_read(const void *buf_dev, int64_t bytes, uint32_t *sink_dev, int32_t workgroups,
                      hipStream_t stream);

/* Default per-(b, KV head) cap for a fetch ratio of a K-block budget
 * (OasisKV Table 2 sets the cap by a fetch ratio): max(1, floor(ratio * K))
 * for ratio > 0, 0 for ratio <= 0, K for ratio >= 1. */
int32_t oasis_cap_from_ratio(float ratio, int32_t k_blocks);

const char *oasis_strerror(int status);
const char *oasis_last_error(const oasis_t *h);

#ifdef __cplusplus
}
#endif
#endif /* OASIS_H */
