/*
 * OasisKV decode-step oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; the product
 * path never calls it.
 *
 * Sources (cited by page title and figure/table/section):
 *   [OASIS]  "OasisKV: Scaling In-Decode KV Cache Beyond HBM with Lookahead
 *            Sparse Prefetching" (METAL MEDIA explainer of arXiv:2608.08097):
 *            Fig. 7 (compressed keys by per-block min/max pooling, draft
 *            query scans them for the next top-K, sparse KV working set),
 *            Fig. 8 (predict -> select -> transfer per layer), Fig. 9
 *            (head-wise GPU-block -> CPU-block table), Table 2 (fetch cap by
 *            fetch ratio, LRU eviction), the explanatory diagram (compare the
 *            predicted blocks with those on the GPU, cap the per-step
 *            transfer) and the glossary entry on capped eviction (bound the
 *            number of blocks newly loaded in one step).
 *   [KVW2]   "KV cache offloading, week 2" study notes (youwins-lab blog):
 *            section 2 (bytes per token = layers x 2 x KV heads x head dim x
 *            dtype bytes) and section 3 (GQA groups, PagedAttention blocks).
 *
 * Every unit of work is one (batch row, KV head) pair; units are independent.
 * Inputs are the storage arrays (fp32, or bf16 as raw uint16 bits), each
 * element converted exactly to double.  All arithmetic is fp64.
 *
 * Readings of points the pages leave open (listed with reasons in the design
 * notes) are marked READING below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------------ input */

/* Exact value of element i of a storage array: fp32, or bf16 = the upper
 * 16 bits of an IEEE binary32. */
static double elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[i];
    uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------- KV sizes */

/* [KVW2] section 2: KV bytes per token of a model. */
uint64_t orc_kv_bytes_per_token(int64_t layers, int64_t kv_heads, int64_t head_dim,
                                int64_t dtype_bytes)
{
    return (uint64_t)layers * 2u * (uint64_t)kv_heads * (uint64_t)head_dim *
           (uint64_t)dtype_bytes;
}

/* ------------------------------------------------------- block summary */

/* [OASIS] Fig. 7: per-block min/max pooling of the keys.
 * keys: [T][d] storage array of one unit.  Block j covers the valid tokens
 * p in [j*bs, min((j+1)*bs, T)) (READING: a partial tail block is pooled over
 * its valid tokens only).  mx[c] / mn[c] = max / min over those tokens of
 * k[p][c].  Strict comparisons in token order keep the first of equal
 * values, which fixes the sign of a zero.  Returns 0, or -1 if the block has
 * no valid token. */
int orc_block_summary(const void *keys, int dtype, int64_t T, int d, int bs, int64_t j,
                      double *mx, double *mn)
{
    int64_t p0 = j * bs, p1 = (j + 1) * bs;
    if (p1 > T)
        p1 = T;
    if (p0 >= p1)
        return -1;
    for (int c = 0; c < d; ++c) {
        double hi = elem(keys, dtype, p0 * d + c), lo = hi;
        for (int64_t p = p0 + 1; p < p1; ++p) {
            double x = elem(keys, dtype, p * d + c);
            if (x > hi)
                hi = x;
            if (x < lo)
                lo = x;
        }
        mx[c] = hi;
        mn[c] = lo;
    }
    return 0;
}

/* ---------------------------------------------------------------- score */

/* [OASIS] Fig. 7: the next step's top-K blocks are predicted from the
 * min/max-pooled key summaries, scored against the draft queries.
 * READING (score rule): the block score for one query row x is the largest
 * value x.k can take over the block's per-dimension box [mn, mx], i.e.
 * sum_c max(x_c*mx_c, x_c*mn_c).
 * READING (aggregation): the score of a block is the maximum of that bound
 * over all query rows given: the G query heads of the KV head's group, for
 * the current query and every draft.
 * mx, mn: [nb][d]; x: [nq][d]; out: s[nb]. */
void orc_score(const double *mx, const double *mn, int64_t nb, int d, const double *x,
               int nq, double *s)
{
    for (int64_t j = 0; j < nb; ++j) {
        double best = -INFINITY;
        for (int r = 0; r < nq; ++r) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) {
                double a = x[(int64_t)r * d + c] * mx[j * d + c];
                double b = x[(int64_t)r * d + c] * mn[j * d + c];
                acc += (a > b) ? a : b;
            }
            if (acc > best)
                best = acc;
        }
        s[j] = best;
    }
}

/* ----------------------------------------------------------------- top-K */

typedef struct {
    float s;
    int32_t id;
} scored_t;

/* Order for the top-K: higher score first; among equal scores the lower
 * block id first (READING: ties go to the lower block index).  -0 and +0
 * compare equal as floats do. */
static int by_score_desc_id_asc(const void *pa, const void *pb)
{
    const scored_t *a = pa, *b = pb;
    if (a->s > b->s)
        return -1;
    if (a->s < b->s)
        return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

/* [OASIS] explanatory diagram and Fig. 7: top-K block prediction under a
 * fixed token budget (2,048 tokens = K blocks of the block size).
 * s: fp32 scores of blocks 0..nb-1.  ids[0..k-1] receives the min(k, nb)
 * best block ids in (score desc, id asc) order, then -1 padding.
 * Returns 0, or -1 if a score is NaN or infinite. */
int orc_topk(const float *s, int64_t nb, int k, int32_t *ids)
{
    for (int64_t j = 0; j < nb; ++j)
        if (!isfinite(s[j]))
            return -1;
    scored_t *v = malloc((size_t)(nb > 0 ? nb : 1) * sizeof *v);
    if (!v)
        return -2;
    for (int64_t j = 0; j < nb; ++j) {
        v[j].s = s[j];
        v[j].id = (int32_t)j;
    }
    qsort(v, (size_t)nb, sizeof *v, by_score_desc_id_asc);
    for (int i = 0; i < k; ++i)
        ids[i] = (i < nb) ? v[i].id : -1;
    free(v);
    return 0;
}

/* --------------------------------------------------- select / cap / LRU */

typedef struct {
    int32_t last_used;
    int32_t block;
    int32_t slot;
} victim_t;

/* Least recently used first; equal recency -> lower block id first. */
static int by_lru(const void *pa, const void *pb)
{
    const victim_t *a = pa, *b = pb;
    if (a->last_used != b->last_used)
        return (a->last_used < b->last_used) ? -1 : 1;
    return (a->block < b->block) ? -1 : (a->block > b->block);
}

/* [OASIS] explanatory diagram: compare the predicted blocks with the blocks
 * already on the GPU and move only the missing ones, capping the per-step
 * transfer; glossary (capped eviction): bound the blocks newly loaded in one
 * step; Table 2: the cap is set by a fetch ratio, eviction is LRU; Fig. 9:
 * a per-KV-head table maps each GPU block (slot) to a CPU block.
 *
 * State of one unit: slot_block[S] (CPU block held by each HBM slot, -1 =
 * empty) and last_used[S] (step at which the slot's block was last selected
 * or fetched).  ids[0..K-1]: this step's selection in top-K order, -1 padded.
 *
 * Step t:
 *   hits H   = selected blocks already held by a slot (top-K order);
 *   misses M = selected blocks not held (top-K order);
 *   n        = min(cap, |M|): READING, the first n misses in top-K order
 *              (the highest-scoring ones) are fetched;
 *   slots    = empty slots in ascending index first, then victims: held
 *              blocks that are not selected, least recently used first,
 *              ties to the lower block id (READING: only non-selected blocks
 *              are evictable; recency is refreshed when a block is selected
 *              while held or fetched);
 *   last_used = t for every hit and every fetched block.
 * Outputs: fetch_block/fetch_slot[0..n-1]; the attended list (READING: the
 * attention runs over the selected blocks now held) = hits in top-K order
 * followed by the fetched blocks, as block ids and their slots.
 * attend_all != 0 takes the other reading of the attended set, every block
 * held after the step: the hits, then the held blocks that were not
 * selected (kept, not evicted) in slot order, then the fetched blocks;
 * att_block / att_slot then need room for max(K, S) entries.  Residency and
 * recency are the same under both readings.
 * Returns 0, or -1 on an invalid state (a block held twice, not enough
 * slots). */
int orc_select(int32_t *slot_block, int32_t *last_used, int S, const int32_t *ids, int K,
               int cap, int32_t t, int32_t *fetch_block, int32_t *fetch_slot, int32_t *n_fetch,
               int32_t *att_block, int32_t *att_slot, int32_t *n_att, int32_t *n_hit,
               int attend_all)
{
    int32_t *hit_slot = malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    int32_t *miss = malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    int32_t *cand = malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    victim_t *vict = malloc(sizeof(victim_t) * (size_t)(S > 0 ? S : 1));
    int rc = 0;
    if (!hit_slot || !miss || !cand || !vict) {
        rc = -2;
        goto out;
    }
    /* a block may be held by at most one slot */
    for (int a = 0; a < S; ++a)
        for (int b = a + 1; b < S; ++b)
            if (slot_block[a] >= 0 && slot_block[a] == slot_block[b]) {
                rc = -1;
                goto out;
            }

    int nh = 0, nm = 0;
    for (int i = 0; i < K; ++i) {
        if (ids[i] < 0)
            continue;
        int found = -1;
        for (int s = 0; s < S; ++s)
            if (slot_block[s] == ids[i])
                found = s;
        if (found >= 0) {
            att_block[nh] = ids[i];
            hit_slot[nh++] = found;
        } else {
            miss[nm++] = ids[i];
        }
    }
    int n = (nm < cap) ? nm : cap;
    if (n < 0)
        n = 0;

    /* slots to fill: empty ones first (ascending), then LRU victims */
    int nc = 0, nv = 0;
    for (int s = 0; s < S; ++s)
        if (slot_block[s] < 0)
            cand[nc++] = s;
    for (int s = 0; s < S; ++s) {
        if (slot_block[s] < 0)
            continue;
        int selected = 0;
        for (int i = 0; i < K; ++i)
            if (ids[i] >= 0 && ids[i] == slot_block[s])
                selected = 1;
        if (!selected) {
            vict[nv].last_used = last_used[s];
            vict[nv].block = slot_block[s];
            vict[nv].slot = s;
            ++nv;
        }
    }
    qsort(vict, (size_t)nv, sizeof *vict, by_lru);
    for (int i = 0; i < nv; ++i)
        cand[nc++] = vict[i].slot;
    if (nc < n) {
        rc = -1;
        goto out;
    }

    for (int i = 0; i < nh; ++i) {
        last_used[hit_slot[i]] = t;
        att_slot[i] = hit_slot[i];
    }
    for (int i = 0; i < n; ++i) {
        int s = cand[i];
        slot_block[s] = miss[i];
        last_used[s] = t;
        fetch_block[i] = miss[i];
        fetch_slot[i] = s;
    }
    int na = nh;
    if (attend_all) {
        for (int s = 0; s < S; ++s) {
            if (slot_block[s] < 0)
                continue;
            int listed = 0;
            for (int i = 0; i < nh; ++i)
                if (hit_slot[i] == s)
                    listed = 1;
            for (int i = 0; i < n; ++i)
                if (cand[i] == s)
                    listed = 1;
            if (!listed) {
                att_block[na] = slot_block[s];
                att_slot[na] = s;
                ++na;
            }
        }
    }
    for (int i = 0; i < n; ++i) {
        att_block[na + i] = miss[i];
        att_slot[na + i] = cand[i];
    }
    *n_fetch = n;
    *n_hit = nh;
    *n_att = na + n;
out:
    free(hit_slot);
    free(miss);
    free(cand);
    free(vict);
    return rc;
}

/* ------------------------------------------------------------- attention */

/* [OASIS] Fig. 7: attention over the sparse KV working set; [KVW2] section 3:
 * under GQA a group of query heads shares one KV head.
 * q: [nq][d] query rows of one KV head's group (already exact doubles);
 * keys / vals: [T][d] storage arrays of the unit; blocks[0..nblocks-1]: the
 * attended block ids.  For each row, over the valid tokens p of the attended
 * blocks: w_p = softmax_p(q.k_p / sqrt(d)) (max-subtracted), out = sum w_p v_p.
 * READING: scale 1/sqrt(d), no other logit transform.  An empty attended set
 * gives out = 0. */
void orc_attention(const double *q, int nq, const void *keys, const void *vals, int dtype,
                   int d, int bs, int64_t T, const int32_t *blocks, int nblocks, double *out)
{
    int64_t ntok = 0;
    for (int i = 0; i < nblocks; ++i) {
        int64_t p0 = (int64_t)blocks[i] * bs, p1 = p0 + bs;
        if (p1 > T)
            p1 = T;
        if (p1 > p0)
            ntok += p1 - p0;
    }
    int64_t *pos = malloc(sizeof(int64_t) * (size_t)(ntok > 0 ? ntok : 1));
    double *logit = malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
    int64_t n = 0;
    for (int i = 0; i < nblocks; ++i) {
        int64_t p0 = (int64_t)blocks[i] * bs, p1 = p0 + bs;
        if (p1 > T)
            p1 = T;
        for (int64_t p = p0; p < p1; ++p)
            pos[n++] = p;
    }
    double scale = 1.0 / sqrt((double)d);
    for (int r = 0; r < nq; ++r) {
        double *o = out + (int64_t)r * d;
        for (int c = 0; c < d; ++c)
            o[c] = 0.0;
        if (n == 0)
            continue;
        double m = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
                acc += q[(int64_t)r * d + c] * elem(keys, dtype, pos[i] * d + c);
            logit[i] = acc * scale;
            if (logit[i] > m)
                m = logit[i];
        }
        double z = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            double w = exp(logit[i] - m);
            z += w;
            for (int c = 0; c < d; ++c)
                o[c] += w * elem(vals, dtype, pos[i] * d + c);
        }
        for (int c = 0; c < d; ++c)
            o[c] /= z;
    }
    free(pos);
    free(logit);
}

/* Dense attention over all T tokens, coded separately from orc_attention
 * (two passes: log-sum-exp normaliser first, then normalised weights).  Used
 * only to check that sparse attention over every block equals dense
 * attention. */
void orc_dense_attention(const double *q, int nq, const void *keys, const void *vals,
                         int dtype, int d, int64_t T, double *out)
{
    double scale = 1.0 / sqrt((double)d);
    double *l = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int r = 0; r < nq; ++r) {
        const double *qr = q + (int64_t)r * d;
        double *o = out + (int64_t)r * d;
        for (int64_t p = 0; p < T; ++p) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
                acc += qr[c] * elem(keys, dtype, p * d + c);
            l[p] = acc * scale;
        }
        double hi = -INFINITY;
        for (int64_t p = 0; p < T; ++p)
            hi = fmax(hi, l[p]);
        double sum = 0.0;
        for (int64_t p = 0; p < T; ++p)
            sum += exp(l[p] - hi);
        double lse = hi + log(sum);
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t p = 0; p < T; ++p)
                acc += exp(l[p] - lse) * elem(vals, dtype, p * d + c);
            o[c] = (T > 0) ? acc : 0.0;
        }
    }
    free(l);
}
