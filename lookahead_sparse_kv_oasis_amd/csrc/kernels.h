// Host-side launchers of the liboasis kernels.  Each returns the launch's
// hipError_t; shapes are validated by the C-ABI layer before any launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace oasis {

// Timing events for the next launch: when set, the launch carries them in its
// dispatch packet (start/stop timestamps of the kernel itself, no extra
// packets on the stream).  Set and cleared by the C-ABI layer around one
// launcher call; one thread drives a handle.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

#define OASIS_LAUNCH(kernel, grid, block, lds, stream, ...)                                       \
    do {                                                                                         \
        if (::oasis::g_launch_events.start)                                                      \
            hipExtLaunchKernelGGL(kernel, grid, block, lds, stream,                              \
                                  ::oasis::g_launch_events.start,                                \
                                  ::oasis::g_launch_events.stop, 0, __VA_ARGS__);                \
        else                                                                                     \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                   \
    } while (0)

struct Dims {
    int B, Hq, Hkv, G, d, dtype, bs, K, S;
    int64_t NBmax;
    // Summary layout.  Block-major: [unit][block][max | min][d].  Tiled (bf16
    // with the matrix-core score): per unit, tiles of 32 blocks, each tile
    // [k-step i < d / 8][lane < 64][8 elements], where lane l holds block
    // 32 t + l % 32, maxima for l < 32 and minima for l >= 32, dims 8i..8i+8:
    // the B-operand order of v_mfma_f32_32x32x16_bf16, so one k-step of a
    // tile is one contiguous 1 KB load of a wave.
    bool tiled = false;
    // Attended set: the selected blocks now held (false), or every block held
    // after the step (true; needs S <= K so the list fits K entries).
    bool attend_all = false;
    // Compute units the handle's kernels may occupy (0: every CU of the
    // current device).  Launches are sized to fill this many CUs: where the
    // caller runs the handle on a stream limited to a subset of the CUs, a
    // grid planned for the whole chip would leave part of each launch to a
    // second round.
    int cus = 0;
    int64_t units() const { return (int64_t)B * Hkv; }
    int esize() const { return dtype == kF32 ? 4 : 2; }
    int64_t block_elems() const { return 2LL * bs * d; }  // K and V of one block
    int64_t summ_tiles() const { return (NBmax + 31) / 32; }
    int64_t summ_unit_elems() const { return tiled ? summ_tiles() * 64LL * d : NBmax * 2LL * d; }
};

// Compute units a launch of the handle should fill (Dims::cus, else the
// current device's count).
inline int compute_units(const Dims &D) {
    if (D.cus > 0) return D.cus;
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
        return n;
    return 256;
}

// Element offset of dims [c, c + 8) of the maxima (half 0) or minima (half 1)
// of block j in a unit's summary region (see Dims).
__host__ __device__ inline int64_t summ_offset(bool tiled, int d, int64_t j, int half, int c) {
    if (!tiled) return j * 2LL * d + (int64_t)half * d + c;
    return (j >> 5) * 64LL * d + (int64_t)(c >> 3) * 512 + (int64_t)(half * 32 + (int)(j & 31)) * 8;
}

// Append token `pos` of every sequence (host KV, summary, resident slot).
hipError_t launch_append(const Dims &D, const void *k, const void *v, int64_t pos, void *host_kv,
                         void *summ, const int32_t *block_slot, void *slots, hipStream_t st);

// Summaries of blocks [0, ceil(T/bs)) from the host KV.
hipError_t launch_summary_build(const Dims &D, const void *host_kv, int64_t T, void *summ,
                                hipStream_t st);

// Block scores: the bf16 matrix-core kernel on a tiled summary, the VALU
// kernel on a block-major one.
hipError_t launch_score(const Dims &D, const void *summ, const void *q, const void *drafts,
                        int n_drafts, int64_t NB, float *scores, hipStream_t st);

// Per-unit top-K of scores[unit][0..NB).
hipError_t launch_topk(const Dims &D, const float *scores, int64_t NB, int32_t *ids,
                       int32_t *ids_copy, uint32_t *err, hipStream_t st);

// Diff / cap / LRU per unit.
hipError_t launch_select(const Dims &D, const int32_t *ids, int32_t *slot_block,
                         int32_t *last_used, int32_t *block_slot, int cap, int32_t t,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *att_block,
                         int32_t *att_slot, int32_t *counts, DevStats *stats, uint32_t *err,
                         hipStream_t st);

// Copy listed blocks from the host KV into their slots, the rows of tokens
// < T only.  Unit u copies n = counts[u * count_stride + count_index] entries
// of (blocks, slots)[u * list_stride ...].  max_n bounds n for the grid.
hipError_t launch_gather(const Dims &D, const void *host_kv, void *slots, const int32_t *blocks,
                         const int32_t *slot_ids, int list_stride, const int32_t *counts,
                         int count_stride, int count_index, int max_n, int64_t T,
                         hipStream_t st);

// Top-K and diff / cap / LRU of every unit in one kernel (the ids are also
// written to ids).
// Score, top-K and select fused in one workgroup per unit (tiled bf16
// summaries, d = 128, at least as many units as compute units, NB <= 8192);
// score_topk_fusable says whether a shape qualifies.
bool score_topk_fusable(const Dims &D, int64_t NB, int n_rows);
hipError_t launch_score_topk_select(const Dims &D, const void *summ, const void *q,
                                    const void *drafts, int n_drafts, int64_t NB, float *scores,
                                    int32_t *ids, int32_t *slot_block, int32_t *last_used,
                                    int32_t *block_slot, int cap, int32_t t,
                                    int32_t *fetch_block, int32_t *fetch_slot,
                                    int32_t *att_block, int32_t *att_slot, int32_t *counts,
                                    DevStats *stats, uint32_t *err, hipStream_t st);

hipError_t launch_topk_select(const Dims &D, const float *scores, int64_t NB, int32_t *ids,
                              int32_t *slot_block, int32_t *last_used, int32_t *block_slot,
                              int cap, int32_t t, int32_t *fetch_block, int32_t *fetch_slot,
                              int32_t *att_block, int32_t *att_slot, int32_t *counts,
                              DevStats *stats, uint32_t *err, hipStream_t st);

// Forced non-residency: unit u drops blocks[u * max_per_unit + i], i < counts[u].
hipError_t launch_evict(const Dims &D, const int32_t *blocks, const int32_t *counts,
                        int max_per_unit, int32_t *slot_block, int32_t *block_slot,
                        hipStream_t st);

// Forced non-residency from seeded draws [units][K]: unit u empties the slots
// of floor(fraction * n_att) entries of its attended list, those with the
// smallest draws (ties to the lower position).  K <= 1024.
hipError_t launch_evict_attended(const Dims &D, const double *draws, double fraction,
                                const int32_t *att_block, const int32_t *counts,
                                int32_t *slot_block, int32_t *block_slot, hipStream_t st);

// Rebuild block_slot from slot_block (after oasis_set_state).
hipError_t launch_rebuild_block_slot(const Dims &D, const int32_t *slot_block,
                                     int32_t *block_slot, hipStream_t st);

// Split-K sparse attention partials and their combination.  Partials of a
// unit are indexed [0, nsa): fetch splits at [0, nsf), hit splits at
// [nsf_max, nsf_max + ns1).
struct AttnPlan {
    bool mfma;             // bf16, d = 128, block 16, G in {1, 2, 4, 8, 16}, or 32 when flat
    int blocks_per_wave;   // hit entries per wave (MFMA: 4 waves per split)
    int ns1;               // hit splits per unit (split kernel; verification attention)
    int nsf_max;           // fetch splits per unit at cap = K (MFMA only)
    int nsa;               // partial stride per unit
    // Balanced hit path (MFMA layouts whose units fit its LDS prefix sums):
    // flat_waves waves stream equal runs (at least flat_pmin entries) of all
    // units' hit entries and write their partials after the per-unit region,
    // flat_rows per unit.
    bool flat;
    int flat_waves, flat_pmin, flat_rows;
    // Query rows per unit in the kernels and the partials (the row stride of
    // the partial buffers): G, or 16 where the balanced kernel runs G = 8 on
    // the 16-row matrix-core tile (rows past G repeat row 0, their partials
    // unwritten).
    int gt;
    // verification attention: partial rows per (unit, query row) of its
    // buffers (at least the split and balanced strides of every chunk size)
    int vns;
};
AttnPlan plan_attention(const Dims &D);
// Rows (G floats of m and l, G x d of acc each) of the partial buffers.
int64_t attn_partial_rows(const Dims &D, const AttnPlan &P);
// Fetch splits for a cap (fused mode), 0 when the kernel cannot fuse.
int attention_fetch_splits(const Dims &D, const AttnPlan &P, int cap);
// Where the matrix-core attention kernels take the query rows of a unit.
// Row r of a pass over G_pass rows is the unit's query row r0 + r (r0 again
// for r >= real, whose partials are not written); query row j G + g of unit
// (b, h) is head h G + g of query set j: q [B][Hq][d] for j = 0, drafts set
// j - 1 ([n][B][Hq][d], set_stride elements apart) for j >= 1.  The decode
// attention's rows are {q, -, -, Hq, G, 0, G}.
struct QRows {
    const uint16_t *q, *drafts;
    int64_t set_stride;
    int Hq, G;
    int r0, real;
};
// mode 0: every attended entry from its slot.  mode 1 (MFMA only): entries
// [n_hit, n_att) are read from the host KV and written into their slots in
// the same kernel, using nsf fetch splits.  Balanced plans only: mode 2, the
// entries [0, n_hit) alone; mode 3, entries [n_hit, n_att) alone, from their
// slots (into the nsf fetch splits, as mode 1 writes them), so that a mode-2
// launch can run while a gather on another stream fills the slots and a
// mode-3 launch after it.  launch_combine merges the partials into the
// output.  qr (MFMA only; null: the rows of q) gives the
// query rows of a verification pass.
hipError_t launch_attention(const Dims &D, const AttnPlan &P, int mode, int nsf, const void *q,
                            void *slots, const void *host_kv, const int32_t *att_block,
                            const int32_t *att_slot, const int32_t *counts, int64_t T,
                            float *part_m, float *part_l, float *part_acc, hipStream_t st,
                            const QRows *qr = nullptr);
// Partial rows per (unit, query row) the verification attention's buffers
// need for every chunk size.
int verify_stride(const Dims &D);
// Verification attention (normal and draft query sets together, causal over
// the draft tokens): query rows per unit padded to whole passes (-1 when they
// need more than 12 passes), and the whole call (one block attention per
// chunk of rows, combine).  bf16, d = 128, bs = 16.
int verify_rows(const Dims &D, int n_drafts);
hipError_t launch_verify(const Dims &D, const AttnPlan &P, int n_drafts, const void *q,
                         const void *drafts, const void *kd, const void *vd, void *slots,
                         const int32_t *att_block, const int32_t *att_slot,
                         const int32_t *counts, int64_t T, float *vpart_m, float *vpart_l,
                         float *vpart_acc, float *out, hipStream_t st);

hipError_t launch_combine(const Dims &D, const AttnPlan &P, int nsf, const float *part_m,
                          const float *part_l, const float *part_acc, float *out,
                          hipStream_t st);

}  // namespace oasis
