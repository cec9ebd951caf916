"""Oracle trajectories of one (batch row, KV head) unit of a synthetic workload.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
benchmark).  Inputs come from the shared seeded generator module ``synth``;
the arithmetic is the oracle's own (``oracle/oasis_oracle.c``).

Step order (the decode step of one layer): forced evictions (GQA-8 stress
workload only) -> append one token -> score -> top-K -> select/cap/LRU ->
gather -> attention.  Workloads with admission run an untimed step 0 first:
score the prefix and fetch the whole selection (cap = K) into the empty pool.
"""
from __future__ import annotations

import numpy as np

import synth
from . import Unit, cap_from_ratio, draft_rows, to_f64, unit_rows


def workload_cap(w: synth.Workload) -> int:
    return w.cap if w.cap > 0 else cap_from_ratio(w.fetch_ratio, w.k_blocks)


def initial_unit(w: synth.Workload, b: int, h: int, n_steps: int, layer: int = 0, kv=None):
    T_end = w.prefix_tokens + n_steps
    keys, vals = kv if kv is not None else synth.unit_kv(w, b, h, T_end, layer)
    sb = lu = None
    if w.initial_resident_frac > 0:
        sb_all, lu_all = synth.initial_slots(w, layer)
        sb, lu = sb_all[b, h], lu_all[b, h]
    return Unit(keys, vals, w.dtype, w.block_size, w.prefix_tokens, w.k_blocks, w.n_slots,
                sb, lu)


def run_unit(w: synth.Workload, b: int, h: int, n_steps: int, layer: int = 0, cap=None,
             kv=None, scores32_by_step=None, unit: Unit | None = None):
    """Full trajectory of one unit; returns the list of step records."""
    if unit is None:
        unit = initial_unit(w, b, h, n_steps, layer, kv)
    cap = workload_cap(w) if cap is None else cap
    qf = to_f64(synth.queries(w, layer), w.dtype)
    recs = []
    prev_att = None
    if w.admission:
        x, cur = unit_rows(qf, to_f64(synth.drafts(w, 0, layer), w.dtype), b, h, w.group)
        s = None if scores32_by_step is None else scores32_by_step(0)
        recs.append(unit.step(0, x, cur, w.k_blocks, append=False, scores32=s))
        prev_att = recs[-1]["att_block"]
    for t in range(1, n_steps + 1):
        ev = None
        if w.forced_evict_frac > 0 and prev_att is not None:
            draws = synth.evict_draws(w, t, layer)[b, h]
            ev = synth.forced_evictions(w, prev_att, len(prev_att), draws)
        x, cur = unit_rows(qf, to_f64(synth.drafts(w, t, layer), w.dtype), b, h, w.group)
        s = None if scores32_by_step is None else scores32_by_step(t)
        rec = unit.step(t, x, cur, cap, append=True, evict_blocks=ev, scores32=s)
        rec["evicted"] = ev if ev is not None else np.zeros(0, np.int32)
        recs.append(rec)
        prev_att = rec["att_block"]
    return recs


def run_unit_ahead(w: synth.Workload, b: int, h: int, n_steps: int, layer: int = 0, cap=None,
                   kv=None, unit: Unit | None = None):
    """Lookahead trajectory ([OASIS] Fig. 8) of one unit: an admission step 0
    selects (cap = K) from the step-0 drafts; step t appends token t, attends
    with the step-t query over the set chosen at step t-1, and selects the
    set for step t+1 from the step-t drafts alone."""
    if unit is None:
        unit = initial_unit(w, b, h, n_steps, layer, kv)
    cap = workload_cap(w) if cap is None else cap
    recs = []
    x = draft_rows(to_f64(synth.drafts(w, 0, layer), w.dtype), b, h, w.group)
    recs.append(unit.step_ahead(0, x, None, w.k_blocks, append=False, attend=False))
    for t in range(1, n_steps + 1):
        q = to_f64(synth.query_at(w, t, layer), w.dtype)
        cur = q[b, h * w.group:(h + 1) * w.group]
        x = draft_rows(to_f64(synth.drafts(w, t, layer), w.dtype), b, h, w.group)
        recs.append(unit.step_ahead(t, x, cur, cap))
    return recs


def run_unit_corrected(w: synth.Workload, b: int, h: int, n_steps: int, cap_correct: int,
                       layer: int = 0, cap=None, kv=None, unit: Unit | None = None):
    """Lookahead prefetch plus decode-time miss correction for one unit: the
    admission step prefetches (cap = K) from the step-0 drafts; each step
    then corrects with the current query's exact top-K (cap_correct) before
    attending, and prefetches the next step's set from its drafts (cap)."""
    if unit is None:
        unit = initial_unit(w, b, h, n_steps, layer, kv)
    cap = workload_cap(w) if cap is None else cap
    recs = []
    x = draft_rows(to_f64(synth.drafts(w, 0, layer), w.dtype), b, h, w.group)
    recs.append(unit.step_ahead(0, x, None, w.k_blocks, append=False, attend=False))
    for t in range(1, n_steps + 1):
        q = to_f64(synth.query_at(w, t, layer), w.dtype)
        cur = q[b, h * w.group:(h + 1) * w.group]
        x = draft_rows(to_f64(synth.drafts(w, t, layer), w.dtype), b, h, w.group)
        recs.append(unit.step_corrected(t, cur, cap_correct, x, cap))
    return recs
