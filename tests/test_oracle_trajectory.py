"""Whole-trajectory invariants of the oracle on the tiny workload and on
reduced-size versions of the bf16 workloads (CPU only, seconds)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.trajectory import run_unit, workload_cap


def _check_traj(w, recs, n_steps):
    cap = workload_cap(w)
    prev_sb = None
    for r in recs:
        t = r["t"]
        c = w.k_blocks if t == 0 else cap
        sel = [i for i in r["ids"] if i >= 0]
        assert len(sel) == min(w.k_blocks, (r["T"] + w.block_size - 1) // w.block_size)
        assert len(r["fetch_block"]) <= c
        held = [b for b in r["slot_block"] if b >= 0]
        assert len(held) == len(set(held)) and len(held) <= w.n_slots
        assert sorted(r["att_block"]) == sorted(b for b in sel if b in held)
        assert np.all(r["last_used"][r["att_slot"]] == t)
        if prev_sb is not None:
            ev = set(r.get("evicted", []))
            prev_held = {b for b in prev_sb if b >= 0} - ev
            for b in sel:                                    # a held selected block stays
                if b in prev_held:
                    assert b in held
        prev_sb = r["slot_block"]
    assert recs[-1]["t"] == n_steps


@pytest.mark.parametrize("h", [0, 1])
def test_tiny_trajectory_invariants(h):
    w = synth.TINY
    recs = run_unit(w, 0, h, w.steps)
    _check_traj(w, recs, w.steps)
    # the first step appends token 1024, which opens block 64 with one token
    assert recs[0]["T"] == 1025
    assert len(recs) == w.steps


def test_admission_fills_the_pool_with_the_first_selection():
    w = synth.QWEN3_8B.with_(batch=2, prefix_tokens=16 * 300 + 5, budget_tokens=16 * 32)
    recs = run_unit(w, 1, 3, 3)
    r0 = recs[0]
    assert r0["t"] == 0 and r0["T"] == w.prefix_tokens
    assert list(r0["slot_block"]) == list(r0["ids"])      # free slots in ascending order
    assert np.all(r0["last_used"] == 0)
    assert list(r0["att_block"]) == list(r0["ids"])
    _check_traj(w, recs, 3)


def test_forced_evictions_leave_holes_that_are_refilled():
    w = synth.QWEN3_32B.with_(batch=1, prefix_tokens=16 * 200, budget_tokens=16 * 20)
    recs = run_unit(w, 0, 5, 6)
    _check_traj(w, recs, 6)
    for i in range(1, len(recs)):
        n_prev = len(recs[i - 1]["att_block"])
        assert len(recs[i]["evicted"]) == int(np.floor(0.1 * n_prev + 1e-9)) > 0


def test_evict_empties_the_slots_and_the_next_select_refills_them_first():
    """Unit.evict, pinned by a hand-worked case (R8: empty slots are filled
    first, in ascending order, before any LRU victim).  Four slots hold blocks
    5, 2, 7, 9 with recency 3, 1, 2, 0.  Evicting 2 and 9 empties slots 1 and
    3 and leaves recency alone.  Selecting [11, 12, 13, 5] with cap 3 then
    fetches 11 -> slot 1 and 12 -> slot 3 (the holes, ascending), and 13 ->
    slot 2, the least recent held block not selected (7 at step 2; 5 is a
    hit).  A no-op evict would hand slot 1 to the LRU victim 2 instead."""
    w = synth.TINY.with_(prefix_tokens=16 * 14, budget_tokens=16 * 4, slots=4,
                         initial_resident_frac=0.0)
    keys, vals = synth.unit_kv(w, 0, 0, w.prefix_tokens)
    unit = oracle.Unit(keys, vals, w.dtype, w.block_size, w.prefix_tokens, 4, 4,
                       slot_block=[5, 2, 7, 9], last_used=[3, 1, 2, 0])
    unit.evict(np.array([2, 9], np.int32))
    assert unit.slot_block.tolist() == [5, -1, 7, -1]
    assert unit.last_used.tolist() == [3, 1, 2, 0]
    unit.evict(np.array([4], np.int32))          # not held: nothing changes
    assert unit.slot_block.tolist() == [5, -1, 7, -1]
    r = oracle.select(unit.slot_block, unit.last_used, np.array([11, 12, 13, 5], np.int32), 3, 4)
    assert r["fetch_block"].tolist() == [11, 12, 13]
    assert r["fetch_slot"].tolist() == [1, 3, 2]
    assert r["att_block"].tolist() == [5, 11, 12, 13] and r["n_hit"] == 1
    assert unit.slot_block.tolist() == [5, 11, 13, 12]
    assert unit.last_used.tolist() == [4, 4, 4, 4]


def test_forced_evictions_are_gone_at_the_next_select():
    """Along the GQA-8 stress trajectory, every forced-out block is absent
    when the next select runs: if it is held after that step, the step fetched
    it again (it is in the fetch list, not among the hits), and the evicted
    blocks' slots are empty slots, which the select fills first."""
    w = synth.QWEN3_32B.with_(batch=1, prefix_tokens=16 * 200, budget_tokens=16 * 20)
    recs = run_unit(w, 0, 5, 8)
    seen = 0
    for i in range(1, len(recs)):
        ev = set(int(b) for b in recs[i]["evicted"])
        assert ev
        prev_sb = recs[i - 1]["slot_block"]
        holes = sorted(int(s) for s in np.nonzero(np.isin(prev_sb, list(ev)))[0])
        # empty at the select: the new holes and any slot a capped step left empty
        empty = sorted(set(holes) | set(int(s) for s in np.nonzero(prev_sb < 0)[0]))
        hits = set(int(b) for b in recs[i]["att_block"][:recs[i]["n_hit"]])
        fetched = [int(b) for b in recs[i]["fetch_block"]]
        assert not (ev & hits), f"step {i}: an evicted block counted as a hit"
        for b in ev:
            if b in recs[i]["slot_block"]:
                assert b in fetched
        # the first fetches go to the empty slots, ascending, holes included
        nf = len(fetched)
        assert [int(s) for s in recs[i]["fetch_slot"][:min(nf, len(empty))]] == \
            empty[:min(nf, len(empty))]
        assert len(holes) == len(ev)   # every forced-out block was held
        seen += len(ev & set(fetched))
    assert seen > 0   # some evicted blocks were selected again and re-fetched


def test_fetch_all_equals_dense_attention_when_budget_covers_context():
    """Budget >= context and an uncapped fetch: every block is attended, so the
    sparse output is dense attention over the whole context."""
    w = synth.TINY.with_(prefix_tokens=16 * 6 + 3, budget_tokens=16 * 8, slots=8, cap=8,
                         initial_resident_frac=0.0)
    unit = None
    recs = run_unit(w, 0, 1, 4, cap=8, unit=unit)
    keys, vals = synth.unit_kv(w, 0, 1, w.prefix_tokens + 4)
    q = oracle.to_f64(synth.queries(w), w.dtype)[0, 2:4]
    for r in recs:
        dense = oracle.dense_attention(q, keys, vals, w.dtype, r["T"])
        assert np.max(np.abs(r["out"] - dense)) < 1e-12


def test_drafts_redrawn_query_fixed():
    w = synth.QWEN3_8B.with_(batch=1)
    d1, d2 = synth.drafts(w, 1), synth.drafts(w, 2)
    assert not np.array_equal(d1, d2)
    assert np.array_equal(synth.queries(w), synth.queries(w))


def test_unit_kv_prefix_property():
    w = synth.LLAMA31_8B_LONG.with_(batch=1)
    a = synth.unit_kv(w, 0, 2, 1000)
    b = synth.unit_kv(w, 0, 2, 1200)
    assert np.array_equal(a[0], b[0][:1000]) and np.array_equal(a[1], b[1][:1000])


# ------------------------------------------------------------------ lookahead ordering

def _ahead_small(**kw):
    return synth.QWEN3_8B_AHEAD.with_(batch=1, prefix_tokens=16 * 6 + 14, budget_tokens=16 * 16,
                                      **kw)


def test_lookahead_attends_the_previous_steps_selection():
    """Fig. 8 ordering: step t's attention runs over exactly the blocks that
    step t-1 selected, and a capped step never fetches more than the cap."""
    from oracle.trajectory import run_unit_ahead
    w = synth.QWEN3_8B_AHEAD.with_(batch=1, prefix_tokens=16 * 300 + 5, budget_tokens=16 * 32)
    recs = run_unit_ahead(w, 0, 5, 8)
    assert recs[0]["out"] is None and len(recs[0]["attended"]) == 0
    for prev, r in zip(recs, recs[1:]):
        assert np.array_equal(r["attended"], prev["att_block"])
        assert len(r["fetch_block"]) <= workload_cap(w)
        held = set(int(b) for b in r["slot_block"] if b >= 0)
        # the set attended at step t+1 is held after step t's select
        assert set(int(b) for b in r["att_block"]) <= held


def test_lookahead_with_whole_context_budget_is_dense_attention_minus_the_newest_block():
    """Budget and cap covering every block: the attended set at step t is every
    block that existed at step t-1.  When token t lands in an existing block
    that is the whole context (dense attention over T tokens); when token t
    opens a new block, that block was not there to be predicted, so the output
    is dense attention over the first T - 1 tokens."""
    from oracle.trajectory import run_unit_ahead
    w = _ahead_small(cap=16)
    n = 6
    recs = run_unit_ahead(w, 0, 2, n, cap=16)
    keys, vals = synth.unit_kv(w, 0, 2, w.prefix_tokens + n)
    opened = 0
    for r in recs[1:]:
        q = oracle.to_f64(synth.query_at(w, r["t"]), w.dtype)[0, 2 * w.group:3 * w.group]
        T = r["T"]
        new_block = (T - 1) % w.block_size == 0
        opened += new_block
        dense = oracle.dense_attention(q, keys, vals, w.dtype, T - 1 if new_block else T)
        assert np.max(np.abs(r["out"] - dense)) < 1e-12
    assert opened >= 1   # the prompt ends 2 tokens before a block boundary


def test_lookahead_query_drift_and_drafts_follow_the_next_query():
    """The lookahead workload's queries drift between steps and its drafts are
    centred on the next step's query (so they predict it better than the
    previous query does)."""
    w = synth.QWEN3_8B_AHEAD.with_(batch=2)
    f = lambda a: synth.decode_f32(a, w.dtype).astype(np.float64)
    q = [f(synth.query_at(w, t)) for t in range(4)]
    d1 = f(synth.drafts(w, 1))
    assert np.array_equal(q[0], f(synth.queries(w)))
    assert 0.15 < np.std(q[2] - q[1]) < 0.3
    assert np.std(d1 - q[2][None]) < 0.5 * np.std(q[1] - q[2])
    # non-lookahead workloads keep a fixed query
    w0 = synth.QWEN3_8B.with_(batch=2)
    assert np.array_equal(synth.query_at(w0, 5), synth.queries(w0))


# ------------------------------------------------------------------ decode-time miss correction

def test_correction_with_whole_context_budget_is_dense_attention():
    """Budget covering every block and an unbounded correction: the corrected
    set is every block, so the output is dense attention over all T tokens
    (the newest block included, unlike the plain lookahead order)."""
    from oracle.trajectory import run_unit_corrected
    w = _ahead_small(cap=2)
    n = 6
    recs = run_unit_corrected(w, 0, 1, n, cap_correct=16, cap=2)
    keys, vals = synth.unit_kv(w, 0, 1, w.prefix_tokens + n)
    for r in recs[1:]:
        q = oracle.to_f64(synth.query_at(w, r["t"]), w.dtype)[0, w.group:2 * w.group]
        dense = oracle.dense_attention(q, keys, vals, w.dtype, r["T"])
        assert np.max(np.abs(r["out"] - dense)) < 1e-12
        assert len(r["correction"]["att_block"]) == (r["T"] + 15) // 16


def test_correction_fetches_at_most_its_cap_and_attends_the_exact_hits():
    """The corrective select fetches at most cap_correct of the exact top-K's
    missing blocks; attention covers exactly the exact top-K blocks held after
    it; the prefetch that follows fetches at most the prefetch cap."""
    from oracle.trajectory import run_unit_corrected
    w = synth.QWEN3_8B_AHEAD.with_(batch=1, prefix_tokens=16 * 300 + 5, budget_tokens=16 * 32)
    recs = run_unit_corrected(w, 0, 6, 10, cap_correct=3, cap=2)
    for r in recs[1:]:
        c, p = r["correction"], r["prefetch"]
        assert len(c["fetch_block"]) <= 3 and len(p["fetch_block"]) <= 2
        exact = [int(i) for i in r["exact_ids"] if i >= 0]
        assert c["n_hit"] + len(c["fetch_block"]) == len(c["att_block"])
        assert set(int(b) for b in c["att_block"]) <= set(exact)
        # a miss beyond the correction cap is the only reason to skip an exact block
        n_miss = len(exact) - c["n_hit"]
        assert len(exact) - len(c["att_block"]) == max(0, n_miss - 3)
