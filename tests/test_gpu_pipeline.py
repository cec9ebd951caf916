"""Multi-layer decode through oasis_decode_layers: layers sharing a host KV,
prediction/selection overlapped with attention on a second stream.

  - the overlapped schedule gives bit-identical outputs, tables and slot
    payloads to the serial one;
  - sampled (layer, unit) pairs of the 36-layer Qwen3-8B model at full size
    are checked step by step against the oracle (free-running checks:
    scores 1e-4, ids / select / tables bit-exact, attention 2e-3);
  - the fetch-all cap and a restart from the shared prompt (the fetch-ratio
    sweep) keep those checks.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import lookahead_sparse_kv_oasis_amd as L
    L.lib()


def _log(msg):
    print(msg, flush=True)


SMALL = synth.QWEN3_8B_36L.with_(batch=4, prefix_tokens=16 * 300 + 5, layers=6, steps=10,
                                 budget_tokens=16 * 64)

STATE_BUFS = ["IDS", "SLOT_BLOCK", "BLOCK_SLOT", "LAST_USED", "FETCH_BLOCK", "FETCH_SLOT",
              "ATT_BLOCK", "ATT_SLOT", "COUNTS"]


def _runner(w, steps, data_layers=2, **kw):
    from lookahead_sparse_kv_oasis_amd.runner import ModelRunner
    return ModelRunner(w, steps, data_layers=data_layers, threads=8, log=_log, **kw)


def test_overlapped_schedule_matches_serial_bitwise():
    w = SMALL
    a = _runner(w, w.steps)
    b = _runner(w, w.steps)
    side = torch.cuda.Stream()
    a.admission(side=side)
    b.admission()
    for t in range(1, w.steps + 1):
        a.step(t, side=side)
        b.step(t)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
    for l in range(w.layers):
        ha, hb = a.handles[l], b.handles[l]
        for buf in STATE_BUFS:
            assert np.array_equal(ha.read(buf), hb.read(buf)), f"layer {l} {buf}"
        assert np.array_equal(ha.read("SLOTS", np.uint8), hb.read("SLOTS", np.uint8)), \
            f"layer {l} slot payloads"
        sa, sb = ha.oasis_get_stats(), hb.oasis_get_stats()
        assert {k: sa[k] for k in ("hits", "misses", "fetched")} == \
            {k: sb[k] for k in ("hits", "misses", "fetched")}
        ha.oasis_check()
    # layers of one data layer share the host KV and differ in their selections
    assert np.array_equal(a.handles[0].read("HOST_KV", np.uint8),
                          a.handles[2].read("HOST_KV", np.uint8))
    assert not np.array_equal(a.handles[0].read("IDS"), a.handles[2].read("IDS"))
    a.close()
    b.close()


def _check_layers(mr, layers, units, steps, side, cap=None, check_payload_every=4):
    from tests.gpu_parity import PipelineLayer, pipeline_unit_kv
    checks = [PipelineLayer(mr, l, units, pipeline_unit_kv(mr, l, units)) for l in layers]
    cap = mr.cap if cap is None else cap
    reports = [dict(score_err=0.0, attn_err=0.0, steps=0, fetched=0) for _ in checks]
    mr.admission(side=side)
    torch.cuda.synchronize()
    prev = [c.after_admission() for c in checks]
    for t in range(1, steps + 1):
        mr.step(t, side=side, cap=cap)
        torch.cuda.synchronize()
        for i, c in enumerate(checks):
            c.run.h.oasis_check()
            prev[i] = c.verify_step(t, prev[i], reports[i], c.scores(), cap,
                                    check_payload=(t % check_payload_every == 0 or t == steps))
    return reports


def test_reduced_model_against_oracle_and_fetch_all_restart():
    w = SMALL
    mr = _runner(w, w.steps)
    side = torch.cuda.Stream()
    units = [(0, 0), (3, 7), (1, 4)]
    rep = _check_layers(mr, [0, 3, 5], units, w.steps, side)
    _log(f"reduced model, cap {mr.cap}: {rep}")
    # restart every layer from the shared prompt with the fetch-all cap
    mr.reset()
    rep = _check_layers(mr, [1, 4], units, w.steps, side, cap=w.k_blocks)
    _log(f"reduced model, fetch all: {rep}")
    mr.close()


def test_decode_layers_rejects_bad_arguments():
    from lookahead_sparse_kv_oasis_amd import LayerStep, OasisError, Oasis, OASIS_BF16
    w = SMALL.with_(layers=2, steps=2)
    mr = _runner(w, 2)
    bad = LayerStep([mr.handles[0], mr.handles[0]])
    for l in range(2):
        bad.set(l, None, None, mr.q[0], mr.drafts[1][0], mr.out[0])
    with pytest.raises(OasisError):
        bad.run(w.drafts, 2)
    half = LayerStep(mr.handles)
    for l in range(2):
        half.set(l, mr.app_k[0][0], None, mr.q[0], mr.drafts[1][l], mr.out[l])
    with pytest.raises(OasisError):
        half.run(w.drafts, 2)
    # a shared handle must match the owner's host layout
    with pytest.raises(OasisError):
        Oasis(w.batch + 1, w.q_heads, w.kv_heads, w.head_dim, OASIS_BF16, w.drafts,
              w.prefix_tokens + 2, share_host_with=mr.handles[0])
    # reuse of the host prompt needs the same length
    with pytest.raises(OasisError):
        mr.handles[1].oasis_load_prefix(None, None, w.prefix_tokens - 1)
    mr.close()


@pytest.fixture(scope="module")
def full_model():
    """The 36-layer model at batch 64 and 64K context (two data layers)."""
    w = synth.QWEN3_8B_36L
    mr = _runner(w, w.steps)
    yield mr
    mr.close()


@pytest.mark.slow
def test_qwen3_8b_36_layers_full_size_sampled_layers(full_model):
    """Overlapped schedule, fetch ratio 0.02 (cap 2), every step."""
    mr, w = full_model, full_model.w
    mr.reset()
    side = torch.cuda.Stream()
    rep = _check_layers(mr, [0, 19, 35], [(0, 0), (37, 3), (63, 7)], w.steps, side,
                        check_payload_every=8)
    _log(f"{w.name}: {rep}")


@pytest.mark.slow
def test_qwen3_8b_36_layers_full_size_fetch_ratio_sweep(full_model):
    """The fetch-ratio sweep of the 36-layer workload (ratios 0.01, 0.02, 0.05,
    0.10, 0.20 and fetch-all: caps 1, 2, 6, 12, 25, 128 per KV head), each
    from the prompt (reset) for 4 decode steps, layers 0, 19 and 35 checked
    free-running against the oracle at every step."""
    mr, w = full_model, full_model.w
    side = torch.cuda.Stream()
    units = [(0, 0), (37, 3), (63, 7)]
    caps = [oracle_cap(r, w.k_blocks) for r in synth.FETCH_RATIO_SWEEP]
    assert caps == [1, 2, 6, 12, 25, 128]
    for cap in caps:
        mr.reset()
        rep = _check_layers(mr, [0, 19, 35], units, 4, side, cap=cap, check_payload_every=2)
        _log(f"{w.name}, cap {cap}: {rep}")
        assert all(r["steps"] == 4 for r in rep)


def oracle_cap(ratio, k):
    import oracle
    return oracle.cap_from_ratio(ratio, k)


AHEAD_SMALL = synth.QWEN3_8B_36L_AHEAD.with_(batch=4, prefix_tokens=16 * 300 + 5, layers=5,
                                             steps=8, budget_tokens=16 * 64)


def test_lookahead_executor_against_oracle_and_one_stream():
    """oasis_decode_layers_ahead on three streams: sampled layers checked step by
    step against the oracle's lookahead ordering, and every output, table and
    slot bit-identical to the same calls on one stream."""
    from tests.gpu_parity import PipelineLayer, pipeline_unit_kv
    w = AHEAD_SMALL
    a = _runner(w, w.steps)
    b = _runner(w, w.steps)
    cur = torch.cuda.current_stream()
    side, xfer = torch.cuda.Stream(), torch.cuda.Stream()
    units = [(0, 0), (3, 7), (2, 5)]
    checks = [PipelineLayer(a, l, units, pipeline_unit_kv(a, l, units)) for l in (0, 2, 4)]
    reps = [dict(score_err=0.0, attn_err=0.0, steps=0, fetched=0) for _ in checks]
    for c in checks:
        for k in units:
            c.oru[k].slot_block[:] = -1
    empty = {k: (np.full(a.handles[0].slots, -1, np.int32),
                 np.full(a.handles[0].slots, -1, np.int32)) for k in units}
    a.admission_ahead(cur, side, xfer)
    b.admission_ahead(cur, cur, cur)
    torch.cuda.synchronize()
    state = [c.verify_ahead(0, empty, None, r, w.k_blocks) for c, r in zip(checks, reps)]
    for t in range(1, w.steps + 1):
        a.step_ahead(t, cur, side, xfer)
        b.step_ahead(t, cur, cur, cur)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
        state = [c.verify_ahead(t, prev, att, r, a.cap, check_payload=(t % 4 == 0))
                 for c, r, (prev, att) in zip(checks, reps, state)]
    for l in range(w.layers):
        for buf in STATE_BUFS:
            assert np.array_equal(a.handles[l].read(buf), b.handles[l].read(buf)), f"{l} {buf}"
        a.handles[l].oasis_check()
    _log(f"lookahead executor: {reps}")
    a.close()
    b.close()


def test_lookahead_executor_with_miss_correction_matches_one_stream():
    """oasis_decode_layers_ahead with cap_correct: three streams bit-identical to
    one, and every layer's output equal to the single-layer corrected calls."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = AHEAD_SMALL.with_(layers=3)
    a = _runner(w, w.steps)
    b = _runner(w, w.steps)
    single = LayerRunner(w.with_(layers=1), w.steps, layer=0)
    cur = torch.cuda.current_stream()
    side, xfer = torch.cuda.Stream(), torch.cuda.Stream()
    a.admission_ahead(cur, side, xfer)
    b.admission_ahead(cur, cur, cur)
    single.admission_ahead()
    for t in range(1, w.steps + 1):
        a.step_ahead(t, cur, side, xfer, cap_correct=4)
        b.step_ahead(t, cur, cur, cur, cap_correct=4)
        single.step_corrected(t, 4)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
        assert torch.equal(a.out[0], single.out), f"step {t}: layer 0 differs from one layer"
    for l in range(w.layers):
        for buf in STATE_BUFS:
            assert np.array_equal(a.handles[l].read(buf), b.handles[l].read(buf)), f"{l} {buf}"
    a.close()
    b.close()


def test_handle_moving_to_a_second_stream_midway_matches_one_stream():
    """A handle driven on one stream records no ordering events; when its
    predict / select move to a second stream at step 4 (and back for the
    attention), the first cross-stream call orders everything queued before
    it: outputs and tables stay bit-identical to the all-one-stream run."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B.with_(batch=4, prefix_tokens=16 * 300 + 5, budget_tokens=16 * 64)
    n = 8
    a, b = LayerRunner(w, n), LayerRunner(w, n)
    cur, s2 = torch.cuda.current_stream(), torch.cuda.Stream()
    a.admission()
    b.admission()
    for t in range(1, n + 1):
        for r, other in ((a, s2 if t >= 4 else cur), (b, cur)):
            h = r.h
            h.oasis_append_kv(r.app_k[t - 1], r.app_v[t - 1], stream=cur)
            h.oasis_predict(r.q_steps[t], r.drafts[t], w.drafts, stream=other)
            h.oasis_select_and_fetch(r.cap, stream=other)
            h.oasis_sparse_attn(r.q_steps[t], r.out, stream=cur)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
    for buf in STATE_BUFS:
        assert np.array_equal(a.h.read(buf), b.h.read(buf)), buf
    assert np.array_equal(a.h.read("SLOTS", np.uint8), b.h.read("SLOTS", np.uint8))
    a.h.oasis_check()


def test_predict_on_another_stream_than_its_select_and_append():
    """Predict on one stream while append, select and attention run on the
    other, swapping the two streams every step: the select, the next append
    and the next predict wait for the score kernels queued on the other
    stream, and an evict on the predict's stream waits for the select, so
    outputs, tables and slot payloads equal a one-stream run bit for bit."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B.with_(batch=8, prefix_tokens=16 * 1000 + 5, budget_tokens=16 * 64)
    n = 8
    a, b = LayerRunner(w, n), LayerRunner(w, n)
    cur, s2 = torch.cuda.current_stream(), torch.cuda.Stream()
    a.admission()
    b.admission()
    units = w.batch * w.kv_heads
    for t in range(1, n + 1):
        ps, ss = (s2, cur) if t % 2 else (cur, s2)
        for r, (p_st, s_st) in ((a, (ps, ss)), (b, (cur, cur))):
            h = r.h
            h.oasis_append_kv(r.app_k[t - 1], r.app_v[t - 1], stream=s_st)
            h.oasis_predict(r.q_steps[t], r.drafts[t], w.drafts, stream=p_st)
            h.oasis_select_and_fetch(r.cap, stream=s_st)
            h.oasis_sparse_attn(r.q_steps[t], r.out, stream=s_st)
            if t == 4:
                # step 3's first attended block of every unit forced out, on
                # the stream that did not run this step's select (nothing
                # synchronises in between)
                h.oasis_evict(prev_att[id(r)], np.ones(units, np.int32), stream=p_st)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
        if t == 3:
            prev_att = {id(r): r.h.read("ATT_BLOCK").reshape(units, -1)[:, :1].copy()
                        for r in (a, b)}
    for buf in STATE_BUFS:
        assert np.array_equal(a.h.read(buf), b.h.read(buf)), buf
    assert np.array_equal(a.h.read("SLOTS", np.uint8), b.h.read("SLOTS", np.uint8))
    a.h.oasis_check()


def test_lookahead_append_and_attention_on_different_streams():
    """Lookahead order with each step's append on one stream and its
    attention, predict and select on the other (swapped every step), nothing
    synchronising in between.  Budget and cap cover every block, so the
    blocks a pending fetch copies include the one the append writes: the
    attention waits for the append's write-through and for the host token its
    fetch reads, and outputs, tables and slot payloads equal a one-stream run
    bit for bit."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B_AHEAD.with_(batch=2, prefix_tokens=16 * 40 + 5, budget_tokens=16 * 48,
                                   cap=48)
    n = 16
    a, b = LayerRunner(w, n), LayerRunner(w, n)
    cur, s2 = torch.cuda.current_stream(), torch.cuda.Stream()
    a.admission_ahead()
    b.admission_ahead()
    for t in range(1, n + 1):
        st_app, st_rest = (cur, s2) if t % 2 else (s2, cur)
        h = a.h
        h.oasis_append_kv(a.app_k[t - 1], a.app_v[t - 1], stream=st_app)
        h.oasis_sparse_attn(a.q_steps[t], a.out, stream=st_rest)
        h.oasis_predict(None, a.drafts[t], w.drafts, stream=st_rest)
        h.oasis_select_and_fetch(a.cap, stream=st_rest)
        b.step_ahead(t)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
    for buf in STATE_BUFS:
        assert np.array_equal(a.h.read(buf), b.h.read(buf)), buf
    assert np.array_equal(a.h.read("SLOTS", np.uint8), b.h.read("SLOTS", np.uint8))
    a.h.oasis_check()


def test_select_after_append_and_attention_twice_on_other_streams():
    """Per step: append and predict on one stream, a second append on the
    other, the select back on the first (it waits for that append, whose
    write-through reads the block -> slot table the select rewrites), then
    one attention on each stream: the first copies the fetched blocks, the
    second waits for it (same partials, the slots it wrote).  Outputs, tables
    and slot payloads equal the same calls on one stream bit for bit."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B.with_(batch=4, prefix_tokens=16 * 300 + 5, budget_tokens=16 * 64)
    n = 6
    a, b = LayerRunner(w, 2 * n), LayerRunner(w, 2 * n)
    out2 = {id(a): torch.empty_like(a.out), id(b): torch.empty_like(b.out)}
    cur, s2 = torch.cuda.current_stream(), torch.cuda.Stream()
    a.admission()
    b.admission()
    for t in range(1, n + 1):
        k = 2 * (t - 1)
        for r, other in ((a, s2), (b, cur)):
            h = r.h
            h.oasis_append_kv(r.app_k[k], r.app_v[k], stream=cur)
            h.oasis_predict(r.q_steps[t], r.drafts[t], w.drafts, stream=cur)
            h.oasis_append_kv(r.app_k[k + 1], r.app_v[k + 1], stream=other)
            h.oasis_select_and_fetch(r.cap, stream=cur)
            h.oasis_sparse_attn(r.q_steps[t], r.out, stream=other)
            h.oasis_sparse_attn(r.q_steps[t], out2[id(r)], stream=cur)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: first attention differs"
        assert torch.equal(out2[id(a)], out2[id(b)]), f"step {t}: second attention differs"
    for buf in STATE_BUFS:
        assert np.array_equal(a.h.read(buf), b.h.read(buf)), buf
    assert np.array_equal(a.h.read("SLOTS", np.uint8), b.h.read("SLOTS", np.uint8))
    a.h.oasis_check()


def test_verify_and_device_evictions_on_other_streams():
    """Per step: forced evictions (oasis_evict_attended) on a second stream,
    then append, predict, select and attention on the first, then the
    verification attention on the second stream again, nothing synchronising
    in between.  The evictions wait for the previous attention and the append
    for them; the verify waits for the attention's fetch.  Everything equals
    the same calls on one stream bit for bit, and set 0 of the verify equals
    the attention up to the split-K merge order."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner, to_device
    w = synth.QWEN3_32B.with_(batch=4, prefix_tokens=16 * 400 + 5, budget_tokens=16 * 64)
    n = 6
    a, b = LayerRunner(w, n), LayerRunner(w, n)
    cur, s2 = torch.cuda.current_stream(), torch.cuda.Stream()
    D, B, Hkv, d = w.drafts, w.batch, w.kv_heads, w.head_dim
    rng = np.random.default_rng(3)
    vout = {id(r): torch.empty((1 + D, B, w.q_heads, d), dtype=torch.float32, device="cuda")
            for r in (a, b)}
    draws = [torch.from_numpy(np.ascontiguousarray(synth.evict_draws(w, t))).cuda()
             for t in range(n + 1)]
    kd = [to_device(synth.encode(rng.standard_normal((D, B, Hkv, d)).astype(np.float32),
                                 w.dtype)) for _ in range(n + 1)]
    vd = [to_device(synth.encode(rng.standard_normal((D, B, Hkv, d)).astype(np.float32),
                                 w.dtype)) for _ in range(n + 1)]
    a.admission()
    b.admission()
    torch.cuda.synchronize()
    for t in range(1, n + 1):
        for r, other in ((a, s2), (b, cur)):
            h = r.h
            h.oasis_evict_attended(draws[t], w.forced_evict_frac, stream=other)
            h.oasis_append_kv(r.app_k[t - 1], r.app_v[t - 1], stream=cur)
            h.oasis_predict(r.q, r.drafts[t], w.drafts, stream=cur)
            h.oasis_select_and_fetch(r.cap, stream=cur)
            h.oasis_sparse_attn(r.q, r.out, stream=cur)
            h.oasis_sparse_attn_verify(r.q, r.drafts[t], D, kd[t], vd[t], vout[id(r)],
                                       stream=other)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
        assert torch.equal(vout[id(a)], vout[id(b)]), f"step {t}: verify differs"
        assert float((vout[id(a)][0] - a.out).abs().max()) < 1e-5, f"step {t}: set 0"
        st = a.h.oasis_get_stats()
        assert st["misses"] > 0
    for buf in STATE_BUFS:
        assert np.array_equal(a.h.read(buf), b.h.read(buf)), buf
    assert np.array_equal(a.h.read("SLOTS", np.uint8), b.h.read("SLOTS", np.uint8))
    a.h.oasis_check()
