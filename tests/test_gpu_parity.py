"""GPU parity: the HIP path through the C-ABI against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import lookahead_sparse_kv_oasis_amd as L
    L.lib()   # loud failure if the HIP library is missing


def _parity():
    from tests.gpu_parity import Parity, log
    return Parity, log


def test_tiny_workload_full_trajectory():
    """Tiny fp32 workload: every unit, every step, every intermediate."""
    Parity, log = _parity()
    w = synth.TINY
    p = Parity(w, w.steps, [(0, 0), (0, 1)])
    rep = p.run_all()
    log(f"tiny: {rep}")
    assert rep["steps"] == w.steps


def test_tiny_workload_bf16_variant():
    Parity, log = _parity()
    w = synth.TINY.with_(dtype=synth.BF16, head_dim=128)
    p = Parity(w, 8, [(0, 0), (0, 1)])
    log(f"tiny bf16 d128: {p.run_all()}")


def _all_units(w):
    from tests.gpu_parity import every_unit
    return every_unit(w)


@pytest.mark.parametrize("q_heads,kv_heads", [(8, 8), (16, 8), (32, 4), (64, 4), (32, 1)])
def test_group_sizes_reduced_context(q_heads, kv_heads):
    """G = 1, 2, 8, 16, 32 on a reduced context with a ragged prefix (32
    heads per KV head: two 16-row tiles on the matrix cores; 2 drafts, so the
    96 query rows of the score fit the handle's limit)."""
    Parity, log = _parity()
    extra = {"drafts": 2} if q_heads // kv_heads == 32 else {}
    w = synth.QWEN3_8B.with_(batch=2, q_heads=q_heads, kv_heads=kv_heads,
                             prefix_tokens=16 * 300 + 7, budget_tokens=16 * 64, **extra)
    p = Parity(w, 6, _all_units(w))
    log(f"G={q_heads // kv_heads}: {p.run_all()}")


@pytest.mark.parametrize("head_dim", [64, 256])
def test_head_dims_reduced_context(head_dim):
    """bf16 at d = 64 and 256: the tiled summary layout and the matrix-core
    score at the other tile sizes (8 KB and 32 KB per 32 blocks)."""
    Parity, log = _parity()
    w = synth.QWEN3_8B.with_(batch=2, head_dim=head_dim, prefix_tokens=16 * 200 + 3,
                             budget_tokens=16 * 64)
    p = Parity(w, 5, _all_units(w))
    log(f"d={head_dim}: {p.run_all()}")


@pytest.mark.parametrize("block_size,budget_blocks", [(1, 48), (8, 64), (64, 16)])
def test_block_sizes_reduced_context(block_size, budget_blocks):
    """bf16, d = 128 at block sizes other than 16: the matrix-core score on
    summaries of 1, 8 or 64 tokens, the generic attention kernel and the
    eager gather on the copy stream (the fused fetch needs 16-token blocks).
    One-token blocks are the degenerate case where a block's score is the
    exact largest dot product of its key with the query rows."""
    Parity, log = _parity()
    w = synth.QWEN3_8B.with_(batch=2, block_size=block_size,
                             prefix_tokens=block_size * 120 + block_size // 2 + 1,
                             budget_tokens=block_size * budget_blocks)
    p = Parity(w, 6, _all_units(w))
    log(f"block size {block_size}: {p.run_all()}")


def test_tiny_workload_one_token_blocks():
    """fp32 with one-token blocks: the VALU score, block-major summaries and
    the generic attention at the smallest block."""
    Parity, log = _parity()
    w = synth.TINY.with_(block_size=1, prefix_tokens=200, budget_tokens=8, slots=16)
    p = Parity(w, 8, _all_units(w))
    log(f"tiny, one-token blocks: {p.run_all()}")


# ------------------------------------------------------------------ full-size workloads
# Every step of the workload through the C-ABI at its real shape, compared on a
# sample of (batch row, KV head) units that the oracle recomputes one by one.

def test_qwen3_8b_layer_full_size_sampled_units():
    Parity, log = _parity()
    w = synth.QWEN3_8B
    p = Parity(w, w.steps, [(0, 0), (17, 5), (31, 7)])
    rep = p.run_all(check_payload_every=8)
    log(f"{w.name}: {rep}")


def test_llama31_8b_long_context_full_size_sampled_units():
    Parity, log = _parity()
    w = synth.LLAMA31_8B_LONG
    p = Parity(w, w.steps, [(0, 3), (5, 0), (7, 7)])
    rep = p.run_all(check_payload_every=8)
    log(f"{w.name}: {rep}")


def test_qwen3_32b_forced_eviction_full_size_sampled_units():
    Parity, log = _parity()
    w = synth.QWEN3_32B
    p = Parity(w, w.steps, [(0, 0), (9, 4), (15, 7)])
    rep = p.run_all(check_payload_every=16)
    log(f"{w.name}: {rep}")


# Every (batch row, KV head) unit at full size: the admission step and two
# decode steps, each unit recomputed by the oracle on host threads.

def _every_unit(w, steps=2, device_evict=False):
    from tests.gpu_parity import Parity, every_unit, log
    p = Parity(w, steps, every_unit(w))
    p.device_evict = device_evict
    rep = p.run_all(check_payload_every=1)
    log(f"{w.name}, all {len(p.units)} units: {rep}")
    assert rep["steps"] == steps


def test_qwen3_8b_layer_full_size_every_unit():
    _every_unit(synth.QWEN3_8B)


def test_llama31_8b_long_context_full_size_every_unit():
    _every_unit(synth.LLAMA31_8B_LONG)


def test_qwen3_32b_full_size_every_unit_device_evictions():
    """The forced evictions applied by oasis_evict_attended from the seeded
    draws, checked on every unit against the harness rule on the GPU's own
    attended lists and against the oracle's."""
    _every_unit(synth.QWEN3_32B, device_evict=True)


# ------------------------------------------------------------------ free-running
# The GPU selects on its own scores with the fused top-K + select kernel;
# every step is checked against the oracle functions applied to its state.

def test_tiny_workload_free_running():
    from tests.gpu_parity import FreeRunning, log
    w = synth.TINY
    log(f"tiny free: {FreeRunning(w, w.steps, [(0, 0), (0, 1)]).run_free()}")


def test_qwen3_8b_layer_free_running_sampled_units():
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_8B
    rep = FreeRunning(w, 24, [(0, 0), (13, 2), (31, 7)]).run_free(check_payload_every=8)
    log(f"{w.name} free: {rep}")


def test_qwen3_32b_free_running_with_forced_evictions():
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_32B
    rep = FreeRunning(w, 16, [(0, 0), (7, 5), (15, 7)]).run_free(check_payload_every=4)
    log(f"{w.name} free: {rep}")


def test_llama31_8b_long_context_free_running_sampled_units():
    """128K context (8,196 blocks per KV head): the production selection path,
    the top-K + select kernel at 1,024 threads, on the GPU's own scores."""
    from tests.gpu_parity import FreeRunning, log
    w = synth.LLAMA31_8B_LONG
    rep = FreeRunning(w, 12, [(0, 3), (4, 6), (7, 7)]).run_free(check_payload_every=6)
    log(f"{w.name} free: {rep}")


def test_qwen3_32b_free_running_device_evictions():
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_32B
    p = FreeRunning(w, 16, [(0, 0), (7, 5), (15, 7)])
    p.device_evict = True
    rep = p.run_free(check_payload_every=4)
    log(f"{w.name} free, device evictions: {rep}")


def test_select_and_fetch_on_an_explicit_copy_stream():
    """oasis_select_and_fetch(cap, stream, copy) with a copy stream of the
    caller's: the fetched blocks are copied there after the table update and
    the attention waits for them.  Checked free-running against the oracle,
    and equal (tables, payloads bit-exact; outputs up to the split-K merge
    order) to the default placement inside the attention."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_8B.with_(batch=4, prefix_tokens=16 * 600 + 9)
    p = FreeRunning(w, 6, [(0, 0), (3, 7), (2, 4)])
    p.copy_stream = torch.cuda.Stream()
    rep = p.run_free(check_payload_every=2)
    log(f"explicit copy stream: {rep}")
    a, b = LayerRunner(w, 4), LayerRunner(w, 4)
    st = a.h.oasis_get_state()
    assert np.all(st["fetch_list"] == -1) and np.all(st["fetch_n"] == 0)
    assert np.all(st["attended"] == -1) and np.all(st["slot_block"] == -1)
    cp = torch.cuda.Stream()
    for r in (a, b):
        r.admission()
    for t in range(1, 5):
        for r, copy in ((a, cp), (b, None)):
            r.h.oasis_append_kv(r.app_k[t - 1], r.app_v[t - 1])
            r.h.oasis_predict(r.q, r.drafts[t], w.drafts)
            r.h.oasis_select_and_fetch(r.cap, copy=copy)
            r.h.oasis_sparse_attn(r.q, r.out)
        torch.cuda.synchronize()
        assert float((a.out - b.out).abs().max()) <= 1e-5, f"step {t}"
        sa, sb = a.h.oasis_get_state(), b.h.oasis_get_state()
        for k in sa:
            assert np.array_equal(sa[k], sb[k]), f"step {t}: {k}"
    from tests.gpu_parity import assert_held_rows_equal
    assert_held_rows_equal(a.h, b.h)
    a.h.oasis_check()


# ------------------------------------------------------------------ lookahead ordering

def test_lookahead_ordering_reduced_context():
    """[OASIS] Fig. 8 ordering on one layer: attention at step t over the set
    step t-1 predicted from its drafts alone."""
    from tests.gpu_parity import AheadRunning, log
    w = synth.QWEN3_8B_AHEAD.with_(batch=2, prefix_tokens=16 * 300 + 7, budget_tokens=16 * 64)
    p = AheadRunning(w, 10, [(0, 0), (1, 7), (0, 4)])
    log(f"lookahead reduced: {p.run_ahead()}")


def test_lookahead_ordering_full_size_sampled_units():
    from tests.gpu_parity import AheadRunning, log
    w = synth.QWEN3_8B_AHEAD
    p = AheadRunning(w, w.steps, [(0, 0), (17, 5), (31, 7)])
    log(f"{w.name}: {p.run_ahead(check_payload_every=16)}")


def test_lookahead_append_into_a_block_whose_fetch_is_pending():
    """Budget and cap covering every block.  Admission fetches the partly
    filled tail block, and a block opened at step 12 is fetched by that step's
    select; in both cases the next append writes its token into the block
    while the copy is still pending (it runs inside the next attention).  The
    attention over that block and the slot payloads must hold the token."""
    from tests.gpu_parity import AheadRunning, log
    w = synth.QWEN3_8B_AHEAD.with_(batch=2, prefix_tokens=16 * 40 + 5, budget_tokens=16 * 48,
                                   cap=48)
    p = AheadRunning(w, 16, [(0, 0), (1, 7), (0, 4)])
    rep = p.run_ahead(check_payload_every=1)
    log(f"lookahead, fetch all, appends into pending fetches: {rep}")
    assert rep["fetched"] > 0


@pytest.fixture
def cu_streams():
    """A compute stream on all CUs but the first 16 and a copy stream on those
    16 (oasis_stream_create_cus), and the compute stream's CU count."""
    import lookahead_sparse_kv_oasis_amd as L
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    n_copy = 16
    raw = [L.stream_create_cus(n_copy, ncu - n_copy), L.stream_create_cus(0, n_copy)]
    yield ncu - n_copy, torch.cuda.ExternalStream(raw[0]), torch.cuda.ExternalStream(raw[1])
    torch.cuda.synchronize()
    for r in raw:
        L.stream_destroy(r)


@pytest.mark.parametrize("case", ["reduced", "fetch_all", "full_size", "full_size_fused"])
def test_lookahead_with_the_copy_on_its_own_cus(case, cu_streams):
    """[OASIS] Fig. 8 placement: each select's blocks are copied on a copy
    stream with CUs of its own while the next step appends, scores the drafts
    and attends to the held blocks on the compute stream (sized for the
    remaining CUs); the fetched blocks are attended once the copy lands.
    fetch_all: the budget and cap cover every block, so an append writes its
    token into a block whose copy is still running.  Checked against the
    oracle as the one-stream lookahead run is, slot payloads included (at full
    size also with score, top-K and select fused: 256 units fill the 240 CUs'
    one-workgroup-per-unit kernel)."""
    from tests.gpu_parity import AheadRunning, log
    cus, comp, copy = cu_streams
    if case == "reduced":
        w = synth.QWEN3_8B_AHEAD.with_(batch=2, prefix_tokens=16 * 300 + 7,
                                       budget_tokens=16 * 64)
        p, every = AheadRunning(w, 10, [(0, 0), (1, 7), (0, 4)], compute_units=cus), 2
    elif case == "fetch_all":
        w = synth.QWEN3_8B_AHEAD.with_(batch=2, prefix_tokens=16 * 40 + 5,
                                       budget_tokens=16 * 48, cap=48)
        p, every = AheadRunning(w, 16, [(0, 0), (1, 7), (0, 4)], compute_units=cus), 1
    else:
        w = synth.QWEN3_8B_AHEAD
        p, every = AheadRunning(w, 12, [(0, 0), (17, 5), (31, 7)], compute_units=cus), 6
        if case == "full_size_fused":   # score, top-K and select in one kernel
            p.run.h.oasis_set_score_topk_fusion(True)
    rep = p.run_ahead(check_payload_every=every, beside=(comp, copy))
    log(f"lookahead, copy on {torch.cuda.get_device_properties(0).multi_processor_count - cus}"
        f" CUs of its own ({case}): {rep}")
    assert rep["fetched"] > 0


@pytest.mark.parametrize("q_heads", [8, 64, 128])
def test_lookahead_with_the_copy_on_its_own_cus_other_group_sizes(q_heads, cu_streams):
    """The copy-beside lookahead for 1, 8 and 16 query heads per KV head (the
    held-block and fetched-block launches and the combine on the G-row
    partials of each), against the oracle with slot payloads."""
    from tests.gpu_parity import AheadRunning, log
    cus, comp, copy = cu_streams
    w = synth.QWEN3_8B_AHEAD.with_(batch=2, q_heads=q_heads, prefix_tokens=16 * 200 + 11,
                                   budget_tokens=16 * 32, cap=4)
    p = AheadRunning(w, 6, [(0, 0), (1, 7), (0, 5)], compute_units=cus)
    rep = p.run_ahead(check_payload_every=2, beside=(comp, copy))
    log(f"lookahead, copy beside, G = {q_heads // 8}: {rep}")
    assert rep["fetched"] > 0


def test_lookahead_copy_beside_matches_one_stream(cu_streams):
    """The same lookahead run on one stream and with the copy on its own CUs:
    ids, tables and slot payloads bit-identical every step; outputs equal up
    to the order of the sums (the attention runs as two launches)."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    cus, comp, copy = cu_streams
    w = synth.QWEN3_8B_AHEAD.with_(batch=4, prefix_tokens=16 * 500 + 3, budget_tokens=16 * 64)
    a = LayerRunner(w, 12)
    b = LayerRunner(w, 12, compute_units=cus)
    torch.cuda.synchronize()  # inputs were made on torch's stream
    a.admission_ahead()
    b.admission_beside(comp, copy)
    worst = 0.0
    for t in range(1, 13):
        a.step_ahead(t)
        b.step_beside(t, comp, copy)
        torch.cuda.synchronize()
        for name in ("IDS", "SLOT_BLOCK", "LAST_USED", "ATT_BLOCK", "COUNTS", "FETCH_BLOCK"):
            assert np.array_equal(a.h.read(name), b.h.read(name)), f"step {t}: {name}"
        oa, ob = a.out.cpu().numpy(), b.out.cpu().numpy()
        worst = max(worst, float(np.max(np.abs(oa - ob))))
        assert worst <= 1e-5, f"step {t}: outputs differ by {worst:.3g}"
    # every slot's rows of tokens < T
    T, bs, S, d = a.h.oasis_tokens(), w.block_size, a.h.slots, w.head_dim
    sa = a.h.read("SLOTS", np.uint16).reshape(-1, S, 2, bs, d)
    sb = b.h.read("SLOTS", np.uint16).reshape(-1, S, 2, bs, d)
    blk = a.h.read("SLOT_BLOCK").reshape(-1, S)
    for u in range(sa.shape[0]):
        for s_ in range(S):
            if blk[u, s_] >= 0:
                n = max(0, min(bs, T - blk[u, s_] * bs))
                assert np.array_equal(sa[u, s_, :, :n], sb[u, s_, :, :n]), (u, s_)
    from tests.gpu_parity import log
    log(f"lookahead one stream vs copy beside: outputs within {worst:.3g}")


def test_lookahead_recall_measurement():
    """Recall of the drafts' prediction and of the previous query's top-K
    against the exact top-K of the step's own query; the exact ids are checked
    against the oracle top-K of the GPU's scores for sampled units."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner, exact_ids, predicted_ids, recall
    from tests.gpu_parity import log
    w = synth.QWEN3_8B_AHEAD.with_(batch=4, prefix_tokens=16 * 400 + 3, budget_tokens=16 * 64)
    n = 8
    run = LayerRunner(w, n)
    h = run.h
    buf = torch.empty(w.batch * w.kv_heads * w.k_blocks, dtype=torch.int32, device="cuda")
    run.admission_ahead()
    torch.cuda.synchronize()
    prev_exact = None
    r_ahead, r_prev = [], []
    K = h.k_blocks
    for t in range(1, n + 1):
        pred = predicted_ids(h)
        h.oasis_append_kv(run.app_k[t - 1], run.app_v[t - 1])
        ex = exact_ids(h, run.q_steps[t], buf)
        scores = h.read("SCORES", np.float32).reshape(w.batch * w.kv_heads, -1)
        nb = w.blocks_at(w.prefix_tokens + t)
        for u in (0, 9, w.batch * w.kv_heads - 1):
            assert np.array_equal(ex[u], oracle.topk(scores[u, :nb], K)), f"step {t} unit {u}"
        r_ahead.append(recall(pred, ex))
        if prev_exact is not None:
            r_prev.append(recall(prev_exact, ex))
        prev_exact = ex
        h.oasis_sparse_attn(run.q_steps[t], run.out)
        h.oasis_predict(None, run.drafts[t], w.drafts)
        h.oasis_select_and_fetch(run.cap)
    torch.cuda.synchronize()
    a, p = float(np.mean(r_ahead)), float(np.mean(r_prev))
    log(f"recall of the exact next top-K: drafts {a:.3f}, previous query {p:.3f}")
    assert 0.0 < a <= 1.0 and 0.0 < p <= 1.0


# ------------------------------------------------------------------ decode-time miss correction

def test_miss_correction_reduced_context():
    """Lookahead prefetch plus decode-time miss correction, phase by phase
    against the oracle (cap_correct = 3 and the unbounded correction)."""
    from tests.gpu_parity import CorrectedRunning, log
    w = synth.QWEN3_8B_AHEAD.with_(batch=2, prefix_tokens=16 * 300 + 7, budget_tokens=16 * 64)
    for cc in (3, w.k_blocks):
        p = CorrectedRunning(w, 8, [(0, 0), (1, 7), (0, 4)])
        log(f"correction cap {cc}: {p.run_corrected(cc)}")


# ------------------------------------------------------------------ verification attention

@pytest.mark.parametrize("q_heads,n_steps,fewer", [(32, 4, 0), (64, 3, 0), (128, 2, 0),
                                                   (8, 2, 0), (16, 2, 1)])
def test_verification_attention_against_oracle(q_heads, n_steps, fewer):
    """Normal and draft queries together with causal draft tokens ([OASIS]
    Fig. 7 right) after each step of the free-running path: every set of
    sampled units against the oracle over the GPU's attended list; set 0
    equal to oasis_sparse_attn up to summation order.  20 rows per KV head
    run as one padded 32-row pass, 40 as 32 + 8, 80 as 32 + 32 + 16, 5 as
    one padded 8-row pass; `fewer` drafts than the handle was sized for
    (2 heads x 4 sets: one 8-row pass)."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner, to_device
    from tests.gpu_parity import ATTN_TOL, log
    w = synth.QWEN3_8B.with_(batch=3, q_heads=q_heads, prefix_tokens=16 * 300 + 9,
                             budget_tokens=16 * 64)
    run = LayerRunner(w, n_steps)
    h = run.h
    D, B, Hkv, d, G = w.drafts - fewer, w.batch, w.kv_heads, w.head_dim, w.group
    rng = np.random.default_rng(7)
    out = torch.empty((1 + D, B, w.q_heads, d), dtype=torch.float32, device="cuda")
    run.admission()
    worst = 0.0
    units = [(0, 0), (1, 5), (2, 7)]
    kv = {k: synth.unit_kv(w, k[0], k[1], w.prefix_tokens + n_steps) for k in units}
    qf = oracle.to_f64(synth.queries(w), w.dtype)
    for t in range(1, n_steps + 1):
        run.step(t)
        kd = synth.encode(rng.standard_normal((D, B, Hkv, d)).astype(np.float32), w.dtype)
        vd = synth.encode(rng.standard_normal((D, B, Hkv, d)).astype(np.float32), w.dtype)
        h.oasis_sparse_attn_verify(run.q, run.drafts[t][:D].contiguous() if fewer else run.drafts[t],
                                   D, to_device(kd), to_device(vd), out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        # set 0 is the plain attention, summed in other splits (fetched blocks
        # are read from their slots here, inside the fetch waves there)
        assert np.max(np.abs(got[0] - run.out.cpu().numpy())) < 1e-5, f"step {t}: set 0"
        ab, cnt = h.read("ATT_BLOCK"), h.read("COUNTS")
        dr = oracle.to_f64(synth.drafts(w, t), w.dtype)[:D]
        T = w.prefix_tokens + t
        for (b, hh) in units:
            u = b * Hkv + hh
            att = ab[u * w.k_blocks:u * w.k_blocks + int(cnt[u * 4])]
            g0 = hh * G
            sets = np.stack([qf[b, g0:g0 + G]] + [dr[i, b, g0:g0 + G] for i in range(D)])
            exp = oracle.attention_verify(sets, kv[(b, hh)][0], kv[(b, hh)][1], w.dtype,
                                          w.block_size, T, att, oracle.to_f64(kd[:, b, hh], w.dtype),
                                          oracle.to_f64(vd[:, b, hh], w.dtype))
            e = float(np.max(np.abs(got[:, b, g0:g0 + G].astype(np.float64) - exp)))
            worst = max(worst, e)
            assert e <= ATTN_TOL, f"step {t} unit {(b, hh)} verify err {e:.3g}"
    log(f"verify G={G}: max err {worst:.3g}")


# ------------------------------------------------------------------ score + top-K + select fusion

def _state(h, bufs=("IDS", "SLOT_BLOCK", "BLOCK_SLOT", "LAST_USED", "FETCH_BLOCK",
                    "FETCH_SLOT", "ATT_BLOCK", "ATT_SLOT", "COUNTS")):
    return {b: h.read(b) for b in bufs}


def test_score_topk_fusion_bit_identical_full_size():
    """Qwen3-8B layer at batch 32 and 32K context: with the fused kernel every
    step's scores, ids, tables, slot payloads and outputs equal the separate
    kernels' bit for bit; a read of the ids or the scores between predict and
    select runs the deferred work on its own and changes nothing."""
    from lookahead_sparse_kv_oasis_amd import TIME
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    from tests.gpu_parity import log
    w = synth.QWEN3_8B
    n = 10
    a, b = LayerRunner(w, n), LayerRunner(w, n)
    a.h.oasis_set_score_topk_fusion(True)
    a.h.oasis_set_timing(TIME["all"])
    a.admission()
    b.admission()
    for t in range(1, n + 1):
        for r in (a, b):
            r.h.oasis_append_kv(r.app_k[t - 1], r.app_v[t - 1])
            r.h.oasis_predict(r.q_steps[t], r.drafts[t], w.drafts)
        if t == 3:
            assert np.array_equal(a.h.read("IDS"), b.h.read("IDS")), "ids read before select"
        if t == 5:
            assert np.array_equal(a.h.read("SCORES", np.float32), b.h.read("SCORES", np.float32))
        for r in (a, b):
            r.h.oasis_select_and_fetch(r.cap)
            r.h.oasis_sparse_attn(r.q_steps[t], r.out)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
        sa, sb = _state(a.h), _state(b.h)
        for k in sa:
            assert np.array_equal(sa[k], sb[k]), f"step {t}: {k} differs"
        assert np.array_equal(a.h.read("SCORES", np.float32), b.h.read("SCORES", np.float32)), \
            f"step {t}: scores differ"
        if t % 5 == 0:
            assert np.array_equal(a.h.read("SLOTS", np.uint8), b.h.read("SLOTS", np.uint8)), \
                f"step {t}: slot payloads differ"
    tm = a.h.oasis_get_timing()
    # steps 3 and 5 ran the separate kernels, the admission and the rest fused
    assert tm["n_select"] == 2 and tm["n_score"] == n + 1, tm
    log(f"fused score+top-K+select: {n} steps bit-identical, timing {tm}")
    a.h.oasis_check()


def test_fetch_outside_the_attention_bit_identical_full_size():
    """Qwen3-8B layer at full size: fetched blocks copied by the gather kernel
    on the copy stream (fetch-in-attention off from the start, or switched
    off and on again with a copy pending) give the same tables, selections
    and slot payloads (the rows of the tokens held), bit for bit, as the
    copy inside the attention kernel.
    The attention output differs only by rounding: inside the attention each
    fetched block is its own split-K partial, with the gather every block is
    read from its slot by the hit workgroups, so the fp32 merge order
    differs."""
    from lookahead_sparse_kv_oasis_amd import OasisError, OASIS_E_INVAL, TIME
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    from tests.gpu_parity import log
    w = synth.QWEN3_8B
    n = 8
    a, b, c = LayerRunner(w, n), LayerRunner(w, n), LayerRunner(w, n)
    a.h.oasis_set_fetch_in_attention(False)
    a.h.oasis_set_timing(TIME["gather"] | TIME["attn"])
    for r in (a, b, c):
        r.admission()
    for t in range(1, n + 1):
        for r in (a, b, c):
            r.h.oasis_append_kv(r.app_k[t - 1], r.app_v[t - 1])
            r.h.oasis_predict(r.q_steps[t], r.drafts[t], w.drafts)
            r.h.oasis_select_and_fetch(r.cap)
        if t in (3, 6):   # c switches with its copy pending
            c.h.oasis_set_fetch_in_attention(t == 6)
        for r in (a, b, c):
            r.h.oasis_sparse_attn(r.q_steps[t], r.out)
        torch.cuda.synchronize()
        for r in (a, c):
            err = float((r.out - b.out).abs().max())
            assert err <= 1e-5, f"step {t}: outputs differ by {err:.3g}"
            sr, sb = _state(r.h), _state(b.h)
            for k in sb:
                assert np.array_equal(sr[k], sb[k]), f"step {t}: {k} differs"
        if t % 4 == 0:
            from tests.gpu_parity import assert_held_rows_equal
            for r in (a, c):
                assert_held_rows_equal(r.h, b.h, f"step {t}:")
    tm = a.h.oasis_get_timing()
    assert tm["n_gather"] == n + 1 and tm["n_attn"] == n + 1, tm   # admission included
    log(f"fetch outside the attention: {n} steps bit-identical, timing {tm}")
    for r in (a, b, c):
        r.h.oasis_check()
    f32 = LayerRunner(synth.TINY, 1)
    with pytest.raises(OasisError) as e:
        f32.h.oasis_set_fetch_in_attention(True)   # fp32 attention has no fetch waves
    assert e.value.status == OASIS_E_INVAL
    f32.h.oasis_set_fetch_in_attention(False)


def test_score_topk_fusion_free_running_against_oracle():
    """The fused kernel checked step by step against the oracle (scores 1e-4,
    ids, select and tables bit-exact, attention 2e-3) on sampled units."""
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_8B
    rep = FreeRunning(w, 12, [(0, 0), (13, 2), (31, 7)]).run_free(check_payload_every=6,
                                                                   fuse=True)
    log(f"{w.name} fused free: {rep}")


def test_score_topk_fusion_lookahead_executor():
    """The three-stream lookahead executor (Fig. 8 ordering) with fusion on
    every layer: outputs and tables bit-identical to the same run without."""
    from lookahead_sparse_kv_oasis_amd.runner import ModelRunner
    from tests.gpu_parity import log
    w = synth.QWEN3_8B_36L_AHEAD.with_(batch=32, prefix_tokens=16 * 200 + 5, layers=3, steps=6,
                                       budget_tokens=16 * 64)
    a = ModelRunner(w, w.steps, data_layers=1, threads=8, log=log)
    b = ModelRunner(w, w.steps, data_layers=1, threads=8, log=log)
    for h in a.handles:
        h.oasis_set_score_topk_fusion(True)
    cur = torch.cuda.current_stream()
    side, xfer = torch.cuda.Stream(), torch.cuda.Stream()
    a.admission_ahead(cur, side, xfer)
    b.admission_ahead(cur, side, xfer)
    for t in range(1, w.steps + 1):
        a.step_ahead(t, cur, side, xfer, cap_correct=4 if t % 2 else 0)
        b.step_ahead(t, cur, side, xfer, cap_correct=4 if t % 2 else 0)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
    for l in range(w.layers):
        sa, sb = _state(a.handles[l]), _state(b.handles[l])
        for k in sa:
            assert np.array_equal(sa[k], sb[k]), f"layer {l} {k}"
        a.handles[l].oasis_check()
    a.close()
    b.close()


# ------------------------------------------------------------------ attend-all reading

def test_attend_all_resident_tiny_free_running():
    """fp32 path with slots = K: every held block attended, checked against
    the oracle's attend-all select and attention over that list."""
    from tests.gpu_parity import FreeRunning, log
    w = synth.TINY.with_(slots=8)
    rep = FreeRunning(w, w.steps, [(0, 0), (0, 1)]).run_free(attend_all=True)
    log(f"tiny attend-all: {rep}")


def test_attend_all_resident_rejects_more_slots_than_budget():
    from lookahead_sparse_kv_oasis_amd import OasisError
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    run = LayerRunner(synth.TINY, 2)  # 32 slots per KV head, K = 8
    with pytest.raises(OasisError):
        run.h.oasis_set_attend_all_resident(True)
    run.h.oasis_set_attend_all_resident(False)


def test_attend_all_resident_forced_evictions_full_size():
    """Qwen3-32B layer with forced evictions, so fewer than S blocks are held
    and some held blocks are not selected: the attended lists and the fused
    fetch + attention over them against the oracle."""
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_32B
    rep = FreeRunning(w, 12, [(0, 0), (7, 5), (15, 7)]).run_free(check_payload_every=6,
                                                                  attend_all=True)
    log(f"{w.name} attend-all: {rep}")


def test_attend_all_resident_with_fusion_full_size():
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_8B
    rep = FreeRunning(w, 8, [(0, 0), (13, 2), (31, 7)]).run_free(check_payload_every=4, fuse=True,
                                                                  attend_all=True)
    log(f"{w.name} attend-all fused: {rep}")


@pytest.mark.parametrize("q_heads,drafts,prefix", [(128, 4, 16 * 300 + 5), (128, 7, 16 * 300 + 5),
                                                   (128, 4, 16 * 2100 + 3)])
def test_score_topk_fusion_query_row_tiles(q_heads, drafts, prefix):
    """G = 16 with 5 and 8 query sets (80 and 128 rows: three and four 32-row
    tiles per unit), short and 2,100-block contexts: fused equals separate."""
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B.with_(q_heads=q_heads, drafts=drafts, prefix_tokens=prefix)
    n = 4
    a, b = LayerRunner(w, n), LayerRunner(w, n)
    a.h.oasis_set_score_topk_fusion(True)
    for r in (a, b):
        r.admission()
    for t in range(1, n + 1):
        for r in (a, b):
            r.step(t)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), f"step {t}: outputs differ"
        assert np.array_equal(a.h.read("SCORES", np.float32), b.h.read("SCORES", np.float32))
        sa, sb = _state(a.h), _state(b.h)
        for k in sa:
            assert np.array_equal(sa[k], sb[k]), f"step {t}: {k} differs"
    a.h.oasis_check()


# ------------------------------------------------------------------ degenerate and large pools

def test_free_running_cap_zero_attends_hits_only():
    """Cap 0 after an admission: nothing is fetched, the attended list is the
    held selected blocks, and the attention runs over those alone."""
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_8B.with_(batch=2, prefix_tokens=16 * 300 + 7, budget_tokens=16 * 64)
    p = FreeRunning(w, 5, [(0, 0), (1, 7)])
    p.cap = 0
    rep = p.run_free()
    log(f"cap 0: {rep}")
    assert rep["fetched"] == 0


@pytest.mark.parametrize("slots", [300, 2048])
def test_free_running_full_slot_pools(slots):
    """S > K slots per KV head, every slot held from the start: the admission
    and every capped fetch evict, and with more than 256 slots the victims are
    ranked by counting.  300 slots keep the tables in the top-K + select
    kernel's LDS; 2,048 (the largest pool) do not, and the top-K and select
    run as two kernels."""
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_8B.with_(batch=2, prefix_tokens=16 * 2100 + 3, slots=slots,
                             initial_resident_frac=1.0)
    p = FreeRunning(w, 6, [(0, 0), (1, 5)])
    rep = p.run_free()
    log(f"{slots}-slot pool: {rep}")


@pytest.mark.parametrize("fetch_ratio", [0.02, 1.0])
def test_free_running_largest_budget(fetch_ratio):
    """The largest budget the handle takes, 16,384 tokens (K = 1,024 blocks
    per KV head) with 1,024 slots, on a 1,600-block context: the top-K places
    its winners by rank counting (more than 128 of them), the select and the
    balanced attention run K-entry lists (its partial rows per unit grow with
    K), and fetch-all moves up to 1,024 blocks per KV head in one step.  Every
    unit, every step, against the oracle."""
    from tests.gpu_parity import FreeRunning, every_unit, log
    w = synth.QWEN3_8B.with_(batch=2, prefix_tokens=16 * 1600 + 11, budget_tokens=16 * 1024,
                             fetch_ratio=fetch_ratio)
    rep = FreeRunning(w, 4, every_unit(w)).run_free()
    log(f"K = 1024, ratio {fetch_ratio}: {rep}")


def test_free_running_past_the_direct_lookup_table():
    """More than 16,384 blocks per KV head (272K tokens): the select's
    resident-block lookup falls back to the LDS hash; checked step by step
    against the oracle on sampled units."""
    from tests.gpu_parity import FreeRunning, log
    w = synth.QWEN3_8B.with_(batch=1, prefix_tokens=16 * 17000 + 5)
    rep = FreeRunning(w, 4, [(0, 0), (0, 5)]).run_free(check_payload_every=4)
    log(f"17,000-block context: {rep}")
