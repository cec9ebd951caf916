"""GPU tests of single kernels and error paths through the C-ABI."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import lookahead_sparse_kv_oasis_amd as L
    L.lib()


def _handle(batch=1, hq=2, hkv=1, d=64, dtype=0, drafts=0, max_tokens=1024, bs=16, budget=128,
            ratio=0.02, slots=0, compute_units=0):
    from lookahead_sparse_kv_oasis_amd import Oasis
    return Oasis(batch, hq, hkv, d, dtype, drafts, max_tokens, block_size=bs,
                 budget_tokens=budget, fetch_ratio=ratio, slots_per_head=slots,
                 compute_units=compute_units)


def _zeros_prefix(h, T, d, batch=1, hkv=1, dtype=np.float32):
    z = np.zeros((batch, hkv, T, d), dtype)
    h.oasis_load_prefix(z, z, T)


# block counts across the workgroup shapes (256 / 512 / 1,024 threads, 4 to 64
# keys per thread), the largest pool, and K above the one-wave sort
@pytest.mark.parametrize("nb,k,seed", [(1, 8, 0), (5, 8, 1), (300, 128, 2), (1500, 128, 8),
                                       (2048, 64, 9), (2052, 128, 3), (8196, 128, 4),
                                       (20000, 256, 5), (4096, 1024, 6), (65536, 128, 7)])
def test_topk_matches_oracle_with_ties(nb, k, seed):
    bs, d, units = 16, 8, 3
    h = _handle(batch=units, hq=1, hkv=1, d=d, max_tokens=nb * bs, budget=k * bs)
    _zeros_prefix(h, nb * bs, d, batch=units)
    rng = np.random.default_rng(seed)
    s = np.zeros((units, 1, h.nb_max), np.float32)
    s[0, 0, :nb] = rng.integers(-4, 5, nb).astype(np.float32) * 0.5      # heavy ties
    s[1, 0, :nb] = rng.standard_normal(nb).astype(np.float32)
    s[2, 0, :nb] = np.where(rng.random(nb) < 0.5, -0.0, 0.0).astype(np.float32)  # +-0 only
    ids_dev = torch.full((units, 1, k), -7, dtype=torch.int32, device="cuda")
    h.oasis_topk_from_scores(torch.from_numpy(s).cuda(), ids_dev)
    torch.cuda.synchronize()
    got = ids_dev.cpu().numpy()
    internal = h.read("IDS").reshape(units, 1, k)
    for u in range(units):
        exp = oracle.topk(s[u, 0, :nb], k)
        assert np.array_equal(got[u, 0], exp), (u, got[u, 0][:16], exp[:16])
        assert np.array_equal(internal[u, 0], exp)
    h.oasis_check()


def test_topk_rejects_nonfinite_scores():
    from lookahead_sparse_kv_oasis_amd import OasisError, OASIS_E_NONFINITE
    h = _handle(max_tokens=160)
    _zeros_prefix(h, 160, 64)
    s = np.zeros((1, 1, h.nb_max), np.float32)
    s[0, 0, 3] = np.nan
    h.oasis_topk_from_scores(torch.from_numpy(s).cuda())
    with pytest.raises(OasisError) as e:
        h.oasis_check()
    assert e.value.status == OASIS_E_NONFINITE
    h.oasis_check()    # the word is cleared


def test_select_reproduces_hand_worked_lru_trace_on_gpu():
    g = json.load(open(os.path.join(GOLD, "lru_trace.json")))
    bs, d = 16, 8
    T0 = 91                       # six blocks; five appends keep it at six
    h = _handle(hq=1, hkv=1, d=d, max_tokens=96, budget=g["k"] * bs, slots=g["slots"])
    rng = np.random.default_rng(0)
    kv = rng.standard_normal((1, 1, 96, d)).astype(np.float32)
    h.oasis_load_prefix(np.ascontiguousarray(kv[:, :, :T0]), np.ascontiguousarray(kv[:, :, :T0]), T0)
    h.oasis_set_state(np.array(g["initial"]["slot_block"], np.int32),
                      np.array(g["initial"]["last_used"], np.int32))
    q = torch.from_numpy(rng.standard_normal((1, 1, d)).astype(np.float32)).cuda()
    out = torch.empty((1, 1, d), dtype=torch.float32, device="cuda")
    for st in g["steps"]:
        t = st["t"]
        tok = torch.from_numpy(np.ascontiguousarray(kv[:, :, T0 + t - 1])).cuda()
        h.oasis_append_kv(tok, tok)
        s = np.zeros((1, 1, h.nb_max), np.float32)
        s[0, 0, :6] = st["scores"]
        h.oasis_topk_from_scores(torch.from_numpy(s).cuda())
        h.oasis_select_and_fetch(g["cap"])
        h.oasis_sparse_attn(q, out)
        torch.cuda.synchronize()
        cnt = h.read("COUNTS")
        na, nh, nf = int(cnt[0]), int(cnt[1]), int(cnt[2])
        assert list(h.read("IDS")) == st["ids"]
        assert list(h.read("FETCH_BLOCK")[:nf]) == st["fetch_block"], t
        assert list(h.read("FETCH_SLOT")[:nf]) == st["fetch_slot"], t
        assert list(h.read("ATT_BLOCK")[:na]) == st["att_block"], t
        assert list(h.read("ATT_SLOT")[:na]) == st["att_slot"], t
        assert nh == st["n_hit"]
        assert list(h.read("SLOT_BLOCK")) == st["slot_block"], t
        assert list(h.read("LAST_USED")) == st["last_used"], t
        T = T0 + t
        ref = oracle.attention(q.cpu().numpy()[0].astype(np.float64), kv[0, 0, :T], kv[0, 0, :T],
                               synth.F32, bs, T, np.array(st["att_block"], np.int32))
        assert np.max(np.abs(out.cpu().numpy()[0] - ref)) < 2e-3


def test_error_paths():
    from lookahead_sparse_kv_oasis_amd import (OasisError, OASIS_E_CAPACITY, OASIS_E_INVAL,
                                               OASIS_E_STATE)
    h = _handle(max_tokens=33, drafts=1)
    k = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    q = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
    out = torch.empty((1, 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(OasisError) as e:
        h.oasis_predict(q, None, 0)          # nothing loaded yet
    assert e.value.status == OASIS_E_STATE
    _zeros_prefix(h, 32, 64)
    with pytest.raises(OasisError) as e:
        h.oasis_select_and_fetch(2)          # before predict
    assert e.value.status == OASIS_E_STATE
    with pytest.raises(OasisError) as e:
        h.oasis_sparse_attn(q, out)          # before select
    assert e.value.status == OASIS_E_STATE
    with pytest.raises(OasisError) as e:
        h.oasis_predict(q, None, 2)          # more drafts than the layout allows
    assert e.value.status == OASIS_E_INVAL
    h.oasis_append_kv(k, k)
    with pytest.raises(OasisError) as e:
        h.oasis_append_kv(k, k)              # 34th token
    assert e.value.status == OASIS_E_CAPACITY
    with pytest.raises(OasisError) as e:
        h.oasis_set_state(np.array([1, 1, -1, -1, -1, -1, -1, -1], np.int32),
                          np.zeros(8, np.int32))
    assert e.value.status == OASIS_E_INVAL
    with pytest.raises(OasisError) as e:
        h.oasis_set_state(np.array([5] + [-1] * 7, np.int32), np.zeros(8, np.int32))
    assert e.value.status == OASIS_E_INVAL
    h.oasis_predict(q, None, 0)
    h.oasis_select_and_fetch(0)              # cap 0: nothing fetched, nothing attended
    h.oasis_sparse_attn(q, out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    h.oasis_check()


def test_cu_partition_arguments():
    """oasis_stream_create_cus rejects empty ranges and ranges past the
    device's CUs; a handle's compute_units must be 0 or a CU count of the
    device; a valid partition stream runs the handle's work."""
    import lookahead_sparse_kv_oasis_amd as L
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    for first, n in [(0, 0), (-1, 4), (ncu - 8, 16), (0, ncu + 1)]:
        with pytest.raises(L.OasisError) as e:
            L.stream_create_cus(first, n)
        assert e.value.status == L.OASIS_E_INVAL, (first, n)
    for cus in [-1, ncu + 1]:
        with pytest.raises(L.OasisError) as e:
            _handle(max_tokens=33, drafts=1, compute_units=cus)
        assert e.value.status == L.OASIS_E_INVAL, cus
    s = L.stream_create_cus(8, ncu - 8)
    try:
        h = _handle(max_tokens=33, drafts=1, compute_units=ncu - 8)
        _zeros_prefix(h, 32, 64)
        q = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
        out = torch.full((1, 2, 64), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        h.oasis_predict(q, None, 0, stream=s)
        h.oasis_select_and_fetch(2, stream=s)
        h.oasis_sparse_attn(q, out, stream=s)
        torch.cuda.synchronize()
        assert torch.all(out == 0)   # zero keys and values
        h.oasis_check()
    finally:
        torch.cuda.synchronize()
        L.stream_destroy(s)


@pytest.mark.parametrize("hq", [32, 64, 128])
def test_empty_attended_sets_give_zero_output_on_the_matrix_core_path(hq):
    """bf16, d = 128 (the balanced attention kernel, 4, 8 and 16 heads per KV
    head): nothing resident and cap 0, so every unit's attended list is empty;
    the kernel marks every partial row empty and the combine writes exact
    zeros (the rows' sums, never written, are selected away).  Verification
    attention over the same empty lists leaves set 0 at zero and attends set
    j to draft tokens 1..j only."""
    B, hkv, d, T = 4, 8, 128, 16 * 100 + 3
    h = _handle(batch=B, hq=hq, hkv=hkv, d=d, dtype=1, drafts=2, max_tokens=T + 8,
                budget=16 * 64)
    z = np.zeros((B, hkv, T, d), np.uint16)
    h.oasis_load_prefix(z, z, T)
    q = torch.ones((B, hq, d), dtype=torch.int16, device="cuda") * 0x3F80  # bf16 1.0
    out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    h.oasis_predict(q, None, 0)
    h.oasis_select_and_fetch(0)
    h.oasis_sparse_attn(q, out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    assert int(h.read("COUNTS").reshape(-1, 4)[:, 0].max()) == 0
    # verification: set 0 has nothing to attend; draft j attends to draft
    # tokens 1..j, whose values are v_i = i + 1 in every dimension
    D = 2
    drafts = q.unsqueeze(0).repeat(D, 1, 1, 1).contiguous()
    kd = torch.zeros((D, B, hkv, d), dtype=torch.int16, device="cuda")
    vals = [0x3F80, 0x4000]  # bf16 1.0, 2.0
    vd = torch.stack([torch.full((B, hkv, d), v, dtype=torch.int16, device="cuda") for v in vals])
    vout = torch.full((1 + D, B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    h.oasis_sparse_attn_verify(q, drafts, D, kd, vd, vout)
    torch.cuda.synchronize()
    assert torch.all(vout[0] == 0)
    assert torch.all(vout[1] == 1.0)          # one token, value 1
    assert torch.allclose(vout[2], torch.full_like(vout[2], 1.5), atol=1e-6)  # equal logits
    h.oasis_check()


def test_runs_are_bitwise_deterministic():
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B.with_(batch=4, prefix_tokens=16 * 400 + 3)
    outs = []
    for _ in range(2):
        r = LayerRunner(w, 5)
        r.admission()
        res = []
        for t in range(1, 6):
            r.step(t)
            torch.cuda.synchronize()
            res.append((r.out.cpu().numpy().copy(), r.h.read("ATT_BLOCK").copy(),
                        r.h.read("SLOT_BLOCK").copy()))
        outs.append(res)
        r.h.close()
    for a, b in zip(*outs):
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_stats_count_fetches_and_hits():
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B.with_(batch=2, prefix_tokens=16 * 300)
    r = LayerRunner(w, 4)
    r.admission()
    for t in range(1, 5):
        r.step(t)
    st = r.h.oasis_get_stats()
    units = w.batch * w.kv_heads
    assert st["steps"] == 5 and st["tokens"] == w.prefix_tokens + 4
    admission = units * w.k_blocks
    assert admission <= st["fetched"] <= admission + 4 * units * r.cap
    assert st["hits"] + st["misses"] == 5 * units * w.k_blocks
    assert st["bytes_fetched"] == st["fetched"] * 2 * 16 * 128 * 2


def test_sampled_kernel_timing_counts_one_launch_per_period():
    from lookahead_sparse_kv_oasis_amd import TIME, OasisError
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    w = synth.QWEN3_8B.with_(batch=1, prefix_tokens=16 * 200)
    r = LayerRunner(w, 7)
    r.admission()
    r.h.oasis_set_timing(TIME["score"] | TIME["attn"])
    r.h.oasis_set_timing_period(3)
    for t in range(1, 8):
        r.step(t)
    tm = r.h.oasis_get_timing()
    # launches 0, 3 and 6 of each class carry events
    assert tm["n_score"] == 3 and tm["n_attn"] == 3 and tm["n_append"] == 0
    assert tm["ms_score"] > 0 and tm["ms_attn"] > 0
    with pytest.raises(OasisError):
        r.h.oasis_set_timing_period(0)


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (16 * 1007, 3), (64 << 20, 300),
                                        ((64 << 20) + 16 * 5, 2048)])
def test_stream_read_folds_every_word_of_the_buffer(nbytes, wgs):
    """The streaming-read helper behind the measured HBM read peak: the XOR of
    its per-workgroup words equals the XOR of the buffer, for ragged sizes and
    for more workgroups than 16 KB pieces."""
    from lookahead_sparse_kv_oasis_amd import stream_read
    host = np.random.default_rng(nbytes).integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    stream_read(buf, sink, wgs)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)
