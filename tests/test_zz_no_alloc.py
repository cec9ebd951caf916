"""The allocation-free attention entry point (oasis_sparse_attn_noalloc)
against the handle's oasis_sparse_attn on the same state, on two calls in a
row, the second with a smaller input; and its argument and capacity checks."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3     # attention bar against the oracle
SAME = 1e-5    # same kernels, partials merged in another order


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("shape", ["qwen3_8b", "qwen3_32b"])
def test_noalloc_attention_matches_the_handle_on_two_calls(shape):
    """4 heads per KV head (vector-ALU P V) and 8 (the 16-row matrix-core
    tile over resident blocks, twice the partial rows)."""
    import lookahead_sparse_kv_oasis_amd as L
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner
    L.lib()
    if shape == "qwen3_8b":
        w = synth.QWEN3_8B.with_(batch=8, prefix_tokens=16 * 600 + 9)
    else:
        w = synth.QWEN3_32B.with_(batch=4, prefix_tokens=16 * 600 + 9)
    run = LayerRunner(w, 3)
    h = run.h
    run.admission()
    for t in range(1, 4):
        run.step(t)
    torch.cuda.synchronize()
    ref = run.out.clone()
    K, S, T = h.k_blocks, h.slots, h.oasis_tokens()
    slots = _dev(h.read("SLOTS", np.uint8))
    ab, ast, cnt = _dev(h.read("ATT_BLOCK")), _dev(h.read("ATT_SLOT")), _dev(h.read("COUNTS"))
    B, Hq, Hkv = w.batch, w.q_heads, w.kv_heads

    # first call: the whole batch
    desc = L.oasis_attn_desc(B, Hq, Hkv, 128, 16, K, S, 0)
    out = torch.full_like(ref, float("nan"))
    assert L.sparse_attn_noalloc(desc, run.q, slots, ab, ast, cnt, T, out) == L.OASIS_OK
    torch.cuda.synchronize()
    err = float((out - ref).abs().max())
    assert err <= SAME, f"whole batch: {err:.3g}"

    # second call right after, smaller: the first half of the batch rows
    half = B // 2
    desc2 = L.oasis_attn_desc(half, Hq, Hkv, 128, 16, K, S, 0)
    out2 = torch.full((half, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    assert L.sparse_attn_noalloc(desc2, run.q[:half], slots, ab, ast, cnt, T, out2) == L.OASIS_OK
    torch.cuda.synchronize()
    err2 = float((out2 - ref[:half]).abs().max())
    assert err2 <= SAME, f"half batch: {err2:.3g}"

    # and against the oracle on two units of the second call
    qf = oracle.to_f64(synth.queries(w), w.dtype)
    ab_h, cnt_h = h.read("ATT_BLOCK"), h.read("COUNTS")
    got = out2.cpu().numpy()
    G = w.group
    for (b, hh) in [(0, 0), (half - 1, Hkv - 1)]:
        u = b * Hkv + hh
        keys, vals = synth.unit_kv(w, b, hh, T)
        exp = oracle.attention(qf[b, hh * G:(hh + 1) * G], keys, vals, w.dtype, w.block_size, T,
                               ab_h[u * K:u * K + int(cnt_h[u * 4])])
        e = float(np.max(np.abs(got[b, hh * G:(hh + 1) * G].astype(np.float64) - exp)))
        assert e <= TOL, f"unit {(b, hh)}: {e:.3g}"


def test_noalloc_attention_rejects_bad_shapes_and_oversized_calls():
    import lookahead_sparse_kv_oasis_amd as L
    q = torch.zeros((1, 4, 128), dtype=torch.int16, device="cuda")
    slots = torch.zeros(2 * 16 * 128 * 8, dtype=torch.int16, device="cuda")
    lists = torch.zeros(8, dtype=torch.int32, device="cuda")
    counts = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 4, 128), dtype=torch.float32, device="cuda")
    f = L.sparse_attn_noalloc
    assert f(L.oasis_attn_desc(1, 4, 1, 64, 16, 8, 8, 0), q, slots, lists, lists, counts, 16,
             out) == L.OASIS_E_INVAL                   # head_dim
    assert f(L.oasis_attn_desc(1, 12, 1, 128, 16, 8, 8, 0), q, slots, lists, lists, counts, 16,
             out) == L.OASIS_E_INVAL                   # 12 heads per KV head
    assert f(L.oasis_attn_desc(1, 4, 1, 128, 16, 8, 8, 0), q, slots, lists, lists, None, 16,
             out) == L.OASIS_E_INVAL                   # null counts
    # needs more partial rows than the library's array holds: nothing is launched
    assert f(L.oasis_attn_desc(8192, 64, 8, 128, 16, 128, 128, 0), q, slots, lists, lists,
             counts, 16, out) == L.OASIS_E_CAPACITY
    # a valid tiny call still works after the rejected ones (one empty list)
    assert f(L.oasis_attn_desc(1, 4, 1, 128, 16, 8, 8, 0), q, slots, lists, lists, counts, 16,
             out) == L.OASIS_OK
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0
