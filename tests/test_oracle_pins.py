"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these retypes an oracle formula: each checks a printed value, a
closed form, an invariant, a brute-force enumeration or a special case that
reduces to something independent of the code under test.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- KV sizes

def test_kv_bytes_per_token_matches_printed_examples():
    g = json.load(open(os.path.join(GOLD, "kv_bytes.json")))
    for row in g["per_token"]:
        got = oracle.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"],
                                        row["dtype_bytes"])
        if "bytes" in row:
            assert got == row["bytes"], row
        else:
            assert got == row["bytes_approx_kb"] * 1024, row


def test_kv_bytes_per_context_matches_printed_table():
    g = json.load(open(os.path.join(GOLD, "kv_bytes.json")))
    per_tok = oracle.kv_bytes_per_token(80, 8, 128, 2)
    for row in g["per_context_llama3_70b_fp16"]:
        gb = per_tok * row["tokens"] / 1e9
        # the page gives rounded "about" figures (1.34 -> 1.3, 42.9 -> 42)
        assert abs(gb - row["approx_gb"]) / row["approx_gb"] < 0.05, (row, gb)
    per_tok8 = oracle.kv_bytes_per_token(80, 8, 128, 1)
    for row in g["per_context_llama3_70b_int8"]:
        gb = per_tok8 * row["tokens"] / 1e9
        assert abs(gb - row["approx_gb"]) / row["approx_gb"] < 0.05


def test_qwen3_8b_host_kv_footprint():
    # 36 layers x 2 x 8 KV heads x 128 x 2 B; the 36-layer workload's pinned
    # full KV is that times context times batch.
    assert oracle.kv_bytes_per_token(36, 8, 128, 2) == 147456
    w = synth.QWEN3_8B_36L
    total = oracle.kv_bytes_per_token(w.layers, w.kv_heads, w.head_dim, 2) * \
        w.prefix_tokens * w.batch
    assert total == 36 * 64 * 65536 * 8 * 2 * 128 * 2


# ---------------------------------------------------------------- summary

@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_block_summary_is_the_tight_box(dtype):
    rng = _rng(1)
    d, bs, T = 12, 16, 16 * 5 + 7           # ragged tail block of 7 tokens
    x = rng.standard_normal((T + 9, d)).astype(np.float32)
    x[T:] = 1e30                           # tokens past T must not be pooled
    keys = synth.encode(x, dtype)
    vals = oracle.to_f64(keys, dtype)
    for j in range((T + bs - 1) // bs):
        mx, mn = oracle.block_summary(keys, dtype, T, bs, j)
        blk = vals[j * bs:min((j + 1) * bs, T)]
        # every key of the block lies in the box, and each face is attained
        assert np.all(blk <= mx[None]) and np.all(blk >= mn[None])
        for c in range(d):
            assert np.any(blk[:, c] == mx[c]) and np.any(blk[:, c] == mn[c])
        assert np.all(mx < 1e29)


def test_block_summary_single_token_block():
    keys = synth.encode(np.arange(6, dtype=np.float32).reshape(2, 3) - 2.5, synth.F32)
    mx, mn = oracle.block_summary(keys, synth.F32, 1, 16, 0)
    assert np.array_equal(mx, mn) and np.array_equal(mx, [-2.5, -1.5, -0.5])


def test_block_summary_empty_block_rejected():
    keys = np.zeros((4, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.block_summary(keys, synth.F32, 4, 4, 1)


# ---------------------------------------------------------------- score

def test_score_equals_box_corner_enumeration():
    """The block score is the largest x.z over the 2^d corners of [mn, mx]:
    a linear function attains its maximum over a box at a corner."""
    rng = _rng(2)
    d, nb, nq = 6, 9, 3
    mx = rng.standard_normal((nb, d))
    mn = mx - np.abs(rng.standard_normal((nb, d)))
    x = rng.standard_normal((nq, d))
    x[0, 2] = 0.0
    got = oracle.score(mx, mn, x)
    for j in range(nb):
        best = -np.inf
        for pick in itertools.product([0, 1], repeat=d):
            z = np.where(np.array(pick) == 1, mx[j], mn[j])
            best = max(best, float((x @ z).max()))
        assert abs(got[j] - best) <= 1e-12 * max(1.0, abs(best))


def test_score_bounds_every_token_and_is_tight_for_one_token_blocks():
    rng = _rng(3)
    d, bs, T = 16, 16, 16 * 6 + 1          # the last block holds one token
    keys = synth.encode(rng.standard_normal((T, d)).astype(np.float32), synth.F32)
    kf = oracle.to_f64(keys, synth.F32)
    nb = (T + bs - 1) // bs
    mx = np.empty((nb, d))
    mn = np.empty((nb, d))
    for j in range(nb):
        mx[j], mn[j] = oracle.block_summary(keys, synth.F32, T, bs, j)
    x = rng.standard_normal((5, d))
    s = oracle.score(mx, mn, x)
    for j in range(nb):
        dots = x @ kf[j * bs:min((j + 1) * bs, T)].T
        assert s[j] >= dots.max() - 1e-12
    assert abs(s[nb - 1] - (x @ kf[T - 1]).max()) < 1e-12


def test_score_aggregates_by_max_over_rows():
    rng = _rng(4)
    mx = rng.standard_normal((7, 5))
    mn = mx - 1.0
    x = rng.standard_normal((4, 5))
    each = np.stack([oracle.score(mx, mn, x[i:i + 1]) for i in range(4)])
    assert np.array_equal(oracle.score(mx, mn, x), each.max(axis=0))


def test_score_sign_split_identity():
    """sum_c max(x mx, x mn) == x+ . mx + x- . mn (the contraction form)."""
    rng = _rng(5)
    mx = rng.standard_normal((11, 8))
    mn = mx - np.abs(rng.standard_normal((11, 8)))
    x = rng.standard_normal((1, 8))
    xp, xm = np.maximum(x, 0), np.minimum(x, 0)
    ref = (xp @ mx.T + xm @ mn.T)[0]
    assert np.allclose(oracle.score(mx, mn, x), ref, rtol=0, atol=1e-12)


def test_score_degenerate_box_is_the_exact_dot():
    rng = _rng(6)
    k = rng.standard_normal((3, 10))
    x = rng.standard_normal((2, 10))
    assert np.allclose(oracle.score(k, k, x), (x @ k.T).max(axis=0), atol=1e-12)


# ---------------------------------------------------------------- top-K

def _brute_rank_topk(s, k):
    n = len(s)
    sel = [j for j in range(n)
           if sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j)) < k]
    rank = {j: sum(1 for i in sel if s[i] > s[j] or (s[i] == s[j] and i < j)) for j in sel}
    out = [-1] * k
    for j in sel:
        out[rank[j]] = j
    return out


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_rank_count_with_ties(seed):
    rng = _rng(100 + seed)
    n = int(rng.integers(1, 40))
    k = int(rng.integers(1, 12))
    s = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.25)   # many ties
    if seed % 3 == 0:
        s = rng.standard_normal(n).astype(np.float32)
    got = oracle.topk(s, k)
    assert list(got) == _brute_rank_topk(list(s), k)


def test_topk_signed_zero_and_padding():
    s = np.array([-0.0, 0.0, -1.0], np.float32)
    assert list(oracle.topk(s, 5)) == [0, 1, 2, -1, -1]
    s = np.array([0.0, -0.0], np.float32)
    assert list(oracle.topk(s, 1)) == [0]


def test_topk_rejects_nonfinite():
    with pytest.raises(FloatingPointError):
        oracle.topk(np.array([1.0, np.nan], np.float32), 1)
    with pytest.raises(FloatingPointError):
        oracle.topk(np.array([np.inf], np.float32), 1)


# ---------------------------------------------------------------- select

def test_select_reproduces_hand_worked_lru_trace():
    g = json.load(open(os.path.join(GOLD, "lru_trace.json")))
    sb = np.array(g["initial"]["slot_block"], np.int32)
    lu = np.array(g["initial"]["last_used"], np.int32)
    for st in g["steps"]:
        ids = oracle.topk(np.array(st["scores"], np.float32), g["k"])
        assert list(ids) == st["ids"]
        r = oracle.select(sb, lu, ids, g["cap"], st["t"])
        for key in ("fetch_block", "fetch_slot", "att_block", "att_slot"):
            assert list(r[key]) == st[key], (st["t"], key)
        assert r["n_hit"] == st["n_hit"]
        assert list(sb) == st["slot_block"] and list(lu) == st["last_used"], st["t"]


def test_select_attend_all_reading_on_hand_worked_trace():
    """The attend-every-held-block reading on the same trace: the attended
    lists of the worked example, and residency, recency and fetches equal to
    the default reading's at every step."""
    g = json.load(open(os.path.join(GOLD, "lru_trace.json")))
    sb = np.array(g["initial"]["slot_block"], np.int32)
    lu = np.array(g["initial"]["last_used"], np.int32)
    for st in g["steps"]:
        ids = np.array(st["ids"], np.int32)
        r = oracle.select(sb, lu, ids, g["cap"], st["t"], attend_all=True)
        assert list(r["att_block"]) == st["att_block_all"], st["t"]
        assert list(r["att_slot"]) == st["att_slot_all"], st["t"]
        for key in ("fetch_block", "fetch_slot"):
            assert list(r[key]) == st[key], (st["t"], key)
        assert r["n_hit"] == st["n_hit"]
        assert list(sb) == st["slot_block"] and list(lu) == st["last_used"], st["t"]


def _check_select_invariants(sb0, lu0, sb, lu, ids, cap, t, r):
    sel = [i for i in ids if i >= 0]
    held0 = {b for b in sb0 if b >= 0}
    held1 = [b for b in sb if b >= 0]
    assert len(held1) == len(set(held1))                       # slots unique
    assert len(r["fetch_block"]) <= cap                         # transfer cap
    misses = [b for b in sel if b not in held0]
    assert len(r["fetch_block"]) == min(cap, len(misses))
    assert list(r["fetch_block"]) == misses[:len(r["fetch_block"])]
    for b in sel:                                               # hits never evicted
        if b in held0:
            assert b in held1
    if cap >= len(misses):                                      # uncapped => all resident
        assert set(sel) <= set(held1)
    att = list(r["att_block"])
    assert sorted(att) == sorted(b for b in sel if b in held1)  # A = Sel n R'
    for b, s in zip(r["att_block"], r["att_slot"]):
        assert sb[s] == b and lu[s] == t
    changed = [s for s in range(len(sb)) if sb[s] != sb0[s]]
    assert sorted(changed) == sorted(r["fetch_slot"])
    for s in range(len(sb)):                                    # untouched slots keep recency
        if sb[s] >= 0 and sb[s] not in sel:
            assert lu[s] == lu0[s]


@pytest.mark.parametrize("seed", range(30))
def test_select_invariants_random(seed):
    rng = _rng(500 + seed)
    nb = int(rng.integers(2, 40))
    k = int(rng.integers(1, min(nb, 10) + 1))
    S = int(rng.integers(k, k + 8))
    cap = int(rng.integers(0, k + 2))
    sb = np.full(S, -1, np.int32)
    lu = np.full(S, -1, np.int32)
    nres = int(rng.integers(0, min(S, nb) + 1))
    sb[rng.choice(S, nres, replace=False)] = rng.choice(nb, nres, replace=False)
    lu[:] = rng.integers(-1, 5, S)
    for t in range(5, 12):
        s = rng.integers(0, 6, nb).astype(np.float32)
        ids = oracle.topk(s, k)
        sb0, lu0 = sb.copy(), lu.copy()
        r = oracle.select(sb, lu, ids, cap, t)
        _check_select_invariants(sb0, lu0, sb, lu, ids, cap, t, r)


@pytest.mark.parametrize("seed", range(20))
def test_select_attend_all_invariants_random(seed):
    """Attend-all reading: the list is the hits in top-K order, then every
    other held block in slot order, then the fetched blocks; it names each
    held block once with its slot; the state update is the default's; with
    S = K and an uncapped fetch it is the default attended set."""
    rng = _rng(900 + seed)
    nb = int(rng.integers(2, 40))
    k = int(rng.integers(1, min(nb, 10) + 1))
    S = k if seed % 2 else int(rng.integers(k, k + 8))
    cap = k if seed % 4 == 1 else int(rng.integers(0, k + 2))
    sb = np.full(S, -1, np.int32)
    lu = np.full(S, -1, np.int32)
    nres = int(rng.integers(0, min(S, nb) + 1))
    sb[rng.choice(S, nres, replace=False)] = rng.choice(nb, nres, replace=False)
    lu[:] = rng.integers(-1, 5, S)
    for t in range(5, 12):
        s = rng.integers(0, 6, nb).astype(np.float32)
        ids = oracle.topk(s, k)
        sb_d, lu_d = sb.copy(), lu.copy()
        rd = oracle.select(sb_d, lu_d, ids, cap, t)
        ra = oracle.select(sb, lu, ids, cap, t, attend_all=True)
        assert np.array_equal(sb, sb_d) and np.array_equal(lu, lu_d)
        assert np.array_equal(ra["fetch_block"], rd["fetch_block"])
        assert np.array_equal(ra["fetch_slot"], rd["fetch_slot"])
        nh, nf = rd["n_hit"], len(rd["fetch_block"])
        att, ats = list(ra["att_block"]), list(ra["att_slot"])
        assert att[:nh] == list(rd["att_block"][:nh])               # hits, top-K order
        assert att[len(att) - nf:] == list(rd["fetch_block"])       # fetched last
        rest = ats[nh:len(ats) - nf]
        assert rest == sorted(rest)                                  # others in slot order
        held = {int(b): s_ for s_, b in enumerate(sb) if b >= 0}
        assert sorted(att) == sorted(held) and len(att) == len(set(att))
        for b, s_ in zip(att, ats):
            assert held[b] == s_
        if S == k and {int(b) for b in ids if b >= 0} <= set(held):
            assert sorted(att) == sorted(rd["att_block"])


def test_select_rejects_duplicate_residency():
    sb = np.array([3, 3], np.int32)
    lu = np.zeros(2, np.int32)
    with pytest.raises(ValueError):
        oracle.select(sb, lu, np.array([3], np.int32), 1, 1)


def test_cap_from_ratio_reading():
    # fetch ratios of the fetch-cap ablation table, against a 128-block budget
    assert [oracle.cap_from_ratio(r, 128) for r in synth.FETCH_RATIO_SWEEP] == \
        [1, 2, 6, 12, 25, 128]
    assert oracle.cap_from_ratio(0.5, 8) == 4 and oracle.cap_from_ratio(0.001, 8) == 1


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_sparse_attention_over_all_blocks_equals_dense(dtype):
    rng = _rng(7)
    d, bs, T = 32, 16, 16 * 4 + 5
    K = synth.encode(rng.standard_normal((T, d)).astype(np.float32), dtype)
    V = synth.encode(rng.standard_normal((T, d)).astype(np.float32), dtype)
    q = rng.standard_normal((3, d)) * 2
    blocks = np.array([3, 0, 4, 1, 2], np.int32)          # any order
    sp = oracle.attention(q, K, V, dtype, bs, T, blocks)
    de = oracle.dense_attention(q, K, V, dtype, T)
    assert np.max(np.abs(sp - de)) < 1e-12


def test_attention_special_cases():
    rng = _rng(8)
    d, bs = 8, 4
    K = synth.encode(rng.standard_normal((12, d)).astype(np.float32), synth.F32)
    V = synth.encode(rng.standard_normal((12, d)).astype(np.float32), synth.F32)
    Vf = oracle.to_f64(V, synth.F32)
    q = rng.standard_normal((2, d))
    # one valid token (block 2 holds only token 8 when T = 9) -> out = v
    out = oracle.attention(q, K, V, synth.F32, bs, 9, np.array([2], np.int32))
    assert np.allclose(out, Vf[8][None], atol=1e-15)
    # identical keys -> equal weights -> mean of V over the attended tokens
    Ks = np.repeat(K[:1], 12, axis=0)
    out = oracle.attention(q, Ks, V, synth.F32, bs, 12, np.array([0, 2], np.int32))
    assert np.allclose(out, np.concatenate([Vf[0:4], Vf[8:12]]).mean(0)[None], atol=1e-14)
    # two tokens: weight of the first is the logistic of the logit gap
    out = oracle.attention(q, K, V, synth.F32, 1, 12, np.array([5, 7], np.int32))
    Kf = oracle.to_f64(K, synth.F32)
    for r in range(2):
        gap = (q[r] @ Kf[5] - q[r] @ Kf[7]) / math.sqrt(d)
        w = 1.0 / (1.0 + math.exp(-gap))
        assert np.allclose(out[r], w * Vf[5] + (1 - w) * Vf[7], atol=1e-14)
    # empty attended set -> zeros
    assert np.all(oracle.attention(q, K, V, synth.F32, bs, 12, np.zeros(0, np.int32)) == 0)


def test_attention_ignores_tokens_past_T():
    rng = _rng(9)
    d, bs = 8, 4
    x = rng.standard_normal((8, d)).astype(np.float32)
    K1, V1 = x.copy(), x[::-1].copy()
    K2, V2 = K1.copy(), V1.copy()
    K2[6:] = 50.0
    V2[6:] = -50.0
    q = rng.standard_normal((1, d))
    a = oracle.attention(q, K1, V1, synth.F32, bs, 6, np.array([0, 1], np.int32))
    b = oracle.attention(q, K2, V2, synth.F32, bs, 6, np.array([0, 1], np.int32))
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ verification attention

def _verify_case(seed, dtype=None):
    rng = np.random.default_rng(seed)
    d, bs, G, D = 32, 16, 2, 3
    T = 16 * 5 + 7
    dt = synth.BF16 if dtype is None else dtype
    keys = synth.encode(rng.standard_normal((T + 4, d)).astype(np.float32), dt)
    vals = synth.encode(rng.standard_normal((T + 4, d)).astype(np.float32), dt)
    kd = synth.encode(rng.standard_normal((D, d)).astype(np.float32), dt)
    vd = synth.encode(rng.standard_normal((D, d)).astype(np.float32), dt)
    q = rng.standard_normal((1 + D, G, d))
    return keys, vals, kd, vd, q, T, bs, dt


def test_verify_attention_over_every_block_is_dense_attention_of_the_extended_sequence():
    """Every block attended: query set j sees the T context tokens and draft
    tokens 1..j, so each set equals dense attention over the context with the
    first j draft tokens appended (the independent dense routine)."""
    keys, vals, kd, vd, q, T, bs, dt = _verify_case(1)
    nb = (T + bs - 1) // bs
    out = oracle.attention_verify(q, keys, vals, dt, bs, T, np.arange(nb), oracle.to_f64(kd, dt),
                                  oracle.to_f64(vd, dt))
    for j in range(q.shape[0]):
        ke = np.concatenate([keys[:T], kd[:j]], axis=0)
        ve = np.concatenate([vals[:T], vd[:j]], axis=0)
        dense = oracle.dense_attention(q[j], ke, ve, dt, T + j)
        assert np.max(np.abs(out[j] - dense)) < 1e-12


def test_verify_attention_set_zero_is_the_sparse_attention_and_drafts_are_causal():
    """Set 0 (the current query) ignores the draft tokens: it equals the plain
    sparse attention; changing draft token j changes only sets >= j."""
    keys, vals, kd, vd, q, T, bs, dt = _verify_case(2)
    blocks = np.array([4, 1, 3], np.int32)
    kf, vf = oracle.to_f64(kd, dt), oracle.to_f64(vd, dt)
    out = oracle.attention_verify(q, keys, vals, dt, bs, T, blocks, kf, vf)
    plain = oracle.attention(q[0], keys, vals, dt, bs, T, blocks)
    assert np.max(np.abs(out[0] - plain)) < 1e-12
    kf2 = kf.copy()
    kf2[1] += 1.0                       # draft token 2
    out2 = oracle.attention_verify(q, keys, vals, dt, bs, T, blocks, kf2, vf)
    assert np.array_equal(out[:2], out2[:2])
    assert np.all(np.abs(out[2:] - out2[2:]).max(axis=(1, 2)) > 0)
