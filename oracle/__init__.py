"""fp64 CPU oracle for the OasisKV per-layer decode step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it; the product library never imports, links or calls
anything here.  The arithmetic lives in ``oasis_oracle.c`` (plain loops,
fp64); this module loads it with ctypes and sequences one unit's decode
steps in the order append -> score -> top-K -> select/cap/LRU -> gather ->
attention.

Sources: the OasisKV explainer page ("OasisKV: Scaling In-Decode KV Cache
Beyond HBM with Lookahead Sparse Prefetching"): Fig. 7, Fig. 8, Fig. 9,
Table 2, the explanatory diagram and the capped-eviction glossary entry; and
the "KV cache offloading, week 2" study notes, sections 2 and 3.

Parity status of each function (what pins it, outside itself) is listed in
the tests under ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oasis_oracle.c")
_LIB = os.path.join(_HERE, "liboasis_oracle.so")
# OASIS_ORACLE_SANITIZE=1 loads an AddressSanitizer + UndefinedBehaviorSanitizer
# build instead (the process must preload gcc's libasan; tests/test_sanitizers.py
# runs the oracle tests that way in a child process).
_SAN_LIB = os.path.join(os.path.dirname(_HERE), "_build", "san", "liboasis_oracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
             "-fno-sanitize-recover=undefined"]

F32 = 0
BF16 = 1


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with plain gcc (no fast-math, no shared headers).

    sanitize=True builds the AddressSanitizer + UndefinedBehaviorSanitizer
    variant (same source, -O1 -g) into _build/san/."""
    out = _SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        tmp = out + ".tmp%d" % os.getpid()
        opt = SAN_FLAGS if sanitize else ["-O2"]
        subprocess.check_call(["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        san = os.environ.get("OASIS_ORACLE_SANITIZE") == "1"
        path = build(force=False, sanitize=san)
        L = ctypes.CDLL(path)
        vp, dp, ip, fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), \
            ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.orc_kv_bytes_per_token.restype = ctypes.c_uint64
        L.orc_kv_bytes_per_token.argtypes = [i64, i64, i64, i64]
        L.orc_block_summary.restype = ctypes.c_int
        L.orc_block_summary.argtypes = [vp, i32, i64, i32, i32, i64, dp, dp]
        L.orc_score.restype = None
        L.orc_score.argtypes = [dp, dp, i64, i32, dp, i32, dp]
        L.orc_topk.restype = ctypes.c_int
        L.orc_topk.argtypes = [fp, i64, i32, ip]
        L.orc_select.restype = ctypes.c_int
        L.orc_select.argtypes = [ip, ip, i32, ip, i32, i32, ctypes.c_int32,
                                 ip, ip, ip, ip, ip, ip, ip, i32]
        L.orc_attention.restype = None
        L.orc_attention.argtypes = [dp, i32, vp, vp, i32, i32, i32, i64, ip, i32, dp]
        L.orc_dense_attention.restype = None
        L.orc_dense_attention.argtypes = [dp, i32, vp, vp, i32, i32, i64, dp]
        _lib = L
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _storage(a: np.ndarray, dtype: int) -> np.ndarray:
    want = np.float32 if dtype == F32 else np.uint16
    if a.dtype != want:
        raise TypeError(f"storage array must be {want}, got {a.dtype}")
    return np.ascontiguousarray(a)


def to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact double values of a storage array (fp32, or bf16 bits)."""
    if dtype == F32:
        return a.astype(np.float64)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ functions

def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(lib().orc_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def cap_from_ratio(ratio, k_blocks: int) -> int:
    """Per-(b, KV head) blocks fetched per step for a fetch ratio of the budget.

    READING of the fetch-cap ablation (Table 2): the cap is a share of the
    K-block budget, floored, at least one block; ``None`` means fetch all.
    """
    if ratio is None:
        return k_blocks
    if ratio <= 0:
        return 0
    return max(1, int(math.floor(ratio * k_blocks + 1e-9)))


def block_summary(keys: np.ndarray, dtype: int, T: int, bs: int, j: int):
    keys = _storage(keys, dtype)
    d = keys.shape[-1]
    mx = np.empty(d, np.float64)
    mn = np.empty(d, np.float64)
    rc = lib().orc_block_summary(keys.ctypes.data, dtype, T, d, bs, j,
                                 _p(mx, ctypes.c_double), _p(mn, ctypes.c_double))
    if rc != 0:
        raise ValueError("empty block")
    return mx, mn


def score(mx: np.ndarray, mn: np.ndarray, x: np.ndarray) -> np.ndarray:
    mx = np.ascontiguousarray(mx, np.float64)
    mn = np.ascontiguousarray(mn, np.float64)
    x = np.ascontiguousarray(x, np.float64)
    nb, d = mx.shape
    out = np.empty(nb, np.float64)
    lib().orc_score(_p(mx, ctypes.c_double), _p(mn, ctypes.c_double), nb, d,
                    _p(x, ctypes.c_double), x.shape[0], _p(out, ctypes.c_double))
    return out


def topk(s32: np.ndarray, k: int) -> np.ndarray:
    s32 = np.ascontiguousarray(s32, np.float32)
    ids = np.empty(k, np.int32)
    rc = lib().orc_topk(_p(s32, ctypes.c_float), s32.shape[0], k, _p(ids, ctypes.c_int32))
    if rc == -1:
        raise FloatingPointError("non-finite score")
    if rc != 0:
        raise MemoryError
    return ids


def select(slot_block: np.ndarray, last_used: np.ndarray, ids: np.ndarray, cap: int, t: int,
           attend_all: bool = False):
    """Diff / cap / LRU for one unit; updates slot_block and last_used in place.

    attend_all: the attended list is every block held after the step (hits,
    then the other held blocks in slot order, then the fetched ones) instead
    of the selected blocks now held."""
    S = slot_block.shape[0]
    K = ids.shape[0]
    assert slot_block.dtype == np.int32 and last_used.dtype == np.int32
    ids = np.ascontiguousarray(ids, np.int32)
    fb = np.full(max(cap, 1), -1, np.int32)
    fs = np.full(max(cap, 1), -1, np.int32)
    ab = np.full(max(K, S), -1, np.int32)
    ast = np.full(max(K, S), -1, np.int32)
    nf, na, nh = (ctypes.c_int32(0) for _ in range(3))
    I = ctypes.c_int32
    rc = lib().orc_select(_p(slot_block, I), _p(last_used, I), S, _p(ids, I), K, cap, t,
                          _p(fb, I), _p(fs, I), ctypes.byref(nf), _p(ab, I), _p(ast, I),
                          ctypes.byref(na), ctypes.byref(nh), int(bool(attend_all)))
    if rc != 0:
        raise ValueError("invalid residency state")
    return dict(fetch_block=fb[:nf.value].copy(), fetch_slot=fs[:nf.value].copy(),
                att_block=ab[:na.value].copy(), att_slot=ast[:na.value].copy(),
                n_hit=nh.value)


def attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, dtype: int, bs: int, T: int,
              blocks: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    keys, vals = _storage(keys, dtype), _storage(vals, dtype)
    blocks = np.ascontiguousarray(blocks, np.int32)
    nq, d = q.shape
    out = np.empty((nq, d), np.float64)
    lib().orc_attention(_p(q, ctypes.c_double), nq, keys.ctypes.data, vals.ctypes.data, dtype,
                        d, bs, T, _p(blocks, ctypes.c_int32), blocks.shape[0],
                        _p(out, ctypes.c_double))
    return out


def dense_attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, dtype: int, T: int):
    q = np.ascontiguousarray(q, np.float64)
    keys, vals = _storage(keys, dtype), _storage(vals, dtype)
    nq, d = q.shape
    out = np.empty((nq, d), np.float64)
    lib().orc_dense_attention(_p(q, ctypes.c_double), nq, keys.ctypes.data, vals.ctypes.data,
                              dtype, d, T, _p(out, ctypes.c_double))
    return out


# ------------------------------------------------------------ one unit

class _PhaseClock:
    """Adds the wall time since the previous lap to phase_times[name]; does
    nothing when phase_times is None (timing only, no effect on results)."""

    def __init__(self, phase_times):
        self.d = phase_times
        self.t = time.perf_counter() if phase_times is not None else 0.0

    def lap(self, name):
        if self.d is not None:
            now = time.perf_counter()
            self.d[name] = self.d.get(name, 0.0) + (now - self.t)
            self.t = now


class Unit:
    """Decode-step state of one (batch row, KV head) unit.

    keys / vals: storage arrays [n_tokens][d] holding the prefix and every
    token to be appended (the host-resident full KV of [OASIS] Fig. 7).
    """

    def __init__(self, keys, vals, dtype, bs, T0, k_blocks, slots, slot_block=None,
                 last_used=None):
        self.keys, self.vals = _storage(keys, dtype), _storage(vals, dtype)
        self.dtype, self.bs, self.T = dtype, bs, T0
        self.d = keys.shape[1]
        self.K, self.S = k_blocks, slots
        cap_blocks = (keys.shape[0] + bs - 1) // bs
        self.mx = np.zeros((cap_blocks, self.d))
        self.mn = np.zeros((cap_blocks, self.d))
        for j in range(self.nb):
            self.mx[j], self.mn[j] = block_summary(self.keys, dtype, T0, bs, j)
        self.slot_block = (np.full(slots, -1, np.int32) if slot_block is None
                           else np.array(slot_block, np.int32))
        self.last_used = (np.full(slots, -1, np.int32) if last_used is None
                          else np.array(last_used, np.int32))

    @property
    def nb(self) -> int:
        return (self.T + self.bs - 1) // self.bs

    def append(self):
        """Token T becomes valid; its block's summary is pooled again."""
        if self.T >= self.keys.shape[0]:
            raise IndexError("append past the generated tokens")
        self.T += 1
        j = (self.T - 1) // self.bs
        self.mx[j], self.mn[j] = block_summary(self.keys, self.dtype, self.T, self.bs, j)

    def evict(self, blocks):
        for blk in blocks:
            hit = np.nonzero(self.slot_block == blk)[0]
            for s in hit:
                self.slot_block[s] = -1

    def score(self, x_rows) -> np.ndarray:
        return score(self.mx[:self.nb], self.mn[:self.nb], x_rows)

    def step(self, t, x_rows, q_rows, cap, append=True, evict_blocks=None, scores32=None,
             phase_times=None):
        """One decode step.  Returns a record of every intermediate result.

        scores32: if given, the fp32 scores to select on (parity hook);
        otherwise the oracle's own fp64 scores rounded to fp32.
        phase_times: if given, a dict to which the wall time of each phase
        (append, score, topk, select, attention) is added.
        """
        clock = _PhaseClock(phase_times)
        if evict_blocks is not None and len(evict_blocks):
            self.evict(evict_blocks)
        if append:
            self.append()
        clock.lap("append")
        s64 = self.score(x_rows)
        clock.lap("score")
        s32 = s64.astype(np.float32) if scores32 is None else np.asarray(scores32, np.float32)
        ids = topk(s32, self.K)
        clock.lap("topk")
        sel = select(self.slot_block, self.last_used, ids, cap, t)
        clock.lap("select")
        out = attention(q_rows, self.keys, self.vals, self.dtype, self.bs, self.T,
                        sel["att_block"])
        clock.lap("attention")
        rec = dict(t=t, T=self.T, scores64=s64, scores32=s32, ids=ids, out=out,
                   slot_block=self.slot_block.copy(), last_used=self.last_used.copy())
        rec.update(sel)
        return rec


    def step_ahead(self, t, x_rows, q_rows, cap, append=True, scores32=None, attend=True):
        """One decode step in the lookahead order ([OASIS] Fig. 8): token t is
        appended; the current query attends over the blocks that the previous
        step selected (self.att); then the draft rows x_rows are scored and the
        top-K, diff, cap and LRU choose the set for the next step's attention.
        attend=False (the untimed admission step) skips the attention."""
        if append:
            self.append()
        att = getattr(self, "att", np.zeros(0, np.int32))
        out = (attention(q_rows, self.keys, self.vals, self.dtype, self.bs, self.T, att)
               if attend else None)
        s64 = self.score(x_rows)
        s32 = s64.astype(np.float32) if scores32 is None else np.asarray(scores32, np.float32)
        ids = topk(s32, self.K)
        sel = select(self.slot_block, self.last_used, ids, cap, t)
        self.att = sel["att_block"]
        rec = dict(t=t, T=self.T, scores64=s64, scores32=s32, ids=ids, out=out, attended=att,
                   slot_block=self.slot_block.copy(), last_used=self.last_used.copy())
        rec.update(sel)
        return rec


    def step_corrected(self, t, q_rows, cap_correct, x_draft_rows, cap, append=True):
        """One decode step with decode-time miss correction (the corrective
        transfers the OasisKV page names among its limits) on top of the
        lookahead prefetch: token t is appended; the current query alone is
        scored and its top-K selected with cap_correct (the blocks the earlier
        prediction missed are fetched now, synchronously); the current query
        attends over that set; then the drafts alone select (cap) the set to
        prefetch for step t+1.  Both selects use recency t."""
        if append:
            self.append()
        e64 = self.score(q_rows)
        e32 = e64.astype(np.float32)
        exact = topk(e32, self.K)
        corr = select(self.slot_block, self.last_used, exact, cap_correct, t)
        out = attention(q_rows, self.keys, self.vals, self.dtype, self.bs, self.T,
                        corr["att_block"])
        s64 = self.score(x_draft_rows)
        s32 = s64.astype(np.float32)
        ids = topk(s32, self.K)
        pre = select(self.slot_block, self.last_used, ids, cap, t)
        self.att = pre["att_block"]
        return dict(t=t, T=self.T, exact_scores64=e64, exact_scores32=e32, exact_ids=exact,
                    correction=corr, out=out, scores64=s64, scores32=s32, ids=ids,
                    prefetch=pre, slot_block=self.slot_block.copy(),
                    last_used=self.last_used.copy())


def attention_verify(q_sets, keys, vals, dtype: int, bs: int, T: int, blocks, k_drafts, v_drafts):
    """Verification attention ([OASIS] Fig. 7, right): the current query and
    each draft query over the sparse KV in one pass, plain fp64.  q_sets [1 + D][G][d]: set 0 is the current query
    (position T - 1), set j the j-th draft (position T - 1 + j).  Set j attends
    over the valid tokens of the attended blocks plus draft tokens 1..j
    (k_drafts / v_drafts [D][d], exact values): causal within the drafts.
    Returns [1 + D][G][d]."""
    keys, vals = _storage(keys, dtype), _storage(vals, dtype)
    kf = np.asarray(k_drafts, np.float64)
    vf = np.asarray(v_drafts, np.float64)
    toks = []
    for blk in np.asarray(blocks, np.int64):
        p0 = int(blk) * bs
        toks.extend(range(p0, min(p0 + bs, T)))
    toks = np.asarray(toks, np.int64)
    k_ctx = to_f64(keys[toks], dtype) if len(toks) else np.zeros((0, keys.shape[1]))
    v_ctx = to_f64(vals[toks], dtype) if len(toks) else np.zeros((0, vals.shape[1]))
    q_sets = np.asarray(q_sets, np.float64)
    d = q_sets.shape[-1]
    out = np.zeros(q_sets.shape, np.float64)
    for j in range(q_sets.shape[0]):
        kk = np.concatenate([k_ctx, kf[:j]], axis=0)
        vv = np.concatenate([v_ctx, vf[:j]], axis=0)
        if kk.shape[0] == 0:
            continue
        lg = q_sets[j] @ kk.T / np.sqrt(d)
        lg -= lg.max(axis=1, keepdims=True)
        p = np.exp(lg)
        out[j] = (p @ vv) / p.sum(axis=1, keepdims=True)
    return out


def unit_rows(q, drafts_t, b, h, group):
    """Query rows of one unit: the G group heads of the current query, then of
    every draft (scoring), and the current query alone (attention)."""
    g0, g1 = h * group, (h + 1) * group
    cur = q[b, g0:g1]
    rows = [cur] + [drafts_t[i, b, g0:g1] for i in range(drafts_t.shape[0])]
    return np.concatenate(rows, axis=0), cur


def draft_rows(drafts_t, b, h, group):
    """Scoring rows of one unit from the drafts alone (lookahead prediction)."""
    g0, g1 = h * group, (h + 1) * group
    return np.concatenate([drafts_t[i, b, g0:g1] for i in range(drafts_t.shape[0])], axis=0)
