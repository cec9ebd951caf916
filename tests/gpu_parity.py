"""Helpers for the GPU parity tests: run the HIP path and the fp64 oracle on the
same seeded inputs and compare them step by step.

Tolerances (written here, used by every parity test):
  - summaries, top-K ids, fetch lists, slot tables, recency, attended lists,
    slot payload bytes: bit-exact;
  - block scores: |gpu - oracle| <= 1e-4 * N_j, where N_j is the largest
    sum over c of |x_c| * max(|max_jc|, |min_jc|) over the query rows (the
    magnitude scale of the terms being summed; a pure relative error is
    undefined near zero);
  - attention output: max |gpu - oracle| <= 2e-3.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import synth
from lookahead_sparse_kv_oasis_amd import Oasis
from lookahead_sparse_kv_oasis_amd.runner import LayerRunner, to_device
from oracle.trajectory import initial_unit, workload_cap

SCORE_TOL = 1e-4
ATTN_TOL = 2e-3


def log(msg):
    print(msg, flush=True)


_POOL = None


def pool():
    """Host threads for the oracle units (its C calls release the GIL)."""
    global _POOL
    if _POOL is None:
        import os
        _POOL = ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


def every_unit(w):
    return [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]


def device_evictions(w, h, t, layer):
    """Forced evictions of step t applied on the device (oasis_evict_attended)
    from the seeded draws.  Checks the slot table afterwards against the
    harness rule applied to the GPU's own previous attended lists, for every
    unit (bit-exact), and returns the evicted blocks per unit."""
    K, S = h.k_blocks, h.slots
    ab, cnt, sb0 = h.read("ATT_BLOCK"), h.read("COUNTS"), h.read("SLOT_BLOCK")
    draws = synth.evict_draws(w, t, layer)
    h.oasis_evict_attended(torch.from_numpy(np.ascontiguousarray(draws)).cuda(),
                           w.forced_evict_frac)
    sb1 = h.read("SLOT_BLOCK")
    out = {}
    for b in range(w.batch):
        for hh in range(w.kv_heads):
            u = b * w.kv_heads + hh
            na = int(cnt[u * 4])
            ev = synth.forced_evictions(w, ab[u * K:u * K + na], na, draws[b, hh])
            exp = sb0[u * S:(u + 1) * S].copy()
            exp[np.isin(exp, ev)] = -1
            assert np.array_equal(sb1[u * S:(u + 1) * S], exp), \
                f"step {t} unit {(b, hh)}: device evictions differ"
            out[(b, hh)] = ev
    return out


def score_scale(unit: oracle.Unit, x_rows: np.ndarray) -> np.ndarray:
    nb = unit.nb
    amp = np.maximum(np.abs(unit.mx[:nb]), np.abs(unit.mn[:nb]))
    return (np.abs(x_rows) @ amp.T).max(axis=0)


def slot_payload_expected(keys, vals, blk, T, bs, dtype):
    """Rows a slot holding block blk must contain: the K and V rows of its
    tokens < T ([2][n][d]).  Rows of tokens not yet appended are never read
    (the attention bounds every block by T) and copies leave them as they
    are, so they are not compared."""
    p0 = blk * bs
    n = max(0, min(bs, T - p0))
    dt = np.float32 if dtype == synth.F32 else np.uint16
    return np.stack([keys[p0:p0 + n], vals[p0:p0 + n]]).astype(dt, copy=False)


def assert_held_rows_equal(ha, hb, what=""):
    """Two handles hold the same blocks in the same slots, with the same bytes
    in the rows of the tokens held (rows past T are never read: the fetch
    inside the attention copies whole host blocks, the gather kernel the
    held rows only)."""
    assert np.array_equal(ha.read("SLOT_BLOCK"), hb.read("SLOT_BLOCK")), what + " slot tables"
    T, S, bs = ha.oasis_tokens(), ha.slots, ha.block_size
    assert T == hb.oasis_tokens()
    blk = ha.read("SLOT_BLOCK").reshape(-1, S)
    sa = ha.read("SLOTS", np.uint8).reshape(blk.shape[0], S, 2, bs, -1)
    sb = hb.read("SLOTS", np.uint8).reshape(blk.shape[0], S, 2, bs, -1)
    rows = np.clip(T - blk.astype(np.int64) * bs, 0, bs)  # held rows per slot
    keep = np.arange(bs)[None, None, :] < rows[:, :, None]  # [units][S][bs]
    keep &= (blk >= 0)[:, :, None]
    m = np.broadcast_to(keep[:, :, None, :, None], sa.shape)
    assert np.array_equal(sa[m], sb[m]), what + " slot payloads"


class Parity:
    """GPU runner + oracle units for a sample of (b, h) units of a workload."""

    def __init__(self, w: synth.Workload, n_steps: int, units, layer: int = 0,
                 compute_units: int = 0):
        self.w, self.n_steps, self.units, self.layer = w, n_steps, list(units), layer
        n_tok = w.prefix_tokens + n_steps
        K, V = synth.layer_kv(w, n_tok, layer)
        self.K, self.V = K, V
        self.run = LayerRunner(w, n_steps, layer, kv=(K, V), compute_units=compute_units)
        self.cap = workload_cap(w)
        mk = lambda k: initial_unit(w, k[0], k[1], n_steps, layer, kv=(K[k[0], k[1]], V[k[0], k[1]]))
        self.oru = dict(zip(self.units, pool().map(mk, self.units)))
        self.qf = oracle.to_f64(synth.queries(w, layer), w.dtype)
        self.G = w.group
        h = self.run.h
        self.NBmax = h.nb_max
        self.scores_dev = torch.empty((w.batch, w.kv_heads, self.NBmax), dtype=torch.float32,
                                      device="cuda")
        self.prev_att = {}

    # ------------------------------------------------------------ checks
    def check_summary(self):
        w, h = self.w, self.run.h
        dt = np.float32 if w.dtype == synth.F32 else np.uint16
        per_unit = self.NBmax * 2 * w.head_dim
        for (b, hh) in self.units:
            u = b * w.kv_heads + hh
            got = h.read_range("SUMMARY", u * per_unit * np.dtype(dt).itemsize,
                               per_unit * np.dtype(dt).itemsize, dt).reshape(self.NBmax, 2, -1)
            unit = self.oru[(b, hh)]
            nb = unit.nb
            exp_mx = synth.encode(unit.mx[:nb].astype(np.float32), w.dtype)
            exp_mn = synth.encode(unit.mn[:nb].astype(np.float32), w.dtype)
            bits = np.uint32 if w.dtype == synth.F32 else np.uint16
            assert np.array_equal(np.ascontiguousarray(got[:nb, 0]).view(bits), exp_mx.view(bits)), \
                f"summary max differs, unit {(b, hh)}"
            assert np.array_equal(np.ascontiguousarray(got[:nb, 1]).view(bits), exp_mn.view(bits)), \
                f"summary min differs, unit {(b, hh)}"

    def _unit_slice(self, arr, b, hh, width):
        u = b * self.w.kv_heads + hh
        return arr[u * width:(u + 1) * width]

    def check_state(self, t, rec):
        w, h = self.w, self.run.h
        K = h.k_blocks
        S = h.slots
        ids = h.read("IDS")
        sb = h.read("SLOT_BLOCK")
        lu = h.read("LAST_USED")
        fb, fs = h.read("FETCH_BLOCK"), h.read("FETCH_SLOT")
        ab, ast = h.read("ATT_BLOCK"), h.read("ATT_SLOT")
        cnt = h.read("COUNTS")
        bsl = h.read("BLOCK_SLOT")
        st = h.oasis_get_state()   # the same state through oasis_get_state
        for (b, hh) in self.units:
            r = rec[(b, hh)]
            tag = f"step {t} unit {(b, hh)}"
            u = b * w.kv_heads + hh
            nf_o, na_o = len(r["fetch_block"]), len(r["att_block"])
            assert np.array_equal(st["slot_block"][u], r["slot_block"]), tag + " get_state slots"
            assert np.array_equal(st["last_used"][u], r["last_used"]), tag + " get_state lru"
            assert st["fetch_n"][u] == nf_o, tag + " get_state fetch_n"
            assert np.array_equal(st["fetch_list"][u, :nf_o, 0], r["fetch_block"]), tag
            assert np.array_equal(st["fetch_list"][u, :nf_o, 1], r["fetch_slot"]), tag
            assert np.all(st["fetch_list"][u, nf_o:] == -1), tag + " get_state fetch pad"
            assert np.array_equal(st["attended"][u, :na_o], r["att_block"]), tag
            assert np.all(st["attended"][u, na_o:] == -1), tag + " get_state attended pad"
            assert np.array_equal(self._unit_slice(ids, b, hh, K), r["ids"]), tag + " ids"
            c = self._unit_slice(cnt, b, hh, 4)
            na, nh, nf = int(c[0]), int(c[1]), int(c[2])
            assert (na, nh, nf) == (len(r["att_block"]), r["n_hit"], len(r["fetch_block"])), \
                tag + f" counts {(na, nh, nf)}"
            assert np.array_equal(self._unit_slice(fb, b, hh, K)[:nf], r["fetch_block"]), tag
            assert np.array_equal(self._unit_slice(fs, b, hh, K)[:nf], r["fetch_slot"]), tag
            assert np.array_equal(self._unit_slice(ab, b, hh, K)[:na], r["att_block"]), tag
            assert np.array_equal(self._unit_slice(ast, b, hh, K)[:na], r["att_slot"]), tag
            usb = self._unit_slice(sb, b, hh, S)
            assert np.array_equal(usb, r["slot_block"]), tag + " slot_block"
            assert np.array_equal(self._unit_slice(lu, b, hh, S), r["last_used"]), tag + " lru"
            ubs = self._unit_slice(bsl, b, hh, self.NBmax)
            inv = np.full(self.NBmax, -1, np.int32)
            held = usb >= 0
            inv[usb[held]] = np.nonzero(held)[0]
            assert np.array_equal(ubs, inv), tag + " block_slot is not the inverse table"
            self.prev_att[(b, hh)] = r["att_block"]

    def check_payload(self, t):
        w, h = self.w, self.run.h
        dt = np.float32 if w.dtype == synth.F32 else np.uint16
        S, bs, d = h.slots, w.block_size, w.head_dim
        per_slot = 2 * bs * d * np.dtype(dt).itemsize
        sb = h.read("SLOT_BLOCK")
        T = self.run.h.oasis_tokens()
        for (b, hh) in self.units:
            u = b * w.kv_heads + hh
            got = h.read_range("SLOTS", u * S * per_slot, S * per_slot, dt).reshape(S, 2, bs, d)
            usb = sb[u * S:(u + 1) * S]
            for s in range(S):
                if usb[s] < 0:
                    continue
                exp = slot_payload_expected(self.K[b, hh], self.V[b, hh], usb[s], T, bs, w.dtype)
                assert np.array_equal(got[s][:, :exp.shape[1]], exp), \
                    f"step {t} unit {(b, hh)} slot {s} block {usb[s]} payload differs"

    def check_out(self, t, rec):
        out = self.run.out.cpu().numpy()
        worst = 0.0
        for (b, hh) in self.units:
            g0 = hh * self.G
            got = out[b, g0:g0 + self.G].astype(np.float64)
            err = np.max(np.abs(got - rec[(b, hh)]["out"]))
            worst = max(worst, err)
            assert err <= ATTN_TOL, f"step {t} unit {(b, hh)} attention max|err| {err:.3g}"
        return worst

    # ------------------------------------------------------------ stepping
    def _oracle_step(self, t, append, cap, evictions=None):
        drafts = oracle.to_f64(synth.drafts(self.w, t, self.layer), self.w.dtype)

        def one(key):
            b, hh = key
            x, cur = oracle.unit_rows(self.qf, drafts, b, hh, self.G)
            ev = None if evictions is None else evictions[key]
            r = self.oru[key].step(t, x, cur, cap, append=append, evict_blocks=ev)
            r["x"] = x
            return r

        if len(self.units) > 4:
            return dict(zip(self.units, pool().map(one, self.units)))
        return {k: one(k) for k in self.units}

    def _compare_scores(self, t, rec):
        gpu = self.scores_dev.cpu().numpy()
        worst = 0.0
        for (b, hh) in self.units:
            unit = self.oru[(b, hh)]
            nb = unit.nb
            ref = rec[(b, hh)]["scores64"]
            scale = score_scale(unit, rec[(b, hh)]["x"])
            err = np.abs(gpu[b, hh, :nb].astype(np.float64) - ref) / scale
            worst = max(worst, float(err.max()))
            assert err.max() <= SCORE_TOL, f"step {t} unit {(b, hh)} score err {err.max():.3g}"
        return gpu, worst

    def _feed_oracle_scores(self, gpu, rec):
        fed = gpu.copy()
        for (b, hh) in self.units:
            nb = self.oru[(b, hh)].nb
            fed[b, hh, :nb] = rec[(b, hh)]["scores32"]
        self.run.h.oasis_topk_from_scores(torch.from_numpy(fed).cuda())

    device_evict = False   # apply forced evictions with oasis_evict_attended

    def forced_evictions(self, t):
        """Host-side draws of the stress workload applied to the GPU's own
        previous attended lists (read back), same rule as the oracle; by the
        host-built block lists (oasis_evict) or on the device from the draws
        (oasis_evict_attended)."""
        w, h = self.w, self.run.h
        if self.device_evict:
            per_unit = device_evictions(w, h, t, self.layer)
            draws = synth.evict_draws(w, t, self.layer)
            out = {}
            for key in self.units:
                prev = self.prev_att.get(key, np.zeros(0, np.int32))
                mine = synth.forced_evictions(w, prev, len(prev), draws[key[0], key[1]])
                assert np.array_equal(mine, per_unit[key]), f"step {t} unit {key} evictions differ"
                out[key] = mine
            return out
        K = h.k_blocks
        ab, cnt = h.read("ATT_BLOCK"), h.read("COUNTS")
        draws = synth.evict_draws(w, t, self.layer)
        blocks = np.full((w.batch, w.kv_heads, K), -1, np.int32)
        counts = np.zeros((w.batch, w.kv_heads), np.int32)
        per_unit = {}
        for b in range(w.batch):
            for hh in range(w.kv_heads):
                u = b * w.kv_heads + hh
                na = int(cnt[u * 4])
                ev = synth.forced_evictions(w, ab[u * K:u * K + na], na, draws[b, hh])
                blocks[b, hh, :len(ev)] = ev
                counts[b, hh] = len(ev)
                per_unit[(b, hh)] = ev
        h.oasis_evict(blocks.reshape(w.batch * w.kv_heads, K), counts.reshape(-1))
        out = {}
        for key in self.units:   # the oracle's own previous attended list gives the same draw
            prev = self.prev_att.get(key, np.zeros(0, np.int32))
            mine = synth.forced_evictions(w, prev, len(prev), draws[key[0], key[1]])
            assert np.array_equal(mine, per_unit[key]), f"step {t} unit {key} evictions differ"
            out[key] = mine
        return out

    def run_all(self, check_payload_every=1, steps=None):
        """Admission (if any) then every step, comparing after each one."""
        w, run, h = self.w, self.run, self.run.h
        steps = self.n_steps if steps is None else steps
        report = dict(score_err=0.0, attn_err=0.0, steps=0)
        self.check_summary()
        if w.admission:
            h.oasis_predict(run.q, run.drafts[0], w.drafts, scores=self.scores_dev)
            torch.cuda.synchronize()
            rec = self._oracle_step(0, append=False, cap=w.k_blocks)
            gpu, e = self._compare_scores(0, rec)
            self._feed_oracle_scores(gpu, rec)
            h.oasis_select_and_fetch(w.k_blocks)
            h.oasis_sparse_attn(run.q, run.out)
            torch.cuda.synchronize()
            self.check_state(0, rec)
            self.check_payload(0)
            report["attn_err"] = max(report["attn_err"], self.check_out(0, rec))
        for t in range(1, steps + 1):
            ev = None
            if w.forced_evict_frac > 0:
                ev = self.forced_evictions(t)
            h.oasis_append_kv(run.app_k[t - 1], run.app_v[t - 1])
            h.oasis_predict(run.q, run.drafts[t], w.drafts, scores=self.scores_dev)
            torch.cuda.synchronize()
            rec = self._oracle_step(t, append=True, cap=self.cap, evictions=ev)
            gpu, e = self._compare_scores(t, rec)
            report["score_err"] = max(report["score_err"], e)
            self._feed_oracle_scores(gpu, rec)
            h.oasis_select_and_fetch(self.cap)
            h.oasis_sparse_attn(run.q, run.out)
            torch.cuda.synchronize()
            h.oasis_check()
            self.check_state(t, rec)
            if t % check_payload_every == 0 or t == steps:
                self.check_payload(t)
                self.check_summary()
            report["attn_err"] = max(report["attn_err"], self.check_out(t, rec))
            report["steps"] = t
        return report


class FreeRunning(Parity):
    """The GPU runs on its own scores with the fused top-K + select.  Each step
    is checked kernel by kernel: scores against the oracle's, the ids against
    the oracle top-K of the GPU's own fp32 scores, the select outputs against
    the oracle select applied to the GPU's previous tables, and the attention
    against the oracle attention over the GPU's attended list."""

    q_layer = None   # layer whose query the drafts perturb (None: self.layer)
    attend_all = False  # attended set: every block held after the step
    copy_stream = None  # select_and_fetch's copy stream (None: the handle's placement)

    def _tables(self):
        h = self.run.h
        S = h.slots
        sb, lu = h.read("SLOT_BLOCK"), h.read("LAST_USED")
        return {(b, hh): (self._unit_slice(sb, b, hh, S).copy(),
                          self._unit_slice(lu, b, hh, S).copy()) for (b, hh) in self.units}

    def after_admission(self):
        """Admission ran on the GPU: the oracle units only track the KV and
        scores from here (selection is checked against the GPU's tables)."""
        for (b, hh) in self.units:
            self.oru[(b, hh)].slot_block[:] = -1
        return self._tables()

    def verify_step(self, t, prev, report, gpu_scores, cap, check_payload=False):
        """Check step t of the handle against the oracle; returns its tables."""
        w, h = self.w, self.run.h
        K = h.k_blocks
        ids = h.read("IDS")
        fb, fs = h.read("FETCH_BLOCK"), h.read("FETCH_SLOT")
        ab, ast = h.read("ATT_BLOCK"), h.read("ATT_SLOT")
        cnt = h.read("COUNTS")
        out = self.run.out.cpu().numpy()
        drafts = oracle.to_f64(synth.drafts(w, t, self.layer, self.q_layer), w.dtype)
        now = self._tables()
        for (b, hh) in self.units:
            tag = f"free step {t} layer {self.layer} unit {(b, hh)}"
            unit = self.oru[(b, hh)]
            unit.append()
            x, cur = oracle.unit_rows(self.qf, drafts, b, hh, self.G)
            ref = unit.score(x)
            nb = unit.nb
            err = np.abs(gpu_scores[b, hh, :nb].astype(np.float64) - ref) / score_scale(unit, x)
            report["score_err"] = max(report["score_err"], float(err.max()))
            assert err.max() <= SCORE_TOL, tag + f" score err {err.max():.3g}"
            exp_ids = oracle.topk(gpu_scores[b, hh, :nb], K)
            got_ids = self._unit_slice(ids, b, hh, K)
            assert np.array_equal(got_ids, exp_ids), tag + " ids"
            sb0, lu0 = prev[(b, hh)]
            sb_exp, lu_exp = sb0.copy(), lu0.copy()
            r = oracle.select(sb_exp, lu_exp, exp_ids, cap, t, attend_all=self.attend_all)
            c = self._unit_slice(cnt, b, hh, 4)
            na, nh, nf = int(c[0]), int(c[1]), int(c[2])
            assert (na, nh, nf) == (len(r["att_block"]), r["n_hit"], len(r["fetch_block"])), tag
            assert np.array_equal(self._unit_slice(fb, b, hh, K)[:nf], r["fetch_block"]), tag
            assert np.array_equal(self._unit_slice(fs, b, hh, K)[:nf], r["fetch_slot"]), tag
            assert np.array_equal(self._unit_slice(ab, b, hh, K)[:na], r["att_block"]), tag
            assert np.array_equal(self._unit_slice(ast, b, hh, K)[:na], r["att_slot"]), tag
            assert np.array_equal(now[(b, hh)][0], sb_exp), tag + " slot_block"
            assert np.array_equal(now[(b, hh)][1], lu_exp), tag + " last_used"
            exp_out = oracle.attention(cur, unit.keys, unit.vals, w.dtype, w.block_size,
                                       unit.T, r["att_block"])
            g0 = hh * self.G
            e = float(np.max(np.abs(out[b, g0:g0 + self.G].astype(np.float64) - exp_out)))
            report["attn_err"] = max(report["attn_err"], e)
            assert e <= ATTN_TOL, tag + f" attention err {e:.3g}"
            report["fetched"] += nf
        if check_payload:
            self.check_payload(t)
            self.check_summary()
        report["steps"] = t
        return now

    def run_free(self, steps=None, check_payload_every=8, fuse=False, attend_all=False):
        """fuse: score, top-K and select in one kernel (the scores are then
        read back from the handle's SCORES buffer).  attend_all: attend every
        block held after each step."""
        w, run, h = self.w, self.run, self.run.h
        steps = self.n_steps if steps is None else steps
        K = h.k_blocks
        report = dict(score_err=0.0, attn_err=0.0, steps=0, fetched=0)
        if fuse:
            h.oasis_set_score_topk_fusion(True)
        if attend_all:
            h.oasis_set_attend_all_resident(True)
            self.attend_all = True
        if w.admission:
            run.admission()
            torch.cuda.synchronize()
            prev = self.after_admission()
        else:
            prev = self._tables()
        for t in range(1, steps + 1):
            if w.forced_evict_frac > 0 and self.device_evict:
                for key, ev in device_evictions(w, h, t, self.layer).items():
                    if key in prev:
                        sb0 = prev[key][0]
                        sb0[np.isin(sb0, ev)] = -1
            elif w.forced_evict_frac > 0:
                ab, cnt = h.read("ATT_BLOCK"), h.read("COUNTS")
                draws = synth.evict_draws(w, t, self.layer)
                blocks = np.full((w.batch * w.kv_heads, K), -1, np.int32)
                counts = np.zeros(w.batch * w.kv_heads, np.int32)
                for u in range(w.batch * w.kv_heads):
                    na = int(cnt[u * 4])
                    ev = synth.forced_evictions(w, ab[u * K:u * K + na], na,
                                                draws[u // w.kv_heads, u % w.kv_heads])
                    blocks[u, :len(ev)] = ev
                    counts[u] = len(ev)
                    key = (u // w.kv_heads, u % w.kv_heads)
                    if key in prev:
                        sb0 = prev[key][0]
                        for blk in ev:
                            sb0[sb0 == blk] = -1
                h.oasis_evict(blocks, counts)
            h.oasis_append_kv(run.app_k[t - 1], run.app_v[t - 1])
            h.oasis_predict(run.q, run.drafts[t], w.drafts,
                            scores=None if fuse else self.scores_dev)
            h.oasis_select_and_fetch(self.cap, copy=self.copy_stream)
            h.oasis_sparse_attn(run.q, run.out)
            torch.cuda.synchronize()
            h.oasis_check()
            sc = (h.read("SCORES", np.float32).reshape(w.batch, w.kv_heads, self.NBmax) if fuse
                  else self.scores_dev.cpu().numpy())
            prev = self.verify_step(t, prev, report, sc, self.cap,
                                    check_payload=(t % check_payload_every == 0 or t == steps))
        return report


class AheadRunning(FreeRunning):
    """Lookahead ordering ([OASIS] Fig. 8) on one layer, free running: step t
    appends, attends with the step-t query over the set step t-1 selected, and
    selects step t+1's set from the drafts alone.  Checked per step: the draft
    scores against the oracle's, the ids against the oracle top-K of the
    GPU's own fp32 scores, the select against the oracle select on the GPU's
    previous tables, and the attention against the oracle attention over the
    previously selected (and checked) list."""

    def _draft_rows(self, t, b, hh):
        d = oracle.to_f64(synth.drafts(self.w, t, self.layer, self.q_layer), self.w.dtype)
        return oracle.draft_rows(d, b, hh, self.G)

    def verify_ahead(self, t, prev, prev_att, report, cap, check_payload=False):
        w, h = self.w, self.run.h
        K = h.k_blocks
        gpu_scores = h.read("SCORES", np.float32).reshape(w.batch, w.kv_heads, self.NBmax)
        ids = h.read("IDS")
        fb, fs = h.read("FETCH_BLOCK"), h.read("FETCH_SLOT")
        ab, ast = h.read("ATT_BLOCK"), h.read("ATT_SLOT")
        cnt = h.read("COUNTS")
        out = self.run.out.cpu().numpy()
        q = oracle.to_f64(synth.query_at(w, t, self.q_layer if self.q_layer is not None
                                         else self.layer), w.dtype)
        now = self._tables()
        att_now = {}
        for (b, hh) in self.units:
            tag = f"lookahead step {t} layer {self.layer} unit {(b, hh)}"
            unit = self.oru[(b, hh)]
            if t > 0:
                unit.append()
                cur = q[b, hh * self.G:(hh + 1) * self.G]
                exp_out = oracle.attention(cur, unit.keys, unit.vals, w.dtype, w.block_size,
                                           unit.T, prev_att[(b, hh)])
                g0 = hh * self.G
                e = float(np.max(np.abs(out[b, g0:g0 + self.G].astype(np.float64) - exp_out)))
                report["attn_err"] = max(report["attn_err"], e)
                assert e <= ATTN_TOL, tag + f" attention err {e:.3g}"
            x = self._draft_rows(t, b, hh)
            nb = unit.nb
            ref = unit.score(x)
            err = np.abs(gpu_scores[b, hh, :nb].astype(np.float64) - ref) / score_scale(unit, x)
            report["score_err"] = max(report["score_err"], float(err.max()))
            assert err.max() <= SCORE_TOL, tag + f" score err {err.max():.3g}"
            exp_ids = oracle.topk(gpu_scores[b, hh, :nb], K)
            assert np.array_equal(self._unit_slice(ids, b, hh, K), exp_ids), tag + " ids"
            sb0, lu0 = prev[(b, hh)]
            sb_exp, lu_exp = sb0.copy(), lu0.copy()
            r = oracle.select(sb_exp, lu_exp, exp_ids, cap, t, attend_all=self.attend_all)
            c = self._unit_slice(cnt, b, hh, 4)
            na, nh, nf = int(c[0]), int(c[1]), int(c[2])
            assert (na, nh, nf) == (len(r["att_block"]), r["n_hit"], len(r["fetch_block"])), tag
            assert np.array_equal(self._unit_slice(fb, b, hh, K)[:nf], r["fetch_block"]), tag
            assert np.array_equal(self._unit_slice(fs, b, hh, K)[:nf], r["fetch_slot"]), tag
            assert np.array_equal(self._unit_slice(ab, b, hh, K)[:na], r["att_block"]), tag
            assert np.array_equal(self._unit_slice(ast, b, hh, K)[:na], r["att_slot"]), tag
            assert np.array_equal(now[(b, hh)][0], sb_exp), tag + " slot_block"
            assert np.array_equal(now[(b, hh)][1], lu_exp), tag + " last_used"
            att_now[(b, hh)] = r["att_block"].copy()
            report["fetched"] += nf
        if check_payload:
            self.check_payload(t)
            self.check_summary()
        report["steps"] = t
        return now, att_now

    def run_ahead(self, steps=None, check_payload_every=4, beside=None):
        """beside = (stream, copy): the runner's step_beside, the copy of each
        select's blocks on `copy` while the next step scores and attends on
        `stream`."""
        w, run = self.w, self.run
        steps = self.n_steps if steps is None else steps
        report = dict(score_err=0.0, attn_err=0.0, steps=0, fetched=0)
        empty = {k: (np.full(run.h.slots, -1, np.int32), np.full(run.h.slots, -1, np.int32))
                 for k in self.units}
        for k in self.units:
            self.oru[k].slot_block[:] = -1
        if beside is None:
            run.admission_ahead()
        else:
            torch.cuda.synchronize()  # inputs were made on torch's stream
            run.admission_beside(*beside)
        torch.cuda.synchronize()
        prev, att = self.verify_ahead(0, empty, None, report, w.k_blocks)
        for t in range(1, steps + 1):
            if beside is None:
                run.step_ahead(t)
            else:
                run.step_beside(t, *beside)
            torch.cuda.synchronize()
            run.h.oasis_check()
            prev, att = self.verify_ahead(t, prev, att, report, self.cap,
                                          check_payload=(t % check_payload_every == 0 or
                                                         t == steps))
        return report


class PipelineLayer(AheadRunning):
    """Free-running checks of one layer of a ModelRunner (oasis_decode_layers).

    The layer's K, V and query come from its data layer; its drafts from its
    own noise stream around that query."""

    def __init__(self, mr, layer: int, units, unit_kv: dict):
        from types import SimpleNamespace
        w = mr.w
        self.w, self.n_steps, self.units = w, mr.n_steps, list(units)
        self.layer, self.q_layer = layer, mr.group_of(layer)
        h = mr.handles[layer]
        self.run = SimpleNamespace(h=h, out=mr.out[layer])
        self.cap = mr.cap
        self.K = {k: kv[0] for k, kv in unit_kv.items()}
        self.V = {k: kv[1] for k, kv in unit_kv.items()}
        self.oru = {k: initial_unit(w, k[0], k[1], mr.n_steps, self.q_layer, kv=unit_kv[k])
                    for k in self.units}
        self.qf = oracle.to_f64(synth.queries(w, self.q_layer), w.dtype)
        self.G = w.group
        self.NBmax = h.nb_max
        self.prev_att = {}

    def scores(self):
        w = self.w
        return self.run.h.read("SCORES", np.float32).reshape(w.batch, w.kv_heads, self.NBmax)


def pipeline_unit_kv(mr, layer, units):
    """Oracle-side K, V of sampled units of a ModelRunner layer (its data layer's draws)."""
    w, g = mr.w, mr.group_of(layer)
    n_tok = w.prefix_tokens + mr.n_steps
    u = synth.heavy_direction(w, g)
    return {k: synth.unit_kv(w, k[0], k[1], n_tok, g, u[k[0], k[1]]) for k in units}


class CorrectedRunning(AheadRunning):
    """Lookahead prefetch plus decode-time miss correction on one layer, run
    phase by phase: each step's correction (the step query's own top-K,
    cap_correct), its attention, and the drafts' prefetch are each checked
    against the oracle on the GPU's own scores and previous tables."""

    def _phase(self, t, prev, rows_of, cap, report, name):
        w, h = self.w, self.run.h
        K = h.k_blocks
        gpu_scores = h.read("SCORES", np.float32).reshape(w.batch, w.kv_heads, self.NBmax)
        ids = h.read("IDS")
        fb, fs = h.read("FETCH_BLOCK"), h.read("FETCH_SLOT")
        ab, ast = h.read("ATT_BLOCK"), h.read("ATT_SLOT")
        cnt = h.read("COUNTS")
        now = self._tables()
        att, misses = {}, 0
        for (b, hh) in self.units:
            tag = f"{name} step {t} unit {(b, hh)}"
            unit = self.oru[(b, hh)]
            x = rows_of(b, hh)
            nb = unit.nb
            ref = unit.score(x)
            err = np.abs(gpu_scores[b, hh, :nb].astype(np.float64) - ref) / score_scale(unit, x)
            report["score_err"] = max(report["score_err"], float(err.max()))
            assert err.max() <= SCORE_TOL, tag + f" score err {err.max():.3g}"
            exp_ids = oracle.topk(gpu_scores[b, hh, :nb], K)
            assert np.array_equal(self._unit_slice(ids, b, hh, K), exp_ids), tag + " ids"
            sb_exp, lu_exp = prev[(b, hh)][0].copy(), prev[(b, hh)][1].copy()
            r = oracle.select(sb_exp, lu_exp, exp_ids, cap, t, attend_all=self.attend_all)
            c = self._unit_slice(cnt, b, hh, 4)
            na, nh, nf, nm = int(c[0]), int(c[1]), int(c[2]), int(c[3])
            n_sel = int((exp_ids >= 0).sum())
            assert (na, nh, nf, nm) == (len(r["att_block"]), r["n_hit"], len(r["fetch_block"]),
                                        n_sel - r["n_hit"]), tag
            assert np.array_equal(self._unit_slice(fb, b, hh, K)[:nf], r["fetch_block"]), tag
            assert np.array_equal(self._unit_slice(fs, b, hh, K)[:nf], r["fetch_slot"]), tag
            assert np.array_equal(self._unit_slice(ab, b, hh, K)[:na], r["att_block"]), tag
            assert np.array_equal(self._unit_slice(ast, b, hh, K)[:na], r["att_slot"]), tag
            assert np.array_equal(now[(b, hh)][0], sb_exp), tag + " slot_block"
            assert np.array_equal(now[(b, hh)][1], lu_exp), tag + " last_used"
            att[(b, hh)] = r["att_block"].copy()
            misses += nm
        report[name + "_misses"] = report.get(name + "_misses", 0) + misses
        return now, att

    def run_corrected(self, cap_correct, steps=None, check_payload_every=4):
        w, run, h = self.w, self.run, self.run.h
        steps = self.n_steps if steps is None else steps
        report = dict(score_err=0.0, attn_err=0.0, steps=0, fetched=0)
        empty = {k: (np.full(h.slots, -1, np.int32), np.full(h.slots, -1, np.int32))
                 for k in self.units}
        for k in self.units:
            self.oru[k].slot_block[:] = -1
        run.admission_ahead()
        torch.cuda.synchronize()
        prev, _ = self.verify_ahead(0, empty, None, report, w.k_blocks)
        for t in range(1, steps + 1):
            q = oracle.to_f64(synth.query_at(w, t, self.layer), w.dtype)
            cur = {k: q[k[0], k[1] * self.G:(k[1] + 1) * self.G] for k in self.units}
            h.oasis_append_kv(run.app_k[t - 1], run.app_v[t - 1])
            for k in self.units:
                self.oru[k].append()
            h.oasis_predict(run.q_steps[t], None, 0)
            h.oasis_select_and_fetch(cap_correct)
            torch.cuda.synchronize()
            prev, att = self._phase(t, prev, lambda b, hh: cur[(b, hh)], cap_correct, report,
                                    "correction")
            h.oasis_sparse_attn(run.q_steps[t], run.out)
            torch.cuda.synchronize()
            out = run.out.cpu().numpy()
            for (b, hh) in self.units:
                unit = self.oru[(b, hh)]
                exp = oracle.attention(cur[(b, hh)], unit.keys, unit.vals, w.dtype, w.block_size,
                                       unit.T, att[(b, hh)])
                g0 = hh * self.G
                e = float(np.max(np.abs(out[b, g0:g0 + self.G].astype(np.float64) - exp)))
                report["attn_err"] = max(report["attn_err"], e)
                assert e <= ATTN_TOL, f"corrected step {t} unit {(b, hh)} attention err {e:.3g}"
            h.oasis_predict(None, run.drafts[t], w.drafts)
            h.oasis_select_and_fetch(self.cap)
            torch.cuda.synchronize()
            h.oasis_check()
            prev, _ = self._phase(t, prev, lambda b, hh: self._draft_rows(t, b, hh), self.cap,
                                  report, "prefetch")
            if t % check_payload_every == 0 or t == steps:
                self.check_payload(t)
            report["steps"] = t
        return report
