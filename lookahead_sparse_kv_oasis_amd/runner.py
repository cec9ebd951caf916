"""Drive one layer's decode steps through the C-ABI on a synthetic workload.

A thin loop around the library calls (no arithmetic of the method here):
load the prompt, optionally seed the residency tables, then per step
append -> predict -> select_and_fetch -> sparse_attn.  Inputs come from the
seeded generator module ``synth``; device memory and streams come from
PyTorch.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from . import Oasis, OASIS_BF16, OASIS_F32


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Storage array (float32 or bf16 bits as uint16) -> device tensor with the same bytes."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class LayerRunner:
    def __init__(self, w: synth.Workload, n_steps: int, layer: int = 0, device: str = "cuda",
                 kv=None, cap: int | None = None, compute_units: int = 0):
        self.w, self.layer, self.n_steps = w, layer, n_steps
        self.T0 = w.prefix_tokens
        n_tok = w.prefix_tokens + n_steps
        K, V = kv if kv is not None else synth.layer_kv(w, n_tok, layer)
        self.cap = cap if cap is not None else (
            w.cap if w.cap > 0 else _cap_from_ratio(w.fetch_ratio, w.k_blocks))
        self.h = Oasis(w.batch, w.q_heads, w.kv_heads, w.head_dim,
                       OASIS_F32 if w.dtype == synth.F32 else OASIS_BF16, w.drafts, n_tok,
                       block_size=w.block_size, budget_tokens=w.budget_tokens,
                       fetch_ratio=w.fetch_ratio, slots_per_head=w.n_slots,
                       compute_units=compute_units)
        self.h.oasis_load_prefix(np.ascontiguousarray(K[:, :, :self.T0]),
                                 np.ascontiguousarray(V[:, :, :self.T0]), self.T0)
        # appended tokens, one [B][Hkv][d] slab per step
        self.app_k = to_device(np.ascontiguousarray(K[:, :, self.T0:].transpose(2, 0, 1, 3)), device)
        self.app_v = to_device(np.ascontiguousarray(V[:, :, self.T0:].transpose(2, 0, 1, 3)), device)
        del K, V
        self.q = to_device(synth.queries(w, layer), device)
        # current query per step (the same tensor unless the workload drifts)
        self.q_steps = ([to_device(synth.query_at(w, t, layer), device)
                         for t in range(n_steps + 1)] if w.query_drift else
                        [self.q] * (n_steps + 1))
        self.drafts = [to_device(synth.drafts(w, t, layer), device) for t in range(n_steps + 1)]
        self.out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32,
                               device=device)
        if w.initial_resident_frac > 0:
            sb, lu = synth.initial_slots(w, layer)
            self.h.oasis_set_state(sb, lu)
        # the GQA-8 stress workload forces part of the previous attended set out
        # of HBM at each step start: its seeded draws, every step, on the device
        self.evict_draws = None
        if w.forced_evict_frac > 0:
            self.evict_draws = torch.from_numpy(np.ascontiguousarray(np.stack(
                [synth.evict_draws(w, t, layer) for t in range(n_steps + 1)]))).to(device)
        self.t = 0

    def admission(self, stream=None):
        """Untimed step 0: select on the prompt and fetch the whole selection."""
        h = self.h
        h.oasis_predict(self.q, self.drafts[0], self.w.drafts, stream=stream)
        h.oasis_select_and_fetch(self.w.k_blocks, stream=stream)
        h.oasis_sparse_attn(self.q, self.out, stream=stream)

    def step(self, t: int, stream=None, scores_hook=None):
        """Decode step t (1-based): forced evictions (stress workload), append
        token T0 + t - 1, predict, select, attend.

        scores_hook(t) may return device scores [B][Hkv][NBmax] to select on
        instead of the library's own (parity runs)."""
        h = self.h
        if self.evict_draws is not None:
            h.oasis_evict_attended(self.evict_draws[t], self.w.forced_evict_frac, stream=stream)
        h.oasis_append_kv(self.app_k[t - 1], self.app_v[t - 1], stream=stream)
        q = self.q_steps[t]
        h.oasis_predict(q, self.drafts[t], self.w.drafts, stream=stream)
        if scores_hook is not None:
            s = scores_hook(t)
            if s is not None:
                h.oasis_topk_from_scores(s, stream=stream)
        h.oasis_select_and_fetch(self.cap, stream=stream)
        h.oasis_sparse_attn(q, self.out, stream=stream)
        self.t = t

    # ---- lookahead ordering ([OASIS] Fig. 8)
    def admission_ahead(self, stream=None):
        """Untimed step 0: the step-0 drafts select (cap = K) the set that step
        1 attends over."""
        h = self.h
        h.oasis_predict(None, self.drafts[0], self.w.drafts, stream=stream)
        h.oasis_select_and_fetch(self.w.k_blocks, stream=stream)

    def step_ahead(self, t: int, stream=None, cap: int | None = None):
        """Step t: append token T0 + t - 1, attend with the step-t query over
        the set step t-1 selected, then select step t+1's set from the drafts."""
        h = self.h
        h.oasis_append_kv(self.app_k[t - 1], self.app_v[t - 1], stream=stream)
        h.oasis_sparse_attn(self.q_steps[t], self.out, stream=stream)
        h.oasis_predict(None, self.drafts[t], self.w.drafts, stream=stream)
        h.oasis_select_and_fetch(self.cap if cap is None else cap, stream=stream)
        self.t = t

    def admission_beside(self, stream, copy):
        """admission_ahead with the copy on its own stream."""
        h = self.h
        h.oasis_set_attention_beside_copy(True)
        h.oasis_predict(None, self.drafts[0], self.w.drafts, stream=stream)
        h.oasis_select_and_fetch(self.w.k_blocks, stream=stream, copy=copy)

    def step_beside(self, t: int, stream, copy, cap: int | None = None):
        """Lookahead step with the transfer on a copy stream of its own
        ([OASIS] Fig. 8): append token T0 + t - 1, score the step-t drafts,
        attend with the step-t query (the blocks held before the last select
        while the copy of its fetched blocks runs, those once it has landed),
        then select step t+1's set, whose copy starts on `copy`.  The scoring
        and the attention over held blocks hide the transfer."""
        h = self.h
        h.oasis_append_kv(self.app_k[t - 1], self.app_v[t - 1], stream=stream)
        h.oasis_predict(None, self.drafts[t], self.w.drafts, stream=stream)
        h.oasis_sparse_attn(self.q_steps[t], self.out, stream=stream)
        h.oasis_select_and_fetch(self.cap if cap is None else cap, stream=stream, copy=copy)
        self.t = t

    def step_corrected(self, t: int, cap_correct: int, stream=None, cap: int | None = None):
        """Lookahead step with decode-time miss correction: append; the step-t
        query's own top-K selected with cap_correct (missed blocks fetched
        now); attention over it; then the drafts prefetch step t+1's set."""
        h = self.h
        h.oasis_append_kv(self.app_k[t - 1], self.app_v[t - 1], stream=stream)
        h.oasis_predict(self.q_steps[t], None, 0, stream=stream)
        h.oasis_select_and_fetch(cap_correct, stream=stream)
        h.oasis_sparse_attn(self.q_steps[t], self.out, stream=stream)
        h.oasis_predict(None, self.drafts[t], self.w.drafts, stream=stream)
        h.oasis_select_and_fetch(self.cap if cap is None else cap, stream=stream)
        self.t = t


def _cap_from_ratio(ratio, k):
    from . import cap_from_ratio
    return cap_from_ratio(ratio, k)


class ModelRunner:
    """All layers of a multi-layer workload, stepped by oasis_decode_layers.

    Layer l's K, V and current query are those of data layer
    ``synth.data_layer(w, l, data_layers)``: layers of one data layer share a
    pinned host KV (oasis_create_shared) so that the model fits host memory,
    and receive the same appended tokens.  Each layer has its own HBM state
    (summaries, slot pool, tables) and its own draft noise, so selections
    differ between layers.
    """

    def __init__(self, w: synth.Workload, n_steps: int, data_layers: int = 2,
                 device: str = "cuda", cap: int | None = None, threads: int = 16, log=None,
                 compute_units: int = 0):
        from . import LayerStep
        self.w, self.n_steps = w, n_steps
        self.n_layers = w.layers
        self.H = max(1, min(data_layers, w.layers))
        self.T0 = w.prefix_tokens
        n_tok = self.T0 + n_steps
        self.cap = cap if cap is not None else (
            w.cap if w.cap > 0 else _cap_from_ratio(w.fetch_ratio, w.k_blocks))
        dt = OASIS_F32 if w.dtype == synth.F32 else OASIS_BF16
        mk = lambda owner=None: Oasis(w.batch, w.q_heads, w.kv_heads, w.head_dim, dt, w.drafts,
                                      n_tok, block_size=w.block_size,
                                      budget_tokens=w.budget_tokens, fetch_ratio=w.fetch_ratio,
                                      slots_per_head=w.n_slots, share_host_with=owner,
                                      compute_units=compute_units)
        self.handles = [None] * self.n_layers
        self.app_k, self.app_v, self.q, self.q_steps = [], [], [], []
        for g in range(self.H):
            if log:
                log(f"generating data layer {g} of {self.H}")
            Kp, Vp, Ka, Va = synth.layer_kv_split(w, self.T0, n_steps, g, threads)
            owner = mk()
            owner.oasis_load_prefix(Kp, Vp, self.T0)
            del Kp, Vp
            self.app_k.append(to_device(Ka, device))
            self.app_v.append(to_device(Va, device))
            del Ka, Va
            self.q.append(to_device(synth.queries(w, g), device))
            self.q_steps.append([to_device(synth.query_at(w, t, g), device)
                                 for t in range(n_steps + 1)] if w.query_drift else
                                [self.q[-1]] * (n_steps + 1))
            for l in range(g, self.n_layers, self.H):
                if l == g:
                    self.handles[l] = owner
                else:
                    h = mk(owner)
                    h.oasis_load_prefix(None, None, self.T0)
                    self.handles[l] = h
        # draft queries of every (step, layer): [steps + 1][layers] device tensors
        from concurrent.futures import ThreadPoolExecutor
        keys = [(t, l) for t in range(n_steps + 1) for l in range(self.n_layers)]
        with ThreadPoolExecutor(threads) as ex:
            host = list(ex.map(lambda k: synth.drafts(w, k[0], k[1], self.group_of(k[1])), keys))
        flat = [to_device(a, device) for a in host]
        del host
        self.drafts = [flat[t * self.n_layers:(t + 1) * self.n_layers]
                       for t in range(n_steps + 1)]
        self.out = torch.empty((self.n_layers, w.batch, w.q_heads, w.head_dim),
                               dtype=torch.float32, device=device)
        self.step_args = LayerStep(self.handles)
        self.t = 0

    def group_of(self, l: int) -> int:
        return synth.data_layer(self.w, l, self.H)

    def reset(self):
        """Every layer starts over from the prompt (synchronous)."""
        for h in self.handles:
            h.oasis_load_prefix(None, None, self.T0)
        self.t = 0

    def _fill(self, t: int):
        a = self.step_args
        for l in range(self.n_layers):
            g = self.group_of(l)
            k = self.app_k[g][t - 1] if t > 0 else None
            v = self.app_v[g][t - 1] if t > 0 else None
            a.set(l, k, v, self.q_steps[g][t], self.drafts[t][l], self.out[l])

    def admission(self, stream=None, side=None):
        """Untimed step 0 on every layer: select on the prompt, fetch it all."""
        self._fill(0)
        self.step_args.run(self.w.drafts, self.w.k_blocks, stream=stream, side=side)

    def step(self, t: int, stream=None, side=None, cap: int | None = None):
        """Decode step t (1-based) over all layers; side=None serialises."""
        self._fill(t)
        self.step_args.run(self.w.drafts, self.cap if cap is None else cap, stream=stream,
                           side=side)
        self.t = t

    # ---- lookahead ordering ([OASIS] Fig. 8): oasis_decode_layers_ahead
    def admission_ahead(self, stream, side, xfer):
        """Untimed step 0: every layer's step-0 drafts select (cap = K) and
        fetch the set its step-1 attention uses."""
        a = self.step_args
        for l in range(self.n_layers):
            a.set(l, None, None, None, self.drafts[0][l], None)
        a.run_ahead(self.w.drafts, self.w.k_blocks, stream, side, xfer)

    def step_ahead(self, t: int, stream, side, xfer, cap: int | None = None,
                   cap_correct: int = 0):
        a = self.step_args
        for l in range(self.n_layers):
            g = self.group_of(l)
            a.set(l, self.app_k[g][t - 1], self.app_v[g][t - 1], self.q_steps[g][t],
                  self.drafts[t][l], self.out[l])
        a.run_ahead(self.w.drafts, self.cap if cap is None else cap, stream, side, xfer,
                    cap_correct)
        self.t = t

    def close(self):
        for h in self.handles[::-1]:
            if h is not None:
                h.close()


# ---- prediction quality of the lookahead ordering ([OASIS] Fig. 4, Fig. 6)

def predicted_ids(h) -> np.ndarray:
    """The handle's current selection (ids) as [units][K]."""
    return h.read("IDS").reshape(-1, h.k_blocks)


def exact_ids(h, q, buf: torch.Tensor, stream=None) -> np.ndarray:
    """Top-K ids of the current query alone ([units][K]).  Leaves the handle's
    scores and ids changed: call it where the next predict recomputes them."""
    h.oasis_predict(q, None, 0, block_ids=buf, stream=stream)
    torch.cuda.synchronize()
    return buf.cpu().numpy().reshape(-1, h.k_blocks)


def recall(pred: np.ndarray, exact: np.ndarray) -> float:
    """Mean over units of |pred ∩ exact| / |exact| (ids -1 are padding)."""
    hit = (pred[:, :, None] == exact[:, None, :]) & (exact[:, None, :] >= 0)
    n = np.maximum((exact >= 0).sum(axis=1), 1)
    return float((hit.any(axis=1).sum(axis=1) / n).mean())
