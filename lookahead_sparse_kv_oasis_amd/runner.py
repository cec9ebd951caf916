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
                 kv=None, cap: int | None = None):
        self.w, self.layer, self.n_steps = w, layer, n_steps
        self.T0 = w.prefix_tokens
        n_tok = w.prefix_tokens + n_steps
        K, V = kv if kv is not None else synth.layer_kv(w, n_tok, layer)
        self.cap = cap if cap is not None else (
            w.cap if w.cap > 0 else _cap_from_ratio(w.fetch_ratio, w.k_blocks))
        self.h = Oasis(w.batch, w.q_heads, w.kv_heads, w.head_dim,
                       OASIS_F32 if w.dtype == synth.F32 else OASIS_BF16, w.drafts, n_tok,
                       block_size=w.block_size, budget_tokens=w.budget_tokens,
                       fetch_ratio=w.fetch_ratio, slots_per_head=w.n_slots)
        self.h.oasis_load_prefix(np.ascontiguousarray(K[:, :, :self.T0]),
                                 np.ascontiguousarray(V[:, :, :self.T0]), self.T0)
        # appended tokens, one [B][Hkv][d] slab per step
        self.app_k = to_device(np.ascontiguousarray(K[:, :, self.T0:].transpose(2, 0, 1, 3)), device)
        self.app_v = to_device(np.ascontiguousarray(V[:, :, self.T0:].transpose(2, 0, 1, 3)), device)
        del K, V
        self.q = to_device(synth.queries(w, layer), device)
        self.drafts = [to_device(synth.drafts(w, t, layer), device) for t in range(n_steps + 1)]
        self.out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32,
                               device=device)
        if w.initial_resident_frac > 0:
            sb, lu = synth.initial_slots(w, layer)
            self.h.oasis_set_state(sb, lu)
        self.t = 0

    def admission(self, stream=None):
        """Untimed step 0: select on the prompt and fetch the whole selection."""
        h = self.h
        h.oasis_predict(self.q, self.drafts[0], self.w.drafts, stream=stream)
        h.oasis_select_and_fetch(self.w.k_blocks, stream=stream)
        h.oasis_sparse_attn(self.q, self.out, stream=stream)

    def step(self, t: int, stream=None, scores_hook=None):
        """Decode step t (1-based): append token T0 + t - 1, predict, select, attend.

        scores_hook(t) may return device scores [B][Hkv][NBmax] to select on
        instead of the library's own (parity runs)."""
        h = self.h
        h.oasis_append_kv(self.app_k[t - 1], self.app_v[t - 1], stream=stream)
        h.oasis_predict(self.q, self.drafts[t], self.w.drafts, stream=stream)
        if scores_hook is not None:
            s = scores_hook(t)
            if s is not None:
                h.oasis_topk_from_scores(s, stream=stream)
        h.oasis_select_and_fetch(self.cap, stream=stream)
        h.oasis_sparse_attn(self.q, self.out, stream=stream)
        self.t = t


def _cap_from_ratio(ratio, k):
    from . import cap_from_ratio
    return cap_from_ratio(ratio, k)
