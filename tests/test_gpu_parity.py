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


@pytest.mark.parametrize("q_heads,kv_heads", [(8, 8), (16, 8), (32, 4), (64, 4)])
def test_group_sizes_reduced_context(q_heads, kv_heads):
    """G = 1, 2, 8, 16 on a reduced context with a ragged prefix."""
    Parity, log = _parity()
    w = synth.QWEN3_8B.with_(batch=2, q_heads=q_heads, kv_heads=kv_heads,
                             prefix_tokens=16 * 300 + 7, budget_tokens=16 * 64)
    units = [(0, 0), (1, kv_heads - 1)]
    p = Parity(w, 6, units)
    log(f"G={q_heads // kv_heads}: {p.run_all()}")
