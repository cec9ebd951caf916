"""Seeded synthetic inputs for the OasisKV decode-step workloads.

This module is shared by the fp64 oracle harness and the HIP path.  It holds
only the workload recipe (shapes, value distributions, seeds) and contains
none of the method's arithmetic: no scoring, selection, eviction or
attention.  Every random number the method consumes (draft noise, the
residency seed of the tiny case, the forced-eviction draws of the GQA-8
stress case) is drawn here and handed to both sides as an input.

Values are drawn in fp32 with numpy's PCG64, one independent stream per
(config seed, layer, batch row, kv head, tensor kind), so any single
(batch, kv-head) unit can be regenerated on its own and the full batch is
the stack of its units.  bf16 tensors are stored as raw uint16 bit patterns
produced by round-to-nearest-even from the fp32 draw.

The stand-ins follow the layer shapes the OasisKV page evaluates (Qwen3-8B,
Qwen3-32B, Llama-3.1-8B; a 2,048-token KV budget; 32K-128K context; fetch
ratios 0.01-0.20 from the fetch-cap ablation table), with synthetic values
in place of model activations, which are not available.
"""
from __future__ import annotations

import dataclasses
import functools
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = 0
BF16 = 1

# stream kinds
_K, _V, _Q, _DRAFT, _HEAVY, _RESID, _EVICT, _QDRIFT = 1, 2, 3, 4, 5, 6, 7, 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: int                # F32 or BF16
    prefix_tokens: int        # tokens loaded before step 1
    steps: int                # decode steps, one appended token each
    block_size: int = 16
    budget_tokens: int = 2048
    slots: int = 0            # HBM slots per (b, kv head); 0 -> budget blocks
    drafts: int = 4
    draft_sigma: float = 0.3
    heavy_mode: str = "bernoulli"   # "bernoulli" (fraction) or "count"
    heavy_frac: float = 0.05
    heavy_count: int = 0
    heavy_amp: float = 2.0
    drift_amp: float = 0.0
    drift_period: float = 4096.0
    fetch_ratio: float = 0.02
    cap: int = 0              # explicit per-(b, kv head) cap; 0 -> from fetch_ratio
    forced_evict_frac: float = 0.0
    admission: bool = True    # uncapped step 0 fills the pool with the step-0 selection
    initial_resident_frac: float = 0.0
    layers: int = 1
    # Lookahead workloads: the current query drifts between steps (AR(1) around
    # the step-0 query: e_t = rho e_{t-1} + sqrt(1 - rho^2) query_drift xi_t)
    # and the drafts of step t are centred on the next step's query.
    query_drift: float = 0.0
    drift_rho: float = 0.9
    lookahead: bool = False
    seed: int = 0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def k_blocks(self) -> int:
        return self.budget_tokens // self.block_size

    @property
    def n_slots(self) -> int:
        return self.slots if self.slots > 0 else self.k_blocks

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def blocks_at(self, tokens: int) -> int:
        return (tokens + self.block_size - 1) // self.block_size

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Sizes, distributions and knobs as listed for the
# decode-step benchmark; readings where the recipe is silent are noted.
TINY = Workload(
    name="tiny_b1_h4x2_d64_t1k_f32", batch=1, q_heads=4, kv_heads=2, head_dim=64,
    dtype=F32, prefix_tokens=1024, steps=16, budget_tokens=8 * 16, slots=32,
    drafts=2, draft_sigma=0.3, heavy_mode="count", heavy_count=4, heavy_amp=3.0,
    cap=2, admission=False, initial_resident_frac=0.5)
QWEN3_8B = Workload(
    name="qwen3_8b_layer_b32_t32k_bf16", batch=32, q_heads=32, kv_heads=8, head_dim=128,
    dtype=BF16, prefix_tokens=32768, steps=64, heavy_frac=0.05, heavy_amp=2.0,
    fetch_ratio=0.02)
LLAMA31_8B_LONG = Workload(
    name="llama31_8b_layer_b8_t128k_bf16", batch=8, q_heads=32, kv_heads=8, head_dim=128,
    dtype=BF16, prefix_tokens=131072, steps=64, heavy_frac=0.02, heavy_amp=2.0,
    drift_amp=0.5, drift_period=4096.0, fetch_ratio=0.02)
QWEN3_32B = Workload(
    name="qwen3_32b_layer_b16_t32k_bf16", batch=16, q_heads=64, kv_heads=8, head_dim=128,
    dtype=BF16, prefix_tokens=32768, steps=128, draft_sigma=0.5, heavy_frac=0.05,
    heavy_amp=2.0, fetch_ratio=0.05, forced_evict_frac=0.10)
QWEN3_8B_36L = Workload(
    name="qwen3_8b_36layer_b64_t64k_bf16", batch=64, q_heads=32, kv_heads=8, head_dim=128,
    dtype=BF16, prefix_tokens=65536, steps=32, heavy_frac=0.05, heavy_amp=2.0,
    fetch_ratio=0.02, layers=36)

# Lookahead ordering ([OASIS] Fig. 8): the drafts of step t predict the set for
# step t+1's attention.  Queries drift (AR(1), stationary std 0.5 per element,
# rho 0.9, so about 0.22 change per step) and the drafts sit 0.1 around the next
# query, so the previous query and the drafts are both imperfect predictors.
QWEN3_8B_AHEAD = QWEN3_8B.with_(name="qwen3_8b_layer_b32_t32k_bf16_lookahead",
                                query_drift=0.5, drift_rho=0.9, draft_sigma=0.1,
                                lookahead=True)
QWEN3_8B_36L_AHEAD = QWEN3_8B_36L.with_(name="qwen3_8b_36layer_b64_t64k_bf16_lookahead",
                                        query_drift=0.5, drift_rho=0.9, draft_sigma=0.1,
                                        lookahead=True)

WORKLOADS = [TINY, QWEN3_8B, LLAMA31_8B_LONG, QWEN3_32B, QWEN3_8B_36L, QWEN3_8B_AHEAD,
             QWEN3_8B_36L_AHEAD]
FETCH_RATIO_SWEEP = [0.01, 0.02, 0.05, 0.10, 0.20, None]   # None = fetch all


# ---------------------------------------------------------------- encoding

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 draw -> storage array (float32, or uint16 bf16 bits)."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    return round_to_bf16_bits(x)


def decode_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    """storage array -> float32 values (exact)."""
    if dtype == F32:
        return a.astype(np.float32, copy=False)
    return bf16_bits_to_f32(a)


def _rng(w: Workload, layer: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, layer, *key])))


# ---------------------------------------------------------------- queries

def queries(w: Workload, layer: int = 0) -> np.ndarray:
    """Current query q[b][g][d] ~ N(0,1), held fixed over the run; storage dtype."""
    g = _rng(w, layer, _Q)
    x = g.standard_normal((w.batch, w.q_heads, w.head_dim), dtype=np.float32)
    return encode(x, w.dtype)


@functools.lru_cache(maxsize=8)
def _queries_f32(w: Workload, layer: int) -> np.ndarray:
    return decode_f32(queries(w, layer), w.dtype)


@functools.lru_cache(maxsize=8)
def _drift(w: Workload, layer: int, upto: int) -> tuple:
    """Deviations e_0 .. e_upto of the drifting query (e_0 = 0), fp32."""
    shape = (w.batch, w.q_heads, w.head_dim)
    e = [np.zeros(shape, np.float32)]
    c = np.float32(np.sqrt(1.0 - w.drift_rho ** 2) * w.query_drift)
    for t in range(1, upto + 1):
        xi = _rng(w, layer, _QDRIFT, t).standard_normal(shape, dtype=np.float32)
        e.append(np.float32(w.drift_rho) * e[-1] + c * xi)
    return tuple(e)


def query_at(w: Workload, step: int, layer: int = 0) -> np.ndarray:
    """Current query of decode step `step` in storage dtype: the step-0 query,
    plus the AR(1) deviation of a lookahead workload."""
    if w.query_drift == 0.0 or step == 0:
        return queries(w, layer)
    e = _drift(w, layer, max(step, w.steps + 1))[step]
    return encode(_queries_f32(w, layer) + e, w.dtype)


def drafts(w: Workload, step: int, layer: int = 0, q_layer: int | None = None) -> np.ndarray:
    """Draft queries [D][b][g][d] = q + N(0, sigma^2), redrawn every step.

    q is layer q_layer's query (default: the same layer) at this step, or at
    the next step for a lookahead workload (the draft tokens approximate the
    query that comes next); the noise stream is layer's own."""
    ql = layer if q_layer is None else q_layer
    if w.lookahead or w.query_drift != 0.0:
        q = decode_f32(query_at(w, step + 1 if w.lookahead else step, ql), w.dtype)
    else:
        q = _queries_f32(w, ql)
    g = _rng(w, layer, _DRAFT, step)
    noise = g.standard_normal((w.drafts, w.batch, w.q_heads, w.head_dim), dtype=np.float32)
    return encode(q[None] + np.float32(w.draft_sigma) * noise, w.dtype)


def heavy_direction(w: Workload, layer: int = 0) -> np.ndarray:
    """u[b][h] = unit vector of the sum of the group's current queries (fp32)."""
    q = decode_f32(queries(w, layer), w.dtype).astype(np.float64)
    s = q.reshape(w.batch, w.kv_heads, w.group, w.head_dim).sum(axis=2)
    n = np.linalg.norm(s, axis=-1, keepdims=True)
    return (s / np.where(n > 0, n, 1.0)).astype(np.float32)


# ---------------------------------------------------------------- KV

def heavy_blocks(w: Workload, b: int, h: int, n_blocks: int, layer: int = 0) -> np.ndarray:
    """Boolean flag per block index of one (b, kv head) unit."""
    g = _rng(w, layer, _HEAVY, b, h)
    if w.heavy_mode == "count":
        flags = np.zeros(n_blocks, dtype=bool)
        base = min(n_blocks, w.blocks_at(w.prefix_tokens))
        flags[g.choice(base, size=min(w.heavy_count, base), replace=False)] = True
        return flags
    return g.random(n_blocks) < w.heavy_frac


def unit_kv(w: Workload, b: int, h: int, n_tokens: int, layer: int = 0,
            u: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Keys and values [n_tokens][d] of one unit in storage dtype.

    Tokens are the prefix followed by the appended decode tokens, so a longer
    draw extends a shorter one.  Keys of heavy blocks get heavy_amp * u; the
    long-context workload adds a sinusoidal drift along u to every key.
    """
    d = w.head_dim
    if u is None:
        u = heavy_direction(w, layer)[b, h]
    k = _rng(w, layer, _K, b, h).standard_normal((n_tokens, d), dtype=np.float32)
    v = _rng(w, layer, _V, b, h).standard_normal((n_tokens, d), dtype=np.float32)
    nb = w.blocks_at(n_tokens)
    flags = heavy_blocks(w, b, h, nb, layer)
    tok_heavy = np.repeat(flags, w.block_size)[:n_tokens]
    k[tok_heavy] += np.float32(w.heavy_amp) * u[None, :]
    if w.drift_amp != 0.0:
        p = np.arange(n_tokens, dtype=np.float64)
        amp = (w.drift_amp * np.sin(2.0 * np.pi * p / w.drift_period)).astype(np.float32)
        k += amp[:, None] * u[None, :]
    return encode(k, w.dtype), encode(v, w.dtype)


def layer_kv(w: Workload, n_tokens: int, layer: int = 0, threads: int = 8):
    """Full-batch K and V [B][Hkv][n_tokens][d] in storage dtype."""
    dt = np.float32 if w.dtype == F32 else np.uint16
    K = np.empty((w.batch, w.kv_heads, n_tokens, w.head_dim), dtype=dt)
    V = np.empty_like(K)
    u = heavy_direction(w, layer)

    def one(idx):
        b, h = divmod(idx, w.kv_heads)
        K[b, h], V[b, h] = unit_kv(w, b, h, n_tokens, layer, u[b, h])

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(w.batch * w.kv_heads)))
    return K, V


def layer_kv_split(w: Workload, n_prefix: int, n_append: int, layer: int = 0,
                   threads: int = 8):
    """The same draws as layer_kv(w, n_prefix + n_append, layer), split into
    the prompt K, V [B][Hkv][n_prefix][d] and the appended tokens
    [n_append][B][Hkv][d] (one slab per decode step)."""
    dt = np.float32 if w.dtype == F32 else np.uint16
    d = w.head_dim
    Kp = np.empty((w.batch, w.kv_heads, n_prefix, d), dtype=dt)
    Vp = np.empty_like(Kp)
    Ka = np.empty((n_append, w.batch, w.kv_heads, d), dtype=dt)
    Va = np.empty_like(Ka)
    u = heavy_direction(w, layer)

    def one(idx):
        b, h = divmod(idx, w.kv_heads)
        k, v = unit_kv(w, b, h, n_prefix + n_append, layer, u[b, h])
        Kp[b, h], Vp[b, h] = k[:n_prefix], v[:n_prefix]
        Ka[:, b, h], Va[:, b, h] = k[n_prefix:], v[n_prefix:]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(w.batch * w.kv_heads)))
    return Kp, Vp, Ka, Va


def data_layer(w: Workload, layer: int, data_layers: int) -> int:
    """Multi-layer workloads whose full host KV does not fit host memory
    alias layer l's K, V and current query onto data layer l mod data_layers;
    each layer keeps its own draft noise."""
    return layer % max(1, min(data_layers, w.layers))


# ---------------------------------------------------------------- residency / eviction draws

def initial_slots(w: Workload, layer: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Seeded initial pool: slot_block[B][Hkv][S] (-1 empty) and last_used (-1).

    Used by the tiny workload: a random half of the prefix blocks starts
    resident, filling the pool.
    """
    S = w.n_slots
    sb = np.full((w.batch, w.kv_heads, S), -1, dtype=np.int32)
    lu = np.full((w.batch, w.kv_heads, S), -1, dtype=np.int32)
    nb0 = w.blocks_at(w.prefix_tokens)
    n = min(S, int(round(w.initial_resident_frac * nb0)))
    for b in range(w.batch):
        for h in range(w.kv_heads):
            g = _rng(w, layer, _RESID, b, h)
            sb[b, h, :n] = g.choice(nb0, size=n, replace=False)
    return sb, lu


def evict_draws(w: Workload, step: int, layer: int = 0) -> np.ndarray:
    """Uniform draws [B][Hkv][K] used to pick forced evictions at a step start."""
    g = _rng(w, layer, _EVICT, step)
    return g.random((w.batch, w.kv_heads, w.k_blocks))


def forced_evictions(w: Workload, attended: np.ndarray, n_attended: int, draws: np.ndarray) -> np.ndarray:
    """Blocks of the previous attended list to force out of HBM for one unit.

    Takes floor(frac * |A|) entries of A, uniformly without replacement: the
    positions of A with the smallest draws.  Returns the block ids.
    """
    n = int(np.floor(w.forced_evict_frac * n_attended + 1e-9))
    if n <= 0:
        return np.zeros(0, dtype=np.int32)
    pos = np.argsort(draws[:n_attended], kind="stable")[:n]
    return np.asarray(attended[:n_attended][pos], dtype=np.int32)
