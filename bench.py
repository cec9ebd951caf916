"""Decode-step benchmark of the OasisKV per-layer hot path on one MI355X.

One step = append one token -> score every block against the current and
draft queries -> per-KV-head top-K -> diff/cap/LRU -> host->HBM gather ->
sparse GQA attention, for the whole batch of one layer, through the C-ABI.
Inputs are seeded synthetic tensors already resident (prompt KV in pinned host
memory and block summaries in HBM) before the timed region.

Prints one JSON line.  `value` is decode layer-steps/s of the Qwen3-8B layer
workload.  The headline roofline object is the metric's own HBM figure:
the algorithmic bytes of the block scoring and of the sparse attention (its
attended KV, queries and output) over the summed average launch times of the
score, attention and combine kernels, from HIP events attached to their
dispatches on their stream during a timed region (one launch in
--timing-period, spread evenly over the region, so that the events barely
disturb the measured throughput).  It is taken from the leg in which the
fetched blocks are copied by the gather kernel on the copy stream, where
score and attention run as pure HBM kernels; in the main leg the copy runs
inside the attention kernel, which is then bound by the host link (that leg's
figure is hbm_gbps_score_attn).  Per-kernel objects (score, attention,
host_link, split_fetch, fused_score_topk, verify_attention) follow, with
fractions against the 8 TB/s spec, the box's measured streaming-read rate
(2 GiB) and cold plain reads of the kernels' own bytes.  The default run then
adds the Llama-3.1-8B 128K layer, the Qwen3-32B layer (its forced evictions
applied on the device inside every timed step) and a few steps of the
36-layer model under "workloads".  The CPU baseline is the fp64 oracle timed
on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decode steps/s per layer + achieved HBM GB/s (score+sparse attn) at 2,048-token "
          "budget")
HBM_PEAK_GBPS = 8000.0
PCIE_GEN5_X16_GBPS = 64.0   # host link, one direction


KERNEL_SOURCES = {
    "oasis_score": ["score.hip", "score_tile.h"],
    "oasis_sparse_attn": ["attention.hip", "combine.h"],
    "oasis_sparse_attn_hbm": ["attention.hip", "combine.h"],
    "oasis_combine": ["attention.hip", "combine.h"],
    "oasis_topk_select": ["selection.hip"],
    "oasis_score_topk_select": ["selection.hip", "score_tile.h"],
}


def kernel_source_sha(kernel: str) -> str:
    """sha256 of the HIP sources a kernel is built from (its file, plus the
    shared headers), so stored counter readings can be tied to the code."""
    import hashlib
    d = os.path.join(ROOT, "lookahead_sparse_kv_oasis_amd", "csrc")
    h = hashlib.sha256()
    for f in ["common.h", "kernels.h"] + KERNEL_SOURCES[kernel]:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a plain-copy calibration) and stored under profiles/, or None
    when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    e = data.get("workloads", {}).get(workload, {}).get(kernel)
    if not e or e.get("source_sha256") != kernel_source_sha(kernel):
        return None
    return e.get("hbm_bytes_per_launch")


def _workloads():
    import synth
    return {w.name: w for w in synth.WORKLOADS}


def pinned_h2d_peak_gbps(nbytes=1 << 30, reps=10):
    """Best pinned host -> device copy rate (hipMemcpyAsync through torch)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        best = max(best, nbytes / (time.perf_counter() - t0) / 1e9)
    del src, dst
    return best


def hbm_read_peak(same_sizes=(), nbytes=2 << 30, reps=5):
    """The box's streaming-read rate of HBM with oasis_stream_read.

    "gbps": a buffer eight times the 256 MB last-level cache read once, best
    of `reps` launches for each of a few grid sizes.  "same_size": for each
    byte count in same_sizes (the per-launch bytes of a kernel), a buffer of
    that size read once right after the large buffer has evicted the cache,
    best of `reps`: a plain read of the same bytes, with the same launch ramp
    and drain as the kernel it is compared with.  HIP events on the launching
    stream."""
    import torch
    from lookahead_sparse_kv_oasis_amd import stream_read
    big = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    big.fill_(0x01020304)
    sinks = {w: torch.empty(w, dtype=torch.int32, device="cuda")
             for w in (1024, 2048, 4096, 8192, 16384, 32768)}

    def timed(buf, wgs, flush):
        if flush:
            stream_read(big, sinks[8192], 8192)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        stream_read(buf, sinks[wgs], wgs)
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e-3

    best = (0.0, 0)
    for wgs in sinks:
        stream_read(big, sinks[wgs], wgs)   # warm the code path
        mine = max(nbytes / timed(big, wgs, False) / 1e9 for _ in range(reps))
        if mine > best[0]:
            best = (mine, wgs)
        print(f"# HBM streaming read, {wgs} workgroups: {mine:.0f} GB/s", file=sys.stderr,
              flush=True)
    out = {"gbps": best[0], "workgroups": best[1], "bytes": nbytes, "same_size": {}}
    for n in same_sizes:
        n16 = int(n) // 16 * 16
        buf = torch.empty(n16 // 4, dtype=torch.int32, device="cuda")
        buf.fill_(1)
        g = max(n16 / timed(buf, wgs, True) / 1e9 for wgs in (1024, 4096, 8192)
                for _ in range(reps))
        out["same_size"][str(int(n))] = g
        print(f"# HBM streaming read of {n16 / 1e6:.1f} MB after a cache flush: {g:.0f} GB/s",
              file=sys.stderr, flush=True)
        del buf
    del big, sinks
    torch.cuda.synchronize()
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, target_s=12.0, max_threads=16, bytes_per_step=None):
    """The fp64 oracle (as it stands) on a bounded sample of the workload: up
    to 64 (b, KV head) units stepped through the same decode steps (appended
    tokens continue the seeded draws past the workload's step count) on a pool
    of host threads, sized from a one-step calibration to about target_s of
    wall time.  Extrapolated to whole-layer steps/s; with bytes_per_step (the
    algorithmic score + attention bytes of one layer step) also as an
    effective GB/s.  phase_share: each phase's share of the oracle's time."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth
    from oracle.trajectory import initial_unit, workload_cap

    threads = min(max_threads, len(os.sched_getaffinity(0)))
    units_all = w.batch * w.kv_heads
    n_units = min(units_all, 64)
    cap = workload_cap(w)
    qf = oracle.to_f64(synth.queries(w), w.dtype)
    units = [divmod((i * 37) % units_all, w.kv_heads) for i in range(n_units)]
    # calibrate: one unit, two steps
    probe = initial_unit(w, *units[0], 2)
    one = []
    for t in (1, 2):
        x, cur = oracle.unit_rows(qf, oracle.to_f64(synth.drafts(w, t), w.dtype), *units[0],
                                  w.group)
        t0 = time.perf_counter()
        probe.step(t, x, cur, cap)
        one.append(time.perf_counter() - t0)
    per = min(one)
    steps = int(max(2, min(1024, target_s * threads / max(per * n_units, 1e-9))))
    with ThreadPoolExecutor(threads) as ex:
        us = list(ex.map(lambda bh: initial_unit(w, bh[0], bh[1], steps), units))
        drafts = list(ex.map(lambda t: oracle.to_f64(synth.drafts(w, t), w.dtype),
                             range(1, steps + 1)))

    phases = [dict() for _ in range(n_units)]

    def run(i):
        b, h = units[i]
        for t in range(1, steps + 1):
            x, cur = oracle.unit_rows(qf, drafts[t - 1], b, h, w.group)
            us[i].step(t, x, cur, cap, phase_times=phases[i])

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, range(n_units)))
    dt = time.perf_counter() - t0
    unit_steps_per_s = n_units * steps / dt
    total = {}
    for p in phases:
        for k, v in p.items():
            total[k] = total.get(k, 0.0) + v
    tsum = sum(total.values()) or 1.0
    value = unit_steps_per_s / units_all
    return {
        "value": value,
        "unit": "layer-steps/s",
        "cores": threads,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "effective_gbps": value * bytes_per_step / 1e9 if bytes_per_step else None,
        "phase_share": {k: v / tsum for k, v in total.items()},
        "sample": f"{n_units} of {units_all} (batch row, KV head) units x {steps} decode steps "
                  f"of {w.name} (append, fp64 score, top-K, select, attention), {dt:.1f} s "
                  f"wall on {threads} threads, scaled to one whole-layer step",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default=None, choices=sorted(_workloads()),
                    help="one workload only (default: the Qwen3-8B layer, then the other "
                         "layer workloads and the 36-layer model as extra keys)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-h2d-peak", action="store_true")
    ap.add_argument("--no-read-peak", action="store_true",
                    help="skip the HBM streaming-read measurement (2 GiB, a few launches)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB five times "
                         "(reference for the HBM byte counters) and exit")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the per-kernel HIP events (roofline fields become null)")
    ap.add_argument("--timing-period", type=int, default=4,
                    help="attach HIP events to one launch in this many of each timed kernel "
                         "(spread over the timed region)")
    ap.add_argument("--schedule", default="overlap", choices=["overlap", "serial", "both"],
                    help="multi-layer workloads: prediction/selection of later layers on a "
                         "second stream under earlier layers' attention, or one stream")
    ap.add_argument("--data-layers", type=int, default=2,
                    help="multi-layer workloads: distinct host KV buffers the layers alias")
    ap.add_argument("--fetch-ratio", default=None,
                    help="override the workload's fetch ratio ('all' = cap K)")
    ap.add_argument("--layers", type=int, default=None,
                    help="override the workload's layer count (1 = the single-layer path)")
    ap.add_argument("--correct-cap", type=int, default=0,
                    help="lookahead workloads: decode-time miss correction with this cap per "
                         "(b, KV head) and step (0: attention over the prefetched set)")
    ap.add_argument("--fuse-score-topk", action="store_true",
                    help="score, top-K and select in one kernel where the shape allows")
    ap.add_argument("--no-split-leg", action="store_true",
                    help="skip the leg that copies fetched blocks with the gather kernel")
    ap.add_argument("--no-fused-leg", action="store_true",
                    help="single layers: skip the second timed leg with score, top-K and select fused")
    ap.add_argument("--sweep", action="store_true",
                    help="multi-layer workloads: one line per fetch ratio of the sweep")
    ap.add_argument("--extra-steps", type=int, default=16,
                    help="default run: timed steps of each extra workload (36-layer model: 3)")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="default run: the Qwen3-8B layer alone")
    ap.add_argument("--copy-cus", type=int, default=0,
                    help="partition the CUs: copy stream on CUs [0, N), compute (and side) "
                         "streams on the rest, handles sized for them (0: no partition)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch row, KV head) unit of the decode "
              "path is independent, so several GPUs would each run this same measurement on "
              "their own share; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    if args.copy_cus > 0:
        from lookahead_sparse_kv_oasis_amd import stream_destroy
        _partition(args.copy_cus)
        with torch.cuda.stream(_PART["compute"]):
            _run(args)
        torch.cuda.synchronize()
        for k in ("compute", "side", "copy"):
            stream_destroy(_PART[k].cuda_stream)
        return
    _run(args)


# CU partition of the run (--copy-cus): compute units of the compute streams
# and the streams themselves
_PART = {}
# side and transfer streams of the multi-layer executors
_MODEL_STREAMS = {}


def _partition(n_copy):
    import torch

    from lookahead_sparse_kv_oasis_amd import stream_create_cus
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    if not 0 < n_copy < ncu:
        raise SystemExit(f"--copy-cus must be in 1..{ncu - 1}")
    ext = torch.cuda.ExternalStream
    _PART.update(cus=ncu - n_copy, copy_cus=n_copy,
                 compute=ext(stream_create_cus(n_copy, ncu - n_copy)),
                 side=ext(stream_create_cus(n_copy, ncu - n_copy)),
                 copy=ext(stream_create_cus(0, n_copy)))


def _run(args):
    import torch

    default_run = args.workload is None
    w = _workloads()[args.workload or "qwen3_8b_layer_b32_t32k_bf16"]
    if args.layers is not None:
        w = w.with_(layers=args.layers)
    if w.layers > 1:
        for line in bench_model(args, w):
            print(json.dumps(line), flush=True)
        return
    if args.fetch_ratio is not None:
        w = w.with_(fetch_ratio=1.0 if args.fetch_ratio == "all" else float(args.fetch_ratio),
                    cap=0)
    line = bench_layer(args, w, args.steps, args.warmup, main_leg=True)
    if default_run and not args.no_extra_workloads and not args.no_kernel_timing:
        # the other layer workloads and the 36-layer model, each with its own
        # figures, as extra keys of the one line
        line["workloads"] = {}
        shared = dict(h2d=line["host_link"]["pinned_h2d_peak_gbps"],
                      read_peak=(line["hbm_read_peak"] or {}).get("gbps"))
        import gc
        for name in ("llama31_8b_layer_b8_t128k_bf16", "qwen3_32b_layer_b16_t32k_bf16",
                     "qwen3_8b_layer_b32_t32k_bf16_lookahead"):
            print(f"# extra workload {name}", file=sys.stderr, flush=True)
            sub = bench_layer(args, _workloads()[name], args.extra_steps, 2, main_leg=False,
                              shared=shared)
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data",
                      "cpu_baseline", "hbm_read_peak", "_bytes_per_step"):
                sub.pop(k, None)
            line["workloads"][name] = sub
            gc.collect()
            torch.cuda.empty_cache()
        # the 36-layer model within the step (the layer overlap), then in the
        # lookahead order with score, top-K and select fused (its fastest form)
        for mname, fuse in (("qwen3_8b_36layer_b64_t64k_bf16", False),
                            ("qwen3_8b_36layer_b64_t64k_bf16_lookahead", True)):
            m = _workloads()[mname]
            print(f"# extra workload {m.name}", file=sys.stderr, flush=True)
            margs = argparse.Namespace(**vars(args))
            margs.steps, margs.warmup, margs.sweep, margs.fetch_ratio = 3, 1, False, None
            margs.no_cpu_baseline, margs.no_h2d_peak, margs.no_read_peak = True, True, True
            margs.schedule = "overlap"
            margs.fuse_score_topk = fuse
            sub = bench_model(margs, m)[0]
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data",
                      "cpu_baseline"):
                sub.pop(k, None)
            line["workloads"][m.name] = sub
            gc.collect()
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, bytes_per_step=line["_bytes_per_step"])
    line.pop("_bytes_per_step", None)
    print(json.dumps(line), flush=True)


def bench_layer(args, w, steps, warmup, main_leg=True, shared=None):
    """One layer workload: the main timed leg (the handle's default schedule,
    fetch inside the attention), then on the same handle, where the layout
    allows, the fused score + top-K + select leg (main workload only) and the
    split leg (fetch by the gather kernel on the copy stream, so score and
    attention run as pure HBM kernels: the metric's HBM figure comes from it).
    Returns the JSON line as a dict."""
    import numpy as np
    import torch

    import synth
    from lookahead_sparse_kv_oasis_amd import TIME
    from lookahead_sparse_kv_oasis_amd.runner import LayerRunner

    shared = shared or {}
    mfma_layout = (w.dtype == synth.BF16 and w.head_dim == 128 and w.block_size == 16)
    # a second timed leg with score, top-K and select in one kernel, where that
    # kernel applies (tiled bf16 d = 128, >= 256 units)
    fused_leg = (main_leg and not args.fuse_score_topk and not args.no_fused_leg and
                 not w.lookahead and not args.no_kernel_timing and mfma_layout and
                 w.batch * w.kv_heads >= 256)
    # a leg with the fetch as its own kernel, so that score and attention are
    # timed as pure HBM kernels and the host-link copy on its own
    split_leg = (mfma_layout and not w.lookahead and not args.no_split_leg and
                 not args.no_kernel_timing)
    n_main = warmup + steps
    n_fused_end = n_main + (steps if fused_leg else 0)
    n_steps = n_fused_end + (steps if split_leg else 0)
    t_setup = time.perf_counter()
    run = LayerRunner(w, n_steps, compute_units=_PART.get("cus", 0))
    h = run.h
    if args.fuse_score_topk:
        h.oasis_set_score_topk_fusion(True)
    stream = torch.cuda.current_stream()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s: {w.name}, {n_steps} steps",
          file=sys.stderr, flush=True)
    rec = None
    # lookahead order on a CU partition (--copy-cus): each select's blocks are
    # copied on the copy stream while the next step runs on this one
    beside = bool(_PART) and w.lookahead and args.correct_cap == 0
    if w.lookahead:
        # [OASIS] Fig. 8 ordering; the warmup steps also measure prediction recall
        rec = warmup_ahead_with_recall(run, warmup, stream, args.correct_cap)
        if args.correct_cap > 0:
            step = lambda t, st: run.step_corrected(t, args.correct_cap, st)
        elif beside:
            # the transfer on the copy stream's own CUs, beside the next
            # step's scoring and attention over held blocks
            h.oasis_set_attention_beside_copy(True)
            step = lambda t, st: run.step_beside(t, st, _PART["copy"])
        else:
            step = run.step_ahead
    else:
        if w.admission:
            run.admission(stream)
        for t in range(1, warmup + 1):
            run.step(t, stream)
        step = run.step
    torch.cuda.synchronize()
    stats0 = h.oasis_get_stats()
    # with miss correction the prefetch select's blocks are copied by the
    # standalone gather (the next select rewrites the fetch list first)
    correcting = w.lookahead and args.correct_cap > 0
    # events only around the kernels of the metric (score, attention and the
    # combine of its partials), sampled, to keep the step itself unperturbed
    h.oasis_set_timing(0 if args.no_kernel_timing else
                       TIME["score"] | TIME["attn"] | TIME["combine"] |
                       (0 if stats0["fetch_fused"] and not correcting and not beside
                        else TIME["gather"]))
    h.oasis_set_timing_period(args.timing_period)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warmup + 1, n_main + 1):
        step(t, stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    tm = h.oasis_get_timing()
    stats1 = h.oasis_get_stats()
    h.oasis_check()
    verify = None
    if main_leg and mfma_layout and not w.lookahead and not args.no_kernel_timing:
        verify = time_verify(run, w)
    K = steps
    e = w.elem_bytes
    units = w.batch * w.kv_heads
    d, bs = w.head_dim, w.block_size
    blk_bytes = 2 * bs * d * e
    # algorithmic bytes per launch
    nb_avg = np.mean([w.blocks_at(w.prefix_tokens + t) for t in range(warmup + 1, n_main + 1)])
    q_bytes = w.batch * w.q_heads * d * e
    out_bytes = w.batch * w.q_heads * d * 4
    score_bytes = units * nb_avg * 2 * d * e + q_bytes * (1 + w.drafts) + units * nb_avg * 4
    attended = (stats1["attended"] - stats0["attended"]) / K
    fetched = (stats1["fetched"] - stats0["fetched"]) / K
    # with the copy beside, the timed attention launch reads the held blocks
    # only (the fetched ones follow in a second, untimed launch)
    attn_bytes = (attended - (fetched if beside else 0)) * blk_bytes + q_bytes + out_bytes
    base = {"metric": METRIC, "value": K / dt, "unit": "layer-steps/s", "n_gpus": 1,
            "steps": K, "warmup": warmup, "ms_per_step": dt / K * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if w.dtype == synth.BF16 else "f32", "data": "synthetic",
            "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads,
                       "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                       "context": w.prefix_tokens, "block_size": bs,
                       "budget_tokens": w.budget_tokens, "drafts": w.drafts,
                       "fetch_ratio": w.fetch_ratio, "cap_per_kv_head": run.cap,
                       "forced_evict_frac": w.forced_evict_frac,
                       "fuse_score_topk": bool(args.fuse_score_topk),
                       **({"copy_cus": _PART["copy_cus"]} if _PART else {})},
            "_bytes_per_step": score_bytes + attn_bytes}
    if args.no_kernel_timing:
        base.update(roofline=None, cpu_baseline=None)
        return base
    ms_score = tm["ms_score"] / max(tm["n_score"], 1)
    ms_attn = (tm["ms_attn"]) / max(tm["n_attn"], 1)
    ms_comb = tm["ms_combine"] / max(tm["n_combine"], 1)
    ms_gather = tm["ms_gather"] / max(tm["n_gather"], 1)
    score_gbps = score_bytes / (ms_score * 1e-3) / 1e9
    attn_gbps = attn_bytes / (ms_attn * 1e-3) / 1e9
    hbm_gbps = (score_bytes + attn_bytes) / ((ms_score + ms_attn + ms_comb) * 1e-3) / 1e9
    # the fetch runs inside the next attention, in the lookahead order too
    # (the append before it leaves it pending)
    fused = bool(stats1["fetch_fused"]) and not correcting and not beside
    # with the fetch fused into the attention kernel the host-link transfer
    # runs inside it: its rate is bounded below by bytes / attention time.
    # With miss correction the corrective fetch runs inside the attention and
    # the prefetch in the standalone gather, so the step's fetched bytes span
    # both launches.
    g_ms = ms_attn if fused else (ms_attn + ms_gather if correcting else ms_gather)
    fetch_in_attn = fused or correcting
    gather_gbps = fetched * blk_bytes / (g_ms * 1e-3) / 1e9 if g_ms > 0 else None
    h2d = shared.get("h2d") if not main_leg else (
        None if args.no_h2d_peak else pinned_h2d_peak_gbps())
    rpk = None
    if main_leg and not args.no_read_peak:
        rpk = hbm_read_peak((score_bytes, attn_bytes, score_bytes + attn_bytes))
    read_peak = rpk["gbps"] if rpk else shared.get("read_peak")
    link_gbps = h2d if h2d is not None else PCIE_GEN5_X16_GBPS
    attn_link_bound = (fetch_in_attn and fetched * blk_bytes / (link_gbps * 1e9) >=
                       attn_bytes / ((read_peak or 6500.0) * 1e9))

    def same(n):
        return rpk["same_size"].get(str(int(n))) if rpk else None

    def frac_of(x, ref):
        return x / ref if (x and ref) else None

    line = dict(base)
    line.update({
        "hbm_gbps_score_attn": hbm_gbps,
        "score": {"kernel": "oasis_score_topk_select" if args.fuse_score_topk else "oasis_score",
                  "avg_ms": ms_score, "hbm_bytes_per_launch": score_bytes,
                  "hbm_gbps": score_gbps, "hbm_frac": score_gbps / HBM_PEAK_GBPS,
                  "same_size_read_gbps": same(score_bytes),
                  "frac_of_same_size_read": frac_of(score_gbps, same(score_bytes)),
                  "traffic": stored_traffic("oasis_score_topk_select" if args.fuse_score_topk
                                            else "oasis_score", w.name)},
        "attention": {"kernel": "oasis_sparse_attn", "avg_ms": ms_attn,
                      "hbm_bytes_per_launch": attn_bytes, "hbm_gbps": attn_gbps,
                      "hbm_frac": attn_gbps / HBM_PEAK_GBPS,
                      "hbm_frac_of_measured_read_peak": frac_of(attn_gbps, read_peak),
                      "same_size_read_gbps": same(attn_bytes),
                      "bound": "host_link" if attn_link_bound else "hbm",
                      "fetch_inside": fetch_in_attn},
        "host_link": {"kernel": "oasis_sparse_attn (fused fetch)" if fused else
                      "oasis_sparse_attn (corrective fetch) + oasis_gather (prefetch)"
                      if correcting else "oasis_gather (copy stream, CUs of its own)"
                      if beside else "oasis_gather",
                      "achieved_gbps": gather_gbps, "pinned_h2d_peak_gbps": h2d,
                      "frac": frac_of(gather_gbps, h2d),
                      "pcie_gen5_x16_gbps": PCIE_GEN5_X16_GBPS,
                      "blocks_per_step": fetched, "bytes_per_step": fetched * blk_bytes},
        "kernels_avg_ms": {"score": ms_score, "attn": ms_attn, "combine": ms_comb,
                           **({} if fused else {"gather": ms_gather})},
        "timed_launches": {"score": tm["n_score"], "attn": tm["n_attn"],
                           "period": args.timing_period},
        "attended_blocks_per_step": attended,
        "hbm_read_peak": rpk,
    })
    # Headline roofline before the split leg (replaced by it below): the
    # metric's score + attention (+ combine) figure of the main leg, honest
    # but host-link bound whenever the fetch inside the attention outlasts
    # its HBM stream.
    line["roofline"] = {
        "bound": "hbm", "kernel": "oasis_score + oasis_sparse_attn + combine",
        "leg": "main", "achieved": hbm_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": hbm_gbps / HBM_PEAK_GBPS, "traffic": None,
        "per_launch_bytes": score_bytes + attn_bytes, "avg_ms": ms_score + ms_attn + ms_comb,
        "measured_read_peak_gbps": read_peak,
        "frac_of_measured_read_peak": frac_of(hbm_gbps, read_peak)}
    if fused_leg:
        h.oasis_set_score_topk_fusion(True)
        h.oasis_set_timing(TIME["score"] | TIME["select"])
        h.oasis_set_timing_period(args.timing_period)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(n_main + 1, n_fused_end + 1):
            step(t, stream)
        torch.cuda.synchronize()
        dt2 = time.perf_counter() - t0
        tm2 = h.oasis_get_timing()
        h.oasis_check()
        h.oasis_set_score_topk_fusion(False)
        if tm2["n_select"] == 0 and tm2["n_score"] > 0:
            ms_f = tm2["ms_score"] / tm2["n_score"]
            f_gbps = score_bytes / (ms_f * 1e-3) / 1e9
            line["fused_score_topk"] = {
                "value": K / dt2, "ms_per_step": dt2 / K * 1e3,
                "kernel": "oasis_score_topk_select", "avg_ms": ms_f,
                "achieved_gbps": f_gbps, "frac": f_gbps / HBM_PEAK_GBPS,
                "traffic": stored_traffic("oasis_score_topk_select", w.name),
                "steps": K, "note": "same handle, the K steps after the main timed region, "
                "score + top-K + select in one kernel (bit-identical results)"}
    if split_leg:
        h.oasis_set_fetch_in_attention(False)
        h.oasis_set_timing(TIME["score"] | TIME["attn"] | TIME["combine"] | TIME["gather"])
        h.oasis_set_timing_period(args.timing_period)
        st0 = h.oasis_get_stats()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(n_fused_end + 1, n_steps + 1):
            step(t, stream)
        torch.cuda.synchronize()
        dt3 = time.perf_counter() - t0
        tm3 = h.oasis_get_timing()
        st1 = h.oasis_get_stats()
        h.oasis_check()
        h.oasis_set_fetch_in_attention(True)
        if min(tm3["n_score"], tm3["n_attn"], tm3["n_gather"]) > 0:
            s3 = tm3["ms_score"] / tm3["n_score"]
            a3 = tm3["ms_attn"] / tm3["n_attn"]
            g3 = tm3["ms_gather"] / tm3["n_gather"]
            c3 = tm3["ms_combine"] / max(tm3["n_combine"], 1)
            att3 = (st1["attended"] - st0["attended"]) / K
            f3 = (st1["fetched"] - st0["fetched"]) / K
            ab3 = att3 * blk_bytes + q_bytes + out_bytes
            sa3 = (score_bytes + ab3) / ((s3 + a3 + c3) * 1e-3) / 1e9
            g_gbps = f3 * blk_bytes / (g3 * 1e-3) / 1e9
            line["split_fetch"] = {
                "value": K / dt3, "ms_per_step": dt3 / K * 1e3,
                "score_attn_hbm_gbps": sa3, "score_attn_frac": sa3 / HBM_PEAK_GBPS,
                "score_attn_frac_of_measured_read_peak": frac_of(sa3, read_peak),
                "score_avg_ms": s3, "attn_avg_ms": a3, "combine_avg_ms": c3,
                "attn_hbm_gbps": ab3 / (a3 * 1e-3) / 1e9,
                "attn_bytes_per_launch": ab3,
                "gather_avg_ms": g3, "gather_gbps": g_gbps,
                "gather_frac_of_pinned_h2d": frac_of(g_gbps, h2d),
                "steps": K, "note": "same handle, the K steps after the earlier legs, fetched "
                "blocks copied by the gather kernel on the copy stream (the same "
                "selections and payloads; outputs equal up to the split-K merge order): "
                "score and attention timed as pure HBM kernels, the copy on its own; "
                "slower per step than the copy inside the attention"}
            # The metric's HBM figure with score and attention as pure HBM
            # kernels: algorithmic bytes of both over their summed average
            # launch times (the combine of the attention's partials included).
            parts = [stored_traffic(k, w.name) for k in
                     ("oasis_score", "oasis_sparse_attn_hbm", "oasis_combine")]
            line["roofline"] = {
                "bound": "hbm", "kernel": "oasis_score + oasis_sparse_attn + combine",
                "leg": "split_fetch", "achieved": sa3, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": sa3 / HBM_PEAK_GBPS,
                "traffic": sum(parts) if all(x is not None for x in parts) else None,
                "per_launch_bytes": score_bytes + ab3, "avg_ms": s3 + a3 + c3,
                "kernels_avg_ms": {"score": s3, "attn": a3, "combine": c3},
                "measured_read_peak_gbps": read_peak,
                "frac_of_measured_read_peak": frac_of(sa3, read_peak),
                "same_size_read_gbps": same(score_bytes + attn_bytes),
                "frac_of_same_size_read": frac_of(sa3, same(score_bytes + attn_bytes))}
    if verify is not None:
        verify["attended_blocks"] = attended
        # bytes the passes read, and the attended KV once (what the call needs)
        verify["hbm_gbps"] = (verify["passes"] * attended * blk_bytes) / (verify["avg_ms"] * 1e-3) / 1e9
        verify["attended_kv_gbps"] = attended * blk_bytes / (verify["avg_ms"] * 1e-3) / 1e9
        line["verify_attention"] = verify
    if rec is not None:
        line["ordering"] = "lookahead"
        line["config"]["correct_cap"] = args.correct_cap
        line["recall"] = rec
    del run, h
    return line


def time_verify(run, w, calls=20):
    """Attention over the normal and draft query sets together (after the timed
    region; synthetic draft-token K/V): average call time with events on the
    caller's stream, and the number of passes over the attended KV."""
    import numpy as np
    import torch

    import synth
    from lookahead_sparse_kv_oasis_amd.runner import to_device

    D = w.drafts
    rng = np.random.default_rng(11)
    shape = (D, w.batch, w.kv_heads, w.head_dim)
    kd = to_device(synth.encode(rng.standard_normal(shape).astype(np.float32), w.dtype))
    vd = to_device(synth.encode(rng.standard_normal(shape).astype(np.float32), w.dtype))
    out = torch.empty((1 + D, w.batch, w.q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    t = run.t
    run.h.oasis_sparse_attn_verify(run.q, run.drafts[t], D, kd, vd, out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(calls):
        run.h.oasis_sparse_attn_verify(run.q, run.drafts[t], D, kd, vd, out)
    b.record()
    torch.cuda.synchronize()
    # passes of the library's cut: 32 rows while 32 remain, then the next
    # power of two at or above the rest (padded)
    rows = w.group * (1 + D)
    passes, padded, r = 0, 0, rows
    while r > 0:
        g = 32
        if r < 32:
            g = 1
            while g < r:
                g *= 2
        r -= min(r, g)
        padded += g
        passes += 1
    return {"avg_ms": a.elapsed_time(b) / calls, "query_sets": 1 + D, "rows_per_kv_head": rows,
            "padded_rows_per_kv_head": padded, "passes": passes, "calls": calls}


def warmup_ahead_with_recall(run, warmup, stream, cap_correct=0):
    """Admission and `warmup` lookahead steps of a LayerRunner; each step also
    scores the step's own query to get the exact top-K (untimed), giving the
    recall of the drafts' prediction (made one step earlier) and of the
    previous query's exact top-K ([OASIS] Fig. 4, synthetic analog)."""
    import numpy as np
    import torch

    from lookahead_sparse_kv_oasis_amd.runner import exact_ids, predicted_ids, recall

    h, w = run.h, run.w
    buf = torch.empty(w.batch * w.kv_heads * w.k_blocks, dtype=torch.int32, device="cuda")
    run.admission_ahead(stream)
    torch.cuda.synchronize()
    r_ahead, r_prev, prev = [], [], None
    miss, left = [], []
    for t in range(1, warmup + 1):
        pred = predicted_ids(h)
        h.oasis_append_kv(run.app_k[t - 1], run.app_v[t - 1], stream=stream)
        ex = exact_ids(h, run.q_steps[t], buf, stream)
        r_ahead.append(recall(pred, ex))
        if prev is not None:
            r_prev.append(recall(prev, ex))
        prev = ex
        if cap_correct > 0:
            # the exact ids are the selection now: correct with them
            h.oasis_select_and_fetch(cap_correct, stream=stream)
            c = h.read("COUNTS").reshape(-1, 4)
            miss.append(float(c[:, 3].mean()) / w.k_blocks)
            left.append(float(np.maximum(c[:, 3] - cap_correct, 0).mean()) / w.k_blocks)
        h.oasis_sparse_attn(run.q_steps[t], run.out, stream=stream)
        h.oasis_predict(None, run.drafts[t], w.drafts, stream=stream)
        h.oasis_select_and_fetch(run.cap, stream=stream)
    out = {"drafts": float(np.mean(r_ahead)) if r_ahead else None,
           "previous_query": float(np.mean(r_prev)) if r_prev else None,
           "steps": warmup, "what": "mean over units and steps of |predicted top-K ∩ exact "
                                    "top-K of the step's own query| / K"}
    if cap_correct > 0:
        out["decode_time_miss_rate"] = float(np.mean(miss)) if miss else None
        out["left_after_correction"] = float(np.mean(left)) if left else None
        out["correct_cap"] = cap_correct
    return out


def bench_model(args, w):
    """All layers of a multi-layer workload per step through oasis_decode_layers;
    returns one line (dict) per fetch ratio."""
    import numpy as np
    import torch

    import synth
    from lookahead_sparse_kv_oasis_amd import TIME, cap_from_ratio
    from lookahead_sparse_kv_oasis_amd.runner import ModelRunner

    n_steps = args.warmup + args.steps
    if n_steps > w.steps:
        w = w.with_(steps=n_steps)
    t_setup = time.perf_counter()
    log = lambda m: print("# " + m, file=sys.stderr, flush=True)
    mr = ModelRunner(w, n_steps, data_layers=args.data_layers, log=log,
                     compute_units=_PART.get("cus", 0))
    if args.fuse_score_topk:
        for h in mr.handles:
            h.oasis_set_score_topk_fusion(True)
    log(f"setup {time.perf_counter() - t_setup:.1f}s: {w.name}, {w.layers} layers on "
        f"{mr.H} host KV buffers, {n_steps} steps")
    if args.sweep:
        ratios = synth.FETCH_RATIO_SWEEP
    elif args.fetch_ratio is not None:
        ratios = [None if args.fetch_ratio == "all" else float(args.fetch_ratio)]
    else:
        ratios = [w.fetch_ratio]
    schedules = ["overlap", "serial"] if args.schedule == "both" else [args.schedule]
    stream = torch.cuda.current_stream()
    side, xfer = _PART.get("side"), _PART.get("copy")
    if side is None:
        # made once per process: the runtime spreads streams over a few
        # hardware queues (4 here) in creation order, and a later pair of
        # pool streams can land on the queue of the caller's stream, which
        # then serializes the overlap (17.2 against 10.9 ms per 36-layer
        # lookahead step when a second model ran with new streams)
        if "side" not in _MODEL_STREAMS:
            _MODEL_STREAMS.update(side=torch.cuda.Stream(), xfer=torch.cuda.Stream())
        side, xfer = _MODEL_STREAMS["side"], _MODEL_STREAMS["xfer"]
    h2d = None if args.no_h2d_peak else pinned_h2d_peak_gbps()
    rpk = None if args.no_read_peak else hbm_read_peak()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w.with_(layers=1))
    e, d, bs = w.elem_bytes, w.head_dim, w.block_size
    units = w.batch * w.kv_heads
    blk_bytes = 2 * bs * d * e
    q_bytes = w.batch * w.q_heads * d * e
    L = w.layers
    first = True
    lines = []
    for ratio in ratios:
        cap = w.k_blocks if ratio is None else cap_from_ratio(ratio, w.k_blocks)
        res = {}
        for sched in schedules:
            sd = side if sched == "overlap" else None
            if not first:
                mr.reset()
            first = False
            if w.lookahead:
                sd2 = side if sched == "overlap" else stream
                xf = xfer if sched == "overlap" else stream
                mr.admission_ahead(stream, sd2, xf)
                mstep = (lambda t, sd2=sd2, xf=xf:
                         mr.step_ahead(t, stream, sd2, xf, cap, args.correct_cap))
            else:
                mr.admission(stream, sd)
                mstep = lambda t, sd=sd: mr.step(t, stream, sd, cap)
            for t in range(1, args.warmup + 1):
                mstep(t)
            torch.cuda.synchronize()
            s0 = [h.oasis_get_stats() for h in mr.handles]
            for h in mr.handles:
                h.oasis_set_timing(0 if args.no_kernel_timing else TIME["score"] | TIME["attn"])
                h.oasis_set_timing_period(args.timing_period)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for t in range(args.warmup + 1, n_steps + 1):
                mstep(t)
            t_issue = time.perf_counter() - t0
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            s1 = [h.oasis_get_stats() for h in mr.handles]
            tms = [h.oasis_get_timing() for h in mr.handles]
            for h in mr.handles:
                h.oasis_check()
                h.oasis_set_timing(0)
            fetched = sum(b["fetched"] - a["fetched"] for a, b in zip(s0, s1)) / args.steps
            attended = sum(b["attended"] - a["attended"] for a, b in zip(s0, s1)) / args.steps
            res[sched] = dict(dt=dt, fetched=fetched, attended=attended, tms=tms)
            n_sc = max(1, sum(tm["n_score"] for tm in tms))
            n_at = max(1, sum(tm["n_attn"] for tm in tms))
            log(f"ratio {ratio} cap {cap} {sched}: {dt / args.steps * 1e3:.3f} ms/step, "
                f"host issue {t_issue / args.steps * 1e3:.3f} ms/step, score "
                f"{sum(tm['ms_score'] for tm in tms) / n_sc * 1e3:.1f} us, attn "
                f"{sum(tm['ms_attn'] for tm in tms) / n_at * 1e3:.1f} us per launch, "
                f"{fetched:.0f} blocks fetched/step")
        main_sched = schedules[0]
        r = res[main_sched]
        K = args.steps
        dt = r["dt"]
        nb_avg = np.mean([w.blocks_at(w.prefix_tokens + t)
                          for t in range(args.warmup + 1, n_steps + 1)])
        score_bytes = units * nb_avg * 2 * d * e + q_bytes * (1 + w.drafts) + units * nb_avg * 4
        roof = None
        if not args.no_kernel_timing:
            n_sc = sum(tm["n_score"] for tm in r["tms"])
            ms_score = sum(tm["ms_score"] for tm in r["tms"]) / max(n_sc, 1)
            n_at = sum(tm["n_attn"] for tm in r["tms"])
            ms_attn = sum(tm["ms_attn"] for tm in r["tms"]) / max(n_at, 1)
            score_gbps = score_bytes / (ms_score * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": "oasis_score", "achieved": score_gbps,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                    "traffic": None, "per_launch_bytes": score_bytes, "avg_ms": ms_score,
                    "attn_avg_ms": ms_attn,
                    "measured_read_peak_gbps": rpk["gbps"] if rpk else None,
                    "frac_of_measured_read_peak": score_gbps / rpk["gbps"] if rpk else None}
        link_gbps = r["fetched"] * blk_bytes / (dt / K) / 1e9
        # the metric's HBM figure with the layers pipelined: every layer's
        # score and attention bytes of a step over the step's wall time
        pipe_bytes = L * score_bytes + r["attended"] * blk_bytes + \
            L * (q_bytes + w.batch * w.q_heads * d * 4)
        pipe_gbps = pipe_bytes / (dt / K) / 1e9
        line = {
            "metric": METRIC,
            "value": L * K / dt,
            "unit": "layer-steps/s",
            "n_gpus": 1, "steps": K, "warmup": args.warmup,
            "ms_per_step": dt / K * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if w.dtype == synth.BF16 else "f32", "data": "synthetic",
            "config": {"workload": w.name, "layers": L, "batch": w.batch,
                       "q_heads": w.q_heads, "kv_heads": w.kv_heads, "head_dim": d,
                       "context": w.prefix_tokens, "block_size": bs,
                       "budget_tokens": w.budget_tokens, "drafts": w.drafts,
                       "fetch_ratio": "all" if ratio is None else ratio,
                       "cap_per_kv_head": cap, "schedule": main_sched,
                       "ordering": "lookahead" if w.lookahead else "within step",
                       "correct_cap": args.correct_cap if w.lookahead else None,
                       "fuse_score_topk": bool(args.fuse_score_topk),
                       "host_kv_buffers": mr.H,
                       **({"copy_cus": _PART["copy_cus"]} if _PART else {})},
            "model_steps_per_s": K / dt,
            "roofline": roof,
            "pipelined_score_attn": {"hbm_bytes_per_step": pipe_bytes, "gbps": pipe_gbps,
                                     "frac": pipe_gbps / HBM_PEAK_GBPS,
                                     "note": "score + attention bytes of all layers per step "
                                             "over the step's wall time (kernels overlapped)"},
            "host_link": {"achieved_gbps_step_avg": link_gbps, "pinned_h2d_peak_gbps": h2d,
                          "blocks_per_step": r["fetched"],
                          "bytes_per_step": r["fetched"] * blk_bytes},
            "attended_blocks_per_step": r["attended"],
            "cpu_baseline": cpu,
        }
        if "serial" in res and main_sched != "serial":
            line["serial_ms_per_step"] = res["serial"]["dt"] / K * 1e3
            line["overlap_speedup"] = res["serial"]["dt"] / dt
        lines.append(line)
    mr.close()
    return lines


if __name__ == "__main__":
    main()
