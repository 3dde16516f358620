"""DSA decode throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode32k]

A step is one pass of the whole path -- head-gate, pool compression (of the
pools the step's newest row completes; all older pools are cached), index
scores, pool top-k, selection expansion, sparse MLA -- through the fused decode
calls (gate+compress, gated index scores, top-k+expand, sparse MLA) over one batch of
resident synthetic input: the 32K-context decode batch (16 requests x 32768
cached rows, one query each) by default.  Eight input sets (each larger than
the 256 MB last-level cache together with its outputs) are rotated so that
every step streams its keys and latent rows from HBM.  The timed region makes
one dsa_decode_step call per step (the library's step executor: one host call
that enqueues the fused calls on the stream; each set's arguments are
marshalled once, before timing), K steps in all (five equal segments give the
median per-step time too).  Beside it: each set's step captured in a HIP
graph of its own and replayed once per step, the eight sets' steps captured in
sequence in one graph (as a serving loop captures consecutive decode steps,
which spreads the host's graph-launch cost), the single-step graphs replayed
with two and with four
batches in flight (two or four streams, showing how much of the step is
fixed latency rather than throughput), the same step through the six separate calls, the step with
the attention reading a paged copy of the latent cache (64-row pages in
shuffled order, through a block table), and the whole decode step from
device-side live lengths (geometry, the store of the step's indexer row, the
fused calls, the paged attention).

The JSON line also carries, for the call that takes the most time, its
algorithmic bytes per launch over its average launch time (a graph of 32
back-to-back calls of that kind, replayed between HIP events on the launch
stream),
against the 8 TB/s HBM peak and against the lane (a plain coalesced read of
1 GiB, dsa_lane_read, timed in the same run); and the CPU oracle's throughput on a bounded
sample of the same workload, run on every host core before the GPU is used.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_attention_fp32_amd import dsa  # noqa: E402
from sparse_attention_fp32_amd import workloads as W  # noqa: E402
from sparse_attention_fp32_amd.pipeline import DsaStep  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
# the calls of the timed step (the fused decode calls) ...
STAGES = ("gate_compress", "index_scores_gated", "topk_expand", "sparse_mla_decode")
# ... and the six separate calls, timed for comparison
CALLS = ("head_gate", "kpool_compress", "index_scores", "topk_pools", "expand_selection",
         "sparse_mla_decode")
# kernel source behind each call (a change to it invalidates stored HBM counters)
STAGE_SOURCE = {"head_gate": "head_gate.hip", "kpool_compress": "kpool_compress.hip",
                "index_scores": "index_scores.hip", "topk_pools": "topk.hip",
                "expand_selection": "expand.hip", "sparse_mla_decode": "sparse_mla.hip",
                "gate_compress": "kpool_compress.hip", "index_scores_gated": "index_scores.hip",
                "topk_expand": "topk.hip"}


def algorithmic_bytes(spec: W.Spec, xn: dict, n_pools: np.ndarray, tok: np.ndarray) -> dict:
    """Bytes each call must move at least once (inputs read once, outputs
    written once), for the cached-pool decode step.  A pooled key or latent
    row that several queries of one request use (prefill) counts once."""
    Q, H, D, Hm, L = spec.Q, spec.index_heads, spec.index_dim, spec.mla_heads, spec.latent
    kp = spec.kpool
    req = np.asarray(xn["q_req"]).astype(np.int64)
    P_r = int(n_pools[np.unique(req)].astype(np.int64).sum())  # pools of the requests queried
    pst = spec.pstride()
    touched = len(spec.lengths)                        # one pool per request
    lat_row = L * (1 if spec.latent_fp8 else 2) + (4 if spec.latent_fp8 else 0)
    sel = tok >= 0                                     # distinct (request, row) pairs selected
    n_sel = int(np.unique(req[:, None].repeat(tok.shape[1], 1)[sel] * (1 << 32)
                          + tok[sel].astype(np.int64)).size)
    b = {
        "head_gate": 4 * (Q * spec.hidden + spec.hidden * H + Q * H),
        # kpool rows of k and gate per touched pool, ape, LN params, key + meta out,
        # the valid flags of each pool, offsets
        "kpool_compress": touched * (2 * kp * D * 2 + kp + D * 2 + 5) + kp * D * 2 + 8 * D
        + 4 * (2 * (spec.B + 1) + 2 * spec.B),
        "index_scores": P_r * (D * 2 + 5) + Q * H * (D * 2 + 4) + Q * pst * 5 + 12 * Q,
        "topk_pools": Q * pst * 5 + Q * spec.select_k * 4,
        "expand_selection": Q * spec.select_k * 8 + Q * spec.out_width * 4 + 8 * Q,
        "sparse_mla_decode": n_sel * lat_row + Q * Hm * L * 2 * 2 + Q * spec.out_width * 4
        + Q * Hm * 4 + 8 * Q,
    }
    # fused calls: the head-gate partials are written once and read once; sel is
    # written but not read back
    part = 4 * Q * H * max(1, spec.hidden // 128)
    b["gate_compress"] = b["head_gate"] - 4 * Q * H + part + b["kpool_compress"]
    b["index_scores_gated"] = b["index_scores"] - 4 * Q * H + part + 4 * Q * H
    b["topk_expand"] = b["topk_pools"] + b["expand_selection"] - Q * spec.select_k * 4
    return b


def source_sha(stage: str) -> str:
    p = os.path.join(ROOT, "sparse_attention_fp32_amd", "csrc", STAGE_SOURCE[stage])
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# kernels behind each call, by name (counters of a call add up over its kernels)
CALL_KERNELS = {
    "sparse_mla_decode": (r"sparse_mla_kernel<(true|false), false, (true|false)>",
                          r"mla_combine_kernel"),
    "index_scores_gated": (r"index_scores(_qblock)?_kernel<\d+, true",),
    # (a row selected in two stages runs the stage-1 kernel, shared by both
    # top-k calls, then the call's stage-2 kernel)
    "topk_expand": (r"topk_kernel<\d+, \d+, (true|false), true(, 0)?>",
                    r"topk_kernel<\d+, \d+, false, false, 1>",
                    r"topk_kernel<\d+, \d+, false, true, 2>"),
    "index_scores": (r"index_scores(_qblock)?_kernel<\d+, false",),
    "topk_pools": (r"topk_kernel<\d+, \d+, (true|false), false(, 0)?>",
                   r"topk_kernel<\d+, \d+, false, false, 1>",
                   r"topk_kernel<\d+, \d+, false, false, 2>"),
}


def stored_counters(stage: str, workload: str):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE scaled by the copy
    calibration) and MFMA / VALU busy of a call's kernels, from the rocprofv3
    summary stored in profiles/counters_<workload>.json, if it was taken on
    this call's current kernel source.  For each kernel of the call the grid
    launched most often (the timed step's) counts."""
    import re
    p = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if stage not in CALL_KERNELS or not os.path.exists(p):
        return None
    with open(p) as f:
        rows = json.load(f)["kernels"]
    cur = source_sha(stage)
    picked = []
    for pat in CALL_KERNELS[stage]:
        cand = [r for r in rows if re.match(pat, r["kernel"])]
        if not cand:
            continue
        r = max(cand, key=lambda r: r.get("dispatches", 0))
        if r["source_sha"] != cur:
            return None
        picked.append(r)
    if not picked:
        return None
    main = picked[0]
    return {"hbm_bytes": sum(r["fetch_bytes"] + r["write_bytes"] for r in picked),
            "mfma_util_pct": round(main["mfma_util_pct"], 2),
            "valu_busy_pct": round(main["valu_busy_pct"], 2), "kernel": main["kernel"]}


def _cpu_worker(xn, spec, q, core, budget_s, start, results):
    """One host core: the cached-pool oracle step of query q, repeated for
    budget_s seconds after every worker has compressed its request."""
    import oracle as O
    try:
        os.sched_setaffinity(0, {core})
    except OSError:  # pragma: no cover
        pass
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        r = int(xn["q_req"][q])
        prev = O.kpool_compress(xn["k"], xn["gate"], xn["ape"], xn["valid"], xn["tok_off"],
                                xn["pool_off"], xn["ln_w"], xn["ln_b"], spec.eps, spec.kpool,
                                requests=[r])
        start.wait()
        reps, t0 = 0, time.perf_counter()
        while True:
            O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                       spec.sm_scale, new_from=xn["new_from"], prev=prev, queries=[q])
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    results.put((q, reps, el))


def cpu_baseline(spec: W.Spec, seed: int, budget_s: float = 10.0) -> dict:
    """The oracle, untuned, on a bounded sample of the workload: the
    cached-pool step (each query's request compressed beforehand, untimed),
    one query per host core of this process's affinity set, every core
    running its query's step repeatedly for budget_s seconds (queries/s = all
    steps done / the longest worker's time), then one query on one thread.

    Runs before anything touches the GPU: the workers are forked from this
    process and read its input arrays in place."""
    import multiprocessing as mp

    import oracle as O
    from threadpoolctl import threadpool_limits
    cores = sorted(os.sched_getaffinity(0))
    n = max(1, min(len(cores), spec.Q, 16))        # at most 16: the host share of one GPU
    xn = W.make_inputs(spec, seed=seed).numpy()   # the first timed input set, on the host
    ctx = mp.get_context("fork")
    start, results = ctx.Barrier(n + 1), ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker,
                         args=(xn, spec, q, cores[q % len(cores)], budget_s, start, results))
             for q in range(n)]
    for p in procs:
        p.start()
    start.wait()
    got = [results.get(timeout=budget_s * 10 + 300) for _ in procs]
    for p in procs:
        p.join()
    steps = sum(g[1] for g in got)
    el = max(g[2] for g in got)
    out = {"value": round(steps / el, 3), "unit": "queries/s", "cores": n, "kind": "oracle",
           "sample": f"{spec.name} (input set of seed {seed}): cached-pool step, queries "
                     f"0..{n - 1} one per host core (each core one process, one BLAS thread), "
                     f"{steps} query steps in {el:.1f} s; host cores in the affinity set: "
                     f"{len(cores)}"}
    # one query on one thread
    r = int(xn["q_req"][0])
    with threadpool_limits(limits=1):
        prev = O.kpool_compress(xn["k"], xn["gate"], xn["ape"], xn["valid"], xn["tok_off"],
                                xn["pool_off"], xn["ln_w"], xn["ln_b"], spec.eps, spec.kpool,
                                requests=[r])
        reps, t0 = 0, time.perf_counter()
        while True:
            O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                       spec.sm_scale, new_from=xn["new_from"], prev=prev, queries=[0])
            reps += 1
            el1 = time.perf_counter() - t0
            if el1 >= budget_s / 2:
                break
    out["single_thread"] = {"value": round(reps / el1, 3), "unit": "queries/s", "cores": 1,
                            "sample": f"query 0, {reps} steps in {el1:.1f} s"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode32k", choices=W.WORKLOADS)
    ap.add_argument("--sets", type=int, default=8)
    ap.add_argument("--stage-reps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--page-rows", type=int, default=64,
                    help="also time the step over a paged copy of the latent cache (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    a = ap.parse_args()
    if a.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    spec = W.spec_by_name(a.workload)
    # the CPU baseline first: its workers are forked, so nothing may have
    # touched the GPU yet (counting devices does not)
    cpu = None
    if not a.no_cpu_baseline and torch.cuda.device_count() > 0:
        cpu = cpu_baseline(spec, seed=1000)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    dsa.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)

    # -- resident input sets and their output buffers ---------------------------
    sets, steps = [], []
    for i in range(a.sets):
        x = W.make_inputs(spec, seed=1000 + i, device=dev)
        st = DsaStep(x)
        st.run(incremental=False)       # cache every pool once (set-up, untimed)
        sets.append(x)
        steps.append(st)
    torch.cuda.synchronize()
    print(f"[bench] {a.sets} input sets of {spec.name} resident", file=sys.stderr, flush=True)

    def capture(fn):
        graphs = []
        for st in steps:
            fn(st)                      # warm the path once before capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(st)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    def capture_seq(fn):
        """One graph over every set's step, in set order."""
        for st in steps:
            fn(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for st in steps:
                fn(st)
        torch.cuda.synchronize()
        return g

    def timed_seq(gseq, singles, n, warm, segments=5):
        """n steps: n // len(singles) replays of the sequence graph, then the
        remainder as single-step graphs.  Events also split the replays into
        `segments` runs of equal replay count; returns the total time, the
        wall time and the median per-step time of the segments (us)."""
        k = len(singles)
        for _ in range(max(1, warm // k)):
            gseq.replay()
        torch.cuda.synchronize()
        reps = n // k
        nseg = max(1, min(segments, reps))
        bounds = [reps * i // nseg for i in range(nseg + 1)]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(reps):
            gseq.replay()
            if i + 1 in bounds[1:]:
                ev[bounds.index(i + 1)].record()
        for i in range(n % k):
            singles[i].replay()
        e1.record()
        torch.cuda.synchronize()
        seg = sorted(ev[j].elapsed_time(ev[j + 1]) / ((bounds[j + 1] - bounds[j]) * k) * 1e3
                     for j in range(nseg) if bounds[j + 1] > bounds[j])
        med = seg[len(seg) // 2] if seg else None
        return ev[0].elapsed_time(e1), time.perf_counter() - t0, med

    def timed(graphs, n, warm, segments=1):
        """n steps, one graph replay each (graphs in rotation); events split
        them into `segments` runs of equal length.  Returns the total time
        (ms), the wall time and the median per-step time of the segments (us)."""
        for i in range(warm):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        nseg = max(1, min(segments, n))
        bounds = [n * i // nseg for i in range(nseg + 1)]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(n):
            graphs[i % len(graphs)].replay()
            if i + 1 in bounds[1:]:
                ev[bounds.index(i + 1)].record()
        torch.cuda.synchronize()
        seg = sorted(ev[j].elapsed_time(ev[j + 1]) / (bounds[j + 1] - bounds[j]) * 1e3
                     for j in range(nseg) if bounds[j + 1] > bounds[j])
        return ev[0].elapsed_time(ev[-1]), time.perf_counter() - t0, seg[len(seg) // 2]

    def timed_native(argsets, n, warm, segments=5):
        """n steps, one dsa_decode_step call each (the sets in rotation) on the
        current stream; events split them into `segments` runs of equal
        length.  Returns the total time (ms), the wall time and the median
        per-step time of the segments (us)."""
        cur = torch.cuda.current_stream()
        k = len(argsets)
        for i in range(warm):
            dsa.dsa_decode_step(argsets[i % k], stream=cur)
        torch.cuda.synchronize()
        nseg = max(1, min(segments, n))
        bounds = [n * i // nseg for i in range(nseg + 1)]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(n):
            dsa.dsa_decode_step(argsets[i % k], stream=cur)
            if i + 1 in bounds[1:]:
                ev[bounds.index(i + 1)].record()
        torch.cuda.synchronize()
        seg = sorted(ev[j].elapsed_time(ev[j + 1]) / (bounds[j + 1] - bounds[j]) * 1e3
                     for j in range(nseg) if bounds[j + 1] > bounds[j])
        return ev[0].elapsed_time(ev[-1]), time.perf_counter() - t0, seg[len(seg) // 2]

    # the step: the fused decode calls over cached pools, one dsa_decode_step
    # call per step (the timed figure); beside it, the same steps as one graph
    # replay per step and as graphs of eight consecutive steps
    argsets = [st.step_args(incremental=True) for st in steps]
    ms, wall, seg_med_us = timed_native(argsets, a.steps, a.warmup)
    ms_per_step = ms / a.steps
    qps = spec.Q * a.steps / (ms / 1e3)
    graphs = capture(lambda st: st.run_fused(incremental=True))
    gseq = capture_seq(lambda st: st.run_fused(incremental=True))
    msg, _, seg_med_g_us = timed(graphs, a.steps, a.warmup, segments=5)
    ms8, _, seg_med8_us = timed_seq(gseq, graphs, a.steps, a.warmup)
    # the same step graphs with two (four) batches in flight: set i replays on
    # side stream i mod 2 (4), default priority, bracketed by events on the
    # launch stream; each set always replays on the same stream
    def in_flight(nstreams):
        side = [torch.cuda.Stream() for _ in range(nstreams)]
        cur = torch.cuda.current_stream()
        n2 = max(nstreams, a.steps // nstreams * nstreams)
        for rep2 in range(2):  # (the first pass warms the streams)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            for sd in side:
                sd.wait_event(e0)
            for i in range(n2):
                with torch.cuda.stream(side[i % nstreams]):
                    graphs[i % len(graphs)].replay()
            for sd in side:
                ev = torch.cuda.Event()
                ev.record(sd)
                cur.wait_event(ev)
            e1.record(cur)
            torch.cuda.synchronize()
        ms2 = e0.elapsed_time(e1)
        return {"streams": nstreams, "value": round(spec.Q * n2 / (ms2 / 1e3), 1),
                "unit": "queries/s", "us_per_step": round(ms2 / n2 * 1e3, 2)}
    # (only when the sets divide evenly, so no set is in flight on two streams)
    concurrent = in_flight(2) if len(graphs) % 2 == 0 else None
    concurrent4 = in_flight(4) if len(graphs) % 4 == 0 else None
    # the same step through the six separate calls, for comparison
    graphs6 = capture(lambda st: st.run(incremental=True))
    ms6, _, _ = timed(graphs6, max(1, a.steps // 4), max(1, a.warmup // 4))
    six_us = ms6 / max(1, a.steps // 4) * 1e3
    del graphs6
    # the same step with the attention over a paged copy of the latent cache
    paged = None
    if a.page_rows > 0:
        for i, st in enumerate(steps):
            st.pc = W.make_paged_cache(sets[i], a.page_rows, seed=i)
        graphs_p = capture(lambda st: st.run_fused(incremental=True, paged=st.pc))
        ms_p, _, _ = timed(graphs_p, max(1, a.steps // 4), max(1, a.warmup // 4))
        paged = {"page_rows": a.page_rows,
                 "table_cols": int(steps[0].pc.block_table.shape[1]),
                 "step_us": round(ms_p / max(1, a.steps // 4) * 1e3, 2)}
        del graphs_p
    # the whole decode step from device-side live lengths: geometry, the store
    # of the step's indexer row, the fused step, the attention (paged when
    # timed above)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    for st in steps:
        st.seq_len = torch.tensor(spec.live_lengths(), dtype=torch.int32, device=dev)
        st.k_new = torch.randn(spec.B, spec.index_dim, generator=gen, device=dev) \
            .to(torch.bfloat16).view(torch.int16)
        st.gate_new = torch.randn(spec.B, spec.index_dim, generator=gen, device=dev) \
            .to(torch.bfloat16).view(torch.int16)
        st.slot = torch.empty(spec.B, dtype=torch.int32, device=dev)
    graphs_l = capture(lambda st: st.run_live(st.k_new, st.gate_new, paged=getattr(st, "pc", None),
                                              slot=st.slot if paged is not None else None))
    ms_l, _, _ = timed(graphs_l, max(1, a.steps // 4), max(1, a.warmup // 4))
    del graphs_l
    graphs_l = capture(lambda st: st.run_live(st.k_new, st.gate_new, paged=getattr(st, "pc", None),
                                              fused=True))
    ms_lf, _, _ = timed(graphs_l, max(1, a.steps // 4), max(1, a.warmup // 4))
    del graphs_l
    live = {"step_us": round(ms_l / max(1, a.steps // 4) * 1e3, 2),
            "fused_step_us": round(ms_lf / max(1, a.steps // 4) * 1e3, 2)}

    # -- per-call launch times: a graph of kCallsPerGraph back-to-back calls of
    # one kind (the input sets in rotation), replayed between HIP events on the
    # launch stream; the time per call is what the step's own graph sees, with
    # the host's graph-launch cost spread over many calls
    stream = torch.cuda.current_stream()
    kCallsPerGraph = 32

    def call_graph(fn):
        for st in steps:
            fn(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(kCallsPerGraph):
                fn(steps[i % len(steps)])
        torch.cuda.synchronize()
        return g

    fns = {
        "gate_compress": lambda s: s.gate_compress(incremental=True),
        "index_scores_gated": lambda s: s.index_scores_gated(),
        "topk_expand": lambda s: s.topk_expand(),
        "head_gate": lambda s: s.head_gate(),
        "kpool_compress": lambda s: s.compress(incremental=True),
        "index_scores": lambda s: s.index_scores(),
        "topk_pools": lambda s: s.topk(),
        "expand_selection": lambda s: s.expand(),
        "sparse_mla_decode": lambda s: s.mla(),
    }
    if paged is not None:
        fns["sparse_mla_decode_paged"] = lambda s: s.mla_paged(s.pc)
    fns["write_geom"] = lambda s: s.write_geom(getattr(s, "pc", None),
                                               s.slot if paged is not None else None)
    fns["indexer_store"] = lambda s: s.store(s.k_new, s.gate_new)
    fns["gate_compress_live"] = lambda s: s.gate_compress_live(s.k_new, s.gate_new)
    call_us = {}
    reps = max(1, a.stage_reps // kCallsPerGraph)
    for name, fn in fns.items():
        g = call_graph(fn)
        ms_c, _, _ = timed([g], reps, 1)
        call_us[name] = ms_c / (reps * kCallsPerGraph) * 1e3
        del g
    stage_us = {k: call_us[k] for k in STAGES}
    if paged is not None:
        paged["mla_us"] = round(call_us["sparse_mla_decode_paged"], 2)
    live["write_geom_us"] = round(call_us["write_geom"], 2)
    live["indexer_store_us"] = round(call_us["indexer_store"], 2)
    live["gate_compress_live_us"] = round(call_us["gate_compress_live"], 2)

    # the lane: a plain coalesced 16-byte-per-lane read of 1 GiB on this part
    lane_bytes = 1 << 30
    lane_buf = torch.empty(lane_bytes, dtype=torch.uint8, device=dev)
    lane_buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        dsa.dsa_lane_read(lane_buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dsa.dsa_lane_read(lane_buf, sink)
    e1.record()
    torch.cuda.synchronize()
    lane_gbs = lane_bytes / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del lane_buf

    xn0 = {"q_req": sets[0].q_req.cpu().numpy()}
    nb = algorithmic_bytes(spec, xn0, steps[0].n_pools.cpu().numpy(), steps[0].tok.cpu().numpy())
    step_bytes = sum(nb[k] for k in STAGES)
    dom = max(STAGES, key=lambda n: stage_us[n])
    ach = nb[dom] / (stage_us[dom] * 1e-6) / 1e9
    ctr = stored_counters(dom, spec.name)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": None if ctr is None else int(ctr["hbm_bytes"]),
                "algorithmic_bytes": int(nb[dom]), "avg_launch_us": round(stage_us[dom], 2),
                "lane_GBps": round(lane_gbs, 1), "frac_of_lane": round(ach / lane_gbs, 4)}
    if dom == "sparse_mla_decode":
        # the attention's dense MFMA work over the selected rows (QK and PV)
        n_tok = int((steps[0].tok >= 0).sum().item())
        fl = 4.0 * spec.latent * spec.mla_heads * n_tok
        roofline["mfma"] = {"flops": int(fl), "achieved_TFLOPs": round(fl / (stage_us[dom] * 1e-6) / 1e12, 1),
                            "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                            "frac": round(fl / (stage_us[dom] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if ctr is not None:
        roofline["counters"] = {"kernel": ctr["kernel"], "MfmaUtil_pct": ctr["mfma_util_pct"],
                                "VALUBusy_pct": ctr["valu_busy_pct"],
                                "source": f"profiles/counters_{spec.name}.json"}

    line = {
        "metric": "DSA decode queries/s (gate+indexer+top-k+sparse MLA) and % of HBM peak",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "precision": "bf16 MFMA operands with f32 accumulation; f32 head-gate and pooling",
        "data": "synthetic, seeded",
        "config": {"workload": spec.name, "requests": spec.B, "queries": spec.Q,
                   "context_rows": spec.lengths[0] if len(set(spec.lengths)) == 1 else "ragged",
                   "kpool": spec.kpool, "select_k": spec.select_k, "out_width": spec.out_width,
                   "index_heads": spec.index_heads, "index_dim": spec.index_dim,
                   "mla_heads": spec.mla_heads, "latent": spec.latent,
                   "latent_dtype": "fp8_e4m3" if spec.latent_fp8 else "bf16",
                   "pools": "cached; the step recompresses the pool of its newest row",
                   "input_sets": a.sets,
                   "launch": "one dsa_decode_step call per step (the input sets in "
                             "rotation): the fused decode calls (gate+compress, gated index "
                             "scores, top-k+expand, sparse MLA) enqueued on the stream by "
                             "the library's step executor"},
        "median_of_5_segments_us": round(seg_med_us, 2),
        "single_step_graph": {"us_per_step": round(msg / a.steps * 1e3, 2),
                              "value": round(spec.Q * a.steps / (msg / 1e3), 1),
                              "unit": "queries/s",
                              "median_of_5_segments_us": round(seg_med_g_us, 2),
                              "graph": "each input set's step captured in a HIP graph of its "
                                       "own, one replay per step"},
        "eight_step_graph": {"us_per_step": round(ms8 / a.steps * 1e3, 2),
                             "value": round(spec.Q * a.steps / (ms8 / 1e3), 1),
                             "unit": "queries/s",
                             "median_of_5_segments_us": None if seg_med8_us is None
                             else round(seg_med8_us, 2),
                             "graph": "the eight input sets' steps captured in sequence "
                                      "in one graph"},
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": int(step_bytes),
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
        "stage_bytes": {k: int(nb[k]) for k in STAGES},
        "six_call_step_us": round(six_us, 2),
        "call_us": {k: round(call_us[k], 2) for k in CALLS},
        "two_batches_in_flight": concurrent,
        "four_batches_in_flight": concurrent4,
        "paged": paged,
        "live_step": live,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
