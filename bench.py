#!/usr/bin/env python3
"""Benchmark: GDN tree verify + persist per layer call on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config batched]

A step is one pass of the whole hot path over one batch of synthetic input:
gdn_tree_plan, then gdn_tree_verify and gdn_tree_persist for every layer of
the workload ("batched": 32 sequences x one layer; "stress": 64 sequences x 48
layers).  Inputs and states are resident in HBM before timing starts.  To keep
the 256 MB Infinity Cache from serving repeated reads, the timed loop rotates
through R independent copies of the states and inputs (each layer of the
workload is its own copy), so consecutive steps never touch the same bytes.
A one-layer workload (R >= 4) persists on the copy half a rotation away from
the one verify read: in a model, the other layers' verify calls separate a
layer's verify from its persist.

The timed loop replays the steps as a HIP graph holding one rotation cycle of
consecutive steps (the same library calls, captured once; `--eager` times host
launches instead).  Per-call durations come from one graph per call kind
(that call alone over the rotation, replayed between two events on the
kernels' stream); a separate eager pass with an event pair around every call
gives the eager breakdown, which adds the host's launch gaps.

`--schedule fused` times the deferred-persist schedule instead: a step is the
plan and, per layer, one gdn_tree_persist_verify (the previous step's persist
fused with this step's verify); two workspaces alternate between steps.

Prints ONE JSON line.  `value` = tree nodes verified per second per layer call
(plan + verify + persist); `roofline` describes the dominant kernel, timed with
HIP events on the stream it runs on; `cpu_baseline` times the fp64 CPU oracle
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="batched")
    ap.add_argument("--rotate", type=int, default=0, help="independent copies (default: >= 512 MB in flight)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-accept", action="store_true", help="skip the greedy-acceptance measurement")
    ap.add_argument("--accept-steps", type=int, default=50)
    ap.add_argument("--no-draft", action="store_true", help="skip the draft top-k / tree-builder measurement")
    ap.add_argument("--no-snapshot", action="store_true", help="skip the prefix-cache snapshot measurement")
    ap.add_argument("--no-store-path", action="store_true",
                    help="skip the per-node fp16 state path (verify-and-store + persist-by-copy) comparison")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--path", choices=["auto", "recurrent"], default="auto",
                    help="recurrent: run the per-node recurrent kernels on every call (GDN_KERNEL_PATH)")
    ap.add_argument("--distinct", type=int, default=0,
                    help="generate this many layers' inputs and place each in several copies (0: every copy)")
    ap.add_argument("--no-stress", action="store_true", help="skip the stress-workload sub-object")
    ap.add_argument("--stress-steps", type=int, default=10)
    ap.add_argument("--stress-warmup", type=int, default=3)
    ap.add_argument("--seqs", type=int, default=0,
                    help="run the workload with this many sequences (its own slots) instead of its own count")
    ap.add_argument("--stress-distinct", type=int, default=4,
                    help="independently generated layers of the stress sub-object (the rest are copies)")
    ap.add_argument("--sweep", default="64,128,256",
                    help="sequence counts of the batch sweep sub-object (the same tree recipe; empty: none)")
    ap.add_argument("--sweep-steps", type=int, default=20)
    ap.add_argument("--schedule", choices=["separate", "fused"], default="separate",
                    help="fused: a step is the plan and one gdn_tree_persist_verify per layer (the previous "
                         "step's persist with this step's verify), for workloads the fused kernel takes")
    return ap.parse_args()


def algorithmic_bytes(cfg, T, path_lens, s_in):
    """Bytes the method must move per layer call: verify reads every sequence's
    committed state once, the node inputs (q, k, v at s_in bytes, gates at 4) and the
    tree indices, and writes one output row per (node, value head); persist reads and
    writes each state once and reads the inputs of the accepted path's nodes (no q)."""
    B, Hk, Hv, D = cfg.num_seqs, cfg.num_k_heads, cfg.num_v_heads, cfg.head_dim
    state = B * Hv * D * D * 4
    verify = state + T * (2 * Hk * D + Hv * D) * s_in + T * Hv * 8 + T * Hv * D * 4 + 4 * (T + 2 * B + 1)
    P = int(np.sum(path_lens))
    persist = 2 * state + P * (Hk * D + Hv * D) * s_in + P * Hv * 8 + 4 * B
    return verify, persist


def rotation(per_copy, layers):
    """Independent copies the timed loop rotates through: enough that >= 512 MB separate
    two reads of the same bytes (the Infinity Cache holds 256 MB), at least 4 for a
    one-layer workload, and at most 128: below ~4 MB per copy (the batch-1 and tiny
    workloads) the data is cache-sized whatever the rotation, and a graph of tens of
    thousands of steps is more than the runtime should be asked to capture."""
    return min(128, max(4 if layers == 1 else 1, int(np.ceil(512e6 / (per_copy * layers)))))


def pct(xs):
    """median, p10 and p90 of a list of timings"""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(a.mean()), "samples": int(a.size)}


def cpu_model_name():
    """The host CPU's model name (the `lscpu` "Model name" line, read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def memory_ceilings(G, dev):
    """Plain streaming rates of this part, the practical ceilings beside the 8 TB/s
    peak: the library's diagnostic pass reading 1 GiB, and copying 1 GiB into another
    buffer (read + write).  Each sample times 4 back-to-back launches queued behind a
    fifth, so the events see the device busy throughout and no host launch gap; the
    rate is the median over 10 samples."""
    import torch
    x = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    partial = torch.empty((x.numel() * 4 + 65535) // 65536 * 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn, nbytes in (("read", lambda: G.gdn_probe_stream("read", x, partial), x.numel() * 4),
                             ("copy", lambda: G.gdn_probe_stream("copy", x, y), 2 * x.numel() * 4)):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fn()
            e0.record(stream)
            for _ in range(4):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / 4)
        res[name + "_gbs"] = nbytes / float(np.median(ts)) / 1e9
    del x, y, partial
    torch.cuda.synchronize()
    res["how"] = ("gdn_probe_stream reading 1 GiB (read) and copying 1 GiB (read + write bytes); "
                  "4 launches queued behind a fifth per sample, median of 10 samples")
    return res


def fused_supported(cfg):
    """The workloads gdn_tree_persist_verify runs as one kernel (other shapes run the two calls)."""
    return cfg.dtype == "bf16" and cfg.head_dim in (64, 128) and cfg.max_nodes <= 32


def measure(G, W, cfg, args, steps, warmup, distinct=0, path_label="auto", schedule="separate"):
    """Times one workload: a step = plan + verify and persist for each layer, or with
    schedule "fused" the plan + one fused persist + verify call per layer (each layer's
    persist deferred to its next verify; two workspaces alternate between steps).
    Returns the workload's result fields and the state the extra measurements use."""
    import torch
    dev = torch.device("cuda:0")
    trees = W.make_trees(cfg)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    slots = W.make_slots(cfg)
    acc = W.make_accepts(cfg, trees)
    s_in = 2 if cfg.dtype == "bf16" else 4
    qkv_dtype = G.GDN_BF16 if cfg.dtype == "bf16" else G.GDN_F32
    dims = G.make_dims(cfg.num_seqs, T, cfg.max_nodes, cfg.num_k_heads, cfg.num_v_heads, cfg.head_dim,
                       cfg.num_slots, qkv_dtype, max_depth=cfg.max_depth)
    path_lens = [int(W.tree_depths(t)[m]) for t, m in zip(trees, acc)]
    vbytes, pbytes = algorithmic_bytes(cfg, T, path_lens, s_in)

    def to_dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    layers = cfg.num_layers
    per_copy = vbytes + T * cfg.num_v_heads * cfg.head_dim * 4
    rotate = args.rotate or rotation(per_copy, layers)
    copies = layers * rotate
    # distinct > 0: that many independently generated layers' inputs and prefills,
    # each placed in several copies (every copy is its own HBM buffer; only the
    # values repeat, which the kernels' timing does not depend on)
    n_gen = copies if distinct <= 0 else min(distinct, copies)
    print("# config %s: B=%d T=%d layers=%d copies=%d (%d generated, %.0f MB per layer copy)"
          % (cfg.name, cfg.num_seqs, T, layers, copies, n_gen, per_copy / 1e6), file=sys.stderr, flush=True)

    slot_d = to_dev(slots)
    acc_d = to_dev(acc)
    parent_d = to_dev(np.concatenate(trees).astype(np.int32))
    cu_d = to_dev(cu.astype(np.int32))
    ws = G.new_workspace(dims)
    wss = [ws, G.new_workspace(dims)] if schedule == "fused" else [ws]
    for w_ in wss[1:]:
        G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, w_)
    # committed states: each generated copy's cache is filled by the library's own
    # chain kernel running that copy's prefill tokens from a zero state
    pre_cu = torch.arange(0, (cfg.num_seqs + 1) * cfg.prefill_steps, cfg.prefill_steps, dtype=torch.int32,
                          device=dev)
    pre_dims = G.make_dims(cfg.num_seqs, cfg.num_seqs * cfg.prefill_steps, cfg.prefill_steps, cfg.num_k_heads,
                           cfg.num_v_heads, cfg.head_dim, cfg.num_slots, qkv_dtype)
    zero_cache = torch.zeros((cfg.num_slots, cfg.num_v_heads, cfg.head_dim, cfg.head_dim), device=dev)
    flen = torch.full((cfg.num_seqs,), cfg.prefill_steps, dtype=torch.int32, device=dev)
    ident = torch.arange(cfg.num_seqs, dtype=torch.int32, device=dev)
    sets = []
    for c in range(copies):
        if c < n_gen:
            inp = W.make_layer_inputs(cfg, c, trees)
            pre = W.make_prefill(cfg, c)
            d = {k: to_dev(v) for k, v in inp.items()}
            pk = to_dev(pre["k"].reshape(-1, cfg.num_k_heads, cfg.head_dim))
            pv = to_dev(pre["v"].reshape(-1, cfg.num_v_heads, cfg.head_dim))
            pa = to_dev(pre["a"].reshape(-1, cfg.num_v_heads))
            pb = to_dev(pre["b"].reshape(-1, cfg.num_v_heads))
            fin = torch.empty((cfg.num_seqs, cfg.num_v_heads, cfg.head_dim, cfg.head_dim), device=dev)
            G.gdn_chain_verify(pre_dims, pre_cu, None, pk, pv, pa, pb, zero_cache, ident, None, flen, fin)
            cache = torch.zeros((cfg.num_slots, cfg.num_v_heads, cfg.head_dim, cfg.head_dim), device=dev)
            cache[slot_d.long()] = fin
            d["cache"] = cache
            del pk, pv, pa, pb, fin
        else:
            d = {k: v.clone() for k, v in sets[c % n_gen].items() if k != "out"}
        d["out"] = torch.empty((T, cfg.num_v_heads, cfg.head_dim), device=dev)
        sets.append(d)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * layers + 2)] for _ in range(steps)]

    def step(i, events=None):
        r = i % rotate
        if schedule == "fused":
            # this step's plan goes to one workspace; the other holds the previous step's
            # plan (the same trees), whose accepted paths the fused calls persist
            wn, wp = wss[i % 2], wss[(i + 1) % 2]
            rp = (r + rotate // 2) % rotate if layers == 1 else r
            if events:
                events[0].record(stream)
            G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, wn)
            if events:
                events[1].record(stream)
            for l in range(layers):
                d, p = sets[r * layers + l], sets[rp * layers + l]
                G.gdn_tree_persist_verify(dims, p["k"], p["v"], p["a"], p["b"], acc_d, wp, dims, d["q"], d["k"],
                                          d["v"], d["a"], d["b"], d["cache"], slot_d, d["out"], wn)
                if events:
                    events[2 + l].record(stream)
            return
        if events:
            events[0].record(stream)
        G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, ws)
        if events:
            events[1].record(stream)
        for l in range(layers):
            d = sets[r * layers + l]
            G.gdn_tree_verify(dims, d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], slot_d, d["out"], ws)
            if events:
                events[2 + l].record(stream)
        # one-layer workloads persist on the copy half a rotation ahead: in a model every other
        # layer's verify runs between a layer's verify and its persist, so its states are no
        # longer cached, and no copy is read again within two steps of being written
        rp = (r + rotate // 2) % rotate if layers == 1 else r
        for l in range(layers):
            d = sets[rp * layers + l]
            G.gdn_tree_persist(dims, d["k"], d["v"], d["a"], d["b"], acc_d, d["cache"], slot_d, ws)
            if events:
                events[2 + layers + l].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    for w_ in wss:
        rc, bad, code = G.gdn_tree_status(w_)
        if rc != 0:
            break
    if rc != 0:
        print(json.dumps({"error": "library rejected the %s workload: %d %d %d" % (cfg.name, rc, bad, code)}))
        sys.exit(1)

    # per-call breakdown: K eager steps with an event pair around every call
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, ev[i])
    torch.cuda.synchronize()
    eager_ms_per_step = (time.perf_counter() - t0) * 1e3 / steps

    # main timed loop: exactly K steps as HIP graph replays (the same calls, without the
    # host's launch gaps).  One graph holds one rotation cycle of consecutive steps
    # (copies 0 .. R-1): each graph launch costs the GPU several microseconds, which a
    # decode loop pays per launch, not per step.  Each cycle's replay sits between two
    # events, which give the per-step spread.
    cycle = None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for r in range(rotate):
                step(r)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        cycle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cycle):
            for r in range(rotate):
                step(r)
        cycle.replay()
    torch.cuda.synchronize()
    full, rest = divmod(steps, rotate) if cycle is not None else (0, steps)
    cyc_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(full)]
    t0 = time.perf_counter()
    for e0, e1 in cyc_ev:
        e0.record(stream)
        cycle.replay()
        e1.record(stream)
    for i in range(rest):  # a partial cycle (or every step with --eager) runs eagerly
        step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    if cyc_ev:
        step_samples = [a.elapsed_time(b) / rotate for a, b in cyc_ev]
        step_how = "one sample per graph replay of %d consecutive steps (events on the kernels' stream)" % rotate
    else:
        step_samples = [e[0].elapsed_time(e[-1]) for e in ev]
        step_how = "eager steps, first to last event"

    # per-kernel launch durations under graph replay, the launch mode of the timed loop:
    # one graph per call kind holding that call alone over the rotation, each replay
    # between two events on the stream the kernels run on (events cannot sit inside a
    # graph here).  Each graph holds enough launches that the graph launch's own
    # start-up (several microseconds) adds little per launch.
    def graph_us(call, per_cycle):
        cycles = max(1, 32 // per_cycle)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for r in range(rotate):
                call(r)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(cycles):
                for r in range(rotate):
                    call(r)
        g.replay()
        torch.cuda.synchronize()
        reps = max(5, 400 // (cycles * per_cycle))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        per_launch = [a.elapsed_time(b) * 1e3 / (cycles * per_cycle) for a, b in evs]
        del g
        return pct(per_launch)

    def plan_call(r):
        G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, ws)

    def verify_call(r):
        for l in range(layers):
            d = sets[r * layers + l]
            G.gdn_tree_verify(dims, d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], slot_d, d["out"], ws)

    def persist_call(r):
        for l in range(layers):
            d = sets[r * layers + l]
            G.gdn_tree_persist(dims, d["k"], d["v"], d["a"], d["b"], acc_d, d["cache"], slot_d, ws)

    gp = graph_us(plan_call, rotate)
    gv = graph_us(verify_call, rotate * layers)
    gs = graph_us(persist_call, rotate * layers)
    g_plan, g_ver, g_per = gp["mean"] * 1e-6, gv["mean"] * 1e-6, gs["mean"] * 1e-6

    # the fused layer call of a decode loop that defers each layer's persist to its next
    # verify: gdn_tree_persist_verify replays the previous step's accepted path into the
    # cache and verifies this step's trees from the same registers (one state read and one
    # write instead of two reads and a write).  The previous step's inputs come from the
    # copy half a rotation away, as persist's do above; both steps use the workload's trees.
    fused = None
    if fused_supported(cfg) and path_label == "auto":
        ws_prev = G.new_workspace(dims)
        G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, ws_prev)
        G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, ws)

        def fused_call(r):
            rp = (r + rotate // 2) % rotate if layers == 1 else r
            for l in range(layers):
                d, p = sets[r * layers + l], sets[rp * layers + l]
                G.gdn_tree_persist_verify(dims, p["k"], p["v"], p["a"], p["b"], acc_d, ws_prev, dims, d["q"], d["k"],
                                          d["v"], d["a"], d["b"], d["cache"], slot_d, d["out"], ws)

        gf = graph_us(fused_call, rotate * layers)
        rc, bad, code = G.gdn_tree_status(ws_prev)
        if rc != 0:
            print(json.dumps({"error": "fused call rejected the %s workload: %d %d %d" % (cfg.name, rc, bad, code)}))
            sys.exit(1)
        g_fu = gf["mean"] * 1e-6
        state_bytes = cfg.num_seqs * cfg.num_v_heads * cfg.head_dim * cfg.head_dim * 4
        fbytes = vbytes + pbytes - state_bytes  # one state read fewer than verify + persist
        fused = {"us": g_fu * 1e6, "us_pct": gf, "bytes": fbytes, "hbm_gbs": fbytes / g_fu / 1e9,
                 "hbm_frac": fbytes / g_fu / 1e9 / HBM_PEAK_GBS, "traffic": measured_traffic("fused", cfg.name),
                 "nodes_per_s": T / g_fu,
                 # a decode step of this schedule: the plan, then the fused call for each layer
                 "step_nodes_per_s": T * layers / (g_plan + layers * g_fu),
                 "vs_verify_plus_persist": (g_ver + g_per) / g_fu,
                 "bytes_note": "verify + persist bytes less one read of the touched state slices",
                 "timing": "graph replay of the fused call alone over the rotation (mean; spread in us_pct)"}
        del ws_prev
    G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, ws)
    torch.cuda.synchronize()

    plan_ms, ver_ms, per_ms, fu_ms = [], [], [], []
    for e in ev:
        plan_ms.append(e[0].elapsed_time(e[1]))
        prev = e[1]
        if schedule == "fused":
            for l in range(layers):
                fu_ms.append(prev.elapsed_time(e[2 + l]))
                prev = e[2 + l]
            continue
        for l in range(layers):
            ver_ms.append(prev.elapsed_time(e[2 + l]))
            prev = e[2 + l]
        for l in range(layers):
            per_ms.append(prev.elapsed_time(e[2 + layers + l]))
            prev = e[2 + layers + l]
    t_plan = float(np.mean(plan_ms)) * 1e-3
    # eager per-call figures of the calls the timed steps make
    t_ver = float(np.mean(ver_ms)) * 1e-3 if ver_ms else None
    t_per = float(np.mean(per_ms)) * 1e-3 if per_ms else None
    nodes_per_s = T * layers / (ms_per_step * 1e-3)
    hbm_gbs = (vbytes + pbytes) / (g_ver + g_per) / 1e9

    # dominant kernel of the layer call: both stream the state cache and run far below the
    # ridge point of the matrix cores, so the bound is HBM bandwidth.  Its launch duration
    # is the graph-replay mean (the timed loop's launch mode); the eager figure, which adds
    # the host launch gap, is reported beside it.
    if schedule == "fused":  # one kernel per layer call
        dom, t_dom, t_dom_eager, dom_bytes, dom_pct = ("fused", fused["us"] * 1e-6, float(np.mean(fu_ms)) * 1e-3,
                                                       fused["bytes"], fused["us_pct"])
    elif g_ver >= g_per:
        dom, t_dom, t_dom_eager, dom_bytes, dom_pct = "tree_verify", g_ver, t_ver, vbytes, gv
    else:
        dom, t_dom, t_dom_eager, dom_bytes, dom_pct = "persist", g_per, t_per, pbytes, gs
    roof = {"bound": "hbm", "achieved": dom_bytes / t_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, cfg.name)
    roof["kernel"] = dom
    roof["bytes_per_launch"] = dom_bytes
    roof["launch_us"] = t_dom * 1e6
    roof["launch_us_pct"] = dom_pct
    roof["launch_us_eager"] = t_dom_eager * 1e6

    res = {
        "value": nodes_per_s,
        "ms_per_step": ms_per_step,
        "step_ms": dict(pct(step_samples), how=step_how),
        "eager_ms_per_step": eager_ms_per_step,
        "config": {"workload": cfg.name, "sequences": cfg.num_seqs, "layers": layers, "nodes": T,
                   "v_heads": cfg.num_v_heads, "k_heads": cfg.num_k_heads, "head_dim": cfg.head_dim,
                   "qkv": cfg.dtype, "rotated_copies": rotate, "generated_copies": n_gen, "seed": cfg.seed,
                   "kernels": path_label, "schedule": schedule,
                   "launch": "eager" if args.eager else "hip_graph_per_%d_steps" % rotate},
        "layer_call": {"verify_us": g_ver * 1e6, "persist_us": g_per * 1e6, "plan_us": g_plan * 1e6,
                       "verify_us_pct": gv, "persist_us_pct": gs, "plan_us_pct": gp,
                       # one plan per decode step serves every GDN layer; 48 layers as in the
                       # 64-sequence stress workload
                       "plan_amortized_us": g_plan * 1e6 / 48, "plan_amortized_over_layers": 48,
                       "verify_bytes": vbytes, "persist_bytes": pbytes, "hbm_gbs": hbm_gbs,
                       "hbm_frac": hbm_gbs / HBM_PEAK_GBS,
                       "verify_gbs": vbytes / g_ver / 1e9, "persist_gbs": pbytes / g_per / 1e9,
                       "nodes_per_s": T / (g_ver + g_per),
                       "timing": "graph replay of each call alone over the rotation (mean; spread in *_pct)",
                       "eager": ({"verify_us": t_ver * 1e6, "persist_us": t_per * 1e6, "plan_us": t_plan * 1e6}
                                 if schedule == "separate" else
                                 {"fused_us": float(np.mean(fu_ms)) * 1e3, "plan_us": t_plan * 1e6})},
        "roofline": roof,
    }
    if fused is not None:
        res["fused_layer_call"] = fused
    ctx = dict(trees=trees, cu=cu, acc=acc, dims=dims, parent_d=parent_d, cu_d=cu_d, slot_d=slot_d, acc_d=acc_d,
               ws=ws, sets=sets, rotate=rotate, layers=layers, vbytes=vbytes, pbytes=pbytes, t_ver=t_ver,
               t_per=t_per)
    return res, ctx


PRECISION = ("bf16 q/k/v; fp32 gates, state and outputs.  The dense products (S0 K^T, S0 Q^T, the output "
             "operator and the persist update) run on bf16 MFMA with each fp32 operand split into bf16 hi + lo "
             "(about 16 significant bits per product) and fp32 accumulation; the per-path recurrences run in "
             "fp32 on the vector ALU")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; --gpus %d is not supported "
                                   "(sequences shard across GPUs with no exchange, so one GPU's "
                                   "share at its real shape is the measured unit)" % args.gpus}))
        sys.exit(2)
    if args.path == "recurrent":
        os.environ["GDN_KERNEL_PATH"] = "recurrent"
    import torch
    import gated_deltanet_tree_amd as G
    import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    G.load_library()
    cfg = W.get_config(args.config)
    if args.seqs > 0:  # the same tree recipe at another batch size
        import dataclasses
        cfg = dataclasses.replace(cfg, num_seqs=args.seqs, num_slots=args.seqs)
    if args.schedule == "fused" and (not fused_supported(cfg) or args.path != "auto"):
        print(json.dumps({"error": "--schedule fused needs bf16 inputs, head dim 64 or 128, trees of at most 32 "
                                   "nodes and the default kernels; workload %s does not qualify" % cfg.name}))
        sys.exit(2)
    res, ctx = measure(G, W, cfg, args, args.steps, args.warmup, distinct=args.distinct, path_label=args.path,
                       schedule=args.schedule)
    # calibration for memory-traffic counters: one plain device copy of a known size
    # (256 MiB read + 256 MiB written), outside the timed region
    cal_src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst
    torch.cuda.synchronize()

    result = {
        "metric": "GDN tree-verify nodes/sec per layer call + achieved HBM GB/s (% of peak)",
        "value": res["value"],
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "split-bf16 MFMA (fp32 state as bf16 hi + lo), fp32 accumulate" if cfg.dtype == "bf16"
                 and args.path == "auto" else "f32",
        "precision": PRECISION,
        "data": "synthetic",
    }
    result.update({k: v for k, v in res.items() if k not in ("value", "ms_per_step")})
    result["memory_ceilings"] = memory_ceilings(G, "cuda")
    if not args.no_accept:
        result["accept"] = bench_accept(G, W, cfg, ctx["trees"], ctx["dims"], ctx["parent_d"], ctx["cu_d"],
                                        ctx["slot_d"], args.accept_steps)
    if not args.no_draft and cfg.tree[0] == "ddtree":
        result["draft"] = bench_draft(G, W, cfg, args.accept_steps)
    if not args.no_store_path and ctx["layers"] == 1 and ctx["t_ver"] is not None:  # beside the two-call steps
        result["store_path"] = bench_store_path(G, cfg, ctx["dims"], ctx["sets"], ctx["slot_d"], ctx["acc_d"],
                                                ctx["ws"], ctx["rotate"], args.accept_steps, ctx["vbytes"],
                                                ctx["pbytes"], ctx["t_ver"], ctx["t_per"])
    if not args.no_snapshot:
        result["snapshot"] = bench_snapshot(G, cfg, ctx["sets"], ctx["slot_d"], ctx["rotate"], ctx["layers"],
                                            args.accept_steps)
    del ctx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # the largest single-GPU workload, as its own sub-object: 64 sequences x 65-node
    # trees x 48 layer calls per step, a few steps
    if not args.no_stress and cfg.name != "stress":
        scfg = W.get_config("stress")
        sres, sctx = measure(G, W, scfg, args, args.stress_steps, args.stress_warmup, distinct=args.stress_distinct,
                             path_label=args.path)
        sres["nodes_per_s"] = sres.pop("value")
        if not args.no_cpu_baseline:
            sres["cpu_baseline"] = cpu_baseline(scfg, sctx["trees"], sctx["cu"], sctx["acc"], args.cpu_seconds / 2,
                                                layer_calls=1, single_thread=False)
        del sctx
        result["stress"] = sres
    # the same tree recipe at larger batches: where the fixed per-workgroup latencies
    # are amortized, the layer call's share of peak bandwidth
    sweep = [int(x) for x in args.sweep.split(",") if x.strip()] if cfg.name == "batched" and args.seqs <= 0 else []
    if sweep:
        import dataclasses
        rows = []
        for nseq in sweep:
            torch.cuda.empty_cache()
            bcfg = dataclasses.replace(cfg, num_seqs=nseq, num_slots=nseq)
            bres, bctx = measure(G, W, bcfg, args, args.sweep_steps, 3, distinct=2, path_label=args.path)
            lc = bres["layer_call"]
            rows.append({"sequences": nseq, "nodes": bres["config"]["nodes"], "verify_us": lc["verify_us"],
                         "persist_us": lc["persist_us"], "verify_frac": lc["verify_gbs"] / HBM_PEAK_GBS,
                         "persist_frac": lc["persist_gbs"] / HBM_PEAK_GBS, "hbm_gbs": lc["hbm_gbs"],
                         "hbm_frac": lc["hbm_frac"], "layer_call_nodes_per_s": lc["nodes_per_s"],
                         "step_nodes_per_s": bres["value"], "rotated_copies": bres["config"]["rotated_copies"]})
            if "fused_layer_call" in bres:
                fl = bres["fused_layer_call"]
                rows[-1]["fused"] = {"us": fl["us"], "hbm_frac": fl["hbm_frac"], "nodes_per_s": fl["nodes_per_s"]}
            del bctx
        result["batch_sweep"] = {"recipe": "the %s workload's trees and heads at other sequence counts" % cfg.name,
                                 "timing": "graph replay of each call alone over the rotation (mean)",
                                 "rows": rows}
    if not args.no_cpu_baseline:
        trees, cu, acc = W.make_trees(cfg), None, None
        cu = W.cu_from_trees(trees)
        acc = W.make_accepts(cfg, trees)
        result["cpu_baseline"] = cpu_baseline(cfg, trees, cu, acc, args.cpu_seconds)
    print(json.dumps(result))


def bench_accept(G, W, cfg, trees, dims, parent_d, cu_d, slot_d, steps):
    """Greedy acceptance over the step's verify logits (one fp32 row of the
    vocabulary per node), timed per call with HIP events on its stream.  Not
    part of the step: it runs once per decode step after the last layer."""
    import torch
    from workloads import draft
    T = dims.total_nodes
    tok = draft.make_draft_tokens(cfg, trees)
    logits = torch.from_numpy(draft.make_verify_logits(cfg, trees, tok)).cuda()
    tok_d = torch.from_numpy(tok).cuda()
    B = cfg.num_seqs
    acc, alen, nxt = (torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(3))
    ws = G.new_workspace(dims)
    G.gdn_tree_plan(dims, parent_d, cu_d, slot_d, ws)
    stream = torch.cuda.current_stream()
    for _ in range(5):
        G.gdn_tree_accept(dims, logits, tok_d, acc, alen, nxt, ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        G.gdn_tree_accept(dims, logits, tok_d, acc, alen, nxt, ws)
        e1.record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    vocab = int(logits.shape[1])
    # algorithmic bytes: every logit once, the draft tokens, the plan's depth and
    # path rows read by the walk, three int32 outputs per sequence
    nbytes = T * vocab * 4 + T * 4 + T * (4 + 4) + B * 12
    gbs = nbytes / t / 1e9
    return {"vocab": vocab, "nodes": T, "call_us": t * 1e6, "bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("accept", cfg.name)},
            "mean_accept_len": float(alen.float().mean().item())}


def bench_draft(G, W, cfg, steps):
    """The drafter side of a decode step: top-W candidates of every drafted
    position over the full vocabulary (gdn_draft_topk), then the trees
    (gdn_ddtree_build), each timed per call with HIP events on its stream.  Not
    part of the step: both run once per decode step before the plan."""
    import torch
    from workloads import draft
    B, L = cfg.num_seqs, draft.DRAFT_LEVELS
    _, budget, width, _ = cfg.tree
    x = torch.from_numpy(draft.make_draft_logits(cfg).reshape(B * L, draft.VOCAB)).cuda()
    roots = torch.from_numpy(draft.make_root_tokens(cfg)).cuda()
    tk = torch.empty((B * L, width), dtype=torch.int32, device="cuda")
    lp = torch.empty((B * L, width), dtype=torch.float32, device="cuda")
    n = G.ddtree_nodes(L, width, budget)
    par = torch.empty(B * n, dtype=torch.int32, device="cuda")
    ntok = torch.empty(B * n, dtype=torch.int32, device="cuda")
    cu = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def topk():
        G.gdn_draft_topk(x, width, tk, lp)

    def build():
        G.gdn_ddtree_build(roots, tk.view(B, L, width), lp.view(B, L, width), budget, par, ntok, cu)

    times = {}
    for name, fn in (("topk", topk), ("build", build)):
        for _ in range(5):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        times[name] = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    # algorithmic bytes of the top-k: every logit once, W (token, log p) pairs per row out
    nbytes = B * L * draft.VOCAB * 4 + B * L * width * 8
    gbs = nbytes / times["topk"] / 1e9
    return {"rows": B * L, "vocab": draft.VOCAB, "width": width, "budget": budget, "tree_nodes": n,
            "topk_us": times["topk"] * 1e6, "topk_bytes": nbytes,
            "topk_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("draft_topk", cfg.name)},
            "build_us": times["build"] * 1e6}


def bench_store_path(G, cfg, dims, sets, slot_d, acc_d, ws, rotate, steps, vbytes, pbytes, t_ver, t_per):
    """The pages' own tree path for comparison: verify that also stores every
    node's state in fp16 (gdn_tree_verify_store), and a commit that copies the
    accepted node's stored state (gdn_tree_persist_copy), each timed per call
    with HIP events, beside this library's replay path."""
    import torch
    T, Hv, D, B = dims.total_nodes, cfg.num_v_heads, cfg.head_dim, cfg.num_seqs
    node_states = torch.empty((T, Hv, D, D), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    t = {}
    for name in ("verify_store", "persist_copy"):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps + 3):
            d = sets[i % rotate]
            if name == "persist_copy":
                # the stored states must be this copy's: store first, outside the events
                G.gdn_tree_verify_store(dims, d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], slot_d, d["out"],
                                        node_states, ws)
            e = ev[i - 3] if i >= 3 else None
            if e:
                e[0].record(stream)
            if name == "verify_store":
                G.gdn_tree_verify_store(dims, d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], slot_d, d["out"],
                                        node_states, ws)
            else:
                G.gdn_tree_persist_copy(dims, acc_d, node_states, d["cache"], slot_d, ws)
            if e:
                e[1].record(stream)
        torch.cuda.synchronize()
        t[name] = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    stored = T * Hv * D * D * 2
    return {"verify_store_us": t["verify_store"] * 1e6, "persist_copy_us": t["persist_copy"] * 1e6,
            "verify_store_bytes": vbytes + stored, "persist_copy_bytes": B * Hv * D * D * (2 + 4),
            "replay_verify_us": t_ver * 1e6, "replay_persist_us": t_per * 1e6,
            "replay_bytes": vbytes + pbytes,
            "store_path_over_replay": (t["verify_store"] + t["persist_copy"]) / (t_ver + t_per)}


def bench_snapshot(G, cfg, sets, slot_d, rotate, layers, steps):
    """Prefix-cache restore: every sequence's committed state of one layer copied
    from a prefix pool into its cache slot (gdn_state_copy), timed per call with
    HIP events, rotating over the workload's independent cache copies."""
    import torch
    B = cfg.num_seqs
    copies = [sets[r * layers]["cache"] for r in range(rotate)]
    pools = [c[slot_d.long()].clone() for c in copies]
    pool_slots = torch.arange(B, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(5):
        G.gdn_state_copy(pools[i % rotate], pool_slots, copies[i % rotate], slot_d)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        G.gdn_state_copy(pools[i % rotate], pool_slots, copies[i % rotate], slot_d)
        e1.record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    nbytes = 2 * B * cfg.num_v_heads * cfg.head_dim * cfg.head_dim * 4 + 8 * B
    gbs = nbytes / t / 1e9
    return {"slots": B, "call_us": t * 1e6, "bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("snapshot", cfg.name)}}


# the sources each measured kernel is built from: counters recorded for one of
# them stay valid while these files keep their code
KERNEL_SOURCES = {
    "tree_verify": ("gdn_fast.hip", "gdn_internal.h"),
    "persist": ("gdn_fast.hip", "gdn_internal.h"),
    "fused": ("gdn_fast.hip", "gdn_internal.h"),
    "accept": ("gdn_accept.hip", "gdn_internal.h"),
    "draft_topk": ("gdn_ddtree.hip", "gdn_internal.h"),
    "snapshot": ("gdn_snapshot.hip", "gdn_internal.h"),
}


def kernel_source_digest(kernel: str) -> str:
    """Hash of a kernel's sources with comments and whitespace removed: a
    change of code invalidates recorded counters, a change of comments not."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_tree_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = re.sub(r"\s+", " ", text).strip()
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_digest") != kernel_source_digest(kernel):
        return None
    return ent["bytes_per_launch"]


def cpu_baseline(cfg, trees, cu, acc, seconds, layer_calls=None, single_thread=True):
    """The fp64 oracle (verify + persist) on the host cores.  One layer call is
    every sequence of the workload on one layer's inputs, each sequence from its
    own committed state.  After one warm-up sequence, whole layer calls run while
    about `seconds` of oracle work lasts (at most `layer_calls` of them); `value`
    is the median rate over the calls, a call cut short by the budget counting
    the sequences it finished.  With `single_thread` the same is done again on
    one thread, the budget split between the two runs."""
    import oracle
    import workloads as W
    rng = np.random.default_rng(0)
    inputs = [W.make_layer_inputs(cfg, layer, trees) for layer in range(2)]
    states = [(0.1 * rng.standard_normal((cfg.num_v_heads, cfg.head_dim, cfg.head_dim))).astype(np.float32)
              for _ in range(cfg.num_seqs)]
    T = int(cu[-1])

    def one_seq(inp, s):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = {k: v[lo:hi] for k, v in inp.items()}
        t0 = time.perf_counter()
        oracle.tree(trees[s], sl["q"], sl["k"], sl["v"], sl["a"], sl["b"], states[s])
        oracle.accept_state(trees[s], int(acc[s]), sl["k"], sl["v"], sl["a"], sl["b"], states[s])
        return time.perf_counter() - t0, hi - lo

    def run(budget):
        one_seq(inputs[0], 0)
        rates, nodes, t_total, calls, whole = [], 0, 0.0, 0, 0
        while t_total < budget and (layer_calls is None or calls < layer_calls):
            inp = inputs[calls % len(inputs)]
            t_call, n_call = 0.0, 0
            for s in range(cfg.num_seqs):
                dt, n = one_seq(inp, s)
                t_call, n_call = t_call + dt, n_call + n
                if t_total + t_call >= budget:
                    break
            whole += n_call == T
            rates.append(n_call / t_call)
            nodes, t_total, calls = nodes + n_call, t_total + t_call, calls + 1
        return float(np.median(rates)), nodes, t_total, calls, whole

    share = seconds / 2 if single_thread else seconds
    rate, nodes, t_total, calls, whole = run(share)
    res = {"value": rate, "unit": "nodes/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": "%d layer calls (%d whole) of the %s workload, each every sequence's tree on one layer's "
                     "inputs (%d nodes in all, verify + persist, fp64), %.1f s; median rate over the calls"
                     % (calls, whole, cfg.name, nodes, t_total),
           "nproc": os.cpu_count(), "model_name": cpu_model_name(),
           "layer_call_ms": T / rate * 1e3}
    if cfg.num_layers > 1:
        res["step_ms_extrapolated"] = T / rate * 1e3 * cfg.num_layers
        res["extrapolation"] = "one layer call's rate times %d layer calls per step" % cfg.num_layers
    if single_thread:
        oracle.set_threads(1)
        try:
            rate1, nodes1, t1, calls1, whole1 = run(share)
        finally:
            oracle.set_threads(0)
        res["single_thread"] = {
            "value": rate1, "unit": "nodes/s", "cores": 1,
            "sample": "%d layer calls (%d whole), %d nodes, %.1f s" % (calls1, whole1, nodes1, t1)}
    return res


if __name__ == "__main__":
    main()
