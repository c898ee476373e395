"""Benchmark of the verification hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu]

A step is one spec_verify_chain call over one batch of the headline workload:
chain verification, B=64 requests, gamma=5 drafts, V=128256, bf16 target logits
(N(0, 3^2), 1% of entries +8), fp32 draft distributions, T=0.8 -- 384 verified
positions per step.  Inputs are synthetic (synth.make_config(3)), resident in HBM
before timing starts, and rotated over several device copies whose total exceeds
twice the 256 MB Infinity Cache, so every step streams from HBM.

Prints ONE JSON line: throughput (verified positions/s) over K timed steps, the
roofline of the verification kernel (one launch per call) from HIP events recorded on
the stream it runs on, the oracle's CPU throughput on a bounded sample (measured first,
before the GPU is touched), and secondary measurements: the greedy chain (B=256,
gamma=8, V=128256), membership tree and greedy tree (B=32, N=63, V=152064), residual-update
tree (B=32, N=31, V=32000) workloads, and the headline chain with stop tokens and budgets and
with target logit processors.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_copies(make, per_copy_bytes, min_copies=3):
    n = max(min_copies, int(np.ceil(2 * MALL_BYTES / max(per_copy_bytes, 1))) + 1)
    return [make() for _ in range(n)]


def time_calls(calls, steps, warmup, stream):
    """Runs prepared calls round-robin: `warmup` untimed, then `steps` timed back to back.

    Returns (seconds between the events that bracket the timed steps, per-launch
    durations in ms from a second pass of `steps` calls each bracketed by its own pair of
    events on the same stream)."""
    import torch
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        calls[i % len(calls)]()
    t1.record(stream)
    torch.cuda.synchronize()
    span_ms = t0.elapsed_time(t1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        calls[i % len(calls)]()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return span_ms / 1e3, per


def bench_tree_residual(args, torch, sv, synth):
    x = synth.make_config(6, 0)
    B, N, V = x.B, x.N, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    nt, pt = torch.from_numpy(x.node_tokens).to(dev), torch.from_numpy(x.parents).to(dev)
    ua, ud = torch.from_numpy(x.u_acc).to(dev), torch.from_numpy(x.u_draw).to(dev)
    sets = device_copies(lambda: (lt.clone(), qt.clone(), nt, pt, ua, ud), lt.numel() * 2 + qt.numel() * 4)
    del lt, qt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.tree_residual_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_tree_residual(*s, float(x.temperature), workspace_tensor=ws) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    acc = calls[0].out["accepted_len"].cpu().numpy()
    launch = span / len(per)
    del sets, calls
    return dict(workload="tree with residual updates B=32 N=31 V=32000 bf16 logits, fp32 q, T=1",
                nodes_per_s=B * N * len(per) / span, launch_us=launch * 1e6,
                evented_launch_mean_us=float(per.mean()) * 1e3, mean_accepted=float(acc.mean()),
                dense_equivalent_gbs=B * N * V * (2 + 4) / launch / 1e9)


def traffic_record(name):
    """Per-launch HBM traffic from the committed rocprofv3 counter summary for kernel `name`,
    or None when the kernel sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec if h.hexdigest() == rec["sources_sha256"] else None


def bench_chain(args, torch, sv, synth):
    x = synth.make_config(3, 0)
    B, G, V = x.B, x.gamma, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    tt = torch.from_numpy(x.tokens).to(dev)
    ut = torch.from_numpy(x.u).to(dev)
    per_copy = lt.numel() * 2 + qt.numel() * 4
    sets = device_copies(lambda: (lt.clone(), qt.clone(), tt.clone(), ut.clone()), per_copy)
    del lt, qt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.chain_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_chain(s[0], s[1], s[2], s[3], float(x.temperature), workspace_tensor=ws)
             for s in sets]
    span, per = time_calls(calls, args.steps, args.warmup, stream)
    acc = calls[0].out["accepted_len"].cpu().numpy()
    st = calls[0].out["req_status"].cpu().numpy()
    assert (st == 0).all(), "unexpected request errors in the benchmark workload"
    n_rej = int((acc < G).sum())
    logit_bytes = B * (G + 1) * V * 2
    q_bytes = n_rej * V * 4
    small = B * G * (4 + 4 + 2) + B * (G + 1) * 4 + B * (G + 2) * 4 * 2   # gathers, u, outputs
    alg_bytes = logit_bytes + q_bytes + small
    med_ms = float(np.median(per))
    return dict(x=x, span=span, per=per, n_rej=n_rej, alg_bytes=alg_bytes,
                logit_bytes=logit_bytes, q_bytes=q_bytes, med_ms=med_ms, mean_ms=float(per.mean()),
                positions=B * (G + 1), mean_acc=float(acc.mean()), copies=len(sets))


def bench_greedy(args, torch, sv, synth):
    x = synth.make_config(4, 0)
    B, G, V = x.B, x.gamma, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    tt = torch.from_numpy(x.tokens).to(dev)
    sets = device_copies(lambda: (lt.clone(), tt.clone()), lt.numel() * 2)
    del lt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.greedy_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_greedy(s[0], s[1], workspace_tensor=ws) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    alg = B * (G + 1) * V * 2 + B * G * 4 + B * (G + 2) * 8
    launch = span / len(per)       # seconds per launch over the timed region
    del sets, calls
    trec = traffic_record("greedy_kernel_config4")
    return dict(workload="greedy B=256 gamma=8 V=128256 bf16", positions_per_s=B * (G + 1) * len(per) / span,
                launch_us=launch * 1e6, evented_launch_mean_us=float(per.mean()) * 1e3,
                achieved_gbs=alg / launch / 1e9, frac=alg / launch / 1e9 / HBM_PEAK_GBS, alg_bytes=alg,
                traffic_gbs=None if trec is None else trec["bytes_per_launch"] / launch / 1e9)


def bench_greedy_lazy(args, torch, sv, synth, k):
    """The greedy workload with lazy rows (spec_verify_greedy_ex, lazy_rows = k): rows read in
    groups of k, a group only when every draft before it matched."""
    x = synth.make_config(4, 0)
    B, G, V = x.B, x.gamma, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    tt = torch.from_numpy(x.tokens).to(dev)
    sets = device_copies(lambda: (lt.clone(),), lt.numel() * 2)
    del lt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.greedy_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_greedy(s[0], tt, workspace_tensor=ws, lazy_rows=k) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    acc = calls[0].out["accepted_len"].cpu().numpy()
    assert (calls[0].out["req_status"].cpu().numpy() == 0).all()
    launch = span / len(per)
    R = G + 1
    needed = int((acc + 1).sum())
    read = int(np.minimum(R, -(-(acc + 1) // k) * k).sum())
    alg = needed * V * 2 + B * G * 4 + B * (G + 2) * 8
    del sets, calls
    return dict(workload=f"greedy B=256 gamma=8 V=128256 bf16, lazy rows in groups of {k}",
                positions_per_s=B * R * len(per) / span, us_per_call=launch * 1e6,
                evented_call_mean_us=float(per.mean()) * 1e3, rows_needed=needed, rows_read=read,
                rows_dense=B * R, alg_bytes_per_call=alg, alg_gbs=alg / launch / 1e9,
                alg_frac=alg / launch / 1e9 / HBM_PEAK_GBS)


def bench_tree(args, torch, sv, synth):
    x = synth.make_config(5, 0)
    B, N, V = x.B, x.N, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    nt = torch.from_numpy(x.node_tokens).to(dev)
    pt = torch.from_numpy(x.parents).to(dev)
    ut = torch.from_numpy(x.u).to(dev)
    sets = device_copies(lambda: (lt.clone(), nt.clone(), pt.clone(), ut.clone()), lt.numel() * 2)
    del lt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.tree_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_tree(s[0], s[1], s[2], s[3], float(x.temperature), workspace_tensor=ws) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    acc = calls[0].out["accepted_len"].cpu().numpy()
    visited = int((acc + 1).sum())
    alg = visited * V * 2 + B * N * 12
    launch = span / len(per)
    del sets, calls
    return dict(workload="tree B=32 N=63 V=152064 bf16 T=1", nodes_per_s=B * N * len(per) / span,
                launch_us=launch * 1e6, evented_launch_mean_us=float(per.mean()) * 1e3,
                visited_rows=visited, achieved_gbs_visited=alg / launch / 1e9,
                dense_equivalent_gbs=B * N * V * 2 / launch / 1e9)


def bench_tree_greedy(args, torch, sv, synth):
    x = synth.make_config(5, 0)
    B, N, V = x.B, x.N, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    nt = torch.from_numpy(x.node_tokens).to(dev)
    pt = torch.from_numpy(x.parents).to(dev)
    sets = device_copies(lambda: (lt.clone(), nt.clone(), pt.clone()), lt.numel() * 2)
    del lt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.tree_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_tree_greedy(s[0], s[1], s[2], workspace_tensor=ws) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    acc = calls[0].out["accepted_len"].cpu().numpy()
    visited = int((acc + 1).sum())
    alg = visited * V * 2 + B * N * 8
    launch = span / len(per)
    del sets, calls
    return dict(workload="greedy tree B=32 N=63 V=152064 bf16", nodes_per_s=B * N * len(per) / span,
                launch_us=launch * 1e6, evented_launch_mean_us=float(per.mean()) * 1e3,
                visited_rows=visited, achieved_gbs_visited=alg / launch / 1e9,
                dense_equivalent_gbs=B * N * V * 2 / launch / 1e9)


def bench_chain_stop(args, torch, sv, synth):
    """The headline chain workload through spec_verify_chain_stop: 64 stop tokens (48 of
    them draft tokens), budgets uniform on [0, 7]."""
    x = synth.make_config(3, 0)
    stop, budget = synth.make_stop(x.tokens, x.V, seed=301, n_stop=64, from_drafts=48)
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    tt, ut = torch.from_numpy(x.tokens).to(dev), torch.from_numpy(x.u).to(dev)
    st, bt = torch.from_numpy(stop).to(dev), torch.from_numpy(budget).to(dev)
    sets = device_copies(lambda: (lt.clone(), qt.clone()), lt.numel() * 2 + qt.numel() * 4)
    del lt, qt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.chain_workspace_bytes(x.B, x.gamma, x.V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_chain(s[0], s[1], tt, ut, float(x.temperature), workspace_tensor=ws, stop_tokens=st,
                              budget=bt) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    fin = np.bincount(calls[0].out["finish"].cpu().numpy(), minlength=3)
    launch = span / len(per)
    del sets, calls
    return dict(workload="chain B=64 gamma=5 V=128256 bf16 with 64 stop tokens and budgets 0..7",
                positions_per_s=x.B * (x.gamma + 1) * len(per) / span, launch_us=launch * 1e6,
                evented_launch_mean_us=float(per.mean()) * 1e3,
                finish_counts=dict(open=int(fin[0]), stop=int(fin[1]), budget=int(fin[2])))


def bench_chain_sparse(args, torch, sv, synth):
    """The headline chain workload with a top-K drafter (K = 64): draft rows given as K
    (index, value) pairs, so a rejecting request reads 8 K bytes of its q row instead of 4 V.
    Algorithmic bytes: every target row once, the K pairs of each rejecting request's row."""
    K = 64
    spec = dict(synth.CONFIGS[3])
    spec.pop("kind")
    B, G, V = spec.pop("B"), spec.pop("gamma"), spec.pop("V")
    x, idx, vals = synth.make_chain_sparse(B, G, V, K, seed=0, **spec)
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    it, vt = torch.from_numpy(idx).to(dev), torch.from_numpy(vals).to(dev)
    tt, ut = torch.from_numpy(x.tokens).to(dev), torch.from_numpy(x.u).to(dev)
    sets = device_copies(lambda: lt.clone(), lt.numel() * 2)
    del lt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.chain_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_chain(s, vt, tt, ut, float(x.temperature), workspace_tensor=ws, q_index=it) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    acc = calls[0].out["accepted_len"].cpu().numpy()
    n_rej = int((acc < G).sum())
    alg = B * (G + 1) * V * 2 + n_rej * K * 8 + B * G * 10 + B * (G + 1) * 4
    launch = span / len(per)
    del sets, calls
    return dict(workload=f"chain B={B} gamma={G} V={V} bf16 logits, sparse draft rows K={K}, T={spec['temperature']}",
                positions_per_s=B * (G + 1) * len(per) / span, us_per_call=launch * 1e6,
                evented_call_mean_us=float(per.mean()) * 1e3, rejecting_requests=n_rej, alg_bytes_per_call=alg,
                alg_gbs=alg / launch / 1e9, alg_frac=alg / launch / 1e9 / HBM_PEAK_GBS)


def bench_chain_proc(args, torch, sv, synth, truncate):
    """The headline chain workload through spec_verify_chain_ex with target logit processors:
    fp32 bias and 90%-allowed masks per row, plus (truncate) top-k in {0, 1, 20, 1000} and
    top-p in {1, 0.5, 0.9, 0.99} per request, which add the threshold pre-pass."""
    x = synth.make_config(3, 0)
    bias, words, k, p = synth.make_processors(x.B, x.gamma + 1, x.V, seed=11, with_top_k=truncate,
                                              with_top_p=truncate)
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    tt, ut = torch.from_numpy(x.tokens).to(dev), torch.from_numpy(x.u).to(dev)
    bt = torch.from_numpy(bias).to(dev)
    wt = torch.from_numpy(words.view(np.int32)).to(dev)
    kt = None if k is None else torch.from_numpy(k).to(dev)
    pt = None if p is None else torch.from_numpy(p).to(dev)
    sets = device_copies(lambda: (lt.clone(), qt.clone()), lt.numel() * 2 + qt.numel() * 4)
    del lt, qt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.chain_workspace_bytes(x.B, x.gamma, x.V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_chain(s[0], s[1], tt, ut, float(x.temperature), workspace_tensor=ws, bias=bt, allowed=wt,
                              top_k=kt, top_p=pt) for s in sets]
    span, per = time_calls(calls, max(100, args.steps // 2), args.warmup, stream)
    launch = span / len(per)
    del sets, calls
    what = "bias, masks, top-k, top-p (threshold pass + verification)" if truncate else "bias and masks"
    return dict(workload=f"chain B=64 gamma=5 V=128256 bf16 with {what}",
                positions_per_s=x.B * (x.gamma + 1) * len(per) / span, us_per_call=launch * 1e6,
                evented_call_mean_us=float(per.mean()) * 1e3)


def bench_chain_lazy(args, torch, sv, synth, k, fp32=False):
    """The headline chain workload (fp32: its fp32-logit variant at T = 1), with lazy rows
    when k >= 1 (spec_verify_chain_ex, lazy_rows = k: rows read in groups of k, a group only
    when every draft before it was accepted), or every row read (k = 0)."""
    x = synth.make_config(3, 0, logit_dtype="f32", temperature=1.0) if fp32 else synth.make_config(3, 0)
    B, G, V = x.B, x.gamma, x.V
    dev = "cuda:0"
    if fp32:
        lt = torch.from_numpy(x.logits).to(dev)
    else:
        lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    tt, ut = torch.from_numpy(x.tokens).to(dev), torch.from_numpy(x.u).to(dev)
    sl = lt.element_size()
    sets = device_copies(lambda: (lt.clone(), qt.clone()), lt.numel() * sl + qt.numel() * 4)
    del lt, qt
    stream = torch.cuda.current_stream()
    ws = torch.zeros(sv.chain_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_chain(s[0], s[1], tt, ut, float(x.temperature), workspace_tensor=ws, lazy_rows=k)
             for s in sets]
    span, per = time_calls(calls, args.steps, args.warmup, stream)
    acc = calls[0].out["accepted_len"].cpu().numpy()
    assert (calls[0].out["req_status"].cpu().numpy() == 0).all()
    launch = span / len(per)
    R = G + 1
    needed = int((acc + 1).sum()) if k else B * R                  # rows 0..A of every request
    read = int(np.minimum(R, -(-(acc + 1) // k) * k).sum()) if k else B * R   # whole groups
    n_rej = int((acc < G).sum())
    alg = needed * V * sl + n_rej * V * 4 + B * G * 10 + B * R * 4 + B * (G + 2) * 8
    del sets, calls
    what = f"lazy rows in groups of {k}" if k else "every row read"
    dt = "fp32 logits, T=1" if fp32 else "bf16 logits, T=0.8"
    return dict(workload=f"chain B=64 gamma=5 V=128256 {dt}, {what}",
                positions_per_s=B * R * len(per) / span, us_per_call=launch * 1e6,
                evented_call_mean_us=float(per.mean()) * 1e3, rows_needed=needed, rows_read=read,
                rows_dense=B * R, alg_bytes_per_call=alg, alg_gbs=alg / launch / 1e9,
                alg_frac=alg / launch / 1e9 / HBM_PEAK_GBS)


def bench_sweep(args, torch, sv, synth):
    """Bandwidth sweep of the chain verifier: config 3's recipe (gamma = 5, V = 128256) with
    bf16 logits at T = 0.8 and fp32 logits at T = 1, over batch sizes B (the first B requests
    of a 256-request batch); one JSON line per point with the time per call and the achieved
    GB/s on the algorithmic bytes (every row once plus each rejecting request's fp32 q row)."""
    dev = "cuda:0"
    sizes = (8, 16, 32, 64, 128, 256)
    for fp32 in (False, True):
        # the largest batch once; smaller ones are its first B requests (requests are independent)
        x = synth.make_config(3, 0, B=sizes[-1], **(dict(logit_dtype="f32", temperature=1.0) if fp32 else {}))
        G, V = x.gamma, x.V
        for B in sizes:
            if fp32:
                lt = torch.from_numpy(x.logits[:B]).to(dev)
            else:
                lt = torch.from_numpy(x.logits[:B].view(np.int16)).to(dev).view(torch.bfloat16)
            qt = torch.from_numpy(x.q[:B]).to(dev)
            tt, ut = torch.from_numpy(x.tokens[:B]).to(dev), torch.from_numpy(x.u[:B]).to(dev)
            sl = lt.element_size()
            sets = device_copies(lambda: (lt.clone(), qt.clone()), lt.numel() * sl + qt.numel() * 4)
            del lt, qt
            ws = torch.zeros(sv.chain_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=dev)
            calls = [sv.prepare_chain(s_[0], s_[1], tt, ut, float(x.temperature), workspace_tensor=ws) for s_ in sets]
            span, per = time_calls(calls, args.steps, args.warmup, torch.cuda.current_stream())
            acc = calls[0].out["accepted_len"].cpu().numpy()
            n_rej = int((acc < G).sum())
            alg = B * (G + 1) * V * sl + n_rej * V * 4 + B * G * 10 + B * (G + 1) * 4 + B * (G + 2) * 8
            launch = span / len(per)
            print(json.dumps(dict(sweep="chain", logits="fp32" if fp32 else "bf16", B=B, gamma=G, V=V,
                                  us_per_call=launch * 1e6, alg_bytes=alg, alg_gbs=alg / launch / 1e9,
                                  frac=alg / launch / 1e9 / HBM_PEAK_GBS,
                                  positions_per_s=B * (G + 1) / launch)), flush=True)
            del sets, calls, ws
            torch.cuda.empty_cache()


TRACE_WORDS = 16         # words per record of the timeline-trace build
TRACE_KERNELS = 5        # kernel slots: 0 chain, 1 exact redraw, 2 tree, 3 residual tree, 4 thresholds
TICK_US = 0.01           # s_memrealtime runs at 100 MHz


def _trace_records(buf, cap):
    """The trace buffer as {slot: (tag fields, stamps in us)} for the blocks that wrote a tag."""
    a = buf.cpu().numpy().view(np.uint64).reshape(TRACE_KERNELS, cap, TRACE_WORDS)
    out = {}
    for k in range(TRACE_KERNELS):
        r = a[k][(a[k][:, 0] >> np.uint64(63)) == 1]
        tag = r[:, 0]
        out[k] = dict(kind=((tag >> np.uint64(56)) & np.uint64(0x7f)).astype(int),
                      b=((tag >> np.uint64(24)) & np.uint64(0xffffffff)).astype(int),
                      idx=(tag & np.uint64(0xffffff)).astype(int),
                      t=r[:, 1:].astype(np.int64))
    return out


def _med(v):
    v = np.asarray(v, dtype=float)
    v = v[np.isfinite(v)]
    return float(np.median(v)) if v.size else float("nan")


def timeline_chain(args, torch, sv, synth, lib, proc=False):
    """Per-block timeline of the headline chain call from the trace build: when the statistics
    stream ends, and each selector's steps (decision, own chunk mass, every mass in, rescan,
    outputs, workspace cleared), then the exact-redraw kernel.  Prints a markdown summary.
    With proc, the chain kernel of the processors line (bias, masks, top-k, top-p; the
    threshold pass runs first and is not part of the times)."""
    import ctypes
    x = synth.make_config(3, 0)
    B, G, V = x.B, x.gamma, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    tt, ut = torch.from_numpy(x.tokens).to(dev), torch.from_numpy(x.u).to(dev)
    sets = device_copies(lambda: (lt.clone(), qt.clone()), lt.numel() * 2 + qt.numel() * 4)
    del lt, qt
    ws = torch.zeros(sv.chain_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=dev)
    kw = {}
    if proc:
        bias, words, k, p = synth.make_processors(B, G + 1, V, seed=11)
        kw = dict(bias=torch.from_numpy(bias).to(dev), allowed=torch.from_numpy(words.view(np.int32)).to(dev),
                  top_k=torch.from_numpy(k).to(dev), top_p=torch.from_numpy(p).to(dev))
    calls = [sv.prepare_chain(s_[0], s_[1], tt, ut, float(x.temperature), workspace_tensor=ws, **kw)
             for s_ in sets]
    stream = torch.cuda.current_stream()
    cap = 8192
    buf = torch.zeros(TRACE_KERNELS * cap * TRACE_WORDS, dtype=torch.int64, device=dev)
    assert lib.spec_trace_set(ctypes.c_void_p(0), 0) == 0
    span_off, _ = time_calls(calls, args.steps, args.warmup, stream)
    assert lib.spec_trace_set(ctypes.c_void_p(buf.data_ptr()), cap) == 0
    span_on, _ = time_calls(calls, args.steps, args.warmup, stream)
    rows = []
    for rep in range(args.timeline_calls):
        buf.zero_()
        torch.cuda.synchronize()
        calls[rep % len(calls)]()
        torch.cuda.synchronize()
        rec = _trace_records(buf, cap)
        c, e = rec[0], rec[1]
        t = c["t"].astype(float)
        t[t == 0] = np.nan
        base = np.nanmin(t[:, 0])
        t = (t - base) * TICK_US
        kind, b = c["kind"], c["b"]
        S, L = kind == 0, kind == 3
        if L.sum() != B:
            raw = buf.cpu().numpy().view(np.uint64).reshape(TRACE_KERNELS, cap, TRACE_WORDS)
            if os.environ.get("SPEC_TRACE_DUMP"):
                np.save(os.environ["SPEC_TRACE_DUMP"], raw)
            nz = np.nonzero(raw[0][:, 0])[0]
            raise RuntimeError(f"trace records: {len(kind)} blocks, kinds {np.bincount(kind).tolist()}, "
                               f"selectors for requests {np.unique(b[L]).tolist()}; tagged records "
                               f"{nz.min()}..{nz.max()} ({nz.size}); slot-1 records tagged "
                               f"{np.count_nonzero(raw[1][:, 0])}")
        chain_end = np.nanmax(t)
        T = kind == 2
        term_start = _med(t[T, 0]) if T.any() else float("nan")
        stats_done = np.array([np.nanmax(t[S & (b == r), 1]) for r in range(B)])
        sel = {r: t[L & (b == r)][0] for r in range(B)}
        steps = np.array([[sel[r][1] - sel[r][0],                 # start -> decided
                           sel[r][2] - sel[r][1],                 # decided -> own chunk mass
                           sel[r][3] - sel[r][2],                 # own mass -> every mass in
                           sel[r][4] - sel[r][3],                 # masses in -> rescan done
                           sel[r][5] - sel[r][4],                 # rescan -> outputs written
                           sel[r][6] - sel[r][5]] for r in range(B)])
        sub = np.array([[sel[r][7] - sel[r][0],                   # start -> rows combined
                         sel[r][8] - sel[r][7],                   # -> gather records in
                         sel[r][9] - sel[r][8],                   # -> decided
                         sel[r][1] - sel[r][9],                   # -> past the block barrier
                         sel[r][10] - sel[r][3],                  # masses in -> chunk picked
                         sel[r][11] - sel[r][10],                 # -> chunk reloaded
                         sel[r][4] - sel[r][11]] for r in range(B)])   # -> rescan scans done
        sel_end = np.array([sel[r][6] for r in range(B)])
        last = int(np.argmax(sel_end))
        et = e["t"].astype(float)
        et[et == 0] = np.nan
        et = (et - base) * TICK_US
        k3_start, k3_end = np.nanmin(et[:, 0]), np.nanmax(et)
        rows.append(dict(chain_end=chain_end, stream_end=float(np.nanmax(t[S, 1])),
                         stats_item=_med(t[S, 2] - t[S, 0]), last_req_stats=float(stats_done.max()),
                         sel_start_last=float(sel[last][0]), sel_end_last=float(sel_end[last]),
                         steps_med=np.median(steps, axis=0), steps_last=steps[last],
                         sub_med=np.nanmedian(sub, axis=0), sub_last=sub[last],
                         after_stats_last=float(sel_end[last] - stats_done[last]),
                         k3_gap=float(k3_start - chain_end), k3_span=float(k3_end - k3_start),
                         k3_exact=int((e["kind"] == 5).sum()), total=float(k3_end), term_start=term_start))
    assert lib.spec_trace_set(ctypes.c_void_p(0), 0) == 0
    g = lambda k: _med([r_[k] for r_ in rows])
    sm = np.median(np.array([r_["steps_med"] for r_ in rows]), axis=0)
    sl = np.median(np.array([r_["steps_last"] for r_ in rows]), axis=0)
    names = ["dispatch -> decision", "decision -> own chunk mass", "own mass -> every mass in",
             "masses in -> rescan done", "rescan -> outputs written", "outputs -> workspace cleared"]
    what = ", bias, masks, top-k, top-p (chain kernel after the threshold pass)" if proc else ""
    print(f"## chain_kernel timeline: B={B} gamma={G} V={V} bf16 logits, fp32 q, T={x.temperature}{what}")
    print()
    print(f"Trace build, {args.timeline_calls} traced calls; medians over calls. Times in us from the "
          f"first block's start (s_memrealtime, 10 ns ticks). Calls of the trace build: "
          f"{span_off / args.steps * 1e6:.1f} us with tracing off, {span_on / args.steps * 1e6:.1f} us on "
          f"(event span / {args.steps} back-to-back calls).")
    print()
    print("| event | us |")
    print("|---|---|")
    print(f"| median statistics item (start -> published) | {g('stats_item'):.2f} |")
    print(f"| statistics stream ends (last item's stream done) | {g('stream_end'):.2f} |")
    print(f"| median terminal item start | {g('term_start'):.2f} |")
    print(f"| last-finishing request: its statistics done | {g('last_req_stats'):.2f} |")
    print(f"| last-finishing request: selector dispatched | {g('sel_start_last'):.2f} |")
    print(f"| last-finishing request: selector done | {g('sel_end_last'):.2f} |")
    print(f"| chain kernel's last stamp | {g('chain_end'):.2f} |")
    print(f"| exact-redraw kernel: first block starts after the chain's last stamp | {g('k3_gap'):.2f} |")
    print(f"| exact-redraw kernel: first start -> last stamp | {g('k3_span'):.2f} |")
    print(f"| call: first start -> last stamp | {g('total'):.2f} |")
    print()
    print("| selector step | median over the requests | request that finishes last |")
    print("|---|---|---|")
    for n_, a_, b_ in zip(names, sm, sl):
        print(f"| {n_} | {a_:.2f} | {b_:.2f} |")
    print()
    sub_names = ["dispatch -> summaries in, rows combined", "-> gather records in", "-> decision taken",
                 "-> past the block barrier", "masses in -> chunk picked", "chunk picked -> chunk reloaded",
                 "chunk reloaded -> rescan scans done"]
    sbm = np.median(np.array([r_["sub_med"] for r_ in rows]), axis=0)
    sbl = np.median(np.array([r_["sub_last"] for r_ in rows]), axis=0)
    print("| selector sub-step | median over the requests | request that finishes last |")
    print("|---|---|---|")
    for n_, a_, b_ in zip(sub_names, sbm, sbl):
        print(f"| {n_} | {a_:.2f} | {b_:.2f} |")
    print()
    print(f"Last-finishing request: {g('after_stats_last'):.2f} us from its statistics' end to its selector's end; "
          f"exact redraws per call: {g('k3_exact'):.0f} blocks.")


def _traced_calls(args, torch, lib, calls, cap, slot):
    """Times `calls` with tracing off and on, then runs args.timeline_calls traced calls one at
    a time; returns (us per call off, us per call on, [records of kernel slot `slot`, base])."""
    import ctypes
    stream = torch.cuda.current_stream()
    buf = torch.zeros(TRACE_KERNELS * cap * TRACE_WORDS, dtype=torch.int64, device="cuda:0")
    assert lib.spec_trace_set(ctypes.c_void_p(0), 0) == 0
    span_off, per = time_calls(calls, args.steps, args.warmup, stream)
    assert lib.spec_trace_set(ctypes.c_void_p(buf.data_ptr()), cap) == 0
    span_on, _ = time_calls(calls, args.steps, args.warmup, stream)
    out = []
    for rep in range(args.timeline_calls):
        buf.zero_()
        torch.cuda.synchronize()
        calls[rep % len(calls)]()
        torch.cuda.synchronize()
        r = _trace_records(buf, cap)[slot]
        r["raw"] = r["t"].copy()
        t = r["t"].astype(float)
        t[t == 0] = np.nan
        base = np.nanmin(t[:, 0])
        r["t"] = (t - base) * TICK_US
        out.append(r)
    assert lib.spec_trace_set(ctypes.c_void_p(0), 0) == 0
    return span_off / args.steps * 1e6, span_on / args.steps * 1e6, out


def timeline_tree(args, torch, sv, synth, lib):
    """Per-hop timeline of the membership tree (B=32, N=63, V=152064): for each hop of each
    request's walk, the wait for the row's summaries (the root stream at hop 0, the helpers'
    round trip after that), the sample (chunk select and rescan), and the child search plus
    the next order."""
    x = synth.make_config(5, 0)
    B, N, V = x.B, x.N, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    nt, pt, ut = (torch.from_numpy(a).to(dev) for a in (x.node_tokens, x.parents, x.u))
    sets = device_copies(lambda: (lt.clone(), nt, pt, ut), lt.numel() * 2)
    del lt
    ws = torch.zeros(sv.tree_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_tree(s_[0], s_[1], s_[2], s_[3], float(x.temperature), workspace_tensor=ws) for s_ in sets]
    off, on, recs = _traced_calls(args, torch, lib, calls, 8192, 2)
    per_hop = {}
    ends, root_ends, walk_starts = [], [], []
    for r in recs:
        t, kind, b = r["t"], r["kind"], r["b"]
        node = kind == 8
        root = kind == 0
        root_ends.append(np.nanmax(t[(kind == 0) | (kind == 2), 1]))
        walk_starts.append(_med(t[kind == 2, 1]))
        ends.append(np.nanmax(t))
        for req in range(B):
            h = t[node & (b == req)]
            h = h[np.argsort(h[:, 0])]
            for j in range(len(h)):
                wait = h[j, 1] - (h[j - 1, 3] if j else h[j, 0])
                per_hop.setdefault(j, []).append((wait, h[j, 2] - h[j, 1], h[j, 3] - h[j, 2], h[j, 3]))
    print(f"## tree_kernel timeline (membership): B={B} N={N} V={V} bf16 logits, T={x.temperature}")
    print()
    print(f"Trace build, {args.timeline_calls} traced calls; times in us from the first block's start. "
          f"Calls of the trace build: {off:.1f} us with tracing off, {on:.1f} us on.")
    print()
    print(f"Root stream: the last root chunk summary published at {_med(root_ends):.2f} us (median over "
          f"calls); the call's last stamp at {_med(ends):.2f} us.")
    print()
    print("| hop | walks reaching it | wait for the row's summaries | sample (select + rescan) | "
          "child search + order | hop done at (median) |")
    print("|---|---|---|---|---|---|")
    for j in sorted(per_hop):
        a = np.array(per_hop[j])
        what = "root row (stream)" if j == 0 else "helpers' round trip"
        print(f"| {j} | {len(a) // max(1, args.timeline_calls)} | {_med(a[:, 0]):.2f} ({what}) | "
              f"{_med(a[:, 1]):.2f} | {_med(a[:, 2]):.2f} | {_med(a[:, 3]):.2f} |")


def timeline_tree_residual(args, torch, sv, synth, lib):
    """Per-hop timeline of the residual-update tree (B=32, N=31, V=32000): node visits (wait for
    the row's summaries, normalizer) and residual passes (order -> every chunk mass in -> W)."""
    x = synth.make_config(6, 0)
    B, N, V = x.B, x.N, x.V
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    nt, pt = torch.from_numpy(x.node_tokens).to(dev), torch.from_numpy(x.parents).to(dev)
    ua, ud = torch.from_numpy(x.u_acc).to(dev), torch.from_numpy(x.u_draw).to(dev)
    sets = device_copies(lambda: (lt.clone(), qt.clone(), nt, pt, ua, ud), lt.numel() * 2 + qt.numel() * 4)
    del lt, qt
    ws = torch.zeros(sv.tree_residual_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_tree_residual(*s_, float(x.temperature), workspace_tensor=ws) for s_ in sets]
    off, on, recs = _traced_calls(args, torch, lib, calls, 8192, 3)
    node_wait, node_z, node_root, pass_in, pass_w, tests, draws, accept_order = [], [], [], [], [], [], [], []
    n_nodes, n_pass, ends, walk_ends = [], [], [], []
    for r in recs:
        t, kind, b = r["t"], r["kind"], r["b"]
        ends.append(np.nanmax(t))
        walk_ends.append(_med([np.nanmax(t[(kind >= 8) & (b == q)]) for q in range(B)]))
        n_nodes.append((kind == 8).sum() / B)
        n_pass.append((kind == 9).sum() / B)
        for req in range(B):
            sel = (kind >= 8) & (b == req)
            ev = sorted(zip(t[sel, 0], kind[sel], map(tuple, t[sel])), key=lambda e: e[0])
            prev_order = None   # when the order for the current node's row was published
            k = 0
            while k < len(ev):
                s_ = ev[k][2]           # a node visit: slots top, staged, Z, child order, draw
                if prev_order is None:
                    node_root.append(s_[1])
                else:
                    node_wait.append(s_[1] - prev_order)
                node_z.append(s_[2] - s_[1])
                last = s_[2]
                k += 1
                while k < len(ev) and ev[k][1] == 9:   # its residual passes: order, masses in, W
                    p_ = ev[k][2]
                    tests.append(p_[0] - last)
                    pass_in.append(p_[1] - p_[0])
                    pass_w.append(p_[2] - p_[1])
                    last = p_[2]
                    k += 1
                if np.isfinite(s_[3]):
                    accept_order.append(s_[3] - last)
                    prev_order = s_[3]
                if np.isfinite(s_[4]):
                    draws.append(s_[4] - last)
    print(f"## tree_kernel timeline (residual-update): B={B} N={N} V={V} bf16 logits, fp32 q, T={x.temperature}")
    print()
    print(f"Trace build, {args.timeline_calls} traced calls; times in us. Calls of the trace build: "
          f"{off:.1f} us with tracing off, {on:.1f} us on. Per request: {_med(n_nodes):.1f} node visits and "
          f"{_med(n_pass):.1f} residual passes (medians over calls); median walk ends at {_med(walk_ends):.2f} us, "
          f"the call's last stamp at {_med(ends):.2f} us.")
    print()
    print("| step | count per call | median us |")
    print("|---|---|---|")
    nc = max(1, args.timeline_calls)
    print(f"| root row: summaries in (from the first block's start) | {len(node_root) // nc} | {_med(node_root):.2f} |")
    print(f"| node below the root: order for its row -> summaries in (helpers' round trip) | {len(node_wait) // nc} | {_med(node_wait):.2f} |")
    print(f"| summaries in -> normalizer Z | {len(node_z) // nc} | {_med(node_z):.2f} |")
    print(f"| accept test of a child (after Z or the last pass) -> pass order | {len(tests) // nc} | {_med(tests):.2f} |")
    print(f"| residual pass: order -> every chunk mass in (helpers' round trip) | {len(pass_in) // nc} | {_med(pass_in):.2f} |")
    print(f"| residual pass: masses in -> W published | {len(pass_w) // nc} | {_med(pass_w):.2f} |")
    print(f"| accepted child: accept test -> its row's order published | {len(accept_order) // nc} | {_med(accept_order):.2f} |")
    print(f"| terminal draw (after Z or the last W) -> token | {len(draws) // nc} | {_med(draws):.2f} |")


def timeline_thresh(args, torch, sv, synth, lib):
    """Per-row timeline of the top-k / top-p threshold pass on the processors workload (B=64,
    gamma=5, V=128256 bf16 with bias, masks, top-k in {0, 1, 20, 1000} and top-p in {1, 0.5,
    0.9, 0.99}): each row's phases and the slowest rows."""
    x = synth.make_config(3, 0)
    bias, words, k, p = synth.make_processors(x.B, x.gamma + 1, x.V, seed=11)
    dev = "cuda:0"
    lt = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    qt = torch.from_numpy(x.q).to(dev)
    tt, ut = torch.from_numpy(x.tokens).to(dev), torch.from_numpy(x.u).to(dev)
    bt, wt = torch.from_numpy(bias).to(dev), torch.from_numpy(words.view(np.int32)).to(dev)
    kt, pt = torch.from_numpy(k).to(dev), torch.from_numpy(p).to(dev)
    sets = device_copies(lambda: (lt.clone(), qt.clone()), lt.numel() * 2 + qt.numel() * 4)
    del lt, qt
    ws = torch.zeros(sv.chain_workspace_bytes(x.B, x.gamma, x.V) + 512, dtype=torch.uint8, device=dev)
    calls = [sv.prepare_chain(s_[0], s_[1], tt, ut, float(x.temperature), workspace_tensor=ws, bias=bt, allowed=wt,
                              top_k=kt, top_p=pt) for s_ in sets]
    off, on, recs = _traced_calls(args, torch, lib, calls, 8192, 4)
    rows = []
    for r in recs:
        t, kind, kk = r["t"], r["kind"], r["idx"]
        raw = r["raw"].astype(np.uint64)
        for i in range(len(kind)):
            tp = float(np.array([raw[i, 8] & np.uint64(0xffffffff)], dtype=np.uint64).astype(np.uint32).view(np.float32)[0])
            n1 = int(raw[i, 9] & np.uint64(0xffffffff))
            rows.append(dict(kind=int(kind[i]), k=int(kk[i]), p=tp, n=n1, radix=int(raw[i, 10]),
                             block=i, where=int(raw[i, 11]), rep=len(rows) // max(1, len(kind)),
                             dur=t[i, 6] - t[i, 0], p0=t[i, 1] - t[i, 0],
                             p1=t[i, 2] - t[i, 1], col=t[i, 3] - t[i, 2], res=t[i, 4] - t[i, 3],
                             topp=t[i, 5] - t[i, 4], rest=t[i, 6] - t[i, 5], start=t[i, 0], end=t[i, 6]))
    print(f"## thresh_kernel timeline: B={x.B} rows of gamma+1={x.gamma + 1}, V={x.V} bf16, bias, masks, top-k, top-p")
    print()
    print(f"Trace build, {args.timeline_calls} traced calls; per row (block) times in us. Calls of the trace build: "
          f"{off:.1f} us with tracing off, {on:.1f} us on (the whole processed chain call).")
    print()
    print("Stamps, window path: sample and window choice | window pass | window bins | top-k | top-p | end. "
          "Full path (top-1, and any row whose window fell back): sample and counting pass | (none) | collect | "
          "top-k | top-p | radix and end.")
    print()
    print("| rows (top-k, top-p) | count per call | median duration | max duration | stamp 1→2 | 2→3 | 3→4 | "
          "4→5 | 5→6 | 6→end |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    nc = max(1, args.timeline_calls)
    for kval in sorted(set(r_["k"] for r_ in rows if r_["kind"] != 0)):
        for pval in sorted(set(r_["p"] for r_ in rows if r_["kind"] != 0 and r_["k"] == kval)):
            sel = [r_ for r_ in rows if r_["kind"] != 0 and r_["k"] == kval and r_["p"] == pval]
            if not sel:
                continue
            f = lambda key: _med([r_[key] for r_ in sel])
            nrad = sum(1 for r_ in sel if r_["radix"] == 1)
            nfb = sum(1 for r_ in sel if r_["radix"] == 2)
            note = (f" (radix in {nrad})" if nrad else "") + (f" (window fell back in {nfb})" if nfb else "")
            print(f"| k={kval}, p={pval:g} | {len(sel) // nc} | {f('dur'):.2f} | {max(r_['dur'] for r_ in sel):.2f} | "
                  f"{f('p0'):.2f} | {f('p1'):.2f} | {f('col'):.2f} | {f('res'):.2f} | {f('topp'):.2f} | "
                  f"{f('rest'):.2f}{note} |")
    slow = sorted(rows, key=lambda r_: -r_["dur"] if np.isfinite(r_["dur"]) else 0)[:8]
    print()
    print("Slowest rows: " + "; ".join(f"k={r_['k']} p={r_['p']:g} {r_['dur']:.1f} us"
                                      f"{' (radix)' if r_['radix'] == 1 else (' (window fell back)' if r_['radix'] == 2 else '')}"
                                      for r_ in slow))
    ends = [r_["end"] for r_ in rows if np.isfinite(r_["end"])]
    print()
    print(f"Last row ends at {np.percentile(ends, 100):.2f} us (p90 {np.percentile(ends, 90):.2f}, "
          f"median {np.median(ends):.2f}) after the first row's start.")
    # placement (first traced call): which blocks share a CU
    first = [r_ for r_ in rows[:len(recs[0]["kind"])]]
    by_cu = {}
    for r_ in first:
        by_cu.setdefault(r_["where"], []).append(r_)
    shared = [sorted(v, key=lambda r_: r_["block"]) for v in by_cu.values() if len(v) > 1]
    gaps = {}
    for v in shared:
        g_ = v[-1]["block"] - v[0]["block"]
        gaps[g_] = gaps.get(g_, 0) + 1
    top = sorted(gaps.items(), key=lambda kv: -kv[1])[:4]
    low = sum(1 for v in shared for r_ in v if r_["block"] < 256)
    print()
    print(f"Placement (first traced call, from the hardware IDs): {len(by_cu)} CUs used, {len(shared)} with more "
          f"than one row; block-index gaps within a shared CU (gap: CUs): "
          + ", ".join(f"{g_}: {c_}" for g_, c_ in top)
          + f"; blocks below 256 among the shared: {low}.")


class _CachedSynth:
    """The synth module with make_config memoized, so that the lines that share a workload
    generate its inputs once (they only read them)."""

    def __init__(self, mod):
        self._mod, self._cache = mod, {}

    def make_config(self, k, run=0, **override):
        key = (k, run, tuple(sorted(override.items())))
        if key not in self._cache:
            self._cache[key] = self._mod.make_config(k, run, **override)
        return self._cache[key]

    def __getattr__(self, name):
        return getattr(self._mod, name)


_CPU_X = None   # the workload a forked oracle worker reads


def _oracle_worker(args):
    """Runs the oracle on requests k, k+stride, ... (cycling over the batch) for budget_s."""
    import oracle
    k, stride, budget_s = args
    x = _CPU_X
    t0 = time.perf_counter()
    n = 0
    while True:
        b = (k + n * stride) % x.B
        oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype, requests=[b])
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            return n


def cpu_baseline(x, budget_s):
    """The float64 oracle, as it stands, on requests of the headline workload: one process on
    one core, then a pool of forked processes over requests, one per core this process may
    run on up to 16 (a one-GPU machine's CPU share), each for about budget_s; nproc and the
    affinity count are reported beside the pool size.  Runs before anything touches the GPU, so the fork is of a plain CPU
    process."""
    import multiprocessing as mp
    global _CPU_X
    _CPU_X = x
    G = x.gamma
    t0 = time.perf_counter()
    n1 = _oracle_worker((0, 1, budget_s))
    el1 = time.perf_counter() - t0
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    # one worker per core this process may run on, up to 16: a one-GPU machine's CPU share
    workers = max(1, min(16, avail))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        counts = pool.map(_oracle_worker, [(k, workers, budget_s) for k in range(workers)])
    elp = time.perf_counter() - t0
    n = sum(counts)
    return dict(value=n * (G + 1) / elp, unit="verified positions/s", cores=workers, kind="oracle",
                nproc=os.cpu_count(), affinity_cores=avail,
                sample=f"{n} requests of the chain B=64 gamma=5 V=128256 bf16 workload (its 64 requests "
                       f"cycled), float64 NumPy oracle, {workers} forked processes for {elp:.1f} s "
                       f"wall including pool start-up",
                single_core=dict(value=n1 * (G + 1) / el1, cores=1,
                                 sample=f"{n1} requests on one core in {el1:.1f} s"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="all",
                    help="comma-separated secondary lines to run (greedy, tree, tree_residual, tree_greedy, "
                         "chain_stop, chain_bias_mask, chain_processors, chain_sparse, chain_lazy, chain_f32, greedy_lazy), or all")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sweep", action="store_true",
                    help="print the chain bandwidth sweep over batch sizes (one JSON line per point) instead")
    ap.add_argument("--timeline", choices=["chain", "chain_proc", "tree", "tree_residual", "thresh"],
                    help="print a per-block timeline summary (markdown) of one workload instead, from the "
                         "trace build (python -m exact_rejection_sampling_amd.build --trace)")
    ap.add_argument("--timeline-calls", type=int, default=5)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps(dict(error="this benchmark runs on one GPU only; run with --gpus 1")))
        sys.exit(2)

    import torch
    import exact_rejection_sampling_amd as sv
    import synth as synth_module
    synth = _CachedSynth(synth_module)
    cpu = None
    if not args.no_cpu and not args.sweep and not args.timeline:
        log("[bench] oracle CPU baseline")
        cpu = cpu_baseline(synth.make_config(3, 0), args.cpu_seconds)
    if not torch.cuda.is_available():
        print(json.dumps(dict(error="no GPU visible")))
        sys.exit(1)
    if args.timeline:
        from exact_rejection_sampling_amd import build as _build
        lib = sv.load_library(_build.TRACE_LIB, install=True)
        fn = dict(chain=timeline_chain, tree=timeline_tree, tree_residual=timeline_tree_residual,
                  thresh=timeline_thresh,
                  chain_proc=lambda *a: timeline_chain(*a, proc=True))[args.timeline]
        fn(args, torch, sv, synth, lib)
        return
    sv.load_library()
    if args.sweep:
        bench_sweep(args, torch, sv, synth)
        return

    log("[bench] chain headline workload")
    c = bench_chain(args, torch, sv, synth)
    value = c["positions"] * args.steps / c["span"]
    # the timed region's average launch duration: one launch per call, back to back
    launch_ms = c["span"] * 1e3 / args.steps
    achieved = c["alg_bytes"] / (launch_ms * 1e-3) / 1e9
    # traffic: HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counters (scaled
    # by what the counters read for device copies of known size), over the same launch time
    trec = traffic_record("chain_kernel_config3")
    traffic = None if trec is None else trec["bytes_per_launch"] / (launch_ms * 1e-3) / 1e9
    line = dict(
        metric="verified positions/s + achieved HBM GB/s (% peak), B=64 gamma=5 V=128256 bf16",
        value=value, unit="verified positions/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=c["span"] * 1e3 / args.steps, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="chain verify B=64 gamma=5 V=128256 bf16 logits, fp32 q, T=0.8",
                    B=64, gamma=5, V=128256, logits="bf16", q="fp32", temperature=0.8,
                    input_copies=c["copies"]),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=traffic,
                      kernel="chain_kernel (one launch per spec_verify_chain call)",
                      launch_us=launch_ms * 1e3,
                      evented_launch_mean_us=c["mean_ms"] * 1e3, evented_launch_median_us=c["med_ms"] * 1e3,
                      p10_us=float(np.percentile(c["per"], 10)) * 1e3,
                      p90_us=float(np.percentile(c["per"], 90)) * 1e3,
                      alg_bytes_per_call=c["alg_bytes"], rejecting_requests=c["n_rej"],
                      traffic_bytes_per_launch=None if trec is None else trec["bytes_per_launch"],
                      mean_accepted=c["mean_acc"]),
    )
    if not args.no_secondary:
        want = None if args.secondary == "all" else set(args.secondary.split(","))
        sec = line["secondary"] = {}

        def run(name, key, what, fn):
            if want is not None and name not in want:
                return
            torch.cuda.empty_cache()
            log(f"[bench] {what}")
            sec[key] = fn()

        run("greedy", "greedy", "greedy workload", lambda: bench_greedy(args, torch, sv, synth))
        run("tree", "tree", "tree workload", lambda: bench_tree(args, torch, sv, synth))
        run("tree_residual", "tree_residual", "tree with residual updates",
            lambda: bench_tree_residual(args, torch, sv, synth))
        run("tree_greedy", "tree_greedy", "greedy tree", lambda: bench_tree_greedy(args, torch, sv, synth))
        run("chain_stop", "chain_stop", "chain with stop tokens and budgets",
            lambda: bench_chain_stop(args, torch, sv, synth))
        run("chain_bias_mask", "chain_bias_mask", "chain with bias and masks",
            lambda: bench_chain_proc(args, torch, sv, synth, False))
        run("chain_processors", "chain_processors", "chain with every processor",
            lambda: bench_chain_proc(args, torch, sv, synth, True))
        run("chain_sparse", "chain_sparse", "chain with sparse draft rows",
            lambda: bench_chain_sparse(args, torch, sv, synth))
        for k in (3, 2):
            run("chain_lazy", f"chain_lazy{k}", f"chain with lazy rows, groups of {k}",
                lambda: bench_chain_lazy(args, torch, sv, synth, k))
        for k in (0, 3):
            run("chain_f32", f"chain_f32_lazy{k}", f"chain, fp32 logits, lazy rows {k}",
                lambda: bench_chain_lazy(args, torch, sv, synth, k, fp32=True))
        for k in (3, 2, 1):
            run("greedy_lazy", f"greedy_lazy{k}", f"greedy with lazy rows, groups of {k}",
                lambda: bench_greedy_lazy(args, torch, sv, synth, k))
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
