#!/usr/bin/env python3
"""Benchmark of the sparse-gradient compression hot path on one MI355X.

Metric: gradient elements per second of top-1% compress + Rice encode on a
flat fp32 gradient of 2^30 elements (99% ~ Normal(0, 1e-4), 1% ~
Laplace(0, 1e-2)), exact global selection, residual carried across steps,
Rice parameter b = 6 (the optimum at 1% density).  Inputs are synthetic and
resident in HBM before the timed region; two gradients alternate.

One timed step = sgc_compress (residual add, exact top-1%, emit, residual
zeroing) + sgc_encode of its indices.  The JSON line also carries, measured
in the same run: the dominant kernel's roofline (the fused residual-add +
candidate pass, timed with HIP events recorded on its own stream around its
launch), the remaining rows of the path at the same scale (accumulate-only,
exact and sampled compress at 0.1% and 1%, exact compress + encode at 5%,
10% and 25% (the warm-up densities), exact compress with momentum
correction, Rice encode at both densities,
SBC binarize, decode-accumulate of 16 workers' Rice messages), every other
workload on its own shapes (flat 2^20; the MLP with 2-bit messages; the
NMT-style model with its global+local sum; ResNet-50 per tensor with delay,
SBC and Rice: worker step exact and sampled, and the receive step), a grid
of communication delay (1, 10, 100) against kept fraction (25% to 0.1%),
each cell timed as its real sequence of calls, with time and bits per
element per iteration, the warm-up schedule (kept fraction 25% -> 0.1% over
20 carried steps) with per-step time and bits, and the CPU oracle timed on
a bounded sample as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gradient elems/sec (GB/s, % of HBM peak) for top-1% compress+encode at 1 GPU"
PEAK_HBM_GBS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "pass1_flat1G_top1pct_pmc.txt")
# sources the fused pass is compiled from (the 2^30 step takes the window pipeline;
# its tile geometry lives in the header)
PASS_SRCS = [os.path.join(ROOT, "compressed_sgd_amd", "csrc", f) for f in ("compress_window.hip", "sgc_common.h")]


def pass_traffic():
    """HBM bytes per launch of the fused pass from the committed PMC summary,
    or None when the kernel source changed since the counters were taken."""
    return summary_traffic(PMC_FILE, PASS_SRCS)


def timed(fn, reps, stream):
    import torch
    fn()  # workspace allocation and first-touch outside the timed region
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_timed(fn, reps, stream):
    """fn captured once in a HIP graph (after an eager warm-up call) and
    replayed: the launch cost of its kernels leaves the timed region.  Every
    library call in fn passes its own workspace (ws=)."""
    import torch
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / reps


def sparsity_grid(sgc, W, torch, dev, stream, grads, reps=2):
    """Temporal versus gradient sparsity ([SBC] §III; §II Communication
    Delay): communication delay n crossed with the kept fraction p, at the
    full 2^30 elements.  Each cell is timed as the real sequence it stands
    for -- n - 1 accumulate-only calls, then one exchange (exact top-p
    compress + Rice encode) -- with the residual carried, `reps` times, HIP
    events around every sequence.  Per cell: time per training iteration
    (sequence time / n) and the bits sent per element per iteration,
    (Rice position bits + 32 value bits per kept entry) / (n x elements)."""
    N = grads[0].numel()
    L = sgc.Layout([N])
    r = torch.zeros(N, dtype=torch.float32, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    cells = []
    for p in (250000, 100000, 10000, 1000):
        b = sgc.rice_param(p / 1e6)
        c = sgc.compress(L, grads[0], r, keep_ppm=p)
        e = sgc.encode(L, c.idx, c.counts, c.cap, b=b)
        wsc = torch.empty(sgc.compress_workspace_bytes(L, keep_ppm=p), **u8)
        wse = torch.empty(sgc.encode_workspace_bytes(L, sgc.GLOBAL, c.cap), **u8)
        for n_delay in (1, 10, 100):
            it = [0]

            def sequence():
                for _ in range(n_delay - 1):
                    sgc.compress(L, grads[it[0] % 2], r, mode=sgc.ACCUMULATE_ONLY)
                    it[0] += 1
                sgc.compress(L, grads[it[0] % 2], r, keep_ppm=p, out=c, ws=wsc)
                sgc.encode(L, c.idx, c.counts, c.cap, b=b, out=e, ws=wse)
                it[0] += 1
            r.zero_()
            t = timed(sequence, reps, stream)
            cells.append({"delay": n_delay, "keep_pct": p / 1e4, "rice_b": b, "ms_per_sequence": t,
                          "ms_per_iteration": t / n_delay, "kept": c.total(),
                          "bits_per_element_per_iteration": (int(e.nbits[0].item()) + 32.0 * c.total())
                          / (n_delay * N)})
        del c, e, wsc, wse
    return {"elements": N, "timed": "each cell as n - 1 accumulate-only calls + one exchange, residual carried",
            "cells": cells}


def warmup_run(sgc, torch, dev, stream, grads, steps=20, start_ppm=250000, end_ppm=1000):
    """Warm-up training ([SBC] appendix A: the kept fraction falls
    exponentially from 25% to 0.1% over the first epochs) as a carried
    sequence at 2^30 elements: step t keeps sgc_warmup_ppm(t, steps) parts
    per million (exact global selection, residual carried from the step
    before) and Rice-codes them with the parameter that suits that density.
    The schedule runs once on a scratch residual (it sizes every buffer),
    then for real, each step between its own HIP events."""
    N = grads[0].numel()
    L = sgc.Layout([N])
    ppms = [sgc.warmup_ppm(t, steps, start_ppm, end_ppm) for t in range(steps)]
    u8 = dict(dtype=torch.uint8, device=dev)
    cap = max(L.keep_total(sgc.GLOBAL, p) for p in ppms)
    ws_c = torch.empty(max(sgc.compress_workspace_bytes(L, keep_ppm=p) for p in ppms), **u8)
    ws_e = torch.empty(sgc.encode_workspace_bytes(L, sgc.GLOBAL, cap), **u8)
    r = torch.zeros(N, dtype=torch.float32, device=dev)
    comp = sgc.compress(L, grads[0], r, keep_ppm=ppms[0], cap=cap, ws=ws_c)
    enc = None
    for t, p in enumerate(ppms):  # sizing pass
        k = L.keep_total(sgc.GLOBAL, p)
        sgc.compress(L, grads[t % 2], r, keep_ppm=p, cap=k, out=comp, ws=ws_c)
        enc = sgc.encode(L, comp.idx, comp.counts, k, b=sgc.rice_param(p / 1e6), out=enc, ws=ws_e)
    r.zero_()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ppms]
    for t, p in enumerate(ppms):
        k = L.keep_total(sgc.GLOBAL, p)
        a, z = ev[t]
        a.record(stream)
        sgc.compress(L, grads[t % 2], r, keep_ppm=p, cap=k, out=comp, ws=ws_c)
        sgc.encode(L, comp.idx, comp.counts, k, b=sgc.rice_param(p / 1e6), out=enc, ws=ws_e)
        z.record(stream)
        ev[t] = (a, z, comp.counts[-1].clone(), enc.nbits[0].clone())
    torch.cuda.synchronize()
    rows = []
    for t, p in enumerate(ppms):
        a, z, kept, nbits = ev[t]
        kept, nbits = int(kept.item()), int(nbits.item())
        ms = a.elapsed_time(z)
        rows.append({"step": t, "keep_ppm": p, "rice_b": sgc.rice_param(p / 1e6), "kept": kept, "ms": ms,
                     "elements_per_s": N / (ms / 1e3),
                     "alg_GBps": (12.0 * N + 12.0 * kept + nbits / 8.0) / (ms / 1e3) / 1e9,
                     "bits_per_position": nbits / max(kept, 1),
                     "bits_per_element": (nbits + 32.0 * kept) / N})
    total = sum(x["ms"] for x in rows)
    return {"elements": N, "steps": steps, "start_ppm": start_ppm, "end_ppm": end_ppm,
            "schedule": "kept ppm = start * (end/start)^(t/(steps-1)), rounded", "total_ms": total,
            "bits_per_element_total": sum(x["bits_per_element"] for x in rows), "per_step": rows}


def workload_rows(sgc, W, torch, dev, stream, reps=10):
    """Every workload besides the 2^30 one, on its own shapes: the worker step
    (compress exact and sampled, plus the binarize / Rice / delay steps the
    workload uses) and the receive step (decode-accumulate of its workers'
    messages).  Working sets of 4-204 MB fit the 256 MB last-level cache, so
    these report elements/s only, no roofline; the Python binding's launch
    cost is included (small steps can be host-bound)."""
    rows = {}

    def el(n, t):
        return n / (t / 1e3)

    # flat-1M: exact / sampled global top-1%, residual carried over 3 gradients in turn
    w = W.FLAT_1M
    L = sgc.Layout(w.seg_numel)
    n = w.numel
    gs = [W.gradient(w, 0, s, device=dev) for s in range(w.steps)]
    row = {}
    for mode, tag in ((sgc.EXACT, "exact"), (sgc.SAMPLED, "sampled")):
        r = torch.zeros(n, dtype=torch.float32, device=dev)
        c = sgc.compress(L, gs[0], r, mode=mode, keep_ppm=w.keep_ppm)
        it = [0]

        def step():
            sgc.compress(L, gs[it[0] % len(gs)], r, mode=mode, keep_ppm=w.keep_ppm, out=c)
            it[0] += 1
        t = timed(step, reps, stream)
        row[f"compress_{tag}"] = {"ms": t, "elements_per_s": el(n, t), "kept": c.total()}
    # the same step with its Rice encode, replayed from a HIP graph (no launch cost)
    r = torch.zeros(n, dtype=torch.float32, device=dev)
    g_in = gs[0].clone()
    c = sgc.compress(L, g_in, r, keep_ppm=w.keep_ppm)
    bf = sgc.rice_param(w.keep_ppm / 1e6)
    e = sgc.encode(L, c.idx, c.counts, c.cap, b=bf)
    u8 = dict(dtype=torch.uint8, device=dev)
    wsc = torch.empty(sgc.compress_workspace_bytes(L, keep_ppm=w.keep_ppm), **u8)
    wse = torch.empty(sgc.encode_workspace_bytes(L, sgc.GLOBAL, c.cap), **u8)

    def step_enc():
        sgc.compress(L, g_in, r, keep_ppm=w.keep_ppm, out=c, ws=wsc)
        sgc.encode(L, c.idx, c.counts, c.cap, b=bf, out=e, ws=wse)
    t = timed(step_enc, reps, stream)
    tg = graph_timed(step_enc, reps, stream)
    row["compress_encode_exact"] = {"ms": t, "ms_graph": tg, "elements_per_s_graph": el(n, tg)}
    rows[w.name] = row

    # mlp-mnist: global top-1% + 2-bit per worker; 4 raw 2-bit messages summed into zeros
    w = W.MLP_MNIST
    L = sgc.Layout(w.seg_numel)
    n = w.numel
    gs = [W.gradient(w, k, 0, device=dev) for k in range(w.workers)]
    rs = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(w.workers)]
    msgs = []
    for k in range(w.workers):
        c = sgc.compress(L, gs[k], rs[k], keep_ppm=w.keep_ppm, hold=True)
        bn = sgc.binarize(L, c, rs[k], sgc.BIN_2BIT, held=True)
        msgs.append(sgc.Message(sgc.MSG_RAW_2BIT, bn.counts, bn.cap, idx=c.idx, codes=bn.codes, means=bn.means))
    row = {}
    for mode, tag in ((sgc.EXACT, "exact"), (sgc.SAMPLED, "sampled")):
        ct = sgc.compress(L, gs[0], rs[0], mode=mode, keep_ppm=w.keep_ppm)

        def step():
            sgc.compress(L, gs[1], rs[0], mode=mode, keep_ppm=w.keep_ppm, out=ct, hold=True)
            sgc.binarize(L, ct, rs[0], sgc.BIN_2BIT, held=True)
        t = timed(step, reps, stream)
        row[f"worker_step_{tag}"] = {"ms": t, "elements_per_s": el(n, t), "steps": "compress (hold flag) + 2-bit (held)"}
    out = torch.empty(n, dtype=torch.float32, device=dev)
    t = timed(lambda: sgc.decode_accumulate(L, msgs, out), reps, stream)
    row["receive"] = {"ms": t, "elements_per_s": el(n, t), "messages": len(msgs), "format": "raw 2-bit"}
    rows[w.name] = row
    del gs, rs, msgs, out

    # nmt-rnn: global top-1% per worker; 4 raw messages added onto the local gradient
    w = W.NMT_RNN
    L = sgc.Layout(w.seg_numel)
    n = w.numel
    gs = [W.gradient(w, k, 0, device=dev) for k in range(w.workers)]
    msgs = []
    r = torch.zeros(n, dtype=torch.float32, device=dev)
    for k in range(w.workers):
        r.zero_()
        msgs.append(sgc.raw_message(sgc.compress(L, gs[k], r, keep_ppm=w.keep_ppm)))
    row = {}
    for mode, tag in ((sgc.EXACT, "exact"), (sgc.SAMPLED, "sampled")):
        ct = sgc.compress(L, gs[0], r, mode=mode, keep_ppm=w.keep_ppm)
        t = timed(lambda: sgc.compress(L, gs[1], r, mode=mode, keep_ppm=w.keep_ppm, out=ct), reps, stream)
        row[f"compress_{tag}"] = {"ms": t, "elements_per_s": el(n, t), "GBps": 12.0 * n / (t / 1e3) / 1e9}
    out = torch.empty(n, dtype=torch.float32, device=dev)
    t = timed(lambda: sgc.decode_accumulate(L, msgs, out, init=sgc.INIT_BASE, base=gs[0]), reps, stream)
    row["receive_on_local"] = {"ms": t, "elements_per_s": el(n, t), "messages": len(msgs), "format": "raw fp32"}
    rows[w.name] = row
    del gs, msgs, r, out

    # resnet50: 7 delayed accumulations + per-tensor top-0.1% + SBC + per-tensor Rice (b = 9)
    # per worker round; 8 workers' messages summed into zeros
    w = W.RESNET50
    L = sgc.Layout(w.seg_numel)
    n = w.numel
    b = sgc.rice_param(w.keep_ppm / 1e6)
    gs = [W.gradient(w, 0, s, device=dev) for s in range(2)]
    msgs = []
    r = torch.zeros(n, dtype=torch.float32, device=dev)
    for k in range(w.workers):
        r.zero_()
        c = sgc.compress(L, gs[k % 2], r, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm, hold=True)
        bn = sgc.binarize(L, c, r, sgc.BIN_SBC, held=True)
        e = sgc.encode(L, bn.idx, bn.counts, bn.cap, scope=sgc.PER_SEGMENT, b=b)
        msgs.append(sgc.golomb_message(bn, e))
    row = {}
    for mode, tag in ((sgc.EXACT, "exact"), (sgc.SAMPLED, "sampled")):
        ct = sgc.compress(L, gs[0], r, mode=mode, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm)
        u8 = dict(dtype=torch.uint8, device=dev)
        wsc = torch.empty(sgc.compress_workspace_bytes(L, mode=mode, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm), **u8)
        wsb = torch.empty(sgc.binarize_workspace_bytes(L, ct.cap), **u8)
        wse = torch.empty(sgc.encode_workspace_bytes(L, sgc.PER_SEGMENT, ct.cap), **u8)

        def exchange():
            sgc.compress(L, gs[1], r, mode=mode, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm, out=ct, ws=wsc,
                         hold=True)
            bt = sgc.binarize(L, ct, r, sgc.BIN_SBC, ws=wsb, held=True)
            sgc.encode(L, bt.idx, bt.counts, bt.cap, scope=sgc.PER_SEGMENT, b=b, ws=wse)

        def rnd():
            for s_ in range(w.delay - 1):
                sgc.compress(L, gs[s_ % 2], r, mode=sgc.ACCUMULATE_ONLY)
            exchange()
        t = timed(exchange, reps, stream)
        tr = timed(rnd, reps, stream)
        row[f"exchange_{tag}"] = {"ms": t, "elements_per_s": el(n, t), "steps": "compress (hold flag) + SBC (held) + Rice"}
        row[f"round_{tag}"] = {"ms": tr, "steps": f"{w.delay - 1} accumulations + exchange"}
        if mode == sgc.EXACT:  # the same, replayed from a HIP graph
            row[f"exchange_{tag}"]["ms_graph"] = graph_timed(exchange, reps, stream)
            row[f"round_{tag}"]["ms_graph"] = graph_timed(rnd, reps, stream)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    t = timed(lambda: sgc.decode_accumulate(L, msgs, out), reps, stream)
    row["receive"] = {"ms": t, "elements_per_s": el(n, t), "messages": len(msgs), "format": "Rice + SBC mean"}
    rows[w.name] = row
    return rows


def cpu_configs(W, log):
    """The CPU oracle (single-threaded, as it stands) on every workload's own
    shapes: the worker step and the receive step, timed with perf_counter on
    host copies of the same synthetic inputs.  Receive steps sum one worker's
    message W times (the same work as W distinct messages)."""
    import numpy as np
    import oracle as orc

    res = {}

    def clock(f):
        t0 = time.perf_counter()
        out = f()
        return time.perf_counter() - t0, out

    # flat-1M: exact global top-1%, residual carried over 3 steps
    w = W.FLAT_1M
    off = np.array(w.seg_off, np.int64)
    r = np.zeros(w.numel, np.float32)
    ts = []
    for s in range(w.steps):
        g = W.gradient(w, 0, s).numpy()
        ts.append(clock(lambda: orc.compress_exact(g, r, off, orc.GLOBAL, w.keep_ppm))[0])
    res[w.name] = {"worker_step_s": sum(ts) / len(ts), "worker_elements_per_s": w.numel / (sum(ts) / len(ts)),
                   "steps": "compress (exact global 1%)"}
    log(f"[cpu] {w.name} done")
    # mlp-mnist: exact global 1% + 2-bit; receive 4 raw 2-bit messages into zeros
    w = W.MLP_MNIST
    off = np.array(w.seg_off, np.int64)
    g = W.gradient(w, 0, 0).numpy()
    r = np.zeros(w.numel, np.float32)
    t1, sp = clock(lambda: orc.compress_exact(g, r, off, orc.GLOBAL, w.keep_ppm))
    t2, bn = clock(lambda: orc.binarize(sp, len(off) - 1, orc.BIN_2BIT, r))
    msg = orc.Message(bn.counts, vkind=orc.VAL_2BIT, idx=sp.idx, codes=bn.codes, means=bn.means)
    out = np.zeros(w.numel, np.float32)
    t3, _ = clock(lambda: orc.decode_accumulate([msg] * w.workers, off, out))
    res[w.name] = {"worker_step_s": t1 + t2, "worker_elements_per_s": w.numel / (t1 + t2),
                   "receive_s": t3, "receive_elements_per_s": w.numel / t3,
                   "steps": "compress (exact global 1%) + 2-bit; receive 4 raw 2-bit messages"}
    log(f"[cpu] {w.name} done")
    # nmt-rnn: exact global 1%; receive 4 raw messages onto the local gradient
    w = W.NMT_RNN
    off = np.array(w.seg_off, np.int64)
    g = W.gradient(w, 0, 0).numpy()
    r = np.zeros(w.numel, np.float32)
    t1, sp = clock(lambda: orc.compress_exact(g, r, off, orc.GLOBAL, w.keep_ppm))
    out = g.copy()
    msg = orc.Message(sp.counts, idx=sp.idx, val=sp.val)
    t3, _ = clock(lambda: orc.decode_accumulate([msg] * w.workers, off, out))
    res[w.name] = {"worker_step_s": t1, "worker_elements_per_s": w.numel / t1,
                   "receive_s": t3, "receive_elements_per_s": w.numel / t3,
                   "steps": "compress (exact global 1%); receive 4 raw messages onto the local gradient"}
    log(f"[cpu] {w.name} done")
    # resnet50: 7 accumulations + per-tensor 0.1% + SBC + Rice (b = 9); receive 8 messages
    w = W.RESNET50
    off = np.array(w.seg_off, np.int64)
    b = orc.rice_param(w.keep_ppm / 1e6)
    gs = [W.gradient(w, 0, s).numpy() for s in range(w.delay)]
    r = np.zeros(w.numel, np.float32)

    def rnd():
        for s in range(w.delay - 1):
            orc.accumulate(gs[s], r)
        sp = orc.compress_exact(gs[-1], r, off, orc.PER_SEGMENT, w.keep_ppm)
        bn = orc.binarize(sp, len(off) - 1, orc.BIN_SBC, r)
        return bn, orc.encode(bn.idx, bn.counts, off, orc.PER_SEGMENT, b)
    t1, (bn, enc) = clock(rnd)
    msg = orc.Message(bn.counts, vkind=orc.VAL_SBC, golomb=True, scope=orc.PER_SEGMENT, b=b, means=bn.means,
                      enc=enc)
    out = np.zeros(w.numel, np.float32)
    t3, _ = clock(lambda: orc.decode_accumulate([msg] * w.workers, off, out))
    res[w.name] = {"worker_round_s": t1, "worker_elements_per_s": w.numel / t1,
                   "receive_s": t3, "receive_elements_per_s": w.numel / t3,
                   "steps": "7 accumulations + compress (exact per-tensor 0.1%) + SBC + Rice; receive 8 messages"}
    log(f"[cpu] {w.name} done")
    # the 2^30 headline recipe: its first 2^28 elements, exact global top-1% + Rice (b = 6); a
    # second point (besides the benchmark's own 2^26 sample) for the n log n extrapolation to 2^30
    w = W.FLAT_1G
    m = 1 << 28
    g = W.gradient(w, 0, 0, numel=m).numpy()
    r = np.zeros(m, np.float32)
    off = np.array([0, m], np.int64)

    def step28():
        sp = orc.compress_exact(g, r, off, orc.GLOBAL, w.keep_ppm)
        return orc.encode(sp.idx, sp.counts, off, orc.GLOBAL, orc.rice_param(w.keep_ppm / 1e6))
    t1, _ = clock(step28)
    res["flat-2^28-of-1G"] = {"worker_step_s": t1, "worker_elements_per_s": m / t1,
                              "extrapolated_2e30_s": t1 * 4 * (30.0 / 28.0),
                              "steps": "compress (exact global 1%) + Rice b=6 on the first 2^28 elements of the "
                                       "2^30 recipe; 2^30 extrapolated as n log n, not measured"}
    log(f"[cpu] flat-2^28 done")
    return res


RECV_PMC_FILE = os.path.join(ROOT, "profiles", "receive_flat1G_16x1pct_pmc.txt")
RECV_SRCS = [os.path.join(ROOT, "compressed_sgd_amd", "csrc", f) for f in ("accumulate.hip", "sgc_common.h")]


def summary_traffic(path, srcs):
    """HBM bytes per call from a committed PMC summary, or None when a source
    it was taken from has changed since."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    if vals.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def receive_rows(sgc, W, torch, dev, stream, layout, reps=3):
    """a7: decode-accumulate of 16 workers' Rice + fp32 messages (flat 2^30
    recipe, workers 0..15, exact top-1% / top-0.1%) into 4 GiB, onto zeros and
    onto the local dense gradient.  Algorithmic bytes: the dense write (+ the
    dense read of the local gradient) + the messages (code words + 4 B per
    value).  The 1% row onto zeros carries a roofline entry."""
    w = W.FLAT_1G
    n = w.numel
    rows = {}
    r16 = torch.zeros(n, dtype=torch.float32, device=dev)
    outd = torch.empty(n, dtype=torch.float32, device=dev)
    local = W.gradient(w, 0, 0, device=dev)
    for p, tag in ((1000, "0.1pct"), (10000, "1pct")):
        msgs = []
        for wk in range(16):
            g = W.gradient(w, wk, 0, device=dev)
            r16.zero_()
            c = sgc.compress(layout, g, r16, keep_ppm=p)
            e = sgc.encode(layout, c.idx, c.counts, c.cap, b=sgc.rice_param(p / 1e6))
            msgs.append(sgc.golomb_message(c, e))
            del g
        kp = layout.keep_total(sgc.GLOBAL, p)
        msg_bytes = sum(4.0 * kp + 4.0 * int(m.enc.word_off[-1].item()) for m in msgs)
        t = timed(lambda: sgc.decode_accumulate(layout, msgs, outd), reps, stream)
        alg = 4.0 * n + msg_bytes
        rows[f"decode_accumulate_16x{tag}"] = {
            "ms": t, "entries": 16 * kp, "GBps_alg": alg / (t / 1e3) / 1e9}
        if tag == "1pct":
            traffic = summary_traffic(RECV_PMC_FILE, RECV_SRCS)
            achieved = alg / (t / 1e3) / 1e9
            rows[f"decode_accumulate_16x{tag}"]["roofline"] = {
                "kernels": "k_msg_setup, k_msg_decode, k_fill_max, k_fill (one batch of 16), k_merge",
                "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "alg_bytes_per_call": alg, "traffic": traffic,
                "traffic_over_alg": None if traffic is None else traffic / alg}
        t = timed(lambda: sgc.decode_accumulate(layout, msgs, outd, init=sgc.INIT_BASE, base=local), reps, stream)
        rows[f"decode_accumulate_16x{tag}_on_local"] = {
            "ms": t, "entries": 16 * kp, "GBps_alg": (8.0 * n + msg_bytes) / (t / 1e3) / 1e9}
        del msgs
    del r16, outd, local
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample-log2", type=int, default=26)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="only time the CPU oracle on every workload's own shapes (no GPU needed)")
    ap.add_argument("--no-rows", action="store_true", help="skip the extra rows and workloads (e.g. under a profiler)")
    ap.add_argument("--receive-only", action="store_true",
                    help="only the 16-worker decode-accumulate rows at 2^30 (e.g. under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of 2^28 fp32 (1 GiB each way) three times: "
                         "the reference the HBM byte counters are scaled by")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no cross-GPU step); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W

    if args.cpu_configs:
        log = lambda m: print(m, file=sys.stderr, flush=True)
        print(json.dumps({"cpu_configs": cpu_configs(W, log), "cores": 1, "kind": "oracle",
                          "host_cpus": os.cpu_count()}), flush=True)
        return

    import compressed_sgd_amd as sgc

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        x = torch.randn(1 << 28, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.add(x, 0.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": 4 << 28, "launches": 3}))
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.receive_only:
        print(json.dumps({"rows": receive_rows(sgc, W, torch, dev, stream, sgc.Layout(W.FLAT_1G.seg_numel))}),
              flush=True)
        return
    w = W.FLAT_1G
    n = w.numel
    ppm = 10000
    b = sgc.rice_param(ppm / 1e6)
    layout = sgc.Layout(w.seg_numel)
    k = layout.keep_total(sgc.GLOBAL, ppm)
    print(f"[bench] generating 2 x 2^30 gradients (k={k}, b={b})", file=sys.stderr, flush=True)
    grads = [W.gradient(w, 0, s, device=dev) for s in range(2)]
    res = torch.zeros(n, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    comp = sgc.compress(layout, grads[0], res, keep_ppm=ppm)
    enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b)
    res.zero_()

    def step(i):
        sgc.compress(layout, grads[i % 2], res, keep_ppm=ppm, out=comp)
        sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b, out=enc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # per-step HIP events around the fused pass, on the stream it is launched on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, z in ev:
        a.record(stream)
        z.record(stream)
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        sgc.set_pass_events(*ev[i])
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sgc.set_pass_events(None, None)
    ms = e0.elapsed_time(e1) / args.steps
    pass_ms = [a.elapsed_time(z) for a, z in ev]
    pass_avg = sum(pass_ms) / len(pass_ms)
    # per-step times (separate run of the same steps, each bracketed by its own events)
    st_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i, (a, z) in enumerate(st_ev):
        a.record(stream)
        step(args.warmup + args.steps + i)
        z.record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(z) for a, z in st_ev)
    status = int(comp.status.item())
    kept = comp.total()
    nbits = int(enc.nbits[0].item())

    # Rice code length at the page's parameter (b = 7) for the same message
    enc7 = sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=7)
    nbits7 = int(enc7.nbits[0].item())
    del enc7
    # the same 12 B/element stream without any selection work (the library's
    # accumulate-only pass, r <- r + g over the same 2^30 elements): the
    # practical ceiling of the fused pass's access pattern on this GPU
    rs = res.clone()
    stream_ms = timed(lambda: sgc.compress(layout, grads[0], rs, mode=sgc.ACCUMULATE_ONLY), 5, stream)
    del rs

    pass_bytes = 12.0 * n                          # read g, read r, write r
    alg_bytes = 12.0 * n + 8.0 * kept + 4.0 * kept + nbits / 8.0 + 8.0 * ((kept + 255) // 256)
    achieved = pass_bytes / (pass_avg / 1e3) / 1e9
    traffic = pass_traffic()

    out = {
        "metric": METRIC,
        "value": n / (ms / 1e3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded flat fp32 gradient, 99% Normal(0,1e-4) + 1% Laplace(0,1e-2), resident in HBM",
        "config": {
            "workload": "flat-2^30 gradient, exact global top-1% with residual, Rice-coded index gaps (b=6)",
            "n": n, "keep_ppm": ppm, "kept": kept, "mode": "exact", "scope": "global", "rice_b": b,
        },
        "ms_per_step_median": step_ms[len(step_ms) // 2],
        "ms_per_step_min": step_ms[0],
        "alg_GBps": alg_bytes / (ms / 1e3) / 1e9,
        "alg_frac_of_8TBps": alg_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "bits_per_position": nbits / max(kept, 1),
        "bits_per_position_b7": nbits7 / max(kept, 1),
        "compression_ratio_vs_dense_fp32": 32.0 * n / (nbits + 32.0 * kept),
        "status": status,
        "wall_s_timed": wall,
        "roofline": {
            "kernel": "k_pass1 (fused residual add + candidate emission)",
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
            "alg_bytes_per_launch": pass_bytes, "avg_launch_ms": pass_avg,
            "traffic_over_alg": None if traffic is None else traffic / pass_bytes,
            "same_pattern_stream_GBps": pass_bytes / (stream_ms / 1e3) / 1e9,
        },
    }

    if not args.no_rows:
        rows = {}
        # a1: accumulate-only (communication delay), 12 B/elem
        t = timed(lambda: sgc.compress(layout, grads[0], res, mode=sgc.ACCUMULATE_ONLY), 5, stream)
        rows["accumulate_only"] = {"ms": t, "GBps": 12.0 * n / (t / 1e3) / 1e9}
        # compress alone and encode alone
        t = timed(lambda: sgc.compress(layout, grads[1], res, keep_ppm=ppm, out=comp), 5, stream)
        rows["compress_exact_1pct"] = {"ms": t, "GBps": (12.0 * n + 8.0 * kept) / (t / 1e3) / 1e9}
        t = timed(lambda: sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b, out=enc), 5, stream)
        rows["encode_1pct"] = {"ms": t, "codes": kept}
        # exact mode at 0.1% (compress, then Rice encode at that density's parameter)
        c01 = sgc.compress(layout, grads[1], res, keep_ppm=1000)
        b01 = sgc.rice_param(1000 / 1e6)
        t = timed(lambda: sgc.compress(layout, grads[1], res, keep_ppm=1000, out=c01), 5, stream)
        rows["compress_exact_0.1pct"] = {"ms": t, "GBps": (12.0 * n + 8.0 * c01.total()) / (t / 1e3) / 1e9,
                                         "kept": c01.total()}
        e01 = sgc.encode(layout, c01.idx, c01.counts, c01.cap, b=b01)
        t = timed(lambda: sgc.encode(layout, c01.idx, c01.counts, c01.cap, b=b01, out=e01), 5, stream)
        rows["encode_0.1pct"] = {"ms": t, "codes": c01.total(), "rice_b": b01,
                                 "bits_per_position": int(e01.nbits[0].item()) / max(c01.total(), 1)}
        del c01, e01
        # density sweep (warm-up sparsity runs from 25% down to 0.1%): exact compress + Rice encode
        for p in (250000, 100000, 50000):
            cp = sgc.compress(layout, grads[1], res, keep_ppm=p)
            tp = timed(lambda: sgc.compress(layout, grads[1], res, keep_ppm=p, out=cp), 3, stream)
            bp = sgc.rice_param(p / 1e6)
            ep = sgc.encode(layout, cp.idx, cp.counts, cp.cap, b=bp)
            te = timed(lambda: sgc.encode(layout, cp.idx, cp.counts, cp.cap, b=bp, out=ep), 3, stream)
            rows[f"compress_encode_exact_{p / 1e4:g}pct"] = {
                "compress_ms": tp, "encode_ms": te, "kept": cp.total(), "rice_b": bp,
                "compress_GBps": (12.0 * n + 8.0 * cp.total()) / (tp / 1e3) / 1e9,
                "bits_per_position": int(ep.nbits[0].item()) / max(cp.total(), 1)}
            del cp, ep
        # momentum correction + masking, exact top-1%: 20 B/elem (g, r, u read; r, u written)
        mom = torch.zeros(n, dtype=torch.float32, device=dev)
        cm = sgc.compress_momentum(layout, grads[0], mom, res, 0.9, keep_ppm=ppm)
        t = timed(lambda: sgc.compress_momentum(layout, grads[1], mom, res, 0.9, keep_ppm=ppm, out=cm), 5, stream)
        rows["compress_momentum_exact_1pct"] = {"ms": t, "GBps": (20.0 * n + 12.0 * kept) / (t / 1e3) / 1e9,
                                                "beta": 0.9}
        del mom, cm
        # sampled-threshold mode at 0.1% and 1%
        for p, name in ((1000, "compress_sampled_0.1pct"), (10000, "compress_sampled_1pct")):
            cs = sgc.compress(layout, grads[0], res, keep_ppm=p, mode=sgc.SAMPLED)
            t = timed(lambda: sgc.compress(layout, grads[0], res, keep_ppm=p, mode=sgc.SAMPLED, out=cs), 5, stream)
            rows[name] = {"ms": t, "GBps": 12.0 * n / (t / 1e3) / 1e9, "kept": cs.total()}
        # a5: SBC binarize of a 1% message (one segment)
        sgc.compress(layout, grads[0], res, keep_ppm=ppm, out=comp)
        rsave = res.clone()
        t = timed(lambda: sgc.binarize(layout, comp, res, sgc.BIN_SBC), 5, stream)
        rows["binarize_sbc_1pct"] = {"ms": t, "entries": kept}
        # the same after compress with the hold flag: only the sent side is written
        res.copy_(rsave)
        sgc.compress(layout, grads[0], res, keep_ppm=ppm, out=comp, hold=True)
        t = timed(lambda: sgc.binarize(layout, comp, res, sgc.BIN_SBC, held=True), 5, stream)
        rows["binarize_sbc_1pct_held"] = {"ms": t, "entries": kept}
        res.copy_(rsave)
        del rsave
        rows.update(receive_rows(sgc, W, torch, dev, stream, layout))
        out["rows"] = rows
        print("[bench] the other workloads", file=sys.stderr, flush=True)
        out["workloads"] = workload_rows(sgc, W, torch, dev, stream)
        print("[bench] warm-up schedule 25% -> 0.1% over 20 steps", file=sys.stderr, flush=True)
        out["warmup_schedule"] = warmup_run(sgc, torch, dev, stream, grads)
        print("[bench] temporal x gradient sparsity grid", file=sys.stderr, flush=True)
        out["sparsity_grid"] = sparsity_grid(sgc, W, torch, dev, stream, grads)

    if not args.no_cpu_baseline:
        import oracle as orc
        m = 1 << args.cpu_sample_log2
        g0 = grads[0][:m].cpu().numpy()
        r0 = np.zeros(m, np.float32)
        print(f"[bench] oracle on the first 2^{args.cpu_sample_log2} elements", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        sp = orc.compress_exact(g0, r0, np.array([0, m], np.int64), orc.GLOBAL, ppm)
        orc.encode(sp.idx, sp.counts, np.array([0, m], np.int64), orc.GLOBAL, b)
        dt = time.perf_counter() - t0
        # the full sort dominates: n log n from the sample size to the headline's 2^30
        L2 = args.cpu_sample_log2
        scale = (n / m) * (30.0 / L2)
        out["cpu_baseline"] = {
            "value": m / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"first 2^{L2} elements of the step-0 gradient: exact top-1% "
                      f"(full sort) + Rice b={b} encode, single-threaded C oracle ({dt:.1f} s)",
            "host_cpus": os.cpu_count(),
            "extrapolated_2e30": {"value": n / (dt * scale), "seconds": dt * scale,
                                  "how": f"n log n extrapolation from the 2^{L2} measurement (x{scale:.2f}), "
                                         "not measured"},
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
