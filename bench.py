#!/usr/bin/env python3
"""Gated-prefill benchmark on one MI355X.

Default workload (stage_32k): the full gated-prefill stage at Qwen3-1.7B
shape -- N = 32768 tokens (r = 64 question tokens), d = 2048 bf16 residual,
gate MLP 2048 -> 256 -> 1, K = 3277 (10 %) kept, then 24 upper-layer
token-gated causal GQA attention calls (16q / 8kv heads, d_h 128) on the
compacted stream.

One step = one pass of the whole path over one input:
    tg_gate_score -> tg_gate_select (sequence norm, top-K, compaction)
    -> 24 x tg_gated_attention
(--separate-gate runs tg_seq_rmsnorm, tg_topk_select and tg_compact instead
of tg_gate_select; the results are the same bit for bit)
with every input already resident in HBM.  Calls are launched directly on
one stream with no host synchronisation; --graph captures each phase of a
step (each gate call, the run of attention calls) once as a HIP graph and
replays it instead.  The residual is rotated over
several copies (> the 256 MiB Infinity Cache) so the HBM-bound kernels read
HBM.  The per-layer Q/K/V are the upper layers' projections of the compacted
stream (seeded random weights); they are produced before the timed region by
plain bf16 GEMMs outside the library and are timed separately ("glue").

Prints ONE JSON line: tokens/s = N / (GPU time per step), the roofline of
the dominant kernel (gated attention, bf16 MFMA), per-kernel figures and the
CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated-prefill tokens/s at N=16k–128k; HBM GB/s % and MFMA % of peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(kernel_file: str):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they
    were taken on the current source of the kernel; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
        src = os.path.join(ROOT, "learned_token_pruning_07_amd", "csrc", kernel_file)
        ent = t.get(kernel_file)
        if not ent or ent.get("source_sha256") != _sha(src):
            return None
        return float(ent["bytes_per_launch"])
    except Exception:
        return None


class Events:
    """HIP events on torch's current stream (the stream the library launches
    on) at the boundaries between the phases of a step: one event ends a phase
    and starts the next, so a step records 6 events rather than a pair per
    call (each record costs a few microseconds of GPU time between kernels).
    A phase is one library call, or the run of consecutive calls of one entry
    point; its per-call average is the phase time over the calls it holds."""

    def __init__(self, torch):
        self.torch = torch
        self.spans = {}   # name -> [(start_event, end_event, calls)]
        self.last = None

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.last = e
        return e

    def phase(self, name, fn, calls=1):
        a = self.last if self.last is not None else self.mark()
        r = fn()
        b = self.mark()
        self.spans.setdefault(name, []).append((a, b, calls))
        return r

    def avg_us(self, name):
        ps = self.spans.get(name, [])
        n = sum(c for _, _, c in ps)
        return 1000.0 * sum(a.elapsed_time(b) for a, b, _ in ps) / max(1, n)

    def count(self, name):
        return sum(c for _, _, c in self.spans.get(name, []))


def time_backward(torch, tg, qkv, b_S, kept_idx, layer, attn_out, heads, M, stream_reps=20):
    """The backward of one token-gated attention layer at the stage's shape,
    timed on its own (it is not part of the prefill step): the layer's
    forward gives O and lse, a seeded bf16 upstream gradient stands in for
    the loss, and HIP events on the launch stream bracket `stream_reps`
    back-to-back calls.  Algorithmic work: the five products of the usual
    flash-attention backward (S, dP, dV, dK, dQ), 2.5x the forward's flops."""
    q, k, v = qkv
    Hq, Hkv, dh = heads["Hq"], heads["Hkv"], heads["dh"]
    out, lse = tg.tg_gated_attention(q, k, v, b_S, kept_idx, layer.gain, layer.temp, want_lse=True)
    g = torch.Generator(device=q.device).manual_seed(1234)
    d_out = torch.randn(q.shape, generator=g, device=q.device).bfloat16()
    ws = tg.attention_backward_workspace(1, M, Hq, Hkv, dh, q.device)
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty((1, M), device=q.device), torch.empty(Hq, device=q.device), torch.empty(Hq, device=q.device)]
    call = lambda: tg.tg_gated_attention_backward(q, k, v, out, lse, d_out, b_S, kept_idx, layer.gain,  # noqa: E731
                                                  layer.temp, None, *grads, ws=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(stream_reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / stream_reps
    flops = 5 * dh * Hq * M * (M + 1)
    tf = flops / (us * 1e-6) / 1e12
    return {"call": "tg_gated_attention_backward", "avg_us": round(us, 3), "calls_timed": stream_reps,
            "algorithmic_flops": flops, "achieved_TFLOPs": round(tf, 2),
            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "shape": {"M": M, "Hq": Hq, "Hkv": Hkv, "d_h": dh}}


def time_varlen(torch, tg, layer, heads, M, n_seq=16, reps=20):
    """Token-gated attention over a packed batch of `n_seq` gated prompts
    (kept lengths uniform in [M/8, M], seeded; random bf16 q, k, v, scores and
    sorted original positions), timed on its own: one tg_gated_attention_varlen
    call, and for context the same sequences as one batch-of-one
    tg_gated_attention call each.  Algorithmic work: the forward's two causal
    products per sequence, 2 d_h Hq m (m + 1) flops."""
    Hq, Hkv, dh = heads["Hq"], heads["Hkv"], heads["dh"]
    g = torch.Generator().manual_seed(2468)
    lens = torch.randint(max(M // 8, 1), M + 1, (n_seq,), generator=g).tolist()
    cu = [0]
    for m in lens:
        cu.append(cu[-1] + m)
    T = cu[-1]
    dev = layer.gain.device
    q = torch.randn((T, Hq, dh), generator=g).bfloat16().to(dev)
    k = torch.randn((T, Hkv, dh), generator=g).bfloat16().to(dev)
    v = torch.randn((T, Hkv, dh), generator=g).bfloat16().to(dev)
    ks = torch.randn(T, generator=g).to(dev)
    pos = torch.cat([torch.sort(torch.randperm(4 * m, generator=g)[:m]).values for m in lens]).int().to(dev)
    out = torch.empty_like(q)
    ws = tg.attention_workspace(1, T + 63 * n_seq, Hq, Hkv, dh, dev)
    packed = lambda: tg.tg_gated_attention_varlen(q, k, v, cu, ks, pos, layer.gain, layer.temp,  # noqa: E731
                                                  out=out, ws=ws)
    views = [(q[None, a:b], k[None, a:b], v[None, a:b], ks[None, a:b], pos[None, a:b], out[None, a:b])
             for a, b in zip(cu[:-1], cu[1:])]

    def per_sequence():
        for qq, kk, vv, ss, pp, oo in views:
            tg.tg_gated_attention(qq, kk, vv, ss, pp, layer.gain, layer.temp, out=oo, ws=ws)

    res = {}
    for name, call in (("avg_us", packed), ("per_sequence_calls_us", per_sequence)):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / reps, 3)
    flops = sum(2 * dh * Hq * m * (m + 1) for m in lens)
    tf = flops / (res["avg_us"] * 1e-6) / 1e12
    return {"call": "tg_gated_attention_varlen", "avg_us": res["avg_us"], "calls_timed": reps,
            "per_sequence_calls_us": res["per_sequence_calls_us"], "algorithmic_flops": flops,
            "achieved_TFLOPs": round(tf, 2), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "shape": {"sequences": n_seq, "rows": T, "min_M": min(lens), "max_M": max(lens), "Hq": Hq,
                      "Hkv": Hkv, "d_h": dh}}


STAGE_GATE_LAYER = 4  # the stage workload's gate layer L: layers 0..L hold full-length KV caches


def time_kv_prune(torch, tg, kept_idx, N, M, heads, n_layers, reps=20):
    """Post-prefill pruning of the K/V caches of layers 0..L (seeded bf16
    caches of the prompt length N) to the stage's kept set, timed on its own
    (it runs once after prefill, outside the step).  Algorithmic bytes: every
    kept row read once and written once, K and V, every layer."""
    Hkv, dh = heads["Hkv"], heads["dh"]
    g = torch.Generator(device=kept_idx.device).manual_seed(4321)
    shape = (n_layers, 1, N, Hkv, dh)
    kc = torch.randn(shape, generator=g, device=kept_idx.device).bfloat16()
    vc = torch.randn(shape, generator=g, device=kept_idx.device).bfloat16()
    ko = torch.empty((n_layers, 1, M, Hkv, dh), dtype=torch.bfloat16, device=kept_idx.device)
    vo = torch.empty_like(ko)
    call = lambda: tg.tg_kv_cache_prune(kc, vc, kept_idx, k_out=ko, v_out=vo)  # noqa: E731
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = 2 * 2 * n_layers * M * Hkv * dh * 2 + 4 * M * 2 * n_layers
    gbs = nbytes / (us * 1e-6) / 1e9
    del kc, vc
    return {"call": "tg_kv_cache_prune", "avg_us": round(us, 3), "calls_timed": reps, "layers": n_layers,
            "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "shape": {"N": N, "M": M, "Hkv": Hkv, "d_h": dh}}


def cpu_baseline(c, layer0_qkv, kept_idx, b_S, gain, temp, n_layers, max_rows=1024):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    t0 = time.perf_counter()
    raw = oracle.gate_score(c.resid, c.r, c.norm_w, c.W1, c.b1, c.w2, c.b2, c.eps_row)
    b = oracle.seq_rmsnorm(raw, c.r, c.eps_seq)
    keep = oracle.topk_select(b.astype(np.float32), c.r, c.K)
    oracle.compact(c.resid, keep, b.astype(np.float32))
    t_gate = time.perf_counter() - t0
    q, k, v = layer0_qkv
    M = q.shape[1]
    R = min(M, max_rows)
    rows = np.linspace(0, M - 1, R).astype(np.int64)
    t0 = time.perf_counter()
    oracle.gated_attention(q, k, v, b_S, kept_idx, gain, temp, q.shape[-1] ** -0.5, rows=rows)
    t_rows = time.perf_counter() - t0
    t_layer = t_rows * M / R
    per_step = t_gate + n_layers * t_layer
    return {
        "value": c.N / per_step, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"gate (score, seq-norm, top-K, compaction) on the full N={c.N} input: {t_gate:.2f} s; "
                   f"one attention layer on {R} of {M} query rows (all {q.shape[2]} heads): {t_rows:.2f} s, "
                   f"extrapolated linearly to {M} rows x {n_layers} layers"),
        "seconds_per_step": per_step,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stage_32k", choices=["stage_32k", "gate_16k", "sweep_128k"])
    ap.add_argument("--frac", type=float, default=0.10, help="budget fraction for sweep_128k")
    ap.add_argument("--layers", type=int, default=None, help="upper layers (default: 24 for stage_32k, else 1)")
    ap.add_argument("--copies", type=int, default=0, help="residual copies rotated per step (0: enough for 512 MiB)")
    ap.add_argument("--separate-gate", action="store_true",
                    help="run sequence norm, top-K and compaction as three calls instead of tg_gate_select")
    ap.add_argument("--graph", action="store_true",
                    help="capture each phase of a step as a HIP graph once and replay it (slower on this ROCm: "
                         "a replay costs several microseconds more than direct launches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv-prune", action="store_true",
                    help="skip the separate timing of tg_kv_cache_prune (layers 0..L of the stage)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed varying-length attention timing")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the separate timing of tg_gated_attention_backward at the attention shape")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB (5 times): the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: the gated-prefill path is measured on one MI355X only; a multi-GPU run is not "
              "implemented (the batch and head dimensions shard without communication). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import learned_token_pruning_07_amd as tg
    from learned_token_pruning_07_amd import stage_glue
    from learned_token_pruning_07_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 5}), flush=True)
        return
    tg.load_library()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------- inputs ----------------
    if args.workload == "stage_32k":
        c = wl.preset_gate_case("stage_32k")
        n_layers = 24 if args.layers is None else args.layers
    elif args.workload == "gate_16k":
        c = wl.preset_gate_case("gate_16k")
        n_layers = 0 if args.layers is None else args.layers
    else:
        c = wl.preset_gate_case("sweep_128k", K=int(round(args.frac * (131072 - 128))))
        n_layers = 1 if args.layers is None else args.layers
    N, r, K, d, h, M = c.N, c.r, c.K, c.d, c.h, c.M
    heads = wl.STAGE_HEADS
    log(f"workload {args.workload}: N={N} r={r} K={K} M={M} d={d} h={h} layers={n_layers}")

    def bits(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    resid0 = bits(c.resid)
    row_bytes = d * 2
    ncopy = args.copies or max(1, -(-(512 << 20) // (N * row_bytes)))
    resids = [resid0] + [resid0.clone() for _ in range(ncopy - 1)]
    norm_w, W1, w2 = bits(c.norm_w), bits(c.W1), bits(c.w2)
    b1, b2 = torch.from_numpy(c.b1).to(dev), torch.from_numpy(c.b2).to(dev)
    # preallocated outputs: nothing is allocated inside a step
    score = torch.empty((1, N), dtype=torch.float32, device=dev)
    keep = torch.empty((1, N), dtype=torch.uint8, device=dev)
    kept_idx = torch.empty((1, M), dtype=torch.int32, device=dev)
    resid_S = torch.empty((1, M, d), dtype=torch.bfloat16, device=dev)
    b_S = torch.empty((1, M), dtype=torch.float32, device=dev)
    gate_ws = tg.gate_workspace(h, d, dev)
    seq_ws = tg.seq_rmsnorm_workspace(1, N, dev)   # None up to N = 32768
    topk_ws = tg.topk_workspace(1, N, dev)
    sel_ws = tg.gate_select_workspace(1, N, dev)   # None up to N = 32768
    sel_phases = ("seq_rmsnorm", "topk_select", "compact") if args.separate_gate else ("gate_select",)

    def gate_calls(x):
        """The gate's library calls on residual x, as (phase name, call)."""
        calls = [("gate_score", lambda: tg.tg_gate_score(x, r, norm_w, W1, b1, w2, b2, c.eps_row, score_raw=score,
                                                          ws=gate_ws))]
        if args.separate_gate:
            calls += [("seq_rmsnorm", lambda: tg.tg_seq_rmsnorm(score, r, c.eps_seq, score=score, ws=seq_ws)),
                      ("topk_select", lambda: tg.tg_topk_select(score, r, K, keep=keep, ws=topk_ws)),
                      ("compact", lambda: tg.tg_compact(x, keep, score, M, kept_idx=kept_idx, resid_out=resid_S,
                                                         score_out=b_S))]
        else:
            calls += [("gate_select", lambda: tg.tg_gate_select(score, x, r, K, c.eps_seq, score=score, keep=keep,
                                                                 kept_idx=kept_idx, resid_out=resid_S,
                                                                 score_out=b_S, ws=sel_ws))]
        return calls

    for _, fn in gate_calls(resid0):
        fn()
    torch.cuda.synchronize()

    # upper-layer Q/K/V (glue, outside the library and outside the timed step)
    layers = stage_glue.stage_layers(n_layers, d, **heads) if n_layers else []
    qkv = [p.qkv(resid_S) for p in layers]
    attn_out = torch.empty((1, M, heads["Hq"], heads["dh"]), dtype=torch.bfloat16, device=dev)
    attn_ws = tg.attention_workspace(1, M, heads["Hq"], heads["Hkv"], heads["dh"], dev)
    torch.cuda.synchronize()
    glue_ms = 0.0
    if layers:
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for p in layers:
            p.qkv(resid_S)
        g0.record()
        for _ in range(3):
            for p in layers:
                p.qkv(resid_S)
        g1.record()
        torch.cuda.synchronize()
        glue_ms = g0.elapsed_time(g1) / 3

    def attention_layers():
        for l, p in enumerate(layers):
            q, k, v = qkv[l]
            tg.tg_gated_attention(q, k, v, b_S, kept_idx, p.gain, p.temp, out=attn_out, ws=attn_ws)

    def step_phases(i):
        """(phase name, call, library calls in it) of step i; the residual copy rotates."""
        ph = [(name, fn, 1) for name, fn in gate_calls(resids[i % ncopy])]
        if layers:
            ph.append(("gated_attention", attention_layers, len(layers)))
        return ph

    graphs = {}
    if args.graph:
        # each phase of a step is captured once as a HIP graph (per residual
        # copy for the gate phases) and replayed; events between the replays
        # time the phases.  The calls allocate nothing, so capture is legal.
        for i in range(ncopy):  # eager warm-up of every call shape first
            for _, fn, _ in step_phases(i):
                fn()
        torch.cuda.synchronize()
        for i in range(ncopy):
            for name, fn, _ in step_phases(i):
                key = (i if name != "gated_attention" else 0, name)
                if key not in graphs:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        fn()
                    graphs[key] = g
        torch.cuda.synchronize()

    def step(i, ev=None):
        for name, fn, calls in step_phases(i):
            if graphs:
                fn = graphs[(i % ncopy if name != "gated_attention" else 0, name)].replay
            if ev:
                ev.phase(name, fn, calls=calls)
            else:
                fn()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---------------- timed region ----------------
    # events at the phase boundaries of every step give per-call durations on
    # the library's stream; the first and last of them bracket the K steps
    ev = Events(torch)
    torch.cuda.synchronize()
    t_start = ev.mark()
    for i in range(args.steps):
        step(i, ev)
    t_end = ev.last
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    log(f"{ms_per_step:.4f} ms/step over {args.steps} steps ({ncopy} residual copies, "
        f"{'HIP graph replays' if args.graph else 'direct launches'})")

    # ---------------- figures ----------------
    e = 2
    P = N - r
    algo = {"gate_score": dict(bytes=P * d * e + h * d * e + 4 * N, flops=2 * P * d * h, bound="hbm")}
    if args.separate_gate:
        algo["seq_rmsnorm"] = dict(bytes=4 * P + 4 * N, flops=2 * P, bound="latency")
        algo["topk_select"] = dict(bytes=4 * P + N, flops=0, bound="latency")
        algo["compact"] = dict(bytes=N + 2 * M * d * e + 12 * M, flops=0, bound="hbm")
    else:
        # raw scores in, normalised scores, keep mask, kept_idx and kept scores
        # out, kept_idx read back by the gather, kept rows read and written
        algo["gate_select"] = dict(bytes=4 * P + 4 * N + N + 12 * M + 2 * M * d * e, flops=2 * P, bound="latency")
    if layers:
        Hq, Hkv, dh = heads["Hq"], heads["Hkv"], heads["dh"]
        algo["gated_attention"] = dict(bytes=M * dh * e * (2 * Hq + 2 * Hkv) + 8 * M,
                                       flops=2 * dh * Hq * M * (M + 1), bound="mfma")
    kernels = {}
    for name, a in algo.items():
        us = ev.avg_us(name)
        ent = {"avg_us": round(us, 3), "launches_per_step": ev.count(name) // args.steps,
               "algorithmic_bytes": a["bytes"], "algorithmic_flops": a["flops"]}
        gbs = a["bytes"] / (us * 1e-6) / 1e9
        ent["achieved_GBs"] = round(gbs, 1)
        ent["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4)
        if a["flops"]:
            tf = a["flops"] / (us * 1e-6) / 1e12
            ent["achieved_TFLOPs"] = round(tf, 2)
            ent["mfma_frac"] = round(tf / PEAK_BF16_TFLOPS, 4)
        kernels[name] = ent
    kernel_us_sum = sum(kernels[n]["avg_us"] * kernels[n]["launches_per_step"] for n in kernels)
    gate_us = sum(kernels[n]["avg_us"] for n in ("gate_score",) + sel_phases)
    gate_bytes = sum(algo[n]["bytes"] for n in ("gate_score",) + sel_phases)

    if layers:
        dom, dom_file = "gated_attention", "gated_attention.hip"
        a = kernels[dom]
        roofline = {"kernel": dom, "bound": "mfma", "achieved": a["achieved_TFLOPs"], "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": a["mfma_frac"], "traffic": None}
    else:
        dom, dom_file = "gate_score", "gate_score.hip"
        a = kernels[dom]
        roofline = {"kernel": dom, "bound": "hbm", "achieved": a["achieved_GBs"], "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": a["hbm_frac"], "traffic": None}
    roofline["traffic"] = _traffic(dom_file)

    value = N / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded PCG64 draws with the workload's shapes and distributions",
        "config": {"workload": args.workload, "N": N, "r": r, "K": K, "M": M, "d": d, "h": h, "layers": n_layers,
                   "Hq": heads["Hq"], "Hkv": heads["Hkv"], "d_h": heads["dh"], "batch": 1,
                   "residual_copies": ncopy},
        "roofline": roofline,
        "kernels": kernels,
        "launch": "hip_graph" if args.graph else "direct",
        "gate_op": {"calls": ["tg_gate_score"] + ["tg_" + n for n in sel_phases],
                    "avg_us": round(gate_us, 3), "algorithmic_bytes": gate_bytes,
                    "achieved_GBs": round(gate_bytes / (gate_us * 1e-6) / 1e9, 1),
                    "hbm_frac": round(gate_bytes / (gate_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "library_kernel_tokens_per_s": round(N / (kernel_us_sum * 1e-6), 1),
        "glue_qkv_ms_per_step": round(glue_ms, 4),
        "tokens_per_s_with_glue": round(N / ((ms_per_step + glue_ms) * 1e-3), 1),
    }

    if layers and not args.no_varlen:
        out["varlen_attention"] = time_varlen(torch, tg, layers[0], heads, M)
    if layers and not args.no_backward:
        out["attention_backward"] = time_backward(torch, tg, qkv[0], b_S, kept_idx, layers[0], attn_out, heads, M,
                                                  stream_reps=20)
        log(f"attention backward: {out['attention_backward']['avg_us']:.2f} us per call")

    if layers and not args.no_kv_prune and args.workload == "stage_32k":
        out["kv_cache_prune"] = time_kv_prune(torch, tg, kept_idx, N, M, heads, n_layers=STAGE_GATE_LAYER + 1)
        log(f"kv cache prune: {out['kv_cache_prune']['avg_us']:.2f} us per call")

    if not args.no_cpu_baseline and layers:
        log("timing the CPU oracle on a bounded sample")
        q, k, v = qkv[0]
        host = lambda t: t.detach().cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
        out["cpu_baseline"] = cpu_baseline(c, (host(q), host(k), host(v)), kept_idx.cpu().numpy(),
                                           b_S.cpu().numpy(), layers[0].gain.cpu().numpy(),
                                           layers[0].temp.cpu().numpy(), n_layers)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
