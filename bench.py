#!/usr/bin/env python3
"""Gated-prefill benchmark on one MI355X.

Default workload (stage_32k): the full gated-prefill stage at Qwen3-1.7B
shape -- N = 32768 tokens (r = 64 question tokens), d = 2048 bf16 residual,
gate MLP 2048 -> 256 -> 1, K = 3277 (10 %) kept, then 24 upper-layer
token-gated causal GQA attention calls (16q / 8kv heads, d_h 128) on the
compacted stream.

One step = one pass of the whole path over one input:
    tg_gate_score_folded -> tg_gate_select (sequence norm, top-K, compaction)
    -> 24 x tg_gated_attention
(the scorer's first-layer weights are folded with the RMSNorm weight once,
by tg_gate_fold_weights, as a model would at load time)
(--separate-gate runs tg_seq_rmsnorm, tg_topk_select and tg_compact instead
of tg_gate_select; the results are the same bit for bit)
with every input already resident in HBM.  Calls are launched directly on
one stream with no host synchronisation; --graph also captures each whole
step once as one HIP graph from the padded entry points (the budget read
from device memory, launches sized by the kept length padded to a multiple
of 256, as one graph per padded length serves every budget of its bucket)
and times its replays.  The residual is rotated over
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


# every source a call's kernels are compiled from, beyond its own file
PROFILE_DEPS = {
    "gated_attention.hip": ["rope_device.h", "tg_device.h"],
    "gate_score.hip": ["gate_select_row.h", "select_device.h", "row_gather.h", "compact.hip", "tg_device.h"],
    "gate_select.hip": ["gate_select_row.h", "select_device.h", "row_gather.h", "compact.hip", "tg_device.h"],
    "gated_attention_bwd.hip": ["rope_device.h", "tg_device.h"],
    "kv_prune.hip": ["row_gather.h", "tg_device.h"],
}


def _sources_sha(kernel_file: str):
    """sha256 over the kernel file and the sources it depends on."""
    d = os.path.join(ROOT, "learned_token_pruning_07_amd", "csrc")
    files = [kernel_file] + PROFILE_DEPS.get(kernel_file, [])
    return hashlib.sha256("".join(_sha(os.path.join(d, f)) for f in files).encode()).hexdigest()


def _traffic(kernel_file: str):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they
    were taken on the current sources of the kernel; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
        ent = t.get(kernel_file)
        if not ent or ent.get("sources_sha256") != _sources_sha(kernel_file):
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


def time_rope(torch, tg, qkv, b_S, kept_idx, layer, heads, M, base=1e6, reps=20, rounds=3):
    """The rotary variant of one attention layer beside the plain call, at the
    stage's shape: q and k turned by the kept tokens' original positions
    (kept_idx) inside the call.  Rounds of `reps` plain calls, then `reps`
    rotary calls, alternate on the launch stream (HIP events around each
    block); the best round of each is reported, and their ratio."""
    q, k, v = qkv
    Hq, Hkv, dh = heads["Hq"], heads["Hkv"], heads["dh"]
    out = torch.empty((1, M, Hq, dh), dtype=torch.bfloat16, device=q.device)
    ws_p = tg.attention_workspace(1, M, Hq, Hkv, dh, q.device)
    ws_r = tg.attention_rope_workspace(1, M, Hq, Hkv, dh, q.device)
    plain = lambda: tg.tg_gated_attention(q, k, v, b_S, kept_idx, layer.gain, layer.temp, out=out,  # noqa: E731
                                          ws=ws_p)
    rope = lambda: tg.tg_gated_attention_rope(q, k, v, b_S, kept_idx, layer.gain, layer.temp, base,  # noqa: E731
                                              out=out, ws=ws_r)
    for fn in (plain, rope, plain, rope):
        fn()
    torch.cuda.synchronize()
    best = {"plain": float("inf"), "rope": float("inf")}
    for _ in range(rounds):
        for name, fn in (("plain", plain), ("rope", rope)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            best[name] = min(best[name], e0.elapsed_time(e1) * 1e3 / reps)
    flops = 2 * dh * Hq * M * (M + 1)
    return {"call": "tg_gated_attention_rope", "rope_base": base, "plain_us": round(best["plain"], 3),
            "rope_us": round(best["rope"], 3), "rope_over_plain": round(best["rope"] / best["plain"], 4),
            "rope_mfma_frac": round(flops / (best["rope"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "calls_per_round": reps, "rounds": rounds}


def time_fused_gate(torch, tg, resids, c, W1f, b1, w2, b2, reps=20, rounds=3):
    """The whole gate as one tg_gate call (the scorer whose last workgroup of
    each batch row runs that row's selection, then the gather) beside the
    separate calls the step makes (tg_gate_score_folded, tg_gate_select), at
    the step's shape: rounds of `reps` calls of each alternate on the launch
    stream, the best round of each is reported, and the outputs of the two
    are compared bit for bit."""
    dev = resids[0].device
    B, N = 1, c.N
    M = tg.kept_count(N, c.r, c.K)

    def outs():
        return (torch.empty((B, N), dtype=torch.float32, device=dev),
                torch.empty((B, N), dtype=torch.float32, device=dev),
                torch.empty((B, N), dtype=torch.uint8, device=dev),
                torch.empty((B, M), dtype=torch.int32, device=dev),
                torch.empty((B, M, c.d), dtype=torch.bfloat16, device=dev),
                torch.empty((B, M), dtype=torch.float32, device=dev))

    o_sep, o_fus = outs(), outs()
    counters = tg.gate_counters(B, dev)

    def separate(i):
        raw, score, keep, ki, ro, so = o_sep
        x = resids[i % len(resids)]
        tg.tg_gate_score_folded(x, c.r, W1f, c.h, b1, w2, b2, c.eps_row, score_raw=raw)
        tg.tg_gate_select(raw, x, c.r, c.K, c.eps_seq, score=score, keep=keep, kept_idx=ki, resid_out=ro,
                          score_out=so)

    def fused(i):
        raw, score, keep, ki, ro, so = o_fus
        tg.tg_gate(resids[i % len(resids)], c.r, c.K, W1f, c.h, b1, w2, b2, c.eps_row, c.eps_seq, score_raw=raw,
                   score=score, keep=keep, kept_idx=ki, resid_out=ro, score_out=so, counters=counters)

    for fn in (separate, fused, separate, fused):
        fn(0)
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.uint8), b.view(torch.uint8)) for a, b in zip(o_sep, o_fus))
    best = {"separate": float("inf"), "fused": float("inf")}
    for _ in range(rounds):
        for name, fn in (("separate", separate), ("fused", fused)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            best[name] = min(best[name], e0.elapsed_time(e1) * 1e3 / reps)
    return {"call": "tg_gate", "separate_calls": ["tg_gate_score_folded", "tg_gate_select"],
            "separate_us": round(best["separate"], 3), "fused_us": round(best["fused"], 3),
            "fused_over_separate": round(best["fused"] / best["separate"], 4), "bit_identical": bool(same),
            "calls_per_round": reps, "rounds": rounds}


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


def time_graph(torch, tg, resids, c, W1f, b1, w2, b2, layers, heads, steps, warmup):
    """Each whole step (scorer, selection with the budget read from device
    memory, every attention layer) captured once as one HIP graph per residual
    copy, with the padded entry points: the launches are sized by the kept
    length padded to a multiple of 256, so the same graph would serve any
    budget of that bucket.  Timed by HIP events around `steps` replays."""
    dev = resids[0].device
    N, r, K, d, M, h = c.N, c.r, c.K, c.d, c.M, c.h
    M_pad = min(N, -(-M // 256) * 256)
    Hq, Hkv, dh = heads["Hq"], heads["Hkv"], heads["dh"]
    K_dev = torch.full((1,), K, dtype=torch.int32, device=dev)
    score = torch.empty((1, N), dtype=torch.float32, device=dev)
    keep = torch.empty((1, N), dtype=torch.uint8, device=dev)
    kept_idx = torch.zeros((1, M_pad), dtype=torch.int32, device=dev)
    resid_S = torch.zeros((1, M_pad, d), dtype=torch.bfloat16, device=dev)
    b_S = torch.zeros((1, M_pad), dtype=torch.float32, device=dev)
    kept_count = torch.empty((1,), dtype=torch.int32, device=dev)
    out = torch.empty((1, M_pad, Hq, dh), dtype=torch.bfloat16, device=dev)
    ws = tg.attention_workspace(1, M_pad, Hq, Hkv, dh, dev)

    def gate(x):
        tg.tg_gate_score_folded(x, r, W1f, h, b1, w2, b2, c.eps_row, score_raw=score)
        tg.tg_gate_select_padded(score, x, r, K_dev, M_pad, c.eps_seq, score=score, keep=keep, kept_idx=kept_idx,
                                 resid_out=resid_S, score_out=b_S, kept_count=kept_count)

    gate(resids[0])
    torch.cuda.synchronize()
    qkv = [p.qkv(resid_S) for p in layers]  # glue on the padded stream, outside the graph

    def run(x):
        gate(x)
        for l, p in enumerate(layers):
            q, k, v = qkv[l]
            tg.tg_gated_attention_padded(q, k, v, kept_count, b_S, kept_idx, p.gain, p.temp, out=out, ws=ws)

    graphs = []
    for x in resids:
        run(x)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(x)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return {"ms_per_step": e0.elapsed_time(e1) / steps, "M_pad": M_pad, "kept": int(kept_count.item()),
            "entry_points": ["tg_gate_score_folded", "tg_gate_select_padded", "tg_gated_attention_padded"],
            "graphs": len(graphs)}


def time_phases(torch, phases, steps, warmup):
    """Per-phase average microseconds (HIP events on the launch stream at the
    phase boundaries) and the step time, over `steps` steps; phases is a
    list of (name, call(step_index))."""
    for i in range(warmup):
        for _, fn in phases:
            fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps * len(phases) + 1)]
    ev[0].record()
    n = 0
    for i in range(steps):
        for _, fn in phases:
            fn(i)
            n += 1
            ev[n].record()
    torch.cuda.synchronize()
    per = {}
    for j, (name, _) in enumerate(phases):
        per[name] = 1000.0 * sum(ev[i * len(phases) + j].elapsed_time(ev[i * len(phases) + j + 1])
                                 for i in range(steps)) / steps
    return per, ev[0].elapsed_time(ev[-1]) / steps


def sub_records(torch, tg, wl, stage_glue, heads, steps=10, warmup=3):
    """The metric's other lengths, measured with the same calls as the main
    step: gate_16k (N = 16384, the gate op alone) and sweep_128k (N = 131072,
    heavy-tailed rows, budgets 1/5/10/25 % of the prunable tokens, each gate
    followed by one token-gated attention layer on its kept set)."""
    import numpy as np
    dev = "cuda:0"
    e = 2
    Hq, Hkv, dh = heads["Hq"], heads["Hkv"], heads["dh"]

    def bits(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    def gate_setup(c):
        ncopy = max(1, -(-(512 << 20) // (c.N * c.d * 2)))
        x0 = bits(c.resid)
        xs = [x0] + [x0.clone() for _ in range(ncopy - 1)]
        W1f = tg.tg_gate_fold_weights(bits(c.W1), bits(c.norm_w))
        return xs, W1f, torch.from_numpy(c.b1).to(dev), bits(c.w2), torch.from_numpy(c.b2).to(dev)

    def gate_figures(c, M, per):
        P = c.N - c.r
        sb = P * c.d * e + c.h * c.d * e + 4 * c.N
        gb = 4 * P + 4 * c.N + c.N + 12 * M + 2 * M * c.d * e
        f = {"gate_score_us": round(per["gate_score"], 3),
             "gate_score_hbm_frac": round(sb / (per["gate_score"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
             "gate_select_us": round(per["gate_select"], 3),
             "gate_op_hbm_frac": round((sb + gb) / ((per["gate_score"] + per["gate_select"]) * 1e-6) / 1e9
                                       / PEAK_HBM_GBS, 4)}
        return f

    out = {}
    # gate_16k: the gate op alone
    c = wl.preset_gate_case("gate_16k")
    xs, W1f, b1, w2, b2 = gate_setup(c)
    score = torch.empty((1, c.N), dtype=torch.float32, device=dev)
    keep = torch.empty((1, c.N), dtype=torch.uint8, device=dev)
    ki = torch.empty((1, c.M), dtype=torch.int32, device=dev)
    rs = torch.empty((1, c.M, c.d), dtype=torch.bfloat16, device=dev)
    bs = torch.empty((1, c.M), dtype=torch.float32, device=dev)
    phases = [("gate_score", lambda i: tg.tg_gate_score_folded(xs[i % len(xs)], c.r, W1f, c.h, b1, w2, b2, c.eps_row,
                                                                 score_raw=score)),
              ("gate_select", lambda i: tg.tg_gate_select(score, xs[i % len(xs)], c.r, c.K, c.eps_seq, score=score,
                                                          keep=keep, kept_idx=ki, resid_out=rs, score_out=bs))]
    per, ms = time_phases(torch, phases, steps, warmup)
    out["gate_16k"] = {"N": c.N, "K": c.K, "M": c.M, "ms_per_step": round(ms, 5),
                       "tokens_per_s": round(c.N / (ms * 1e-3), 1), **gate_figures(c, c.M, per)}
    del xs, c
    # sweep_128k: one residual, four budgets
    c = wl.preset_gate_case("sweep_128k", K=1)
    xs, W1f, b1, w2, b2 = gate_setup(c)
    score = torch.empty((1, c.N), dtype=torch.float32, device=dev)
    sel_ws = tg.gate_select_workspace(1, c.N, dev)
    rows = []
    for n, K in enumerate(wl.sweep_budgets(c.N, c.r)):
        M = tg.kept_count(c.N, c.r, K)
        ki = torch.empty((1, M), dtype=torch.int32, device=dev)
        rs = torch.empty((1, M, c.d), dtype=torch.bfloat16, device=dev)
        bs = torch.empty((1, M), dtype=torch.float32, device=dev)
        keep = torch.empty((1, c.N), dtype=torch.uint8, device=dev)
        tg.tg_gate_score_folded(xs[0], c.r, W1f, c.h, b1, w2, b2, c.eps_row, score_raw=score)
        tg.tg_gate_select(score, xs[0], c.r, K, c.eps_seq, score=score, keep=keep, kept_idx=ki, resid_out=rs,
                          score_out=bs, ws=sel_ws)
        lay = stage_glue.stage_layers(1, c.d, seed0=500 + n, **heads)[0]
        q, k, v = lay.qkv(rs)
        ao = torch.empty((1, M, Hq, dh), dtype=torch.bfloat16, device=dev)
        aws = tg.attention_workspace(1, M, Hq, Hkv, dh, dev)
        phases = [("gate_score", lambda i: tg.tg_gate_score_folded(xs[0], c.r, W1f, c.h, b1, w2, b2, c.eps_row,
                                                                     score_raw=score)),
                  ("gate_select", lambda i: tg.tg_gate_select(score, xs[0], c.r, K, c.eps_seq, score=score,
                                                              keep=keep, kept_idx=ki, resid_out=rs, score_out=bs,
                                                              ws=sel_ws)),
                  ("attention", lambda i: tg.tg_gated_attention(q, k, v, bs, ki, lay.gain, lay.temp, out=ao, ws=aws))]
        per, ms = time_phases(torch, phases, steps, warmup)
        flops = 2 * dh * Hq * M * (M + 1)
        tf = flops / (per["attention"] * 1e-6) / 1e12
        rows.append({"frac": wl.SWEEP_FRACTIONS[n], "K": K, "M": M, "ms_per_step": round(ms, 5),
                     "tokens_per_s": round(c.N / (ms * 1e-3), 1), **gate_figures(c, M, per),
                     "attention_us": round(per["attention"], 3), "attention_TFLOPs": round(tf, 2),
                     "attention_mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        del q, k, v, ao, aws, ki, rs, bs
    out["sweep_128k"] = {"N": c.N, "r": c.r, "budgets": rows}
    return out


def ceilings(torch, reps=5):
    """Measured ceilings of this device, for context beside the spec peaks: a
    plain device-to-device copy of 1 GiB (bytes read + written per second)
    and a large bf16 GEMM through torch (hipBLASLt), 8192^3."""
    dev = "cuda:0"
    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).bfloat16()
    b = torch.randn(8192, 8192, device=dev).bfloat16()
    # the scorer's first layer as a plain library GEMM (no norm, no epilogue,
    # the [N, h] product written out): residual [32768, 2048] x W1^T [2048, 256]
    xs = torch.randn(32768, 2048, device=dev).bfloat16()
    w1 = torch.randn(256, 2048, device=dev).bfloat16()
    res = {}
    for name, fn, work in (("copy", lambda: dst.copy_(src), 2 * (1 << 30)),
                           ("gemm_bf16", lambda: torch.mm(a, b), 2 * 8192 ** 3),
                           ("gemm_scorer", lambda: torch.mm(xs, w1.t()), 32768 * 2048 * 2)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = work * reps / (e0.elapsed_time(e1) * 1e-3)
    del src, dst, a, b, xs, w1
    scorer_us = 32768 * 2048 * 2 / res["gemm_scorer"] * 1e6  # (work counted as the residual bytes read)
    return {"copy_GBs": round(res["copy"] / 1e9, 1), "copy_frac_of_spec": round(res["copy"] / 1e9 / PEAK_HBM_GBS, 4),
            "gemm_bf16_TFLOPs": round(res["gemm_bf16"] / 1e12, 1),
            "gemm_bf16_frac_of_spec": round(res["gemm_bf16"] / 1e12 / PEAK_BF16_TFLOPS, 4),
            "gemm_shape": [8192, 8192, 8192],
            "scorer_gemm_library_us": round(scorer_us, 2), "scorer_gemm_shape": [32768, 2048, 256],
            "scorer_gemm_residual_GBs": round(res["gemm_scorer"] / 1e9, 1)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(c, layer0_qkv, kept_idx, b_S, gain, temp, n_layers, max_rows=1024):
    """The oracle, as it stands, on a bounded sample of the same workload,
    once with its BLAS thread pool at its default size and once on one
    thread (elementwise numpy steps are single-threaded either way)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    full = _cpu_sample(c, layer0_qkv, kept_idx, b_S, gain, temp, n_layers, max_rows)
    with threadpool_limits(limits=1):
        one = _cpu_sample(c, layer0_qkv, kept_idx, b_S, gain, temp, n_layers, max_rows)
    return {"value": full["value"], "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": full["sample"], "seconds_per_step": full["seconds_per_step"], "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "single_thread": {"value": one["value"], "seconds_per_step": one["seconds_per_step"], "cores": 1}}


def _cpu_sample(c, layer0_qkv, kept_idx, b_S, gain, temp, n_layers, max_rows):
    import numpy as np

    import oracle
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
        "value": c.N / per_step,
        "sample": (f"gate (score, seq-norm, top-K, compaction) on the full N={c.N} input: {t_gate:.2f} s; "
                   f"one attention layer on {R} of {M} query rows (all {q.shape[2]} heads): {t_rows:.2f} s, "
                   f"extrapolated linearly to {M} rows x {n_layers} layers"),
        "seconds_per_step": per_step,
    }


# ---------------------------------------------------------------------------
# Profile summaries (CPU only): rocprofv3 CSV output -> the files under profiles/
STAGE_SHAPE = dict(N=32768, r=64, d=2048, h=256, M=3341, Hq=16, Hkv=8, dh=128, kv_layers=STAGE_GATE_LAYER + 1)
PROFILE_RUN_FLAGS = "--no-cpu-baseline --no-sub-records --no-ceilings --no-varlen --no-rope --no-fused-gate"
# library call -> (source file, kernels of one call at the stage shape)
PROFILE_CALLS = {
    "tg_gated_attention": ("gated_attention.hip",
                           ["attn_prepass_kernel<128, false, false>", "gated_attn_kernel<128, 2, false, false>"]),
    "tg_gate_score_folded": ("gate_score.hip", ["gate_score_bf16_kernel<256, 128, 8, 32, false>"]),
    "tg_gate_select": ("gate_select.hip", ["gate_select_kernel", "compact_gather_kernel"]),
    "tg_gated_attention_backward": ("gated_attention_bwd.hip",
                                    ["bwd_rows_kernel<128>", "bwd_dkdv_kernel<128, 2, false>",
                                     "bwd_dq_kernel<128, 2, false>", "bwd_reduce_kernel"]),
    "tg_kv_cache_prune": ("kv_prune.hip", ["kv_prune_kernel"]),
}


def stage_algorithmic_bytes():
    """Bytes each library call must move at the stage shape (inputs read once,
    outputs written once)."""
    S = STAGE_SHAPE
    N, r, d, h, M, Hq, Hkv, dh = (S[k] for k in ("N", "r", "d", "h", "M", "Hq", "Hkv", "dh"))
    P = N - r
    return {
        # residual span, W1 (bf16), raw scores out
        "tg_gate_score_folded": P * d * 2 + h * d * 2 + 4 * N,
        # raw scores in, normalised scores, keep mask, kept_idx and kept scores out, kept_idx read back by the
        # gather, kept rows read and written
        "tg_gate_select": 4 * P + 4 * N + N + 12 * M + 2 * M * d * 2,
        # q, k, v in, out written (bf16); key scores and positions
        "tg_gated_attention": M * dh * 2 * (2 * Hq + 2 * Hkv) + 8 * M,
        # q, k, v, out, d_out in (bf16), lse, key scores, positions; d_q, d_k, d_v (bf16), d_key_score out
        "tg_gated_attention_backward": 2 * M * dh * (3 * Hq + 2 * Hkv) + 4 * M * Hq + 8 * M
                                       + 2 * M * dh * (Hq + 2 * Hkv) + 4 * M,
        # the kept rows of every layer's K and V read and written, kept_idx
        "tg_kv_cache_prune": S["kv_layers"] * 2 * M * Hkv * dh * 2 * 2 + 4 * M,
    }


def _short_kernel(name: str) -> str:
    """'void tg::(anonymous namespace)::k<1, 2>(args...)' -> 'k<1, 2>'."""
    n = name[5:] if name.startswith("void ") else name
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0 and not n[:i].endswith("anonymous namespace") and \
                not n[i:].startswith("(anonymous"):
            n = n[:i]
            break
    return n.replace("tg::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")


def _csv_rows(root, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {root}")
    return list(csv.DictReader(open(files[0])))


def _counter_kib(root):
    """Average counter value (KiB) per dispatch of every kernel in a --pmc run."""
    acc = {}
    for r in _csv_rows(root, "counter_collection.csv"):
        acc.setdefault(_short_kernel(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_profiles(run_dir: str):
    """Writes profiles/kernel_trace_stage_32k.txt, profiles/hbm_traffic_stage_32k.txt and
    profiles/traffic.json from the rocprofv3 output of the commands they list,
    run from the repository root with their -d directories under run_dir."""
    prof = os.path.join(ROOT, "profiles")
    cmds = {
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {{dir}}/trace -o stage -- "
                 f"python3 bench.py --steps 5 --warmup 2 {PROFILE_RUN_FLAGS}",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {{dir}}/fetch -o stage -- "
                 f"python3 bench.py --steps 2 --warmup 1 {PROFILE_RUN_FLAGS}",
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {{dir}}/write -o stage -- "
                 f"python3 bench.py --steps 2 --warmup 1 {PROFILE_RUN_FLAGS}",
        "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/copy_fetch -o copy -- "
                      "python3 bench.py --copy-calibration",
        "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/copy_write -o copy -- "
                      "python3 bench.py --copy-calibration",
    }
    S = STAGE_SHAPE
    head = (f"stage_32k (N={S['N']}, r={S['r']}, K=3277 -> M={S['M']}, d={S['d']}, h={S['h']}, "
            f"{S['Hq']}q/{S['Hkv']}kv heads, d_h {S['dh']}, 24 gated attention layers)")
    # ---- kernel trace ----
    stats = _csv_rows(os.path.join(run_dir, "trace"), "kernel_stats.csv")
    lines = [f"# Kernel trace: {head}", "", "Commands (repository root, one MI355X):",
             "    " + cmds["trace"].format(dir="<dir>"),
             "    python3 bench.py --summarize-profiles <dir>   (writes this file)", "",
             "rocprofv3 --stats summary (durations in microseconds).  Cijk_* are the Q/K/V projection glue",
             "(hipBLASLt GEMMs, outside the library and outside the timed step); __amd_rocclr_* and at::native",
             "kernels are torch copies, fills and draws of the set-up.", "",
             f"{'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total%':>7s}"]
    avg = {}
    for r in stats:
        k = _short_kernel(r["Name"])
        avg[k] = float(r["AverageNs"]) / 1e3
        lines.append(f"{k[:58]:58s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}")
    lines += ["", "Per library call at the stage shape (sum of its kernels' averages):"]
    for call, (_, ks) in PROFILE_CALLS.items():
        if all(k in avg for k in ks):
            parts = " + ".join(f"{avg[k]:.2f}" for k in ks)
            lines.append(f"    {call} = {' + '.join(ks)}")
            lines.append(f"        = {parts} = {sum(avg[k] for k in ks):.2f} us")
    lines += ["", "bench.py times the same calls with HIP events on the launch stream; its per-call averages",
              "include the gaps between kernels, so they read slightly above these sums."]
    open(os.path.join(prof, "kernel_trace_stage_32k.txt"), "w").write("\n".join(lines) + "\n")
    # ---- HBM traffic ----
    fetch, write = _counter_kib(os.path.join(run_dir, "fetch")), _counter_kib(os.path.join(run_dir, "write"))
    cf, cw = _counter_kib(os.path.join(run_dir, "copy_fetch")), _counter_kib(os.path.join(run_dir, "copy_write"))
    copy_k = [k for k in cf if "copyBuffer" in k]
    if not copy_k:
        raise SystemExit("no copy kernel in the calibration runs")
    nbytes = 1 << 30
    fscale = nbytes / (cf[copy_k[0]] * 1024)  # bytes moved per KiB of counter
    wscale = nbytes / (cw[copy_k[0]] * 1024)
    algo = stage_algorithmic_bytes()
    t = {"calibration": {"copy_bytes": nbytes, "fetch_kib_read": cf[copy_k[0]], "write_kib_read": cw[copy_k[0]],
                         "fetch_scale": fscale, "write_scale": wscale},
         "commands": [cmds[k].format(dir="<dir>") for k in ("fetch", "write", "copy_fetch", "copy_write")],
         "shape": S}
    lines = [f"# HBM traffic per library call: {head}", "", "Commands (repository root):"]
    lines += ["    " + cmds[k].format(dir="<dir>") for k in ("fetch", "write", "copy_fetch", "copy_write")]
    lines += ["    python3 bench.py --summarize-profiles <dir>   (writes this file)", "",
              f"Calibration: a plain 1 GiB device copy (torch copy_ -> {copy_k[0]}) reads FETCH_SIZE "
              f"{cf[copy_k[0]]:.1f} KiB and WRITE_SIZE {cw[copy_k[0]]:.1f} KiB per dispatch for 1048576 KiB moved",
              f"each way: below, one FETCH_SIZE KiB counts as {fscale:.4f} KiB read and one WRITE_SIZE KiB as "
              f"{wscale:.4f} KiB written.", "",
              f"{'call / kernel':48s} {'FETCH KiB':>11s} {'WRITE KiB':>11s} {'bytes (scaled)':>16s}"]
    for call, (src, ks) in PROFILE_CALLS.items():
        if not all(k in fetch and k in write for k in ks):
            lines.append(f"{call}: not in the counter runs")
            continue
        tot = 0.0
        for k in ks:
            b = fetch[k] * 1024 * fscale + write[k] * 1024 * wscale
            tot += b
            lines.append(f"  {k[:46]:46s} {fetch[k]:11.1f} {write[k]:11.1f} {b / 1e6:13.2f} MB")
        lines.append(f"{call:48s} {'':11s} {'':11s} {tot / 1e6:13.2f} MB   algorithmic {algo[call] / 1e6:.2f} MB "
                     f"(ratio {tot / algo[call]:.3f})")
        t[src] = {"call": call, "kernels": ks, "bytes_per_launch": tot, "algorithmic_bytes": algo[call],
                  "fetch_kib": {k: fetch[k] for k in ks}, "write_kib": {k: write[k] for k in ks},
                  "sources": [src] + PROFILE_DEPS.get(src, []), "sources_sha256": _sources_sha(src)}
    open(os.path.join(prof, "hbm_traffic_stage_32k.txt"), "w").write("\n".join(lines) + "\n")
    json.dump(t, open(os.path.join(prof, "traffic.json"), "w"), indent=1)
    print("\n".join(lines))
    bench_line = os.path.join(run_dir, "bench.json")
    if os.path.exists(bench_line):
        summarize_bench_line(bench_line, os.path.join(prof, "bench_stage_32k.txt"))
    for name, (wflags, what) in OTHER_TRACES.items():
        if os.path.isdir(os.path.join(run_dir, "trace_" + name)):
            summarize_other_trace(run_dir, name, wflags, what, prof)


# kernel traces at the metric's other lengths: directory suffix -> (bench.py workload flags, description)
OTHER_TRACES = {
    "gate_16k": ("--workload gate_16k", "gate_16k (N=16384, r=64, K=1638 -> M=1702, d=2048, h=256): "
                                        "scorer and fused selection"),
    "sweep_128k_f25": ("--workload sweep_128k --frac 0.25",
                       "sweep_128k at a 25 % budget (N=131072, r=128, K=32736 -> M=32864, d=2048, h=256; "
                       "one gated attention layer, 16q/8kv, d_h 128)"),
}


def summarize_other_trace(run_dir: str, name: str, wflags: str, what: str, prof: str):
    """profiles/kernel_trace_<name>.txt from a rocprofv3 kernel trace of that workload."""
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace_{name} -o run -- "
           f"python3 bench.py {wflags} --steps 5 --warmup 2 {PROFILE_RUN_FLAGS} --no-backward --no-kv-prune")
    stats = _csv_rows(os.path.join(run_dir, "trace_" + name), "kernel_stats.csv")
    lines = [f"# Kernel trace: {what}", "", "Commands (repository root, one MI355X):", "    " + cmd,
             "    python3 bench.py --summarize-profiles <dir>   (writes this file)", "",
             "rocprofv3 --stats summary (durations in microseconds); __amd_rocclr_*, at::native and Cijk_* kernels",
             "are torch copies, fills, draws and the Q/K/V projection glue of the set-up, outside the timed step.", "",
             f"{'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total%':>7s}"]
    for r in stats:
        k = _short_kernel(r["Name"])
        lines.append(f"{k[:58]:58s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}")
    open(os.path.join(prof, f"kernel_trace_{name}.txt"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_bench_line(path: str, dst: str):
    """profiles/bench_stage_32k.txt: the figures of one default bench.py line
    (the step, per-call times, roofline, the measured ceilings, the other
    lengths and the CPU oracle), from `python3 bench.py > <dir>/bench.json`."""
    d = json.loads(open(path).read().strip().splitlines()[-1])
    L = [f"# bench.py line: {d['config'].get('workload')} on one MI355X", "",
         "Command (repository root):", "    python3 bench.py > <dir>/bench.json",
         "    python3 bench.py --summarize-profiles <dir>   (writes this file)", "",
         f"{d['metric']}", f"value {d['value']:.4g} {d['unit']}; {d['ms_per_step']:.4f} ms per step "
         f"({d['steps']} steps after {d['warmup']} warm-up, dtype {d['dtype']})", "",
         f"{'call':24s} {'us/call':>9s} {'per step':>9s} {'HBM frac':>9s} {'MFMA frac':>10s}"]
    for k, v in d["kernels"].items():
        L.append(f"{k:24s} {v['avg_us']:9.2f} {v['launches_per_step']:9d} {v.get('hbm_frac', 0):9.3f} "
                 f"{v.get('mfma_frac', 0):10.3f}")
    r = d["roofline"]
    L += ["", f"roofline ({r['kernel']}, {r['bound']}): {r['achieved']:.1f} of {r['peak']:.0f} {r['unit']} = "
          f"{r['frac']:.4f} of the spec peak; {r.get('frac_of_measured_ceiling', 0):.4f} of the measured bf16 GEMM "
          f"rate; counter traffic {r['traffic'] / 1e6 if r.get('traffic') else float('nan'):.2f} MB per call"]
    c = d.get("ceilings")
    if c:
        L += ["", "measured ceilings (same box, same run):",
              f"  device copy of 1 GiB: {c['copy_GBs']:.0f} GB/s = {c['copy_frac_of_spec']:.3f} of 8 TB/s",
              f"  bf16 GEMM {c['gemm_shape']} through torch (hipBLASLt): {c['gemm_bf16_TFLOPs']:.0f} TFLOP/s = "
              f"{c['gemm_bf16_frac_of_spec']:.3f} of 2.5 PFLOP/s",
              f"  the scorer's product {c['scorer_gemm_shape']} as a library GEMM: {c['scorer_gemm_library_us']:.2f} us "
              f"({c['scorer_gemm_residual_GBs']:.0f} GB/s of residual)"]
    for name, rec in (d.get("sub_records") or {}).items():
        L.append("")
        for b in rec.get("budgets", [rec]):
            L.append(f"{name} N={rec['N']} M={b['M']}: {b['ms_per_step'] * 1000:.1f} us per step, "
                     f"{b['tokens_per_s'] / 1e6:.1f} M tokens/s; score {b['gate_score_us']:.1f} us "
                     f"({b['gate_score_hbm_frac']:.3f} HBM), selection {b['gate_select_us']:.1f} us"
                     + (f", attention {b['attention_us']:.1f} us ({b['attention_mfma_frac']:.3f} MFMA)"
                        if "attention_us" in b else ""))
    cb = d.get("cpu_baseline")
    if cb:
        st = cb.get("single_thread", {})
        L += ["", f"CPU oracle ({cb.get('cpu_model')}, {cb['cores']} threads): {cb['value']:.0f} {cb['unit']}; "
              f"one thread: {st.get('value', float('nan')):.0f}", f"  sample: {cb['sample']}"]
    open(dst, "w").write("\n".join(L) + "\n")
    print("\n".join(L))


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
                    help="after the direct-launch timing, capture each whole step as one HIP graph (padded entry "
                         "points: budget in device memory, kept length padded to a multiple of 256) and time "
                         "its replays; value and ms_per_step then come from the replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub-records", action="store_true",
                    help="skip the gate_16k and sweep_128k (1/5/10/25 %%) records of the metric's other lengths")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured copy and bf16 GEMM ceilings")
    ap.add_argument("--no-kv-prune", action="store_true",
                    help="skip the separate timing of tg_kv_cache_prune (layers 0..L of the stage)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed varying-length attention timing")
    ap.add_argument("--no-rope", action="store_true",
                    help="skip the rotary attention timing beside the plain call")
    ap.add_argument("--no-fused-gate", action="store_true",
                    help="skip the timing of the one-call gate (tg_gate) beside the separate calls")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the separate timing of tg_gated_attention_backward at the attention shape")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="(CPU only) turn the rocprofv3 output of the profile commands, run with their -d "
                         "directories under DIR, into the summaries under profiles/, then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB (5 times): the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return

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
    W1f = tg.tg_gate_fold_weights(W1, norm_w)      # once per weight set
    seq_ws = tg.seq_rmsnorm_workspace(1, N, dev)   # None up to N = 32768
    topk_ws = tg.topk_workspace(1, N, dev)
    sel_ws = tg.gate_select_workspace(1, N, dev)   # None up to N = 32768
    sel_phases = ("seq_rmsnorm", "topk_select", "compact") if args.separate_gate else ("gate_select",)

    def gate_calls(x):
        """The gate's library calls on residual x, as (phase name, call)."""
        calls = [("gate_score", lambda: tg.tg_gate_score_folded(x, r, W1f, h, b1, w2, b2, c.eps_row,
                                                                 score_raw=score))]
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

    def step(i, ev=None):
        for name, fn, calls in step_phases(i):
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
    log(f"{ms_per_step:.4f} ms/step over {args.steps} steps ({ncopy} residual copies, direct launches)")
    direct_ms = ms_per_step
    graph_info = None
    if args.graph and not args.separate_gate and N <= 32768:
        graph_info = time_graph(torch, tg, resids, c, W1f, b1, w2, b2, layers, heads, args.steps, args.warmup)
        ms_per_step = graph_info["ms_per_step"]
        log(f"{ms_per_step:.4f} ms/step over {args.steps} graph replays (padded kept length "
            f"{graph_info['M_pad']})")

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
    # (the committed counters are per call at the stage shape)
    roofline["traffic"] = _traffic(dom_file) if args.workload == "stage_32k" and n_layers == 24 else None
    ceil = None if args.no_ceilings else ceilings(torch)
    if ceil:
        if roofline["unit"] == "TFLOP/s":
            roofline["measured_ceiling"] = ceil["gemm_bf16_TFLOPs"]
        else:
            roofline["measured_ceiling"] = ceil["copy_GBs"]
        roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / roofline["measured_ceiling"], 4)

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
        "launch": "hip_graph" if graph_info else "direct",
        "gate_op": {"calls": ["tg_gate_score_folded"] + ["tg_" + n for n in sel_phases],
                    "avg_us": round(gate_us, 3), "algorithmic_bytes": gate_bytes,
                    "achieved_GBs": round(gate_bytes / (gate_us * 1e-6) / 1e9, 1),
                    "hbm_frac": round(gate_bytes / (gate_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "library_kernel_tokens_per_s": round(N / (kernel_us_sum * 1e-6), 1),
        "glue_qkv_ms_per_step": round(glue_ms, 4),
        "tokens_per_s_with_glue": round(N / ((ms_per_step + glue_ms) * 1e-3), 1),
    }
    if ceil:
        out["ceilings"] = ceil
    if graph_info:
        out["direct_ms_per_step"] = round(direct_ms, 5)
        out["graph"] = {k: v for k, v in graph_info.items() if k != "ms_per_step"}

    if layers and not args.no_varlen:
        out["varlen_attention"] = time_varlen(torch, tg, layers[0], heads, M)
    if layers and not args.no_rope:
        out["rope_attention"] = time_rope(torch, tg, qkv[0], b_S, kept_idx, layers[0], heads, M)
        log(f"rotary attention: {out['rope_attention']['rope_us']:.2f} us per call, "
            f"{out['rope_attention']['rope_over_plain']:.3f} x the plain call")
    if not args.no_fused_gate:
        out["fused_gate"] = time_fused_gate(torch, tg, resids, c, W1f, b1, w2, b2)
        log(f"one-call gate: {out['fused_gate']['fused_us']:.2f} us vs {out['fused_gate']['separate_us']:.2f} us "
            f"for the separate calls (bit-identical: {out['fused_gate']['bit_identical']})")
    if layers and not args.no_backward:
        out["attention_backward"] = time_backward(torch, tg, qkv[0], b_S, kept_idx, layers[0], attn_out, heads, M,
                                                  stream_reps=20)
        log(f"attention backward: {out['attention_backward']['avg_us']:.2f} us per call")

    if layers and not args.no_kv_prune and args.workload == "stage_32k":
        out["kv_cache_prune"] = time_kv_prune(torch, tg, kept_idx, N, M, heads, n_layers=STAGE_GATE_LAYER + 1)
        log(f"kv cache prune: {out['kv_cache_prune']['avg_us']:.2f} us per call")

    if not args.no_sub_records and args.workload == "stage_32k":
        log("sub-records: gate_16k and sweep_128k at 1/5/10/25 %")
        out["sub_records"] = sub_records(torch, tg, wl, stage_glue, heads)

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
