"""The gated-prefill stage captured as one HIP graph: the gate (score, then
selection and compaction in one call), two token-gated attention layers on
the compacted stream, the second layer's backward and the KV-cache pruning of
two lower layers, replayed several times.  Each replay must reproduce the
eager results bit for bit, also after the input buffer is refilled between
replays (the graph reads the buffers live) and with eager work and
synchronisations between the replays.  The library's calls launch kernels
only (no allocation, no memset, no host synchronisation), which is what makes
them capturable."""
import numpy as np
import pytest
import torch

import learned_token_pruning_07_amd as tg
from learned_token_pruning_07_amd import workloads as wl
from _gpu_util import DEV, dev, dev_bits, say

pytestmark = pytest.mark.gpu

N, R, D, H, K = 4096, 32, 512, 256, 400
HQ, HKV, DH = 4, 2, 128
M = tg.kept_count(N, R, K)


def _gate_inputs(seed):
    c = wl.gate_case(N=N, r=R, d=D, h=H, K=K, dtype="bf16", seed=seed, w_std=0.1, salient_frac=0.02)
    return c, dict(resid=dev_bits(c.resid), norm_w=dev_bits(c.norm_w), W1=dev_bits(c.W1),
                   b1=dev(c.b1), w2=dev_bits(c.w2), b2=dev(c.b2))


class Stage:
    """Preallocated buffers and the stage's library calls on the current stream."""

    def __init__(self, w, c):
        self.w, self.c = w, c
        self.resid = torch.empty((1, N, D), dtype=torch.bfloat16, device=DEV)
        self.score = torch.empty((1, N), dtype=torch.float32, device=DEV)
        self.keep = torch.empty((1, N), dtype=torch.uint8, device=DEV)
        self.kept_idx = torch.empty((1, M), dtype=torch.int32, device=DEV)
        self.resid_S = torch.empty((1, M, D), dtype=torch.bfloat16, device=DEV)
        self.b_S = torch.empty((1, M), dtype=torch.float32, device=DEV)
        self.gate_ws = tg.gate_workspace(H, D, DEV)
        self.sel_ws = tg.gate_select_workspace(1, N, DEV)
        g = torch.Generator(device=DEV).manual_seed(5)
        # two layers' Q/K/V: fixed random tensors (the stage's glue is not in the graph)
        self.qkv = [(torch.randn(1, M, HQ, DH, device=DEV, generator=g).bfloat16(),
                     torch.randn(1, M, HKV, DH, device=DEV, generator=g).bfloat16(),
                     torch.randn(1, M, HKV, DH, device=DEV, generator=g).bfloat16()) for _ in range(2)]
        self.gain = [torch.rand(HQ, device=DEV, generator=g) + 0.5 for _ in range(2)]
        self.temp = torch.full((HQ,), 1.2, device=DEV)
        self.out = [torch.empty((1, M, HQ, DH), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
        self.attn_ws = tg.attention_workspace(1, M, HQ, HKV, DH, DEV)
        self.lse = torch.empty((1, HQ, M), dtype=torch.float32, device=DEV)
        # the last layer's backward and the KV-cache pruning of two lower layers
        self.d_out = torch.randn(1, M, HQ, DH, device=DEV, generator=g).bfloat16()
        self.grads = [torch.empty((1, M, HQ, DH), dtype=torch.bfloat16, device=DEV),
                      torch.empty((1, M, HKV, DH), dtype=torch.bfloat16, device=DEV),
                      torch.empty((1, M, HKV, DH), dtype=torch.bfloat16, device=DEV),
                      torch.empty((1, M), dtype=torch.float32, device=DEV), torch.empty(HQ, device=DEV),
                      torch.empty(HQ, device=DEV)]
        self.bwd_ws = tg.attention_backward_workspace(1, M, HQ, HKV, DH, DEV)
        self.kv = [torch.randn(2, 1, N, HKV, DH, device=DEV, generator=g).bfloat16() for _ in range(2)]
        self.kv_out = [torch.empty((2, 1, M, HKV, DH), dtype=torch.bfloat16, device=DEV) for _ in range(2)]

    def run(self):
        w, c = self.w, self.c
        tg.tg_gate_score(self.resid, R, w["norm_w"], w["W1"], w["b1"], w["w2"], w["b2"], c.eps_row,
                         score_raw=self.score, ws=self.gate_ws)
        tg.tg_gate_select(self.score, self.resid, R, K, c.eps_seq, score=self.score, keep=self.keep,
                          kept_idx=self.kept_idx, resid_out=self.resid_S, score_out=self.b_S, ws=self.sel_ws)
        for l in range(2):
            q, k, v = self.qkv[l]
            tg.tg_gated_attention(q, k, v, self.b_S, self.kept_idx, self.gain[l], self.temp, out=self.out[l],
                                  lse=self.lse if l == 1 else None, ws=self.attn_ws)
        q, k, v = self.qkv[1]
        tg.tg_gated_attention_backward(q, k, v, self.out[1], self.lse, self.d_out, self.b_S, self.kept_idx,
                                       self.gain[1], self.temp, None, *self.grads, ws=self.bwd_ws)
        tg.tg_kv_cache_prune(self.kv[0], self.kv[1], self.kept_idx, k_out=self.kv_out[0], v_out=self.kv_out[1])

    def results(self):
        return [t.clone() for t in (self.score, self.keep, self.kept_idx, self.resid_S, self.b_S, *self.out, self.lse,
                                    *self.grads, *self.kv_out)]

    def poison(self):
        for t in (self.score, self.b_S, self.lse, *self.grads[3:]):
            t.fill_(float("nan"))
        for t in (self.keep, self.kept_idx, self.resid_S, *self.out, *self.grads[:3], *self.kv_out):
            t.view(torch.uint8).fill_(0xA5)


def _same(got, ref, what):
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: output {i} differs"


def test_stage_graph_replays_match_eager():
    say(f"graph: gate N={N} d={D} K={K} + 2 attention layers M={M}")
    c0, w = _gate_inputs(0)
    c1, _ = _gate_inputs(1)  # a second residual for the same weights
    st = Stage(w, c0)
    inputs = [dev_bits(c0.resid), dev_bits(c1.resid)]

    # eager references for both inputs
    ref = []
    for x in inputs:
        st.resid.copy_(x)
        st.run()
        torch.cuda.synchronize()
        ref.append(st.results())
    assert int(st.keep.sum()) == M

    # capture (the calls were warmed up above; nothing is allocated inside)
    graph = torch.cuda.CUDAGraph()
    st.resid.copy_(inputs[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()

    for rep, which in enumerate([0, 1, 0, 1]):
        st.poison()
        st.resid.copy_(inputs[which])
        graph.replay()
        torch.cuda.synchronize()
        _same(st.results(), ref[which], f"replay {rep} (input {which})")
        # eager work between replays: an eager pass on the other input, checked too
        st.resid.copy_(inputs[1 - which])
        st.run()
        torch.cuda.synchronize()
        _same(st.results(), ref[1 - which], f"eager pass after replay {rep}")
    say("  4 replays and 4 eager passes bit-identical")


def test_varlen_graph_replays_match_eager():
    """The packed varying-length attention and its backward captured in one
    graph (72 sequences: two launches of each kernel; their sequence tables
    travel in the kernel arguments): every replay, with its outputs poisoned
    before it and eager work after it, equals the eager call bit for bit."""
    lens = [300, 0, 129, 64, 1, 500] * 12
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()
    T, B = cu[-1], len(lens)
    say(f"graph: varlen attention + backward, {B} sequences, {T} rows")
    g = torch.Generator(device=DEV).manual_seed(9)
    q = torch.randn(T, HQ, DH, device=DEV, generator=g).bfloat16()
    k = torch.randn(T, HKV, DH, device=DEV, generator=g).bfloat16()
    v = torch.randn(T, HKV, DH, device=DEV, generator=g).bfloat16()
    d_out = torch.randn(T, HQ, DH, device=DEV, generator=g).bfloat16()
    ks = torch.randn(T, device=DEV, generator=g)
    pos = torch.cat([torch.arange(m, dtype=torch.int32, device=DEV) * 3 for m in lens])
    gain, temp = torch.rand(HQ, device=DEV, generator=g) + 0.5, torch.full((HQ,), 1.2, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(T * HQ, dtype=torch.float32, device=DEV)
    ws_f = tg.attention_workspace(1, T + 63 * B, HQ, HKV, DH, DEV)
    ws_b = tg.attention_backward_workspace(1, T + 63 * B, HQ, HKV, DH, DEV)

    def run():
        tg.tg_gated_attention_varlen(q, k, v, cu, ks, pos, gain, temp, out=out, lse=lse, ws=ws_f)
        return tg.tg_gated_attention_backward_varlen(q, k, v, out, lse, d_out, cu, ks, pos, gain, temp, ws=ws_b)

    ref_grads = [x.clone() for x in run()]
    torch.cuda.synchronize()
    ref = [out.clone(), lse.clone()] + ref_grads
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grads = run()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in [out, lse] + list(grads):
            x.view(torch.uint8).fill_(0xFF)  # NaN in both dtypes
        graph.replay()
        torch.cuda.synchronize()
        for x, y, name in zip([out, lse] + list(grads), ref, ["out", "lse", "d_q", "d_k", "d_v", "d_key_score",
                                                              "d_gain", "d_temp"]):
            assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), \
                f"replay {rep}: {name}"
        # eager work between replays (the batched attention on another shape)
        tg.tg_gated_attention(q[None, :500].contiguous(), k[None, :500].contiguous(), v[None, :500].contiguous(),
                              ks[None, :500].contiguous(), torch.arange(500, dtype=torch.int32, device=DEV)[None],
                              gain, temp)
        torch.cuda.synchronize()
    say("  3 replays bit-identical")


def test_padded_graph_serves_every_budget_of_its_bucket():
    """One graph per padded kept length (paper, Section 5, "Implementation and
    timing": the pruned forward is captured once per padded length).  The gate
    (scorer, then the selection with its budget read from device memory) and
    two attention layers sized by M_pad are captured once; replays at several
    budgets, each set by writing K into device memory, equal the plain entry
    points called with that budget bit for bit, leave the rows past the kept
    length untouched, and match the oracle.  A budget past the bucket is cut
    to it."""
    import oracle
    from _gpu_util import TOL_BF16, TOL_LSE, assert_close, host_bits

    M_pad = 512
    budgets = [100, 333, 480, 700, 100]  # kept 132, 365, 512, 512 (cut), 132
    c, w = _gate_inputs(3)
    resid = dev_bits(c.resid)
    g = torch.Generator(device=DEV).manual_seed(17)
    qkv = [(torch.randn(1, M_pad, HQ, DH, device=DEV, generator=g).bfloat16(),
            torch.randn(1, M_pad, HKV, DH, device=DEV, generator=g).bfloat16(),
            torch.randn(1, M_pad, HKV, DH, device=DEV, generator=g).bfloat16()) for _ in range(2)]
    gains = [torch.rand(HQ, device=DEV, generator=g) + 0.5 for _ in range(2)]
    temp = torch.full((HQ,), 1.2, device=DEV)
    K_dev = torch.zeros(1, dtype=torch.int32, device=DEV)
    score = torch.empty((1, N), dtype=torch.float32, device=DEV)
    keep = torch.empty((1, N), dtype=torch.uint8, device=DEV)
    kept_idx = torch.empty((1, M_pad), dtype=torch.int32, device=DEV)
    resid_S = torch.empty((1, M_pad, D), dtype=torch.bfloat16, device=DEV)
    b_S = torch.empty((1, M_pad), dtype=torch.float32, device=DEV)
    kept_count = torch.empty(1, dtype=torch.int32, device=DEV)
    outs = [torch.empty((1, M_pad, HQ, DH), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    lse = torch.empty((1, HQ, M_pad), dtype=torch.float32, device=DEV)
    gate_ws = tg.gate_workspace(H, D, DEV)
    attn_ws = tg.attention_workspace(1, M_pad, HQ, HKV, DH, DEV)

    def run_padded():
        tg.tg_gate_score(resid, R, w["norm_w"], w["W1"], w["b1"], w["w2"], w["b2"], c.eps_row, score_raw=score,
                         ws=gate_ws)
        tg.tg_gate_select_padded(score, resid, R, K_dev, M_pad, c.eps_seq, score=score, keep=keep, kept_idx=kept_idx,
                                 resid_out=resid_S, score_out=b_S, kept_count=kept_count)
        for l in range(2):
            q, k, v = qkv[l]
            tg.tg_gated_attention_padded(q, k, v, kept_count, b_S, kept_idx, gains[l], temp, out=outs[l],
                                         lse=lse if l == 1 else None, ws=attn_ws)

    def eager(Kb):
        """The plain entry points at budget Kb (host M), on fresh buffers."""
        Kc = min(Kb, M_pad - R)
        raw = tg.tg_gate_score(resid, R, w["norm_w"], w["W1"], w["b1"], w["w2"], w["b2"], c.eps_row)
        ki, rs, bs, kp, sc = tg.tg_gate_select(raw, resid, R, Kc, c.eps_seq)
        M = ki.shape[1]
        res = [sc, kp, ki, rs, bs]
        for l in range(2):
            q, k, v = (t[:, :M].contiguous() for t in qkv[l])
            o, ls = tg.tg_gated_attention(q, k, v, bs, ki, gains[l], temp, want_lse=True)
            res += [o, ls]
        return M, res

    K_dev.fill_(budgets[0])
    run_padded()  # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_padded()
    torch.cuda.synchronize()
    say(f"graph: gate N={N} + 2 attention layers, padded kept length {M_pad}")
    for rep, Kb in enumerate(budgets):
        for t in (score, b_S, lse):
            t.fill_(float("nan"))
        for t in (keep, kept_idx, resid_S, *outs):
            t.view(torch.uint8).fill_(0xA5)
        K_dev.fill_(Kb)
        graph.replay()
        torch.cuda.synchronize()
        M, ref = eager(Kb)  # eager work between the replays
        torch.cuda.synchronize()
        assert int(kept_count.item()) == M
        got = [score, keep, kept_idx[:, :M], resid_S[:, :M], b_S[:, :M], outs[0][:, :M], None, outs[1][:, :M],
               lse[:, :, :M]]
        names = ["score", "keep", "kept_idx", "resid_S", "b_S", "out0", None, "out1", "lse1"]
        for x, y, name in zip(got, ref, names):
            if x is None:
                continue
            assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), \
                f"replay {rep} (K={Kb}): {name} differs from the plain calls"
        # rows past the kept length are untouched
        assert bool((kept_idx[:, M:].view(torch.uint8) == 0xA5).all())
        assert bool((outs[0][:, M:].view(torch.uint8) == 0xA5).all())
        assert bool(torch.isnan(lse[:, :, M:]).all())
        # the oracle: selection and compaction on the GPU's scores, attention
        # of layer 1 on the kept set
        sc = score.cpu().numpy()
        k_ref = oracle.topk_select(sc, R, min(Kb, M_pad - R))
        np.testing.assert_array_equal(keep.cpu().numpy(), k_ref)
        ki, rs, bs = oracle.compact(c.resid, k_ref, sc)
        np.testing.assert_array_equal(kept_idx[:, :M].cpu().numpy(), ki)
        np.testing.assert_array_equal(host_bits(resid_S[:, :M]), rs)
        q, k, v = (host_bits(t[:, :M]) for t in qkv[1])
        O, L = oracle.gated_attention(q, k, v, bs.astype(np.float32), ki, gains[1].cpu().numpy(),
                                      temp.cpu().numpy(), DH ** -0.5)
        assert_close(wl.bf16_bits_to_f32(host_bits(outs[1][:, :M])), O, TOL_BF16, f"K={Kb} O")
        assert_close(lse[:, :, :M].cpu().numpy(), L, TOL_LSE, f"K={Kb} lse")
        say(f"  replay {rep}: K={Kb} -> M={M}, bit-identical to the plain calls, oracle-checked")
