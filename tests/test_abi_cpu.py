"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before enqueueing anything.

Every call here fails validation, so no kernel is launched and no HIP call is
made; the pointers passed are fake (aligned, never dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")

import learned_token_pruning_07_amd as tgb  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(tgb.LIB_PATH),
                                reason="libtokengate.so not built (run __graft_entry__.build())")

FAKE = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10002)  # misaligned
NULL = None


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(tg_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return tgb.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(tgb.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_workspace(lib):
    assert lib.tg_version() == 10000
    # scorer: W1 with the RMSNorm weight folded in (bf16)
    assert lib.tg_workspace_size(tgb.TG_OP_GATE_SCORE, 1, 16384, 2048, 256, 1638) == 256 * 2048 * 2
    for op in (tgb.TG_OP_SEQ_RMSNORM, tgb.TG_OP_TOPK_SELECT, tgb.TG_OP_COMPACT):
        assert lib.tg_workspace_size(op, 1, 16384, 2048, 256, 1638) == 0
        assert lib.tg_workspace_size(op, 1, 32768, 2048, 256, 1638) == 0
    # rows beyond 32768 tokens: fp64 partial sums per 8192-score slice; digit histograms
    assert lib.tg_workspace_size(tgb.TG_OP_SEQ_RMSNORM, 2, 131072, 0, 0, 0) == 2 * 16 * 8
    assert lib.tg_workspace_size(tgb.TG_OP_SEQ_RMSNORM, 1, 32769, 0, 0, 0) == 5 * 8
    assert lib.tg_workspace_size(tgb.TG_OP_TOPK_SELECT, 2, 131072, 0, 0, 0) == 2 * (2048 + 2048 + 1024 + 4) * 4
    assert lib.tg_workspace_size(tgb.TG_OP_COMPACT, 1, 131072, 2048, 0, 0) == 0
    # fused selection: none up to 32768 tokens, else the larger of the two it runs in sequence
    assert lib.tg_workspace_size(tgb.TG_OP_GATE_SELECT, 1, 32768, 2048, 0, 0) == 0
    assert lib.tg_workspace_size(tgb.TG_OP_GATE_SELECT, 2, 131072, 2048, 0, 0) == 2 * (2048 + 2048 + 1024 + 4) * 4
    # attention: fp16 V^T copy and fp32 per-head key-score terms, kept length padded to 64 keys
    # V^T (fp16) plus one key-term row per query head and one V^T scale row per KV head
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 1, 3341, 8 * 128, 16, 128) == \
        3392 * (8 * 128 * 2 + (16 + 8) * 4)
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 2, 64, 2 * 64, 4, 64) == 2 * 64 * (2 * 64 * 2 + 6 * 4)
    # K = 0: sized for the largest possible Hkv (= Hq)
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 1, 3341, 8 * 128, 16, 0) == \
        3392 * (8 * 128 * 2 + 32 * 4)
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 1, 64, 2 * 64, 0, 64) == 0   # Hq is required
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 1, 64, 2 * 64, 4, 48) == 0   # d_h must divide d
    # the rotary variant adds the rotated k [B, M, Hkv, d_h] (bf16) and the angle table of the
    # padded slots [B, round_up(M, 64), d_h / 2] (cos, sin) (fp32); K = d_h
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_ROPE, 1, 3341, 8 * 128, 16, 128) == \
        3392 * (8 * 128 * 2 + (16 + 8) * 4) + 3341 * 128 * 2 * 8 + 3392 * 128 * 4
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_ROPE, 1, 64, 2 * 64, 4, 0) == 0   # d_h is required


def _err(lib):
    return lib.tg_last_error().decode()


def test_gate_score_validation(lib):
    args = dict(resid=FAKE, dt=tgb.TG_BF16, B=1, N=128, d=256, r=4, norm_w=FAKE, eps=1e-6, W1=FAKE, b1=FAKE,
                h=256, w2=FAKE, b2=FAKE, out=FAKE, ws=NULL, ws_bytes=0)

    def call(**kw):
        a = dict(args, **kw)
        return lib.tg_gate_score(a["resid"], a["dt"], a["B"], a["N"], a["d"], a["r"], a["norm_w"], a["eps"],
                                 a["W1"], a["b1"], a["h"], a["w2"], a["b2"], a["out"], a["ws"], a["ws_bytes"], None)

    assert call(resid=NULL) == tgb.TG_EINVAL and "null" in _err(lib)
    assert call(N=0) == tgb.TG_EINVAL
    assert call(r=129) == tgb.TG_EINVAL and "outside" in _err(lib)
    assert call(r=-1) == tgb.TG_EINVAL
    assert call(dt=7) == tgb.TG_EINVAL
    assert call(resid=FAKE_ODD) == tgb.TG_EINVAL and "aligned" in _err(lib)
    assert call(d=250) == tgb.TG_EUNSUPPORTED
    assert call(d=136) == tgb.TG_EUNSUPPORTED              # bf16 MFMA path streams 64-column chunks
    assert call() == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(ws=FAKE, ws_bytes=1000) == tgb.TG_EINVAL
    assert call(ws=FAKE_ODD, ws_bytes=1 << 20) == tgb.TG_EINVAL
    assert call(h=96) == tgb.TG_EUNSUPPORTED
    assert call(dt=tgb.TG_F32, d=8192) == tgb.TG_EUNSUPPORTED
    assert call(eps=-1.0) == tgb.TG_EINVAL


def test_seq_rmsnorm_and_topk_validation(lib):
    assert lib.tg_seq_rmsnorm(NULL, 1, 10, 0, 1e-6, FAKE, None, 0, None) == tgb.TG_EINVAL
    assert lib.tg_seq_rmsnorm(FAKE, 1, 10, 11, 1e-6, FAKE, None, 0, None) == tgb.TG_EINVAL
    assert lib.tg_seq_rmsnorm(FAKE, 0, 10, 0, 1e-6, FAKE, None, 0, None) == tgb.TG_EINVAL
    assert lib.tg_topk_select(FAKE, 1, 10, 0, -1, FAKE, None, 0, None) == tgb.TG_EINVAL
    assert "K=-1" in _err(lib)
    assert lib.tg_topk_select(FAKE, 1, 10, 0, 3, NULL, None, 0, None) == tgb.TG_EINVAL
    assert lib.tg_topk_select(FAKE, 1, 10, 12, 3, FAKE, None, 0, None) == tgb.TG_EINVAL
    # long rows need a workspace
    assert lib.tg_seq_rmsnorm(FAKE, 1, 40000, 0, 1e-6, FAKE, None, 0, None) == tgb.TG_EINVAL
    assert "workspace" in _err(lib)
    assert lib.tg_seq_rmsnorm(FAKE, 1, 40000, 0, 1e-6, FAKE, FAKE, 8, None) == tgb.TG_EINVAL
    assert lib.tg_seq_rmsnorm(FAKE, 1, 40000, 0, 1e-6, FAKE, FAKE_ODD, 1 << 20, None) == tgb.TG_EINVAL
    assert lib.tg_topk_select(FAKE, 1, 40000, 0, 3, FAKE, None, 0, None) == tgb.TG_EINVAL
    assert "workspace" in _err(lib)
    assert lib.tg_topk_select(FAKE, 1, 40000, 0, 3, FAKE, FAKE, 100, None) == tgb.TG_EINVAL


def test_compact_validation(lib):
    def call(**kw):
        a = dict(resid=FAKE, dt=tgb.TG_BF16, B=1, N=100, d=64, keep=FAKE, score=FAKE, M=10, ki=FAKE, ro=FAKE,
                 so=FAKE)
        a.update(kw)
        return lib.tg_compact(a["resid"], a["dt"], a["B"], a["N"], a["d"], a["keep"], a["score"], a["M"], a["ki"],
                              a["ro"], a["so"], None, 0, None)

    assert call(M=101) == tgb.TG_EINVAL
    assert call(M=-1) == tgb.TG_EINVAL
    assert call(ki=NULL) == tgb.TG_EINVAL
    assert call(d=4) == tgb.TG_EUNSUPPORTED      # 8-byte rows
    assert call(ro=FAKE_ODD) == tgb.TG_EINVAL


def test_gate_select_validation(lib):
    def call(**kw):
        a = dict(raw=FAKE, B=1, N=100, r=4, eps=1e-6, K=10, resid=FAKE, dt=tgb.TG_BF16, d=64, score=FAKE, keep=FAKE,
                 ki=FAKE, ro=FAKE, so=FAKE, ws=NULL, ws_bytes=0)
        a.update(kw)
        return lib.tg_gate_select(a["raw"], a["B"], a["N"], a["r"], a["eps"], a["K"], a["resid"], a["dt"], a["d"],
                                  a["score"], a["keep"], a["ki"], a["ro"], a["so"], a["ws"], a["ws_bytes"], None)

    assert call(raw=NULL) == tgb.TG_EINVAL and "null" in _err(lib)
    assert call(K=-1) == tgb.TG_EINVAL and "K=-1" in _err(lib)
    assert call(r=101) == tgb.TG_EINVAL and "outside" in _err(lib)
    assert call(dt=3) == tgb.TG_EINVAL
    assert call(d=4) == tgb.TG_EUNSUPPORTED      # 8-byte rows
    assert call(ro=FAKE_ODD) == tgb.TG_EINVAL and "misaligned" in _err(lib)
    assert call(eps=-1.0) == tgb.TG_EINVAL
    assert call(ki=NULL) == tgb.TG_EINVAL
    # long rows need the workspace of the calls they run
    assert call(N=40000) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(N=40000, ws=FAKE, ws_bytes=100) == tgb.TG_EINVAL
    assert call(N=40000, ws=FAKE_ODD, ws_bytes=1 << 20) == tgb.TG_EINVAL


def test_attention_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, M=64, Hq=16, Hkv=8, dh=128, ks=FAKE, pos=FAKE, gain=FAKE, temp=FAKE,
                 scale=0.088, out=FAKE, lse=NULL, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.tg_gated_attention(a["q"], a["k"], a["v"], a["B"], a["M"], a["Hq"], a["Hkv"], a["dh"], a["ks"],
                                      a["pos"], a["gain"], a["temp"], a["scale"], a["out"], a["lse"], a["ws"],
                                      a["ws_bytes"], None)

    assert call(Hkv=5) == tgb.TG_EINVAL and "multiple" in _err(lib)
    assert call(dh=96) == tgb.TG_EUNSUPPORTED
    assert call(Hq=16, Hkv=2) == tgb.TG_EUNSUPPORTED   # group of 8
    assert call(q=NULL) == tgb.TG_EINVAL
    assert call(out=FAKE_ODD) == tgb.TG_EINVAL
    assert call(scale=0.0) == tgb.TG_EINVAL
    assert call(B=0) == tgb.TG_EINVAL
    assert call(M=0, q=NULL) == tgb.TG_OK             # empty kept set: a no-op that touches nothing
    assert call(ws=NULL) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(ws_bytes=1000) == tgb.TG_EINVAL
    assert call(ws=FAKE_ODD) == tgb.TG_EINVAL


def test_attention_rope_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, M=64, Hq=16, Hkv=8, dh=128, ks=FAKE, pos=FAKE, gain=FAKE, temp=FAKE,
                 scale=0.088, base=1e6, out=FAKE, lse=NULL, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.tg_gated_attention_rope(a["q"], a["k"], a["v"], a["B"], a["M"], a["Hq"], a["Hkv"], a["dh"],
                                           a["ks"], a["pos"], a["gain"], a["temp"], a["scale"], a["base"], a["out"],
                                           a["lse"], a["ws"], a["ws_bytes"], None)

    assert call(base=1.0) == tgb.TG_EINVAL and "rope_base" in _err(lib)
    assert call(base=float("nan")) == tgb.TG_EINVAL
    assert call(base=float("inf")) == tgb.TG_EINVAL
    assert call(dh=96) == tgb.TG_EUNSUPPORTED
    assert call(q=NULL) == tgb.TG_EINVAL
    # the plain attention's workspace is too small for the rotated copies
    plain = lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 1, 64, 8 * 128, 16, 0)
    assert call(ws_bytes=plain) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(M=0, q=NULL) == tgb.TG_OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tgb.tg_gate_score(x, 0, torch.ones(16, dtype=torch.bfloat16), torch.zeros(64, 16, dtype=torch.bfloat16),
                          torch.zeros(64), torch.zeros(64, dtype=torch.bfloat16), torch.zeros(1))


def test_attention_backward_workspace_size(lib):
    for B, M, Hq, Hkv, dh in [(1, 3341, 16, 8, 128), (2, 100, 4, 4, 64), (1, 64, 8, 2, 128)]:
        Mp = (M + 63) // 64 * 64
        want = B * Mp * (12 * Hq + 4 * Hkv) + 8 * B * (Mp // 64) * Hq
        assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_BACKWARD, B, M, Hkv * dh, Hq, dh) == want
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_BACKWARD, 1, 0, 1024, 16, 128) == 0
    assert lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_BACKWARD, 1, 64, 1000, 16, 128) == 0  # d % d_h != 0


def test_attention_backward_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, B=1, M=64, Hq=16, Hkv=8, dh=128, ks=FAKE,
                 pos=FAKE, gain=FAKE, temp=FAKE, scale=0.088, dq=FAKE, dk=FAKE, dv=FAKE, db=FAKE, dg=FAKE, dt=FAKE,
                 ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.tg_gated_attention_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["B"], a["M"],
                                               a["Hq"], a["Hkv"], a["dh"], a["ks"], a["pos"], a["gain"], a["temp"],
                                               a["scale"], a["dq"], a["dk"], a["dv"], a["db"], a["dg"], a["dt"],
                                               a["ws"], a["ws_bytes"], None)

    assert call(dh=96) == tgb.TG_EUNSUPPORTED
    assert call(Hq=24, Hkv=3) == tgb.TG_EUNSUPPORTED          # group of 8
    assert call(Hq=16, Hkv=6) == tgb.TG_EINVAL                # not a multiple
    assert call(B=0) == tgb.TG_EINVAL and call(B=65536) == tgb.TG_EINVAL
    assert call(M=-1) == tgb.TG_EINVAL
    for name in ("q", "k", "v", "o", "lse", "do", "ks", "pos", "dq", "dk", "dv", "db", "dg", "dt", "gain", "temp"):
        assert call(**{name: NULL}) == tgb.TG_EINVAL, name
    assert call(do=FAKE_ODD) == tgb.TG_EINVAL and "misaligned" in _err(lib)
    assert call(scale=0.0) == tgb.TG_EINVAL
    need = lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_BACKWARD, 1, 64, 8 * 128, 16, 128)
    assert call(ws_bytes=need - 1) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(ws=NULL) == tgb.TG_EINVAL
    assert call(M=1 << 20, Hq=64, Hkv=16) == tgb.TG_EUNSUPPORTED  # a 32-bit buffer range would overflow


def test_kv_cache_prune_validation(lib):
    def call(**kw):
        a = dict(k=FAKE, v=FAKE, L=5, B=1, N=100, H=8, dh=128, idx=FAKE, M=10, ko=FAKE, vo=FAKE)
        a.update(kw)
        return lib.tg_kv_cache_prune(a["k"], a["v"], a["L"], a["B"], a["N"], a["H"], a["dh"], a["idx"], a["M"],
                                     a["ko"], a["vo"], None)

    assert call(M=101) == tgb.TG_EINVAL and "outside" in _err(lib)
    assert call(M=-1) == tgb.TG_EINVAL
    assert call(dh=12) == tgb.TG_EUNSUPPORTED
    assert call(L=-1) == tgb.TG_EINVAL and call(B=0) == tgb.TG_EINVAL and call(N=0) == tgb.TG_EINVAL
    for name in ("k", "v", "idx", "ko", "vo"):
        assert call(**{name: NULL}) == tgb.TG_EINVAL, name
    assert call(ko=FAKE_ODD) == tgb.TG_EINVAL and "misaligned" in _err(lib)
    # nothing to do: no GPU call is made
    assert call(M=0, k=NULL) == tgb.TG_OK
    assert call(L=0, k=NULL) == tgb.TG_OK


def test_span_entry_points_validate_the_span(lib):
    # a span outside [0, N] or reversed is refused before anything runs
    assert lib.tg_seq_rmsnorm_span(FAKE, 1, 100, 50, 40, 1e-6, FAKE, NULL, 0, None) == tgb.TG_EINVAL
    assert "span" in _err(lib)
    assert lib.tg_seq_rmsnorm_span(FAKE, 1, 100, 0, 101, 1e-6, FAKE, NULL, 0, None) == tgb.TG_EINVAL
    assert lib.tg_topk_select_span(FAKE, 1, 100, -1, 50, 5, FAKE, NULL, 0, None) == tgb.TG_EINVAL
    assert lib.tg_gate_select_span(FAKE, 1, 100, 60, 50, 1e-6, 5, FAKE, tgb.TG_BF16, 64, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, NULL, 0, None) == tgb.TG_EINVAL
    assert lib.tg_gate_score_span(FAKE, tgb.TG_BF16, 1, 100, 256, 10, 120, FAKE, 1e-6, FAKE, FAKE, 64, FAKE, FAKE,
                                  FAKE, FAKE, 1 << 20, None) == tgb.TG_EINVAL
    assert "tg_gate_score_span" in _err(lib)


def test_attention_rope_backward_validation(lib):
    def call(base=1e6, ws_bytes=1 << 30, **kw):
        a = dict(q=FAKE, M=64)
        a.update(kw)
        return lib.tg_gated_attention_rope_backward(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, 1, a["M"], 16, 8, 128, FAKE,
                                                    FAKE, FAKE, FAKE, 0.088, base, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                    FAKE, ws_bytes, None)

    assert call(base=1.0) == tgb.TG_EINVAL and "rope_base" in _err(lib)
    assert call(base=float("nan")) == tgb.TG_EINVAL
    assert call(q=NULL) == tgb.TG_EINVAL
    plain = lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_BACKWARD, 1, 64, 8 * 128, 16, 128)
    rope = lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_ROPE_BACKWARD, 1, 64, 8 * 128, 16, 128)
    assert rope == (plain + 15) // 16 * 16 + 6 * 64 * 24 * 128
    assert call(ws_bytes=plain) == tgb.TG_EINVAL and "workspace" in _err(lib)


def test_attention_varlen_validation(lib):
    def call(cu, ws_bytes=1 << 30):
        arr = (ctypes.c_int32 * len(cu))(*cu)
        return lib.tg_gated_attention_varlen(FAKE, FAKE, FAKE, len(cu) - 1, arr, 16, 8, 128, FAKE, FAKE, FAKE, FAKE,
                                             0.088, FAKE, NULL, FAKE, ws_bytes, None)

    assert call([1, 5]) == tgb.TG_EINVAL and "cu_seqlens[0]" in _err(lib)
    assert call([0, 5, 3]) == tgb.TG_EINVAL and "non-decreasing" in _err(lib)
    small = lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 1, 100, 8 * 128, 16, 0)
    assert call([0, 100, 300], ws_bytes=small) == tgb.TG_EINVAL and "workspace" in _err(lib)  # sized by the longest
    assert call([0, 0, 0]) == tgb.TG_OK  # nothing to do: no GPU call


def test_attention_varlen_checks_heads_before_sizing(lib):
    """Bad head counts are refused as such, before the workspace is sized."""
    cu = (ctypes.c_int32 * 2)(0, 100)

    def call(Hq, Hkv, dh=128):
        return lib.tg_gated_attention_varlen(FAKE, FAKE, FAKE, 1, cu, Hq, Hkv, dh, FAKE, FAKE, FAKE, FAKE, 0.088,
                                             FAKE, NULL, FAKE, 1 << 30, None)

    assert call(-16, 8) == tgb.TG_EINVAL and "bad sizes" in _err(lib)
    assert call(16, -8) == tgb.TG_EINVAL and "bad sizes" in _err(lib)
    assert call(16, 0) == tgb.TG_EINVAL and "bad sizes" in _err(lib)
    assert call(12, 8) == tgb.TG_EINVAL and "multiple" in _err(lib)
    assert call(16, 8, dh=96) == tgb.TG_EUNSUPPORTED and "d_h" in _err(lib)


def test_attention_varlen_validates_every_sequence_first(lib):
    """A bad second sequence is refused before the first is launched (no GPU
    call is made here: a launch would fail on this CPU-only machine)."""
    cu = (ctypes.c_int32 * 3)(0, 100, 200)
    # sequence 1 fine, sequence 2 fine in size, but d_h unsupported for both -> refused up front
    assert lib.tg_gated_attention_varlen(FAKE, FAKE, FAKE, 2, cu, 16, 8, 96, FAKE, FAKE, FAKE, FAKE, 0.088, FAKE,
                                         NULL, FAKE, 1 << 30, None) == tgb.TG_EUNSUPPORTED
    # misaligned key_score for the second sequence only (offset 100 * 4 bytes keeps alignment, so use the base)
    assert lib.tg_gated_attention_varlen(FAKE, FAKE, FAKE, 2, cu, 16, 8, 128, FAKE_ODD, FAKE, FAKE, FAKE, 0.088,
                                         FAKE, NULL, FAKE, 1 << 30, None) == tgb.TG_EINVAL


def test_attention_varlen_workspace_covers_every_sequence(lib):
    """The packed call needs every sequence's padded rows side by side:
    2 x 128 rows x (8 x 128 x 2 + 16 x 4) bytes for two sequences of 100."""
    cu = (ctypes.c_int32 * 3)(0, 100, 200)
    need = 256 * (8 * 128 * 2 + (16 + 8) * 4)
    assert lib.tg_gated_attention_varlen(FAKE, FAKE, FAKE, 2, cu, 16, 8, 128, FAKE, FAKE, FAKE, FAKE, 0.088, FAKE,
                                         NULL, FAKE, need - 1, None) == tgb.TG_EINVAL
    assert b"workspace" in lib.tg_last_error()


def test_gate_score_noalloc_refuses_oversized_weights(lib):
    """The no-allocation scorer holds the folded W1 in a fixed 4 MiB scratch:
    256 x 16384 bf16 (8 MiB) is refused before anything is launched."""
    def call(d, h=256, dt=tgb.TG_BF16):
        return lib.tg_gate_score_noalloc(FAKE, dt, 1, 8, d, 0, FAKE, 1e-6, FAKE, FAKE, h, FAKE, FAKE, FAKE, None)

    assert call(16384) == tgb.TG_EINVAL and "static scratch" in _err(lib)
    assert call(8192 + 64) == tgb.TG_EINVAL and "static scratch" in _err(lib)
    assert call(100) == tgb.TG_EUNSUPPORTED  # the plain scorer's shape rules still apply
    assert call(2048, h=96) == tgb.TG_EUNSUPPORTED


def test_padded_entry_points_validate(lib):
    """The budget and the kept length come from device memory; the host sizes
    (padded length, r, N) are checked before anything is launched."""
    def sel(N=4096, r=32, M_pad=512, kc=FAKE, K=FAKE):
        return lib.tg_gate_select_padded(FAKE, 1, N, r, 1e-6, K, M_pad, FAKE, tgb.TG_BF16, 512, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, kc, None)

    assert sel(M_pad=31) == tgb.TG_EINVAL and "M_pad" in _err(lib)      # below r
    assert sel(M_pad=4097) == tgb.TG_EINVAL and "M_pad" in _err(lib)    # above N
    assert sel(N=40000, M_pad=512) == tgb.TG_EUNSUPPORTED
    assert sel(kc=NULL) == tgb.TG_EINVAL and "null" in _err(lib)
    assert sel(K=FAKE_ODD) == tgb.TG_EINVAL and "misaligned" in _err(lib)

    def attn(kc=FAKE, ws_bytes=1 << 30, dh=128):
        return lib.tg_gated_attention_padded(FAKE, FAKE, FAKE, 1, 512, kc, 16, 8, dh, FAKE, FAKE, FAKE, FAKE, 0.088,
                                             FAKE, NULL, FAKE, ws_bytes, None)

    assert attn(kc=NULL) == tgb.TG_EINVAL and "null" in _err(lib)
    assert attn(kc=FAKE_ODD) == tgb.TG_EINVAL and "misaligned" in _err(lib)
    assert attn(dh=96) == tgb.TG_EUNSUPPORTED
    need = lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION, 1, 512, 8 * 128, 16, 128)
    assert attn(ws_bytes=need - 1) == tgb.TG_EINVAL and "workspace" in _err(lib)


def test_fold_weights_and_folded_scorer_validate(lib):
    assert lib.tg_gate_fold_weights(FAKE, FAKE, tgb.TG_F32, 256, 2048, FAKE, 1 << 20, None) == tgb.TG_EUNSUPPORTED
    assert lib.tg_gate_fold_weights(FAKE, FAKE, tgb.TG_BF16, 256, 2048, FAKE, 256 * 2048 * 2 - 1, None) == \
        tgb.TG_EINVAL and "needed" in _err(lib)
    assert lib.tg_gate_fold_weights(FAKE, FAKE, tgb.TG_BF16, 96, 2048, FAKE, 1 << 30, None) == tgb.TG_EUNSUPPORTED
    assert lib.tg_gate_fold_weights(FAKE_ODD, FAKE, tgb.TG_BF16, 256, 2048, FAKE, 1 << 30, None) == tgb.TG_EINVAL

    def score(r=0, N=64, d=2048, h=256, dt=tgb.TG_BF16, w=FAKE):
        return lib.tg_gate_score_folded(FAKE, dt, 1, N, d, r, w, 1e-6, FAKE, h, FAKE, FAKE, FAKE, None)

    assert score(dt=tgb.TG_F32) == tgb.TG_EUNSUPPORTED
    assert score(r=65) == tgb.TG_EINVAL
    assert score(w=NULL) == tgb.TG_EINVAL and "null" in _err(lib)
    assert score(d=100) == tgb.TG_EUNSUPPORTED


def test_attention_rope_backward_varlen_validation(lib):
    """The rotary packed backward refuses a bad base and sizes its workspace as
    the packed backward's (each sequence padded to 64 rows) rounded to 16
    bytes, then T rows of rotated q and k (bf16) and their fp32 gradients;
    the documented tg_workspace_size bound covers it."""
    cu = (ctypes.c_int32 * 3)(0, 100, 200)
    Hq, Hkv, dh = 16, 8, 128

    def call(base=1e6, ws_bytes=1 << 30, dh_=dh):
        return lib.tg_gated_attention_rope_backward_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, cu, Hq, Hkv, dh_,
                                                           FAKE, FAKE, FAKE, FAKE, 0.088, base, FAKE, FAKE, FAKE,
                                                           FAKE, FAKE, FAKE, FAKE, ws_bytes, None)

    assert call(base=0.5) == tgb.TG_EINVAL and "rope_base" in _err(lib)
    assert call(base=float("inf")) == tgb.TG_EINVAL
    assert call(dh_=96) == tgb.TG_EUNSUPPORTED and "d_h" in _err(lib)
    slots = 256
    plain = slots * (12 * Hq + 4 * Hkv) + 8 * (slots // 64) * Hq
    need = (plain + 15) // 16 * 16 + 200 * (Hq + Hkv) * dh * 6
    assert call(ws_bytes=need - 1) == tgb.TG_EINVAL and "workspace" in _err(lib)
    bound = lib.tg_workspace_size(tgb.TG_OP_GATED_ATTENTION_ROPE_BACKWARD, 1, 200 + 63 * 2, Hkv * dh, Hq, dh)
    assert bound >= need


def test_gate_select_varlen_long_rows_need_the_workspace(lib):
    """Rows past 32768 tokens are selected by the sliced kernels, which need
    the workspace of TG_OP_GATE_SELECT at the padded width N."""
    B, N = 2, 70000
    arr = lambda: FAKE  # noqa: E731

    def call(ws, ws_bytes):
        return lib.tg_gate_select_varlen(FAKE, B, N, arr(), arr(), arr(), arr(), arr(), 1000, 1e-6, FAKE,
                                         tgb.TG_BF16, 256, FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)

    need = lib.tg_workspace_size(tgb.TG_OP_GATE_SELECT, B, N, 0, 0, 0)
    assert need == max(B * 9 * 8, B * 5124 * 4)  # 9 fp64 slice sums per row vs the digit histograms
    assert call(NULL, 0) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(FAKE, need - 1) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(FAKE_ODD, need) == tgb.TG_EINVAL and "misaligned" in _err(lib)


def test_gate_fused_validation(lib):
    """tg_gate: bf16 rows of up to 32768 tokens, d a multiple of 64, h of
    64 / 128 / 256, and B zeroed counting words in the workspace."""
    args = dict(resid=FAKE, dt=tgb.TG_BF16, B=2, N=4096, d=256, r=4, W1=FAKE, eps_row=1e-6, b1=FAKE, h=128,
                w2=FAKE, b2=FAKE, eps_seq=1e-6, K=100, raw=FAKE, score=FAKE, keep=FAKE, ki=FAKE, ro=FAKE, so=FAKE,
                ws=FAKE, ws_bytes=8)

    def call(**kw):
        a = dict(args, **kw)
        return lib.tg_gate(a["resid"], a["dt"], a["B"], a["N"], a["d"], a["r"], a["W1"], a["eps_row"], a["b1"],
                           a["h"], a["w2"], a["b2"], a["eps_seq"], a["K"], a["raw"], a["score"], a["keep"], a["ki"],
                           a["ro"], a["so"], a["ws"], a["ws_bytes"], None)

    assert call(dt=tgb.TG_F32) == tgb.TG_EUNSUPPORTED and "bf16" in _err(lib)
    assert call(N=32769) == tgb.TG_EUNSUPPORTED and "32768" in _err(lib)
    assert call(N=0) == tgb.TG_EINVAL
    assert call(B=0) == tgb.TG_EINVAL
    assert call(r=4097) == tgb.TG_EINVAL and "outside" in _err(lib)
    assert call(K=-1) == tgb.TG_EINVAL
    assert call(eps_seq=-1.0) == tgb.TG_EINVAL
    assert call(resid=NULL) == tgb.TG_EINVAL and "null" in _err(lib)
    assert call(ki=NULL) == tgb.TG_EINVAL and "null" in _err(lib)
    assert call(resid=FAKE_ODD) == tgb.TG_EINVAL and "misaligned" in _err(lib)
    assert call(d=136) == tgb.TG_EUNSUPPORTED
    assert call(h=96) == tgb.TG_EUNSUPPORTED
    assert call(ws=NULL, ws_bytes=0) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(ws_bytes=7) == tgb.TG_EINVAL and "workspace" in _err(lib)
    assert call(ws=FAKE_ODD) == tgb.TG_EINVAL and "misaligned" in _err(lib)


def test_attention_backward_varlen_sizes_checked_before_the_workspace(lib):
    """Bad head counts and d_h are reported as such, not as a workspace of
    some size derived from them (both packed backward entry points)."""
    cu = (ctypes.c_int32 * 3)(0, 100, 200)

    def call(Hq, Hkv, dh, rope):
        if rope:
            return lib.tg_gated_attention_rope_backward_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, cu, Hq, Hkv, dh,
                                                               FAKE, FAKE, FAKE, FAKE, 0.088, 1e6, FAKE, FAKE, FAKE,
                                                               FAKE, FAKE, FAKE, NULL, 0, None)
        return lib.tg_gated_attention_backward_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, cu, Hq, Hkv, dh, FAKE,
                                                      FAKE, FAKE, FAKE, 0.088, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                      NULL, 0, None)

    for rope in (False, True):
        assert call(-16, 8, 128, rope) == tgb.TG_EINVAL and "bad sizes" in _err(lib)
        assert call(16, 0, 128, rope) == tgb.TG_EINVAL and "bad sizes" in _err(lib)
        assert call(16, 6, 128, rope) == tgb.TG_EINVAL and "multiple" in _err(lib)
        assert call(16, 8, 96, rope) == tgb.TG_EUNSUPPORTED and "d_h" in _err(lib)
        assert call(16, 8, 128, rope) == tgb.TG_EINVAL and "workspace" in _err(lib)
