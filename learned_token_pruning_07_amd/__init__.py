"""TokenGate gated-prefill path on MI355X (gfx950): Python binding.

A thin ctypes layer over ``libtokengate.so`` (C ABI declared in
``include/tokengate.h``).  Each function takes torch tensors that already live
on the GPU, checks their dtype/shape/contiguity, and passes raw device
pointers plus torch's current HIP stream to the library.  Every step of the
path runs in the library's HIP kernels; nothing here computes.

If the shared library has not been built, every call raises: there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtokengate.so")

TG_OK, TG_EINVAL, TG_EUNSUPPORTED, TG_EHIP = 0, 1, 2, 3
TG_F32, TG_BF16 = 0, 1
(TG_OP_GATE_SCORE, TG_OP_SEQ_RMSNORM, TG_OP_TOPK_SELECT, TG_OP_COMPACT, TG_OP_GATED_ATTENTION, TG_OP_GATE_SELECT,
 TG_OP_GATED_ATTENTION_ROPE, TG_OP_GATED_ATTENTION_BACKWARD, TG_OP_GATED_ATTENTION_ROPE_BACKWARD) = range(9)

EXPORTED = ("tg_gate_score", "tg_seq_rmsnorm", "tg_topk_select", "tg_compact", "tg_gate_select", "tg_gated_attention",
            "tg_gated_attention_rope", "tg_gated_attention_backward", "tg_gated_attention_rope_backward", "tg_kv_cache_prune", "tg_gate_score_span", "tg_seq_rmsnorm_span",
            "tg_topk_select_span", "tg_gate_select_span", "tg_gate_select_varlen", "tg_gate_score_varlen", "tg_gated_attention_varlen",
            "tg_gated_attention_backward_varlen", "tg_gate_score_noalloc", "tg_gate_select_padded",
            "tg_gated_attention_padded", "tg_gate_fold_weights", "tg_gate_score_folded",
            "tg_gated_attention_rope_varlen", "tg_gated_attention_rope_backward_varlen", "tg_gate", "tg_workspace_size",
            "tg_last_error", "tg_version")

_lib = None


class TokenGateError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[tg status {code}] {msg}")
        self.code = code


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libtokengate.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it first (python -m learned_token_pruning_07_amd._build)")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.tg_gate_score.argtypes = [vp, i, i, i, i, i, vp, f, vp, vp, i, vp, vp, vp, vp, sz, vp]
    lib.tg_seq_rmsnorm.argtypes = [vp, i, i, i, f, vp, vp, sz, vp]
    lib.tg_topk_select.argtypes = [vp, i, i, i, i, vp, vp, sz, vp]
    lib.tg_compact.argtypes = [vp, i, i, i, i, vp, vp, i, vp, vp, vp, vp, sz, vp]
    lib.tg_gated_attention.argtypes = [vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, f, vp, vp, vp, sz, vp]
    lib.tg_gate_select.argtypes = [vp, i, i, i, f, i, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tg_gated_attention_rope.argtypes = [vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, f, ctypes.c_double, vp, vp,
                                            vp, sz, vp]
    lib.tg_gated_attention_backward.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, f, vp, vp, vp,
                                                vp, vp, vp, vp, sz, vp]
    lib.tg_gated_attention_rope_backward.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, f,
                                                     ctypes.c_double, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tg_kv_cache_prune.argtypes = [vp, vp, i, i, i, i, i, vp, i, vp, vp, vp]
    lib.tg_gate_score_span.argtypes = [vp, i, i, i, i, i, i, vp, f, vp, vp, i, vp, vp, vp, vp, sz, vp]
    lib.tg_gate_score_noalloc.argtypes = [vp, i, i, i, i, i, vp, f, vp, vp, i, vp, vp, vp, vp]
    lib.tg_gate_fold_weights.argtypes = [vp, vp, i, i, i, vp, sz, vp]
    lib.tg_gate_score_folded.argtypes = [vp, i, i, i, i, i, vp, f, vp, i, vp, vp, vp, vp]
    lib.tg_gate.argtypes = [vp, i, i, i, i, i, vp, f, vp, i, vp, vp, f, i, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tg_gate_select_padded.argtypes = [vp, i, i, i, f, vp, i, vp, i, i, vp, vp, vp, vp, vp, vp, vp]
    lib.tg_gated_attention_padded.argtypes = [vp, vp, vp, i, i, vp, i, i, i, vp, vp, vp, vp, f, vp, vp, vp, sz, vp]
    lib.tg_seq_rmsnorm_span.argtypes = [vp, i, i, i, i, f, vp, vp, sz, vp]
    lib.tg_topk_select_span.argtypes = [vp, i, i, i, i, i, vp, vp, sz, vp]
    lib.tg_gated_attention_backward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, i, i, i, vp, vp, vp, vp, f,
                                                       vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tg_gated_attention_rope_backward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, i, i, i, vp, vp, vp, vp,
                                                            f, ctypes.c_double, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tg_gated_attention_varlen.argtypes = [vp, vp, vp, i, vp, i, i, i, vp, vp, vp, vp, f, vp, vp, vp, sz, vp]
    lib.tg_gated_attention_rope_varlen.argtypes = [vp, vp, vp, i, vp, i, i, i, vp, vp, vp, vp, f, ctypes.c_double,
                                                   vp, vp, vp, sz, vp]
    lib.tg_gate_score_varlen.argtypes = [vp, i, i, i, i, vp, vp, i, vp, f, vp, vp, i, vp, vp, vp, vp, sz, vp]
    lib.tg_gate_select_varlen.argtypes = [vp, i, i, vp, vp, vp, vp, vp, i, f, vp, i, i, vp, vp, vp, vp, vp, vp, sz,
                                          vp]
    lib.tg_gate_select_span.argtypes = [vp, i, i, i, i, f, i, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tg_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.tg_workspace_size.restype = sz
    lib.tg_last_error.argtypes = []
    lib.tg_last_error.restype = ctypes.c_char_p
    lib.tg_version.argtypes = []
    lib.tg_version.restype = i
    for name in ("tg_gate_score", "tg_seq_rmsnorm", "tg_topk_select", "tg_compact", "tg_gated_attention",
                 "tg_gate_select", "tg_gated_attention_rope", "tg_gated_attention_backward",
                 "tg_gated_attention_rope_backward", "tg_kv_cache_prune", "tg_gate_score_span", "tg_seq_rmsnorm_span", "tg_topk_select_span",
                 "tg_gate_select_span", "tg_gate_select_varlen", "tg_gate_score_varlen",
                 "tg_gated_attention_varlen", "tg_gated_attention_backward_varlen", "tg_gate_score_noalloc",
                 "tg_gate_select_padded", "tg_gated_attention_padded", "tg_gate_fold_weights",
                 "tg_gate_score_folded", "tg_gated_attention_rope_varlen",
                 "tg_gated_attention_rope_backward_varlen", "tg_gate"):
        getattr(lib, name).restype = i
    if path is None:
        _lib = lib
    return lib


def _check(code: int) -> None:
    if code != TG_OK:
        msg = load_library().tg_last_error().decode(errors="replace")
        raise TokenGateError(code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TG_BF16
    if t.dtype == torch.float32:
        return TG_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


# --------------------------------------------------------------- entry points
def gate_workspace(h: int, d: int, device="cuda") -> torch.Tensor:
    """A workspace tensor large enough for tg_gate_score at these sizes."""
    n = int(load_library().tg_workspace_size(TG_OP_GATE_SCORE, 1, 1, d, h, 0))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def tg_gate_score(resid, r: int, norm_w, W1, b1, w2, b2, eps_row: float = 1e-6, score_raw=None, ws=None,
                  stream=None, span_end: int | None = None):
    """Row RMSNorm + scoring MLP -> raw scores ``[B, N]`` fp32 (0 outside the
    prunable span ``[r, span_end)``; ``span_end`` None means N).

    ``ws`` is a uint8 GPU tensor from :func:`gate_workspace` (allocated here
    when omitted)."""
    lib = load_library()
    _need(resid, "resid")
    B, N, d = resid.shape
    h = W1.shape[0]
    _need(norm_w, "norm_w", resid.dtype, (d,))
    _need(W1, "W1", resid.dtype, (h, d))
    _need(b1, "b1", torch.float32, (h,))
    _need(w2, "w2", resid.dtype, (h,))
    _need(b2, "b2", torch.float32, (1,))
    if score_raw is None:
        score_raw = torch.empty((B, N), dtype=torch.float32, device=resid.device)
    _need(score_raw, "score_raw", torch.float32, (B, N))
    if ws is None:
        ws = gate_workspace(h, d, resid.device)
    _need(ws, "ws", torch.uint8)
    rest = (_ptr(norm_w), eps_row, _ptr(W1), _ptr(b1), h, _ptr(w2), _ptr(b2), _ptr(score_raw), _ptr(ws), ws.numel(),
            _stream(stream))
    if span_end is None:
        _check(lib.tg_gate_score(_ptr(resid), _dt(resid), B, N, d, r, *rest))
    else:
        _check(lib.tg_gate_score_span(_ptr(resid), _dt(resid), B, N, d, r, span_end, *rest))
    return score_raw


def tg_gate_fold_weights(W1, norm_w, out=None, stream=None):
    """W1 [h, d] bf16 with the RMSNorm weight folded in, in the scorer's
    fragment order: a uint8 GPU tensor of h * d * 2 bytes for
    :func:`tg_gate_score_folded` (fold once per weight set)."""
    lib = load_library()
    h, d = W1.shape
    _need(W1, "W1", torch.bfloat16, (h, d))
    _need(norm_w, "norm_w", torch.bfloat16, (d,))
    if out is None:
        out = torch.empty(h * d * 2, dtype=torch.uint8, device=W1.device)
    _need(out, "out", torch.uint8)
    _check(lib.tg_gate_fold_weights(_ptr(W1), _ptr(norm_w), TG_BF16, h, d, _ptr(out), out.numel(), _stream(stream)))
    return out


def tg_gate_score_folded(resid, r: int, W1_folded, h: int, b1, w2, b2, eps_row: float = 1e-6, score_raw=None,
                         stream=None):
    """:func:`tg_gate_score` (bf16) on weights folded by :func:`tg_gate_fold_weights`."""
    lib = load_library()
    _need(resid, "resid", torch.bfloat16)
    B, N, d = resid.shape
    _need(W1_folded, "W1_folded", torch.uint8, (h * d * 2,))
    _need(b1, "b1", torch.float32, (h,))
    _need(w2, "w2", torch.bfloat16, (h,))
    _need(b2, "b2", torch.float32, (1,))
    if score_raw is None:
        score_raw = torch.empty((B, N), dtype=torch.float32, device=resid.device)
    _need(score_raw, "score_raw", torch.float32, (B, N))
    _check(lib.tg_gate_score_folded(_ptr(resid), TG_BF16, B, N, d, r, _ptr(W1_folded), eps_row, _ptr(b1), h, _ptr(w2),
                                    _ptr(b2), _ptr(score_raw), _stream(stream)))
    return score_raw


def gate_counters(B: int, device="cuda") -> torch.Tensor:
    """The row counters :func:`tg_gate` takes: B zeroed 32-bit words (every
    call leaves them zero, so one buffer serves all later calls that do not
    overlap in time)."""
    return torch.zeros(max(B, 1), dtype=torch.int32, device=device)


def tg_gate(resid, r: int, K: int, W1_folded, h: int, b1, w2, b2, eps_row: float = 1e-6, eps_seq: float = 1e-6,
            score_raw=None, score=None, keep=None, kept_idx=None, resid_out=None, score_out=None, counters=None,
            stream=None):
    """The whole gate in one call (bf16, N <= 32768): :func:`tg_gate_score_folded`
    then :func:`tg_gate_select`, bit for bit, in two launches.  Returns
    ``(kept_idx, resid_out, score_out, keep, score)`` as :func:`tg_gate_select`;
    ``counters`` from :func:`gate_counters` (made here when omitted)."""
    lib = load_library()
    _need(resid, "resid", torch.bfloat16)
    B, N, d = resid.shape
    _need(W1_folded, "W1_folded", torch.uint8, (h * d * 2,))
    dev = resid.device
    M = kept_count(N, r, K)
    if score_raw is None:
        score_raw = torch.empty((B, N), dtype=torch.float32, device=dev)
    if score is None:
        score = score_raw
    if keep is None:
        keep = torch.empty((B, N), dtype=torch.uint8, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((B, M), dtype=torch.int32, device=dev)
    if resid_out is None:
        resid_out = torch.empty((B, M, d), dtype=resid.dtype, device=dev)
    if score_out is None:
        score_out = torch.empty((B, M), dtype=torch.float32, device=dev)
    if counters is None:
        counters = gate_counters(B, dev)
    _need(counters, "counters", torch.int32)
    _check(lib.tg_gate(_ptr(resid), TG_BF16, B, N, d, r, _ptr(W1_folded), eps_row, _ptr(b1), h, _ptr(w2), _ptr(b2),
                       eps_seq, K, _ptr(score_raw), _ptr(score), _ptr(keep), _ptr(kept_idx), _ptr(resid_out),
                       _ptr(score_out), _ptr(counters), counters.numel() * 4, _stream(stream)))
    return kept_idx, resid_out, score_out, keep, score


def tg_gate_score_noalloc(resid, r: int, norm_w, W1, b1, w2, b2, eps_row: float = 1e-6, score_raw=None,
                          stream=None):
    """:func:`tg_gate_score` without a workspace: the library's fixed 4 MiB
    scratch holds the folded W1 (h * d * 2 bytes at most 4 MiB).  Calls that may
    overlap on one device race on that scratch.  ``score_raw`` must be given
    by callers that may not allocate."""
    lib = load_library()
    _need(resid, "resid")
    B, N, d = resid.shape
    h = W1.shape[0]
    _need(norm_w, "norm_w", resid.dtype, (d,))
    _need(W1, "W1", resid.dtype, (h, d))
    _need(b1, "b1", torch.float32, (h,))
    _need(w2, "w2", resid.dtype, (h,))
    _need(b2, "b2", torch.float32, (1,))
    if score_raw is None:
        score_raw = torch.empty((B, N), dtype=torch.float32, device=resid.device)
    _need(score_raw, "score_raw", torch.float32, (B, N))
    _check(lib.tg_gate_score_noalloc(_ptr(resid), _dt(resid), B, N, d, r, _ptr(norm_w), eps_row, _ptr(W1), _ptr(b1),
                                     h, _ptr(w2), _ptr(b2), _ptr(score_raw), _stream(stream)))
    return score_raw


def _op_workspace(op: int, B: int, N: int, device) -> torch.Tensor | None:
    n = int(load_library().tg_workspace_size(op, B, N, 0, 0, 0))
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def seq_rmsnorm_workspace(B: int, N: int, device="cuda") -> torch.Tensor | None:
    """A workspace for tg_seq_rmsnorm at these sizes (None when it needs none: N <= 32768)."""
    return _op_workspace(TG_OP_SEQ_RMSNORM, B, N, device)


def topk_workspace(B: int, N: int, device="cuda") -> torch.Tensor | None:
    """A workspace for tg_topk_select at these sizes (None when it needs none: N <= 32768)."""
    return _op_workspace(TG_OP_TOPK_SELECT, B, N, device)


def _ws_args(ws):
    if ws is None:
        return None, 0
    _need(ws, "ws", torch.uint8)
    return _ptr(ws), ws.numel()


def tg_seq_rmsnorm(score_raw, r: int, eps_seq: float = 1e-6, score=None, ws=None, stream=None,
                   span_end: int | None = None):
    """Sequence RMSNorm of the raw scores -> ``[B, N]`` fp32 (0 outside the
    prunable span ``[r, span_end)``; ``span_end`` None means N).

    ``ws``: from :func:`seq_rmsnorm_workspace` (allocated here when needed and omitted)."""
    lib = load_library()
    _need(score_raw, "score_raw", torch.float32)
    B, N = score_raw.shape
    if score is None:
        score = torch.empty_like(score_raw)
    _need(score, "score", torch.float32, (B, N))
    if ws is None:
        ws = seq_rmsnorm_workspace(B, N, score_raw.device)
    wp, wn = _ws_args(ws)
    if span_end is None:
        _check(lib.tg_seq_rmsnorm(_ptr(score_raw), B, N, r, eps_seq, _ptr(score), wp, wn, _stream(stream)))
    else:
        _check(lib.tg_seq_rmsnorm_span(_ptr(score_raw), B, N, r, span_end, eps_seq, _ptr(score), wp, wn,
                                       _stream(stream)))
    return score


def tg_topk_select(score, r: int, K: int, keep=None, ws=None, stream=None, span_end: int | None = None):
    """Keep mask ``[B, N]`` uint8 with :func:`kept_count` ones per row (the
    prunable span is ``[r, span_end)``; ``span_end`` None means N).

    ``ws``: from :func:`topk_workspace` (allocated here when needed and omitted)."""
    lib = load_library()
    _need(score, "score", torch.float32)
    B, N = score.shape
    if keep is None:
        keep = torch.empty((B, N), dtype=torch.uint8, device=score.device)
    _need(keep, "keep", torch.uint8, (B, N))
    if ws is None:
        ws = topk_workspace(B, N, score.device)
    wp, wn = _ws_args(ws)
    if span_end is None:
        _check(lib.tg_topk_select(_ptr(score), B, N, r, K, _ptr(keep), wp, wn, _stream(stream)))
    else:
        _check(lib.tg_topk_select_span(_ptr(score), B, N, r, span_end, K, _ptr(keep), wp, wn, _stream(stream)))
    return keep


def kept_count(N: int, r: int, K: int, span_end: int | None = None) -> int:
    """M = N - P + min(K, P), P = span_end - r (N - r by default): the number
    of kept tokens per sequence."""
    P = (N if span_end is None else span_end) - r
    return N - P + max(0, min(K, P))


def tg_compact(resid, keep, score, M: int, kept_idx=None, resid_out=None, score_out=None, stream=None):
    """Compact the residual stream to the kept set.

    Returns ``(kept_idx [B, M] int32, resid_out [B, M, d], score_out [B, M] fp32)``.
    """
    lib = load_library()
    _need(resid, "resid")
    B, N, d = resid.shape
    _need(keep, "keep", torch.uint8, (B, N))
    _need(score, "score", torch.float32, (B, N))
    dev = resid.device
    if kept_idx is None:
        kept_idx = torch.empty((B, M), dtype=torch.int32, device=dev)
    if resid_out is None:
        resid_out = torch.empty((B, M, d), dtype=resid.dtype, device=dev)
    if score_out is None:
        score_out = torch.empty((B, M), dtype=torch.float32, device=dev)
    _need(kept_idx, "kept_idx", torch.int32, (B, M))
    _need(resid_out, "resid_out", resid.dtype, (B, M, d))
    _need(score_out, "score_out", torch.float32, (B, M))
    _check(lib.tg_compact(_ptr(resid), _dt(resid), B, N, d, _ptr(keep), _ptr(score), M, _ptr(kept_idx),
                          _ptr(resid_out), _ptr(score_out), None, 0, _stream(stream)))
    return kept_idx, resid_out, score_out


def gate_select_workspace(B: int, N: int, device="cuda") -> torch.Tensor | None:
    """A workspace for tg_gate_select at these sizes (None when it needs none: N <= 32768)."""
    return _op_workspace(TG_OP_GATE_SELECT, B, N, device)


def tg_gate_select(score_raw, resid, r: int, K: int, eps_seq: float = 1e-6, score=None, keep=None, kept_idx=None,
                   resid_out=None, score_out=None, ws=None, stream=None, span_end: int | None = None):
    """tg_seq_rmsnorm, tg_topk_select and tg_compact in one call (bit-identical results).

    Returns ``(kept_idx [B, M] int32, resid_out [B, M, d], score_out [B, M] fp32, keep [B, N] uint8,
    score [B, N] fp32)`` with ``M = r + min(K, N - r)``.  ``score`` may be ``score_raw`` (in place).
    ``ws``: from :func:`gate_select_workspace` (allocated here when needed and omitted).
    """
    lib = load_library()
    _need(resid, "resid")
    B, N, d = resid.shape
    _need(score_raw, "score_raw", torch.float32, (B, N))
    dev = resid.device
    M = kept_count(N, r, K, span_end)
    if score is None:
        score = torch.empty((B, N), dtype=torch.float32, device=dev)
    if keep is None:
        keep = torch.empty((B, N), dtype=torch.uint8, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((B, M), dtype=torch.int32, device=dev)
    if resid_out is None:
        resid_out = torch.empty((B, M, d), dtype=resid.dtype, device=dev)
    if score_out is None:
        score_out = torch.empty((B, M), dtype=torch.float32, device=dev)
    _need(score, "score", torch.float32, (B, N))
    _need(keep, "keep", torch.uint8, (B, N))
    _need(kept_idx, "kept_idx", torch.int32, (B, M))
    _need(resid_out, "resid_out", resid.dtype, (B, M, d))
    _need(score_out, "score_out", torch.float32, (B, M))
    if ws is None:
        ws = gate_select_workspace(B, N, dev)
    wp, wn = _ws_args(ws)
    rest = (eps_seq, K, _ptr(resid), _dt(resid), d, _ptr(score), _ptr(keep), _ptr(kept_idx), _ptr(resid_out),
            _ptr(score_out), wp, wn, _stream(stream))
    if span_end is None:
        _check(lib.tg_gate_select(_ptr(score_raw), B, N, r, *rest))
    else:
        _check(lib.tg_gate_select_span(_ptr(score_raw), B, N, r, span_end, *rest))
    return kept_idx, resid_out, score_out, keep, score


def tg_gate_select_padded(score_raw, resid, r: int, K, M_pad: int, eps_seq: float = 1e-6, score=None, keep=None,
                          kept_idx=None, resid_out=None, score_out=None, kept_count=None, stream=None):
    """:func:`tg_gate_select` with the budgets ``K`` (int32 GPU tensor ``[B]``)
    read on the device and the kept sets written into ``M_pad`` rows per batch
    row.  Returns ``(kept_idx [B, M_pad], resid_out [B, M_pad, d], score_out
    [B, M_pad], kept_count [B] int32, keep, score)``; row b's first
    ``kept_count[b]`` rows are its kept set (the rest untouched).  No host
    value depends on K, so the call can be captured once and replayed with
    new budgets."""
    lib = load_library()
    _need(resid, "resid")
    B, N, d = resid.shape
    _need(score_raw, "score_raw", torch.float32, (B, N))
    _need(K, "K", torch.int32, (B,))
    dev = resid.device
    if score is None:
        score = torch.empty((B, N), dtype=torch.float32, device=dev)
    if keep is None:
        keep = torch.empty((B, N), dtype=torch.uint8, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((B, M_pad), dtype=torch.int32, device=dev)
    if resid_out is None:
        resid_out = torch.empty((B, M_pad, d), dtype=resid.dtype, device=dev)
    if score_out is None:
        score_out = torch.empty((B, M_pad), dtype=torch.float32, device=dev)
    if kept_count is None:
        kept_count = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(score, "score", torch.float32, (B, N))
    _need(keep, "keep", torch.uint8, (B, N))
    _need(kept_idx, "kept_idx", torch.int32, (B, M_pad))
    _need(resid_out, "resid_out", resid.dtype, (B, M_pad, d))
    _need(score_out, "score_out", torch.float32, (B, M_pad))
    _need(kept_count, "kept_count", torch.int32, (B,))
    _check(lib.tg_gate_select_padded(_ptr(score_raw), B, N, r, eps_seq, _ptr(K), M_pad, _ptr(resid), _dt(resid), d,
                                     _ptr(score), _ptr(keep), _ptr(kept_idx), _ptr(resid_out), _ptr(score_out),
                                     _ptr(kept_count), _stream(stream)))
    return kept_idx, resid_out, score_out, kept_count, keep, score


def tg_gated_attention_padded(q, k, v, kept_count, key_score, pos, gain, temp, sm_scale: float | None = None,
                              out=None, lse=None, ws=None, stream=None):
    """:func:`tg_gated_attention` on tensors padded to ``M_pad`` rows (q ``[B,
    M_pad, Hq, dh]`` ...), where batch row b uses its first ``kept_count[b]``
    rows (int32 GPU tensor ``[B]``, read on the device).  Returns ``out`` (and
    ``lse [B, Hq, M_pad]`` when given)."""
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    B, M_pad, Hq, dh = q.shape
    Hkv = k.shape[2]
    _need(k, "k", torch.bfloat16, (B, M_pad, Hkv, dh))
    _need(v, "v", torch.bfloat16, (B, M_pad, Hkv, dh))
    _need(kept_count, "kept_count", torch.int32, (B,))
    _need(key_score, "key_score", torch.float32, (B, M_pad))
    _need(pos, "pos", torch.int32, (B, M_pad))
    if sm_scale is None:
        sm_scale = dh ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, (B, M_pad, Hq, dh))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, M_pad))
    if ws is None:
        ws = attention_workspace(B, M_pad, Hq, Hkv, dh, q.device)
    _check(lib.tg_gated_attention_padded(_ptr(q), _ptr(k), _ptr(v), B, M_pad, _ptr(kept_count), Hq, Hkv, dh,
                                         _ptr(key_score), _ptr(pos), _ptr(gain), _ptr(temp), float(sm_scale),
                                         _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return (out, lse) if lse is not None else out


def varlen_kept_counts(seq_len, span_begin, span_end, K):
    """Host-side M_b = len_b - P_b + min(K_b, P_b) of a varying-length batch
    (lists or arrays of ints), with the same clamping as the kernel."""
    out = []
    for n, p0, p1, k in zip(seq_len, span_begin, span_end, K):
        p1 = min(max(int(p1), 0), int(n))
        p0 = min(max(int(p0), 0), p1)
        P = p1 - p0
        out.append(int(n) - P + min(max(int(k), 0), P))
    return out


def tg_gate_score_varlen(resid, span_begin, span_end, norm_w, W1, b1, w2, b2, eps_row: float = 1e-6, score_raw=None,
                         ws=None, stream=None):
    """Raw scores ``[B, N]`` of a varying-length batch: row b scored on its span
    ``[span_begin[b], span_end[b])`` (host lists), 0 elsewhere."""
    lib = load_library()
    _need(resid, "resid")
    B, N, d = resid.shape
    h = W1.shape[0]
    dev = resid.device
    if score_raw is None:
        score_raw = torch.empty((B, N), dtype=torch.float32, device=dev)
    _need(score_raw, "score_raw", torch.float32, (B, N))
    if ws is None:
        ws = gate_workspace(h, d, dev)
    sb = torch.tensor([int(x) for x in span_begin], dtype=torch.int32, device=dev)
    se = torch.tensor([int(x) for x in span_end], dtype=torch.int32, device=dev)
    max_span = max([max(0, min(int(e), N) - max(0, int(b_))) for b_, e in zip(span_begin, span_end)] + [0])
    _check(lib.tg_gate_score_varlen(_ptr(resid), _dt(resid), B, N, d, _ptr(sb), _ptr(se), max_span, _ptr(norm_w),
                                    eps_row, _ptr(W1), _ptr(b1), h, _ptr(w2), _ptr(b2), _ptr(score_raw), _ptr(ws),
                                    ws.numel(), _stream(stream)))
    return score_raw


def tg_gate_select_varlen(score_raw, resid, seq_len, span_begin, span_end, K, eps_seq: float = 1e-6, score=None,
                          keep=None, ws=None, stream=None):
    """Gate selection of a batch of sequences of different lengths, spans and
    budgets (per-row host lists).  Returns ``(kept_idx, resid_out, score_out,
    keep, score, cu_kept)`` with the kept rows packed: row b's are
    ``cu_kept[b] .. cu_kept[b+1]-1`` (``cu_kept`` a host list).  Rows longer
    than 32768 tokens use a workspace (allocated here unless ``ws`` is given)."""
    lib = load_library()
    _need(resid, "resid")
    B, N, d = resid.shape
    _need(score_raw, "score_raw", torch.float32, (B, N))
    dev = resid.device
    Ms = varlen_kept_counts(seq_len, span_begin, span_end, K)
    cu = [0]
    for m in Ms:
        cu.append(cu[-1] + m)
    T = cu[-1]
    arr = lambda x: torch.tensor([int(v) for v in x], dtype=torch.int32, device=dev)  # noqa: E731
    rows = [arr(seq_len), arr(span_begin), arr(span_end), arr(K), arr(cu)]
    if score is None:
        score = torch.empty((B, N), dtype=torch.float32, device=dev)
    if keep is None:
        keep = torch.empty((B, N), dtype=torch.uint8, device=dev)
    kept_idx = torch.empty((max(T, 1),), dtype=torch.int32, device=dev)
    resid_out = torch.empty((max(T, 1), d), dtype=resid.dtype, device=dev)
    score_out = torch.empty((max(T, 1),), dtype=torch.float32, device=dev)
    if ws is None:
        n = int(lib.tg_workspace_size(TG_OP_GATE_SELECT, B, N, 0, 0, 0))
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    _check(lib.tg_gate_select_varlen(_ptr(score_raw), B, N, *[_ptr(t) for t in rows], max(Ms) if Ms else 0, eps_seq,
                                     _ptr(resid), _dt(resid), d, _ptr(score), _ptr(keep), _ptr(kept_idx),
                                     _ptr(resid_out), _ptr(score_out), _ptr(ws), ws.numel(), _stream(stream)))
    return kept_idx[:T], resid_out[:T], score_out[:T], keep, score, cu


def tg_gated_attention_varlen(q, k, v, cu_seqlens, key_score, pos, gain, temp, sm_scale: float | None = None,
                              out=None, lse=None, ws=None, stream=None, rope_base: float | None = None):
    """Token-gated attention over packed sequences: q ``[T, Hq, dh]``, k/v
    ``[T, Hkv, dh]``, key_score/pos ``[T]``, ``cu_seqlens`` a host list of B + 1
    row offsets (e.g. from :func:`tg_gate_select_varlen`).  Returns ``out``
    (and ``lse`` when given: sequence b's [Hq, M_b] block at cu_seqlens[b] * Hq)."""
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    T, Hq, dh = q.shape
    Hkv = k.shape[1]
    _need(k, "k", torch.bfloat16, (T, Hkv, dh))
    _need(v, "v", torch.bfloat16, (T, Hkv, dh))
    _need(key_score, "key_score", torch.float32, (T,))
    _need(pos, "pos", torch.int32, (T,))
    cu = [int(x) for x in cu_seqlens]
    if cu[0] != 0 or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0 and end at the number of packed rows")
    B = len(cu) - 1
    if sm_scale is None:
        sm_scale = dh ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, (T, Hq, dh))
    if lse is not None:
        _need(lse, "lse", torch.float32, (T * Hq,))
    if ws is None:  # every sequence padded to 64 rows, side by side
        mk = attention_workspace if rope_base is None else attention_rope_workspace
        ws = mk(1, max(T + 63 * B, 1), Hq, Hkv, dh, q.device)
    cu_arr = (ctypes.c_int32 * len(cu))(*cu)
    args = (_ptr(q), _ptr(k), _ptr(v), B, cu_arr, Hq, Hkv, dh, _ptr(key_score), _ptr(pos), _ptr(gain), _ptr(temp),
            float(sm_scale))
    tail = (_ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
    if rope_base is None:
        _check(lib.tg_gated_attention_varlen(*args, *tail))
    else:
        _check(lib.tg_gated_attention_rope_varlen(*args, float(rope_base), *tail))
    return (out, lse) if lse is not None else out


def tg_gated_attention_rope_varlen(q, k, v, cu_seqlens, key_score, pos, gain, temp, rope_base: float,
                                   sm_scale: float | None = None, out=None, lse=None, ws=None, stream=None):
    """:func:`tg_gated_attention_varlen` with the rotary embedding of
    :func:`tg_gated_attention_rope` (each packed row turned by its own
    original position ``pos``)."""
    return tg_gated_attention_varlen(q, k, v, cu_seqlens, key_score, pos, gain, temp, sm_scale, out=out, lse=lse,
                                     ws=ws, stream=stream, rope_base=rope_base)


def tg_gated_attention_backward_varlen(q, k, v, out, lse, d_out, cu_seqlens, key_score, pos, gain, temp,
                                       sm_scale: float | None = None, ws=None, stream=None,
                                       rope_base: float | None = None):
    """Gradients of :func:`tg_gated_attention_varlen` (same packed layouts;
    ``lse`` as it wrote it).  Returns ``(d_q, d_k, d_v, d_key_score, d_gain
    [B, Hq], d_temp [B, Hq])``: per-sequence gain and temperature gradients.
    With ``rope_base`` the gradients of the rotary variant (q and k passed
    un-rotated)."""
    lib = load_library()
    T, Hq, dh = q.shape
    Hkv = k.shape[1]
    for t_, n_, shp in ((q, "q", (T, Hq, dh)), (k, "k", (T, Hkv, dh)), (v, "v", (T, Hkv, dh)),
                        (out, "out", (T, Hq, dh)), (d_out, "d_out", (T, Hq, dh))):
        _need(t_, n_, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (T * Hq,))
    _need(key_score, "key_score", torch.float32, (T,))
    _need(pos, "pos", torch.int32, (T,))
    cu = [int(x) for x in cu_seqlens]
    if cu[0] != 0 or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0 and end at the number of packed rows")
    B = len(cu) - 1
    if sm_scale is None:
        sm_scale = dh ** -0.5
    dev = q.device
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty(T, device=dev),
             torch.empty((B, Hq), device=dev), torch.empty((B, Hq), device=dev)]
    if ws is None:  # every sequence padded to 64 rows, side by side
        wsf = attention_backward_workspace if rope_base is None else attention_rope_backward_workspace
        ws = wsf(1, max(T + 63 * B, 1), Hq, Hkv, dh, dev)
    cu_arr = (ctypes.c_int32 * len(cu))(*cu)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(d_out), B, cu_arr, Hq, Hkv, dh, _ptr(key_score),
            _ptr(pos), _ptr(gain), _ptr(temp), float(sm_scale))
    tail = (*[_ptr(g_) for g_ in grads], _ptr(ws), ws.numel(), _stream(stream))
    if rope_base is None:
        _check(lib.tg_gated_attention_backward_varlen(*head, *tail))
    else:
        _check(lib.tg_gated_attention_rope_backward_varlen(*head, float(rope_base), *tail))
    return tuple(grads)


def tg_gated_attention_rope_backward_varlen(q, k, v, out, lse, d_out, cu_seqlens, key_score, pos, gain, temp,
                                            rope_base: float, sm_scale: float | None = None, ws=None, stream=None):
    """Gradients of :func:`tg_gated_attention_rope_varlen` (q and k passed
    un-rotated); outputs as :func:`tg_gated_attention_backward_varlen`."""
    return tg_gated_attention_backward_varlen(q, k, v, out, lse, d_out, cu_seqlens, key_score, pos, gain, temp,
                                              sm_scale, ws=ws, stream=stream, rope_base=rope_base)


def attention_workspace(B: int, M: int, Hq: int, Hkv: int, dh: int, device="cuda") -> torch.Tensor:
    """A workspace tensor large enough for tg_gated_attention at these sizes."""
    n = int(load_library().tg_workspace_size(TG_OP_GATED_ATTENTION, B, M, Hkv * dh, Hq, dh))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _attention_call(entry, q, k, v, key_score, pos, gain, temp, sm_scale, out, lse, want_lse, ws, stream,
                    rope_base=None):
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    B, M, Hq, dh = q.shape
    Hkv = k.shape[2]
    _need(k, "k", torch.bfloat16, (B, M, Hkv, dh))
    _need(v, "v", torch.bfloat16, (B, M, Hkv, dh))
    _need(key_score, "key_score", torch.float32, (B, M))
    _need(pos, "pos", torch.int32, (B, M))
    _need(gain, "gain", torch.float32, (Hq,))
    _need(temp, "temp", torch.float32, (Hq,))
    if sm_scale is None:
        sm_scale = dh ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, (B, M, Hq, dh))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, M), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, M))
    if ws is None:
        ws = (attention_workspace(B, M, Hq, Hkv, dh, q.device) if rope_base is None
              else attention_rope_workspace(B, M, Hq, Hkv, dh, q.device))
    _need(ws, "ws", torch.uint8)
    args = [_ptr(q), _ptr(k), _ptr(v), B, M, Hq, Hkv, dh, _ptr(key_score), _ptr(pos), _ptr(gain), _ptr(temp),
            float(sm_scale)]
    if rope_base is not None:
        args.append(float(rope_base))
    args += [_ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)]
    _check(getattr(lib, entry)(*args))
    return (out, lse) if lse is not None else out


def tg_gated_attention(q, k, v, key_score, pos, gain, temp, sm_scale: float | None = None, out=None,
                       lse=None, want_lse: bool = False, ws=None, stream=None):
    """Token-gated causal GQA attention.  q ``[B, M, Hq, dh]``, k/v ``[B, M, Hkv, dh]`` bf16.

    Returns ``out`` (and ``lse [B, Hq, M]`` when ``want_lse`` or ``lse`` is given).
    ``ws`` is a uint8 GPU tensor from :func:`attention_workspace` (allocated
    here when omitted).
    """
    return _attention_call("tg_gated_attention", q, k, v, key_score, pos, gain, temp, sm_scale, out, lse,
                           want_lse, ws, stream)


def attention_rope_workspace(B: int, M: int, Hq: int, Hkv: int, dh: int, device="cuda") -> torch.Tensor:
    """A workspace tensor large enough for tg_gated_attention_rope at these sizes."""
    n = int(load_library().tg_workspace_size(TG_OP_GATED_ATTENTION_ROPE, B, M, Hkv * dh, Hq, dh))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def tg_gated_attention_rope(q, k, v, key_score, pos, gain, temp, rope_base: float, sm_scale: float | None = None,
                            out=None, lse=None, want_lse: bool = False, ws=None, stream=None):
    """tg_gated_attention on q and k rotated by the rotary embedding at the
    original positions ``pos`` (base ``rope_base``); q and k are passed
    un-rotated.  ``ws`` from :func:`attention_rope_workspace`."""
    return _attention_call("tg_gated_attention_rope", q, k, v, key_score, pos, gain, temp, sm_scale, out, lse,
                           want_lse, ws, stream, rope_base=rope_base)


def attention_backward_workspace(B: int, M: int, Hq: int, Hkv: int, dh: int, device="cuda") -> torch.Tensor:
    """A workspace tensor large enough for tg_gated_attention_backward at these sizes."""
    n = int(load_library().tg_workspace_size(TG_OP_GATED_ATTENTION_BACKWARD, B, M, Hkv * dh, Hq, dh))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def attention_rope_backward_workspace(B: int, M: int, Hq: int, Hkv: int, dh: int, device="cuda") -> torch.Tensor:
    """A workspace tensor large enough for tg_gated_attention_rope_backward at these sizes."""
    n = int(load_library().tg_workspace_size(TG_OP_GATED_ATTENTION_ROPE_BACKWARD, B, M, Hkv * dh, Hq, dh))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def tg_gated_attention_rope_backward(q, k, v, out, lse, d_out, key_score, pos, gain, temp, rope_base: float,
                                     sm_scale: float | None = None, ws=None, stream=None, **outs):
    """Gradients of tg_gated_attention_rope (q, k passed un-rotated, as to the
    forward).  Same outputs as :func:`tg_gated_attention_backward`; ``ws`` from
    :func:`attention_rope_backward_workspace`."""
    if ws is None:
        ws = attention_rope_backward_workspace(q.shape[0], q.shape[1], q.shape[2], k.shape[2], q.shape[3], q.device)
    return tg_gated_attention_backward(q, k, v, out, lse, d_out, key_score, pos, gain, temp, sm_scale, ws=ws,
                                       stream=stream, _rope_base=rope_base, **outs)


def tg_gated_attention_backward(q, k, v, out, lse, d_out, key_score, pos, gain, temp, sm_scale: float | None = None,
                                d_q=None, d_k=None, d_v=None, d_key_score=None, d_gain=None, d_temp=None, ws=None,
                                stream=None, _rope_base: float | None = None):
    """Gradients of tg_gated_attention from its outputs ``out`` and ``lse``
    and the upstream gradient ``d_out``.  Returns ``(d_q, d_k, d_v,
    d_key_score, d_gain, d_temp)``: bf16 like q/k/v, fp32 ``[B, M]``, and
    fp32 ``[Hq]`` summed over the batch.  ``ws`` from
    :func:`attention_backward_workspace`."""
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    B, M, Hq, dh = q.shape
    Hkv = k.shape[2]
    dev = q.device
    _need(k, "k", torch.bfloat16, (B, M, Hkv, dh))
    _need(v, "v", torch.bfloat16, (B, M, Hkv, dh))
    _need(out, "out", torch.bfloat16, (B, M, Hq, dh))
    _need(d_out, "d_out", torch.bfloat16, (B, M, Hq, dh))
    _need(lse, "lse", torch.float32, (B, Hq, M))
    _need(key_score, "key_score", torch.float32, (B, M))
    _need(pos, "pos", torch.int32, (B, M))
    _need(gain, "gain", torch.float32, (Hq,))
    _need(temp, "temp", torch.float32, (Hq,))
    if sm_scale is None:
        sm_scale = dh ** -0.5
    d_q = torch.empty_like(q) if d_q is None else d_q
    d_k = torch.empty_like(k) if d_k is None else d_k
    d_v = torch.empty_like(v) if d_v is None else d_v
    if d_key_score is None:
        d_key_score = torch.empty((B, M), dtype=torch.float32, device=dev)
    if d_gain is None:
        d_gain = torch.empty((Hq,), dtype=torch.float32, device=dev)
    if d_temp is None:
        d_temp = torch.empty((Hq,), dtype=torch.float32, device=dev)
    _need(d_q, "d_q", torch.bfloat16, (B, M, Hq, dh))
    _need(d_k, "d_k", torch.bfloat16, (B, M, Hkv, dh))
    _need(d_v, "d_v", torch.bfloat16, (B, M, Hkv, dh))
    _need(d_key_score, "d_key_score", torch.float32, (B, M))
    _need(d_gain, "d_gain", torch.float32, (Hq,))
    _need(d_temp, "d_temp", torch.float32, (Hq,))
    if ws is None:
        ws = attention_backward_workspace(B, M, Hq, Hkv, dh, dev)
    _need(ws, "ws", torch.uint8)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(d_out), B, M, Hq, Hkv, dh, _ptr(key_score),
            _ptr(pos), _ptr(gain), _ptr(temp), float(sm_scale))
    tail = (_ptr(d_q), _ptr(d_k), _ptr(d_v), _ptr(d_key_score), _ptr(d_gain), _ptr(d_temp), _ptr(ws), ws.numel(),
            _stream(stream))
    if _rope_base is None:
        _check(lib.tg_gated_attention_backward(*head, *tail))
    else:
        _check(lib.tg_gated_attention_rope_backward(*head, float(_rope_base), *tail))
    return d_q, d_k, d_v, d_key_score, d_gain, d_temp


def tg_kv_cache_prune(k_cache, v_cache, kept_idx, k_out=None, v_out=None, stream=None):
    """Keep only the kept set in the K/V caches of the layers at and below the
    gate: caches ``[layers, B, N, Hkv, dh]`` (2-byte elements), ``kept_idx
    [B, M]`` int32 -> ``(k_out, v_out)`` ``[layers, B, M, Hkv, dh]``."""
    lib = load_library()
    _need(k_cache, "k_cache")
    if k_cache.dim() != 5 or k_cache.element_size() != 2:
        raise ValueError("k_cache must be [layers, B, N, Hkv, dh] with 2-byte elements")
    L, B, N, Hkv, dh = k_cache.shape
    _need(v_cache, "v_cache", k_cache.dtype, (L, B, N, Hkv, dh))
    _need(kept_idx, "kept_idx", torch.int32)
    if kept_idx.dim() != 2 or kept_idx.shape[0] != B:
        raise ValueError("kept_idx must be [B, M]")
    M = kept_idx.shape[1]
    if k_out is None:
        k_out = torch.empty((L, B, M, Hkv, dh), dtype=k_cache.dtype, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty((L, B, M, Hkv, dh), dtype=k_cache.dtype, device=k_cache.device)
    _need(k_out, "k_out", k_cache.dtype, (L, B, M, Hkv, dh))
    _need(v_out, "v_out", k_cache.dtype, (L, B, M, Hkv, dh))
    _check(lib.tg_kv_cache_prune(_ptr(k_cache), _ptr(v_cache), L, B, N, Hkv, dh, _ptr(kept_idx), M, _ptr(k_out),
                                 _ptr(v_out), _stream(stream)))
    return k_out, v_out


def tg_workspace_size(op: int, B: int, N: int, d: int, h: int, K: int) -> int:
    return int(load_library().tg_workspace_size(op, B, N, d, h, K))


def tg_version() -> int:
    return int(load_library().tg_version())


def gated_prefill_gate(resid, r: int, K: int, norm_w, W1, b1, w2, b2, eps_row=1e-6, eps_seq=1e-6, ws=None,
                       sel_ws=None, stream=None):
    """The gate at layer L, end to end: score -> sequence norm -> top-K -> compaction.

    Returns ``(kept_idx, resid_S, b_S, keep, score)``.  Two library calls
    (tg_gate_score, tg_gate_select) on one stream, no host synchronisation
    (M is known on the host).  ``ws``: the scorer's workspace; ``sel_ws``:
    tg_gate_select's.
    """
    raw = tg_gate_score(resid, r, norm_w, W1, b1, w2, b2, eps_row, ws=ws, stream=stream)
    kept_idx, resid_S, b_S, keep, score = tg_gate_select(raw, resid, r, K, eps_seq, score=raw, ws=sel_ws,
                                                         stream=stream)
    return kept_idx, resid_S, b_S, keep, score
