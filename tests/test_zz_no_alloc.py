"""tg_gate_score_noalloc, the scorer entry point for callers that cannot
allocate, against tg_gate_score through the C ABI.

Both run the same kernels; the no-allocation call puts the folded W1 into the
library's fixed per-device scratch instead of a caller's workspace.  Two calls
in a row, the second on a smaller input (so the scratch still holds the first
call's larger fold), must each equal tg_gate_score bit for bit and match the
oracle within the bf16 score tolerance.  An fp32 call (no scratch) is checked
the same way.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import learned_token_pruning_07_amd as tg
from learned_token_pruning_07_amd import workloads as wl
from _gpu_util import DEV, TOL_BF16, TOL_F32, assert_close, gate_dev, say

pytestmark = pytest.mark.gpu


def _lib():
    lib = ctypes.CDLL(tg.LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.tg_gate_score.argtypes = [vp, i, i, i, i, i, vp, f, vp, vp, i, vp, vp, vp, vp, sz, vp]
    lib.tg_gate_score_noalloc.argtypes = [vp, i, i, i, i, i, vp, f, vp, vp, i, vp, vp, vp, vp]
    lib.tg_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.tg_workspace_size.restype = sz
    lib.tg_last_error.restype = ctypes.c_char_p
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(lib, c):
    """(tg_gate_score result, tg_gate_score_noalloc result) on case c."""
    t = gate_dev(c)
    dt = tg.TG_BF16 if c.dtype == "bf16" else tg.TG_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n = lib.tg_workspace_size(tg.TG_OP_GATE_SCORE, c.B, c.N, c.d, c.h, c.K)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
    ref = torch.full((c.B, c.N), float("nan"), dtype=torch.float32, device=DEV)
    got = torch.full((c.B, c.N), float("nan"), dtype=torch.float32, device=DEV)
    args = (_p(t["norm_w"]), ctypes.c_float(c.eps_row), _p(t["W1"]), _p(t["b1"]), c.h, _p(t["w2"]), _p(t["b2"]))
    rc = lib.tg_gate_score(_p(t["resid"]), dt, c.B, c.N, c.d, c.r, *args, _p(ref), _p(ws), ctypes.c_size_t(ws.numel()),
                           stream)
    assert rc == 0, lib.tg_last_error()
    rc = lib.tg_gate_score_noalloc(_p(t["resid"]), dt, c.B, c.N, c.d, c.r, *args, _p(got), stream)
    assert rc == 0, lib.tg_last_error()
    torch.cuda.synchronize()
    return ref, got


def _oracle(c):
    return oracle.gate_score(c.resid, c.r, c.norm_w, c.W1, c.b1, c.w2, c.b2, c.eps_row)


def test_noalloc_scorer_equals_gate_score():
    lib = _lib()
    # the first call folds a 256 x 4096 W1 (2 MiB of scratch); the second a
    # 128 x 1024 W1 into the start of the same scratch, with a different
    # norm weight, so a stale fold would show
    cases = [wl.gate_case(N=3000, r=40, d=4096, h=256, K=300, dtype="bf16", seed=11, B=2),
             wl.gate_case(N=777, r=5, d=1024, h=128, K=80, dtype="bf16", seed=12)]
    rng = wl.make_rng(13)
    cases[1].norm_w = wl.f32_to_bf16_bits(rng.uniform(0.5, 1.5, size=1024).astype(np.float32))
    for c in cases:
        say(f"noalloc scorer bf16 B={c.B} N={c.N} d={c.d} h={c.h}")
        ref, got = _both(lib, c)
        assert torch.equal(got, ref), "tg_gate_score_noalloc differs from tg_gate_score"
        err = assert_close(got.cpu().numpy(), _oracle(c), TOL_BF16, "noalloc score")
        say(f"  bit-identical to tg_gate_score; max |err| vs oracle {err:.3g}")
    c = wl.gate_case(N=500, r=10, d=256, h=64, K=50, dtype="f32", seed=14, w_std=0.05)
    ref, got = _both(lib, c)
    assert torch.equal(got, ref)
    assert_close(got.cpu().numpy(), _oracle(c), TOL_F32, "noalloc score f32")

