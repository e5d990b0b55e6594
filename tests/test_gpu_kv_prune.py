"""GPU parity of the post-prefill KV-cache pruning (paper, Section 5,
"Implementation and timing", with Appendix B) against the oracle: a row
gather, so the comparison is bit-exact, at small ragged sizes and at the
stage's full size (5 layers at and below gate layer 4, N = 32768, 8 KV heads,
d_h 128, M = 3341 kept)."""
import numpy as np
import pytest
import torch

import oracle
import learned_token_pruning_07_amd as tg
from _gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _case(L, B, N, H, dh, M, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    kc = torch.randint(-32768, 32768, (L, B, N, H, dh), generator=g, device=DEV, dtype=torch.int32).to(torch.int16)
    vc = torch.randint(-32768, 32768, (L, B, N, H, dh), generator=g, device=DEV, dtype=torch.int32).to(torch.int16)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(N, M, replace=False)) for _ in range(B)]).astype(np.int32)
    return kc.view(torch.bfloat16), vc.view(torch.bfloat16), idx


def _check(kc, vc, idx, what):
    ko, vo = tg.tg_kv_cache_prune(kc, vc, torch.from_numpy(idx).to(DEV))
    host = lambda t: t.view(torch.int16).cpu().numpy()  # noqa: E731
    rk, rv = oracle.kv_cache_prune(host(kc), host(vc), idx)
    assert np.array_equal(host(ko), rk), f"{what}: K rows differ"
    assert np.array_equal(host(vo), rv), f"{what}: V rows differ"


@pytest.mark.parametrize("L,B,N,H,dh,M", [
    (1, 1, 100, 2, 64, 37),
    (5, 2, 1000, 8, 128, 333),
    (2, 1, 257, 1, 8, 257),     # every token kept: the identity
    (3, 3, 64, 4, 16, 1),
    (1, 1, 300, 16, 256, 77),   # 8 KiB rows: two passes per row
    (2, 1, 100, 3, 8, 50),      # 48-byte rows: 3 chunks, most lanes idle
])
def test_kv_cache_prune(L, B, N, H, dh, M):
    say(f"kv_cache_prune L={L} B={B} N={N} H={H} dh={dh} M={M}")
    kc, vc, idx = _case(L, B, N, H, dh, M, seed=N + M)
    _check(kc, vc, idx, f"L={L} N={N} M={M}")


def test_kv_cache_prune_empty_leaves_outputs():
    kc, vc, _ = _case(1, 1, 32, 2, 64, 1, seed=3)
    ko = torch.full((1, 1, 0, 2, 64), 1.0, dtype=torch.bfloat16, device=DEV)
    tg.tg_kv_cache_prune(kc, vc, torch.empty((1, 0), dtype=torch.int32, device=DEV), k_out=ko, v_out=ko.clone())


def test_kv_cache_prune_stage_size():
    say("kv_cache_prune full size: 5 layers, N=32768, 8 KV heads, d_h 128, M=3341")
    kc, vc, idx = _case(5, 1, 32768, 8, 128, 3341, seed=7)
    _check(kc, vc, idx, "stage size")
