"""Pins for the oracle's post-prefill KV-cache pruning (paper, Section 5,
"Implementation and timing", with Appendix B): every output row must be the
cache row of the kept token it names (rows encoded with their own
coordinates), the whole kept set gives the cache back, and one layer's result
equals the oracle's compaction (itself pinned to its definition) of that
layer's rows."""
import numpy as np

import oracle


def _encoded_cache(L, B, N, H, dh, salt):
    l, b, j, h, d = np.meshgrid(np.arange(L), np.arange(B), np.arange(N), np.arange(H), np.arange(dh), indexing="ij")
    return (((((l * B + b) * N + j) * H + h) * dh + d) * 2 + salt).astype(np.int64)


def _kept(B, N, M, seed):
    rng = np.random.default_rng(seed)
    return np.stack([np.sort(rng.choice(N, M, replace=False)) for _ in range(B)]).astype(np.int32)


def test_rows_come_from_their_kept_tokens():
    L, B, N, H, dh, M = 3, 2, 50, 2, 8, 17
    kc, vc = _encoded_cache(L, B, N, H, dh, 0), _encoded_cache(L, B, N, H, dh, 1)
    idx = _kept(B, N, M, 0)
    ko, vo = oracle.kv_cache_prune(kc, vc, idx)
    assert ko.shape == (L, B, M, H, dh) and vo.shape == (L, B, M, H, dh)
    # decode the coordinates back from the values
    for out, salt in ((ko, 0), (vo, 1)):
        assert np.all(out % 2 == salt)
        flat = out // 2
        d = flat % dh
        h = (flat // dh) % H
        j = (flat // (dh * H)) % N
        b = (flat // (dh * H * N)) % B
        lay = flat // (dh * H * N * B)
        assert np.array_equal(j[:, :, :, 0, 0], np.broadcast_to(idx[None], (L, B, M)))
        assert np.array_equal(b[:, :, 0, 0, 0], np.broadcast_to(np.arange(B)[None], (L, B)))
        assert np.array_equal(lay[:, 0, 0, 0, 0], np.arange(L))
        assert np.array_equal(h[0, 0, 0, :, 0], np.arange(H)) and np.array_equal(d[0, 0, 0, 0], np.arange(dh))


def test_keeping_every_token_is_the_identity():
    kc = np.random.default_rng(1).integers(0, 1 << 16, size=(2, 1, 40, 3, 8)).astype(np.uint16)
    vc = kc[::-1].copy()
    ko, vo = oracle.kv_cache_prune(kc, vc, np.arange(40, dtype=np.int32)[None])
    assert np.array_equal(ko, kc) and np.array_equal(vo, vc)


def test_matches_compaction_of_one_layer():
    L, B, N, H, dh, M = 2, 1, 64, 2, 8, 20
    rng = np.random.default_rng(2)
    kc = rng.standard_normal((L, B, N, H, dh)).astype(np.float32)
    idx = _kept(B, N, M, 3)
    keep = np.zeros((B, N), np.uint8)
    keep[0, idx[0]] = 1
    ko, _ = oracle.kv_cache_prune(kc, kc, idx)
    for l in range(L):
        kept_idx, resid_S, _ = oracle.compact(kc[l].reshape(B, N, H * dh), keep, np.zeros((B, N), np.float32))
        assert np.array_equal(kept_idx, idx)
        assert np.array_equal(resid_S.reshape(B, M, H, dh), ko[l])
