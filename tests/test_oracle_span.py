"""Pins for the oracle's gate with the prunable document anywhere in the
prompt (a span [p0, p1) with non-prunable text on both sides; the paper's
public interface marks the document with a placeholder inside the prompt).

The tokens outside the span are non-prunable however they are placed, so
moving the text after the span to the front of the prompt must give the
same scores, normalised scores and keep decisions, token for token (the
prefix-only oracle is pinned by its own tests); top-K is also checked by
brute-force rank counting inside the span, and the kept set's order by the
compaction."""
import numpy as np
import pytest

import oracle


def _perm(N, p1):
    """Order that moves tokens [p1, N) to the front, the rest after them."""
    return np.concatenate([np.arange(p1, N), np.arange(p1)])


@pytest.mark.parametrize("N,p0,p1", [(40, 5, 30), (40, 0, 33), (25, 7, 25), (30, 10, 10), (12, 0, 12)])
def test_span_equals_moved_suffix(N, p0, p1):
    rng = np.random.default_rng(N + p0 + p1)
    d, h, B = 16, 8, 2
    resid = rng.standard_normal((B, N, d))
    norm_w = rng.uniform(0.5, 1.5, d)
    W1, b1 = rng.standard_normal((h, d)) * 0.3, rng.standard_normal(h) * 0.1
    w2, b2 = rng.standard_normal(h), rng.standard_normal(1)
    perm = _perm(N, p1)
    inv = np.argsort(perm)
    r_moved = (N - p1) + p0
    raw_span = oracle.gate_score(resid, p0, norm_w, W1, b1, w2, b2, 1e-6, span_end=p1)
    raw_moved = oracle.gate_score(resid[:, perm], r_moved, norm_w, W1, b1, w2, b2, 1e-6)
    np.testing.assert_array_equal(raw_span, raw_moved[:, inv])
    sc_span = oracle.seq_rmsnorm(raw_span, p0, 1e-6, span_end=p1)
    sc_moved = oracle.seq_rmsnorm(raw_moved, r_moved, 1e-6)
    np.testing.assert_array_equal(sc_span, sc_moved[:, inv])
    for K in (0, 1, 5, p1 - p0, p1 - p0 + 3):
        keep_span = oracle.topk_select(sc_span, p0, K, span_end=p1)
        keep_moved = oracle.topk_select(sc_moved, r_moved, K)
        np.testing.assert_array_equal(keep_span, keep_moved[:, inv])
        assert np.all(keep_span.sum(axis=1) == N - (p1 - p0) + min(K, p1 - p0))


def test_span_topk_brute_force():
    rng = np.random.default_rng(5)
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, np.inf, -np.inf, np.nan])
    for trial in range(20):
        N = int(rng.integers(3, 14))
        p0 = int(rng.integers(0, N))
        p1 = int(rng.integers(p0, N + 1))
        s = rng.choice(vals, size=(1, N))
        for K in range(0, p1 - p0 + 2):
            keep = oracle.topk_select(s, p0, K, span_end=p1)[0]
            assert np.all(keep[:p0] == 1) and np.all(keep[p1:] == 1)
            Kp = min(K, p1 - p0)
            span = s[0, p0:p1]
            for i in range(p1 - p0):
                # rank: how many span tokens come strictly before token i in
                # the order (larger score first, NaN last, lower index first)
                def before(j, i=i):
                    a, b = span[j], span[i]
                    if np.isnan(a) or np.isnan(b):
                        return (not np.isnan(a) and np.isnan(b)) or (np.isnan(a) and np.isnan(b) and j < i)
                    return a > b or (a == b and j < i)
                rank = sum(before(j) for j in range(p1 - p0) if j != i)
                assert keep[p0 + i] == (1 if rank < Kp else 0), (trial, N, p0, p1, K, i)


def test_span_kept_order():
    """Compaction of a span keep mask: question, kept document tokens, trailing text, ascending."""
    N, p0, p1, K = 30, 4, 22, 6
    rng = np.random.default_rng(1)
    sc = oracle.seq_rmsnorm(rng.standard_normal((1, N)), p0, 1e-6, span_end=p1)
    keep = oracle.topk_select(sc, p0, K, span_end=p1)
    kept_idx, _, b_S = oracle.compact(rng.standard_normal((1, N, 8)).astype(np.float32), keep, sc)
    ki = kept_idx[0]
    assert ki.shape[0] == N - (p1 - p0) + K
    assert np.array_equal(ki[:p0], np.arange(p0)) and np.array_equal(ki[-(N - p1):], np.arange(p1, N))
    assert np.all(np.diff(ki) > 0) and np.all((ki[p0:p0 + K] >= p0) & (ki[p0:p0 + K] < p1))
    assert np.all(b_S[0, :p0] == 0) and np.all(b_S[0, -(N - p1):] == 0)


def test_varlen_uniform_rows_equal_the_batched_gate():
    """Rows of one length, span and budget give the uniform batched gate."""
    rng = np.random.default_rng(3)
    B, N, p0, p1, K = 3, 50, 6, 44, 9
    raw = rng.standard_normal((B, N))
    resid = rng.standard_normal((B, N, 8)).astype(np.float32)
    ki, rs, bs, keep, score, cu = oracle.gate_select_varlen(raw, resid, [N] * B, [p0] * B, [p1] * B, [K] * B, 1e-6)
    sc = oracle.seq_rmsnorm(raw, p0, 1e-6, span_end=p1)
    kp = oracle.topk_select(sc, p0, K, span_end=p1)
    i2, r2, s2 = oracle.compact(resid, kp, sc)
    assert cu == [0, i2.shape[1], 2 * i2.shape[1], 3 * i2.shape[1]]
    assert np.array_equal(ki, i2.reshape(-1)) and np.array_equal(rs, r2.reshape(-1, 8))
    assert np.array_equal(bs, s2.reshape(-1)) and np.array_equal(keep, kp) and np.array_equal(score, sc)


def test_varlen_padding_changes_nothing():
    """Padding tokens (any scores, any rows) past a row's length are ignored."""
    rng = np.random.default_rng(4)
    N, n = 60, 41
    raw = rng.standard_normal((1, N))
    resid = rng.standard_normal((1, N, 8)).astype(np.float32)
    a = oracle.gate_select_varlen(raw, resid, [n], [3], [35], [7], 1e-6)
    raw2, resid2 = raw.copy(), resid.copy()
    raw2[0, n:] = 1e9
    resid2[0, n:] = -7.0
    b = oracle.gate_select_varlen(raw2, resid2, [n], [3], [35], [7], 1e-6)
    for x, y in zip(a[:5], b[:5]):
        assert np.array_equal(x, y)
    assert np.all(a[3][0, n:] == 0) and np.all(a[4][0, n:] == 0)
