"""Pins for the oracle's backward of token-gated attention (Eq. 8).

The key score b_j reaches the loss only through the logits of the layers
above the gate (TokenGate paper, Section 4, token-gated attention: the
gradient path that makes the top-K selector trainable), so the backward
gives dq, dk, dv and the key-score gradient db together with the gradients
of the per-head gain and temperature (the trainable scale factors of Section
4, "Putting everything together").

The oracle's hand-derived gradients are tied to: central finite differences
of the oracle's own forward (already pinned to SDPA and the gate form) in
float64, torch CPU autograd through ``scaled_dot_product_attention`` in
float64 for the general case (the temperature folded into the queries, the
gain times the key score as an additive mask), softmax shift invariance
(sum_j db_j = 0), and the single-query case where the softmax is constant.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(seed, B=2, M=6, Hq=4, Hkv=2, dh=4):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, M, Hq, dh))
    k = rng.normal(size=(B, M, Hkv, dh))
    v = rng.normal(size=(B, M, Hkv, dh))
    b = rng.normal(size=(B, M))
    # original positions of kept tokens: increasing, pos_i >= i, equal to i on
    # a prefix (the non-prunable question) and larger after it
    pos = np.zeros((B, M), np.int64)
    for bi in range(B):
        pos[bi] = np.concatenate([np.arange(min(M, 2)),
                                  2 + np.sort(rng.choice(np.arange(1, 4 * M), max(M - 2, 0), replace=False))])
    gain = rng.uniform(0.5, 1.5, size=Hq)
    temp = rng.uniform(0.8, 1.3, size=Hq)
    dO = rng.normal(size=(B, M, Hq, dh))
    return q, k, v, b, pos, gain, temp, 1.0 / np.sqrt(dh), dO


def _loss(args, dO):
    q, k, v, b, pos, gain, temp, sm = args
    O, _ = oracle.gated_attention(q, k, v, b, pos, gain, temp, sm)
    return float(np.sum(O * dO))


def _grads(args, dO):
    q, k, v, b, pos, gain, temp, sm = args
    O, lse = oracle.gated_attention(q, k, v, b, pos, gain, temp, sm)
    return oracle.gated_attention_backward(q, k, v, b, pos, gain, temp, sm, O, lse, dO)


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed):
    q, k, v, b, pos, gain, temp, sm, dO = _case(seed)
    args = [q, k, v, b, pos, gain, temp, sm]
    grads = _grads(args, dO)
    h = 1e-5
    for slot, g in zip([0, 1, 2, 3, 5, 6], grads):
        x = args[slot]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[slot], am[slot] = xp, xm
            fd[idx] = (_loss(ap, dO) - _loss(am, dO)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=f"input {slot}")


def test_backward_matches_sdpa_autograd():
    """General case through torch autograd: queries pre-scaled by 1/tau_i (a
    differentiable function of temp), the additive float mask gain_h * b_j on
    j <= i and -inf above the diagonal."""
    q, k, v, b, pos, gain, temp, sm, dO = _case(7, B=2, M=9, Hq=6, Hkv=2, dh=8)
    B, M, Hq, dh = q.shape
    group = Hq // k.shape[2]
    O, lse = oracle.gated_attention(q, k, v, b, pos, gain, temp, sm)
    want = oracle.gated_attention_backward(q, k, v, b, pos, gain, temp, sm, O, lse, dO)

    T = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for n, a in dict(q=q, k=k, v=v, b=b, gain=gain, temp=temp).items()}
    ratio = torch.tensor([[oracle.temperature_ratio(pos[bi, i], i) for i in range(M)] for bi in range(B)],
                         dtype=torch.float64)
    tau = T["temp"][None, None, :] * ratio[:, :, None]                       # [B, M, Hq]
    Qs = (T["q"] / tau[..., None]).permute(0, 2, 1, 3)
    Kr = T["k"].repeat_interleave(group, dim=2).permute(0, 2, 1, 3)
    Vr = T["v"].repeat_interleave(group, dim=2).permute(0, 2, 1, 3)
    bias = T["gain"][None, :, None, None] * T["b"][:, None, None, :]         # [B, Hq, 1, M]
    causal = torch.ones(M, M, dtype=torch.bool).tril()
    mask = torch.where(causal, bias, torch.tensor(-torch.inf, dtype=torch.float64))
    Ot = torch.nn.functional.scaled_dot_product_attention(Qs, Kr, Vr, attn_mask=mask, scale=sm)
    np.testing.assert_allclose(Ot.permute(0, 2, 1, 3).detach().numpy(), O, rtol=1e-12, atol=1e-12)
    (Ot.permute(0, 2, 1, 3) * torch.from_numpy(dO)).sum().backward()
    for name, g in zip(["q", "k", "v", "b", "gain", "temp"], want):
        np.testing.assert_allclose(g, T[name].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_key_score_gradient_sums_to_zero():
    """A constant added to every key score leaves every softmax unchanged."""
    q, k, v, b, pos, gain, temp, sm, dO = _case(3, B=1, M=11, Hq=4, Hkv=1, dh=8)
    _, _, _, db, dgain, _ = _grads([q, k, v, b, pos, gain, temp, sm], dO)
    assert abs(db.sum()) < 1e-12 * np.abs(db).sum()
    # the same invariance per head: shifting b by c changes nothing, so the
    # gain gradient equals its value with b centred
    _, _, _, _, dgain_c, _ = _grads([q, k, v, b - b.mean(), pos, gain, temp, sm], dO)
    np.testing.assert_allclose(dgain, dgain_c, rtol=1e-10, atol=1e-13)


def test_single_query_row():
    """One kept token: the softmax is the constant 1, so only dv = dO survives."""
    q, k, v, b, pos, gain, temp, sm, dO = _case(4, B=1, M=1, Hq=4, Hkv=2, dh=8)
    dq, dk, dv, db, dgain, dtemp = _grads([q, k, v, b, np.zeros((1, 1), np.int64), gain, temp, sm], dO)
    for g in (dq, dk, db, dgain, dtemp):  # dP - D vanishes up to rounding
        assert np.max(np.abs(g)) < 1e-13
    np.testing.assert_allclose(dv[0, 0, 0], dO[0, 0, 0] + dO[0, 0, 1], rtol=1e-14)
    np.testing.assert_allclose(dv[0, 0, 1], dO[0, 0, 2] + dO[0, 0, 3], rtol=1e-14)


def test_l1_scales_bound_the_gradients():
    """Triangle inequality everywhere, and equality where every summand has
    one sign (d_v with a non-negative upstream gradient)."""
    q, k, v, b, pos, gain, temp, sm, dO = _case(5, B=2, M=13, Hq=4, Hkv=2, dh=8)
    O, lse = oracle.gated_attention(q, k, v, b, pos, gain, temp, sm)
    g = oracle.gated_attention_backward(q, k, v, b, pos, gain, temp, sm, O, lse, dO)
    l1 = oracle.gated_attention_backward_l1(q, k, v, b, pos, gain, temp, sm, O, lse, dO)
    for x, m in zip(g, l1):
        assert np.all(np.abs(x) <= m * (1 + 1e-12) + 1e-15)
    dOp = np.abs(dO)
    gp = oracle.gated_attention_backward(q, k, v, b, pos, gain, temp, sm, O, lse, dOp)
    lp = oracle.gated_attention_backward_l1(q, k, v, b, pos, gain, temp, sm, O, lse, dOp)
    np.testing.assert_allclose(gp[2], lp[2], rtol=1e-13)


def test_rope_backward_matches_finite_differences():
    """The rotary variant without the bf16 rounding of q', k': central
    differences of sum(dO * O) with O = Eq. 8 on rope(q), rope(k)."""
    q, k, v, b, pos, gain, temp, sm, dO = _case(11, B=1, M=5, Hq=2, Hkv=1, dh=4)
    base = 100.0
    pos = pos * 37  # angles well away from 0

    def loss(qx, kx):
        O, _ = oracle.gated_attention(oracle.rope(qx, pos, base), oracle.rope(kx, pos, base), v, b, pos, gain, temp,
                                      sm)
        return float(np.sum(O * dO))

    O, lse = oracle.gated_attention(oracle.rope(q, pos, base), oracle.rope(k, pos, base), v, b, pos, gain, temp, sm)
    dq, dk, *_ = oracle.gated_attention_rope_backward(q, k, v, b, pos, gain, temp, sm, base, O, lse, dO,
                                                      round_qk=False)
    h = 1e-5
    for x, g, which in ((q, dq, 0), (k, dk, 1)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = ((loss(xp, k) - loss(xm, k)) if which == 0 else (loss(q, xp) - loss(q, xm))) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_rope_backward_at_position_zero_is_the_plain_backward():
    q, k, v, b, _, gain, temp, sm, dO = _case(12, B=1, M=6, Hq=4, Hkv=2, dh=8)
    pos = np.zeros((1, 6), np.int64)
    O, lse = oracle.gated_attention(q, k, v, b, pos, gain, temp, sm)
    a = oracle.gated_attention_rope_backward(q, k, v, b, pos, gain, temp, sm, 1e4, O, lse, dO, round_qk=False)
    p = oracle.gated_attention_backward(q, k, v, b, pos, gain, temp, sm, O, lse, dO)
    for x, y in zip(a, p):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-15)
