"""Pins for the oracle's token-gated attention and temperature.

The oracle is tied to: a hand-derived worked example, torch CPU
``scaled_dot_product_attention`` in float64 (plain causal GQA attention when
b = 0 and the temperature is 1, and the general case through an additive
float mask and pre-scaled queries), the unsimplified gate form (Eq. 5 with
Eq. 6), softmax shift invariance, monotonicity in the key score, and the
first row attending only to itself.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from learned_token_pruning_07_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _sdpa(q, k, v, mask, scale):
    """torch CPU SDPA over [B,M,H,dh] float64 tensors with GQA repeat."""
    group = q.shape[2] // k.shape[2]
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    Kt = torch.from_numpy(np.repeat(k, group, axis=2)).permute(0, 2, 1, 3)
    Vt = torch.from_numpy(np.repeat(v, group, axis=2)).permute(0, 2, 1, 3)
    if mask is None:
        O = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True, scale=scale)
    else:
        O = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=torch.from_numpy(mask),
                                                             scale=scale)
    return O.permute(0, 2, 1, 3).numpy()


def test_attention_worked_example():
    g = json.load(open(os.path.join(GOLD, "attention_worked.json")))
    q = np.array(g["q"], np.float32).reshape(1, 2, 1, 1)
    k = np.array(g["k"], np.float32).reshape(1, 2, 1, 1)
    v = np.array(g["v"], np.float32).reshape(1, 2, 1, 1)
    b = np.array([g["b"]], np.float64)
    for case in g["cases"]:
        pos = np.array([case["pos"]], np.int32)
        O, lse = oracle.gated_attention(q, k, v, b, pos, np.ones(1), np.ones(1), 1.0)
        np.testing.assert_allclose(O[0, :, 0, 0], case["O"], rtol=1e-14, atol=0)
        np.testing.assert_allclose(lse[0, 0], case["lse"], rtol=1e-14, atol=0)


def test_temperature_ratio_reading():
    # full context (position == rank) gives exactly 1 (temperature 1 at init)
    for i in range(50):
        assert oracle.temperature_ratio(i, i) == 1.0
    # p = 4 keys at full context, m = 2 kept: ln 4 / ln 2 = 2
    assert oracle.temperature_ratio(3, 1) == 2.0
    assert abs(oracle.temperature_ratio(99, 9) - math.log(100) / math.log(10)) == 0.0
    assert oracle.temperature_ratio(99, 9) == 2.0
    # m = 1 with p > 1 is clamped to 2 (only reachable with no question span)
    assert oracle.temperature_ratio(7, 0) == 3.0
    # pruning only removes keys, so the ratio is never below 1
    for i in range(1, 40):
        for p in range(i, 90):
            assert oracle.temperature_ratio(p, i) >= 1.0


@pytest.mark.parametrize("Hq,Hkv,dh", [(4, 2, 16), (6, 6, 8), (8, 2, 32)])
def test_plain_causal_gqa_special_case(Hq, Hkv, dh):
    # b = 0 and unit temperature at full context: plain (top-K) causal attention
    c = wl.attn_case(M=37, Hq=Hq, Hkv=Hkv, dh=dh, seed=Hq * 7 + dh, r_zero=37, gain=1.3, temp=1.0)
    assert np.all(c.b_raw == 0)
    O, lse = oracle.gated_attention(c.q, c.k, c.v, c.b_raw, c.pos, c.gain, c.temp, c.sm_scale)
    ref = _sdpa(_f32(c.q), _f32(c.k), _f32(c.v), None, c.sm_scale)
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("pos", ["arange", "sparse"])
def test_general_case_against_sdpa_with_bias_mask(pos):
    c = wl.attn_case(M=41, Hq=4, Hkv=2, dh=16, seed=3, r_zero=5, gain=(0.5, 1.5), temp=1.2, pos=pos)
    b = oracle.seq_rmsnorm(c.b_raw, 5, 1e-6)
    O, lse = oracle.gated_attention(c.q, c.k, c.v, b, c.pos, c.gain, c.temp, c.sm_scale)
    M = c.M
    q = _f32(c.q)
    # fold 1/(temp_h * ratio_i) into query row i; the mask adds gain_h * b_j
    ratio = np.array([oracle.temperature_ratio(c.pos[0, i], i) for i in range(M)])
    qs = q / (c.temp[None, None, :, None].astype(np.float64) * ratio[None, :, None, None])
    mask = np.full((1, c.Hq, M, M), -np.inf)
    causal = np.tril(np.ones((M, M), bool))
    for h in range(c.Hq):
        mask[0, h] = np.where(causal, float(c.gain[h]) * b[0][None, :], -np.inf)
    ref = _sdpa(qs, _f32(c.k), _f32(c.v), mask, c.sm_scale)
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-12)
    # lse of the first row: a single key
    for h in range(c.Hq):
        kv = h // 2
        s = float(q[0, 0, h] @ _f32(c.k)[0, 0, kv]) * c.sm_scale / (c.temp[h] * ratio[0])
        assert abs(lse[0, h, 0] - (s + c.gain[h] * b[0, 0])) < 1e-12
        np.testing.assert_allclose(O[0, 0, h], _f32(c.v)[0, 0, kv], rtol=0, atol=1e-15)


def test_gate_form_equals_bias_form():
    c = wl.attn_case(M=29, Hq=4, Hkv=1, dh=8, seed=12, r_zero=3, gain=(0.5, 1.5), temp=0.9, pos="sparse")
    b = oracle.seq_rmsnorm(c.b_raw, 3, 1e-6)
    O8, _ = oracle.gated_attention(c.q, c.k, c.v, b, c.pos, c.gain, c.temp, c.sm_scale)
    O56 = oracle.gated_attention_gate_form(c.q, c.k, c.v, b, c.pos, c.gain, c.temp, c.sm_scale)
    np.testing.assert_allclose(O8, O56, rtol=1e-12, atol=1e-12)


def test_constant_key_score_is_a_no_op():
    c = wl.attn_case(M=33, Hq=2, Hkv=1, dh=8, seed=4, r_zero=33, gain=1.7, temp=1.1)
    O0, l0 = oracle.gated_attention(c.q, c.k, c.v, np.zeros((1, 33)), c.pos, c.gain, c.temp, c.sm_scale)
    O1, l1 = oracle.gated_attention(c.q, c.k, c.v, np.full((1, 33), 2.5), c.pos, c.gain, c.temp, c.sm_scale)
    np.testing.assert_allclose(O1, O0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l0 + float(c.gain[0]) * 2.5, rtol=1e-12, atol=1e-12)


def test_higher_score_means_higher_weight():
    # the gain is positive, so raising b_j raises key j's weight for every
    # query that sees it (read the weight out through a one-hot value)
    M, j = 20, 6
    c = wl.attn_case(M=M, Hq=2, Hkv=1, dh=4, seed=8, r_zero=0, gain=(0.5, 1.5), temp=1.0)
    v = np.zeros((1, M, 1, 4), np.float32)
    v[0, j, 0, 0] = 1.0
    b = np.zeros((1, M))
    O_lo, _ = oracle.gated_attention(c.q, c.k, v, b, c.pos, c.gain, c.temp, c.sm_scale)
    b[0, j] = 0.75
    O_hi, _ = oracle.gated_attention(c.q, c.k, v, b, c.pos, c.gain, c.temp, c.sm_scale)
    w_lo, w_hi = O_lo[0, :, :, 0], O_hi[0, :, :, 0]
    assert np.all(w_lo[:j] == 0) and np.all(w_hi[:j] == 0)
    assert np.all(w_hi[j:] > w_lo[j:])
    assert np.all(w_hi[j:] < 1.0)


def test_sampled_rows_equal_full_rows():
    c = wl.attn_case(M=50, Hq=4, Hkv=2, dh=8, seed=5, r_zero=4, pos="sparse")
    O, lse = oracle.gated_attention(c.q, c.k, c.v, c.b_raw, c.pos, c.gain, c.temp, c.sm_scale)
    rows = np.array([0, 3, 4, 17, 49])
    Os, ls = oracle.gated_attention(c.q, c.k, c.v, c.b_raw, c.pos, c.gain, c.temp, c.sm_scale, rows=rows)
    np.testing.assert_array_equal(Os, O[:, rows])
    np.testing.assert_array_equal(ls, lse[:, :, rows])


# ------------------------------------------------------------ rotary (RoPE) --
def test_rope_position_zero_is_identity():
    x = np.random.default_rng(3).standard_normal((1, 5, 2, 8))
    y = oracle.rope(x.astype(np.float32), np.zeros((1, 5), np.int64), 10000.0)
    np.testing.assert_array_equal(y, x.astype(np.float32).astype(np.float64))


def test_rope_is_complex_rotation():
    # independent form: pair (x_i, x_{i+d/2}) as the complex number
    # x_i + 1j x_{i+d/2}, multiplied by exp(1j * p * base^(-2i/d))
    rng = np.random.default_rng(4)
    d, base = 16, 500.0
    x = rng.standard_normal((2, 7, 3, d)).astype(np.float32)
    pos = rng.integers(0, 100000, (2, 7))
    y = oracle.rope(x, pos, base)
    z = x[..., : d // 2].astype(np.float64) + 1j * x[..., d // 2:].astype(np.float64)
    theta = pos[:, :, None, None].astype(np.float64) * base ** (-np.arange(d // 2) * 2.0 / d)
    w = z * np.exp(1j * theta)
    np.testing.assert_allclose(y[..., : d // 2], w.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[..., d // 2:], w.imag, rtol=0, atol=1e-12)


def test_rope_preserves_pair_norms_and_depends_on_relative_position():
    rng = np.random.default_rng(5)
    d, base = 64, 1e6
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 1, d))
    y = oracle.rope(q, np.array([[12345]]), base)
    h = d // 2
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, q[..., :h] ** 2 + q[..., h:] ** 2, rtol=1e-12)
    # q.k after rotation depends only on the position difference
    dots = []
    for shift in (0, 1000, 70000):
        qr = oracle.rope(q, np.array([[300 + shift]]), base)
        kr = oracle.rope(k, np.array([[17 + shift]]), base)
        dots.append(float(np.sum(qr * kr)))
    np.testing.assert_allclose(dots, dots[0], rtol=0, atol=1e-9)


def test_bf16_round_matches_torch_on_fp32_values_and_ties():
    x = np.random.default_rng(6).standard_normal(50000).astype(np.float32)
    one_half = np.float32(1.5).view(np.uint32)
    ties = np.array([one_half | 0x8000, (one_half + 0x10000) | 0x8000, 0xBF818000], np.uint32).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 3e38, -1e-30], np.float32)])
    got = oracle.bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    # ties go to the even neighbour
    assert list(got[-7:-4]) == [0x3FC0, 0x3FC2, 0xBF82]


def test_bf16_round_rounds_float64_once():
    # 1 + 2^-8 + 2^-30 is just above the midpoint between bf16 1.0 and the next
    # value: direct rounding goes up, rounding through fp32 first (which drops
    # the 2^-30) lands on the tie and goes to even (down)
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert oracle.bf16_round(x)[0] == 0x3F81
    assert torch.tensor(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).item() == 0x3F80


def test_rope_attention_at_position_zero_equals_plain():
    c = wl.attn_case(M=40, Hq=4, Hkv=2, dh=16, seed=8, r_zero=40, gain=1.0, temp=1.0)
    zeros = np.zeros((1, 40), np.int64)
    b = np.zeros((1, 40), np.float32)
    O1, L1 = oracle.gated_attention_rope(c.q, c.k, c.v, b, zeros, c.gain, c.temp, c.sm_scale, 10000.0)
    O2, L2 = oracle.gated_attention(c.q, c.k, c.v, b, zeros, c.gain, c.temp, c.sm_scale)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_rope_attention_worked_example():
    """Rotary attention at sparse original positions against a hand-derived
    closed form (d_h = 2), within the bf16 rounding of the rotated q and k;
    the same inputs rotated the wrong way, or by rank instead of position,
    land far outside that bound."""
    g = json.load(open(os.path.join(GOLD, "rope_attention_worked.json")))
    q = np.array(g["q"], np.float32).reshape(1, 3, 1, 2)
    k = np.array(g["k"], np.float32).reshape(1, 3, 1, 2)
    v = np.array(g["v"], np.float32).reshape(1, 3, 1, 2)
    b = np.array([g["b"]], np.float64)
    pos = np.array([g["pos"]], np.int32)
    gain, one = np.full(1, g["gain"]), np.ones(1)
    O, L = oracle.gated_attention_rope(q, k, v, b, pos, gain, one, 1.0, g["base"])
    np.testing.assert_allclose(O[0, :, 0, :], g["O"], rtol=0, atol=g["tol"])
    np.testing.assert_allclose(L[0, 0], g["lse"], rtol=0, atol=g["tol"])
    # teeth: negated angles (the transposed rotation) and rank-based angles miss by far more
    for wrong in (-pos, np.broadcast_to(np.arange(3, dtype=np.int32), (1, 3))):
        qr = oracle.bf16_round(oracle.rope(q, wrong, g["base"]))
        kr = oracle.bf16_round(oracle.rope(k, wrong, g["base"]))
        Ow, Lw = oracle.gated_attention(qr, kr, v, b, pos, gain, one, 1.0)
        assert np.abs(Ow[0, :, 0, :] - np.array(g["O"])).max() > 4 * g["tol"] or \
            np.abs(Lw[0, 0] - np.array(g["lse"])).max() > 4 * g["tol"]
