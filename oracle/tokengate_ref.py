"""Plain CPU oracle for the TokenGate gated-prefill path (fp64).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does, and it
shares no code with the HIP library.

Source: "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill with
Learned Token Pruning" (the paper), Section 4 ("Scoring Network", "Top-K
Selector", token-gated attention with its "Head-wise" and "Temperature
Scaling" paragraphs, and "Putting everything together") and Appendix C.4.
The paper's display equations did not survive extraction; every formula below
is the plainest reading of the surrounding prose, and the readings are listed
where they are used.

Every function is the definition written out, in float64, over the exact
values the GPU sees (bf16 inputs are widened exactly).  Library primitives
(matrix products, a stable sort) serve as single steps; nothing is blocked,
fused or reordered beyond processing independent rows in chunks to bound
memory.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, invariants stated by the paper, torch CPU library routines on
special cases, and brute force on tiny inputs.  The temperature's log-ratio
form (Eq. 7) is a reading of the prose; it is pinned to that reading's closed
form and to the paper's statement that the temperature is 1 at full context,
but the reading itself is not fixed by the paper.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.4426950408889634


def widen(x) -> np.ndarray:
    """Exact float64 copy of an fp32 array or of bf16 bit patterns (uint16)."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# Eq. 1 + Eq. 3 (first half): row RMSNorm of the post-attention residual and
# the scoring MLP.  Paper, Section 4, "Scoring Network"; Appendix C.4 (the
# scorer reads the normalised residual after layer L's mixer).
#
# Readings: RMSNorm with weight w and eps inside the square root; the MLP is
# Linear(d,h) + b1 -> SiLU -> Linear(h,1) + b2 (the activation named by the
# workload shapes "d->h->1 SiLU").
# --------------------------------------------------------------------------
def score_rows(rows, norm_w, W1, b1, w2, b2, eps_row: float) -> np.ndarray:
    """Raw score b~ for each given residual row ``rows[R, d]`` -> ``[R]``."""
    a = widen(rows)
    w = widen(norm_w)
    W = widen(W1)
    c1 = widen(b1)
    v2 = widen(w2)
    c2 = float(widen(b2).reshape(-1)[0])
    d = a.shape[-1]
    out = np.empty(a.shape[0], np.float64)
    step = 4096
    for s in range(0, a.shape[0], step):
        x = a[s:s + step]
        ms = np.sum(x * x, axis=1) / d                  # mean square of the row
        xt = x / np.sqrt(ms + eps_row)[:, None] * w[None, :]   # Eq. 1
        u = xt @ W.T + c1[None, :]                      # first linear layer
        act = u / (1.0 + np.exp(-u))                    # SiLU
        out[s:s + step] = act @ v2 + c2                 # second linear layer
    return out


def gate_score(resid, r: int, norm_w, W1, b1, w2, b2, eps_row: float, span_end=None) -> np.ndarray:
    """Raw scores ``[B, N]`` for a residual ``[B, N, d]``.

    The prunable tokens are the span ``[r, span_end)`` (``span_end`` None: N,
    the prompt x = [x_R, x_D] with the question first).  Every other token
    is non-prunable and its score is fixed to 0.
    """
    a = np.asarray(resid)
    B, N, _ = a.shape
    p1 = N if span_end is None else span_end
    out = np.zeros((B, N), np.float64)
    for bi in range(B):
        if p1 > r:
            out[bi, r:p1] = score_rows(a[bi, r:p1], norm_w, W1, b1, w2, b2, eps_row)
    return out


# --------------------------------------------------------------------------
# Eq. 3 (second half): RMSNorm of the scalar scores along the sequence.
# Paper, Section 4, "Scoring Network": scores are normalised along the
# sequence with RMSNorm and fixed to zero on the non-prunable tokens; a
# zero-output MLP gives b = 0 everywhere.
#
# Readings: the mean square runs over the prunable span only, there is no
# learnable gain, and eps sits inside the square root (so 0 maps to 0).
# --------------------------------------------------------------------------
def seq_rmsnorm(score_raw, r: int, eps_seq: float, span_end=None) -> np.ndarray:
    """Normalised scores; the prunable span is ``[r, span_end)`` (None: N)."""
    s = widen(score_raw)
    B, N = s.shape
    p1 = N if span_end is None else span_end
    out = np.zeros((B, N), np.float64)
    P = p1 - r
    if P <= 0:
        return out
    for bi in range(B):
        x = s[bi, r:p1]
        ms = np.sum(x * x) / P
        out[bi, r:p1] = x / math.sqrt(ms + eps_seq)
    return out


# --------------------------------------------------------------------------
# Eq. 4: top-K selector.  Paper, Section 4, "Top-K Selector": S holds the K
# highest-scoring prunable tokens plus every non-prunable token.
#
# Readings: K' = min(K, |P|); equal scores go to the lower index; -0.0 and
# +0.0 are equal; a NaN score ranks below every number (including -inf).
# --------------------------------------------------------------------------
def topk_select(score, r: int, K: int, span_end=None) -> np.ndarray:
    """Keep mask ``[B, N]`` (uint8) holding exactly N - P + min(K, P) ones,
    where the prunable span is ``[r, span_end)`` (None: N) of P tokens."""
    s = widen(score)
    B, N = s.shape
    p1 = N if span_end is None else span_end
    keep = np.zeros((B, N), np.uint8)
    keep[:, :r] = 1
    keep[:, p1:] = 1
    P = p1 - r
    Kp = min(K, P)
    if Kp <= 0:
        return keep
    idx = np.arange(P)
    for bi in range(B):
        b = s[bi, r:p1]
        is_nan = np.isnan(b)
        neg = np.where(is_nan, 0.0, -b)
        # ascending order of (is_nan, -b, index): a stable total order
        order = np.lexsort((idx, neg, is_nan))
        keep[bi, r + order[:Kp]] = 1
    return keep


# --------------------------------------------------------------------------
# Compaction.  Paper, Section 4, "Top-K Selector" (the residual stream of
# pruned tokens stops at layer L; S continues through the layer-L MLP and the
# layers above) and Appendix C.4 (kept tokens keep their original positions).
#
# Readings: S keeps ascending original order; the un-normalised residual is
# copied bit for bit; the kept index doubles as the original position.
# --------------------------------------------------------------------------
def compact(resid, keep, score):
    """Return ``kept_idx [B, M]`` int32, ``resid_S [B, M, d]`` (same dtype and
    bits as ``resid``) and ``b_S [B, M]`` (the scores of the kept tokens)."""
    a = np.asarray(resid)
    k = np.asarray(keep)
    sc = np.asarray(score)
    B, N = k.shape
    counts = [int(sum(1 for j in range(N) if k[bi, j])) for bi in range(B)]
    if len(set(counts)) != 1:
        raise ValueError("every batch row must keep the same number of tokens")
    M = counts[0]
    kept_idx = np.zeros((B, M), np.int32)
    resid_S = np.zeros((B, M) + a.shape[2:], a.dtype)
    b_S = np.zeros((B, M), sc.dtype)
    for bi in range(B):
        dst = 0                       # running count of kept tokens before j
        for j in range(N):
            if k[bi, j]:
                kept_idx[bi, dst] = j
                resid_S[bi, dst] = a[bi, j]
                b_S[bi, dst] = sc[bi, j]
                dst += 1
    return kept_idx, resid_S, b_S


# --------------------------------------------------------------------------
# Eq. 7: temperature.  Paper, Section 4, "Temperature Scaling": pruning
# shrinks the number of keys query i sees from its original position count
# p_i to its rank count m_i among kept tokens; the learnable positive
# temperature is scaled by the log-ratio of the two counts and is 1 at full
# context.
#
# Reading: tau_i = temp * ln(p_i) / ln(m_i) with 1-based counts
# p_i = pos_i + 1, m_i = i + 1; the ratio is exactly 1 when p_i == m_i, and
# counts below 2 are clamped to 2 otherwise.
# --------------------------------------------------------------------------
def temperature_ratio(pos_i: int, i: int) -> float:
    p = int(pos_i) + 1
    m = int(i) + 1
    if p == m:
        return 1.0
    return math.log(max(p, 2)) / math.log(max(m, 2))


# --------------------------------------------------------------------------
# Eq. 8 (= Eq. 5 with Eq. 6 substituted): token-gated causal GQA attention.
# Paper, Section 4, token-gated attention, "Head-wise", "Putting everything
# together"; Appendix C.4 (applied in the full-attention layers above L).
#
#   z_ij = (q_i . k_j) * sm_scale / tau_{h,i} + gain_h * b_j,   j <= i
#   O_i  = sum_j softmax_j(z_i) v_j,   lse_i = log sum_j exp(z_ij)
#
# Readings: q-head h reads kv-head h // (Hq / Hkv); the gain multiplies the
# key score outside the temperature; causality runs over kept order.
# --------------------------------------------------------------------------
def gated_attention(q, k, v, b_S, pos, gain, temp, sm_scale: float, rows=None,
                    chunk: int = 1024):
    """Return ``(O, lse)``: ``O [B, R, Hq, dh]`` and ``lse [B, Hq, R]`` in fp64,
    for the query rows ``rows`` (all rows when None)."""
    Q = widen(q)
    Kx = widen(k)
    V = widen(v)
    b = widen(b_S)
    P = np.asarray(pos)
    g = widen(gain)
    t = widen(temp)
    B, M, Hq, dh = Q.shape
    Hkv = Kx.shape[2]
    group = Hq // Hkv
    rows = np.arange(M) if rows is None else np.asarray(rows)
    R = rows.shape[0]
    O = np.zeros((B, R, Hq, dh), np.float64)
    lse = np.zeros((B, Hq, R), np.float64)
    for bi in range(B):
        for h in range(Hq):
            kv = h // group
            Kh = Kx[bi, :, kv, :]
            Vh = V[bi, :, kv, :]
            for s in range(0, R, chunk):
                rr = rows[s:s + chunk]
                tau = t[h] * np.array([temperature_ratio(P[bi, i], i) for i in rr])
                logits = (Q[bi, rr, h, :] @ Kh.T) * sm_scale / tau[:, None]
                z = logits + g[h] * b[bi][None, :]
                causal = np.arange(M)[None, :] <= rr[:, None]
                z = np.where(causal, z, -np.inf)
                zmax = np.max(z, axis=1, keepdims=True)
                e = np.exp(z - zmax)
                den = np.sum(e, axis=1, keepdims=True)
                O[bi, s:s + chunk, h, :] = (e @ Vh) / den
                lse[bi, h, s:s + chunk] = zmax[:, 0] + np.log(den[:, 0])
    return O, lse


def gated_attention_gate_form(q, k, v, b_S, pos, gain, temp, sm_scale: float, rows=None):
    """The same attention in its unsimplified form (Eq. 5 with Eq. 6).

    The gate value of each kept key is ``g_j = softmax_j(gain_h * b_j)`` over
    all kept keys; the attention weight of key j for query i is
    ``g_j * exp(s_ij / tau) / sum_{k<=i} g_k * exp(s_ik / tau)``.  The softmax
    normaliser of g is one constant per head and cancels, which is why Eq. 8
    is a plain additive logit bias.
    """
    Q = widen(q)
    Kx = widen(k)
    V = widen(v)
    b = widen(b_S)
    P = np.asarray(pos)
    gn = widen(gain)
    t = widen(temp)
    B, M, Hq, dh = Q.shape
    group = Hq // Kx.shape[2]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    O = np.zeros((B, rows.shape[0], Hq, dh), np.float64)
    for bi in range(B):
        for h in range(Hq):
            kv = h // group
            x = gn[h] * b[bi]
            gate = np.exp(x - x.max())
            gate = gate / gate.sum()                       # Eq. 6
            for n, i in enumerate(rows):
                tau = t[h] * temperature_ratio(P[bi, i], i)
                s = (Kx[bi, :i + 1, kv, :] @ Q[bi, i, h, :]) * sm_scale / tau
                wgt = gate[:i + 1] * np.exp(s - s.max())   # Eq. 5
                O[bi, n, h, :] = (wgt @ V[bi, :i + 1, kv, :]) / wgt.sum()
    return O


# --------------------------------------------------------------------------
# Rotary position embedding on the original positions.  The paper keeps every
# kept token's original position for the position encoding of the layers
# above L (Appendix C.4) but does not define the encoding itself.
#
# Reading: the rotate-half rotary embedding of the model family the pages
# evaluate.  For a head vector x of even width d at position p, each pair
# (x_i, x_{i+d/2}), i < d/2, is rotated by the angle p * base^(-2i/d).  The
# rotated q and k enter the attention products as bf16 (round to nearest
# even), as the model's own q/k tensors are bf16.
# --------------------------------------------------------------------------
def rope_inv_freq(d: int, base: float) -> np.ndarray:
    """base^(-2i/d), i < d/2, in float64."""
    return np.power(float(base), -2.0 * np.arange(d // 2, dtype=np.float64) / d)


def rope(x, pos, base: float) -> np.ndarray:
    """Rotated copy (float64) of x [B, M, H, d] at positions pos [B, M]."""
    X = widen(x)
    d = X.shape[-1]
    h = d // 2
    ang = np.asarray(pos, np.float64)[:, :, None] * rope_inv_freq(d, base)[None, None, :]
    c = np.cos(ang)[:, :, None, :]
    s = np.sin(ang)[:, :, None, :]
    x1, x2 = X[..., :h], X[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def bf16_round(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of float64 values, rounded to nearest even
    directly from float64 (no intermediate fp32 rounding).  Zeros and values
    in bf16's normal range only."""
    a = np.ascontiguousarray(np.asarray(x, np.float64))
    u = a.view(np.uint64)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    exp = (mag >> np.uint64(52)).astype(np.int64) - 1023
    nz = mag != 0
    if np.any(nz & ((exp < -126) | (exp > 127))):
        raise ValueError("bf16_round: value outside bf16's normal range")
    top = u >> np.uint64(45)                        # sign, exponent, 7 mantissa bits
    rem = u & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (rem > half) | ((rem == half) & ((top & np.uint64(1)) == np.uint64(1)))
    top = top + up.astype(np.uint64)
    r64 = (top << np.uint64(45)).view(np.float64)   # exactly representable in bf16
    bits = (r64.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(nz, bits, (u >> np.uint64(48)).astype(np.uint16))  # keep the sign of zeros


def gated_attention_rope(q, k, v, b_S, pos, gain, temp, sm_scale: float, base: float, rows=None):
    """Token-gated attention (gated_attention) on the rotary-embedded q and k:
    q and k rotated at the original positions pos, rounded to bf16, then Eq. 8."""
    qr = bf16_round(rope(q, pos, base))
    kr = bf16_round(rope(k, pos, base))
    return gated_attention(qr, kr, v, b_S, pos, gain, temp, sm_scale, rows=rows)


# --------------------------------------------------------------------------
# Backward of the token-gated attention (Eq. 8), the path through which the
# gate is trained: the key score b_j enters every logit of key j through
# gain_h * b_j (paper Section 4, token-gated attention and "Putting everything
# together"), so dL/db_j = sum_h gain_h sum_i dZ_{h,ij}.
#
# With z_ij = s_ij c_i + gain_h b_j, c_i = sm_scale / tau_{h,i}, s = q.k,
# P = exp(z - lse) on j <= i and O = P V, for an upstream gradient dO:
#   D_i   = dO_i . O_i
#   dZ_ij = P_ij (dO_i . v_j - D_i)
#   dq_i  = c_i sum_j dZ_ij k_j          dk_j = sum_i c_i dZ_ij q_i
#   dv_j  = sum_i P_ij dO_i              db_j = sum_h gain_h sum_i dZ_{h,ij}
#   dgain_h = sum_ij dZ_{h,ij} b_j       dtemp_h = -(1/temp_h) sum_ij dZ_{h,ij} s_ij c_i
# Reading: like the usual flash-attention backward, D and P are formed from
# the forward's own outputs O (bf16) and lse, which are inputs here.
# --------------------------------------------------------------------------
def gated_attention_backward(q, k, v, b_S, pos, gain, temp, sm_scale: float, O, lse, dO):
    """Return ``(dq, dk, dv, db, dgain, dtemp)`` in float64."""
    Q = widen(q)
    Kx = widen(k)
    V = widen(v)
    b = widen(b_S)
    P_ = np.asarray(pos)
    g = widen(gain)
    t = widen(temp)
    Ox = widen(O)
    L = widen(lse)
    dOx = widen(dO)
    B, M, Hq, dh = Q.shape
    Hkv = Kx.shape[2]
    group = Hq // Hkv
    dq = np.zeros_like(Q)
    dk = np.zeros_like(Kx)
    dv = np.zeros_like(V)
    db = np.zeros((B, M), np.float64)
    dgain = np.zeros(Hq, np.float64)
    dtemp = np.zeros(Hq, np.float64)
    causal = np.arange(M)[None, :] <= np.arange(M)[:, None]
    for bi in range(B):
        for h in range(Hq):
            kv = h // group
            tau = t[h] * np.array([temperature_ratio(P_[bi, i], i) for i in range(M)])
            c = sm_scale / tau
            S = Q[bi, :, h, :] @ Kx[bi, :, kv, :].T
            z = S * c[:, None] + g[h] * b[bi][None, :]
            Pm = np.where(causal, np.exp(np.where(causal, z, 0.0) - L[bi, h][:, None]), 0.0)
            dP = dOx[bi, :, h, :] @ V[bi, :, kv, :].T
            D = np.sum(dOx[bi, :, h, :] * Ox[bi, :, h, :], axis=1)
            dZ = Pm * (dP - D[:, None])
            dS = dZ * c[:, None]
            dq[bi, :, h, :] = dS @ Kx[bi, :, kv, :]
            dk[bi, :, kv, :] += dS.T @ Q[bi, :, h, :]
            dv[bi, :, kv, :] += Pm.T @ dOx[bi, :, h, :]
            col = dZ.sum(axis=0)
            db[bi] += g[h] * col
            dgain[h] += float(col @ b[bi])
            dtemp[h] += -float(np.sum(dS * S)) / t[h]
    return dq, dk, dv, db, dgain, dtemp


def gated_attention_backward_l1(q, k, v, b_S, pos, gain, temp, sm_scale: float, O, lse, dO):
    """Error scales for the backward: each gradient's sum with every summand
    replaced by its absolute value (``sum |dZ| |k| c``, ``sum P |dO|``, ...).
    A result whose summands carry relative errors up to u differs from the
    exact sum by at most u times this L1 sum; the parity tests state their
    tolerances in these units.  Returns the same six arrays as
    :func:`gated_attention_backward`."""
    Q = np.abs(widen(q))
    Kx = np.abs(widen(k))
    V = widen(v)
    b = widen(b_S)
    P_ = np.asarray(pos)
    g = widen(gain)
    t = widen(temp)
    Ox = widen(O)
    L = widen(lse)
    dOx = widen(dO)
    B, M, Hq, dh = Q.shape
    Hkv = Kx.shape[2]
    group = Hq // Hkv
    out = [np.zeros_like(Q), np.zeros_like(Kx), np.zeros_like(V), np.zeros((B, M)), np.zeros(Hq), np.zeros(Hq)]
    causal = np.arange(M)[None, :] <= np.arange(M)[:, None]
    for bi in range(B):
        for h in range(Hq):
            kv = h // group
            tau = t[h] * np.array([temperature_ratio(P_[bi, i], i) for i in range(M)])
            c = sm_scale / tau
            S = widen(q)[bi, :, h, :] @ widen(k)[bi, :, kv, :].T
            z = S * c[:, None] + g[h] * b[bi][None, :]
            Pm = np.where(causal, np.exp(np.where(causal, z, 0.0) - L[bi, h][:, None]), 0.0)
            dP = dOx[bi, :, h, :] @ V[bi, :, kv, :].T
            D = np.sum(dOx[bi, :, h, :] * Ox[bi, :, h, :], axis=1)
            aZ = Pm * np.abs(dP - D[:, None])
            aS = aZ * c[:, None]
            out[0][bi, :, h, :] = aS @ Kx[bi, :, kv, :]
            out[1][bi, :, kv, :] += aS.T @ Q[bi, :, h, :]
            out[2][bi, :, kv, :] += Pm.T @ np.abs(dOx[bi, :, h, :])
            col = aZ.sum(axis=0)
            out[3][bi] += abs(g[h]) * col
            out[4][h] += float(col @ np.abs(b[bi]))
            out[5][h] += float(np.sum(aS * np.abs(S))) / t[h]
    return tuple(out)


# --------------------------------------------------------------------------
# Post-prefill KV-cache pruning of the layers at and below the gate.  Paper,
# Section 5, "Implementation and timing" (with Appendix B): once prefill is
# done, the KV cache of every layer l <= L may keep only the selected tokens,
# so that decoding holds the same kept entries at every layer.  The plain
# definition: a row gather of each layer's K and V cache by the kept set.
# --------------------------------------------------------------------------
def kv_cache_prune(k_cache, v_cache, kept_idx):
    """``k_cache, v_cache [layers, B, N, Hkv, dh]`` (any dtype, rows copied as
    they are), ``kept_idx [B, M]`` -> ``(k_out, v_out) [layers, B, M, Hkv, dh]``."""
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    idx = np.asarray(kept_idx)
    L, B = k_cache.shape[:2]
    M = idx.shape[1]
    k_out = np.empty((L, B, M) + k_cache.shape[3:], k_cache.dtype)
    v_out = np.empty_like(k_out)
    for b in range(B):
        k_out[:, b] = k_cache[:, b, idx[b]]
        v_out[:, b] = v_cache[:, b, idx[b]]
    return k_out, v_out


# --------------------------------------------------------------------------
# Backward of the rotary variant: the gradients with respect to the rotated
# q' = R q, k' = R k (the backward above, on the rotated operands), mapped
# back by the transposed rotation R^T, i.e. the rotation by minus the angle.
# With round_qk, q' and k' are rounded to bf16 as the forward rounds them and
# that rounding is passed through as the identity (the straight-through
# reading of a rounding step); without it, the composition is differentiated
# exactly (used by the finite-difference pin).
# --------------------------------------------------------------------------
def gated_attention_rope_backward(q, k, v, b_S, pos, gain, temp, sm_scale: float, base: float, O, lse, dO,
                                  round_qk: bool = True):
    """Return ``(dq, dk, dv, db, dgain, dtemp)`` in float64 (dq, dk with
    respect to the un-rotated q, k)."""
    qr = rope(q, pos, base)
    kr = rope(k, pos, base)
    if round_qk:
        qr, kr = bf16_round(qr), bf16_round(kr)
    dqr, dkr, dv, db, dgain, dtemp = gated_attention_backward(qr, kr, v, b_S, pos, gain, temp, sm_scale, O, lse, dO)
    neg = -np.asarray(pos, np.float64)
    return rope(dqr, neg, base), rope(dkr, neg, base), dv, db, dgain, dtemp


# --------------------------------------------------------------------------
# A batch of sequences of different lengths, document spans and budgets
# (padded to a common N): each row is the single-sequence gate on its first
# seq_len[b] tokens; padding tokens score 0 and are never kept; the kept sets
# are concatenated in batch order.
# --------------------------------------------------------------------------
def gate_select_varlen(score_raw, resid, seq_len, span_begin, span_end, K, eps_seq: float):
    """Return ``(kept_idx, resid_S, b_S, keep, score, cu_kept)`` with the kept
    rows of all sequences packed (row b's at cu_kept[b] .. cu_kept[b+1]-1)."""
    raw = widen(score_raw)
    res = np.asarray(resid)
    B, N = raw.shape
    score = np.zeros((B, N), np.float64)
    keep = np.zeros((B, N), np.uint8)
    ki, rows, bs, cu = [], [], [], [0]
    for b in range(B):
        n = int(seq_len[b])
        p1 = min(max(int(span_end[b]), 0), n)
        p0 = min(max(int(span_begin[b]), 0), p1)
        k = max(int(K[b]), 0)
        sc = seq_rmsnorm(raw[b:b + 1, :n], p0, eps_seq, span_end=p1)
        kp = topk_select(sc, p0, k, span_end=p1)
        i, r, s = compact(res[b:b + 1, :n], kp, sc)
        score[b, :n] = sc[0]
        keep[b, :n] = kp[0]
        ki.append(i[0])
        rows.append(r[0])
        bs.append(s[0])
        cu.append(cu[-1] + i.shape[1])
    return np.concatenate(ki), np.concatenate(rows), np.concatenate(bs), keep, score, cu
