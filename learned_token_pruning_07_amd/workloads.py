"""Seeded synthetic inputs for the gated-prefill path.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic (no normalisation, scoring, selection or attention).
Both the HIP path and the CPU oracle are fed from here, so the two sides see
the same bytes.

Conventions
-----------
* One ``numpy.random.Generator(PCG64(seed))`` per case; tensors are drawn in
  the order the case lists them, from that one stream.
* bf16 tensors are carried as ``numpy.uint16`` bit patterns, produced from
  fp32 draws by round-to-nearest-even.  fp32 tensors are ``numpy.float32``.
* Weights are N(0, std) as listed, biases are 0, the RMSNorm weight is 1,
  ``eps_row = eps_seq = 1e-6`` and ``sm_scale = 1/sqrt(d_h)``.

The named presets mirror the workloads of the TokenGate paper (Qwen3-1.7B
shapes, 16k-128k contexts, budgets of 1-25 % of the prunable span); the
paper's datasets are not available, so lengths and budget fractions stand in
for them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

EPS_ROW = 1e-6
EPS_SEQ = 1e-6


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# gate inputs (scorer, sequence norm, top-K, compaction)
# --------------------------------------------------------------------------
@dataclass
class GateCase:
    name: str
    B: int
    N: int
    r: int
    d: int
    h: int
    K: int
    dtype: str                 # "bf16" or "f32"
    resid: np.ndarray          # [B,N,d] uint16 bits (bf16) or float32
    norm_w: np.ndarray         # [d]   same dtype as resid
    W1: np.ndarray             # [h,d] same dtype as resid
    b1: np.ndarray             # [h]   float32
    w2: np.ndarray             # [h]   same dtype as resid
    b2: np.ndarray             # [1]   float32
    eps_row: float = EPS_ROW
    eps_seq: float = EPS_SEQ
    extra: dict = field(default_factory=dict)

    @property
    def P(self) -> int:
        return self.N - self.r

    @property
    def Kp(self) -> int:
        return min(self.K, self.N - self.r)

    @property
    def M(self) -> int:
        return self.r + self.Kp


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(dtype)


def gate_case(*, N: int, r: int, d: int, h: int, K: int, dtype: str = "bf16",
              w_std: float = 0.02, seed: int = 0, B: int = 1,
              salient_frac: float = 0.0, salient_scale: float = 4.0,
              heavy_tail_nu: float | None = None, zero_w2: bool = False,
              name: str = "custom") -> GateCase:
    """Draw one gate case.

    Draw order: residual ``[B,N,d]`` ~ N(0,1) (times |t_j| per row when
    ``heavy_tail_nu`` is set: Student-t row norms), then the salient rows
    (``round(salient_frac*N)`` rows drawn without replacement from the
    prunable span of each batch, scaled by ``salient_scale``, an exact power of
    two), then ``W1[h,d]``, then ``w2[h]``, both N(0, w_std).
    """
    rng = make_rng(seed)
    resid = rng.standard_normal((B, N, d), dtype=np.float32)
    if heavy_tail_nu is not None:
        t = rng.standard_t(heavy_tail_nu, size=(B, N)).astype(np.float32)
        resid *= np.abs(t)[..., None]
    salient = None
    if salient_frac > 0.0 and N > r:
        n_sal = int(round(salient_frac * N))
        n_sal = min(n_sal, N - r)
        salient = np.stack([r + rng.choice(N - r, size=n_sal, replace=False)
                            for _ in range(B)])
        for bi in range(B):
            resid[bi, salient[bi]] *= np.float32(salient_scale)
    W1 = (rng.standard_normal((h, d), dtype=np.float32) * np.float32(w_std))
    w2 = (rng.standard_normal((h,), dtype=np.float32) * np.float32(w_std))
    if zero_w2:
        w2[:] = 0.0
    return GateCase(
        name=name, B=B, N=N, r=r, d=d, h=h, K=K, dtype=dtype,
        resid=_cast(resid, dtype),
        norm_w=_cast(np.ones(d, np.float32), dtype),
        W1=_cast(W1, dtype),
        b1=np.zeros(h, np.float32),
        w2=_cast(w2, dtype),
        b2=np.zeros(1, np.float32),
        extra={"salient_rows": salient},
    )


# --------------------------------------------------------------------------
# attention inputs
# --------------------------------------------------------------------------
@dataclass
class AttnCase:
    name: str
    B: int
    M: int
    Hq: int
    Hkv: int
    dh: int
    q: np.ndarray          # [B,M,Hq,dh]  bf16 bits
    k: np.ndarray          # [B,M,Hkv,dh] bf16 bits
    v: np.ndarray          # [B,M,Hkv,dh] bf16 bits
    b_raw: np.ndarray      # [B,M] float32 raw key scores (0 on the first r_zero)
    r_zero: int
    pos: np.ndarray        # [B,M] int32
    gain: np.ndarray       # [Hq] float32 (effective, positive)
    temp: np.ndarray       # [Hq] float32 (effective, positive)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)


def attn_case(*, M: int, Hq: int, Hkv: int, dh: int, seed: int = 0, B: int = 1,
              r_zero: int = 64, gain=(0.5, 1.5), temp: float = 1.2,
              pos: str | np.ndarray = "arange", qkv_std: float = 1.0,
              b_std: float = 1.0, name: str = "custom") -> AttnCase:
    """Draw one attention case.

    Draw order: Q ``[B,M,Hq,dh]``, K, V ``[B,M,Hkv,dh]`` ~ N(0, qkv_std), raw key
    scores ``[B,M]`` ~ N(0, b_std) with the first ``r_zero`` set to 0, then the
    per-head gain ~ U(lo, hi) when ``gain`` is a pair (else the scalar is
    broadcast).  ``pos`` is ``"arange"`` (full-context positions) or
    ``"sparse"`` (sorted distinct positions drawn from ``[0, 2M)`` with
    ``pos[i] >= i``, as after pruning), or an explicit array.
    """
    rng = make_rng(seed)
    q = rng.standard_normal((B, M, Hq, dh), dtype=np.float32) * np.float32(qkv_std)
    k = rng.standard_normal((B, M, Hkv, dh), dtype=np.float32) * np.float32(qkv_std)
    v = rng.standard_normal((B, M, Hkv, dh), dtype=np.float32) * np.float32(qkv_std)
    b = rng.standard_normal((B, M), dtype=np.float32) * np.float32(b_std)
    b[:, :min(r_zero, M)] = 0.0
    if isinstance(gain, tuple):
        g = rng.uniform(gain[0], gain[1], size=Hq).astype(np.float32)
    else:
        g = np.full(Hq, gain, np.float32)
    if isinstance(pos, str):
        if pos == "arange":
            p = np.broadcast_to(np.arange(M, dtype=np.int32), (B, M)).copy()
        elif pos == "sparse":
            # a pruned kept set: the first r_zero ranks are the question span
            # (position == rank), the rest are sorted distinct positions drawn
            # from twice as many candidates, so pos[i] >= i
            rz = min(r_zero, M)
            rows = []
            for _ in range(B):
                tail = np.sort(rng.choice(2 * (M - rz), size=M - rz, replace=False)) + rz
                rows.append(np.concatenate([np.arange(rz), tail]))
            p = np.stack(rows).astype(np.int32)
        else:
            raise ValueError(pos)
    else:
        p = np.ascontiguousarray(pos, dtype=np.int32).reshape(B, M)
    return AttnCase(name=name, B=B, M=M, Hq=Hq, Hkv=Hkv, dh=dh,
                    q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
                    b_raw=b, r_zero=r_zero, pos=p, gain=g,
                    temp=np.full(Hq, temp, np.float32))


# --------------------------------------------------------------------------
# Q/K/V projection glue for the stage workloads.  Not a step of the method:
# it stands in for the projections of the layers above the gate.
# --------------------------------------------------------------------------
@dataclass
class LayerWeights:
    Wq: np.ndarray   # [Hq*dh, d] float32
    Wk: np.ndarray   # [Hkv*dh, d]
    Wv: np.ndarray   # [Hkv*dh, d]
    gain: np.ndarray  # [Hq]
    temp: np.ndarray  # [Hq]


def layer_weights(*, d: int, Hq: int, Hkv: int, dh: int, w_std: float, seed: int,
                  gain=(0.5, 1.5), temp: float = 1.2) -> LayerWeights:
    rng = make_rng(seed)
    Wq = rng.standard_normal((Hq * dh, d), dtype=np.float32) * np.float32(w_std)
    Wk = rng.standard_normal((Hkv * dh, d), dtype=np.float32) * np.float32(w_std)
    Wv = rng.standard_normal((Hkv * dh, d), dtype=np.float32) * np.float32(w_std)
    if isinstance(gain, tuple):
        g = rng.uniform(gain[0], gain[1], size=Hq).astype(np.float32)
    else:
        g = np.full(Hq, gain, np.float32)
    return LayerWeights(Wq=Wq, Wk=Wk, Wv=Wv, gain=g, temp=np.full(Hq, temp, np.float32))


def project_qkv_host(resid_S_f32: np.ndarray, lw: LayerWeights, Hq: int, Hkv: int, dh: int):
    """Host-side glue: fp32 projections of the compacted stream, rounded to bf16 bits."""
    x = np.asarray(resid_S_f32, np.float32)
    B, M, _ = x.shape
    q = (x @ lw.Wq.T).reshape(B, M, Hq, dh)
    k = (x @ lw.Wk.T).reshape(B, M, Hkv, dh)
    v = (x @ lw.Wv.T).reshape(B, M, Hkv, dh)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


# --------------------------------------------------------------------------
# named presets
# --------------------------------------------------------------------------
PRESETS = {
    # tiny end-to-end: fp32 residual, 256->64->1 scorer, one 4q/2kv d_h=64 layer
    "tiny_e2e": dict(N=1024, r=32, d=256, h=64, K=256, dtype="f32", w_std=0.05),
    # gate op at Qwen3-1.7B width, 16k context, 2 % salient rows x4, 10 % budget
    "gate_16k": dict(N=16384, r=64, d=2048, h=256, K=1638, dtype="bf16", w_std=0.02,
                     salient_frac=0.02),
    # full stage: 32k context, 10 % budget, then 24 gated attention layers
    "stage_32k": dict(N=32768, r=64, d=2048, h=256, K=3277, dtype="bf16", w_std=0.02),
    # long-context sweep: 128k context, heavy-tailed row norms (Student-t, nu=3)
    "sweep_128k": dict(N=131072, r=128, d=2048, h=256, K=None, dtype="bf16", w_std=0.02,
                       heavy_tail_nu=3.0),
}

SWEEP_FRACTIONS = (0.01, 0.05, 0.10, 0.25)

# attention-only workload: kept length 4096, 16q/8kv heads, d_h 128
ATTN_4K = dict(M=4096, Hq=16, Hkv=8, dh=128, r_zero=64, gain=(0.5, 1.5), temp=1.2,
               pos="arange")

STAGE_LAYERS = 24
STAGE_HEADS = dict(Hq=16, Hkv=8, dh=128)
TINY_HEADS = dict(Hq=4, Hkv=2, dh=64)


def preset_gate_case(name: str, *, seed: int = 0, K: int | None = None, **over) -> GateCase:
    kw = dict(PRESETS[name])
    kw.update(over)
    if K is not None:
        kw["K"] = K
    if kw.get("K") is None:
        raise ValueError("this preset needs an explicit K")
    return gate_case(seed=seed, name=name, **kw)


def sweep_budgets(N: int = 131072, r: int = 128):
    P = N - r
    return [int(round(f * P)) for f in SWEEP_FRACTIONS]
