"""Q/K/V projections for the stage workloads, outside the library.

Not a step of the method: the layers above the gate project the compacted
residual stream into Q/K/V before their token-gated attention.  These plain
bf16 GEMMs (torch -> hipBLASLt) stand in for those projections with seeded
random weights; the library's attention consumes their output.
"""
from __future__ import annotations

import numpy as np
import torch

from . import workloads as wl


class LayerProj:
    """One layer's projection weights on the GPU (bf16, stored transposed and
    contiguous so every product is a plain 2-D GEMM)."""

    def __init__(self, lw: wl.LayerWeights, Hq: int, Hkv: int, dh: int, device="cuda:0"):
        def up(w):
            bits = wl.f32_to_bf16_bits(np.ascontiguousarray(w.T))
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)

        self.WqT, self.WkT, self.WvT = up(lw.Wq), up(lw.Wk), up(lw.Wv)
        self.gain = torch.from_numpy(lw.gain).to(device)
        self.temp = torch.from_numpy(lw.temp).to(device)
        self.Hq, self.Hkv, self.dh = Hq, Hkv, dh

    def qkv(self, resid_S: torch.Tensor):
        """resid_S [B, M, d] bf16 -> q [B, M, Hq, dh], k, v [B, M, Hkv, dh] bf16."""
        B, M, d = resid_S.shape
        x = resid_S.reshape(B * M, d)
        q = torch.mm(x, self.WqT).view(B, M, self.Hq, self.dh)
        k = torch.mm(x, self.WkT).view(B, M, self.Hkv, self.dh)
        v = torch.mm(x, self.WvT).view(B, M, self.Hkv, self.dh)
        return q, k, v


def stage_layers(n_layers: int, d: int, Hq: int, Hkv: int, dh: int, w_std: float = 0.02, seed0: int = 1000,
                 device="cuda:0"):
    """Seeded projections for n_layers upper layers (layer l uses seed seed0 + l)."""
    return [LayerProj(wl.layer_weights(d=d, Hq=Hq, Hkv=Hkv, dh=dh, w_std=w_std, seed=seed0 + l), Hq, Hkv, dh,
                      device) for l in range(n_layers)]
