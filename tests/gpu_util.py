"""Helpers shared by the GPU tests: device upload, the accuracy bars, and oracle runs on
sampled heads. The bars are the ones the hot path is held to:
  float32 storage: normwise relative error max|g - o| / max|o| <= 1e-5 per tensor
                   (max|o| replaced by 1 for a tensor that is identically zero);
  bf16 storage:    max |g - o| <= 2e-2 and mean |g - o| <= 2e-3 on values (outputs and
                   float32 gradients), against the float64 oracle on the same inputs.
A key/value head shared by several query heads gets the sum of their gradients: the GPU
tests hold each summand to the bar above (the same layer with K, V repeated per query head)
and the shared gradient to their float32 sum.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import saf_oracle

FP32_REL = 1e-5
BF16_MAX = 2e-2
BF16_MEAN = 2e-3
LSE_ABS = 1e-3


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device")
    return torch.device("cuda:0")


def up(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def down(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(gpu: np.ndarray, ref: np.ndarray, dtype: str, name: str, lse: bool = False):
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    err = np.abs(gpu - ref)
    if lse:
        assert err.max() <= LSE_ABS, f"{name}: max abs err {err.max():.3e}"
        return err.max()
    if dtype == "fp32":
        # A tensor that vanishes identically (dQ, dK at T = 1, where the softmax over a single
        # key has zero gradient) is held to the same 1e-5 against unit scale.
        scale = np.abs(ref).max()
        rel = err.max() / (scale if scale > 0 else 1.0)
        assert rel <= FP32_REL, f"{name}: normwise rel err {rel:.3e}"
        return rel
    assert err.max() <= BF16_MAX, f"{name}: max abs err {err.max():.3e}"
    assert err.mean() <= BF16_MEAN, f"{name}: mean abs err {err.mean():.3e}"
    return err.max()


def layer_on_device(L: dict):
    dt = L["dtype"]
    g = dict(q=up(L["q"], dt), k=up(L["k"], dt), v=up(L["v"], dt), do=up(L["do"], dt),
             alpha=torch.from_numpy(L["alpha"]).to(dev()), rho=torch.from_numpy(L["rho"]).to(dev()))
    return g


def oracle_head(L: dict, b: int, h: int, scale: float):
    """Oracle O, lse, dQ, dK, dV of one (b, h) of a layer dict (full length)."""
    sl = lambda x: x[b:b + 1, h:h + 1]
    fz = L["frozen"][h:h + 1]
    al, rh = L["alpha"][h:h + 1], L["rho"][h:h + 1]
    O, lse = saf_oracle.attn_fwd(sl(L["q"]), sl(L["k"]), sl(L["v"]), fz, al, rh, scale)
    dq, dk, dv = saf_oracle.attn_bwd(sl(L["q"]), sl(L["k"]), sl(L["v"]), sl(L["do"]), fz, al, rh, scale)
    return O[0, 0], lse[0, 0], dq[0, 0], dk[0, 0], dv[0, 0]
