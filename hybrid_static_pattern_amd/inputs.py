"""Seeded synthetic inputs for the SAF hybrid attention layer and its calibration score.

This module only draws random numbers and rounds them to the storage type. It holds
none of the attention arithmetic, so the CPU oracle and the HIP path can both be fed
from it without sharing any of the method's code.

Workload recipe (the pages train on a web-text corpus whose activations are not
available; these draws stand in for them):
  * Q, K, V, dO ~ N(0, 1), drawn in float32 and rounded to bfloat16 (round to nearest
    even) when the storage type is bf16.
  * alpha(j) = 0.5 * N(0, 1) per frozen-head key position, with alpha(0) = +4 so the
    first key acts as an attention sink.
  * rho(d) = -0.5 * ln(1 + d) + 0.1 * N(0, 1) for distances d = 0 .. T-1 (recency decay).
  * frozen heads: a seeded sample of k of the H heads, sorted.
  * calibration inputs: per-head logit temperature tau_h, log-spaced over [0.1, 4] and
    permuted by the seed, applied by dividing Q of head h by tau_h before rounding.

Draw order is fixed: Q, K, V, dO, alpha, rho, frozen set (then tau for calibration).
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = (rounded << 16).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already exactly bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return round_to_bf16(x)
    if dtype == FP32:
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def choose_frozen(rng: np.random.Generator, H: int, n_frozen: int) -> np.ndarray:
    """Seeded choice of n_frozen distinct heads out of H, sorted; as a uint8 mask [H]."""
    mask = np.zeros(H, dtype=np.uint8)
    if n_frozen > 0:
        mask[np.sort(rng.choice(H, size=n_frozen, replace=False))] = 1
    return mask


def make_tables(rng: np.random.Generator, H: int, T: int):
    """alpha [H,T] and rho [H,T] in float32, drawn as described in the module docstring."""
    alpha = (0.5 * rng.standard_normal((H, T), dtype=np.float32)).astype(np.float32)
    alpha[:, 0] = 4.0
    d = np.arange(T, dtype=np.float64)
    rho = (-0.5 * np.log1p(d))[None, :] + 0.1 * rng.standard_normal((H, T))
    return alpha, rho.astype(np.float32)


def make_layer(B: int, H: int, T: int, D: int, dtype: str = BF16, seed: int = 0,
               n_frozen: int | None = None, frozen_heads=None, kv_heads: int | None = None) -> dict:
    """Inputs of one hybrid attention layer.

    Returns a dict with q, do ([B,H,T,D]) and k, v ([B,H_kv,T,D]) float32 arrays holding
    dtype-exact values, alpha, rho ([H,T] float32), frozen (uint8 [H]), and the shape/dtype
    fields. H_kv = kv_heads (default H) key/value heads, each shared by H / H_kv query heads.
    Either n_frozen (seeded choice) or frozen_heads (explicit list) selects the frozen set.
    """
    rng = np.random.default_rng(seed)
    H_kv = H if kv_heads is None else kv_heads
    shape, kv_shape = (B, H, T, D), (B, H_kv, T, D)
    q = _store(rng.standard_normal(shape, dtype=np.float32), dtype)
    k = _store(rng.standard_normal(kv_shape, dtype=np.float32), dtype)
    v = _store(rng.standard_normal(kv_shape, dtype=np.float32), dtype)
    do = _store(rng.standard_normal(shape, dtype=np.float32), dtype)
    alpha, rho = make_tables(rng, H, T)
    if frozen_heads is not None:
        frozen = np.zeros(H, dtype=np.uint8)
        frozen[list(frozen_heads)] = 1
    else:
        frozen = choose_frozen(rng, H, int(n_frozen or 0))
    return dict(q=q, k=k, v=v, do=do, alpha=alpha, rho=rho, frozen=frozen,
                B=B, H=H, H_kv=H_kv, T=T, D=D, dtype=dtype, seed=seed)


def randn_bf16_device(torch, shapes, seed: int, device: str = "cuda:0"):
    """Seeded N(0, 1) tensors drawn on the device by torch's generator, in float32 and rounded
    to bfloat16 (nearest even), one per shape, in order. For the workloads too large to draw
    on the host in reasonable time (the longest prefill: 2.4e9 values take minutes with
    numpy); alpha, rho and the frozen set still come from make_tables / choose_frozen."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return [torch.randn(tuple(s), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
            for s in shapes]


def temperatures(rng: np.random.Generator, H: int, lo: float = 0.1, hi: float = 4.0):
    """Per-head logit temperatures, log-spaced over [lo, hi] and permuted by the seed."""
    tau = np.exp(np.linspace(np.log(lo), np.log(hi), H))
    return tau[rng.permutation(H)]


def make_calibration(N: int, H: int, T: int, D: int, dtype: str = BF16, seed: int = 4,
                     tau_range=(0.1, 4.0)) -> dict:
    """Calibration batch for the variance score: q, k [N,H,T,D] and tau [H]."""
    rng = np.random.default_rng(seed)
    shape = (N, H, T, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    tau = temperatures(rng, H, *tau_range)
    q = q / tau.astype(np.float32)[None, :, None, None]
    return dict(q=_store(q, dtype), k=_store(k, dtype), tau=tau,
                N=N, H=H, T=T, D=D, dtype=dtype, seed=seed)


# The workloads, by name. Sizes follow the layer shapes the method is measured on:
# a 124M-parameter model (12 heads of width 64) and a 1B-parameter model (16 heads of
# width 128), at the context lengths used for them.
WORKLOADS = {
    "tiny_fwd_fp32": dict(B=1, H=4, T=256, D=64, dtype=FP32, seed=0, frozen_heads=[3]),
    "l124m_fwd": dict(B=8, H=12, T=4096, D=64, dtype=BF16, seed=1, n_frozen=3),
    "l124m_fwdbwd": dict(B=8, H=12, T=4096, D=64, dtype=BF16, seed=2, n_frozen=3),
    "l1b_fwdbwd": dict(B=2, H=16, T=8192, D=128, dtype=BF16, seed=3, n_frozen=4),
}
CALIBRATION = dict(N=64, H=12, T=1024, D=64, dtype=BF16, seed=4)
# Causal prefill on the 124M shape (forward only): batch 64 over a range of lengths at
# r = 0, 25% and 50%, and the single-sequence case B = 1, T = 4096. The entries below are the
# parity cases; bench.py times the whole range.
WORKLOADS.update({
    "prefill_t512": dict(B=64, H=12, T=512, D=64, dtype=BF16, seed=5, n_frozen=3),
    "prefill_t2048": dict(B=64, H=12, T=2048, D=64, dtype=BF16, seed=6, n_frozen=6),
    "prefill_b1_t4096": dict(B=1, H=12, T=4096, D=64, dtype=BF16, seed=8, n_frozen=6),
})
# Grouped-query attention on the shape of a 4B-parameter model with shared key/value heads
# (32 query heads over 8 key/value heads of width 128), at a 4096-token context.
WORKLOADS.update({
    "gqa_4b": dict(B=1, H=32, T=4096, D=128, dtype=BF16, seed=9, n_frozen=8, kv_heads=8),
})
PREFILL = dict(B=64, H=12, D=64, T=(512, 1024, 2048, 4096, 8192, 16384), n_frozen=(0, 3, 6),
               single=dict(B=1, T=4096), seed=7)
