"""Seeded synthetic inputs for the BinaryAttention forward workloads.

This module only draws random numbers and arranges them into the shapes of the
workloads; it holds none of the method's arithmetic, so both the GPU path's
tests and the CPU oracle consume the same arrays without sharing any code.

The pages evaluate DeiT-T/S/B on ImageNet-1K (224^2 and 384^2) and DiT-XL/2 on
256^2 latents ("BinaryAttention" paper notes, CVPR 2026, Tables 1 and 3).  The
datasets and trained checkpoints are not available, so seeded Gaussian
activations with those attention shapes stand in for them.

Recipe (per workload, seed = workload index unless given):
  rng = numpy.random.default_rng(seed)  (PCG64)
  Q, K, V = rng.standard_normal([B,H,N,d], float32) drawn in that order;
  then the bias: dense [H,N,N] or relative-position table [H,(2gh-1)*(2gw-1)],
  both standard_normal * 0.02 (float32);
  then, for workloads with outlier channels, round(frac*H*d) (head, channel)
  pairs chosen without replacement, scaled x8 in Q, K and V for every batch item
  and token (in float32, before the cast);
  finally a round-to-nearest-even cast to the workload dtype (fp16 or fp32).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str = "f16"          # "f16" or "f32": dtype of Q, K, V, bias and O
    bias: str = "dense"         # "none", "dense" or "relpos"
    grid: tuple = ()            # (gh, gw) for relpos, gh * gw == N
    outlier_frac: float = 0.0   # fraction of (head, channel) pairs scaled x8
    note: str = field(default="", compare=False)

    @property
    def np_dtype(self):
        return np.float16 if self.dtype == "f16" else np.float32

    def ops(self) -> float:
        """Effective operations of one forward call: 2*B*H*N^2*d for QK^T plus the same for PV."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d


WORKLOADS = [
    Workload("deit_t_toy", 1, 3, 197, 64, "f32", "dense",
             note="DeiT-T-shaped toy: fp32, dense per-head bias"),
    Workload("deit_s_224", 64, 6, 197, 64, "f16", "dense",
             note="DeiT-S 224^2 batch 64: dense per-head bias"),
    Workload("deit_b_384", 32, 12, 577, 64, "f16", "dense", outlier_frac=0.01,
             note="DeiT-B 384^2 batch 32: 1% outlier channels x8, dense per-head bias"),
    Workload("dit_xl2_256", 64, 16, 256, 72, "f16", "relpos", grid=(16, 16),
             note="DiT-XL/2 256^2 latent: d=72, relative-position table bias"),
    Workload("highres_16k", 2, 16, 16384, 64, "f16", "relpos", grid=(128, 128),
             note="high-resolution 128x128 token grid: relative-position table bias"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def make(w: Workload, seed: int | None = None):
    """Draw Q, K, V and the bias for workload w.

    Returns a dict with numpy arrays q, k, v [B,H,N,d] in the workload dtype,
    'bias' (dense [H,N,N], relpos table [H,(2gh-1)(2gw-1)] or None), and the
    workload itself.
    """
    if seed is None:
        seed = WORKLOADS.index(w) if w in WORKLOADS else 0
    rng = np.random.default_rng(seed)
    shape = (w.B, w.H, w.N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    bias = None
    if w.bias == "dense":
        bias = rng.standard_normal((w.H, w.N, w.N), dtype=np.float32) * np.float32(0.02)
    elif w.bias == "relpos":
        gh, gw = w.grid
        assert gh * gw == w.N, "relative-position grid must cover N tokens"
        bias = rng.standard_normal((w.H, (2 * gh - 1) * (2 * gw - 1)), dtype=np.float32) * np.float32(0.02)
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * w.H * w.d))
        pick = rng.choice(w.H * w.d, size=n_out, replace=False)
        for p in pick:
            h, c = divmod(int(p), w.d)
            q[:, h, :, c] *= 8
            k[:, h, :, c] *= 8
            v[:, h, :, c] *= 8
    dt = w.np_dtype
    out = dict(q=q.astype(dt), k=k.astype(dt), v=v.astype(dt),
               bias=None if bias is None else bias.astype(dt), workload=w)
    return out


def custom(B, H, N, d, dtype="f16", bias="dense", grid=(), seed=0, outlier_frac=0.0):
    """Inputs for an ad-hoc shape with the same recipe (used for ragged / edge cases)."""
    return make(Workload(f"custom_{B}x{H}x{N}x{d}", B, H, N, d, dtype, bias, tuple(grid), outlier_frac), seed)


def projection_inputs(B, N, H, d, bias=True, seed=0):
    """Inputs of the QKV projection that produces a workload's Q, K and V.

    Recipe: rng = numpy.random.default_rng(seed); x = standard_normal([B,N,H d]) (the tokens'
    hidden states); w = standard_normal([3 H d, H d]) / sqrt(H d) (so every projected entry has
    unit variance); bias = standard_normal([3 H d]) * 0.02 when asked; all drawn in float32 in
    that order and cast to fp16 (round-to-nearest-even)."""
    rng = np.random.default_rng(seed)
    C = H * d
    x = rng.standard_normal((B, N, C), dtype=np.float32)
    w = rng.standard_normal((3 * C, C), dtype=np.float32) / np.float32(np.sqrt(C))
    b = rng.standard_normal(3 * C, dtype=np.float32) * np.float32(0.02) if bias else None
    return dict(x=x.astype(np.float16), w=w.astype(np.float16), bias=None if b is None else b.astype(np.float16))
