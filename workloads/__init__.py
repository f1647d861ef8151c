"""Seeded synthetic inputs for video-DiT self-attention with 3D RoPE.

This module only describes workload shapes and draws random numbers. It holds
none of the attention method's arithmetic (no RoPE, rotation, quantization or
softmax), so both the CPU oracle side and the GPU side can take their inputs
from here without sharing any of the method.

Shapes follow the video workloads that the RotateAttention abstract and the
RainFusion2.0 paper discuss (latent token grids laid out frame, height, width;
token counts in the 10K-80K range quoted in RainFusion2.0's introduction).
The pages measure on trained video DiTs that are not available here; these
seeded Gaussian stand-ins take their place, with outlier channels planted per
RoPE frequency group to mimic the RoPE-dependent outliers RotateAttention's
abstract describes.

Every array is drawn in float32 and rounded to float16 (round to nearest
even). Each (batch, head, tensor) has its own counter-free seed derived from a
``numpy.random.SeedSequence``, so a single head can be regenerated without
drawing the others.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ROT_FULL = 0       # one Walsh-Hadamard over the whole head dim
ROT_GROUP64 = 1    # one 64-point Walsh-Hadamard per RoPE group, zero padded
ROT_PAIR = 2       # the mergeable rotation: every RoPE pair turned by pi/4, folded into RoPE

_TENSOR_ID = {"q": 0, "k": 1, "v": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    grid: tuple            # (T, Hh, W) latent token grid
    prefix: int            # text tokens placed before the video tokens (no RoPE)
    split: tuple           # RoPE dims for the (t, h, w) axes, contiguous, in that order
    rotation: int          # ROT_FULL, ROT_GROUP64 or ROT_PAIR
    std: float             # standard deviation of the Gaussian body
    outliers: str          # "group_const", "t3", "lognormal"
    outlier_factor: float  # multiplier for "group_const"
    outliers_per_group: int
    n_t3_channels: int
    head_fallback_frac: float  # share of heads the caller sends to the FP16 path
    tau: float             # block error threshold; inf disables block routing
    seed: int
    base: float = 10000.0

    @property
    def L(self) -> int:
        T, Hh, W = self.grid
        return self.prefix + T * Hh * W

    @property
    def Dp(self) -> int:
        """Head dim after the rotation (192 for the per-group padded Hadamard)."""
        return 3 * 64 if self.rotation == ROT_GROUP64 else self.D

    def credited_ops(self) -> float:
        """4*B*H*L^2*D with the nominal head dim: the attention throughput metric's numerator."""
        return 4.0 * self.B * self.H * float(self.L) ** 2 * self.D

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # 4x8x8 grid, two heads: the small case every test can run in full.
    "tiny": Workload("tiny", B=1, H=2, D=128, grid=(4, 8, 8), prefix=0, split=(44, 42, 42),
                     rotation=ROT_FULL, std=1.0, outliers="group_const", outlier_factor=20.0,
                     outliers_per_group=4, n_t3_channels=0, head_fallback_frac=0.0,
                     tau=math.inf, seed=1001),
    # 480p-style latent grid 21x30x52; heavy-tailed scales on 8 channels; per-group Hadamard.
    "480p": Workload("480p", B=1, H=12, D=128, grid=(21, 30, 52), prefix=0, split=(44, 42, 42),
                     rotation=ROT_GROUP64, std=1.0, outliers="t3", outlier_factor=0.0,
                     outliers_per_group=0, n_t3_channels=8, head_fallback_frac=0.0,
                     tau=math.inf, seed=1002),
    # head dim 64 with a 226-token text prefix that takes no RoPE.
    "smalld": Workload("smalld", B=1, H=48, D=64, grid=(13, 30, 45), prefix=226, split=(22, 21, 21),
                       rotation=ROT_FULL, std=0.5, outliers="group_const", outlier_factor=15.0,
                       outliers_per_group=4, n_t3_channels=0, head_fallback_frac=0.0,
                       tau=math.inf, seed=1003),
    # 480p inputs with 25% of heads on the FP16 path and the 5% block-error rule on.
    "mixed": Workload("mixed", B=1, H=12, D=128, grid=(21, 30, 52), prefix=0, split=(44, 42, 42),
                      rotation=ROT_GROUP64, std=1.0, outliers="t3", outlier_factor=0.0,
                      outliers_per_group=0, n_t3_channels=8, head_fallback_frac=0.25,
                      tau=0.05, seed=1002),
    # 720p-style latent grid 21x45x80 (75600 tokens), 40 heads, lognormal channel scales.
    "720p": Workload("720p", B=1, H=40, D=128, grid=(21, 45, 80), prefix=0, split=(44, 42, 42),
                     rotation=ROT_FULL, std=1.0, outliers="lognormal", outlier_factor=0.0,
                     outliers_per_group=0, n_t3_channels=0, head_fallback_frac=0.0,
                     tau=math.inf, seed=1005),
}

# the order in which the workloads are reported
WORKLOAD_ORDER = ["tiny", "480p", "smalld", "mixed", "720p"]


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def _group_ranges(split):
    off = 0
    out = []
    for g in split:
        out.append((off, off + g))
        off += g
    return out


def _channel_factors(w: Workload, b: int, h: int, tensor: str) -> np.ndarray:
    """Per-channel multipliers for one (batch, head, tensor).

    Q and K share the channel indices of a head (outliers that come from the
    RoPE frequency partition sit in the same channels of both); V draws its
    own indices. Multipliers that are random are drawn per tensor.
    """
    D = w.D
    f = np.ones(D, dtype=np.float32)
    tid = _TENSOR_ID[tensor]
    idx_key = 0 if tensor in ("q", "k") else 1
    ch_rng = _rng(w.seed, b, h, 100 + idx_key)
    val_rng = _rng(w.seed, b, h, 200 + tid)
    if w.outliers == "group_const":
        for lo, hi in _group_ranges(w.split):
            sel = ch_rng.choice(np.arange(lo, hi), size=w.outliers_per_group, replace=False)
            f[sel] = np.float32(w.outlier_factor)
    elif w.outliers == "t3":
        sel = ch_rng.choice(D, size=w.n_t3_channels, replace=False)
        f[sel] = np.abs(val_rng.standard_t(3, size=w.n_t3_channels)).astype(np.float32)
    elif w.outliers == "lognormal":
        f[:] = np.exp(val_rng.standard_normal(D)).astype(np.float32)
    elif w.outliers == "none":
        pass
    else:
        raise ValueError(w.outliers)
    return f


def head_tensor(w: Workload, b: int, h: int, tensor: str, L: int | None = None) -> np.ndarray:
    """One (batch, head) slice of Q, K or V as float16 [L, D]."""
    L = w.L if L is None else L
    rng = _rng(w.seed, b, h, _TENSOR_ID[tensor])
    x = rng.standard_normal((L, w.D), dtype=np.float32)
    x *= np.float32(w.std)
    x *= _channel_factors(w, b, h, tensor)[None, :]
    return x.astype(np.float16)


def head_inputs(w: Workload, b: int, h: int) -> dict:
    return {t: head_tensor(w, b, h, t) for t in ("q", "k", "v")}


def full_inputs(w: Workload, threads: int = 8) -> dict:
    """Q, K, V as float16 [B, H, L, D] arrays (contiguous)."""
    out = {t: np.empty((w.B, w.H, w.L, w.D), dtype=np.float16) for t in ("q", "k", "v")}
    jobs = [(b, h, t) for b in range(w.B) for h in range(w.H) for t in ("q", "k", "v")]

    def run(job):
        b, h, t = job
        out[t][b, h] = head_tensor(w, b, h, t)

    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return out


def head_fallback_mask(w: Workload) -> np.ndarray | None:
    """uint8 [B*H]: 1 for heads the caller routes to the FP16 path; None if none are."""
    n = w.B * w.H
    k = int(round(w.head_fallback_frac * n))
    if k == 0:
        return None
    perm = _rng(w.seed, 7777).permutation(n)
    m = np.zeros(n, dtype=np.uint8)
    m[perm[:k]] = 1
    return m


def random_qkv(L: int, D: int, seed: int, std: float = 1.0, B: int = 1, H: int = 1) -> dict:
    """Plain Gaussian fp16 Q, K, V [B, H, L, D] for edge-case tests."""
    rng = _rng(seed, 4242)
    return {t: (rng.standard_normal((B, H, L, D), dtype=np.float32) * np.float32(std)).astype(np.float16)
            for t in ("q", "k", "v")}
