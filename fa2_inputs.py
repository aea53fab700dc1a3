"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no attention arithmetic: it only names the workloads and
draws their fp16 tensors, so that the HIP path and the oracle are fed the very
same bits. Nothing here imports either of them.

Recipe (one generator per tensor):
    numpy.random.Generator(PCG64(seed)).standard_normal(shape, float64) * sigma
    -> .astype(float16) (round to nearest even)
with seed = 1000*config + {0: Q, 1: K, 2: V}. Causal and non-causal runs of a
config share the same tensors.

The workloads are the shapes the FlashAttention-2 teaching page measures
(fp16 Q, K, V in [B,H,N,D], head dim 64, scale 1/8, iid inputs, plus a
"concentrated softmax" input made by enlarging Q and K) widened to the sizes
below; there is no public dataset behind them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    cid: int            # workload number, 1..5
    name: str
    B: int
    H: int
    S: int
    D: int
    causal_modes: tuple  # which of (False, True) the workload is run in
    sigma_qk: float      # standard deviation of Q and K entries
    sigma_v: float       # standard deviation of V entries

    @property
    def scale(self) -> float:
        """The softmax scale as the float32 value the kernel receives."""
        return float(np.float32(1.0 / np.sqrt(float(self.D))))

    @property
    def shape(self):
        return (self.B, self.H, self.S, self.D)

    def flops(self, causal: bool) -> float:
        """Attention FLOP count 4*B*H*S^2*D, halved when causal."""
        f = 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2 if causal else f


WORKLOADS = {
    1: Workload(1, "tiny B1 H1 S128 D64", 1, 1, 128, 64, (False, True), 1.0, 1.0),
    2: Workload(2, "B4 H8 S4096 D64", 4, 8, 4096, 64, (False, True), 1.0, 1.0),
    3: Workload(3, "B2 H16 S8192 D128", 2, 16, 8192, 128, (True,), 1.0, 1.0),
    4: Workload(4, "B16 H12 S1000 D64 concentrated", 16, 12, 1000, 64, (False, True), 3.0, 1.0),
    5: Workload(5, "long B1 H32 S16384 D64", 1, 32, 16384, 64, (True,), 1.0, 1.0),
}


def normal_f16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """iid N(0, sigma^2) values rounded to fp16."""
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal(shape, dtype=np.float64) * sigma).astype(np.float16)


def make_inputs(cid: int):
    """(q, k, v) fp16 arrays of shape [B,H,S,D] for workload ``cid``."""
    w = WORKLOADS[cid]
    q = normal_f16(1000 * cid + 0, w.shape, w.sigma_qk)
    k = normal_f16(1000 * cid + 1, w.shape, w.sigma_qk)
    v = normal_f16(1000 * cid + 2, w.shape, w.sigma_v)
    return q, k, v


def make_random(seed: int, B: int, H: int, S: int, D: int, sigma_qk: float = 1.0,
                sigma_v: float = 1.0):
    """(q, k, v) for an arbitrary shape, seeds seed+0/1/2."""
    shape = (B, H, S, D)
    return (normal_f16(seed, shape, sigma_qk), normal_f16(seed + 1, shape, sigma_qk),
            normal_f16(seed + 2, shape, sigma_v))


# ---- workloads of the production features (GQA/MQA, local window, packed
# variable-length sequences, dropout). The page lists these features without
# measuring them; the shapes below keep the head dimension and value
# distribution of the workloads above.

@dataclass(frozen=True)
class FeatureWorkload:
    key: str
    name: str
    B: int                  # batch, or number of packed sequences
    H: int
    H_kv: int
    S: int                  # sequence length, or the longest packed sequence
    D: int
    window: tuple           # (left, right); -1 = unbounded side
    dropout_p: float
    seed: int
    lens: tuple = ()        # packed sequence lengths (varlen only)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(float(self.D))))

    @property
    def packed(self) -> bool:
        return bool(self.lens)


def _packed_lengths(seed: int, n: int, lo: int, hi: int) -> tuple:
    g = np.random.Generator(np.random.PCG64(seed))
    return tuple(int(x) for x in g.integers(lo, hi + 1, size=n))


FEATURES = {
    "gqa": FeatureWorkload("gqa", "GQA B4 H8 H_kv2 S4096 D64", 4, 8, 2, 4096, 64, (-1, -1), 0.0, 6000),
    "mqa": FeatureWorkload("mqa", "MQA B4 H8 H_kv1 S4096 D64", 4, 8, 1, 4096, 64, (-1, -1), 0.0, 6100),
    "window": FeatureWorkload("window", "local window (1024, 1024) B4 H8 S8192 D64", 4, 8, 8, 8192, 64,
                              (1024, 1024), 0.0, 6200),
    "varlen": FeatureWorkload("varlen", "packed 24 sequences of 64..4096 rows, H8 D64", 24, 8, 8, 4096, 64,
                              (-1, -1), 0.0, 6300, _packed_lengths(6399, 24, 64, 4096)),
    "dropout": FeatureWorkload("dropout", "dropout p=0.1 B4 H8 S4096 D64", 4, 8, 8, 4096, 64, (-1, -1),
                               float(np.float32(0.1)), 6400),
}


def make_packed(seed: int, lens, H: int, H_kv: int, D: int, sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """(q [total,H,D], k [total,H_kv,D], v [total,H_kv,D], cu_seqlens int32
    [n+1]) for packed sequences of the given lengths; seeds seed+0/1/2."""
    cu = np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)
    total = int(cu[-1])
    return (normal_f16(seed, (total, H, D), sigma_qk), normal_f16(seed + 1, (total, H_kv, D), sigma_qk),
            normal_f16(seed + 2, (total, H_kv, D), sigma_v), cu)


def make_feature_inputs(key: str):
    """Inputs of feature workload ``key``: (q, k, v) dense [B,H,S,D] /
    [B,H_kv,S,D], or (q, k, v, cu_seqlens) packed."""
    f = FEATURES[key]
    if f.packed:
        return make_packed(f.seed, f.lens, f.H, f.H_kv, f.D)
    return (normal_f16(f.seed, (f.B, f.H, f.S, f.D)), normal_f16(f.seed + 1, (f.B, f.H_kv, f.S, f.D)),
            normal_f16(f.seed + 2, (f.B, f.H_kv, f.S, f.D)))
