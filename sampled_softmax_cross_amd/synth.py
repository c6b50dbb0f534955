"""Seeded synthetic inputs for the sampled-softmax cross-entropy step.

This module draws inputs only; it holds none of the method's arithmetic, so the
GPU path and the CPU oracle can both take their inputs from it.

Recipe (one microbatch of T tokens, hidden size d, vocabulary V):

* every field has its own numpy ``Generator(PCG64)`` seeded from
  ``SeedSequence([seed, field_id])``, so fields are independent and reproducible;
* x ~ N(0, 1) and W ~ N(0, 0.02^2) (0.02 is the standard deviation), drawn in
  float64, rounded to float32 (round-to-nearest-even) and, for bf16 inputs,
  rounded again to bfloat16 (round-to-nearest-even on the float32 bits);
* targets follow a truncated Zipf law over class ranks, P(rank r) ~ r^-s for
  r = 1..V, sampled by inverse CDF (binary search of a float64 CDF with a
  53-bit uniform), and rank r is class ``perm[r - 1]`` for a seeded permutation
  of the vocabulary; this mimics the heavy-tailed token frequencies of LM
  training text (a few thousand to ~11k distinct targets per microbatch);
* prefix targets, where a workload has them, are an independent draw from the
  same Zipf law (one per token).

The five named workloads are the sizes of the training schedule the method runs
in: P = 10240 through the first stages, 14336 and then 24576 late in stage 2,
and the full 50304-class softmax (P = 0) at the end.
"""
from dataclasses import dataclass, replace

import numpy as np

_FIELD_X, _FIELD_W, _FIELD_PERM, _FIELD_Y, _FIELD_P = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    V: int
    P: int          # 0 = full softmax
    dtype: str      # "bf16" or "f32"
    zipf_s: float
    prefix: bool
    stride: int
    seed: int
    calls: int = 1  # consecutive calls; the candidate offset advances by P per call

    @property
    def offset(self) -> int:
        """Sweep offset of the first call: seed * T mod V."""
        return (self.seed * self.T) % self.V

    def call_offset(self, i: int) -> int:
        return (self.offset + i * self.P) % self.V


WORKLOADS = {
    "tiny": Workload("tiny", 512, 128, 4096, 2048, "f32", 1.1, False, 1021, 0),
    "stage01": Workload("stage01", 16384, 768, 50304, 10240, "bf16", 1.1, False, 20011, 1),
    "s2early": Workload("s2early", 49152, 768, 50304, 14336, "bf16", 1.05, True, 20011, 2),
    "s2late": Workload("s2late", 49152, 768, 50304, 24576, "bf16", 1.05, True, 20011, 3, 4),
    "full": Workload("full", 49152, 768, 50304, 0, "bf16", 1.05, True, 20011, 4),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _rng(seed: int, field: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), field])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 widening of a stored input (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def normal(seed: int, field: int, shape, std: float, dtype: str) -> np.ndarray:
    v = (_rng(seed, field).standard_normal(shape) * std).astype(np.float32)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def zipf_classes(seed: int, field: int, n: int, V: int, s: float, perm: np.ndarray) -> np.ndarray:
    """n class ids: Zipf(s) over ranks 1..V mapped through perm."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = _rng(seed, field).random(n)
    r = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1)
    return perm[r].astype(np.int64)


def class_permutation(seed: int, V: int) -> np.ndarray:
    return _rng(seed, _FIELD_PERM).permutation(V).astype(np.int64)


def make_weights(w: Workload):
    """(x, W) for a workload: x [T,d], W [V,d] as bf16 bits (uint16) or float32."""
    x = normal(w.seed, _FIELD_X, (w.T, w.d), 1.0, w.dtype)
    W = normal(w.seed, _FIELD_W, (w.V, w.d), 0.02, w.dtype)
    return x, W


def make_labels(w: Workload, call: int = 0):
    """(targets, prefix_targets or None) for call `call` of a workload."""
    perm = class_permutation(w.seed, w.V)
    s = w.seed + call
    y = zipf_classes(s, _FIELD_Y, w.T, w.V, w.zipf_s, perm)
    p = zipf_classes(s, _FIELD_P, w.T, w.V, w.zipf_s, perm) if w.prefix else None
    return y, p


def small_case(seed: int, T: int, d: int, V: int, dtype: str = "f32", zipf_s: float = 1.1,
               prefix: bool = True, ignore_frac: float = 0.0):
    """Small random case for parity tests: (x, W, targets, prefix or None).

    A fraction ``ignore_frac`` of targets and prefix targets is set to -1.
    """
    x = normal(seed, _FIELD_X, (T, d), 1.0, dtype)
    W = normal(seed, _FIELD_W, (V, d), 0.02 if d >= 64 else 0.3, dtype)
    perm = class_permutation(seed, V)
    y = zipf_classes(seed, _FIELD_Y, T, V, zipf_s, perm)
    p = zipf_classes(seed, _FIELD_P, T, V, zipf_s, perm) if prefix else None
    if ignore_frac > 0:
        r = _rng(seed, 99)
        y[r.random(T) < ignore_frac] = -1
        if p is not None:
            p[r.random(T) < ignore_frac] = -1
    return x, W, y, p
