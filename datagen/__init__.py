"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it draws random tensors on the host
in float32, rounds each once (round-to-nearest-even, torch's CPU cast) to the
storage dtype, and describes the workload shapes.  Both the HIP path and the CPU
oracle receive exactly these tensors.

Workloads.  The shapes follow the pages' workloads: the forward constants of the
TVM Discuss thread "Developing a faster schedule for Longformer's kernel" (post 6:
b=1, n=4096, h=12, hidden 768 so d=64, w=w_upper=256, 2w+1=513 diagonals), its two
benchmark settings (post 4: dilation 0 and 3), and its typical range (post 3:
sequence up to 512*64, window up to 8192).  No dataset or trained weights are used;
random tensors of these shapes and distributions stand in for the model's
activations.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    b: int
    n: int
    h: int
    d: int
    w: int
    w_upper: int
    dilation: int
    dtype: str          # storage dtype of every input
    out_dtype: str      # dtype of pv / pvT outputs (and of qk's band)
    seed: int
    ops: tuple = field(default=())
    qk_scale: float = 1.0   # Q, K ~ N(0, qk_scale^2)
    padding: float = 0.0

    @property
    def K(self) -> int:
        return self.w + self.w_upper + 1


# The five workloads.  "small" is the oracle-sized case; the others are the
# production shapes (n = 4096 with a 513-slot window, its dilated twin, the
# autoregressive backward pair, and the long-document chain at n = 32768).
WORKLOADS = {
    "small_f32": Workload("small_f32", 1, 512, 1, 64, 32, 32, 0, "f32", "f32", 0,
                          ("qk", "pv")),
    "fwd_n4096_dil0": Workload("fwd_n4096_dil0", 1, 4096, 12, 64, 256, 256, 0, "f16", "f16",
                               1, ("qk",), qk_scale=0.125),
    "fwd_n4096_dil3": Workload("fwd_n4096_dil3", 1, 4096, 12, 64, 256, 256, 3, "f16", "f16",
                               2, ("qk", "pv"), qk_scale=0.125),
    "bwd_n4096_causal": Workload("bwd_n4096_causal", 12, 4096, 12, 64, 256, 0, 0, "bf16", "f32",
                                 3, ("pv", "pvT")),
    "long_n32768": Workload("long_n32768", 1, 32768, 12, 64, 4096, 4096, 0, "f16", "f16", 4,
                            ("qk", "softmax", "pv")),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_dtype(x: np.ndarray, dtype) -> torch.Tensor:
    """float32 host array -> torch CPU tensor of ``dtype`` (one RNE rounding)."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def normal(g: np.random.Generator, shape, dtype, scale: float = 1.0) -> torch.Tensor:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return to_dtype(x, dtype)


def small_ints(g: np.random.Generator, shape, lo: int, hi: int, dtype) -> torch.Tensor:
    """Uniform integers in [lo, hi] stored in ``dtype`` (exact in every float dtype)."""
    return to_dtype(g.integers(lo, hi + 1, size=shape).astype(np.float32), dtype)


def uniform_rows(g: np.random.Generator, shape, dtype) -> torch.Tensor:
    """U(0,1) values, each last-axis row divided by its sum (in float32)."""
    u = g.random(size=shape, dtype=np.float32)
    u /= u.sum(axis=-1, keepdims=True)
    return to_dtype(u, dtype)


def uniform(g: np.random.Generator, shape) -> torch.Tensor:
    """float32 U[0, 1) values (the random numbers a dropout compares with its p)."""
    return torch.from_numpy(g.random(size=shape, dtype=np.float32))


def softmax_rows(g: np.random.Generator, shape, dtype) -> torch.Tensor:
    """Probabilities: a float32 softmax over the whole last axis of N(0,1) logits."""
    z = torch.from_numpy(g.standard_normal(size=shape, dtype=np.float32))
    return torch.softmax(z, dim=-1).to(DTYPES[dtype] if isinstance(dtype, str) else dtype)


def make(wl: Workload, parts=("q", "k", "v", "band")) -> dict:
    """Inputs of a workload, drawn in the fixed order Q, K, V, band from its seed.

    The band operand is the one pv / pvT consume: row-normalised U(0,1) for the
    small fp32 case, a softmax over all K slots of N(0,1) logits for the dilated
    forward, N(0,1) for the backward pair (a gradient band).  Parts that are not
    asked for are still drawn (and dropped) so every part has a fixed stream."""
    g = rng(wl.seed)
    dense = (wl.b, wl.n, wl.h, wl.d)
    band_shape = (wl.b, wl.n, wl.h, wl.K)
    out = {}
    out["q"] = normal(g, dense, wl.dtype, wl.qk_scale)
    out["k"] = normal(g, dense, wl.dtype, wl.qk_scale)
    if "v" in parts or "band" in parts:
        out["v"] = normal(g, dense, wl.dtype)
    if "band" in parts:
        if wl.name.startswith("small"):
            out["band"] = uniform_rows(g, band_shape, wl.dtype)
        elif wl.name.startswith("fwd"):
            out["band"] = softmax_rows(g, band_shape, wl.dtype)
        else:
            out["band"] = normal(g, band_shape, wl.dtype)
    return {k: v for k, v in out.items() if k in parts}


def sample_rows(n: int, w: int, count: int = 64, seed: int = 1004) -> np.ndarray:
    """Positions checked on the long-document workload: the two ends of the sequence
    and the two window edges, then distinct random positions up to ``count``."""
    forced = [0, w - 1, n - w, n - 1]
    forced = sorted({min(max(p, 0), n - 1) for p in forced})
    g = np.random.RandomState(seed)
    rest = [p for p in g.permutation(n) if p not in forced][: max(0, count - len(forced))]
    return np.array(sorted(forced + [int(p) for p in rest]), dtype=np.int64)
