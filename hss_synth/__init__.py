"""Seeded synthetic inputs for the sparse + low-rank linear layer.

This module only draws random numbers and converts storage types.  It holds
none of the method's arithmetic (no top-k, no factorisation, no products), so
both the CPU oracle's tests and the GPU path's tests/bench can take their
inputs from it without sharing any of the computation under test.

The workloads (WORKLOADS, keyed by name) are the five the layer is measured on: Llama-class
projection shapes with heavy-tailed (Student-t, nu = 3) or Gaussian weights,
optionally with 0.5 % outliers scaled x20 -- the heavy-tailed magnitude
histogram that the HSS page ("LLMの階層的スパース+低ランク圧縮", section
"2段階階層的スパース+低ランク圧縮", actionable-implications paragraph) names
as the case where sparse + low-rank compression pays, and the ~0.5 % outlier
fraction of the SqueezeLLM explainer page (Dense-and-Sparse decomposition).

Storage conventions
-------------------
* fp32 arrays are ``numpy.float32``.
* bf16 arrays are carried as their bit patterns in ``numpy.uint16`` (numpy has
  no bfloat16); ``bf16_bits_to_f32`` widens them exactly.
* Every draw is fp64 first, then rounded fp64 -> fp32 (numpy's RNE cast) and,
  for bf16, fp32 -> bf16 with round-to-nearest-even on the fp32 bits.

Seeding
-------
Each stream is ``numpy.random.Generator(PCG64(SeedSequence([seed, tag, ...])))``
with a fixed tag per role, so changing the batch size never changes W.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "WORKLOADS",
    "Workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "weight",
    "activations",
    "factors",
    "random_matrix",
]

# Stream tags (second entry of the SeedSequence entropy list).
_TAG_W, _TAG_OUT, _TAG_X, _TAG_FAC, _TAG_SMALL, _TAG_DQ = 0, 1, 2, 3, 4, 5


class Workload:
    """One measured workload (shapes, dtype, distribution, S format, rank, batches)."""

    def __init__(self, key, name, shapes, dtype, dist, scale, outliers, fmt, frac, rank, batches,
                 seed, tokens=None, proj_names=None):
        self.key = key
        self.name = name
        self.shapes = list(shapes)        # list of (m, n): out features x in features
        self.dtype = dtype                # "f32" | "bf16"
        self.dist = dist                  # "t3" | "normal"
        self.scale = scale                # multiplier of the unit draw
        self.outliers = outliers          # 0.5 % of entries x20 when True
        self.fmt = fmt                    # "csr" | "2:4"
        self.frac = frac                  # kept fraction (num, den) for CSR; (1, 2) for 2:4
        self.rank = list(rank)            # one rank per shape
        self.batches = tuple(batches)
        self.seed = seed
        self.tokens = tokens              # sequential decode tokens (decoder-layer workload)
        self.proj_names = proj_names or [f"w{i}" for i in range(len(self.shapes))]

    def __repr__(self):
        return f"Workload({self.key!r}, {self.name})"


_L = (4096, 4096)
_UP = (11008, 4096)
_DOWN = (4096, 11008)

WORKLOADS = {
    "csr1024_f32": Workload(
        "csr1024_f32", "1024x1024 f32, top 5% CSR, rank 64, b=1", [(1024, 1024)], "f32", "t3", 0.02,
        False, "csr", (5, 100), [64], (1,), seed=0),
    "csr4096": Workload(
        "csr4096", "4096x4096 bf16 + 0.5% outliers, top 5% CSR, rank 256, b=1,16", [_L], "bf16",
        "t3", 0.02, True, "csr", (5, 100), [256], (1, 16), seed=1),
    "nm24_11008x4096": Workload(
        "nm24_11008x4096", "11008x4096 bf16 + 0.5% outliers, 2:4, rank 64, b=1,8,64", [_UP], "bf16",
        "normal", 0.02, True, "2:4", (1, 2), [64], (1, 8, 64), seed=2),
    # Seven projections of one decoder layer; rank = 10 % of min(m, n), floored: 409.
    "decoder_layer": Workload(
        "decoder_layer", "decoder layer q,k,v,o,gate,up,down bf16, top 3% CSR, rank 409, 256 tokens",
        [_L, _L, _L, _L, _UP, _UP, _DOWN], "bf16", "t3", 0.02, False, "csr", (3, 100),
        [409] * 7, (1,), seed=3, tokens=256, proj_names=["q", "k", "v", "o", "gate", "up", "down"]),
    "csr8192_prefill": Workload(
        "csr8192_prefill", "8192x8192 bf16, top 3% CSR, rank 512, prefill b=2048", [(8192, 8192)], "bf16",
        "t3", 0.015, False, "csr", (3, 100), [512], (2048,), seed=4),
}


def _rng(*entropy):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def f32_to_bf16_bits(a):
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Only finite inputs are expected (the generator never makes NaN)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a64, dtype):
    a32 = a64.astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(dtype)


def _student_t3(rng, size):
    # Student-t with 3 degrees of freedom (numpy's sampler).
    return rng.standard_t(3, size=size)


def weight(cfg: Workload, which: int = 0):
    """W (m x n, row-major) of projection ``which`` of ``cfg``, in the workload's storage type."""
    m, n = cfg.shapes[which]
    rng = _rng(cfg.seed, _TAG_W, which)
    if cfg.dist == "t3":
        w = _student_t3(rng, m * n)
    elif cfg.dist == "normal":
        w = rng.standard_normal(m * n)
    else:
        raise ValueError(cfg.dist)
    w *= cfg.scale
    if cfg.outliers:
        count = (m * n * 5) // 1000
        pos = _rng(cfg.seed, _TAG_OUT, which).choice(m * n, size=count, replace=False)
        w[pos] *= 20.0
    return _store(w, cfg.dtype).reshape(m, n)


def activations(cfg: Workload, b: int, which: int = 0, step: int = 0):
    """X (b x n, row-major) ~ N(0, 1) for projection ``which`` at decode step ``step``."""
    n = cfg.shapes[which][1]
    x = _rng(cfg.seed, _TAG_X, which, step, b).standard_normal(b * n)
    return _store(x, cfg.dtype).reshape(b, n)


def factors(m: int, n: int, r: int, dtype: str, seed: int, which: int = 0, sigma_w: float = 0.02):
    """Stand-in low-rank factors U (m x r) and V (n x r) with an SVD's shapes and scale.

    V has i.i.d. N(0, 1/n) entries (columns of ~unit norm, as singular vectors
    have); column l of U has i.i.d. N(0, (s_l)^2 / m) entries where s_l falls
    linearly from sigma_w*(sqrt(m)+sqrt(n)) to half that across l, roughly the
    leading singular values of an m x n noise matrix with entry scale sigma_w.
    Used where a real factorisation of the residual would cost minutes of CPU;
    the apply step's cost and its error bound do not depend on the values."""
    rng = _rng(seed, _TAG_FAC, which, m, n, r)
    v = rng.standard_normal((n, r)) / np.sqrt(n)
    top = sigma_w * (np.sqrt(m) + np.sqrt(n))
    s = top * np.linspace(1.0, 0.5, num=max(r, 1))[:r]
    u = rng.standard_normal((m, r)) * (s / np.sqrt(m))[None, :]
    return _store(u, dtype).reshape(m, r), _store(v, dtype).reshape(n, r)


def quantised_standin(m: int, n: int, dtype: str, seed: int, sigma_w: float = 0.02):
    """Stand-in 4-bit quantised dense part: codes m x n/2 bytes (two uniform
    random 4-bit codes per byte) and per-row levels m x 16 (16 sorted N(0,
    sigma_w^2) draws), with the shapes and scale a k-means of a weight row
    gives.  Used where quantising a full-size matrix would cost minutes of CPU;
    the apply step's cost and its error bound do not depend on the values."""
    rng = _rng(seed, _TAG_DQ, m, n)
    codes = rng.integers(0, 256, size=(m, n // 2), dtype=np.uint8)
    levels = np.sort(rng.standard_normal((m, 16)) * sigma_w, axis=1)
    return codes, _store(levels, dtype).reshape(m, 16)


_KINDS = ("t3", "normal", "ties", "equal", "zeros", "ints")


def random_matrix(m: int, n: int, dtype: str, seed: int, kind: str = "t3", scale: float = 0.02):
    """Small test matrices with a chosen structure.

    kind: "t3"      Student-t nu=3 x scale
          "normal"  N(0, scale^2)
          "ties"    values drawn from 5 magnitudes with random signs (heavy ties)
          "equal"   every entry +-scale (all magnitudes tie)
          "zeros"   +0 / -0 only
          "ints"    small signed integers (exact in any dtype; many ties)"""
    rng = _rng(seed, _TAG_SMALL, m, n, _KINDS.index(kind))
    size = m * n
    if kind == "t3":
        w = _student_t3(rng, size) * scale
    elif kind == "normal":
        w = rng.standard_normal(size) * scale
    elif kind == "ties":
        mags = np.array([0.0, 0.25, 0.5, 1.0, 2.0]) * scale
        w = mags[rng.integers(0, len(mags), size)] * rng.choice([-1.0, 1.0], size)
    elif kind == "equal":
        w = rng.choice([-1.0, 1.0], size) * scale
    elif kind == "zeros":
        w = rng.choice([-0.0, 0.0], size)
    elif kind == "ints":
        w = rng.integers(-3, 4, size).astype(np.float64)
    else:
        raise ValueError(kind)
    return _store(w, dtype).reshape(m, n)
