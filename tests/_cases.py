"""Shared helpers for the GPU parity tests: cached workload inputs, oracle
results computed on the CPU from the same seeded inputs, and torch <-> numpy
storage conversions.  Oracle inputs never come from the GPU path."""
from __future__ import annotations

import functools

import numpy as np

import hss_synth as syn
import oracle as O


def dt_of(cfg_dtype):
    return O.F32 if cfg_dtype == "f32" else O.BF16


def to_dev(a, dtype):
    import torch
    a = np.ascontiguousarray(a)
    if not a.flags.writeable:
        a = a.copy()
    if dtype == O.F32:
        return torch.from_numpy(a.astype(np.float32, copy=False)).cuda()
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def to_host(t):
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def meta_to_dev(meta):
    import torch
    return torch.from_numpy(np.ascontiguousarray(meta).view(np.int32)).cuda()


@functools.lru_cache(maxsize=None)
def weight(wl, which=0):
    w = syn.weight(syn.WORKLOADS[wl], which)
    w.setflags(write=False)
    return w


@functools.lru_cache(maxsize=None)
def oracle_split(wl, which=0):
    cfg = syn.WORKLOADS[wl]
    W = weight(wl, which)
    dt = dt_of(cfg.dtype)
    if cfg.fmt == "2:4":
        return O.split_24(W, dt)
    m, n = W.shape
    return O.split_csr(W, dt, O.topk_count(m, n, *cfg.frac))


def check_topk_properties(W, dtype, k, row_ptr, col_idx, values, residual=None):
    """The GPU CSR split satisfies the properties that define S uniquely:
    exactly k kept, every kept |w| >= every dropped |w|, ties at the threshold
    kept in row-major order, bits copied, residual = W with +0 on supp(S).
    Pure numpy on the CPU (independent of both the oracle and the GPU)."""
    m, n = W.shape
    bits = W.view(np.uint32) if dtype == O.F32 else W.view(np.uint16).astype(np.uint32)
    mask_bits = 0x7FFFFFFF if dtype == O.F32 else 0x7FFF
    key = (bits & mask_bits).reshape(-1)
    assert row_ptr[0] == 0 and row_ptr[-1] == k and np.all(np.diff(row_ptr) >= 0)
    counts = np.diff(row_ptr.astype(np.int64))
    rows = np.repeat(np.arange(m, dtype=np.int64), counts)
    cols = col_idx.astype(np.int64)
    assert cols.size == k and np.all((cols >= 0) & (cols < n))
    lin = rows * n + cols
    if k > 1:
        d = np.diff(lin)
        assert np.all(d > 0), "columns not strictly ascending within rows"
    kept = np.zeros(m * n, dtype=bool)
    kept[lin] = True
    assert kept.sum() == k
    if 0 < k < m * n:
        T = key[kept].min()
        assert key[~kept].max() <= T
        gt = int(np.count_nonzero(key > T))
        eq_pos = np.flatnonzero(key == T)
        kept_eq = np.flatnonzero(kept & (key == T))
        assert np.array_equal(kept_eq, eq_pos[: k - gt])
    vb = values.view(np.uint32) if dtype == O.F32 else values.view(np.uint16)
    wb = W.reshape(-1).view(vb.dtype)
    assert np.array_equal(vb, wb[lin])
    if residual is not None:
        expect = wb.copy()
        expect[lin] = 0
        assert np.array_equal(residual.reshape(-1).view(vb.dtype), expect)
