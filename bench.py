#!/usr/bin/env python3
"""Throughput of the sparse + low-rank (HSS) linear layer on one MI355X.

Headline workload (one step = one decode token through one decoder layer):
the seven projections of a Llama-7B-class decoder layer (q, k, v, o 4096 x
4096; gate, up 11008 x 4096; down 4096 x 11008), bf16 Student-t (nu = 3) x
0.02 weights, each S = the top 3 % by |w| in CSR (this library's hss_split of
the seeded W) plus factors of rank 409 (10 % of min(m, n)); batch-1 decode.
q/k/v and gate/up read the same input and run as grouped calls, so a token
is four launches.  The factors are seeded stand-ins with a truncated SVD's
shapes and scale (the factorisation is offline; its values do not change
the work -- the parity tests run the oracle's real factors).

Cold-HBM protocol (every timed figure): the compressed operands are
replicated into enough distinct device copies that a pass over them spans
>= 1 GiB, and consecutive steps use consecutive copies.  Exactly K steps are
captured into one HIP graph; before each timed replay a 1 GiB read-write
flush evicts the 256 MB last-level cache, so the steps read HBM whatever K
is.  Several trials give p10 / p50 / p90; `value` is from the median trial.

Also measured (extra JSON keys, each with its own roofline): the 1024^2 fp32
layer (b = 1); the 4096^2 5 % rank-256 layer at b = 1 and 16, its 16-bit
column form, its batched routes side by side, its hierarchical and
dense-and-sparse forms; the 11008 x 4096 2:4 layer at b = 1 / 8 / 64 and its
routes; the 8192^2 prefill at b = 2048 with the low-rank GEMMs alone; a
training step on that layer; hss_split.  `cpu_baseline` times the fp64 CPU
oracle (CSR apply) on a bounded sample of the headline workload.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

METRIC = "sparse+low-rank linear tokens/s + compressed-weight GB/s (% HBM peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROOT = os.path.dirname(os.path.abspath(__file__))
GIB = float(1 << 30)
LAYER_GROUPS = [[0, 1, 2], [3], [4, 5], [6]]          # q k v | o | gate up | down
GROUP_NAMES = ["qkv", "o", "gate_up", "down"]


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="decode tokens per timed region")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--trials", type=int, default=9, help="timed regions (for p10/p50/p90)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip the other workloads")
    ap.add_argument("--only", default=None,
                    help="comma-separated sections to run (headline, csr1024, csr4096, nm24, prefill, train); "
                         "for profiling runs: the JSON line then lacks the sections left out")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run three plain 256 MiB device-to-device copies (a known-size "
                         "reference for hardware byte counters)")
    return ap.parse_args()


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _decode_source_hash():
    """sha256 of the decode kernel's code: the csrc/decode* sources and
    csrc/hss_internal.h in name order, with // comments and blank space
    removed (an edit to a comment does not make measured counters stale)."""
    import re
    csrc = os.path.join(ROOT, "sparse_rank_linear_hss_amd", "csrc")
    names = sorted(f for f in os.listdir(csrc) if f.startswith("decode")) + ["hss_internal.h"]
    code = []
    for f in names:
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        text = re.sub(r"//[^\n]*", "", text)
        code.append(re.sub(r"\s+", " ", text).strip())
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def _measured_traffic(kernel_key):
    """HBM bytes per launch of a decode kernel as two hardware-counter runs
    measured them (profiles/k_decode_hbm_counters.txt), or None when the
    kernels' sources have changed since (the stored hash no longer matches)."""
    path = os.path.join(ROOT, "profiles", "k_decode_hbm_counters.txt")
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    fields = dict(ln.split(":", 1) for ln in lines if ":" in ln and not ln.startswith((" ", "#")))
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("source_sha256") != _decode_source_hash():
        return None
    v = fields.get(f"traffic_bytes_per_launch[{kernel_key}]")
    return float(v) if v else None


def _bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _dev(a, dtype):
    import numpy as np
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return _bf16(a)


def _tdtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


class Layer:
    """One compressed matrix (this library's split of W, stand-in factors)
    and its rotation copies on the device."""

    def __init__(self, H, W, fmt, frac, r, seed, which=0, dtype="bf16", rotation_bytes=GIB, copies=None):
        import hss_synth as syn
        m, n = W.shape
        es = 4 if dtype == "f32" else 2
        self.m, self.n, self.r, self.dtype = m, n, r, dtype
        self.split = H.hss_split(W, fmt, frac=frac)
        U, V = syn.factors(m, n, r, dtype, seed, which)
        self.U, self.Vt = _dev(U, dtype), _dev(V.T, dtype)
        if fmt == "csr":
            self.w_bytes = self.split.k * (es + 4) + 4 * (m + 1) + (m + n) * r * es
        else:
            self.w_bytes = m * n // 2 * es + m * ((n + 31) // 32) * 4 + (m + n) * r * es
        self.copies = copies if copies is not None else max(1, math.ceil(rotation_bytes / self.w_bytes))
        sp = self.split
        td = _tdtype(dtype)
        self.mats = []
        for _ in range(self.copies):
            if fmt == "csr":
                self.mats.append(H.HSSMatrix("csr", m, n, td, U=self.U.clone(), Vt=self.Vt.clone(),
                                             row_ptr=sp.row_ptr.clone(), col_idx=sp.col_idx.clone(),
                                             values=sp.values.clone(), nnz=sp.k))
            else:
                self.mats.append(H.HSSMatrix("2:4", m, n, td, U=self.U.clone(), Vt=self.Vt.clone(),
                                             nm_values=sp.nm_values.clone(), nm_meta=sp.nm_meta.clone()))

    def flops(self, b):
        nnz = self.split.k
        return 2.0 * b * (nnz + self.r * (self.m + self.n))


class Timer:
    """Cold-HBM timing of K steps: one HIP graph of exactly K calls fn(0 ..
    K-1); warm-up calls continue the rotation (fn(K ..)); before each timed
    replay a 1 GiB read-write flush evicts the last-level cache."""

    def __init__(self, trials):
        import torch
        self.trials = trials
        self.flush_buf = torch.zeros(int(GIB), dtype=torch.uint8, device="cuda")

    def flush(self):
        self.flush_buf.add_(1)

    def graph(self, fn, steps, warmup):
        """ms per step of every trial (a list)."""
        import torch
        for i in range(warmup):
            fn(steps + i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        self.flush()
        g.replay()                      # first replay: graph upload (untimed)
        torch.cuda.synchronize()
        out = []
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(self.trials):
            self.flush()
            torch.cuda.synchronize()
            t0.record()
            g.replay()
            t1.record()
            torch.cuda.synchronize()
            out.append(t0.elapsed_time(t1) / steps)
        del g
        return out

    def eager(self, fn, steps, warmup):
        """ms per step of stream launches (no graph), one trial after a flush."""
        import torch
        for i in range(warmup):
            fn(steps + i)
        self.flush()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            fn(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps


def _pct(v):
    import numpy as np
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)), "p90": float(np.percentile(v, 90))}


def _hbm_roofline(bytes_per_launch, ms, kernel, traffic=None):
    gbs = bytes_per_launch / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic, "kernel": kernel, "algorithmic_bytes_per_launch": bytes_per_launch}


def _apply_loop(H, layer, xs, ys, ws):
    mats = layer.mats

    def fn(i):
        H.hss_apply(mats[i % len(mats)], xs[i % len(xs)], ys[i % len(ys)], ws)
    return fn


def _acts(cfg, b, which, count, m, dtype="bf16"):
    import torch
    import hss_synth as syn
    xs = [_dev(syn.activations(cfg, b, which, step), dtype) for step in range(count)]
    ys = [torch.empty((b, m), dtype=_tdtype(dtype), device="cuda") for _ in range(2)]
    return xs, ys


# ---------------------------------------------------------------------------
# Headline: one decoder layer, batch-1 decode
# ---------------------------------------------------------------------------

def _decoder_layer(H, timer, args):
    import torch
    import hss_synth as syn
    wl = syn.WORKLOADS["decoder_layer"]
    tok_bytes = 0
    for (m, n), r in zip(wl.shapes, wl.rank):
        tok_bytes += H.hss_topk_count(m, n, *wl.frac) * 6 + 4 * (m + 1) + (m + n) * r * 2
    copies = max(1, math.ceil(GIB / tok_bytes))          # whole-layer copies: >= 1 GiB per rotation
    projs = []
    for which in range(7):
        Wp = _bf16(syn.weight(wl, which))
        projs.append(Layer(H, Wp, "csr", wl.frac, wl.rank[which], wl.seed, which, copies=copies))
        del Wp
    assert sum(p.w_bytes for p in projs) == tok_bytes
    _log(f"decoder layer ready: {tok_bytes} compressed bytes per token, {copies} layer copies")
    ws = H.apply_workspace(max(H.hss_apply_group_workspace_size([projs[w].mats[0] for w in grp], 1)
                               for grp in LAYER_GROUPS), "cuda")
    xin = [[_bf16(syn.activations(wl, 1, grp[0], s)) for s in range(4)] for grp in LAYER_GROUPS]
    ys = [torch.empty((1, p.m), dtype=torch.bfloat16, device="cuda") for p in projs]
    group_bytes = [sum(projs[w].w_bytes for w in grp) for grp in LAYER_GROUPS]

    def call(gi, i):
        grp = LAYER_GROUPS[gi]
        mats = [projs[w].mats[i % copies] for w in grp]
        if len(grp) == 1:
            H.hss_apply(mats[0], xin[gi][i % 4], ys[grp[0]], ws)
        else:
            H.hss_apply_group(mats, xin[gi][i % 4], [ys[w] for w in grp], ws)

    def step(i):
        for gi in range(len(LAYER_GROUPS)):
            call(gi, i)

    def step_7(i):
        for gi, grp in enumerate(LAYER_GROUPS):
            for w in grp:
                H.hss_apply(projs[w].mats[i % copies], xin[gi][i % 4], ys[w], ws)

    K = args.steps
    trials = timer.graph(step, K, args.warmup)
    ms = sorted(trials)[len(trials) // 2]
    # the config's own 256-token sequence, and the seven-launch order, for reference
    seq = timer.graph(step, wl.tokens, 5) if K != wl.tokens else trials
    ms7 = sorted(timer.graph(step_7, wl.tokens, 5))[len(trials) // 2]

    # per-launch durations: each launch's share of the token, measured as
    # the token graph's time less that of the same graph without the launch
    # (HIP events around the replays on the library's stream, torch's current
    # stream), so a launch's time includes its start after the one before it,
    # as a kernel trace of the sequence records it
    def step_without(skip):
        def f(i):
            for gi in range(len(LAYER_GROUPS)):
                if gi != skip:
                    call(gi, i)
        return f

    per_ms = []
    for gi in range(len(LAYER_GROUPS)):
        t = timer.graph(step_without(gi), K, 5)
        per_ms.append(ms - sorted(t)[len(t) // 2])
    launches = []
    for gi, grp in enumerate(LAYER_GROUPS):
        launches.append({"group": GROUP_NAMES[gi], "projections": [wl.proj_names[w] for w in grp],
                         "algorithmic_bytes": group_bytes[gi], "us_in_sequence": per_ms[gi] * 1e3,
                         "gbs": group_bytes[gi] / (per_ms[gi] * 1e-3) / 1e9,
                         "hbm_frac": group_bytes[gi] / (per_ms[gi] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic_bytes": _measured_traffic(f"decoder_layer.{GROUP_NAMES[gi]}")})
    dom = max(range(len(LAYER_GROUPS)), key=lambda g: per_ms[g])
    roof = _hbm_roofline(group_bytes[dom], per_ms[dom], f"k_decode ({GROUP_NAMES[dom]} launch of the decoder layer)",
                         _measured_traffic(f"decoder_layer.{GROUP_NAMES[dom]}"))
    roof["launch_duration_us"] = per_ms[dom] * 1e3
    roof["traffic_unit"] = "HBM bytes per launch (FETCH_SIZE x read scale + WRITE_SIZE x write scale)"
    res = {"ms_per_token": ms, "trials_ms_per_token": trials, "ms_per_token_pct": _pct(trials),
           "tokens_per_s": 1 / (ms * 1e-3), "bytes_per_token": tok_bytes,
           "gbs": tok_bytes / (ms * 1e-3) / 1e9, "hbm_frac": tok_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "layer_copies": copies, "launches_per_token": len(LAYER_GROUPS), "launches": launches,
           "seq256_ms_per_token_pct": _pct(seq), "ms_per_token_7_launches": ms7,
           "stream_ms_per_token": timer.eager(step, K, 5)}
    del projs
    torch.cuda.empty_cache()
    return res, roof


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle's CSR apply of the same decoder layer
# ---------------------------------------------------------------------------

def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(seconds):
    import numpy as np
    import oracle as O
    import hss_synth as syn
    from threadpoolctl import threadpool_limits
    wl = syn.WORKLOADS["decoder_layer"]
    cores = len(os.sched_getaffinity(0))
    t_prep = time.perf_counter()
    mats = []
    for which in range(7):
        W = syn.weight(wl, which)
        m, n = W.shape
        sp = O.split_csr(W, O.BF16, O.topk_count(m, n, *wl.frac))
        U, V = syn.factors(m, n, wl.rank[which], "bf16", wl.seed, which)
        mats.append((m, n, sp["row_ptr"], sp["col_idx"], sp["values"], O.widen(U, O.BF16), O.widen(V, O.BF16)))
        del W, sp
    xs = [[O.widen(syn.activations(wl, 1, grp[0], s), O.BF16) for s in range(4)] for grp in LAYER_GROUPS]
    t_prep = time.perf_counter() - t_prep

    def token(i):
        for gi, grp in enumerate(LAYER_GROUPS):
            for w in grp:
                m, n, rp, ci, v, U64, V64 = mats[w]
                O.apply_csr(m, n, rp, ci, v, O.BF16, U64, V64, xs[gi][i % 4])

    def run(threads, budget):
        with threadpool_limits(limits=threads):
            token(0)
            calls, t0 = 0, time.perf_counter()
            while True:
                token(calls)
                calls += 1
                el = time.perf_counter() - t0
                if el >= budget or calls >= 100000:
                    return calls, el
    calls, el = run(cores, seconds)
    calls1, el1 = run(1, seconds / 2)
    tok_bytes = sum(len(mm[3]) * 6 + 4 * (mm[0] + 1) + (mm[0] + mm[1]) * mm[5].shape[1] * 2 for mm in mats)
    return {"value": calls / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": _cpu_model(), "single_thread_tokens_per_s": calls1 / el1,
            "gbs": tok_bytes * calls / el / 1e9,
            "sample": f"{calls} decode tokens (b=1) of the decoder layer's 7 projections (top-3% CSR + rank 409) "
                      f"through the fp64 oracle apply_csr (scipy.sparse CSR times x, plus (x V) U^T), "
                      f"{el:.1f} s with BLAS at {cores} threads; {calls1} tokens in {el1:.1f} s at 1 thread; "
                      f"oracle split of the 7 weights took {t_prep:.1f} s (not in value)"}


# ---------------------------------------------------------------------------
# Other workloads
# ---------------------------------------------------------------------------

def _single_layer(H, timer, args, key, b_list, ws_b, extra_routes=None):
    import torch
    import hss_synth as syn
    wl = syn.WORKLOADS[key]
    W = _dev(syn.weight(wl), wl.dtype)
    L = Layer(H, W, "csr" if wl.fmt == "csr" else "2:4", wl.frac, wl.rank[0], wl.seed, dtype=wl.dtype)
    _log(f"{key} ready: {L.copies} rotation copies")
    ws = L.mats[0].workspace(ws_b)
    out = {"w_bytes": L.w_bytes, "rotation_copies": L.copies}
    for b in b_list:
        xs, ys = _acts(wl, b, 0, 4, L.m, wl.dtype)
        steps = max(8, args.steps if b == 1 else args.steps // 4)
        trials = timer.graph(_apply_loop(H, L, xs, ys, ws), steps, args.warmup)
        ms = sorted(trials)[len(trials) // 2]
        out[f"b{b}"] = {"ms": ms, "ms_pct": _pct(trials), "tokens_per_s": b / (ms * 1e-3),
                        "roofline": _hbm_roofline(L.w_bytes, ms, f"hss_apply b={b} (one call)")}
    return L, W, ws, out


def _routes(H, timer, L, wl, batches, routes, skip):
    import hss_synth as syn
    res = {}
    for bq in batches:
        wsq = L.mats[0].workspace(bq)
        xq, yq = _acts(wl, bq, 0, 4, L.m)
        row = {}
        for route in routes:
            if skip(route, bq):
                continue
            with H.option("batch_route", route):
                row[route] = sorted(timer.graph(_apply_loop(H, L, xq, yq, wsq), 16, 4))[timer.trials // 2] * 1e3
        res[f"b{bq}_us"] = row
    return res


def _others(H, timer, args, extra, want):
    if want("csr1024"):
        _csr1024(H, timer, args, extra)
    if want("csr4096"):
        _csr4096(H, timer, args, extra)
    if want("nm24"):
        _nm24(H, timer, args, extra)
    if want("prefill") or want("train"):
        _prefill_train(H, timer, args, extra, want)


def _csr1024(H, timer, args, extra):
    # 1024^2 fp32, top 5 %, rank 64, b = 1 (launch-bound correctness scale)
    L1, W1, _, r1 = _single_layer(H, timer, args, "csr1024_f32", [1], 1)
    extra["csr1024_f32"] = r1
    del L1, W1


def _csr4096(H, timer, args, extra):
    import numpy as np
    import torch
    import hss_synth as syn

    # 4096^2 5 % + rank 256: b = 1, 16; 16-bit columns; routes; hierarchical; dense-and-sparse
    wl = syn.WORKLOADS["csr4096"]
    L, W, ws, r2 = _single_layer(H, timer, args, "csr4096", [1, 16], 16)
    m, n = L.m, L.n
    xs, ys = _acts(wl, 1, 0, 16, m)
    L16 = type("L16", (), {"mats": [A.with_col16() for A in L.mats]})
    bytes16 = L.split.k * (2 + 2) + 4 * (m + 1) + (m + n) * wl.rank[0] * 2
    t16 = timer.graph(_apply_loop(H, L16, xs, ys, ws), args.steps, args.warmup)
    ms16 = sorted(t16)[len(t16) // 2]
    r2["b1_col16"] = {"ms": ms16, "tokens_per_s": 1 / (ms16 * 1e-3),
                      "roofline": _hbm_roofline(bytes16, ms16, "hss_apply b=1, 16-bit columns")}
    del L16
    r2["batch_routes"] = _routes(H, timer, L, wl, (8, 16, 64, 128, 256), ("decode", "spmm", "densify"),
                                 lambda rt, b: (rt == "decode" and b > 64) or (rt == "densify" and b < 24))
    extra["csr4096"] = r2

    # hierarchical form: RCM order of S's support (host), concentration ratio
    # before / after it, 2 x 2 block factors (seeded stand-ins, ranks 96
    # diagonal / 32 off), decode b = 1 three ways: the compact block form in
    # the permuted order (S' = P S P^T; only the blocks' 2 MB of factors),
    # the same blocks packed into zero-padded flat factors (R = 256, 4 MB),
    # and a flat layer of the compact rank 128 (2 MB) on the same S'
    rp_h = L.split.row_ptr.cpu().numpy()
    ci_h = L.split.col_idx.cpu().numpy()
    t0 = time.perf_counter()
    perm = H.hss_rcm_order(rp_h, ci_h, n)
    rcm_ms = (time.perf_counter() - t0) * 1e3
    pos = np.empty(n, dtype=np.int64)
    pos[perm] = np.arange(n)
    rows_h = np.repeat(np.arange(m), np.diff(rp_h))
    bw = [int(np.abs(rows_h - ci_h).max()), int(np.abs(pos[rows_h] - pos[ci_h]).max())]
    perm_d = torch.from_numpy(perm).cuda()
    rho = [float(H.hss_concentration(W)[0]), float(H.hss_concentration(W, perm_d)[0])]
    rd, ro = 96, 32
    hU, hVt = [], []
    for blk in range(4):
        rb = rd if blk in (0, 3) else ro
        Ub, Vb = syn.factors(m // 2, n // 2, rb, "bf16", wl.seed, 10 + blk)
        hU.append(_bf16(Ub))
        hVt.append(_bf16(np.ascontiguousarray(Vb.T)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    Ucat, Vtcat = H.hss_hier_pack(hU, hVt, m, n, perm_d)
    e1.record()
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1)
    sp = L.split
    LH = type("LH", (), {"mats": [H.HSSMatrix("csr", m, n, torch.bfloat16, U=Ucat.clone(), Vt=Vtcat.clone(),
                                              row_ptr=sp.row_ptr.clone(), col_idx=sp.col_idx.clone(),
                                              values=sp.values.clone(), nnz=sp.k) for _ in range(L.copies)]})
    th = timer.graph(_apply_loop(H, LH, xs, ys, ws), args.steps, args.warmup)
    msh = sorted(th)[len(th) // 2]
    del LH, Ucat, Vtcat
    # the compact form in the permuted order
    t0 = time.perf_counter()
    prp, pci, src = H.hss_csr_permute(rp_h, ci_h, perm, n)
    permute_ms = (time.perf_counter() - t0) * 1e3
    prp_d, pci_d = torch.from_numpy(prp).cuda(), torch.from_numpy(pci).cuda()
    pvals = H.hss_gather_values(sp.values, torch.from_numpy(src).cuda())
    Uc, Vtc = H.hss_hier_pack_compact(hU, hVt, m, n)
    hr = [rd, ro, ro, rd]
    LC = type("LC", (), {"mats": [H.HSSMatrix("csr", m, n, torch.bfloat16, U=Uc.clone(), Vt=Vtc.clone(),
                                              row_ptr=prp_d.clone(), col_idx=pci_d.clone(), values=pvals.clone(),
                                              nnz=sp.k, hier_r=hr) for _ in range(L.copies)]})
    wsc = LC.mats[0].workspace(1)
    tc = timer.graph(_apply_loop(H, LC, xs, ys, wsc), args.steps, args.warmup)
    msc = sorted(tc)[len(tc) // 2]
    del LC
    U128, V128 = syn.factors(m, n, rd + ro, "bf16", wl.seed, 20)
    U128, Vt128 = _bf16(U128), _bf16(np.ascontiguousarray(V128.T))
    LF = type("LF", (), {"mats": [H.HSSMatrix("csr", m, n, torch.bfloat16, U=U128.clone(), Vt=Vt128.clone(),
                                              row_ptr=prp_d.clone(), col_idx=pci_d.clone(), values=pvals.clone(),
                                              nnz=sp.k) for _ in range(L.copies)]})
    wsf = LF.mats[0].workspace(1)
    tf = timer.graph(_apply_loop(H, LF, xs, ys, wsf), args.steps, args.warmup)
    msf = sorted(tf)[len(tf) // 2]
    del LF, U128, Vt128
    R_h = 2 * (rd + ro)
    comp_bytes = (m + n) * (rd + ro) * 2
    s_bytes = sp.k * 6 + 4 * (m + 1)
    extra["hier2x2_4096_b1"] = {
        "ms": msc, "tokens_per_s": 1 / (msc * 1e-3), "form": "compact blocks (HSS_HIER2), permuted order",
        "ms_pct": _pct(tc), "ranks_diag_off": [rd, ro],
        "factor_bytes_compact": comp_bytes, "factor_bytes_zero_padded": (m + n) * R_h * 2,
        "roofline": _hbm_roofline(s_bytes + comp_bytes, msc, "hss_apply b=1, compact 2 x 2 blocks"),
        "zero_padded_flat_ms": msh, "flat_rank128_same_bytes_ms": msf,
        "rcm_host_ms": rcm_ms, "csr_permute_host_ms": permute_ms, "pack_ms": pack_ms,
        "rho_identity_rcm": rho, "bandwidth_identity_rcm": bw}
    del Uc, Vtc, hU, hVt, perm_d, prp_d, pci_d, pvals

    # dense-and-sparse form of the same weight: 0.5 % outliers in CSR (this
    # library's split) + a 4-bit quantised dense part (seeded stand-in codes
    # and levels), decode b = 1 and 8
    spo = H.hss_split(W, "csr", frac=(5, 1000))
    codes, levels = syn.quantised_standin(m, n, "bf16", wl.seed)
    codes_d, levels_d = torch.from_numpy(codes).cuda(), _bf16(levels)
    bytes_dq = m * n // 2 + m * 16 * 2 + spo.k * (2 + 4) + 4 * (m + 1)
    dq_copies = max(1, math.ceil(GIB / bytes_dq))
    LDQ = type("LDQ", (), {"mats": [H.HSSMatrix("csr", m, n, torch.bfloat16, row_ptr=spo.row_ptr.clone(),
                                                col_idx=spo.col_idx.clone(), values=spo.values.clone(), nnz=spo.k,
                                                dq_codes=codes_d.clone(), dq_levels=levels_d.clone())
                                   for _ in range(dq_copies)]})
    dq = {"bytes_per_apply": bytes_dq, "outliers": spo.k, "rotation_copies": dq_copies}
    for bq in (1, 8):
        xq, yq = _acts(wl, bq, 0, 4, m)
        tq = timer.graph(_apply_loop(H, LDQ, xq, yq, ws), max(8, args.steps // (1 if bq == 1 else 4)), args.warmup)
        msq = sorted(tq)[len(tq) // 2]
        dq[f"b{bq}"] = {"ms": msq, "tokens_per_s": bq / (msq * 1e-3),
                        "roofline": _hbm_roofline(bytes_dq, msq, f"k_decode_dq b={bq}")}
    extra["dense_sparse_4096_q4"] = dq
    del LDQ, codes_d, levels_d, spo

    # split (offline, once per weight)
    sms = []
    for _ in range(5):
        e0.record()
        H.hss_split(W, "csr", frac=wl.frac, check_finite=False)
        e1.record()
        torch.cuda.synchronize()
        sms.append(e0.elapsed_time(e1))
    split_ms = sorted(sms)[2]
    extra["split_4096sq_bf16"] = {"ms": split_ms, "w_read_gbs": m * n * 2 / (split_ms * 1e-3) / 1e9}
    del L, W
    torch.cuda.empty_cache()


def _nm24(H, timer, args, extra):
    import torch
    import hss_synth as syn
    # 11008 x 4096 2:4, rank 64, b = 1, 8, 64, and its routes
    wl3 = syn.WORKLOADS["nm24_11008x4096"]
    L3, W3, _, r3 = _single_layer(H, timer, args, "nm24_11008x4096", list(wl3.batches), 64)
    r3["batch_routes"] = _routes(H, timer, L3, wl3, (2, 8, 16, 64), ("smfmac", "decode", "densify"),
                                 lambda rt, b: (rt == "decode" and b > 8) or (rt == "densify" and b < 16))
    # the 2:4 split of this weight (offline, once per weight): W read once,
    # from cold HBM (a flush before each call)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sms = []
    for _ in range(5):
        timer.flush()
        torch.cuda.synchronize()
        e0.record()
        H.hss_split(W3, "2:4", check_finite=False)
        e1.record()
        torch.cuda.synchronize()
        sms.append(e0.elapsed_time(e1))
    split_ms = sorted(sms)[2]
    r3["split_ms"] = split_ms
    r3["split_w_read_gbs"] = W3.numel() * 2 / (split_ms * 1e-3) / 1e9
    extra["nm24_11008x4096"] = r3
    del L3, W3
    torch.cuda.empty_cache()


def _prefill_train(H, timer, args, extra, want):
    import ctypes
    import torch
    import hss_synth as syn
    # prefill: 8192^2 CSR 3 %, rank 512, b = 2048 (matrix cores; rotation keeps
    # the densify's read of S honest), and the low-rank products alone
    wl5 = syn.WORKLOADS["csr8192_prefill"]
    W5 = _bf16(syn.weight(wl5))
    L5 = Layer(H, W5, "csr", wl5.frac, wl5.rank[0], wl5.seed, rotation_bytes=GIB / 4)
    _log(f"8192^2 layer ready: {L5.copies} rotation copies")
    b = wl5.batches[0]
    ws5 = L5.mats[0].workspace(b)
    xs5, ys5 = _acts(wl5, b, 0, 2, L5.m)
    if want("prefill"):
        t5 = timer.graph(_apply_loop(H, L5, xs5, ys5, ws5), 8, 2)
        ms5 = sorted(t5)[len(t5) // 2]
        lr = type("LR", (), {"mats": [H.HSSMatrix("csr", L5.m, L5.n, torch.bfloat16, U=mat.U, Vt=mat.Vt,
                                                  row_ptr=torch.zeros(L5.m + 1, dtype=torch.int32, device="cuda"),
                                                  nnz=0) for mat in L5.mats]})
        t5l = timer.graph(_apply_loop(H, lr, xs5, ys5, ws5), 8, 2)
        ms5_lr = sorted(t5l)[len(t5l) // 2]
        lr_flops = 2.0 * b * L5.r * (L5.m + L5.n)
        lr_tf = lr_flops / (ms5_lr * 1e-3) / 1e12
        extra["prefill_8192sq_b2048"] = {
            "ms": ms5, "ms_pct": _pct(t5), "tokens_per_s": b / (ms5 * 1e-3),
            "useful_tflops": L5.flops(b) / (ms5 * 1e-3) / 1e12,
            "dense_equiv_tflops": 2.0 * b * L5.m * L5.n / (ms5 * 1e-3) / 1e12,
            "lowrank_only_ms": ms5_lr, "lowrank_tflops": lr_tf, "lowrank_mfma_frac": lr_tf / BF16_PEAK_TFLOPS,
            "roofline": {"bound": "mfma", "achieved": lr_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": lr_tf / BF16_PEAK_TFLOPS, "traffic": None,
                         "kernel": "low-rank products (T^T = X V, Y = T U^T) of one call with an empty S",
                         "algorithmic_flops_per_call": lr_flops}}
        del lr

    if want("train"):
        # training step on the same layer, b = 2048: forward, parameter gradients
        # (hss_grad) and the input gradient (apply of the transposed layer)
        A5 = L5.mats[0]
        t0 = time.perf_counter()
        At5 = H.hss_transposed_layer(A5)
        torch.cuda.synchronize()
        at_ms = (time.perf_counter() - t0) * 1e3
        gs5 = [_bf16(syn.random_matrix(b, L5.m, "bf16", seed=70 + i, kind="normal", scale=1.0)) for i in range(2)]
        gsz = ctypes.c_size_t(0)
        H._lib.check(H._lib.lib.hss_grad_workspace_size(ctypes.byref(A5.struct), b, ctypes.byref(gsz)), "ws")
        gws = torch.empty(gsz.value, dtype=torch.uint8, device="cuda")
        wst = At5.workspace(b)
        dxs = torch.empty((b, L5.n), dtype=torch.bfloat16, device="cuda")
        ms_fwd = timer.eager(lambda i: H.hss_apply(A5, xs5[i % 2], ys5[i % 2], ws5), 10, 3)
        ms_grad = timer.eager(lambda i: H.hss_grad(A5, xs5[i % 2], gs5[i % 2], ws=gws), 10, 3)
        ms_dx = timer.eager(lambda i: H.hss_apply(At5, gs5[i % 2], dxs, wst), 10, 3)
        ms_gather = timer.eager(lambda i: H.hss_gather_values(A5.values, At5.perm_from_s), 10, 3)
        grad_flops = 2.0 * b * (2 * L5.r * (L5.m + L5.n) + L5.split.k)
        step_ms = ms_fwd + ms_grad + ms_dx + ms_gather
        extra["train_8192sq_b2048"] = {
            "step_ms": step_ms, "tokens_per_s": b / (step_ms * 1e-3),
            "useful_tflops": (2 * L5.flops(b) + grad_flops) / (step_ms * 1e-3) / 1e12,
            "forward_ms": ms_fwd, "grad_ms": ms_grad, "grad_useful_tflops": grad_flops / (ms_grad * 1e-3) / 1e12,
            "dX_ms": ms_dx, "gather_values_ms": ms_gather, "transposed_layer_setup_ms": at_ms,
            "note": "one copy of the weights (compute-bound shape), stream launches"}
        del At5, gs5, gws, wst, dxs, A5, L5, W5
    torch.cuda.empty_cache()


def main():
    args = _args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch

    import sparse_rank_linear_hss_amd as H

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    timer = Timer(args.trials)

    sections = {"headline"} if args.only_headline else (set(args.only.split(",")) if args.only else None)
    want = (lambda name: True) if sections is None else (lambda name: name in sections)
    extra = {}
    if not want("headline"):
        _others(H, timer, args, extra, want)
        print(json.dumps({"metric": METRIC, "value": None, "sections": sorted(sections), **extra}), flush=True)
        return
    head, roof = _decoder_layer(H, timer, args)
    _others(H, timer, args, extra, want)
    ms = head["ms_per_token"]
    out = {
        "metric": METRIC,
        "value": 1.0 / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decoder layer, 7 projections (q,k,v,o 4096x4096; gate,up 11008x4096; down "
                               "4096x11008), bf16 Student-t(3) x0.02, each top-3% CSR + rank-409 factors; batch-1 "
                               "decode, q/k/v and gate/up as grouped calls (4 launches per token); cold HBM "
                               f"({head['layer_copies']} layer copies, 1 GiB flush before each timed region), "
                               "HIP-graph replay",
                   "tokens_per_step": 1, "batch": 1, "rank": 409, "kept_fraction": "3%"},
        "roofline": roof,
        "compressed_gbs_per_token": head["gbs"],
        "hbm_frac_per_token": head["hbm_frac"],
        "decoder_layer_7proj": head,
    }
    out.update(extra)
    out["cpu_baseline"] = None if args.no_cpu_baseline else _cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
