"""Truncated-SVD factors of the full-size workloads, written by the CPU oracle.

    python tests/golden/make_svd_factors.py            # (re)write every factor file
    python tests/golden/make_svd_factors.py --check    # verify the cache against the manifest

Stage 2 of the HSS page ("LLMの階層的スパース+低ランク圧縮", section
"2段階階層的スパース+低ランク圧縮"): after stage 1 keeps the top fraction of
weights by magnitude, the dense residual is factored at rank r.  For each
full-size workload this script draws the seeded W (hss_synth), splits it with
the oracle (top-k CSR or 2:4), factors the +0-residual with the oracle's
truncated SVD in fp64 and rounds U and V to the workload's storage type (RNE),
exactly as the oracle's own pipeline does for the small cases.  Nothing here
touches the GPU library: every number comes from oracle/ and hss_synth/.

The factors are large (about 87 MB in all), so they live in a cache directory
that is not committed (tests/_svd_cache/); the committed manifest next to this
script records, for every file, the sha256 of the array bytes, the shape and
two closed-form checks taken when it was written:
  * Eckart-Young: ||R - U_r V_r^T||_F (fp64 factors) equals the root-sum-square
    of the discarded singular values;
  * the largest kept and the largest dropped singular value.
A test that finds the cache missing rebuilds it with the same calls (minutes of
CPU); one that finds a file whose hash differs from the manifest fails.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import hss_synth as syn  # noqa: E402  (seeded inputs only)
import oracle as O  # noqa: E402

CACHE = os.path.join(ROOT, "tests", "_svd_cache")
MANIFEST = os.path.join(HERE, "svd_factors_manifest.json")

# (workload key, projection index) of every full-size matrix with a low-rank term
ENTRIES = [("csr4096", 0), ("nm24_11008x4096", 0)] + [("decoder_layer", i) for i in range(7)] + [
    ("csr8192_prefill", 0)]


def _name(key, which):
    return f"{key}.{which}"


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _paths(key, which):
    base = os.path.join(CACHE, _name(key, which))
    return base + ".U.npy", base + ".V.npy"


def compute(key, which):
    """U (m x r), V (n x r) in the workload's storage type, and the record of checks."""
    cfg = syn.WORKLOADS[key]
    dt = O.F32 if cfg.dtype == "f32" else O.BF16
    W = syn.weight(cfg, which)
    m, n = W.shape
    r = cfg.rank[which]
    if cfg.fmt == "2:4":
        sp = O.split_24(W, dt)
    else:
        sp = O.split_csr(W, dt, O.topk_count(m, n, *cfg.frac))
    R64 = O.widen(sp["residual"], dt)
    U64, V64, s = O.truncated_svd(R64, r)
    ey_lhs = float(np.linalg.norm(R64 - U64 @ V64.T))
    ey_rhs = float(np.sqrt(np.sum(s[r:] ** 2)))
    U, V = O.narrow(U64, dt), O.narrow(V64, dt)
    rec = {"m": m, "n": n, "r": r, "dtype": dt,
           "eckart_young_lhs": ey_lhs, "eckart_young_rhs": ey_rhs,
           "sigma_r_minus_1": float(s[r - 1]), "sigma_r": float(s[r]) if r < len(s) else 0.0,
           "sha256_U": _sha(U), "sha256_V": _sha(V)}
    return U, V, rec


def _write(key, which):
    os.makedirs(CACHE, exist_ok=True)
    U, V, rec = compute(key, which)
    pu, pv = _paths(key, which)
    for p, a in ((pu, U), (pv, V)):
        tmp = p + ".tmp.npy"
        np.save(tmp, a)
        os.replace(tmp, p)
    return U, V, rec


def _manifest():
    if not os.path.exists(MANIFEST):
        return {}
    with open(MANIFEST) as f:
        return json.load(f)


def load(key, which):
    """(U, V) of one full-size matrix: from the cache when its bytes match the
    manifest, rebuilt by the oracle when the cache is missing.  A cached file
    whose hash differs from the manifest raises."""
    man = _manifest().get("entries", {}).get(_name(key, which))
    pu, pv = _paths(key, which)
    rebuilt = os.path.join(CACHE, _name(key, which) + ".rebuilt")
    if os.path.exists(pu) and os.path.exists(pv):
        U, V = np.load(pu, allow_pickle=False), np.load(pv, allow_pickle=False)
        # a cache rebuilt on another machine may differ in a few roundings
        # (LAPACK's summation order follows its thread count): the manifest
        # pins only the files written with it
        if man is not None and not os.path.exists(rebuilt) and (
                _sha(U) != man["sha256_U"] or _sha(V) != man["sha256_V"]):
            raise RuntimeError(f"factor cache {_name(key, which)} does not match the manifest")
        return U, V
    U, V, _ = _write(key, which)
    with open(rebuilt, "w") as f:
        f.write("rebuilt by the oracle on this machine\n")
    return U, V


def main(argv):
    check = "--check" in argv
    man = _manifest()
    entries = man.get("entries", {})
    for key, which in ENTRIES:
        name = _name(key, which)
        t0 = time.time()
        if check:
            U, V = load(key, which)
            ok = entries.get(name) and _sha(U) == entries[name]["sha256_U"] and _sha(V) == entries[name]["sha256_V"]
            print(f"{name}: {'ok' if ok else 'MISMATCH'}", flush=True)
            continue
        _, _, rec = _write(key, which)
        entries[name] = rec
        print(f"{name}: {rec['m']}x{rec['n']} r={rec['r']}  EY {rec['eckart_young_lhs']:.6e} vs "
              f"{rec['eckart_young_rhs']:.6e}  ({time.time() - t0:.0f} s)", flush=True)
    if not check:
        out = {"written_by": "tests/golden/make_svd_factors.py (oracle.split_* + oracle.truncated_svd + "
                             "oracle.narrow on hss_synth.weight)",
               "cache_dir": "tests/_svd_cache", "entries": entries}
        with open(MANIFEST, "w") as f:
            json.dump(out, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])
