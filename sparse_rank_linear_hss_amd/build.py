"""Build libhss.so (the C-ABI library) in-tree with hipcc for gfx950.

    python sparse_rank_linear_hss_amd/build.py   (standalone: it does not import the package,
                                                 which loads the library it builds)

Each source compiles to an object in _build/ (in parallel), then one link
step writes sparse_rank_linear_hss_amd/libhss.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhss.so")
ARCH = os.environ.get("HSS_OFFLOAD_ARCH", "gfx950")

# decode.hip's kernel instances are spread over the decode_inst_*.hip files so
# that they compile in parallel (the longest first).
SOURCES = ["decode_inst_bf16_csr_b1.hip", "decode_inst_bf16_csr_bn.hip", "decode_inst_bf16_csr16_b1.hip",
           "decode_inst_bf16_csr16_bn.hip", "decode_inst_bf16_nm.hip", "decode_inst_f32.hip", "decode.hip",
           "mfma.hip", "spmm.hip", "nm_mma.hip", "grad.hip", "split.hip", "apply.hip", "hier.hip", "noalloc.hip", "hss_api.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # packed fp32 (v_pk_*_f32) stays off: plain fp32 VALU code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (need ROCm)")


def _compile(src, bdir, extra):
    obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


# Host-sanitizer build (tests/test_host_sanitizers.py): the host code of every
# source instrumented with AddressSanitizer and UndefinedBehaviorSanitizer, the
# device code left as it is (each -fsanitize= applies to the host pass only).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build(verbose: bool = True, sanitize: bool = False, lib: str = None, build_dir: str = None) -> str:
    """Compile every source and link the library (in-tree by default).
    sanitize: the host-sanitizer variant, written to `lib` (required)."""
    bdir = build_dir or (os.path.join(ROOT, "_build", "sanitize") if sanitize else BUILD)
    out = lib or LIB
    if sanitize and lib is None:
        raise ValueError("the sanitizer build needs its own output path")
    os.makedirs(bdir, exist_ok=True)
    extra = SANITIZE if sanitize else []
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, 16, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, bdir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
    sys.exit(0)
