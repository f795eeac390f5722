"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A sanitizer build of libhss.so (every source's host pass instrumented, see
build.py) runs tests/_sanitize_driver.py in a child process with the ASan
runtime preloaded: argument checks, diagnostic switches, workspace sizing,
the host RCM order and CSR transpose (the last two against the oracle).  Any
sanitizer report, or a result differing from the oracle, fails the test.
CPU only: no call in the driver reaches the device."""
import glob
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")


def _sources_hash():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_hss_build", os.path.join(ROOT, "sparse_rank_linear_hss_amd",
                                                                             "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    h = hashlib.sha256()
    for f in sorted(os.listdir(b.CSRC)) + ["../../include/hss.h"]:
        p = os.path.join(b.CSRC, f)
        if os.path.isfile(p):
            h.update(open(p, "rb").read())
    h.update(" ".join(b.COMMON + b.SANITIZE).encode())
    return b, h.hexdigest()


def _sanitized_lib():
    b, digest = _sources_hash()
    lib = os.path.join(OUT, "libhss_sanitize.so")
    stamp = lib + ".sha256"
    if not (os.path.exists(lib) and os.path.exists(stamp) and open(stamp).read() == digest):
        b.build(verbose=False, sanitize=True, lib=lib, build_dir=OUT)
        with open(stamp, "w") as f:
            f.write(digest)
    return lib


def _asan_runtime():
    cand = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cand[-1] if cand else None


@pytest.mark.slow
def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this toolchain")
    lib = _sanitized_lib()
    env = dict(os.environ, HSS_SANITIZED_LIB=lib, LD_PRELOAD=rt, PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "_sanitize_driver.py")], env=env, cwd=ROOT,
                         capture_output=True, text=True, timeout=900)
    report = out.stdout[-3000:] + out.stderr[-6000:]
    assert "AddressSanitizer" not in out.stderr and "runtime error" not in out.stderr, report
    assert out.returncode == 0, report
    assert "host sanitizer driver ok" in out.stdout, report
