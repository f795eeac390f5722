"""CPU checks of bench.py's host logic: the one-GPU contract and the hash
that keys stored hardware-counter figures to the decode kernel's code."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module(root):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.ROOT = root
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


@pytest.fixture()
def csrc_copy(tmp_path):
    src = os.path.join(ROOT, "sparse_rank_linear_hss_amd", "csrc")
    dst = tmp_path / "sparse_rank_linear_hss_amd" / "csrc"
    shutil.copytree(src, dst)
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "k_decode_hbm_counters.txt"), tmp_path / "profiles")
    return tmp_path


def test_decode_hash_ignores_comments_and_follows_code(csrc_copy):
    b = _bench_module(str(csrc_copy))
    h0 = b._decode_source_hash()
    assert h0 == _bench_module(ROOT)._decode_source_hash()
    p = csrc_copy / "sparse_rank_linear_hss_amd" / "csrc" / "decode_kernel.h"
    text = p.read_text()
    p.write_text(text.replace("namespace hss {", "// a new comment line\nnamespace   hss {", 1))
    assert b._decode_source_hash() == h0                       # comments and blank space only
    p.write_text(text.replace("static constexpr int kTReplicas = 8;", "static constexpr int kTReplicas = 4;"))
    assert b._decode_source_hash() != h0                       # the code changed


def test_stored_traffic_is_reported_only_for_the_measured_code(csrc_copy):
    b = _bench_module(str(csrc_copy))
    stored = b._measured_traffic("decoder_layer.gate_up")
    p = csrc_copy / "sparse_rank_linear_hss_amd" / "csrc" / "decode_kernel.h"
    p.write_text(p.read_text().replace("static constexpr int kTReplicas = 8;", "static constexpr int kTReplicas = 4;"))
    assert b._measured_traffic("decoder_layer.gate_up") is None
    assert stored is None or stored > 41_030_172                 # at least the algorithmic bytes
