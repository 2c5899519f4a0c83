"""bench.py's host-side logic (no GPU): the one-GPU refusal and the GEMM source digest that
gates the committed counter summary."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_digest_ignores_comments_and_whitespace(tmp_path):
    src = os.path.join(ROOT, "mixture_experts_layer_37_amd", "csrc", "gemm.hip")
    text = open(src, encoding="utf-8").read()
    edited = tmp_path / "comments.hip"
    edited.write_text("// a new leading comment\n" + text.replace("{\n", "{  \n", 3)
                      + "\n/* trailing\n   block comment */\n", encoding="utf-8")
    assert bench.kernel_source_digest(str(edited)) == bench.kernel_source_digest(src)
    changed = tmp_path / "code.hip"
    assert text.count("constexpr int kLA = 8;") >= 1
    changed.write_text(text.replace("constexpr int kLA = 8;", "constexpr int kLA = 4;", 1),
                       encoding="utf-8")
    assert bench.kernel_source_digest(str(changed)) != bench.kernel_source_digest(src)



def test_digest_covers_the_kloop_headers():
    """The committed counters cover the GEMM's k-loop and tile order too, which live in three
    headers."""
    assert set(bench.GEMM_SOURCES) == {"gemm.hip", "packed_kloop.h", "kloop_model.h",
                                       "tile_order.h"}
    whole = bench.kernel_source_digest()
    only = bench.kernel_source_digest(os.path.join(ROOT, "mixture_experts_layer_37_amd", "csrc",
                                                   "gemm.hip"))
    assert whole != only
