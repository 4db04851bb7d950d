"""Host-side behaviour of bench.py: the one-GPU guard and the kernel-source digest that keeps the
recorded HBM counters attached to the code they were measured on (no GPU needed)."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration that is not measured


def _digest_of(tmp_path, edit=None):
    csrc = tmp_path / "gated_delta_rule_65_amd" / "csrc"
    if csrc.exists():
        shutil.rmtree(csrc)
    shutil.copytree(os.path.join(ROOT, "gated_delta_rule_65_amd", "csrc"), csrc)
    if edit:
        p = csrc / "kda_decode.hip"
        p.write_text(edit(p.read_text()))
    old = bench.ROOT
    bench.ROOT = str(tmp_path)
    try:
        return bench.kernel_source_digest()
    finally:
        bench.ROOT = old


def test_source_digest_ignores_comments_and_spacing(tmp_path):
    base = _digest_of(tmp_path)
    assert base == bench.kernel_source_digest()
    assert _digest_of(tmp_path, lambda s: "// a new line comment\n/* and a\n block one */\n" + s + "\n\n") == base
    assert _digest_of(tmp_path, lambda s: s.replace("\n", "\n  ", 5)) == base


def test_source_digest_follows_code_changes(tmp_path):
    base = _digest_of(tmp_path)
    assert _digest_of(tmp_path, lambda s: s + "\nstatic int unused_marker = 1;\n") != base
