"""Host-side checks of bench.py's record handling (no GPU): the kernel source
hash that keys the committed HBM counter summaries ignores comments and blank
lines but not code, and the committed summaries are keyed to the current
kernel sources (so the bench line's ``roofline.traffic`` is not null)."""
from __future__ import annotations

import json
import os
import shutil

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hash_of(tmp_path, edit=None):
    src = os.path.join(ROOT, "quantization_aware_attention_amd", "csrc")
    dst = tmp_path / "quantization_aware_attention_amd" / "csrc"
    shutil.copytree(src, dst)
    if edit:
        edit(dst)
    shutil.copy(os.path.join(ROOT, "bench.py"), tmp_path / "bench.py")
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_copy", tmp_path / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.kernel_source_hash()


def test_hash_ignores_comments_but_not_code(tmp_path):
    base = _hash_of(tmp_path / "a")

    def add_comments(d):
        p = d / "common.hpp"
        p.write_text("// a new line comment\n/* a block\n   comment */\n\n" + p.read_text() + "\n// trailing\n")

    def change_code(d):
        p = d / "common.hpp"
        p.write_text(p.read_text() + "\nconstexpr int kUnusedForHashTest = 1;\n")

    assert _hash_of(tmp_path / "b", add_comments) == base
    assert _hash_of(tmp_path / "c", change_code) != base
    assert base == bench.kernel_source_hash()


@pytest.mark.parametrize("workload", ["dit_image", "cross_fp8v"])
def test_committed_hbm_summaries_match_the_sources(workload):
    rec = json.load(open(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")))
    assert rec["source_hash"] == bench.kernel_source_hash()
    assert bench.measured_traffic("dkdv_kernel", workload) is not None
