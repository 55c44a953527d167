"""Host logic of bench.py: the kernel-source hash that keeps a counter summary
valid is blind to comments and whitespace and sees every code change."""

import importlib.util
import os
import shutil

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_source_hash_ignores_comments_not_code(tmp_path):
    bench = load_bench()
    csrc = tmp_path / "exact_io_aware_52_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "exact_io_aware_52_amd", "csrc"), csrc)
    bench.ROOT = str(tmp_path)
    base = {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES}
    f = csrc / "fa_common.h"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("namespace fa {", "namespace fa {  /* x */\n\n", 1))
    assert {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES} == base
    f.write_text(text.replace("kCusPerXcd = 32", "kCusPerXcd = 16", 1))
    changed = {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES}
    assert all(changed[k] != base[k] for k in base)   # every kernel includes fa_common.h
    f.write_text(text)
    b = csrc / "fa_bwd_impl.h"
    b.write_text(b.read_text().replace("constexpr int NS = 4;", "constexpr int NS = 3;", 1))
    after = {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES}
    assert after["fwd"] == base["fwd"] and after["bwd_dkdv"] != base["bwd_dkdv"]
