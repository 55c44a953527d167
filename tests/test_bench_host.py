"""Host logic of bench.py and the build: counter summaries are tied to the
machine code of the kernel they were taken on.  The build hashes each
kernel's gfx950 code; the bench reads a summary's traffic only while the
hash it carries equals the built one."""

import importlib.util
import json
import os
import shutil
import subprocess

import pytest

from exact_io_aware_52_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_manifest_names_every_kernel():
    if not os.path.exists(build_lib.CODE_MANIFEST):
        build_lib.build()
    hashes = json.load(open(build_lib.CODE_MANIFEST))
    assert {k for k in hashes if not k.startswith("instance:")} == set(build_lib.KERNELS)
    assert all(isinstance(h, str) and len(h) == 16 for h in hashes.values())
    for kern in build_lib.KERNELS:   # every kernel has its instances hashed one by one
        assert any(k.startswith("instance:") and kern + "I" in k for k in hashes), kern


def test_read_traffic_only_for_matching_code(tmp_path, monkeypatch):
    bench = load_bench()
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "code_hashes", lambda: {"fa_bwd_dkdv_kernel": "abcd" * 4})
    path = tmp_path / "profiles" / "fa_bwd_dkdv_kernel_w_traffic.txt"
    path.write_text("kernel: fa_bwd_dkdv_kernel\ncode_sha256: " + "abcd" * 4 +
                    "\ntraffic_bytes_per_launch: 1234.5\n")
    assert bench.read_traffic("fa_bwd_dkdv_kernel", "w") == 1234.5
    path.write_text("code_sha256: " + "ffff" * 4 + "\ntraffic_bytes_per_launch: 1234.5\n")
    assert bench.read_traffic("fa_bwd_dkdv_kernel", "w") is None
    assert bench.read_traffic("fa_bwd_dkdv_kernel", "other") is None
    # a summary naming its instance is matched against that instance's hash
    monkeypatch.setattr(bench, "code_hashes", lambda: {"fa_bwd_dkdv_kernel": "abcd" * 4,
                                                       "instance:_Zinst": "1234" * 4})
    path.write_text("kernel: fa_bwd_dkdv_kernel\ninstance: _Zinst\ncode_sha256: " + "1234" * 4 +
                    "\ntraffic_bytes_per_launch: 99.0\n")
    assert bench.read_traffic("fa_bwd_dkdv_kernel", "w") == 99.0
    path.write_text("instance: _Zinst\ncode_sha256: " + "abcd" * 4 + "\ntraffic_bytes_per_launch: 9\n")
    assert bench.read_traffic("fa_bwd_dkdv_kernel", "w") is None


KERNEL = """#include <hip/hip_runtime.h>
%s
__global__ void fa_probe_kernelI(float* x) { x[threadIdx.x] = x[threadIdx.x] * %s + 1.f; }
"""


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_code_hash_sees_code_not_comments(tmp_path, monkeypatch):
    # The hash is over machine code: a comment changes nothing, a constant does.
    monkeypatch.setattr(build_lib, "BUILD", str(tmp_path))
    monkeypatch.setattr(build_lib, "KERNELS", ("fa_probe_kernel",))

    def hash_of(comment, factor, name):
        src = tmp_path / f"{name}.hip"
        src.write_text(KERNEL % (comment, factor))
        obj = tmp_path / f"{name}.o"
        subprocess.run([build_lib.hipcc(), "-O3", f"--offload-arch={build_lib.ARCH}", "-c",
                        str(src), "-o", str(obj)], check=True, capture_output=True)
        # the probe's mangled name carries the kernel name followed by 'I'
        return build_lib.kernel_code_hashes([str(obj)])["fa_probe_kernel"]

    a = hash_of("", "2.f", "a")
    b = hash_of("// a comment\n/* and another */", "2.f", "b")
    c = hash_of("", "3.f", "c")
    assert a is not None and a == b and a != c


def test_bench_global_names_resolve():
    # Every global name a function of bench.py (or of the package's binding)
    # reads must exist once the module is imported: a missing import would
    # otherwise only fail on the GPU, in the middle of a run.
    import builtins
    import symtable

    from exact_io_aware_52_amd import _binding

    for path, mod in ((os.path.join(ROOT, "bench.py"), load_bench()),
                      (_binding.__file__, _binding)):
        table = symtable.symtable(open(path).read(), path, "exec")
        missing = set()

        def walk(t):
            for child in t.get_children():
                for sym in child.get_symbols():
                    if sym.is_referenced() and (sym.is_global() or
                                                (sym.is_free() and t.get_type() == "module")):
                        name = sym.get_name()
                        if not hasattr(mod, name) and not hasattr(builtins, name):
                            missing.add((child.get_name(), name))
                walk(child)
        walk(table)
        assert not missing, f"{os.path.basename(path)}: unresolved global names {sorted(missing)}"
