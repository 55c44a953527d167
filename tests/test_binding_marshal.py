"""CPU tests of the Python binding's marshalling: with a stand-in for libfa.so
that records each call, every binding function must call the entry point of
its own name (or the documented _ex variant), with as many arguments as
include/fa.h declares for it, and put the tile options and output pointers in
the declared positions.  No GPU and no library calls are involved."""

import os
import re

import pytest
import torch

from exact_io_aware_52_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_params():
    """{function: [parameter names]} from the header's prototypes."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(fa_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text):
        params = [p.strip() for p in m.group(2).replace("\n", " ").split(",") if p.strip()]
        if params == ["void"]:
            params = []
        out[m.group(1)] = [re.findall(r"\w+", p)[-1] for p in params]
    return out


class FakeLib:
    """Records (name, args) of each call; returns FA_OK and fixed sizes."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append((name, args))
            if name.endswith("_workspace_bytes"):
                return 4096
            if name == "fa_forward_block_rows_for":
                return 128
            return 0
        return fn


@pytest.fixture
def fake(monkeypatch):
    lib = FakeLib()
    monkeypatch.setattr(_binding, "load_library", lambda: lib)
    monkeypatch.setattr(_binding, "_stream", lambda device: None)
    # the binding refuses CPU tensors (the library has no CPU path); only the
    # marshalling is under test here
    monkeypatch.setattr(_binding, "_shape", lambda q, k, v: q.shape)
    return lib


def tensors(B=1, H=2, N=100, d=64):
    q, k, v, o, do = (torch.zeros(B, H, N, d, dtype=torch.bfloat16) for _ in range(5))
    lse = torch.zeros(B, H, N, dtype=torch.float32)
    return q, k, v, o, do, lse


def check_call(call, params, **want):
    name, args = call
    assert len(args) == len(params[name]), (name, len(args), params[name])
    got = dict(zip(params[name], args))
    for key, value in want.items():
        assert got[key] == value, (name, key, got[key], value)
    return got


def test_forward_ex_tile_options(fake):
    params = declared_params()
    q, k, v, o, do, lse = tensors()
    _binding.fa_forward_ex(q, k, v, block_rows=128, block_keys=32)
    check_call(fake.calls[-1], params, block_rows=128, block_keys=32)
    _binding.fa_forward(q, k, v)
    assert fake.calls[-1][0] == "fa_forward"
    check_call(fake.calls[-1], params)


def test_backward_entry_points_and_tile_options(fake):
    params = declared_params()
    q, k, v, o, do, lse = tensors()
    _binding.fa_backward(q, k, v, o, do, lse)
    assert fake.calls[-1][0] == "fa_backward"
    check_call(fake.calls[-1], params)
    _binding.fa_backward_ex(q, k, v, o, do, lse, dq_rows=64, dkdv_rows=256)
    got = check_call(fake.calls[-1], params, dq_rows=64, dkdv_rows=256, grad_dtype=2)
    assert got["o"] is not None and got["dk"] is not None
    _binding.fa_backward(q, k, v, o, do, lse, grad_dtype=torch.float32)
    assert fake.calls[-1][0] == "fa_backward_ex"
    check_call(fake.calls[-1], params, grad_dtype=0, dq_rows=0, dkdv_rows=0)
    # the separate passes keep their own entry points with a rows argument
    _, ws = _binding.fa_backward_dq(q, k, v, o, do, lse, rows=256)
    got = check_call(fake.calls[-1], params, rows=256)
    assert fake.calls[-1][0] == "fa_backward_dq" and got["o"] is not None
    _binding.fa_backward_dkdv(q, k, v, do, ws, rows=64)
    got = check_call(fake.calls[-1], params, rows=64)
    assert fake.calls[-1][0] == "fa_backward_dkdv" and got["dk"] is not None


def test_noalloc_backward(fake):
    params = declared_params()
    q, k, v, o, do, lse = tensors()
    _binding.fa_backward_noalloc(q, k, v, o, do, lse, causal=True)
    got = check_call(fake.calls[-1], params, causal=1, N=100, d=64)
    assert fake.calls[-1][0] == "fa_backward_noalloc" and got["dv"] is not None


def test_every_declared_compute_call_has_a_binding_of_its_name():
    params = declared_params()
    for name in params:
        if name in ("fa_status_string", "fa_last_error_detail", "fa_stamps_arm",
                    "fa_stamps_read"):
            continue
        assert hasattr(_binding, name), name
