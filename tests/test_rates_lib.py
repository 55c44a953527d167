"""The unit-rate measurement library (libfa_rates.so): on the CPU, that it
loads, exports fa_rates_run and refuses out-of-range arguments before any
device call; on the GPU, that every rate kernel runs and each wave records a
loop that took shader and wall clock time at a plausible clock."""

import ctypes
import os

import pytest
import torch

from exact_io_aware_52_amd import build_lib

OPS = range(9)


@pytest.fixture(scope="module")
def rates():
    if not os.path.exists(build_lib.RATES_LIB):
        pytest.fail(f"{build_lib.RATES_LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(build_lib.RATES_LIB)
    lib.fa_rates_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    return lib


def test_rates_argument_checks(rates):
    buf = ctypes.c_void_p(1)  # never dereferenced: every call below is refused first
    assert rates.fa_rates_run(-1, 1, 1, buf, buf, None) == 1
    assert rates.fa_rates_run(9, 1, 1, buf, buf, None) == 1
    assert rates.fa_rates_run(0, 0, 1, buf, buf, None) == 1
    assert rates.fa_rates_run(0, (1 << 16) + 1, 1, buf, buf, None) == 1
    assert rates.fa_rates_run(0, 1, 0, buf, buf, None) == 1
    assert rates.fa_rates_run(0, 1, 1, None, buf, None) == 1
    assert rates.fa_rates_run(0, 1, 1, buf, None, None) == 1


@pytest.mark.gpu
@pytest.mark.parametrize("op", OPS)
def test_rates_kernels_run(rates, op):
    print(f"[rates] op {op}", flush=True)
    wpg = 8 if op == 6 else 4
    grid = 64
    sink = torch.full((grid * 64 * wpg,), float("nan"), device="cuda")
    clocks = torch.zeros(grid * wpg * 5, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream()
    assert rates.fa_rates_run(op, grid, 500, ctypes.c_void_p(sink.data_ptr()),
                              ctypes.c_void_p(clocks.data_ptr()),
                              ctypes.c_void_p(st.cuda_stream)) == 0
    torch.cuda.synchronize()
    c = clocks.view(-1, 5).cpu()
    cycles, wall_ns = c[:, 1] - c[:, 0], 10 * (c[:, 3] - c[:, 2])
    assert (cycles > 0).all() and (wall_ns > 0).all()
    ghz = (cycles.double() / wall_ns.double()).median().item()
    assert 0.3 < ghz < 3.5, ghz
    # every wave says where it ran: a SIMD id 0-3 and at most 8 XCDs
    hw = c[:, 4]
    assert ((hw >> 32) < 8).all()
    assert (((hw & 0xFFFFFFFF) >> 4) & 3).unique().numel() >= 2
    # every thread wrote its result (values may be +inf: the exponential chains overflow)
    assert not torch.isnan(sink).any()
