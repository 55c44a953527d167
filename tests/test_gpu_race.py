"""Race check: the library built with every LDS ring stage fenced on both
sides (FA_SERIALIZE_STAGES: each tile copy completed and the work-group
synchronised right after it is issued and again after each step) computes
the same arithmetic in the same order as the normal build, with no way for a
tile to be read before it lands or overwritten while still read.  Its
outputs must equal the normal build's bit for bit; a missing wait or barrier
in the normal build's ring would show up as a difference.  Both libraries
are called through the C ABI on the same device buffers."""

import ctypes

import pytest
import torch

from exact_io_aware_52_amd import _binding, build_lib, inputs
from test_gpu_parity import dev, log

pytestmark = pytest.mark.gpu

CODE = {"fp32": 0, "fp16": 1, "bf16": 2}


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_lib(lib, prob, block_rows=0, block_keys=0, bwd_rows=0, key_groups=0):
    q, k, v, do = (dev(x, prob.dtype) for x in (prob.q, prob.k, prob.v, prob.do))
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).cuda()
    bm = None if prob.block_mask is None else torch.from_numpy(prob.block_mask).cuda()
    o, dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(4))
    lse = torch.full((prob.B, prob.H, prob.N), float("nan"), dtype=torch.float32, device="cuda")
    need = lib.fa_backward_workspace_bytes(prob.B, prob.H, prob.N, prob.d)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = (prob.B, prob.H, prob.N, prob.d, float(prob.scale), int(prob.causal), ptr(kl))
    st = lib.fa_forward_ex(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), *common, ptr(bm),
                           prob.block_size, block_rows, block_keys, key_groups, CODE[prob.dtype],
                           stream)
    assert st == 0, lib.fa_last_error_detail()
    st = lib.fa_backward_ex(ptr(q), ptr(k), ptr(v), ptr(o), ptr(do), ptr(lse), ptr(dq), ptr(dk),
                            ptr(dv), *common, ptr(bm), prob.block_size, CODE[prob.dtype],
                            CODE[prob.dtype], bwd_rows, bwd_rows, 0, ptr(ws), need, stream)
    assert st == 0, lib.fa_last_error_detail()
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}


CASES = [
    # workload or make_problem arguments, forward query rows and keys per tile, backward
    # rows per work-group of both passes
    ("gpt2_small", None, 0, 0, 0),
    ("block_sparse", None, 0, 0, 0),
    ("small", dict(B=2, H=4, N=600, d=128, dtype="bf16", seed=31, causal=True), 256, 0, 256),
    ("small", dict(B=2, H=3, N=300, d=64, dtype="fp16", seed=32, key_len_range=(1, 300)), 64, 0,
     64),
    ("small", dict(B=1, H=2, N=333, d=128, dtype="fp32", seed=33, block_keep_p=0.5), 0, 0, 0),
    ("small", dict(B=1, H=2, N=257, d=64, dtype="fp32", seed=34, causal=True), 0, 0, 0),
    ("small", dict(B=2, H=4, N=1000, d=64, dtype="bf16", seed=35, causal=True), 128, 32, 256),
    ("small", dict(B=1, H=4, N=1100, d=128, dtype="fp16", seed=36, block_keep_p=0.5), 128, 128,
     64),
    # two key groups (chosen automatically for grids this small), d = 128, ragged
    ("small", dict(B=2, H=2, N=1500, d=128, dtype="bf16", seed=37, causal=True,
                   key_len_range=(700, 1500)), 0, 0, 0),
    # d = 128 with a block mask: the dK/dV pass's split query tiles (two-slot ring, K and V in
    # LDS) over skipped tiles
    ("small", dict(B=1, H=3, N=777, d=128, dtype="bf16", seed=38, block_keep_p=0.5), 0, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0] if c[1] is None else
                         "N{N}d{d}_{dtype}_keys{k}_bwd{b}".format(k=c[3], b=c[4], **c[1]))
def test_serialized_stages_bitwise(case):
    name, kw, rows, keys, brows = case
    prob = inputs.workload(name) if kw is None else inputs.make_problem(**kw)
    log(f"[race] {name} {kw} rows={rows} keys={keys} bwd rows={brows}")
    main = run_lib(_binding.load_library(), prob, rows, keys, brows)
    serial = run_lib(_binding.open_library(build_lib.SERIAL_LIB), prob, rows, keys, brows)
    for n in main:
        a, b = main[n], serial[n]
        assert not torch.isnan(a).any(), n
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (
            f"{name} {n}: {int((a != b).sum())} elements differ between the builds")
    log(f"[race] {name}: all outputs bitwise equal")


def run_split(lib, prob, chunk_blocks):
    q, k, v, do = (dev(x, prob.dtype) for x in (prob.q, prob.k, prob.v, prob.do))
    bm = torch.from_numpy(prob.block_mask).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((prob.B, prob.H, prob.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    need = lib.fa_backward_blocksparse_split_workspace_bytes(prob.B, prob.H, prob.N, prob.d,
                                                             chunk_blocks)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = (prob.B, prob.H, prob.N, prob.d, float(prob.scale), int(prob.causal), None)
    st = lib.fa_forward_ex(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), *common, ptr(bm),
                           prob.block_size, 0, 0, 0, CODE[prob.dtype], stream)
    assert st == 0, lib.fa_last_error_detail()
    st = lib.fa_backward_blocksparse_split(ptr(q), ptr(k), ptr(v), ptr(o), ptr(do), ptr(lse),
                                           ptr(dq), ptr(dk), ptr(dv), *common, ptr(bm),
                                           prob.block_size, chunk_blocks, CODE[prob.dtype],
                                           ptr(ws), need, stream)
    assert st == 0, lib.fa_last_error_detail()
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}


@pytest.mark.parametrize("causal", [False, True])
def test_serialized_stages_split_backward(causal):
    # The split backward's passes (three tiles ahead in the ring), its
    # preparation and reduction kernels, fenced and unfenced: bit for bit.
    prob = inputs.make_problem(1, 2, 4096, 64, "bf16", seed=41 + causal, causal=causal,
                               block_keep_p=1 / 8, block_band=1, block_global=1)
    log(f"[race] split backward causal={causal}")
    main = run_split(_binding.load_library(), prob, 3)
    serial = run_split(_binding.open_library(build_lib.SERIAL_LIB), prob, 3)
    for n in main:
        a, b = main[n], serial[n]
        assert not torch.isnan(a).any(), n
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (
            f"split {n}: {int((a != b).sum())} elements differ between the builds")
