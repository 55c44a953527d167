"""The allocation-free backward (fa_backward_noalloc) against fa_backward with
a caller-owned workspace, through the C ABI, on two calls in a row, the
second with a smaller problem (the device scratch keeps the first call's
contents), and against the fp64 oracle.  Named to be collected last."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_52_amd import _binding, inputs
from test_gpu_parity import dev, log

pytestmark = pytest.mark.gpu

CODE = {"fp32": 0, "fp16": 1, "bf16": 2}


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def both_backwards(lib, prob):
    q, k, v, do = (dev(x, prob.dtype) for x in (prob.q, prob.k, prob.v, prob.do))
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).cuda()
    bm = None if prob.block_mask is None else torch.from_numpy(prob.block_mask).cuda()
    o = torch.empty_like(q)
    lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = (prob.B, prob.H, prob.N, prob.d, float(prob.scale), int(prob.causal), ptr(kl))
    assert lib.fa_forward_ex(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), *common, ptr(bm),
                             prob.block_size, 0, 0, 0, CODE[prob.dtype], stream) == 0
    ref = [torch.full_like(q, float("nan")) for _ in range(3)]
    need = lib.fa_backward_workspace_bytes(prob.B, prob.H, prob.N, prob.d)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert lib.fa_backward(ptr(q), ptr(k), ptr(v), ptr(o), ptr(do), ptr(lse),
                           *(ptr(t) for t in ref), *common, ptr(bm), prob.block_size,
                           CODE[prob.dtype], ptr(ws), need, stream) == 0
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    st = lib.fa_backward_noalloc(ptr(q), ptr(k), ptr(v), ptr(o), ptr(do), ptr(lse),
                                 *(ptr(t) for t in got), *common, ptr(bm), prob.block_size,
                                 CODE[prob.dtype], stream)
    assert st == 0, lib.fa_last_error_detail()
    torch.cuda.synchronize()
    return [t.cpu() for t in ref], [t.cpu() for t in got]


def test_noalloc_backward_two_calls():
    lib = _binding.load_library()
    probs = [inputs.make_problem(2, 4, 1000, 64, "bf16", seed=601, causal=True),
             inputs.make_problem(1, 3, 300, 128, "fp16", seed=602, key_len_range=(50, 300),
                                 block_keep_p=0.5)]
    for prob in probs:
        log(f"[no-alloc] B{prob.B} H{prob.H} N{prob.N} d{prob.d} {prob.dtype}")
        ref, got = both_backwards(lib, prob)
        for n, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert not torch.isnan(b).any(), n
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), n
        args = [x.astype(np.float64) for x in (prob.q, prob.k, prob.v)]
        want = oracle.backward(*args, prob.do.astype(np.float64), float(prob.scale),
                               causal=prob.causal, key_lens=prob.key_lens,
                               block_mask=prob.block_mask, block_size=prob.block_size)
        for n, g, r in zip(("dq", "dk", "dv"), got, want):
            err = float(np.abs(g.double().numpy() - r).max())
            log(f"[no-alloc] {n} max-abs error vs oracle {err:.3g}")
            assert err <= 2e-2, n


def test_noalloc_backward_rejects_too_large():
    lib = _binding.load_library()
    rows = lib.fa_backward_noalloc_max_rows()
    assert rows == (16 << 20) // 8
    # B*H*N one tile's worth above the limit: refused on the host, nothing launched
    fake = ctypes.c_void_p(0x10000)
    st = lib.fa_backward_noalloc(*([fake] * 9), 1, 1, rows + 256, 64, 0.125, 0, None, None, 128,
                                 2, None)
    assert st == _binding.FA_ERR_UNSUPPORTED
    assert b"scratch" in lib.fa_last_error_detail()
