"""Block-sparse backward split by kept mask blocks (fa_backward_blocksparse_split)
against the oracle and against the unsplit backward, through the C ABI.

Each mask row (dQ pass) and column (dK/dV pass) is handed out in items of
chunk_blocks kept blocks; rows and columns with more than that many write
float32 partials that a reduction sums.  The split gradients are rounded to
the input type once, from those sums: against the oracle each element may
differ by the tolerance plus that rounding (half a unit in the last place of
the 16-bit result: 2^-9 |x| for bf16, 2^-12 |x| for fp16); against the
unsplit backward, which rounds its own fp32 sums, by two such roundings."""

import numpy as np
import pytest
import torch

from exact_io_aware_52_amd import (fa_backward, fa_backward_blocksparse_split,
                                   fa_backward_blocksparse_split_workspace_bytes,
                                   fa_forward_blocksparse, inputs)
from test_gpu_parity import (TOL, check_all_heads, check_sampled_rows, check_sum_identities,
                             dev, log, nan_like, run_gpu, run_oracle)

pytestmark = pytest.mark.gpu

ULP_HALF = {"bf16": 2.0 ** -9, "fp16": 2.0 ** -12}
GRADS = ("dq", "dk", "dv")


def split_backward(prob, chunk_blocks, o, lse):
    q, k, v, do = (dev(x, prob.dtype) for x in (prob.q, prob.k, prob.v, prob.do))
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).cuda()
    bm = torch.from_numpy(prob.block_mask).cuda()
    o, lse = torch.from_numpy(o).to(q.dtype).cuda(), torch.from_numpy(lse).float().cuda()
    dq, dk, dv = (nan_like(q) for _ in range(3))
    fa_backward_blocksparse_split(q, k, v, o, do, lse, bm, prob.block_size, chunk_blocks,
                                  scale=float(prob.scale), causal=prob.causal, key_lens=kl,
                                  dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.double().cpu().numpy() for n, t in zip(GRADS, (dq, dk, dv))}


def check_rounded(got, ref, dtype, label, factor=1):
    """|got - ref| <= TOL + factor * (half-ulp rounding of the 16-bit output)."""
    for n in GRADS:
        g, r = got[n], ref[n]
        assert np.all(np.isfinite(g)), f"{label} {n}: non-finite or unwritten elements"
        bound = TOL[dtype] + factor * ULP_HALF[dtype] * np.maximum(np.abs(r), np.abs(g))
        excess = np.abs(g - r) - bound
        log(f"[split bwd] {label} {n}: max |diff| {np.abs(g - r).max():.3g}, "
            f"worst margin {excess.max():.3g}")
        assert np.all(excess <= 0), f"{label} {n}: {int((excess > 0).sum())} elements over bound"


CASES = [
    # B, H, N, d, dtype, causal, key_len_range, keep_p, band, global, chunk_blocks
    (1, 2, 2048, 64, "bf16", False, None, 1 / 8, 1, 1, 3),     # band + global row/column
    (1, 2, 1536, 64, "bf16", True, None, 1 / 4, 1, 1, 1),      # causal, one block per item
    (2, 1, 1000, 128, "fp16", True, (500, 1000), 0.5, None, 0, 2),
    (1, 1, 777, 128, "bf16", False, None, 0.6, None, 0, 4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[2]}d{c[3]}_{c[4]}_chunk{c[10]}")
def test_split_backward(case):
    B, H, N, d, dtype, causal, klr, keep, band, glob, chunk = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=901 + N + chunk, causal=causal,
                               key_len_range=klr, block_keep_p=keep, block_band=band,
                               block_global=glob)
    kept = prob.block_mask.sum(axis=1)
    assert kept.max() > chunk, "the case must split some rows"
    gpu = run_gpu(prob)  # forward + unsplit backward (float32 gradients under dq, dk, dv)
    split = split_backward(prob, chunk, gpu["o"], gpu["lse"])
    label = f"split chunk={chunk} {case}"
    ref = run_oracle(prob)
    check_rounded(split, ref, dtype, label + " vs oracle")
    unsplit16 = {n: gpu[n + "_16"] for n in GRADS}
    check_rounded(split, unsplit16, dtype, label + " vs unsplit", factor=2)


def test_split_backward_one_item_is_the_unsplit_backward():
    # chunk_blocks at least the blocks per row: every row and column is one
    # item, no partials, and the gradients are the unsplit backward's (with
    # one key group, as the split instances run), bit for bit.  The
    # workspace is then only the unsplit one plus three one-item partial
    # arrays.
    prob = inputs.make_problem(1, 2, 900, 64, "bf16", seed=933, causal=True, block_keep_p=0.5,
                               block_band=1, block_global=1)
    gpu = run_gpu(prob, bwd_key_groups=1)
    split = split_backward(prob, 8, gpu["o"], gpu["lse"])
    for n in GRADS:
        assert np.array_equal(split[n], gpu[n + "_16"]), n
    nb = (900 + 127) // 128
    assert fa_backward_blocksparse_split_workspace_bytes(1, 2, 900, 64, nb) > 0


def test_split_backward_deterministic():
    prob = inputs.make_problem(1, 2, 1024, 64, "bf16", seed=944, block_keep_p=1 / 4,
                               block_band=1, block_global=1)
    gpu = run_gpu(prob, backward=False)
    a = split_backward(prob, 2, gpu["o"], gpu["lse"])
    b = split_backward(prob, 2, gpu["o"], gpu["lse"])
    for n in GRADS:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("n", [32768, 65536])
def test_config_block_sparse_long_split_backward(n):
    # The long structured masks through the split backward: dQ on sampled
    # rows of every head against the oracle's row function, the dK/dV sum
    # identities on every head, and every head against the unsplit backward.
    prob = inputs.workload("block_sparse_long", n)
    gpu = run_gpu(prob)
    split = split_backward(prob, 64, gpu["o"], gpu["lse"])
    label = f"block_sparse_long N={n} split backward"
    got = dict(gpu, **split)
    check_all_heads(prob, {k: got[k] for k in ("o", "lse") + GRADS}, label)
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, n // 2, n - 129, n - 1],
                                     rng.integers(0, n, 9)]))
    check_sampled_rows(prob, {k: got[k] for k in ("o", "lse", "dq")}, rows, label,
                       heads=[(0, 0), (0, 7)])
    check_sum_identities(prob, got, label)
    check_rounded(split, {k: gpu[k + "_16"] for k in GRADS}, "bf16", label + " vs unsplit",
                  factor=2)
