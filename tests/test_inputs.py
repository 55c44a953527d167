"""CPU tests of the seeded input generator and of the host flop accounting."""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_52_amd import accounting, inputs


def test_generator_is_deterministic_and_rounded():
    a = inputs.make_problem(2, 3, 40, 16, "bf16", seed=11, causal=True)
    b = inputs.make_problem(2, 3, 40, 16, "bf16", seed=11, causal=True)
    for x, y in zip((a.q, a.k, a.v, a.do), (b.q, b.k, b.v, b.do)):
        assert np.array_equal(x, y)
    # values are exactly representable: torch's own RNE cast leaves them unchanged
    t = torch.from_numpy(a.q)
    assert torch.equal(t.to(torch.bfloat16).float(), t)
    c = inputs.make_problem(1, 1, 64, 8, "fp16", seed=3)
    t = torch.from_numpy(c.k)
    assert torch.equal(t.half().float(), t)


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_round_to_dtype_matches_torch_rne(dtype, tdt):
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    # include exact ties: values halfway between two representable numbers
    x[:4] = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 2.0 + 2 ** -7],
                     np.float32)
    ours = inputs.round_to_dtype(x, dtype)
    ref = torch.from_numpy(x).to(tdt).float().numpy()
    assert np.array_equal(ours, ref)


def test_workloads_shapes():
    p = inputs.make_problem(**inputs.config("bert_large_padded"))
    assert p.q.shape == (16, 16, 512, 64) and p.dtype == "fp16"
    assert p.key_lens.min() >= 128 and p.key_lens.max() <= 512
    cfg = inputs.config("block_sparse")
    assert cfg["N"] == 16384 and cfg["block_keep_p"] == 1 / 8
    assert inputs.config("long_causal", 4096, 128)["seed"] == 4 + 10 * 3


def test_block_mask_recipe():
    p = inputs.make_problem(1, 1, 2048, 8, "bf16", seed=5, block_keep_p=1 / 8)
    bm = p.block_mask
    assert bm.shape == (16, 16) and np.all(np.diag(bm) == 1)
    big = inputs.make_problem(1, 1, 128 * 128, 1, "bf16", seed=5, block_keep_p=1 / 8)
    density = big.block_mask.mean()
    assert 0.11 < density < 0.16          # expected (128 + 127*16) / 128^2 = 13.2 %


def test_structured_block_mask_recipe():
    # band of one block each side, first block row and column, i.i.d. 1/32
    p = inputs.make_problem(1, 1, 128 * 64, 1, "bf16", seed=6, block_keep_p=1 / 32,
                            block_band=1, block_global=1)
    bm = p.block_mask.astype(bool)
    ib, jb = np.indices(bm.shape)
    assert bm[np.abs(ib - jb) <= 1].all() and bm[0].all() and bm[:, 0].all()
    rest = ~((np.abs(ib - jb) <= 1) | (ib == 0) | (jb == 0))
    assert 0.015 < bm[rest].mean() < 0.05            # i.i.d. part at p = 1/32
    cfg = inputs.config("block_sparse_long", 65536)
    assert cfg["N"] == 65536 and cfg["block_band"] == 1 and cfg["block_global"] == 1


@pytest.mark.parametrize("kw", [
    dict(causal=False), dict(causal=True), dict(key_len=37), dict(causal=True, key_len=50),
    dict(block="rand"), dict(causal=True, block="rand", key_len=70),
])
def test_kept_pairs_matches_visibility(kw):
    n, bs = 83, 16
    bm = None
    if kw.pop("block", None):
        nb = -(-n // bs)
        bm = (np.random.default_rng(1).random((nb, nb)) < 0.5).astype(np.uint8)
    want = int(oracle.visibility(n, block_mask=bm, block_size=bs, **kw).sum())
    got = accounting.kept_pairs_head(n, block_mask=bm, block_size=bs, **kw)
    assert got == want


def test_flops_gpt2_small():
    p = inputs.make_problem(8, 12, 1024, 64, "bf16", seed=2, causal=True)
    pairs = 96 * 1024 * 1025 // 2
    assert accounting.kept_pairs(p) == pairs
    assert accounting.flops(p, "fwd+bwd") == 14 * 64 * pairs


@pytest.mark.parametrize("kw", [
    dict(causal=False), dict(causal=True), dict(causal=True, key_len_range=(1, 700)),
    dict(block_keep_p=0.5), dict(causal=True, block_keep_p=0.4, key_len_range=(300, 700)),
    dict(block_keep_p=0.3, block_band=1, block_global=1),
])
@pytest.mark.parametrize("rows", [64, 128, 256])
def test_streamed_rows_match_visibility(kw, rows):
    # The backward IO model's count of streamed rows against brute force over
    # the visibility matrix: per work-group of `rows` rows, the keys some of
    # its queries keep (dQ pass) or the queries that keep some of its keys
    # (dK/dV pass).
    p = inputs.make_problem(2, 3, 700, 64, "bf16", seed=5, **kw)
    want = {"dq": 0, "dkdv": 0}
    for b in range(p.B):
        kl = None if p.key_lens is None else int(p.key_lens[b])
        vis = oracle.visibility(p.N, causal=p.causal, key_len=kl, block_mask=p.block_mask,
                                block_size=p.block_size)
        for r0 in range(0, p.N, rows):
            want["dq"] += int(vis[r0:r0 + rows].any(axis=0).sum())
            want["dkdv"] += int(vis[:, r0:r0 + rows].any(axis=1).sum())
    for which in ("dq", "dkdv"):
        assert accounting.streamed_rows(p, which, rows) == p.H * want[which], which
    # whole passes: own rows plus the streamed ones
    s, n, d, heads = 2, p.N, p.d, p.B * p.H
    assert accounting.tiled_backward_pass_bytes(p, "dq", rows) == \
        heads * (4 * n * d * s + 12 * n) + p.H * want["dq"] * 2 * d * s
    assert accounting.tiled_backward_pass_bytes(p, "dkdv", rows) == \
        heads * 4 * n * d * s + p.H * want["dkdv"] * (2 * d * s + 8)
