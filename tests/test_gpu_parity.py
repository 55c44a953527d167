"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded, dtype-rounded inputs.

Bar: max-abs error <= 1e-5 for fp32 inputs and <= 2e-2 for bf16/fp16 inputs,
on O, LSE, dQ, dK and dV (unit-variance data).  For 16-bit inputs the
gradients are compared in float32 (fa_backward_ex), and the 16-bit gradients
the usual call returns must be exactly their round-to-nearest-even: the bar
then measures the computation, not the output format, whose own rounding
already reaches 2^-6 for values of magnitude 4 to 8, as dV of the first keys
under a causal mask does.  Small cases span several
tiles with ragged tails and are compared element by element in full; the
five workloads run at full size in the launch configuration the bench times.
Up to N = 4096 every head is compared in full; beyond, every head is
compared on sampled query rows (the first and last row of every tile among
them) and through the two sum identities of the gradient, and one whole head
in full.  Every output buffer starts as NaN, so an element no work-group
writes cannot pass: all heads are checked for NaN and for the -inf pattern
of LSE (rows without a visible key) before any sampled comparison.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_52_amd import (fa_backward, fa_forward, fa_forward_blocksparse,
                                   fa_forward_blocksparse_split, fa_forward_ex, inputs,
                                   fa_backward_ex, fa_backward_dq, fa_backward_dkdv)

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "fp16": 2e-2, "bf16": 2e-2}
TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
NAMES = ("o", "lse", "dq", "dk", "dv")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[dtype]).cuda()


def nan_like(t):
    return torch.full_like(t, float("nan"))


def run_gpu(prob, backward=True, block_rows=None, block_keys=0, key_groups=0, bwd_key_groups=0):
    """Forward (and backward) through the C ABI into NaN-filled outputs
    (key groups 0: the library's choice)."""
    q, k, v, do = (dev(x, prob.dtype) for x in (prob.q, prob.k, prob.v, prob.do))
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).cuda()
    bm = None if prob.block_mask is None else torch.from_numpy(prob.block_mask).cuda()
    kw = dict(scale=float(prob.scale), causal=prob.causal, key_lens=kl)
    o = nan_like(q)
    lse = torch.full((prob.B, prob.H, prob.N), float("nan"), dtype=torch.float32, device="cuda")
    if block_rows is not None or block_keys or key_groups:
        fa_forward_ex(q, k, v, bm, prob.block_size, block_rows=block_rows or 0,
                      block_keys=block_keys, key_groups=key_groups, o=o, lse=lse, **kw)
    elif bm is not None:
        fa_forward_blocksparse(q, k, v, bm, prob.block_size, o=o, lse=lse, **kw)
    else:
        fa_forward(q, k, v, o=o, lse=lse, **kw)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = (nan_like(q) for _ in range(3))
        fa_backward_ex(q, k, v, o, do, lse, block_mask=bm, block_size=prob.block_size, dq=dq,
                       dk=dk, dv=dv, key_groups=bwd_key_groups, **kw)
        out.update(dq=dq, dk=dk, dv=dv)
        if prob.dtype != "fp32":
            # The same backward with float32 gradients: the 16-bit gradients
            # above must be exactly their round-to-nearest-even, and the
            # float32 ones are what the oracle comparison measures (the
            # computation's error apart from the output's own rounding).
            g32 = fa_backward_ex(q, k, v, o, do, lse, block_mask=bm, block_size=prob.block_size,
                                 grad_dtype=torch.float32, key_groups=bwd_key_groups, **kw)
            torch.cuda.synchronize()
            for n, g in zip(("dq", "dk", "dv"), g32):
                g = g.cpu().numpy()
                assert not np.isnan(g).any(), f"float32 {n}: elements never written"
                want = inputs.round_to_dtype(g, prob.dtype)
                got = out[n].float().cpu().numpy()
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (
                    f"{n}: 16-bit gradients are not the rounding of the float32 ones "
                    f"({int((got != want).sum())} elements)")
                out[n + "_16"] = out[n]
                out[n] = torch.from_numpy(g)
    torch.cuda.synchronize()
    return {n: t.double().cpu().numpy() for n, t in out.items()}


def rows_without_keys(prob, b, chunk=2048):
    """Boolean [N]: query rows of batch b that see no key (from the oracle's
    visibility rule, a chunk of rows at a time)."""
    kl = None if prob.key_lens is None else int(prob.key_lens[b])
    out = np.zeros(prob.N, dtype=bool)
    for r0 in range(0, prob.N, chunk):
        rows = np.arange(r0, min(prob.N, r0 + chunk))
        vis = oracle.visibility(prob.N, prob.causal, kl, prob.block_mask, prob.block_size,
                                rows=rows)
        out[rows] = ~vis.any(axis=1)
    return out


def check_all_heads(prob, gpu, label=""):
    """Every head: no NaN left in any output (each element was written), LSE
    is -inf exactly on the rows without a visible key, everything else finite."""
    for n, g in gpu.items():
        assert not np.isnan(g).any(), f"{label} {n}: {int(np.isnan(g).sum())} elements never written"
    lse = gpu["lse"]
    for b in range(prob.B):
        empty = rows_without_keys(prob, b)
        ninf = np.isneginf(lse[b])
        assert np.array_equal(ninf, np.broadcast_to(empty, ninf.shape)), f"{label} b={b}: -inf rows"
        assert np.all(np.isfinite(lse[b][:, ~empty])), f"{label} b={b}: LSE not finite"
    for n in gpu:
        if n != "lse":
            assert np.all(np.isfinite(gpu[n])), f"{label} {n}: non-finite values"


def run_oracle(prob, heads=None, row_chunk=None, backward=True):
    args = [x.astype(np.float64) for x in (prob.q, prob.k, prob.v)]
    kw = dict(causal=prob.causal, key_lens=prob.key_lens, block_mask=prob.block_mask,
              block_size=prob.block_size, row_chunk=row_chunk, heads=heads)
    o, lse = oracle.forward(*args, float(prob.scale), **kw)
    ref = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = oracle.backward(*args, prob.do.astype(np.float64), float(prob.scale), **kw)
        ref.update(dq=dq, dk=dk, dv=dv)
    return ref


def compare(gpu, ref, tol, heads=None, label="", magnitude_scaled=False):
    """Max-abs comparison against ``tol``.

    The stated tolerances hold for unit-variance data.  With
    ``magnitude_scaled`` (edge cases whose outputs leave that regime) the
    bound of each tensor is tol * max(1, max |reference|), i.e. the same
    accuracy relative to the tensor's scale; LSE keeps the plain bound."""
    errs, bounds = {}, {}
    for n in ref:
        if n not in gpu:
            continue
        g, r = gpu[n], ref[n]
        if heads is not None:
            # unsampled heads: at least every element written and finite
            assert not np.isnan(g).any(), f"{label} {n}: elements never written"
            g = np.stack([g[b, h] for b, h in heads])
            r = np.stack([r[b, h] for b, h in heads])
        # rows without a visible key: LSE must be -inf on both sides
        ninf = np.isneginf(r)
        assert np.array_equal(np.isneginf(g), ninf), f"{label} {n}: -inf pattern differs"
        assert np.all(np.isfinite(g[~ninf])), f"{label} {n}: non-finite values"
        diff = np.abs(g[~ninf] - r[~ninf])
        errs[n] = float(diff.max()) if diff.size else 0.0
        bounds[n] = tol
        if magnitude_scaled and n != "lse" and diff.size:
            bounds[n] = tol * max(1.0, float(np.abs(r[~ninf]).max()))
    log(f"[parity] {label} tol={tol:g}{' (x max|ref|)' if magnitude_scaled else ''} "
        + " ".join(f"{n}={errs[n]:.3g}/{bounds[n]:.3g}" for n in errs))
    bad = {n: e for n, e in errs.items() if e > bounds[n]}
    assert not bad, f"{label}: max-abs errors over bound: {bad}"
    return errs


# ----------------------------------------------------------------------------- small, full compare

SMALL = [
    # B, H, N, d, dtype, causal, key_len_range, block_keep_p
    (1, 2, 300, 64, "bf16", False, None, None),
    (1, 2, 300, 64, "bf16", True, None, None),
    (2, 2, 257, 128, "bf16", True, None, None),
    (2, 3, 300, 64, "fp16", False, (1, 300), None),
    (2, 1, 300, 128, "fp16", True, (50, 280), None),
    (1, 2, 384, 64, "bf16", False, None, 0.5),
    (1, 2, 384, 128, "fp16", True, None, 0.5),
    (2, 2, 200, 64, "fp32", False, None, None),
    (1, 2, 200, 64, "fp32", True, (30, 190), None),
    (1, 2, 130, 128, "fp32", True, None, None),
    (1, 1, 300, 128, "fp32", False, None, 0.5),
    (1, 1, 17, 64, "bf16", True, None, None),
    (1, 1, 17, 128, "fp32", False, None, None),
    (1, 3, 1, 64, "bf16", False, None, None),
    (1, 1, 1, 128, "fp16", True, None, None),
    # Very short key lengths: each row attends to 1-3 keys, so dV and dK sum
    # O(N) rows of one key and leave the unit-variance regime (compared with
    # the tolerance scaled by the output magnitude).  The bf16 form of this
    # case has its own test below (test_short_keys_bf16).
    (3, 2, 130, 64, "fp16", False, (1, 3), None),
    (3, 2, 130, 128, "fp32", True, (1, 3), None),
    # B * H a multiple of 8: the tile schedule's XCD-aware branch (every tile
    # of a head on one XCD), with several tiles per head and ragged tails,
    # compared in full.
    (2, 4, 600, 64, "bf16", True, None, None),
    (2, 8, 333, 128, "fp16", False, (100, 333), None),
    (1, 16, 520, 64, "bf16", False, None, 0.5),
    (4, 2, 257, 64, "fp32", True, None, None),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}H{}N{}d{}_{}_{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full",
    "_pad" if c[6] else "", "_sparse" if c[7] else ""))
def test_small_cases(case):
    B, H, N, d, dtype, causal, klr, p = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=1000 + N + d, causal=causal,
                               key_len_range=klr, block_keep_p=p)
    log(f"[case] {case}")
    # Key lengths of 1-3 concentrate each head's attention on a few keys, so
    # dV sums O(N) unit rows and leaves the unit-variance regime.
    short = klr is not None and klr[1] <= 8
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, str(case))
    compare(gpu, run_oracle(prob), TOL[dtype], label=str(case), magnitude_scaled=short)


GROUPED = [
    # B, H, N, d, dtype, causal, key_len_range: B * H = 24, three heads per
    # XCD whose streamed K/V (or Q/dO) exceed the XCD's 4 MB of L2, so the
    # schedule takes them two at a time (groups of 2 and 1) in every kernel.
    (3, 8, 2800, 128, "bf16", True, None),
    (4, 6, 2900, 128, "fp16", False, (1000, 2900)),
]


@pytest.mark.parametrize("case", GROUPED, ids=lambda c: "B{}H{}N{}d{}_{}".format(*c[:5]))
def test_grouped_head_schedule(case):
    B, H, N, d, dtype, causal, klr = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=2000 + N, causal=causal,
                               key_len_range=klr)
    log(f"[case] grouped heads {case}")
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, f"grouped {case}")
    compare(gpu, run_oracle(prob, row_chunk=1024), TOL[dtype], label=f"grouped {case}")


def test_short_keys_bf16():
    # bf16 with key lengths 1-3.  Beyond the compute error covered by the
    # magnitude-scaled tolerance, dQ and dK carry the error of
    # D = rowsum(dO * O) formed from the O the forward stored in bf16.  To
    # first order (u = 2^-8, the bf16 unit roundoff): the stored O differs
    # from the exact one by at most u (sum_j P_ij |v_jk| + 2 |O_ik|) (P and
    # O each rounded once, plus the normalisation), so
    # |dD_i| <= u sum_k |dO_ik| (sum_j P_ij |v_jk| + 2 |O_ik|), which reaches
    # dQ_i = scale sum_j dS_ij k_j and dK_j = scale sum_i dS_ij q_i through
    # dS_ij = P_ij (dP_ij - D_i) as
    #   |d dQ_i| <= scale |dD_i| sum_j P_ij |k_j|,
    #   |d dK_j| <= scale sum_i P_ij |dD_i| |q_i|.
    # The test allows that propagated bound, element by element, on top of
    # the scaled tolerance (all terms from the oracle's P and O and the inputs).
    prob = inputs.make_problem(3, 2, 130, 64, "bf16", seed=1194, key_len_range=(1, 3))
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, "short keys bf16")
    ref = run_oracle(prob)
    tol, u, sc = TOL["bf16"], 2.0 ** -8, float(prob.scale)
    for b in range(prob.B):
        for h in range(prob.H):
            q, k, v, do = (x[b, h].astype(np.float64) for x in (prob.q, prob.k, prob.v, prob.do))
            P = oracle.head_probabilities(q, k, sc, key_len=int(prob.key_lens[b]))
            dD = u * (np.abs(do) * (P @ np.abs(v) + 2 * np.abs(ref["o"][b, h]))).sum(axis=1)
            extra = {"dq": sc * dD[:, None] * (P @ np.abs(k)),
                     "dk": sc * (P.T @ (dD[:, None] * np.abs(q))),
                     "dv": 0.0, "o": 0.0}
            for n, e in extra.items():
                g, r = gpu[n][b, h], ref[n][b, h]
                bound = tol * max(1.0, float(np.abs(ref[n]).max())) + e
                over = np.abs(g - r) - bound
                log(f"[parity] short keys bf16 ({b},{h}) {n}: max err "
                    f"{np.abs(g - r).max():.3g}, worst margin {over.max():.3g}")
                assert np.all(over <= 0), (b, h, n, float(over.max()))
            assert np.abs(gpu["lse"][b, h] - ref["lse"][b, h]).max() <= tol


@pytest.mark.parametrize("dtype,lens", [("bf16", [0, 200, 150]), ("fp32", [0, 200, 5])])
def test_zero_key_length_rows(dtype, lens):
    """A batch with key length 0 has no visible key: O = 0, LSE = -inf, zero grads."""
    prob = inputs.make_problem(3, 2, 200, 64, dtype, seed=77)
    prob.key_lens = np.array(lens, np.int32)
    gpu = run_gpu(prob)
    assert np.all(gpu["o"][0] == 0) and np.all(np.isneginf(gpu["lse"][0]))
    for n in ("dq", "dk", "dv"):
        assert np.all(gpu[n][0] == 0)
    compare(gpu, run_oracle(prob), TOL[dtype], label=f"key_len 0 {dtype}")


def test_block_mask_with_empty_rows():
    prob = inputs.make_problem(1, 2, 384, 64, "fp16", seed=78, block_keep_p=0.5)
    prob.block_mask = np.array([[0, 0, 0], [1, 0, 1], [0, 0, 1]], np.uint8)
    gpu = run_gpu(prob)
    assert np.all(gpu["o"][:, :, :128] == 0) and np.all(np.isneginf(gpu["lse"][:, :, :128]))
    compare(gpu, run_oracle(prob), TOL["fp16"], label="empty mask rows")


@pytest.mark.parametrize("dtype,d,causal", [("fp16", 64, True), ("fp16", 128, False),
                                             ("bf16", 64, False), ("bf16", 128, True)])
def test_large_scale(dtype, d, causal):
    # scale = 1: Q stays unscaled in every dtype and each fp32 score is
    # multiplied by scale * log2(e) before the exponential.  Scores have
    # standard deviation sqrt(d), so rows are close to one-hot.
    prob = inputs.make_problem(1, 2, 300, d, dtype, seed=83 + d, causal=causal, scale=1.0)
    compare(run_gpu(prob), run_oracle(prob), TOL[dtype], label=f"scale 1 {dtype} d{d}",
            magnitude_scaled=True)


ROW_CASES = [
    # rows, B, H, N, d, dtype, causal, key_len_range, block_keep_p
    (64, 1, 2, 300, 64, "bf16", True, None, None),
    (64, 2, 1, 257, 128, "fp16", False, (1, 257), None),
    (64, 1, 2, 384, 64, "bf16", False, None, 0.5),
    (64, 1, 1, 200, 64, "fp32", True, None, None),
    (256, 1, 2, 600, 64, "bf16", True, None, None),
    (256, 2, 1, 520, 128, "bf16", False, (100, 520), None),
    (256, 1, 1, 300, 64, "fp32", True, None, None),
    # 256-row d = 128 tiles stage V transposed once per work-group
    (256, 1, 2, 1100, 128, "bf16", True, None, None),
    (256, 2, 2, 777, 128, "fp16", True, (300, 777), None),
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "rows{}_N{}d{}_{}".format(c[0], c[3], c[4], c[5]))
def test_forward_block_rows(case):
    # query tiles of 64 and 256 rows (the tile-height setting) give the same
    # results as the oracle
    rows, B, H, N, d, dtype, causal, klr, bkp = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=97 + rows + N, causal=causal,
                               key_len_range=klr, block_keep_p=bkp)
    gpu = run_gpu(prob, block_rows=rows)
    check_all_heads(prob, gpu, f"{rows} rows")
    compare(gpu, run_oracle(prob), TOL[dtype], label=f"{rows} rows {case[1:]}",
            magnitude_scaled=klr is not None and klr[0] < 4)


KEY_CASES = [
    # keys per K/V tile, B, H, N, d, dtype, causal, key_len_range, block_keep_p
    (32, 1, 2, 1000, 64, "bf16", True, None, None),
    (32, 2, 1, 777, 128, "fp16", False, (1, 777), None),
    (32, 1, 2, 1024, 64, "fp16", False, None, 0.5),
    (32, 1, 1, 640, 128, "bf16", True, None, None),
    (128, 1, 2, 1000, 64, "bf16", True, None, None),
    (128, 2, 1, 777, 128, "fp16", False, (1, 777), None),
    (128, 1, 2, 1100, 64, "bf16", False, None, 0.5),
    (128, 1, 1, 640, 128, "bf16", True, None, None),
    (128, 1, 2, 300, 64, "bf16", False, (100, 300), None),
]


@pytest.mark.parametrize("case", KEY_CASES, ids=lambda c: "keys{}_N{}d{}_{}".format(c[0], c[3], c[4], c[5]))
def test_forward_block_keys(case):
    # K/V tiles of 32 and 128 keys (the key-tile width option; 128-row query
    # tiles) against the oracle on every head: causal diagonals inside and
    # across tiles, ragged last tiles, key lengths down to 1, block masks
    keys, B, H, N, d, dtype, causal, klr, bkp = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=131 + keys + N, causal=causal,
                               key_len_range=klr, block_keep_p=bkp)
    gpu = run_gpu(prob, backward=False, block_keys=keys)
    check_all_heads(prob, gpu, f"{keys} keys")
    compare(gpu, run_oracle(prob, backward=False), TOL[dtype], label=f"{keys} keys {case[1:]}",
            magnitude_scaled=klr is not None and klr[0] < 4)


@pytest.mark.parametrize("boost", [1.5, 6.0])
@pytest.mark.parametrize("keys", [32, 128])
def test_forward_block_keys_far_keys(keys, boost):
    # The unchecked sweep and its fall-back with 32- and 128-key tiles (the
    # fixed reference still comes from each row's first 32 keys).
    prob = inputs.make_problem(1, 2, 700, 64, "bf16", seed=653 + keys, causal=True, scale=1.0)
    prob.k[:, :, 300:304] *= boost
    prob.k = inputs.round_to_dtype(prob.k, "bf16")
    gpu = run_gpu(prob, backward=False, block_keys=keys)
    label = f"far keys x{boost} {keys} keys"
    check_all_heads(prob, gpu, label)
    compare(gpu, run_oracle(prob, backward=False), TOL["bf16"], label=label, magnitude_scaled=True)


KG_CASES = [
    # B, H, N, d, dtype, causal, key_len_range
    (1, 2, 1000, 64, "bf16", True, None),
    (2, 1, 777, 128, "fp16", False, (1, 777)),
    (2, 3, 1100, 128, "bf16", True, (0, 1100)),     # batch 0 without keys
    (2, 2, 100, 64, "bf16", True, None),            # one tile of two key tiles
    (1, 2, 64, 64, "fp16", False, None),            # one key tile: group 1 idle
    (1, 1, 200, 64, "bf16", False, (1, 40)),
    (2, 4, 2048, 64, "bf16", True, None),
]


@pytest.mark.parametrize("kg", [1, 2])
@pytest.mark.parametrize("case", KG_CASES, ids=lambda c: "N{}d{}_{}".format(c[2], c[3], c[4]))
def test_forward_key_groups(case, kg):
    # Each tile's key range in one sweep (1) or split between two groups of
    # four waves whose online-softmax states merge on chip (2), against the
    # oracle on every head.
    B, H, N, d, dtype, causal, klr = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=191 + N + d, causal=causal,
                               key_len_range=klr)
    if klr is not None and klr[0] == 0:
        prob.key_lens[0] = 0
    gpu = run_gpu(prob, backward=False, key_groups=kg)
    check_all_heads(prob, gpu, f"{kg} key groups")
    compare(gpu, run_oracle(prob, backward=False), TOL[dtype], label=f"{kg} key groups {case}",
            magnitude_scaled=klr is not None and klr[0] < 4)


@pytest.mark.parametrize("boost", [1.5, 6.0])
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 128)])
def test_forward_key_groups_far_keys(dtype, d, boost):
    # Two key groups with scores far above the fixed reference: planted keys
    # in the first group's half (300..303) and in the second's (1000..1003);
    # the unchecked sweep keeps them or the work-group falls back to the
    # checked sweep, whose two states are merged by rescaling.
    prob = inputs.make_problem(1, 2, 1200, d, dtype, seed=677 + d, causal=True, scale=1.0)
    for j in (300, 1000):
        prob.k[:, :, j:j + 4] *= boost
    prob.k = inputs.round_to_dtype(prob.k, dtype)
    gpu = run_gpu(prob, backward=False, key_groups=2)
    label = f"key groups far keys x{boost} {dtype} d{d}"
    check_all_heads(prob, gpu, label)
    compare(gpu, run_oracle(prob, backward=False), TOL[dtype], label=label, magnitude_scaled=True)


@pytest.mark.parametrize("kg", [1, 2])
@pytest.mark.parametrize("case", KG_CASES, ids=lambda c: "N{}d{}_{}".format(c[2], c[3], c[4]))
def test_backward_key_groups(case, kg):
    # Both backward passes with each tile's sweep in one group of waves (1)
    # or split between two whose partial gradients add on chip (2; the dK/dV
    # pass keeps one group at d = 128), against the oracle on every head; the
    # 16-bit gradients are the rounding of the float32 ones (run_gpu).
    B, H, N, d, dtype, causal, klr = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=211 + N + d, causal=causal,
                               key_len_range=klr)
    if klr is not None and klr[0] == 0:
        prob.key_lens[0] = 0
    gpu = run_gpu(prob, key_groups=1, bwd_key_groups=kg)
    check_all_heads(prob, gpu, f"{kg} key groups backward")
    compare(gpu, run_oracle(prob), TOL[dtype], label=f"{kg} key groups backward {case}",
            magnitude_scaled=klr is not None and klr[0] < 4)


QS_CASES = [
    # B, H, N, d, dtype, causal, key_len_range, block_keep_p
    (1, 2, 1000, 128, "bf16", True, None, None),
    (2, 2, 700, 128, "fp16", False, (1, 700), None),
    (1, 3, 1100, 128, "bf16", False, None, 0.5),
    (1, 2, 100, 128, "bf16", True, None, None),        # one work-group, keys past N
    (2, 1, 1536, 128, "bf16", True, (600, 1536), 0.5),
    (8, 4, 256, 128, "fp16", True, None, None),        # 32 heads: the XCD-grouped schedule
    (1, 2, 64, 128, "bf16", True, None, None),         # half of the work-group's keys exist
    (1, 2, 128, 128, "bf16", False, None, None),       # exactly one work-group
    (2, 2, 300, 128, "bf16", False, (0, 300), None),   # a sequence with no visible key
]


@pytest.mark.parametrize("case", QS_CASES, ids=lambda c: "N{}d{}_{}_c{}".format(c[2], c[3], c[4],
                                                                                int(c[5])))
def test_backward_dkdv_query_halves(case):
    # At d = 128 the dK/dV pass splits every query tile between two groups of
    # waves (one 32-query half each, K and V read from LDS) unless one group is
    # asked for.  Both forms against the oracle on every head, and against
    # each other: the same products, added in another order, so within a few
    # units in the last place of the float32 gradients.
    B, H, N, d, dtype, causal, klr, bkp = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=233 + N, causal=causal, key_len_range=klr,
                               block_keep_p=bkp)
    if klr is not None and klr[0] == 0:
        prob.key_lens[0] = 0
    split = run_gpu(prob)
    one = run_gpu(prob, bwd_key_groups=1)
    check_all_heads(prob, split, "dK/dV query halves")
    ref = run_oracle(prob)
    ms = klr is not None and klr[0] < 4
    compare(split, ref, TOL[dtype], label=f"dK/dV query halves {case}", magnitude_scaled=ms)
    compare(one, ref, TOL[dtype], label=f"dK/dV one group {case}", magnitude_scaled=ms)
    for n in ("dk", "dv"):
        a, b = split[n], one[n]
        scale = max(np.abs(b).max(), 1e-30)
        assert np.abs(a - b).max() <= 1e-5 * scale, (n, float(np.abs(a - b).max()), scale)
    log(f"[dkdv halves] {case}: both forms agree")


BWD_ROW_CASES = [
    # dQ query rows, dK/dV keys per work-group, B, H, N, d, dtype, causal, key_len_range,
    # block_keep_p
    (64, 64, 1, 2, 1000, 64, "bf16", True, None, None),
    (256, 256, 2, 2, 777, 64, "bf16", True, None, None),
    (256, 64, 1, 3, 1100, 128, "fp16", False, (1, 1100), None),
    (64, 256, 1, 2, 1024, 128, "bf16", True, None, None),
    (64, 64, 1, 2, 1024, 64, "fp16", False, None, 0.5),
    (64, 64, 1, 1, 900, 128, "bf16", True, (300, 900), 0.5),
    (256, 256, 2, 4, 520, 128, "bf16", False, (100, 520), None),
]


@pytest.mark.parametrize("case", BWD_ROW_CASES,
                         ids=lambda c: "dq{}_kv{}_N{}d{}_{}".format(c[0], c[1], c[4], c[5], c[6]))
def test_backward_tile_rows(case):
    # dQ work-groups of 64 or 256 query rows and dK/dV work-groups of 64 or
    # 256 keys (the backward's tile-height option): each wave still owns 32
    # rows and sweeps the same tiles in the same order, so the gradients must
    # equal those of 128-row work-groups (one key group) bit for bit, on
    # every head; those are compared with the oracle.
    dqr, kvr, B, H, N, d, dtype, causal, klr, bkp = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=171 + dqr + kvr + N, causal=causal,
                               key_len_range=klr, block_keep_p=bkp)
    gpu = run_gpu(prob, bwd_key_groups=1)
    compare(gpu, run_oracle(prob), TOL[dtype], label=f"bwd rows default {case[2:]}",
            magnitude_scaled=klr is not None and klr[0] < 4)
    q, k, v, do = (dev(x, prob.dtype) for x in (prob.q, prob.k, prob.v, prob.do))
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).cuda()
    bm = None if prob.block_mask is None else torch.from_numpy(prob.block_mask).cuda()
    o = torch.from_numpy(gpu["o"]).to(q.dtype).cuda()
    lse = torch.from_numpy(gpu["lse"]).float().cuda()
    kw = dict(scale=float(prob.scale), causal=prob.causal, key_lens=kl, block_mask=bm,
              block_size=prob.block_size)
    grads = [nan_like(q) for _ in range(3)]
    fa_backward_ex(q, k, v, o, do, lse, dq=grads[0], dk=grads[1], dv=grads[2], dq_rows=dqr,
                   dkdv_rows=kvr, **kw)
    # the separate passes with the same heights
    sep = [nan_like(q) for _ in range(3)]
    _, ws = fa_backward_dq(q, k, v, o, do, lse, dq=sep[0], rows=dqr, **kw)
    fa_backward_dkdv(q, k, v, do, ws, dk=sep[1], dv=sep[2], rows=kvr, **kw)
    torch.cuda.synchronize()
    for n, g, g2 in zip(("dq", "dk", "dv"), grads, sep):
        want = gpu[n + "_16"]
        for label, t in (("fa_backward_ex", g), ("separate passes", g2)):
            got = t.double().cpu().numpy()
            assert not np.isnan(got).any(), f"{label} {n}: elements never written"
            assert np.array_equal(got, want), (
                f"{label} {n} rows {dqr}/{kvr}: {int((got != want).sum())} elements differ "
                f"from the 128-row backward")
    log(f"[bwd rows] {case}: gradients equal to the 128-row backward bit for bit")


@pytest.mark.parametrize("boost", [1.5, 6.0])
@pytest.mark.parametrize("rows", [128, 256])
@pytest.mark.parametrize("dtype,d,causal", [("bf16", 64, True), ("fp16", 128, False),
                                             ("bf16", 128, True)])
def test_forward_far_keys_take_the_recompute_path(dtype, d, causal, rows, boost):
    # Dense 16-bit forwards first sweep with each row's reference point fixed
    # at the largest score among the first 32 keys it sees (the unchecked
    # sweep).  Here a few later keys are scaled so that their scores exceed
    # that reference.  With boost 6 they do so by far more than the sweep
    # allows (a denominator of 2^64; fp16 probabilities overflow sooner and
    # leave the accumulator infinite) and the work-group starts over with the
    # checked sweep; with boost 1.5 bf16 keeps probabilities of up to 2^49 as
    # they are, while fp16 falls back.  Every path must agree with the oracle
    # (rows then attend almost only to the planted keys, so O leaves the
    # unit-variance regime: scaled bound).
    prob = inputs.make_problem(1, 2, 700, d, dtype, seed=611 + d, causal=causal, scale=1.0)
    prob.k[:, :, 300:304] *= boost
    prob.k = inputs.round_to_dtype(prob.k, dtype)
    # How far above the fixed reference the planted scores reach (log2 units).
    s = np.einsum("bhid,bhjd->bhij", prob.q.astype(np.float64), prob.k.astype(np.float64))
    s = s * prob.scale * np.log2(np.e)
    first = s[..., :32].max(axis=-1)
    later = s[..., 300:304].max(axis=-1)
    margin = (later - first)[..., 300:].max()
    assert margin > 64 + 8 if boost > 2 else 16 < margin < 60
    gpu = run_gpu(prob, block_rows=rows)
    label = f"far keys x{boost} {dtype} d{d} rows {rows}"
    check_all_heads(prob, gpu, label)
    compare(gpu, run_oracle(prob), TOL[dtype], label=label, magnitude_scaled=True)


def test_scale_zero_is_uniform_attention():
    prob = inputs.make_problem(1, 2, 200, 64, "fp32", seed=79, causal=True, scale=0.0)
    compare(run_gpu(prob), run_oracle(prob), TOL["fp32"], label="scale 0")


def test_empty_problem():
    z = torch.zeros(2, 3, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = fa_forward(z, z, z)
    dq, dk, dv = fa_backward(z, z, z, o, z, lse)
    torch.cuda.synchronize()
    assert o.shape == z.shape and lse.shape == (2, 3, 0) and dq.shape == z.shape


def test_deterministic():
    prob = inputs.make_problem(2, 4, 1000, 64, "bf16", seed=80, causal=True)
    a = run_gpu(prob)
    b = run_gpu(prob)
    for n in NAMES:
        assert np.array_equal(a[n], b[n], equal_nan=True), n


# Causal 128-row grids small enough to be resident at once take the snake tile
# order: one whole reversed round of 32 slots per XCD (B4 H16), a whole and a
# partial one (B5 H16), and none (B3 H16, 54 slots per XCD), ragged tails.
@pytest.mark.parametrize("B,H,N", [(4, 16, 1000), (5, 16, 1000), (3, 16, 1100)])
def test_forward_one_round_tile_orders(B, H, N):
    prob = inputs.make_problem(B, H, N, 64, "bf16", seed=90 + B, causal=True)
    gpu = run_gpu(prob, backward=False)
    compare(gpu, run_oracle(prob, backward=False), TOL["bf16"], label=f"B{B} H{H} N{N}")


# ----------------------------------------------------------------------------- the five workloads

def test_config_tiny_full():
    prob = inputs.workload("tiny")
    compare(run_gpu(prob), run_oracle(prob), TOL["fp32"], label="tiny")


def test_config_gpt2_small():
    prob = inputs.workload("gpt2_small")
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, "gpt2_small")
    compare(gpu, run_oracle(prob), TOL["bf16"], label="gpt2_small, all 96 heads")


def test_config_bert_large_padded():
    prob = inputs.workload("bert_large_padded")
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, "bert_large_padded")
    compare(gpu, run_oracle(prob), TOL["fp16"], label="bert_large_padded, all 256 heads")


def tile_edge_rows(n, tile=128, extra=16, seed=0):
    """First and last row of every tile, plus a few random rows."""
    t0 = np.arange(0, n, tile)
    rows = np.concatenate([t0, np.minimum(t0 + tile - 1, n - 1),
                           np.random.default_rng(seed).integers(0, n, extra)])
    return np.unique(rows)


def check_sampled_rows(prob, gpu, rows, label, heads=None):
    """O, LSE and dQ of the given query rows of every head (or ``heads``)
    against the oracle's row function."""
    worst = {}
    todo = heads or [(b, h) for b in range(prob.B) for h in range(prob.H)]
    for b, h in todo:
        kl = None if prob.key_lens is None else int(prob.key_lens[b])
        o, lse, dq = oracle.head_rows(*(x[b, h].astype(np.float64)
                                        for x in (prob.q, prob.k, prob.v, prob.do)),
                                      float(prob.scale), rows, causal=prob.causal, key_len=kl,
                                      block_mask=prob.block_mask, block_size=prob.block_size)
        ref = {"o": o, "lse": lse, "dq": dq}
        got = {n: gpu[n][b, h][rows] for n in ref}
        for n, e in compare(got, ref, TOL[prob.dtype], label=f"{label} rows of ({b},{h})").items():
            worst[n] = max(worst.get(n, 0.0), e)
    log(f"[parity] {label}: {len(rows)} rows on {len(todo)} heads, worst {worst}")


def check_sum_identities(prob, gpu, label):
    """Every head: sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 (over the rows
    that see a key; here every row does), within the spread that bf16 or
    fp16 rounding of the stored values (and of P, O) leaves in such sums."""
    u = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 2.0 ** -24}[prob.dtype]
    for b in range(prob.B):
        assert not rows_without_keys(prob, b).any(), "identities below assume every row sees a key"
        for h in range(prob.H):
            dv, dk, do = gpu["dv"][b, h], gpu["dk"][b, h], prob.do[b, h].astype(np.float64)
            q, o = prob.q[b, h].astype(np.float64), gpu["o"][b, h]
            dev_v = np.abs(dv.sum(axis=0) - do.sum(axis=0))
            bound_v = 6 * u * (np.sqrt((dv ** 2).sum(axis=0)) + np.sqrt((do ** 2).sum(axis=0)))
            assert np.all(dev_v <= bound_v), (label, b, h, "sum dV", dev_v.max(), bound_v.min())
            # sum_j dS_ij = D_i(exact O) - D_i(rounded O): spread |dO_i| |O_i| u per row
            spread = float(prob.scale) * np.sqrt(((np.abs(q) * (np.abs(do) * np.abs(o)).sum(
                axis=1, keepdims=True) * u) ** 2).sum(axis=0))
            dev_k = np.abs(dk.sum(axis=0))
            bound_k = 6 * (spread + u * np.sqrt((dk ** 2).sum(axis=0)))
            assert np.all(dev_k <= bound_k), (label, b, h, "sum dK", dev_k.max(), bound_k.min())
    log(f"[parity] {label}: dK, dV sums within bounds on all {prob.B * prob.H} heads")


@pytest.mark.parametrize("point", inputs.LONG_POINTS, ids=lambda p: f"N{p[0]}_d{p[1]}")
def test_config_long_causal(point):
    prob = inputs.workload("long_causal", *point)
    gpu = run_gpu(prob)
    label = f"long_causal {point}"
    check_all_heads(prob, gpu, label)
    if point[0] <= 4096:
        compare(gpu, run_oracle(prob, row_chunk=2048), TOL["bf16"], label=label + ", all heads")
        return
    heads = [(1, 7)]
    compare(gpu, run_oracle(prob, heads=heads, row_chunk=2048), TOL["bf16"], heads, label)
    check_sampled_rows(prob, gpu, tile_edge_rows(point[0], seed=point[0] + point[1]), label)
    check_sum_identities(prob, gpu, label)


def test_config_block_sparse():
    prob = inputs.workload("block_sparse")
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, "block_sparse")
    heads = [(0, 3)]
    compare(gpu, run_oracle(prob, heads=heads, row_chunk=2048), TOL["bf16"], heads,
            "block_sparse")
    check_sampled_rows(prob, gpu, tile_edge_rows(prob.N, seed=5), "block_sparse")
    check_sum_identities(prob, gpu, "block_sparse")


@pytest.mark.parametrize("n", inputs.SPARSE_LONG_N)
def test_config_block_sparse_long(n):
    # Structured block mask (band, global row and column, i.i.d. 1/32) at 32K
    # and 64K keys.  At 32K one whole head is compared.  At both sizes: O,
    # LSE and dQ on sampled rows of two heads (the oracle's row function), and
    # on every head the two identities the closed-form gradient satisfies,
    # sum_j dV_j = sum_i dO_i and sum_j dK_j = 0, within the spread that
    # rounding the stored values (and P, O) to bf16 leaves in such sums.
    prob = inputs.workload("block_sparse_long", n)
    gpu = run_gpu(prob)
    label = f"block_sparse_long N={n}"
    check_all_heads(prob, gpu, label)
    if n <= 32768:
        heads = [(0, 5)]
        compare(gpu, run_oracle(prob, heads=heads, row_chunk=2048), TOL["bf16"], heads, label)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 129, n // 2, n // 2 + 1, n - 129, n - 128,
                                      n - 1], rng.integers(0, n, 22)]))
    check_sampled_rows(prob, gpu, rows, label)
    check_sum_identities(prob, gpu, label)


# ----------------------------------------------------------------------------- split key ranges

SPLIT_CASES = [
    # B, H, N, d, dtype, causal, key_len_range, keep_p, band, global, key_chunk
    (1, 2, 384, 64, "bf16", False, None, 0.5, None, 0, 128),
    (2, 1, 300, 128, "fp16", True, (1, 300), 0.6, None, 0, 64),
    (1, 2, 200, 64, "fp32", True, None, 0.7, None, 0, 128),
    (1, 2, 1024, 64, "bf16", False, None, 1 / 32, 1, 1, 256),   # band + global row/column
    (1, 1, 1000, 128, "bf16", False, (500, 1000), 0.25, None, 0, 320),
]


@pytest.mark.parametrize("case", SPLIT_CASES,
                         ids=lambda c: "B{}H{}N{}d{}_{}_chunk{}".format(*c[:5], c[10]))
def test_blocksparse_split(case):
    # The key range of every query tile split over work-groups and merged:
    # against the oracle, and against the unsplit block-sparse forward.
    B, H, N, d, dtype, causal, klr, keep, band, glob, chunk = case
    prob = inputs.make_problem(B, H, N, d, dtype, seed=301 + N + chunk, causal=causal,
                               key_len_range=klr, block_keep_p=keep, block_band=band,
                               block_global=glob)
    q, k, v = (dev(x, dtype) for x in (prob.q, prob.k, prob.v))
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).cuda()
    bm = torch.from_numpy(prob.block_mask).cuda()
    kw = dict(scale=float(prob.scale), causal=causal, key_lens=kl)
    o, lse = fa_forward_blocksparse_split(q, k, v, bm, prob.block_size, key_chunk=chunk, **kw)
    o1, lse1 = fa_forward_blocksparse(q, k, v, bm, prob.block_size, **kw)
    torch.cuda.synchronize()
    got = {"o": o.double().cpu().numpy(), "lse": lse.double().cpu().numpy()}
    compare(got, run_oracle(prob, backward=False), TOL[dtype],
            label=f"split forward {case}", magnitude_scaled=klr is not None and klr[0] < 4)
    compare(got, {"o": o1.double().cpu().numpy(), "lse": lse1.double().cpu().numpy()},
            TOL[dtype], label=f"split vs unsplit {case}")


def test_blocksparse_split_edge_cases():
    # key_chunk >= N: one split, no workspace, the unsplit forward's results;
    # an all-ones block mask through the split path equals the dense forward
    # (with one key group per tile, as the block-sparse forward runs).
    prob = inputs.make_problem(1, 2, 520, 64, "bf16", seed=503, causal=True)
    q, k, v = (dev(x, "bf16") for x in (prob.q, prob.k, prob.v))
    nb = (520 + 127) // 128
    ones = torch.ones(nb, nb, dtype=torch.uint8, device="cuda")
    kw = dict(scale=float(prob.scale), causal=True)
    o1, l1 = fa_forward_blocksparse_split(q, k, v, ones, 128, key_chunk=1024, **kw)
    o2, l2 = fa_forward_blocksparse_split(q, k, v, ones, 128, key_chunk=192, **kw)
    od, ld = fa_forward_ex(q, k, v, key_groups=1, **kw)
    torch.cuda.synchronize()
    dense = {"o": od.double().cpu().numpy(), "lse": ld.double().cpu().numpy()}
    one = {"o": o1.double().cpu().numpy(), "lse": l1.double().cpu().numpy()}
    assert np.array_equal(one["o"], dense["o"]) and np.array_equal(one["lse"], dense["lse"])
    compare({"o": o2.double().cpu().numpy(), "lse": l2.double().cpu().numpy()}, dense,
            TOL["bf16"], label="3 splits, all-ones mask vs dense")
    compare(dense, run_oracle(prob, backward=False), TOL["bf16"], label="dense vs oracle")


@pytest.mark.parametrize("n", [32768, 65536])
def test_config_block_sparse_long_split(n):
    # The long structured workloads through the split forward (16384 keys per
    # split, the launch the bench times): sampled rows of O and LSE against the
    # oracle's row function, every row against the unsplit forward.
    prob = inputs.workload("block_sparse_long", n)
    q, k, v = (dev(x, prob.dtype) for x in (prob.q, prob.k, prob.v))
    bm = torch.from_numpy(prob.block_mask).cuda()
    o, lse = fa_forward_blocksparse_split(q, k, v, bm, prob.block_size, key_chunk=16384,
                                          scale=float(prob.scale))
    o1, lse1 = fa_forward_blocksparse(q, k, v, bm, prob.block_size, scale=float(prob.scale))
    torch.cuda.synchronize()
    compare({"o": o.double().cpu().numpy(), "lse": lse.double().cpu().numpy()},
            {"o": o1.double().cpu().numpy(), "lse": lse1.double().cpu().numpy()}, TOL["bf16"],
            label=f"block_sparse_long N={n} split vs unsplit")
    rows = np.array([0, 1, 127, 128, n // 2, n - 129, n - 1])
    for b, h in [(0, 3)]:
        ro, rl, _ = oracle.head_rows(*(x[b, h].astype(np.float64)
                                       for x in (prob.q, prob.k, prob.v, prob.do)),
                                     float(prob.scale), rows, block_mask=prob.block_mask,
                                     block_size=prob.block_size)
        compare({"o": o[b, h].double().cpu().numpy()[rows], "lse": lse[b, h].double().cpu().numpy()[rows]},
                {"o": ro, "lse": rl}, TOL["bf16"], label=f"block_sparse_long N={n} split rows")


# ----------------------------------------------------------------------------- maximum sizes

def test_max_block_mask_length():
    # N = 131072: the longest sequence whose block-mask row (1024 blocks) the
    # kernels cache on chip.  Sampled rows of O, LSE and dQ against the
    # oracle's row function; dK, dV through their sum identities.
    n = 131072
    prob = inputs.make_problem(1, 1, n, 64, "bf16", seed=91, block_keep_p=1 / 128, block_band=1)
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, f"N={n}")
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 127, 128, n // 2, n - 129, n - 128, n - 1],
                                     rng.integers(0, n, 9)]))
    check_sampled_rows(prob, gpu, rows, f"N={n} block mask")
    check_sum_identities(prob, gpu, f"N={n} block mask")


def test_many_heads():
    # 4096 (b, h) heads of 130 rows (a ragged second tile): the largest grids of
    # the five workloads have ~2K work-groups; this launches 8K per pass.
    # B * H is a multiple of 8 (the XCD-aware schedule, 512 heads per XCD).
    prob = inputs.make_problem(64, 64, 130, 64, "bf16", seed=92, causal=True)
    gpu = run_gpu(prob)
    check_all_heads(prob, gpu, "4096 heads")
    compare(gpu, run_oracle(prob), TOL["bf16"], label="4096 heads, all compared")
