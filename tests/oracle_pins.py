"""Pins of the fp64 oracle against things other than itself.

Each ``check_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with:
* hand-derived closed forms (tests/golden/closed_form_cases.json);
* central finite differences of L = sum(dO * O) (pins the backward to the
  forward, with every mask kind);
* torch's CPU fp64 attention (math path, autograd) and its CPU flash kernel's
  logsumexp (independent library routines);
* invariants and special cases of softmax attention.

The same checks run against mutated copies of the oracle in the mutation test,
which shows that each plausible slip (dropped term, wrong sign, off-by-one
mask, transposed operand) is caught by at least one of them.
"""

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
_NS = {"log": math.log, "exp": math.exp, "inf": math.inf, "__builtins__": {}}


def _ev(x):
    if isinstance(x, list):
        return [_ev(e) for e in x]
    return float(eval(x, _NS)) if isinstance(x, str) else float(x)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _b(x):
    return np.asarray(x)[None, None]


# ----------------------------------------------------------------------------- golden

def check_golden(orc):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v, do = (np.array(_ev(c[n])) for n in ("q", "k", "v", "do"))
        scale = _ev(c["scale"])
        kl = c["key_len"]
        bm = None if c["block_mask"] is None else np.array(c["block_mask"], np.uint8)
        kw = dict(causal=c["causal"], key_lens=None if kl is None else [kl],
                  block_mask=bm, block_size=c["block_size"])
        o, lse = orc.forward(_b(q), _b(k), _b(v), scale, **kw)
        dq, dk, dv = orc.backward(_b(q), _b(k), _b(v), _b(do), scale, **kw)
        np.testing.assert_allclose(o[0, 0], np.array(_ev(c["o"])), atol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], np.array(_ev(c["lse"])), atol=1e-13,
                                   err_msg=c["name"])
        for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            np.testing.assert_allclose(got[0, 0], np.array(_ev(c[name])), atol=1e-13,
                                       err_msg=f"{c['name']} {name}")


# ----------------------------------------------------------------------------- finite differences

FD_CASES = [
    dict(causal=False),
    dict(causal=True),
    dict(causal=False, key_len=4),
    dict(causal=True, key_len=5),
    dict(causal=False, block_mask=np.array([[1, 0, 1, 0], [0, 1, 1, 0], [1, 1, 1, 0],
                                            [0, 0, 1, 1]], np.uint8), block_size=2),
    dict(causal=True, block_mask=np.array([[1, 0, 0, 0], [1, 0, 0, 0], [0, 1, 1, 0],
                                           [1, 0, 0, 1]], np.uint8), block_size=2),
    dict(causal=False, key_len=0),
]


def check_finite_differences(orc, n=7, d=3, h=1e-6):
    for ci, kw in enumerate(FD_CASES):
        q, k, v, do = (_rand((n, d), 100 + 4 * ci + t) for t in range(4))
        scale = 0.7

        def loss(q_, k_, v_):
            o, _ = orc.head_forward(q_, k_, v_, scale, **kw)
            return float((do * o).sum())

        dq, dk, dv = orc.head_backward(q, k, v, do, scale, **kw)
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            num = np.zeros((n, d))
            for idx in np.ndindex(n, d):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            np.testing.assert_allclose(grad, num, atol=2e-8, rtol=1e-6,
                                       err_msg=f"fd case {ci} input {which}")


# ----------------------------------------------------------------------------- torch reference

TORCH_CASES = [
    dict(causal=False),
    dict(causal=True),
    dict(causal=False, key_lens=[9, 33]),
    dict(causal=True, key_lens=[20, 1]),
    dict(causal=False, block_mask="random", block_size=8),
    dict(causal=True, block_mask="random", block_size=8),
]


def check_torch_reference(orc, B=2, H=2, n=33, d=16):
    for ci, kw in enumerate(TORCH_CASES):
        kw = dict(kw)
        q, k, v, do = (_rand((B, H, n, d), 200 + 4 * ci + t) for t in range(4))
        scale = 0.3
        if isinstance(kw.get("block_mask"), str):
            nb = -(-n // kw["block_size"])
            bm = (np.random.default_rng(300 + ci).random((nb, nb)) < 0.4).astype(np.uint8)
            np.fill_diagonal(bm, 1)
            kw["block_mask"] = bm
        o, lse = orc.forward(q, k, v, scale, **kw)
        dq, dk, dv = orc.backward(q, k, v, do, scale, **kw)
        # The mask is built here from the definitions, independently of the oracle.
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        for b in range(B):
            vis = np.ones((n, n), bool)
            if kw.get("causal"):
                vis &= j <= i
            if kw.get("key_lens") is not None:
                vis &= j < kw["key_lens"][b]
            if kw.get("block_mask") is not None:
                bs = kw["block_size"]
                vis &= kw["block_mask"][i // bs, j // bs] != 0
            tq, tk, tv = (torch.tensor(x[b], requires_grad=True) for x in (q, k, v))
            tmask = torch.tensor(vis)
            to = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=tmask, scale=scale)
            to.backward(torch.tensor(do[b]))
            add = torch.zeros(n, n, dtype=torch.float64).masked_fill(~tmask, -math.inf)
            _, tlse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
                tq.detach()[None], tk.detach()[None], tv.detach()[None], 0.0, False,
                attn_mask=add, scale=scale)[:2]
            msg = f"torch case {ci} batch {b}"
            np.testing.assert_allclose(o[b], to.detach().numpy(), atol=1e-12, err_msg=msg)
            np.testing.assert_allclose(lse[b], tlse[0].numpy(), atol=1e-12, err_msg=msg)
            np.testing.assert_allclose(dq[b], tq.grad.numpy(), atol=1e-12, err_msg=msg)
            np.testing.assert_allclose(dk[b], tk.grad.numpy(), atol=1e-12, err_msg=msg)
            np.testing.assert_allclose(dv[b], tv.grad.numpy(), atol=1e-12, err_msg=msg)


# ----------------------------------------------------------------------------- invariants

def check_invariants(orc, n=23, d=5):
    q, k, v, do = (_rand((n, d), 400 + t) for t in range(4))
    scale = 0.37
    for causal in (False, True):
        # rows of P sum to 1; P vanishes on masked pairs
        p = orc.head_probabilities(q, k, scale, causal=causal, key_len=17)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
        jj = np.arange(n)[None, :]
        ii = np.arange(n)[:, None]
        masked = (jj >= 17) | ((jj > ii) if causal else np.zeros((n, n), bool))
        assert np.all(p[masked] == 0)
        # O lies in the per-column hull of the visible V rows
        o, lse = orc.head_forward(q, k, v, scale, causal=causal)
        for r in range(n):
            vis_v = v[: r + 1] if causal else v
            assert np.all(o[r] <= vis_v.max(axis=0) + 1e-12)
            assert np.all(o[r] >= vis_v.min(axis=0) - 1e-12)
        # constant V rows give that constant
        c = np.array([0.5, -2.0, 3.0, 0.0, 1.25])
        oc, _ = orc.head_forward(q, k, np.tile(c, (n, 1)), scale, causal=causal)
        np.testing.assert_allclose(oc, np.tile(c, (n, 1)), atol=1e-13)
        # identical keys: O = mean of visible V, LSE = scale*q.k + ln|visible|
        kk = np.tile(k[3], (n, 1))
        oi, li = orc.head_forward(q, kk, v, scale, causal=causal)
        counts = np.arange(1, n + 1) if causal else np.full(n, n)
        means = np.cumsum(v, axis=0) / counts[:, None] if causal else np.tile(v.mean(0), (n, 1))
        np.testing.assert_allclose(oi, means, atol=1e-13)
        np.testing.assert_allclose(li, scale * (q @ k[3]) + np.log(counts), atol=1e-13)
        # shifting every key by the same vector leaves O alone and shifts LSE by scale*q.c
        shift = np.array([1.0, -0.5, 2.0, 0.25, -1.0])
        os_, ls_ = orc.head_forward(q, k + shift, v, scale, causal=causal)
        np.testing.assert_allclose(os_, o, atol=1e-12)
        np.testing.assert_allclose(ls_, lse + scale * (q @ shift), atol=1e-12)
        # gradient sums: sum_j dK_j = 0 (softmax shift invariance), sum_j dV_j = sum_i dO_i
        dq, dk, dv = orc.head_backward(q, k, v, do, scale, causal=causal)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
        # D identity: sum_j P_ij dP_ij equals rowsum(dO * O)
        pf = orc.head_probabilities(q, k, scale, causal=causal)
        np.testing.assert_allclose((pf * (do @ v.T)).sum(1), (do * o).sum(1), atol=1e-12)
    # jointly permuting keys and values leaves O unchanged (non-causal, unmasked)
    perm = np.random.default_rng(7).permutation(n)
    o1, l1 = orc.head_forward(q, k, v, scale)
    o2, l2 = orc.head_forward(q, k[perm], v[perm], scale)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)
    # an all-ones block mask equals no block mask; an all-zero one sees nothing
    bm1 = np.ones((3, 3), np.uint8)
    o3, l3 = orc.head_forward(q, k, v, scale, causal=True, block_mask=bm1, block_size=8)
    o4, l4 = orc.head_forward(q, k, v, scale, causal=True)
    np.testing.assert_array_equal(o3, o4)
    np.testing.assert_array_equal(l3, l4)
    o5, l5 = orc.head_forward(q, k, v, scale, block_mask=np.eye(3, dtype=np.uint8) * 0,
                              block_size=8)
    assert np.all(o5 == 0) and np.all(np.isneginf(l5))
    # a block mask is the element mask it stands for: compare with key_len blocks
    bm_lower = np.array([[1, 0, 0], [1, 1, 0], [1, 1, 1]], np.uint8)
    ob, lb = orc.head_forward(q, k, v, scale, block_mask=bm_lower, block_size=8)
    for r in range(n):
        orow, lrow = orc.head_forward(q, k, v, scale, key_len=8 * (r // 8 + 1))
        np.testing.assert_allclose(ob[r], orow[r], atol=1e-14)
        np.testing.assert_allclose(lb[r], lrow[r], atol=1e-14)


def check_special_cases(orc, n=11, d=4):
    q, k, v, do = (_rand((n, d), 500 + t) for t in range(4))
    # a single visible key (key_len = 1) returns exactly its V row; dQ = 0, dK = 0
    o, lse = orc.head_forward(q, k, v, 0.9, key_len=1)
    assert np.array_equal(o, np.tile(v[0], (n, 1)))
    np.testing.assert_allclose(lse, 0.9 * (q @ k[0]), atol=1e-14)
    dq, dk, dv = orc.head_backward(q, k, v, do, 0.9, key_len=1)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)   # dP and D agree up to rounding
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)
    np.testing.assert_allclose(dv[0], do.sum(0), atol=1e-13)
    assert np.all(dv[1:] == 0)
    # causal row 0 sees key 0 only
    oc, _ = orc.head_forward(q, k, v, 0.9, causal=True)
    assert np.array_equal(oc[0], v[0])
    # N = 1
    o1, l1 = orc.head_forward(q[:1], k[:1], v[:1], 0.9, causal=True)
    assert np.array_equal(o1, v[:1])
    np.testing.assert_allclose(l1, 0.9 * q[0] @ k[0], atol=1e-15)
    # scale 0: uniform attention, LSE = ln|visible|, dQ = dK = 0
    for causal in (False, True):
        o0, l0 = orc.head_forward(q, k, v, 0.0, causal=causal)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        np.testing.assert_allclose(l0, np.log(cnt), atol=1e-14)
        mean = np.cumsum(v, 0) / cnt[:, None] if causal else np.tile(v.mean(0), (n, 1))
        np.testing.assert_allclose(o0, mean, atol=1e-14)
        dq0, dk0, dv0 = orc.head_backward(q, k, v, do, 0.0, causal=causal)
        assert np.all(dq0 == 0) and np.all(dk0 == 0)
    # no visible key anywhere: O = 0, LSE = -inf, no gradient
    oz, lz = orc.head_forward(q, k, v, 0.9, key_len=0)
    assert np.all(oz == 0) and np.all(np.isneginf(lz))
    g = orc.head_backward(q, k, v, do, 0.9, key_len=0)
    assert all(np.all(x == 0) for x in g)


def check_row_chunking(orc, n=37, d=6):
    q, k, v, do = (_rand((n, d), 600 + t) for t in range(4))
    bm = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8)
    for kw in (dict(causal=True), dict(key_len=20), dict(block_mask=bm, block_size=16)):
        full_o, full_l = orc.head_forward(q, k, v, 0.4, **kw)
        ch_o, ch_l = orc.head_forward(q, k, v, 0.4, row_chunk=5, **kw)
        np.testing.assert_allclose(ch_o, full_o, atol=1e-14)
        np.testing.assert_allclose(ch_l, full_l, atol=1e-14)
        full_g = orc.head_backward(q, k, v, do, 0.4, **kw)
        ch_g = orc.head_backward(q, k, v, do, 0.4, row_chunk=5, **kw)
        for a, b in zip(full_g, ch_g):
            np.testing.assert_allclose(b, a, atol=1e-13)


def check_rows(orc, n=41, d=6):
    # O, LSE, dQ of sampled rows equal the same rows of the whole-head oracle
    # (itself pinned above), for every mask kind, unsorted and repeated rows,
    # and rows that see no key.
    q, k, v, do = (_rand((n, d), 700 + t) for t in range(4))
    bm = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], np.uint8)
    rows = np.array([40, 0, 7, 7, 23, 16, 31])
    for kw in (dict(), dict(causal=True), dict(key_len=9), dict(key_len=0),
               dict(block_mask=bm, block_size=16), dict(causal=True, key_len=30, block_mask=bm,
                                                        block_size=16)):
        o, lse = orc.head_forward(q, k, v, 0.45, **kw)
        dq, _, _ = orc.head_backward(q, k, v, do, 0.45, **kw)
        ro, rl, rdq = orc.head_rows(q, k, v, do, 0.45, rows, **kw)
        np.testing.assert_allclose(ro, o[rows], atol=1e-14)
        np.testing.assert_array_equal(np.isneginf(rl), np.isneginf(lse[rows]))
        fin = ~np.isneginf(rl)
        np.testing.assert_allclose(rl[fin], lse[rows][fin], atol=1e-14)
        np.testing.assert_allclose(rdq, dq[rows], atol=1e-13)


def check_kv_torch_lower_right(orc, B=2, H=2, d=8):
    # Bottom-right causal against torch's own lower-right causal bias (an
    # independent library definition of the alignment).  The cache fill L is
    # applied here by handing torch only the first L keys.
    from torch.nn.attention.bias import causal_lower_right
    import warnings
    for ci, (nq, nk, lens) in enumerate([(5, 13, None), (1, 40, [40, 17]), (9, 9, None),
                                          (7, 30, [12, 30]), (16, 20, [20, 19])]):
        q = _rand((B, H, nq, d), 800 + ci)
        k, v = (_rand((B, H, nk, d), 810 + 2 * ci + t) for t in range(2))
        for causal in (False, True):
            o, lse = orc.forward_kv(q, k, v, 0.35, causal=causal, key_lens=lens)
            for b in range(B):
                L = nk if lens is None else lens[b]
                tq, tk, tv = (torch.tensor(x[b]) for x in (q, k[:, :, :L], v[:, :, :L]))
                with warnings.catch_warnings():
                    warnings.simplefilter("ignore")
                    mask = causal_lower_right(nq, L) if causal else None
                    to = torch.nn.functional.scaled_dot_product_attention(
                        tq, tk, tv, attn_mask=mask, scale=0.35)
                msg = f"kv case {ci} causal {causal} batch {b}"
                np.testing.assert_allclose(o[b], to.numpy(), atol=1e-12, err_msg=msg)
                # logsumexp from torch's own softmax normaliser over the same keys
                s = 0.35 * (tq @ tk.transpose(-1, -2))
                if causal:
                    keep = mask._materialize(torch.device("cpu"))
                    s = s.masked_fill(~keep, -math.inf)
                np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).numpy(),
                                           atol=1e-12, err_msg=msg)


def check_kv_decode(orc, n=29, d=6):
    # Decoding the newest positions against a cache equals the same rows of
    # full causal self-attention over the filled part (the forward oracle is
    # pinned above); a cache larger than its fill changes nothing.
    x = [_rand((n, d), 900 + t) for t in range(3)]
    o_full, lse_full = orc.head_forward(x[0], x[1], x[2], 0.5, causal=True)
    for nq in (1, 3, n):
        pad = np.full((11, d), 7.0)          # unfilled cache entries (never visible)
        k = np.concatenate([x[1], pad])
        v = np.concatenate([x[2], pad])
        o, lse = orc.head_forward_kv(x[0][n - nq:], k, v, 0.5, causal=True, key_len=n)
        np.testing.assert_allclose(o, o_full[n - nq:], atol=1e-14)
        np.testing.assert_allclose(lse, lse_full[n - nq:], atol=1e-14)
    # one query with causal sees every filled key: the non-causal result
    o1, l1 = orc.head_forward_kv(x[0][:1], x[1], x[2], 0.5, causal=True, key_len=17)
    o2, l2 = orc.head_forward(np.concatenate([x[0][:1], np.zeros((n - 1, d))]), x[1], x[2], 0.5,
                              key_len=17)
    np.testing.assert_allclose(o1[0], o2[0], atol=1e-14)
    np.testing.assert_allclose(l1[0], l2[0], atol=1e-14)
    # more queries than filled keys: the first nq - L rows see nothing
    q8 = np.concatenate([_rand((5, d), 950), x[0][:3]])   # rows 5..7 are positions 0..2
    o, lse = orc.head_forward_kv(q8, x[1], x[2], 0.5, causal=True, key_len=3)
    assert np.all(o[:5] == 0) and np.all(np.isneginf(lse[:5]))
    np.testing.assert_allclose(o[5:], o_full[:3], atol=1e-14)
    # an empty cache: every row sees nothing
    o, lse = orc.head_forward_kv(x[0][:4], x[1], x[2], 0.5, causal=False, key_len=0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # fills outside [0, nk] are clamped: nk + 5 acts as a full cache, -3 as an empty one
    o, lse = orc.head_forward_kv(x[0][n - 4:], x[1], x[2], 0.5, causal=True, key_len=n + 5)
    np.testing.assert_allclose(o, o_full[n - 4:], atol=1e-14)
    o, lse = orc.head_forward_kv(x[0][:4], x[1], x[2], 0.5, causal=True, key_len=-3)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def check_varlen(orc, H=3, d=5):
    # Packed sequences against torch, one sequence at a time: the slices are
    # taken here from the prefix sums, and torch's lower-right causal bias
    # (or none) gives each sequence's attention.
    from torch.nn.attention.bias import causal_lower_right
    import warnings
    lq = [4, 0, 9, 1, 6]
    lk = [7, 3, 9, 0, 2]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    q = _rand((H, cq[-1], d), 960)
    k, v = (_rand((H, ck[-1], d), 961 + t) for t in range(2))
    for causal in (False, True):
        o, lse = orc.forward_varlen(q, k, v, cq, ck, 0.45, causal=causal)
        for b in range(len(lq)):
            rows = slice(cq[b], cq[b + 1])
            if lq[b] == 0:
                continue
            if lk[b] == 0:          # no keys at all: O = 0, LSE = -inf
                assert np.all(o[:, rows] == 0) and np.all(np.isneginf(lse[:, rows]))
                continue
            tq = torch.tensor(q[:, rows])
            tk, tv = (torch.tensor(x[:, ck[b]:ck[b + 1]]) for x in (k, v))
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                mask = causal_lower_right(lq[b], lk[b]) if causal else None
                to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                                      scale=0.45)
            ref = to.numpy()
            seen = ~np.isnan(ref).any(axis=-1)          # torch gives NaN for rows with no key
            np.testing.assert_allclose(o[:, rows][seen], ref[seen], atol=1e-12,
                                       err_msg=f"varlen seq {b} causal {causal}")
            assert np.all(o[:, rows][~seen] == 0) and np.all(np.isneginf(lse[:, rows][~seen]))
    # equal lengths: the packed problem is the batched one, head-major
    B, n = 3, 6
    qb, kb, vb = (_rand((B, H, n, d), 970 + t) for t in range(3))
    pack = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(H, B * n, d))
    cu = np.arange(B + 1) * n
    o, lse = orc.forward_varlen(pack(qb), pack(kb), pack(vb), cu, cu, 0.3, causal=True)
    ob, lb = orc.forward(qb, kb, vb, 0.3, causal=True)
    np.testing.assert_allclose(o, pack(ob), atol=1e-14)
    np.testing.assert_allclose(lse, lb.transpose(1, 0, 2).reshape(H, B * n), atol=1e-14)


ALL_PINS = [check_golden, check_finite_differences, check_torch_reference,
            check_invariants, check_special_cases, check_row_chunking, check_rows,
            check_kv_torch_lower_right, check_kv_decode, check_varlen]
