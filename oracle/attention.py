"""Plain fp64 CPU attention: the correctness oracle for the tiled GPU kernels.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it.  It shares no code with the HIP library.

What it computes is standard attention written out with the full N x N score
matrix materialised, the formulation that the IO-aware method is exact with
respect to:

* review page, "Problem": standard attention materialises the N-by-N matrix;
* visual guide, "standard attention" and the closing results table: the tiled
  method gives the same outputs ("exact", no change to the model math);
* review page, "Method" and claim C7: the forward keeps only the output and
  small normalisation values, the backward recomputes the attention matrix
  from them.  The normalisation value kept here is the per-row logsumexp
  (natural log), which carries the running max m and denominator l of the
  slides' "action grammar" card as LSE = m + ln(l);
* visual guide, block-sparse paragraph: masking whole blocks.  The block-masked
  result is exact with respect to the block mask and approximate with respect
  to dense attention (review page, caveats), so the sparse reference is dense
  attention with the same mask applied.

The backward pass is the closed form of the gradient of L = sum(dO * O):
D = rowsum(dO * O), dV = P^T dO, dP = dO V^T, dS = P * (dP - D),
dQ = scale * dS K, dK = scale * dS^T Q.

Readings where the pages are silent (each is also listed in the design notes):
* layout [B, H, N, d], d innermost; one (b, h) head at a time;
* causal means key j is visible to query i iff j <= i (top-left aligned);
* key padding masks keys only: key j of batch b is visible iff j < key_lens[b];
  padded query rows are computed like any other row;
* the block mask is one uint8 [ceil(N/bs), ceil(N/bs)] array shared by every
  (b, h); entry (I, J) nonzero keeps every (i, j) with i // bs == I and
  j // bs == J; masks combine by logical AND;
* a query row that sees no key at all has O = 0, LSE = -inf and contributes
  nothing to any gradient;
* with nq queries against nk cached keys (inference, ``forward_kv``), the
  queries are the newest nq positions of a sequence of L = key_lens[b] filled
  cache entries, and causal is aligned bottom-right: j <= i + L - nq;
* packed variable-length batches (``forward_varlen``) lay sequences back to
  back per head, [H, T, d], delimited by prefix sums cu[0..B]; each sequence
  is the problem above with its own query and key counts.

Everything is float64.  Inputs are the dtype-rounded values the GPU receives,
upcast; ``scale`` is the float32 value handed to the GPU, upcast.
"""

import numpy as np


def visibility(n, causal=False, key_len=None, block_mask=None, block_size=128, rows=None):
    """Boolean [n, n] matrix: entry (i, j) is True iff query i may attend key j.

    Combines the three masks of the method (causal, key padding, block mask)
    by logical AND, as read above.  With ``rows`` (query indices), only those
    rows: [len(rows), n].
    """
    i = (np.arange(n) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(n)[None, :]
    vis = np.ones((i.shape[0], n), dtype=bool)
    if causal:
        vis &= j <= i
    if key_len is not None:
        vis &= j < int(key_len)
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        vis &= bm[i // block_size, j // block_size]
    return vis


def _head_forward(q, k, v, scale, vis):
    """One head (or a group of its query rows).  Returns (O, LSE, P).

    Softmax over the visible keys of each row, with the row max m subtracted
    before exponentiating and the denominator l = sum exp(S - m):
    P = exp(S - m) / l and LSE = m + ln(l).
    """
    s = scale * (q @ k.T)                       # score matrix S, rows x N
    s = np.where(vis, s, -np.inf)
    seen = vis.any(axis=1)
    m = np.where(seen, s.max(axis=1, initial=-np.inf), 0.0)
    ex = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = ex.sum(axis=1)
    l_safe = np.where(seen, l, 1.0)
    p = ex / l_safe[:, None]
    lse = np.where(seen, m + np.log(l_safe), -np.inf)
    o = p @ v
    return o, lse, p


def _row_chunks(n, row_chunk):
    step = n if not row_chunk else max(1, int(row_chunk))
    for r0 in range(0, n, step):
        yield r0, min(n, r0 + step)


def head_forward(q, k, v, scale, causal=False, key_len=None, block_mask=None,
                 block_size=128, row_chunk=None):
    """Forward for one head: q, k, v are [N, d] float64.  Returns (O, LSE).

    Query rows are independent in the definition (each row's softmax sees all
    its visible keys), so ``row_chunk`` only bounds memory: rows are handled
    in groups, each group with its full set of keys.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    scale = float(scale)
    n = q.shape[0]
    vis_all = visibility(n, causal, key_len, block_mask, block_size)
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for r0, r1 in _row_chunks(n, row_chunk):
        o[r0:r1], lse[r0:r1], _ = _head_forward(q[r0:r1], k, v, scale, vis_all[r0:r1])
    return o, lse


def head_probabilities(q, k, scale, causal=False, key_len=None, block_mask=None,
                       block_size=128):
    """The attention matrix P of one head (rows sum to 1 over visible keys)."""
    q, k = (np.asarray(x, dtype=np.float64) for x in (q, k))
    vis = visibility(q.shape[0], causal, key_len, block_mask, block_size)
    return _head_forward(q, k, np.zeros((k.shape[0], 1)), float(scale), vis)[2]


def head_backward(q, k, v, do, scale, causal=False, key_len=None, block_mask=None,
                  block_size=128, row_chunk=None):
    """Backward for one head from the closed form.  Returns (dQ, dK, dV).

    Runs its own forward (never a GPU result).  dK and dV are sums over query
    rows, so they accumulate across row groups.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    scale = float(scale)
    n = q.shape[0]
    vis_all = visibility(n, causal, key_len, block_mask, block_size)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0, r1 in _row_chunks(n, row_chunk):
        o, _, p = _head_forward(q[r0:r1], k, v, scale, vis_all[r0:r1])
        d_row = (do[r0:r1] * o).sum(axis=1)     # D = rowsum(dO * O)
        dv += p.T @ do[r0:r1]                   # dV = P^T dO
        dp = do[r0:r1] @ v.T                    # dP = dO V^T
        ds = p * (dp - d_row[:, None])          # dS = P * (dP - D)
        dq[r0:r1] = scale * (ds @ k)            # dQ = scale * dS K
        dk += scale * (ds.T @ q[r0:r1])         # dK = scale * dS^T Q
    return dq, dk, dv


def head_rows(q, k, v, do, scale, rows, causal=False, key_len=None, block_mask=None,
              block_size=128):
    """O, LSE and dQ of the given query rows of one head, from the same
    definitions (each row's softmax over all its visible keys; D, dP, dS and
    dQ = scale * dS K row by row).  Costs O(N d) per row, for checking
    sampled rows of problems too large for a whole head.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    rows = np.asarray(rows)
    scale = float(scale)
    vis = visibility(q.shape[0], causal, key_len, block_mask, block_size, rows=rows)
    o_r, lse_r, p_r = _head_forward(q[rows], k, v, scale, vis)
    d_r = np.sum(do[rows] * o_r, axis=1)        # D = rowsum(dO * O)
    dp_r = do[rows] @ v.T                       # dP = dO V^T
    ds_r = p_r * (dp_r - d_r[:, None])          # dS = P * (dP - D)
    return o_r, lse_r, scale * (ds_r @ k)       # dQ = scale * dS K


def visibility_kv(nq, nk, causal=False, key_len=None):
    """Boolean [nq, nk]: query i of nq new queries may attend key j of nk.

    Inference reading (the pages say only that the kernel came to serve
    inference; the alignment is this module's reading): the key/value tensors
    hold a cache of which the first L = key_len (clamped to [0, nk]; nk when
    None) positions are filled, and the nq queries are the newest nq positions
    of that sequence, so query i sits at position i + L - nq.  Causal then
    means key j is visible iff j <= i + L - nq (aligned bottom-right); keys
    j >= L are never visible.  With nq = nk = L this is the top-left causal
    mask of ``visibility``.
    """
    L = nk if key_len is None else min(max(int(key_len), 0), nk)
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    vis = np.broadcast_to(j < L, (nq, nk)).copy()
    if causal:
        vis &= j <= i + (L - nq)
    return vis


def head_forward_kv(q, k, v, scale, causal=False, key_len=None):
    """Forward of nq queries (q: [nq, d]) against nk keys and values (k, v:
    [nk, d]) with the visibility of ``visibility_kv``.  Returns (O, LSE);
    rows that see no key have O = 0 and LSE = -inf."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    vis = visibility_kv(q.shape[0], k.shape[0], causal, key_len)
    o, lse, _ = _head_forward(q, k, v, float(scale), vis)
    return o, lse


def forward_kv(q, k, v, scale, causal=False, key_lens=None, heads=None):
    """Batched ``head_forward_kv``: q [B, H, nq, d], k and v [B, H, nk, d].
    Returns (O [B, H, nq, d], LSE [B, H, nq]); ``heads`` as in ``forward``."""
    B, H, nq, _ = _heads(q)
    o = np.full((B, H, nq, v.shape[-1]), np.nan)
    lse = np.full((B, H, nq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        kl = None if key_lens is None else int(key_lens[b])
        o[b, h], lse[b, h] = head_forward_kv(q[b, h], k[b, h], v[b, h], scale, causal, kl)
    return o, lse


def forward_varlen(q, k, v, cu_q, cu_k, scale, causal=False):
    """Packed variable-length forward.  q: [H, Tq, d] and k, v: [H, Tk, d]
    hold B sequences back to back; sequence b owns query rows
    cu_q[b] .. cu_q[b+1] - 1 and key rows cu_k[b] .. cu_k[b+1] - 1 of every
    head.  Each sequence attends only to its own keys, with the visibility
    of ``visibility_kv`` (nq = its query count, nk = L = its key count, so
    causal is aligned bottom-right; with equal counts it is top-left).
    Returns (O [H, Tq, d], LSE [H, Tq]).  Rows outside every sequence are
    left as NaN."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    H, Tq, _ = q.shape
    o = np.full((H, Tq, v.shape[-1]), np.nan)
    lse = np.full((H, Tq), np.nan)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        for h in range(H):
            o[h, q0:q1], lse[h, q0:q1] = head_forward_kv(q[h, q0:q1], k[h, k0:k1], v[h, k0:k1],
                                                         scale, causal)
    return o, lse


def _heads(x):
    x = np.asarray(x)
    assert x.ndim == 4, "expected [B, H, N, d]"
    return x.shape


def forward(q, k, v, scale, causal=False, key_lens=None, block_mask=None,
            block_size=128, row_chunk=None, heads=None):
    """Batched forward over [B, H, N, d].  Returns (O [B,H,N,d], LSE [B,H,N]).

    ``heads``: optional list of (b, h) pairs; only those heads are computed
    and the others are left as NaN (used to check sampled heads at full size).
    """
    B, H, N, d = _heads(q)
    o = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        kl = None if key_lens is None else int(key_lens[b])
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], scale, causal, kl,
                                          block_mask, block_size, row_chunk)
    return o, lse


def backward(q, k, v, do, scale, causal=False, key_lens=None, block_mask=None,
             block_size=128, row_chunk=None, heads=None):
    """Batched backward over [B, H, N, d].  Returns (dQ, dK, dV)."""
    B, H, N, d = _heads(q)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        kl = None if key_lens is None else int(key_lens[b])
        dq[b, h], dk[b, h], dv[b, h] = head_backward(
            q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, kl, block_mask,
            block_size, row_chunk)
    return dq, dk, dv
