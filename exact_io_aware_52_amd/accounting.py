"""Flop and byte accounting for the tiled attention path (host arithmetic only).

Algorithmic flops per kept (query, key) pair: the forward's two contractions
(S = Q K^T and O = P V) are 2 * d each, so 4 * d; the backward's five
contractions (recomputed S, dV, dP, dK, dQ) are 10 * d, so 14 * d for a forward
plus backward.  A pair is kept when the causal, key-padding and block masks all
keep it.

Compulsory HBM bytes of one head (s = bytes per element): the forward reads
Q, K, V and writes O and the fp32 logsumexp; the backward reads Q, K, V, O, dO
and the logsumexp and writes dQ, dK, dV, plus its fp32 D vector.
"""

import numpy as np

ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


def kept_pairs_head(n, causal=False, key_len=None, block_mask=None, block_size=128):
    """Number of visible (query, key) pairs in one head, without forming N x N."""
    n = int(n)
    i = np.arange(n)
    limit = np.full(n, n, dtype=np.int64)            # keys [0, limit_i) pass causal/len
    if causal:
        limit = np.minimum(limit, i + 1)
    if key_len is not None:
        limit = np.minimum(limit, max(0, min(int(key_len), n)))
    if block_mask is None:
        return int(limit.sum())
    bm = (np.asarray(block_mask) != 0).astype(np.int64)
    nb = bm.shape[1]
    starts = np.arange(nb, dtype=np.int64) * block_size
    total = 0
    for blk in range(-(-n // block_size)):
        rows = slice(blk * block_size, min(n, (blk + 1) * block_size))
        lim = limit[rows][:, None]                    # rows x 1
        per_block = np.clip(lim - starts[None, :], 0, block_size)   # rows x nb
        total += int((per_block * bm[blk][None, :]).sum())
    return total


def kept_pairs(prob):
    """Kept pairs summed over every (b, h) head of a Problem."""
    total = 0
    for b in range(prob.B):
        kl = None if prob.key_lens is None else int(prob.key_lens[b])
        total += prob.H * kept_pairs_head(prob.N, prob.causal, kl, prob.block_mask,
                                          prob.block_size)
    return total


def flops(prob, which):
    """Algorithmic flops: which in {'fwd', 'bwd', 'fwd+bwd'}."""
    per = {"fwd": 4, "bwd": 10, "fwd+bwd": 14}[which]
    return per * prob.d * kept_pairs(prob)


def compulsory_bytes(prob, which):
    s = ELEM_BYTES[prob.dtype]
    heads = prob.B * prob.H
    n, d = prob.N, prob.d
    fwd = heads * (4 * n * d * s + 4 * n)
    # backward: read Q, K, V, O, dO, write dQ, dK, dV; LSE read, -D and
    # LSE*log2(e) written by the dQ pass and read back by the dK/dV pass
    bwd = heads * (8 * n * d * s + 20 * n)
    return {"fwd": fwd, "bwd": bwd, "fwd+bwd": fwd + bwd}[which]


def standard_attention_bytes(prob):
    """HBM bytes of a forward that materialises S and P (write S, read S, write
    P, read P) plus reading Q, K, V and writing O: the Theta(N d + N^2) model."""
    s = ELEM_BYTES[prob.dtype]
    heads = prob.B * prob.H
    n, d = prob.N, prob.d
    return heads * (4 * n * n * s + 4 * n * d * s)


def tiled_forward_bytes(prob, block_rows):
    """HBM bytes of the tiled forward when every Q tile of ``block_rows`` rows
    reads the K and V tiles it keeps: the Theta(N^2 d^2 / M) model's re-read
    term plus the compulsory traffic."""
    s = ELEM_BYTES[prob.dtype]
    n, d = prob.N, prob.d
    dense = prob.B * prob.H * n * n
    frac = kept_pairs(prob) / dense if dense else 0.0
    tiles = -(-n // block_rows)
    return compulsory_bytes(prob, "fwd") + prob.B * prob.H * tiles * 2 * frac * n * d * s


def _limits(prob, b):
    """Per query row i of batch b: keys [0, limit_i) pass the causal and
    key-length masks."""
    n = prob.N
    lim = np.full(n, n, dtype=np.int64)
    if prob.causal:
        lim = np.minimum(lim, np.arange(n, dtype=np.int64) + 1)
    if prob.key_lens is not None:
        lim = np.minimum(lim, max(0, min(int(prob.key_lens[b]), n)))
    return lim


def streamed_rows(prob, which, rows):
    """Rows of the other side that the backward pass ``which`` streams through
    on-chip memory, summed over its work-groups of ``rows`` rows and over every
    head: the dQ pass ('dq', work-groups of queries) reads each key that some
    query of the work-group keeps; the dK/dV pass ('dkdv', work-groups of keys)
    reads each query that keeps some key of the work-group."""
    n, bs = prob.N, prob.block_size
    bm = None if prob.block_mask is None else np.asarray(prob.block_mask) != 0
    total = 0
    for b in range(prob.B):
        lim = _limits(prob, b)
        qblk = np.arange(n) // bs
        for r0 in range(0, n, rows):
            r1 = min(n, r0 + rows)
            if which == "dq":
                if bm is None:
                    total += int(lim[r0:r1].max())   # the union of [0, limit_i)
                    continue
                # per key block, the furthest key some query of the tile keeps
                cover = np.zeros(bm.shape[1], dtype=np.int64)
                for qb in range(r0 // bs, (r1 - 1) // bs + 1):
                    m = int(lim[max(r0, qb * bs):min(r1, (qb + 1) * bs)].max())
                    cover = np.maximum(cover, np.where(bm[qb], m, 0))
                starts = np.arange(bm.shape[1], dtype=np.int64) * bs
                total += int(np.clip(cover - starts, 0, bs).sum())
            else:
                # query i keeps key j of the tile iff j < limit_i (and j's
                # mask block is kept for i's): some key iff limit_i exceeds
                # the first key of a kept block within the tile
                if bm is None:
                    total += int((lim > r0).sum())
                    continue
                keeps = np.zeros(n, dtype=bool)
                for kb in range(r0 // bs, (r1 - 1) // bs + 1):
                    keeps |= bm[qblk, kb] & (lim > max(r0, kb * bs))
                total += int(keeps.sum())
    return total * prob.H


def tiled_backward_pass_bytes(prob, which, rows):
    """HBM bytes one backward pass reads and writes when each work-group of
    ``rows`` rows reads the other side's rows it needs once (streamed_rows):
    the backward's form of the Theta(N^2 d^2 / M) re-read term, plus the
    pass's own rows.  dQ pass: Q, dO, O rows and the logsumexp read, dQ, -D
    and LSE * log2(e) written; K and V rows streamed (2 d s bytes each).  dK/dV
    pass: K and V read, dK and dV written; Q and dO rows streamed with their
    LSE * log2(e) and -D words (2 d s + 8 bytes each)."""
    s = ELEM_BYTES[prob.dtype]
    heads = prob.B * prob.H
    n, d = prob.N, prob.d
    if which == "dq":
        own = heads * (4 * n * d * s + 12 * n)
        return own + streamed_rows(prob, "dq", rows) * 2 * d * s
    own = heads * (4 * n * d * s)
    return own + streamed_rows(prob, "dkdv", rows) * (2 * d * s + 8)


# ----------------------------------------------------------------------------- inference

def kv_fill(prob, b):
    """Visible cache entries of batch b of a KvProblem (key_lens clamped)."""
    if prob.key_lens is None:
        return prob.Nk
    return max(0, min(int(prob.key_lens[b]), prob.Nk))


def kv_kept_pairs(prob):
    """Visible (query, key) pairs of a KvProblem: row i of batch b sees
    min(L, i + L - Nq + 1) keys under the bottom-right causal mask (none when
    that is negative) and all L otherwise."""
    total = 0
    i = np.arange(prob.Nq, dtype=np.int64)
    for b in range(prob.B):
        L = kv_fill(prob, b)
        per = np.clip(i + L - prob.Nq + 1, 0, L) if prob.causal else np.full(prob.Nq, L)
        total += prob.H * int(per.sum())
    return total


def kv_forward_bytes(prob, splits):
    """Algorithmic HBM bytes of the inference forward kernel: Q and the
    visible part of the K and V cache read once (further query tiles re-read
    the cache from L2), and either O and the fp32 LSE written or, with the
    key range split, the fp32 partial O and LSE of every split."""
    s = ELEM_BYTES[prob.dtype]
    heads = prob.B * prob.H
    q = heads * prob.Nq * prob.d * s
    kv = 2 * prob.H * prob.d * s * sum(kv_fill(prob, b) for b in range(prob.B))
    if splits > 1:
        out = splits * heads * prob.Nq * (prob.d + 1) * 4
    else:
        out = heads * prob.Nq * (prob.d * s + 4)
    return q + kv + out


def varlen_kept_pairs(prob):
    """Visible pairs of a packed variable-length problem: each sequence
    counted as an inference problem with its own query and key counts."""
    total = 0
    for nq, nk in zip(prob.lens_q, prob.lens_k):
        i = np.arange(int(nq), dtype=np.int64)
        L = int(nk)
        per = np.clip(i + L - int(nq) + 1, 0, L) if prob.causal else np.full(int(nq), L)
        total += prob.H * int(per.sum())
    return total
