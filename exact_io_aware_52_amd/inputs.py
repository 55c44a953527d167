"""Seeded synthetic inputs for tiled exact attention.

This module draws and rounds numbers; it performs none of the attention
arithmetic.  Both the HIP path (through its tests and the bench) and the fp64
oracle take their inputs from here, and from nowhere else.

Recipe (the pages fix no data; their workloads are GPT-2, BERT-large, Long
Range Arena and Path-X/Path-256 training, which only lend their attention
shapes here):

* ``numpy.random.default_rng(seed)`` draws Q, K, V, dO in that order, each as
  float32 standard normal in C order [B, H, N, d];
* every value is rounded to the compute dtype with round-to-nearest-even, so
  the float32 arrays returned hold exactly what the GPU receives;
* per-batch key lengths (key padding) come from
  ``default_rng(seed + 1_000_003).integers(lo, hi + 1, B)`` (inclusive range);
* the block mask comes from ``default_rng(seed + 2_000_003).random((nb, nb))
  < p`` with the diagonal forced to 1, nb = ceil(N / block_size).

Inference problems (``make_kv_problem``: Nq new queries against a key/value
cache of Nk entries) draw Q [B, H, Nq, d], then K and V [B, H, Nk, d], the
same way; the cache fill per batch comes from
``default_rng(seed + 1_000_003).integers(lo, hi + 1, B)``.  Cache entries past
the fill hold ordinary draws, which the method must never see.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")


def round_to_dtype(x, dtype):
    """Round float32 values to ``dtype`` (round to nearest, ties to even) and
    return them as float32 again."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Problem:
    """One attention problem: inputs, masks and the softmax scale."""
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    scale: np.float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    key_lens: Optional[np.ndarray] = None       # int32 [B]
    block_mask: Optional[np.ndarray] = None     # uint8 [nb, nb]
    block_size: int = 128
    seed: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)


def make_problem(B, H, N, d, dtype, seed, causal=False, scale=None,
                 key_len_range=None, block_keep_p=None, block_size=128, name="",
                 block_band=None, block_global=0):
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q, k, v, do = (round_to_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)
                   for _ in range(4))
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    key_lens = None
    if key_len_range is not None:
        lo, hi = key_len_range
        key_lens = np.random.default_rng(seed + 1_000_003).integers(
            lo, hi + 1, B).astype(np.int32)
    # Block mask: i.i.d. blocks kept with probability block_keep_p, the diagonal
    # always; optionally a band of block_band blocks on each side of the
    # diagonal and block_global "global" blocks (the first block rows and
    # columns kept in full).
    block_mask = None
    if block_keep_p is not None or block_band is not None:
        nb = -(-N // block_size)
        p = 0.0 if block_keep_p is None else block_keep_p
        bm = np.random.default_rng(seed + 2_000_003).random((nb, nb)) < p
        np.fill_diagonal(bm, True)
        if block_band:
            ib, jb = np.indices((nb, nb))
            bm |= np.abs(ib - jb) <= block_band
        if block_global:
            bm[:block_global, :] = True
            bm[:, :block_global] = True
        block_mask = bm.astype(np.uint8)
    return Problem(B, H, N, d, dtype, bool(causal), np.float32(scale), q, k, v, do,
                   key_lens, block_mask, block_size, seed, name)


@dataclass
class KvProblem:
    """Nq new queries against a key/value cache of Nk entries, of which the
    first key_lens[b] are filled (all Nk when key_lens is None)."""
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    scale: np.float32
    q: np.ndarray           # [B, H, Nq, d]
    k: np.ndarray           # [B, H, Nk, d]
    v: np.ndarray
    key_lens: Optional[np.ndarray] = None
    seed: int = 0
    name: str = ""


def make_kv_problem(B, H, Nq, Nk, d, dtype, seed, causal=True, scale=None, fill_range=None,
                    name=""):
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    q = round_to_dtype(rng.standard_normal((B, H, Nq, d), dtype=np.float32), dtype)
    k, v = (round_to_dtype(rng.standard_normal((B, H, Nk, d), dtype=np.float32), dtype)
            for _ in range(2))
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    key_lens = None
    if fill_range is not None:
        lo, hi = fill_range
        key_lens = np.random.default_rng(seed + 1_000_003).integers(
            lo, hi + 1, B).astype(np.int32)
    return KvProblem(B, H, Nq, Nk, d, dtype, bool(causal), np.float32(scale), q, k, v,
                     key_lens, seed, name)


# Inference workloads: one decode step of a batch of sequences against their
# caches (one new query each, fills between half and all of the capacity), and
# a chunk of 512 new queries appended to caches of the same kind.
KV_CONFIGS = {
    "kv_decode": dict(B=16, H=16, Nq=1, Nk=8192, d=128, dtype="bf16", seed=7, causal=True,
                      fill_range=(4096, 8192)),
    "kv_chunk": dict(B=4, H=16, Nq=512, Nk=8192, d=128, dtype="bf16", seed=8, causal=True,
                     fill_range=(4096, 8192)),
}


def kv_workload(name):
    return make_kv_problem(name=name, **KV_CONFIGS[name])


@dataclass
class VarlenProblem:
    """B sequences packed back to back per head: q [H, Tq, d], k and v
    [H, Tk, d]; sequence b owns rows cu_q[b] .. cu_q[b+1]-1 and
    cu_k[b] .. cu_k[b+1]-1."""
    H: int
    d: int
    dtype: str
    causal: bool
    scale: np.float32
    lens_q: np.ndarray
    lens_k: np.ndarray
    cu_q: np.ndarray        # int32 [B+1]
    cu_k: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seed: int = 0
    name: str = ""

    @property
    def B(self):
        return len(self.lens_q)


def make_varlen_problem(H, d, dtype, seed, lens_q=None, lens_k=None, len_range=None, B=None,
                        causal=True, scale=None, name=""):
    """Sequence lengths are given, or drawn from
    default_rng(seed + 1_000_003).integers(lo, hi + 1, B) (keys: the same
    lengths, self-attention, unless lens_k is given); then Q [H, Tq, d], K and
    V [H, Tk, d] are drawn from default_rng(seed) in that order."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    if lens_q is None:
        lo, hi = len_range
        lens_q = np.random.default_rng(seed + 1_000_003).integers(lo, hi + 1, B)
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = lens_q.copy() if lens_k is None else np.asarray(lens_k, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    q = round_to_dtype(rng.standard_normal((H, int(cu_q[-1]), d), dtype=np.float32), dtype)
    k, v = (round_to_dtype(rng.standard_normal((H, int(cu_k[-1]), d), dtype=np.float32), dtype)
            for _ in range(2))
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return VarlenProblem(H, d, dtype, bool(causal), np.float32(scale), lens_q, lens_k, cu_q, cu_k,
                         q, k, v, seed, name)


# Packed variable-length prefill: 16 causal sequences of 128 to 4096 tokens.
VARLEN_CONFIGS = {
    "varlen_prefill": dict(H=16, d=128, dtype="bf16", seed=9, len_range=(128, 4096), B=16,
                           causal=True),
}


def varlen_workload(name):
    return make_varlen_problem(name=name, **VARLEN_CONFIGS[name])


# The five workloads.  Shapes follow GPT-2-small, BERT-large, long-context
# (Long Range Arena / Path-X lengths) and long-context block-sparse attention.
LONG_POINTS = [(n, d) for n in (2048, 4096, 8192, 16384) for d in (64, 128)]
# Longer-context block-sparse attention with a structured pattern: a local
# band (one block on each side of the diagonal), one global block row and
# column, and i.i.d. blocks with probability 1/32.
SPARSE_LONG_N = (32768, 65536)


def config(name, n=None, d=None):
    """Return the keyword arguments of ``make_problem`` for a named workload."""
    if name == "tiny":
        return dict(B=1, H=2, N=128, d=64, dtype="fp32", seed=1, causal=False,
                    scale=1 / 8, name=name)
    if name == "gpt2_small":
        return dict(B=8, H=12, N=1024, d=64, dtype="bf16", seed=2, causal=True,
                    scale=1 / 8, name=name)
    if name == "bert_large_padded":
        return dict(B=16, H=16, N=512, d=64, dtype="fp16", seed=3, causal=False,
                    scale=1 / 8, key_len_range=(128, 512), name=name)
    if name == "long_causal":
        idx = LONG_POINTS.index((n, d))
        return dict(B=2, H=8, N=n, d=d, dtype="bf16", seed=4 + 10 * idx, causal=True,
                    scale=1 / np.sqrt(d), name=f"long_causal_N{n}_d{d}")
    if name == "block_sparse":
        return dict(B=1, H=8, N=16384, d=64, dtype="bf16", seed=5, causal=False,
                    scale=1 / 8, block_keep_p=1 / 8, block_size=128, name=name)
    if name == "block_sparse_long":
        idx = SPARSE_LONG_N.index(n)
        return dict(B=1, H=8, N=n, d=64, dtype="bf16", seed=6 + 10 * idx, causal=False,
                    scale=1 / 8, block_keep_p=1 / 32, block_band=1, block_global=1,
                    block_size=128, name=f"block_sparse_long_N{n}")
    raise KeyError(name)


def workload(name, n=None, d=None):
    return make_problem(**config(name, n, d))
