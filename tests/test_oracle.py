"""CPU tests of the fp64 oracle: its pins, and a mutation test showing that
the pins catch mistakes planted in a copy of the oracle."""

import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as oracle_attention
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_attention)


# Each mutation plants one plausible slip in the oracle's source text.
MUTATIONS = {
    "drop_D_term": ("ds = p * (dp - d_row[:, None])", "ds = p * dp"),
    "flip_dS_sign": ("ds = p * (dp - d_row[:, None])", "ds = p * (d_row[:, None] - dp)"),
    "dQ_without_scale": ("dq[r0:r1] = scale * (ds @ k)", "dq[r0:r1] = (ds @ k)"),
    "dK_untransposed": ("dk += scale * (ds.T @ q[r0:r1])", "dk += scale * (ds @ q[r0:r1])"),
    "dV_untransposed": ("dv += p.T @ do[r0:r1]", "dv += p @ do[r0:r1]"),
    "dP_wrong_operand": ("dp = do[r0:r1] @ v.T", "dp = do[r0:r1] @ k.T"),
    "scores_without_scale": ("s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "causal_strict": ("vis &= j <= i\n", "vis &= j < i\n"),
    "padding_off_by_one": ("vis &= j < int(key_len)", "vis &= j <= int(key_len)"),
    "block_mask_transposed": ("bm[i // block_size, j // block_size]",
                              "bm[j // block_size, i // block_size]"),
    "lse_without_max": ("m + np.log(l_safe)", "np.log(l_safe)"),
    "D_from_dO_only": ("d_row = (do[r0:r1] * o).sum(axis=1)", "d_row = do[r0:r1].sum(axis=1)"),
    "softmax_over_queries": ("p = ex / l_safe[:, None]", "p = ex / ex.sum(axis=0)[None, :]"),
    "rows_drop_D_term": ("ds_r = p_r * (dp_r - d_r[:, None])", "ds_r = p_r * dp_r"),
    "rows_dQ_wrong_operand": ("scale * (ds_r @ k)", "scale * (ds_r @ q)"),
    "rows_mask_ignores_rows": ("i = (np.arange(n) if rows is None else np.asarray(rows))[:, None]",
                               "i = np.arange(n)[:len(rows) if rows is not None else n, None]"),
    "kv_causal_top_left": ("vis &= j <= i + (L - nq)", "vis &= j <= i"),
    "kv_causal_strict": ("vis &= j <= i + (L - nq)", "vis &= j < i + (L - nq)"),
    "kv_shift_from_capacity": ("vis &= j <= i + (L - nq)", "vis &= j <= i + (nk - nq)"),
    "kv_fill_ignored": ("vis = np.broadcast_to(j < L, (nq, nk)).copy()",
                        "vis = np.ones((nq, nk), dtype=bool)"),
    "kv_fill_unclamped": ("L = nk if key_len is None else min(max(int(key_len), 0), nk)",
                          "L = nk if key_len is None else int(key_len)"),
    "varlen_keys_from_query_offsets": ("k0, k1 = int(cu_k[b]), int(cu_k[b + 1])",
                                       "k0, k1 = int(cu_q[b]), int(cu_q[b + 1])"),
    "varlen_end_off_by_one": ("q0, q1 = int(cu_q[b]), int(cu_q[b + 1])",
                              "q0, q1 = int(cu_q[b]), int(cu_q[b + 1]) - 1"),
    "varlen_keys_of_next_sequence": ("k[h, k0:k1], v[h, k0:k1]", "k[h, k0:k1], v[h, k1:k1 + k1 - k0]"),
}


def _mutant(old, new):
    src = open(oracle_attention.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mutant = _mutant(*MUTATIONS[name])
    caught = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mutant)
            except Exception:           # AssertionError, or a shape error
                caught.append(pin.__name__)
    assert caught, f"no pin detects mutation {name}"


def test_package_exports():
    assert set(oracle.__all__) >= {"forward", "backward", "visibility"}


def test_oracle_not_imported_by_product():
    """The product package must not reference the oracle anywhere."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "exact_io_aware_52_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h", ".hpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
