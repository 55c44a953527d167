"""CPU tests of the C ABI: libfa.so loads, exports every function include/fa.h
declares, and rejects bad arguments on the host before any HIP call (so no
GPU is needed).  Pointers passed here are never dereferenced: each call is
built to fail validation."""

import os
import re

import numpy as np
import pytest

from exact_io_aware_52_amd import _binding, build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.library_path()):
        build_lib.build()
    return _binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("fa_forward", "fa_forward_blocksparse", "fa_backward",
                 "fa_backward_workspace_bytes", "fa_status_string", "fa_last_error_detail"):
        assert want in names


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


FAKE = 0x10000           # 16-byte aligned, never dereferenced
BAD_ALIGN = 0x10002


def fwd(lib, q=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=64, d=64, scale=0.125, causal=0,
        key_lens=None, dtype=2):
    return lib.fa_forward(q, FAKE, FAKE, o, lse, B, H, N, d, scale, causal, key_lens, dtype, None)


def detail(lib):
    return lib.fa_last_error_detail().decode()


def test_forward_validation(lib):
    assert fwd(lib, q=None) == _binding.FA_ERR_INVALID_ARG
    assert "q is NULL" in detail(lib)
    assert fwd(lib, q=BAD_ALIGN) == _binding.FA_ERR_INVALID_ARG
    assert "aligned" in detail(lib)
    assert fwd(lib, lse=FAKE + 2) == _binding.FA_ERR_INVALID_ARG
    assert fwd(lib, d=96) == _binding.FA_ERR_UNSUPPORTED
    assert fwd(lib, d=32) == _binding.FA_ERR_UNSUPPORTED
    assert fwd(lib, B=-1) == _binding.FA_ERR_INVALID_ARG
    assert fwd(lib, N=-5) == _binding.FA_ERR_INVALID_ARG
    assert fwd(lib, dtype=7) == _binding.FA_ERR_INVALID_ARG
    assert fwd(lib, scale=-1.0) == _binding.FA_ERR_UNSUPPORTED
    assert fwd(lib, scale=float("nan")) == _binding.FA_ERR_INVALID_ARG
    assert fwd(lib, scale=float("inf")) == _binding.FA_ERR_INVALID_ARG
    assert fwd(lib, key_lens=FAKE + 1, q=None) == _binding.FA_ERR_INVALID_ARG
    assert fwd(lib, B=1 << 20, H=1 << 10, N=1 << 20) == _binding.FA_ERR_INVALID_ARG


def test_empty_problems_are_noops(lib):
    # Nothing to compute: OK without touching any pointer.
    assert fwd(lib, q=None, o=None, lse=None, N=0) == _binding.FA_OK
    assert fwd(lib, q=None, o=None, lse=None, B=0) == _binding.FA_OK
    assert lib.fa_backward(None, None, None, None, None, None, None, None, None, 1, 0, 10, 64,
                           0.1, 0, None, None, 128, 2, None, 0, None) == _binding.FA_OK
    assert lib.fa_backward_workspace_bytes(0, 4, 10, 64) == 0


def test_blocksparse_validation(lib):
    f = lib.fa_forward_blocksparse
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 256, 64, 0.1, 0, None, None, 128, 2, None) \
        == _binding.FA_ERR_INVALID_ARG
    assert "block_mask" in detail(lib)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 256, 64, 0.1, 0, None, FAKE, 64, 2, None) \
        == _binding.FA_ERR_UNSUPPORTED
    # one mask row is cached on chip: at most 1024 blocks (N <= 131072)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 131073, 64, 0.1, 0, None, FAKE, 128, 2, None) \
        == _binding.FA_ERR_UNSUPPORTED
    assert "1024" in detail(lib)


def test_blocksparse_split_validation(lib):
    f = lib.fa_forward_blocksparse_split

    def call(N=256, chunk=128, ws=FAKE, ws_bytes=0):
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, N, 64, 0.1, 0, None, FAKE, 128, chunk, 2, ws,
                 ws_bytes, None)

    for chunk in (0, -64, 100, 65):
        assert call(chunk=chunk) == _binding.FA_ERR_UNSUPPORTED
        assert "key_chunk" in detail(lib)
    assert call(N=65600, chunk=64) == _binding.FA_ERR_UNSUPPORTED     # 1025 splits
    assert "1024" in detail(lib)
    need = lib.fa_forward_blocksparse_split_workspace_bytes(1, 2, 256, 64, 128)
    # 2 splits x 2 heads x 256 rows: fp32 O (d = 64), then fp32 LSE, each rounded to 256 bytes
    assert need == 2 * 2 * 256 * 64 * 4 + 2 * 2 * 256 * 4
    assert call(ws=None) == _binding.FA_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == _binding.FA_ERR_WORKSPACE
    assert str(need) in detail(lib)
    assert call(ws=BAD_ALIGN, ws_bytes=need) == _binding.FA_ERR_INVALID_ARG
    ws_bytes = lib.fa_forward_blocksparse_split_workspace_bytes
    assert ws_bytes(1, 2, 256, 64, 256) == 0        # one split: no workspace
    assert ws_bytes(1, 2, 256, 64, 100) == 0        # invalid chunk
    assert ws_bytes(3, 1, 300, 128, 128) == (3 * 3 * 300 * 128 * 4) + \
        ((3 * 3 * 300 * 4 + 255) // 256 * 256)


def bwd(lib, ws=FAKE, ws_bytes=1 << 30, dq=FAKE, bm=None, bs=128, d=64, N=100):
    return lib.fa_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, 2, 3, N, d, 0.1, 1,
                           None, bm, bs, 1, ws, ws_bytes, None)


def test_backward_validation(lib):
    need = lib.fa_backward_workspace_bytes(2, 3, 100, 64)
    assert need >= 2 * 2 * 3 * 100 * 4 and need % 256 == 0
    assert bwd(lib, ws=None) == _binding.FA_ERR_WORKSPACE
    assert bwd(lib, ws_bytes=need - 1) == _binding.FA_ERR_WORKSPACE
    assert "needed" in detail(lib)
    assert bwd(lib, ws=FAKE + 8) == _binding.FA_ERR_INVALID_ARG
    assert bwd(lib, dq=None) == _binding.FA_ERR_INVALID_ARG
    assert bwd(lib, dq=BAD_ALIGN) == _binding.FA_ERR_INVALID_ARG
    assert bwd(lib, bm=FAKE, bs=256) == _binding.FA_ERR_UNSUPPORTED
    assert bwd(lib, d=80) == _binding.FA_ERR_UNSUPPORTED


def bwd_ex(lib, dq_rows, dkdv_rows, dtype=1, gdtype=None, bm=None, dq=FAKE, B=2, kg=0):
    return lib.fa_backward_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, B, 3, 100, 64,
                              0.1, 1, None, bm, 128, dtype, dtype if gdtype is None else gdtype,
                              dq_rows, dkdv_rows, kg, FAKE, 1 << 30, None)


def test_backward_ex_tile_rows_validation(lib):
    for bad in (32, 96, 512, -128, 1):
        assert bwd_ex(lib, bad, 0) == _binding.FA_ERR_UNSUPPORTED, bad
        assert "dq_rows" in detail(lib)
        assert bwd_ex(lib, 0, bad) == _binding.FA_ERR_UNSUPPORTED, bad
        assert "dkdv_rows" in detail(lib)
    # every height passes for 16-bit inputs and gradients (the call then
    # fails on the null dq, before any launch)
    for dtype in (1, 2):
        for a in (0, 64, 128, 256):
            for b in (0, 64, 128, 256):
                assert bwd_ex(lib, a, b, dtype=dtype, dq=None) == _binding.FA_ERR_INVALID_ARG
                assert "dq is NULL" in detail(lib)
    # 64 and 256 rows: not for float32 inputs or float32 gradients
    for a, b in ((64, 0), (0, 256)):
        assert bwd_ex(lib, a, b, dtype=0) == _binding.FA_ERR_UNSUPPORTED
        assert bwd_ex(lib, a, b, dtype=2, gdtype=0) == _binding.FA_ERR_UNSUPPORTED
        assert "16-bit" in detail(lib)
    assert bwd_ex(lib, 128, 0, dtype=0, dq=None) == _binding.FA_ERR_INVALID_ARG
    # 256 rows span two 128-token mask blocks: not with a block mask
    assert bwd_ex(lib, 256, 0, bm=FAKE) == _binding.FA_ERR_UNSUPPORTED
    assert bwd_ex(lib, 0, 256, bm=FAKE) == _binding.FA_ERR_UNSUPPORTED
    assert "block mask" in detail(lib)
    assert bwd_ex(lib, 64, 64, bm=FAKE, dq=None) == _binding.FA_ERR_INVALID_ARG
    # empty problem: the sizes are still checked, nothing else is
    assert bwd_ex(lib, 96, 0, B=0) == _binding.FA_ERR_UNSUPPORTED
    assert bwd_ex(lib, 256, 64, B=0, dq=None) == _binding.FA_OK


def test_backward_ex_key_groups_validation(lib):
    for bad in (-1, 3):
        assert bwd_ex(lib, 0, 0, kg=bad) == _binding.FA_ERR_UNSUPPORTED
        assert "key_groups" in detail(lib)
    for dtype in (1, 2):
        for kg in (0, 1, 2):
            for gd in (dtype, 0):  # 16-bit or float32 gradients
                assert bwd_ex(lib, 0, 128, dtype=dtype, gdtype=gd, kg=kg, dq=None) == \
                    _binding.FA_ERR_INVALID_ARG
    assert bwd_ex(lib, 0, 0, dtype=0, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert bwd_ex(lib, 0, 0, bm=FAKE, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert bwd_ex(lib, 64, 0, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert bwd_ex(lib, 0, 256, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert "key_groups=2" in detail(lib)
    # other heights keep one group when the library chooses
    assert bwd_ex(lib, 64, 256, kg=0, dq=None) == _binding.FA_ERR_INVALID_ARG
    kg_for = lib.fa_backward_key_groups_for
    assert kg_for(2, 8, 4096, 64, 2, 0) == 2 and kg_for(2, 8, 4096, 128, 1, 0) == 1
    assert kg_for(2, 8, 2048, 128, 1, 0) == 2 and kg_for(2, 8, 2049, 128, 2, 0) == 1
    assert kg_for(2, 8, 4097, 64, 2, 0) == 1 and kg_for(8, 12, 1024, 64, 2, 0) == 1
    assert kg_for(2, 8, 4096, 64, 0, 0) == 1 and kg_for(2, 8, 4096, 64, 2, 1) == 1


def test_backward_blocksparse_split_validation(lib):
    f = lib.fa_backward_blocksparse_split

    def call(N=1000, chunk=2, ws=FAKE, ws_bytes=1 << 40, bm=FAKE, dtype=2, d=64):
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 3, N, d, 0.1, 0, None,
                 bm, 128, chunk, dtype, ws, ws_bytes, None)

    for chunk in (0, -1):
        assert call(chunk=chunk) == _binding.FA_ERR_UNSUPPORTED
        assert "chunk_blocks" in detail(lib)
    assert call(N=131072 + 128, chunk=1) == _binding.FA_ERR_UNSUPPORTED  # 1025 items per row
    assert "1024" in detail(lib)
    assert call(dtype=0) == _binding.FA_ERR_UNSUPPORTED                   # float32 inputs
    assert call(bm=None) == _binding.FA_ERR_INVALID_ARG
    ws_bytes = lib.fa_backward_blocksparse_split_workspace_bytes
    base = lib.fa_backward_workspace_bytes(2, 3, 1000, 64)
    # 8 mask blocks per row in items of 2: 4 items; three fp32 [4][2*3][1000][64] arrays,
    # then int32 counts [2][8] and the transposed 8 x 8 mask, each rounded to 256 bytes
    part = 4 * 2 * 3 * 1000 * 64 * 4
    masks = 256 + 256
    assert ws_bytes(2, 3, 1000, 64, 2) == base + 3 * part + masks
    assert ws_bytes(2, 3, 1000, 64, 8) == base + 3 * (part // 4) + masks   # one item
    assert ws_bytes(2, 3, 1000, 64, 0) == 0
    need = ws_bytes(2, 3, 1000, 64, 2)
    assert call(ws=None) == _binding.FA_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == _binding.FA_ERR_WORKSPACE
    assert str(need) in detail(lib)
    assert call(ws=BAD_ALIGN, ws_bytes=need) == _binding.FA_ERR_INVALID_ARG
    assert call(d=96, ws_bytes=need) == _binding.FA_ERR_UNSUPPORTED


def test_status_strings(lib):
    assert lib.fa_status_string(0) == b"FA_OK"
    assert lib.fa_status_string(3) == b"FA_ERR_WORKSPACE"
    assert lib.fa_status_string(99) == b"FA_ERR_UNKNOWN"


def test_backward_pass_validation(lib):
    # The two passes check only the pointers they use: the dQ pass needs o,
    # lse, dq (not dk, dv); the dK/dV pass needs dk, dv (not o, lse, dq).
    need = lib.fa_backward_workspace_bytes(2, 3, 100, 64)

    def dq_pass(o=FAKE, lse=FAKE, dq=FAKE, ws=FAKE, ws_bytes=need):
        return lib.fa_backward_dq(FAKE, FAKE, FAKE, o, FAKE, lse, dq, 2, 3, 100, 64, 0.1, 1,
                                  None, None, 128, 2, 0, ws, ws_bytes, None)

    def kv_pass(dk=FAKE, dv=FAKE, ws=FAKE, ws_bytes=need, q=FAKE):
        return lib.fa_backward_dkdv(q, FAKE, FAKE, FAKE, dk, dv, 2, 3, 100, 64, 0.1, 1, None,
                                    None, 128, 2, 0, ws, ws_bytes, None)

    for bad in (dict(o=None), dict(lse=None), dict(dq=None), dict(dq=BAD_ALIGN), dict(ws=None),
                dict(ws_bytes=need - 1)):
        assert dq_pass(**bad) != _binding.FA_OK, bad
    for bad in (dict(dk=None), dict(dv=BAD_ALIGN), dict(ws=None), dict(ws_bytes=need - 1),
                dict(q=None)):
        assert kv_pass(**bad) != _binding.FA_OK, bad
    assert "q is NULL" in detail(lib)


def test_no_process_wide_settings(lib):
    # The library keeps no settings between calls: no setter or timing hook
    # is exported.
    for gone in ("fa_set_forward_block_rows", "fa_get_forward_block_rows", "fa_timing_enable",
                 "fa_timing_read", "fa_kernel_name"):
        assert not hasattr(lib, gone), gone


def kv(lib, q=FAKE, k=FAKE, B=2, H=3, Nq=1, Nk=1000, d=64, dtype=2, ws=FAKE, ws_bytes=1 << 30,
       key_lens=None):
    return lib.fa_forward_kv(q, k, FAKE, FAKE, FAKE, B, H, Nq, Nk, d, 0.1, 1, key_lens, dtype,
                             ws, ws_bytes, None)


def test_forward_kv_validation(lib):
    W = lib.fa_forward_kv_workspace_bytes
    # decode against a long cache splits the key range: it needs a workspace
    need = W(2, 3, 1, 1000, 64, 2)
    assert need > 0 and need % 256 == 0
    assert W(2, 3, 1, 1000, 64, 2) == need                      # deterministic plan
    # enough query tiles already fill the chip: no split, no workspace
    assert W(8, 16, 1024, 1024, 64, 2) == 0
    assert W(1, 1, 1, 100, 64, 2) == 0                         # too few keys to split
    assert W(0, 3, 1, 1000, 64, 2) == 0 and W(2, 3, 1, 0, 64, 2) == 0
    assert kv(lib, Nk=-1) == _binding.FA_ERR_INVALID_ARG
    assert kv(lib, d=96) == _binding.FA_ERR_UNSUPPORTED
    assert kv(lib, dtype=7) == _binding.FA_ERR_INVALID_ARG
    assert kv(lib, q=None) == _binding.FA_ERR_INVALID_ARG
    assert kv(lib, k=None) == _binding.FA_ERR_INVALID_ARG
    assert kv(lib, ws=None) == _binding.FA_ERR_WORKSPACE
    assert "workspace" in detail(lib)
    assert kv(lib, ws_bytes=need - 1) == _binding.FA_ERR_WORKSPACE
    assert kv(lib, ws=BAD_ALIGN) == _binding.FA_ERR_INVALID_ARG
    assert kv(lib, key_lens=0x10001) == _binding.FA_ERR_INVALID_ARG
    # empty problems return before touching any pointer
    assert kv(lib, q=None, Nq=0) == _binding.FA_OK
    assert kv(lib, q=None, B=0) == _binding.FA_OK


def varlen(lib, q=FAKE, k=FAKE, cq=FAKE, ck=FAKE, B=3, H=2, Tq=100, Tk=100, mq=50, d=64, dtype=2):
    return lib.fa_forward_varlen(q, k, FAKE, FAKE, FAKE, cq, ck, B, H, Tq, Tk, mq, d, 0.1, 1,
                                 dtype, None)


def test_forward_varlen_validation(lib):
    assert varlen(lib, Tk=-1) == _binding.FA_ERR_INVALID_ARG
    assert varlen(lib, mq=-2) == _binding.FA_ERR_INVALID_ARG
    assert varlen(lib, mq=101) == _binding.FA_ERR_INVALID_ARG
    assert "max_seqlen_q" in detail(lib)
    assert varlen(lib, cq=None) == _binding.FA_ERR_INVALID_ARG
    assert varlen(lib, ck=0x10002) == _binding.FA_ERR_INVALID_ARG
    assert varlen(lib, k=None) == _binding.FA_ERR_INVALID_ARG
    assert varlen(lib, d=80) == _binding.FA_ERR_UNSUPPORTED
    # empty problems return before touching any pointer
    assert varlen(lib, q=None, cq=None, Tq=0, mq=0) == _binding.FA_OK
    assert varlen(lib, q=None, cq=None, B=0) == _binding.FA_OK
    assert varlen(lib, q=None, cq=None, mq=0) == _binding.FA_OK


def fwd_ex(lib, rows, bm=None, N=256, q=FAKE, keys=0, dtype=2, d=64, kg=0):
    return lib.fa_forward_ex(q, FAKE, FAKE, FAKE, FAKE, 1, 1, N, d, 0.1, 0, None, bm, 128, rows,
                             keys, kg, dtype, None)


def test_forward_ex_block_rows_validation(lib):
    for bad in (32, 96, 512, -128, 1):
        assert fwd_ex(lib, bad) == _binding.FA_ERR_UNSUPPORTED, bad
        assert "block_rows" in detail(lib)
    # valid heights pass the row check (and then fail on the null q, before
    # any launch)
    for rows in (0, 64, 128, 256):
        assert fwd_ex(lib, rows, q=None) == _binding.FA_ERR_INVALID_ARG
        assert "q is NULL" in detail(lib)
    # 256-row tiles span two 128-token mask blocks: not with a block mask
    assert fwd_ex(lib, 256, bm=FAKE) == _binding.FA_ERR_UNSUPPORTED
    assert "256" in detail(lib)
    assert fwd_ex(lib, 128, bm=FAKE, q=None) == _binding.FA_ERR_INVALID_ARG
    # a block mask too long for the on-chip row cache
    assert fwd_ex(lib, 0, bm=FAKE, N=131073) == _binding.FA_ERR_UNSUPPORTED
    # empty problem: nothing checked beyond the sizes, nothing launched
    assert fwd_ex(lib, 64, N=0, q=None) == _binding.FA_OK
    # float32 at d = 128: at most 128 rows per tile

    def f32(rows, q=FAKE):
        return lib.fa_forward_ex(q, FAKE, FAKE, FAKE, FAKE, 1, 1, 256, 128, 0.1, 0, None, None,
                                 128, rows, 0, 0, 0, None)
    assert f32(256) == _binding.FA_ERR_UNSUPPORTED
    assert "float32" in detail(lib)
    assert f32(128, q=None) == _binding.FA_ERR_INVALID_ARG


def test_forward_ex_block_keys_validation(lib):
    for bad in (16, 48, 96, 256, -64, 1):
        assert fwd_ex(lib, 0, keys=bad) == _binding.FA_ERR_UNSUPPORTED, bad
        assert "block_keys" in detail(lib)
    # every width passes with 128-row tiles (or 0 rows), 16-bit types, dense
    # or block-sparse; the call then fails on the null q, before any launch
    for dtype in (1, 2):
        for d in (64, 128):
            for keys in (0, 32, 64, 128):
                for rows in (0, 128):
                    assert fwd_ex(lib, rows, keys=keys, dtype=dtype, d=d, q=None) == \
                        _binding.FA_ERR_INVALID_ARG, (dtype, d, keys, rows)
                    assert "q is NULL" in detail(lib)
            assert fwd_ex(lib, 128, bm=FAKE, keys=128, dtype=dtype, d=d, q=None) == \
                _binding.FA_ERR_INVALID_ARG
    # other widths come with 128-row tiles only
    for rows in (64, 256):
        assert fwd_ex(lib, rows, keys=32) == _binding.FA_ERR_UNSUPPORTED
        assert "128 rows only" in detail(lib)
        assert fwd_ex(lib, rows, keys=64, q=None) == _binding.FA_ERR_INVALID_ARG  # the default
    # float32 keeps its 32-key tiles
    for keys in (64, 128):
        assert fwd_ex(lib, 0, keys=keys, dtype=0) == _binding.FA_ERR_UNSUPPORTED
        assert "float32" in detail(lib)
    assert fwd_ex(lib, 0, keys=32, dtype=0, q=None) == _binding.FA_ERR_INVALID_ARG
    # empty problem: the widths are still checked first
    assert fwd_ex(lib, 0, keys=96, N=0, q=None) == _binding.FA_ERR_UNSUPPORTED
    assert fwd_ex(lib, 0, keys=128, N=0, q=None) == _binding.FA_OK


def test_forward_ex_key_groups_validation(lib):
    for bad in (-1, 3, 4):
        assert fwd_ex(lib, 0, kg=bad) == _binding.FA_ERR_UNSUPPORTED, bad
        assert "key_groups" in detail(lib)
    # 1 and 2 pass for 16-bit dense problems with 128-row tiles of 64 keys
    for dtype in (1, 2):
        for d in (64, 128):
            for kg in (0, 1, 2):
                for rows in (0, 128):
                    for keys in (0, 64):
                        assert fwd_ex(lib, rows, keys=keys, dtype=dtype, d=d, kg=kg, q=None) == \
                            _binding.FA_ERR_INVALID_ARG
                        assert "q is NULL" in detail(lib)
    # two key groups: not for float32, block masks, other heights or widths
    assert fwd_ex(lib, 0, dtype=0, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert fwd_ex(lib, 0, bm=FAKE, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert fwd_ex(lib, 64, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert fwd_ex(lib, 256, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert fwd_ex(lib, 0, keys=32, kg=2) == _binding.FA_ERR_UNSUPPORTED
    assert "key_groups=2" in detail(lib)
    assert fwd_ex(lib, 0, dtype=0, kg=1, q=None) == _binding.FA_ERR_INVALID_ARG


def test_forward_key_groups_automatic(lib):
    # two key groups for 16-bit dense grids of at most 512 128-row tiles
    kg_for = lib.fa_forward_key_groups_for
    assert kg_for(8, 12, 1024, 64, 2, 0) == 1      # 768 tiles
    assert kg_for(2, 8, 4096, 64, 2, 0) == 2       # 512
    assert kg_for(2, 8, 4097, 64, 1, 0) == 1       # 528
    assert kg_for(2, 8, 2048, 64, 1, 0) == 2       # 256
    assert kg_for(2, 8, 8192, 64, 2, 0) == 1       # 1024
    assert kg_for(2, 8, 16384, 64, 2, 0) == 1      # 2048
    assert kg_for(2, 8, 4096, 128, 2, 0) == 2      # d = 128, 128-row tiles
    assert kg_for(2, 8, 4096, 64, 0, 0) == 1       # fp32
    assert kg_for(2, 8, 4096, 64, 2, 1) == 1       # block mask


def test_forward_block_rows_automatic(lib):
    # 256-row tiles only for 16-bit d=128 dense problems with at least 512
    # work-groups of 256 rows; 128 otherwise
    rows_for = lib.fa_forward_block_rows_for
    assert rows_for(2, 8, 16384, 128, 2, 0) == 256     # 1024 work-groups
    assert rows_for(2, 8, 8192, 128, 1, 0) == 256      # 512
    assert rows_for(2, 8, 7937, 128, 2, 0) == 256      # 16 x 32 (ragged last tile)
    assert rows_for(2, 8, 7936, 128, 2, 0) == 128      # 16 x 31 = 496
    assert rows_for(2, 8, 4096, 128, 2, 0) == 128      # 256
    assert rows_for(2, 8, 16384, 64, 2, 0) == 128      # d = 64
    assert rows_for(2, 8, 16384, 128, 0, 0) == 128     # fp32
    assert rows_for(2, 8, 16384, 128, 2, 1) == 128     # block-sparse


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(Exception):
        _binding.fa_forward(q, q, q)          # no silent CPU fallback


def test_varlen_binding_checks_max_seqlen():
    # A sequence longer than max_seqlen_q would be left partly unwritten by
    # the kernel's grid: the binding refuses it when the prefix sums are on
    # the host (before any device work).
    import torch
    q = torch.zeros(2, 300, 64)
    cu = np.array([0, 100, 300], np.int32)
    with pytest.raises(ValueError, match="max_seqlen_q"):
        _binding.fa_forward_varlen(q, q, q, cu, cu, 150)
    with pytest.raises(ValueError, match="non-decreasing"):
        _binding.fa_forward_varlen(q, q, q, np.array([0, 200, 100], np.int32), cu, 300)
