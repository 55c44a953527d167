"""Host replay of the dK/dV pass's staging indices (fa_bwd_impl.h,
fa_bwd_dkdv_kernel): for every key tile of a head, the rows each copy into
the LDS ring touches must lie inside the head.  The pass streams query tiles
of BQ rows (64; 32 for fp32 at d = 128) past BK resident keys (128; 64 and
256 with the tile-height option of 16-bit inputs).  Its dense
interior copies tile t + 2 whole, without a row check, and each of two waves
fetches 64 LSE or D words for it; the boundary path copies any tile with
per-row checks.  The replay mirrors the kernel's loop bounds, so a change to
them that lets an unchecked copy pass the end of a head fails here."""

import itertools

import pytest


def dkdv_rows(N, BQ, causal, kend, BK=128):
    """Rows of Q/dO read by unchecked copies and rows of the LSE/D vectors
    read by the 64-lane word copies, over every key tile of one head."""
    nqt = (N + BQ - 1) // BQ
    whole_tile_rows, word_rows = [], []
    for kt in range((N + BK - 1) // BK):
        j0 = kt * BK
        t_begin = j0 // BQ if causal else 0
        t_end = nqt if j0 < kend else t_begin
        # first two tiles (and every boundary tile) go through issue(): rows
        # are checked per row, words are clamped to the head
        for t in range(t_begin, t_end):
            word_rows += [min(t * BQ + lane, N - 1) for lane in range(64)]
        lo, hi = t_end, -1
        if j0 + BK <= kend:
            lo = (j0 + BK - 1 + BQ - 1) // BQ if causal else t_begin
            hi = min(N // BQ - 3, t_end - 3)
        for t in range(t_begin, t_end):
            if lo <= t <= hi:
                qn = (t + 2) * BQ
                whole_tile_rows += list(range(qn, qn + BQ))
                word_rows += [min(qn + lane, N - 1) for lane in range(64)]
    return whole_tile_rows, word_rows


CASES = ([(BQ, causal, 128) for BQ, causal in itertools.product((32, 64), (False, True))] +
         [(64, causal, BK) for causal, BK in itertools.product((False, True), (64, 256))])


@pytest.mark.parametrize("BQ,causal,BK", CASES)
def test_dkdv_copies_stay_inside_the_head(BQ, causal, BK):
    sizes = sorted({1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 384, 511,
                    512, 513, 1000, 1024, 2048 + 32, 4096})
    for N in sizes:
        for kend in sorted({N, max(N - 1, 0), N // 2, 1, 0}):
            rows, words = dkdv_rows(N, BQ, causal, kend, BK)
            assert all(0 <= r < N for r in rows), (N, BQ, causal, kend, BK, max(rows))
            assert all(0 <= r < N for r in words), (N, BQ, causal, kend, BK)


def test_interior_runs_at_the_sizes_the_replay_checks():
    # The replay must reach the unchecked path, else it proves nothing.
    rows, _ = dkdv_rows(4096, 32, False, 4096)
    assert rows and max(rows) == 4095
    rows, _ = dkdv_rows(1024, 64, True, 1024)
    assert rows and max(rows) == 1023
    for BK in (64, 256):
        rows, _ = dkdv_rows(1024, 64, True, 1024, BK)
        assert rows and max(rows) == 1023
