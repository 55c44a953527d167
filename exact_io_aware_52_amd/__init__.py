"""Tiled exact attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fa.h``); this package only marshals torch tensors
(device memory and the current stream) into those calls.

    from exact_io_aware_52_amd import fa_forward, fa_backward, fa_forward_blocksparse
    from exact_io_aware_52_amd import fa_forward_kv     # inference: Nq queries, Nk cache
"""

from ._binding import (  # noqa: F401
    FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP,
    FaError, library_path, load_library, fa_forward, fa_forward_ex, fa_forward_blocksparse,
    fa_forward_blocksparse_split, fa_forward_blocksparse_split_workspace_bytes, fa_backward,
    fa_backward_ex, fa_backward_dq, fa_backward_dkdv, fa_backward_workspace_bytes,
    fa_backward_noalloc, fa_backward_noalloc_max_rows,
    fa_forward_block_rows_for, fa_forward_key_groups_for, fa_backward_key_groups_for,
    fa_backward_blocksparse_split, fa_backward_blocksparse_split_workspace_bytes,
    fa_forward_kv, fa_forward_kv_workspace_bytes, fa_forward_varlen,
)
