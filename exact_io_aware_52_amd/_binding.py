"""ctypes binding of libfa.so: same entry-point names as the C ABI.

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the attention computation runs in the library's
kernels.  There is no fallback: if libfa.so is missing or a call fails, an
exception is raised.
"""

import ctypes
import math
import os

import numpy as np
import torch

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_LIB = None


class FaError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn} failed: {_status_name(status)}: {detail}")


def library_path():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")


def load_library():
    """Load libfa.so (once) and declare the C signatures."""
    global _LIB
    if _LIB is None:
        _LIB = open_library(library_path())
    return _LIB


def open_library(path):
    """Load a build of the library (libfa.so, or the race-check build
    libfa_serial.so) with the C signatures declared; raises if it is missing."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m exact_io_aware_52_amd.build_lib`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, I, P]
    lib.fa_forward_blocksparse.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, P, I, I, P]
    lib.fa_forward_blocksparse_split.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, P, I, I, I,
                                                 P, Z, P]
    lib.fa_forward_blocksparse_split_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_forward_blocksparse_split_workspace_bytes.restype = Z
    lib.fa_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, I, P, Z, P]
    lib.fa_backward_ex.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, I, I, I,
                                   I, I, P, Z, P]
    lib.fa_backward_key_groups_for.argtypes = [I, I, I, I, I, I]
    lib.fa_backward_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, I,
                                        P]
    lib.fa_backward_noalloc_max_rows.argtypes = []
    lib.fa_backward_noalloc_max_rows.restype = Z
    lib.fa_backward_dq.argtypes = [P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, I, I, P, Z, P]
    lib.fa_backward_dkdv.argtypes = [P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, I, I, P, Z, P]
    lib.fa_forward_ex.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, P, I, I, I, I, I, P]
    lib.fa_forward_key_groups_for.argtypes = [I, I, I, I, I, I]
    lib.fa_backward_blocksparse_split.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I,
                                                  P, P, I, I, I, P, Z, P]
    lib.fa_backward_blocksparse_split_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_backward_blocksparse_split_workspace_bytes.restype = Z
    lib.fa_backward_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_backward_workspace_bytes.restype = Z
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error_detail.argtypes = []
    lib.fa_last_error_detail.restype = ctypes.c_char_p
    lib.fa_forward_block_rows_for.argtypes = [I, I, I, I, I, I]
    lib.fa_forward_kv.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, I, P, Z, P]
    lib.fa_forward_kv_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.fa_forward_kv_workspace_bytes.restype = Z
    lib.fa_forward_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P]
    for fn in (lib.fa_forward, lib.fa_forward_blocksparse, lib.fa_forward_blocksparse_split,
               lib.fa_forward_ex, lib.fa_backward, lib.fa_backward_ex, lib.fa_backward_dq,
               lib.fa_backward_dkdv, lib.fa_backward_noalloc,
               lib.fa_forward_block_rows_for, lib.fa_forward_key_groups_for,
               lib.fa_backward_key_groups_for, lib.fa_forward_kv, lib.fa_forward_varlen):
        fn.restype = I
    return lib


def _status_name(status):
    return load_library().fa_status_string(int(status)).decode()


def _check(fn, status):
    if status != FA_OK:
        raise FaError(fn, status, load_library().fa_last_error_detail().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(q, k, v):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device (the library has no CPU path)")
    return q.shape


def _like(name, t, ref, shape=None, dtype=None):
    """Check a caller-supplied tensor: device, shape, dtype, contiguity."""
    if t.device != ref.device:
        raise ValueError(f"{name} must be on {ref.device}")
    if tuple(t.shape) != tuple(ref.shape if shape is None else shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}")
    if t.dtype != (ref.dtype if dtype is None else dtype):
        raise ValueError(f"{name} has dtype {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _lens(key_lens, B, device):
    if key_lens is None:
        return None
    kl = torch.as_tensor(key_lens).to(device=device, dtype=torch.int32).contiguous()
    if kl.shape != (B,):
        raise ValueError("key_lens must have shape [B]")
    return kl


def _mask(block_mask, N, block_size, device):
    if block_mask is None:
        return None
    bm = torch.as_tensor(block_mask).to(device=device, dtype=torch.uint8).contiguous()
    nb = -(-N // int(block_size)) if block_size > 0 else -1
    if tuple(bm.shape) != (nb, nb):
        raise ValueError(f"block_mask must have shape ({nb}, {nb}) for N={N}, "
                         f"block_size={block_size}")
    return bm


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def _forward(name, q, k, v, scale, causal, key_lens, block_mask, block_size, o, lse,
             block_rows=0, block_keys=0, key_groups=0):
    lib = load_library()
    B, H, N, d = _shape(q, k, v)
    o = torch.empty_like(q) if o is None else _like("o", o, q)
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _like("lse", lse, q, (B, H, N), torch.float32))
    kl = _lens(key_lens, B, q.device)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
            _scale(scale, d), int(bool(causal)), _ptr(kl)]
    if name in ("fa_forward_blocksparse", "fa_forward_ex"):
        bm = _mask(block_mask, N, block_size, q.device)
        args += [_ptr(bm), int(block_size)]
    if name == "fa_forward_ex":
        args += [int(block_rows), int(block_keys), int(key_groups)]
    args += [_DTYPE_CODE[q.dtype], _stream(q.device)]
    _check(name, getattr(lib, name)(*args))
    return o, lse


def fa_forward(q, k, v, scale=None, causal=False, key_lens=None, o=None, lse=None):
    """Forward pass: returns (O [B,H,N,d] in q.dtype, LSE [B,H,N] float32)."""
    return _forward("fa_forward", q, k, v, scale, causal, key_lens, None, 128, o, lse)


def fa_forward_blocksparse(q, k, v, block_mask, block_size=128, scale=None, causal=False,
                           key_lens=None, o=None, lse=None):
    """Block-sparse forward: block_mask is uint8 [ceil(N/bs), ceil(N/bs)]."""
    if block_mask is None:
        raise ValueError("block_mask is required")
    return _forward("fa_forward_blocksparse", q, k, v, scale, causal, key_lens, block_mask,
                    block_size, o, lse)


def fa_forward_ex(q, k, v, block_mask=None, block_size=128, block_rows=0, scale=None,
                  causal=False, key_lens=None, o=None, lse=None, block_keys=0, key_groups=0):
    """Forward with the query rows per work-group (64, 128, 256; 0 = the
    library's choice), the keys per K/V tile (32, 64, 128; 0 = the type's
    default) and the key groups per tile (1, 2; 0 = the library's choice)
    given per call; block_mask optional."""
    return _forward("fa_forward_ex", q, k, v, scale, causal, key_lens, block_mask, block_size,
                    o, lse, block_rows, block_keys, key_groups)


def fa_forward_blocksparse_split_workspace_bytes(B, H, N, d, key_chunk):
    return int(load_library().fa_forward_blocksparse_split_workspace_bytes(B, H, N, d,
                                                                          int(key_chunk)))


def fa_forward_blocksparse_split(q, k, v, block_mask, block_size=128, key_chunk=16384, scale=None,
                                 causal=False, key_lens=None, o=None, lse=None, workspace=None):
    """Block-sparse forward with each query tile's key range split into
    key_chunk-key pieces over work-groups, merged by a second pass (for masks
    with a few very long rows).  workspace: uint8 device tensor of at least
    fa_forward_blocksparse_split_workspace_bytes(...) bytes, allocated here
    when not given."""
    if block_mask is None:
        raise ValueError("block_mask is required")
    lib = load_library()
    B, H, N, d = _shape(q, k, v)
    o = torch.empty_like(q) if o is None else _like("o", o, q)
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _like("lse", lse, q, (B, H, N), torch.float32))
    need = fa_forward_blocksparse_split_workspace_bytes(B, H, N, d, key_chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    kl = _lens(key_lens, B, q.device)
    bm = _mask(block_mask, N, block_size, q.device)
    st = lib.fa_forward_blocksparse_split(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _scale(scale, d),
        int(bool(causal)), _ptr(kl), _ptr(bm), int(block_size), int(key_chunk),
        _DTYPE_CODE[q.dtype], _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device))
    _check("fa_forward_blocksparse_split", st)
    return o, lse


def fa_forward_kv_workspace_bytes(B, H, Nq, Nk, d, dtype):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_forward_kv_workspace_bytes(B, H, Nq, Nk, d, code))


def fa_forward_kv(q, k, v, scale=None, causal=False, key_lens=None, o=None, lse=None,
                  workspace=None):
    """Inference forward: q [B,H,Nq,d] against a cache k, v [B,H,Nk,d] whose
    first key_lens[b] entries are filled; causal aligned bottom-right.
    Returns (O [B,H,Nq,d], LSE [B,H,Nq] float32)."""
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (B, H, Nk, d) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be [B, H, Nk, d] with q's dtype and device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device (the library has no CPU path)")
    o = torch.empty_like(q) if o is None else _like("o", o, q)
    lse = (torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None
           else _like("lse", lse, q, (B, H, Nq), torch.float32))
    need = fa_forward_kv_workspace_bytes(B, H, Nq, Nk, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    kl = _lens(key_lens, B, q.device)
    st = lib.fa_forward_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                           _scale(scale, d), int(bool(causal)), _ptr(kl),
                           _DTYPE_CODE[q.dtype], _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(q.device))
    _check("fa_forward_kv", st)
    return o, lse


def fa_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale=None,
                      causal=False, o=None, lse=None):
    """Packed variable-length forward: q [H, Tq, d], k and v [H, Tk, d];
    cu_seqlens_q / cu_seqlens_k int32 [B+1] prefix sums (device or host).
    Returns (O [H, Tq, d], LSE [H, Tq] float32); rows outside every sequence
    are left as allocated."""
    lib = load_library()
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [H, Tq, d] and k, v [H, Tk, d]")
    H, Tq, d = q.shape
    Tk = k.shape[1]
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (H, Tk, d) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be [H, Tk, d] with q's dtype and device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    # The kernel's grid covers max_seqlen_q rows per sequence; a longer
    # sequence would be left partly unwritten.  The library cannot see device
    # prefix sums; check them here whenever they come from the host.
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if isinstance(cu, torch.Tensor) and cu.device.type != "cpu":
            continue
        lens = np.diff(np.asarray(cu, dtype=np.int64))
        if lens.size and np.any(lens < 0):
            raise ValueError(f"{name} must be non-decreasing")
        if name == "cu_seqlens_q" and lens.size and int(lens.max()) > int(max_seqlen_q):
            raise ValueError(f"max_seqlen_q={int(max_seqlen_q)} is below the longest "
                             f"query sequence ({int(lens.max())})")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device (the library has no CPU path)")
    cq = torch.as_tensor(cu_seqlens_q).to(device=q.device, dtype=torch.int32).contiguous()
    ck = torch.as_tensor(cu_seqlens_k).to(device=q.device, dtype=torch.int32).contiguous()
    if cq.dim() != 1 or ck.shape != cq.shape or cq.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    B = cq.numel() - 1
    o = torch.empty_like(q) if o is None else _like("o", o, q)
    lse = (torch.empty((H, Tq), dtype=torch.float32, device=q.device) if lse is None
           else _like("lse", lse, q, (H, Tq), torch.float32))
    st = lib.fa_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cq), _ptr(ck),
                               B, H, Tq, Tk, int(max_seqlen_q), d, _scale(scale, d),
                               int(bool(causal)), _DTYPE_CODE[q.dtype], _stream(q.device))
    _check("fa_forward_varlen", st)
    return o, lse


def fa_backward_workspace_bytes(B, H, N, d):
    return int(load_library().fa_backward_workspace_bytes(B, H, N, d))


def _backward(name, q, k, v, o, dout, lse, scale, causal, key_lens, block_mask, block_size,
              dq, dk, dv, workspace, grad_dtype=None, dq_rows=0, dkdv_rows=0, key_groups=0):
    lib = load_library()
    B, H, N, d = _shape(q, k, v)
    _like("dout", dout, q)
    if name != "fa_backward_dkdv":
        _like("o", o, q)
        _like("lse", lse, q, (B, H, N), torch.float32)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    if gdt not in (q.dtype, torch.float32):
        raise ValueError(f"grad_dtype must be {q.dtype} or torch.float32")
    if name == "fa_backward" and (gdt != q.dtype or dq_rows or dkdv_rows or key_groups):
        name = "fa_backward_ex"

    def grad(t, nm):
        return (torch.empty(q.shape, dtype=gdt, device=q.device) if t is None
                else _like(nm, t, q, dtype=gdt))
    if name != "fa_backward_dkdv":
        dq = grad(dq, "dq")
    if name != "fa_backward_dq":
        dk, dv = grad(dk, "dk"), grad(dv, "dv")
    need = fa_backward_workspace_bytes(B, H, N, d)
    if workspace is None:
        if name == "fa_backward_dkdv":
            raise ValueError("fa_backward_dkdv reads the workspace fa_backward_dq filled")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    kl = _lens(key_lens, B, q.device)
    bm = _mask(block_mask, N, block_size, q.device)
    tail = [B, H, N, d, _scale(scale, d), int(bool(causal)), _ptr(kl), _ptr(bm),
            int(block_size), _DTYPE_CODE[q.dtype]]
    if name == "fa_backward_ex":
        tail += [_DTYPE_CODE[gdt], int(dq_rows), int(dkdv_rows), int(key_groups)]
    elif name in ("fa_backward_dq", "fa_backward_dkdv"):
        tail.append(int(dq_rows if name == "fa_backward_dq" else dkdv_rows))
    tail += [_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)]
    if name in ("fa_backward", "fa_backward_ex"):
        head = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                _ptr(dv)]
    elif name == "fa_backward_dq":
        head = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq)]
    else:
        head = [_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dk), _ptr(dv)]
    _check(name, getattr(lib, name)(*(head + tail)))
    return dq, dk, dv, workspace


def fa_backward(q, k, v, o, dout, lse, scale=None, causal=False, key_lens=None,
                block_mask=None, block_size=128, dq=None, dk=None, dv=None, workspace=None,
                grad_dtype=None):
    """Backward pass: returns (dQ, dK, dV) in q.dtype, or in float32 with
    grad_dtype=torch.float32 (fa_backward_ex: the same computation without the
    final rounding to the 16-bit type)."""
    dq, dk, dv, _ = _backward("fa_backward", q, k, v, o, dout, lse, scale, causal, key_lens,
                              block_mask, block_size, dq, dk, dv, workspace, grad_dtype)
    return dq, dk, dv


def fa_backward_ex(q, k, v, o, dout, lse, scale=None, causal=False, key_lens=None,
                   block_mask=None, block_size=128, dq=None, dk=None, dv=None, workspace=None,
                   grad_dtype=None, dq_rows=0, dkdv_rows=0, key_groups=0):
    """Backward with the gradients' dtype (q.dtype or torch.float32), the
    tile sizes (query rows per dQ work-group, keys per dK/dV work-group: 64,
    128, 256; 0 = 128) and the key groups (1, 2; 0 = the library's choice)
    given per call: returns (dQ, dK, dV).  At d = 128 the dK/dV pass of
    16-bit inputs with 128-key tiles splits each query tile between two wave
    groups unless key_groups is 1."""
    dq, dk, dv, _ = _backward("fa_backward_ex", q, k, v, o, dout, lse, scale, causal, key_lens,
                              block_mask, block_size, dq, dk, dv, workspace, grad_dtype,
                              dq_rows, dkdv_rows, key_groups)
    return dq, dk, dv


def fa_backward_noalloc_max_rows():
    return int(load_library().fa_backward_noalloc_max_rows())


def fa_backward_noalloc(q, k, v, o, dout, lse, scale=None, causal=False, key_lens=None,
                        block_mask=None, block_size=128, dq=None, dk=None, dv=None):
    """fa_backward with its workspace in the library's per-device scratch (no
    allocation by the library; B*H*N at most fa_backward_noalloc_max_rows()).
    Calls on one device share that scratch: they must not overlap."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v)
    _like("dout", dout, q)
    _like("o", o, q)
    _like("lse", lse, q, (B, H, N), torch.float32)
    dq, dk, dv = (torch.empty_like(q) if t is None else _like(nm, t, q)
                  for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")))
    kl = _lens(key_lens, B, q.device)
    bm = _mask(block_mask, N, block_size, q.device)
    _check("fa_backward_noalloc", lib.fa_backward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, N, d, _scale(scale, d), int(bool(causal)), _ptr(kl), _ptr(bm), int(block_size),
        _DTYPE_CODE[q.dtype], _stream(q.device)))
    return dq, dk, dv


def fa_backward_dq(q, k, v, o, dout, lse, scale=None, causal=False, key_lens=None,
                   block_mask=None, block_size=128, dq=None, workspace=None, rows=0):
    """First backward pass: returns (dQ, workspace); the workspace then holds
    -D and LSE * log2(e) for fa_backward_dkdv.  rows: query rows per
    work-group (64, 128, 256; 0 = 128)."""
    dq, _, _, ws = _backward("fa_backward_dq", q, k, v, o, dout, lse, scale, causal, key_lens,
                             block_mask, block_size, dq, None, None, workspace, dq_rows=rows)
    return dq, ws


def fa_backward_dkdv(q, k, v, dout, workspace, scale=None, causal=False, key_lens=None,
                     block_mask=None, block_size=128, dk=None, dv=None, rows=0):
    """Second backward pass, from the workspace fa_backward_dq filled:
    returns (dK, dV).  rows: keys per work-group (64, 128, 256; 0 = 128)."""
    _, dk, dv, _ = _backward("fa_backward_dkdv", q, k, v, None, dout, None, scale, causal,
                             key_lens, block_mask, block_size, None, dk, dv, workspace,
                             dkdv_rows=rows)
    return dk, dv


def fa_backward_blocksparse_split_workspace_bytes(B, H, N, d, chunk_blocks):
    return int(load_library().fa_backward_blocksparse_split_workspace_bytes(
        B, H, N, d, int(chunk_blocks)))


def fa_backward_blocksparse_split(q, k, v, o, dout, lse, block_mask, block_size=128,
                                  chunk_blocks=64, scale=None, causal=False, key_lens=None,
                                  dq=None, dk=None, dv=None, workspace=None):
    """Block-sparse backward with each mask row (dQ pass) and column (dK/dV
    pass) handed out in items of chunk_blocks kept blocks over work-groups,
    longer ones reduced from float32 partials (for masks with a few very long
    rows or columns).  Returns (dQ, dK, dV) in q.dtype.  workspace: uint8
    device tensor of at least fa_backward_blocksparse_split_workspace_bytes(...)
    bytes, allocated here when not given."""
    if block_mask is None:
        raise ValueError("block_mask is required")
    lib = load_library()
    B, H, N, d = _shape(q, k, v)
    for nm, t in (("o", o), ("dout", dout)):
        _like(nm, t, q)
    _like("lse", lse, q, (B, H, N), torch.float32)
    dq = torch.empty_like(q) if dq is None else _like("dq", dq, q)
    dk = torch.empty_like(q) if dk is None else _like("dk", dk, q)
    dv = torch.empty_like(q) if dv is None else _like("dv", dv, q)
    need = fa_backward_blocksparse_split_workspace_bytes(B, H, N, d, chunk_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    kl = _lens(key_lens, B, q.device)
    bm = _mask(block_mask, N, block_size, q.device)
    st = lib.fa_backward_blocksparse_split(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, N, d, _scale(scale, d), int(bool(causal)), _ptr(kl), _ptr(bm), int(block_size),
        int(chunk_blocks), _DTYPE_CODE[q.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check("fa_backward_blocksparse_split", st)
    return dq, dk, dv


def fa_forward_block_rows_for(B, H, N, d, dtype, sparse=False):
    """Query rows per work-group a forward of these sizes would use."""
    return int(load_library().fa_forward_block_rows_for(int(B), int(H), int(N), int(d),
                                                        (_DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)),
                                                        int(bool(sparse))))


def fa_forward_key_groups_for(B, H, N, d, dtype, sparse=False):
    """Key groups per query tile a forward of these sizes would use."""
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_forward_key_groups_for(int(B), int(H), int(N), int(d), code,
                                                        int(bool(sparse))))


def fa_backward_key_groups_for(B, H, N, d, dtype, sparse=False):
    """Key groups per work-group a backward of these sizes would use (at
    d = 128, the dQ pass's; the dK/dV pass splits its query tiles whenever
    key_groups is not 1)."""
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load_library().fa_backward_key_groups_for(int(B), int(H), int(N), int(d), code,
                                                         int(bool(sparse))))
