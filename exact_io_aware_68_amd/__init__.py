"""Python binding of libfa.so, the C-ABI exact tiled attention library for MI355X (gfx950).

Argument marshalling only: every step of the attention path runs in the library's HIP kernels.
torch is used for device memory and for the current HIP stream; nothing here computes any part
of the attention.  If libfa.so is missing or cannot be loaded, importing the functions below
raises — there is no fallback implementation.

The functions carry the C names (see include/fa.h for the full contract):

    fa_fwd(q, k, v, *, scale, causal, key_lens, o, lse)              -> (o, lse)
    fa_bwd(q, k, v, o, dO, lse, *, scale, causal, key_lens, ...)     -> (dq, dk, dv)
    fa_bwd_prep(o, dO, lse, workspace), fa_bwd_dkdv(q, k, v, dO, dk, dv, workspace, ...),
    fa_bwd_dq(q, k, v, dO, dq, workspace, ...)                       (the stages of fa_bwd)
    fa_bwd_workspace_size, fa_fwd_kernel_name, fa_bwd_dkdv_kernel_name, fa_bwd_dq_kernel_name,
    fa_status_str, fa_abi_version
    fa_fwd_splitkv(q, k, v, *, scale, key_lens, num_splits, o, lse)  -> (o, lse)   (decode shapes)
    fa_fwd_window(q, k, v, *, window, scale, key_lens, o, lse)       -> (o, lse)   (local window)
    fa_fwd_blocksparse(q, k, v, block_mask, *, scale, causal, key_lens, o, lse) -> (o, lse)
    fa_fwd_splitkv_splits, fa_fwd_splitkv_workspace_size

Tensors are [B, H, N, d] contiguous ("BHND"); q/k/v/o/dO are bf16 (d in {64, 128}) or fp32
(forward only, d <= 128); lse is fp32 [B, Hq, N]; key_lens int32 [B] on the device; gradients
are fp32.  Outputs not passed in are allocated with torch on the inputs' device.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FAError", "lib_path", "load", "fa_fwd", "fa_bwd", "fa_bwd_prep", "fa_bwd_dkdv", "fa_bwd_dq",
    "fa_bwd_workspace_size", "fa_fwd_kernel_name", "fa_bwd_dkdv_kernel_name",
    "fa_bwd_dq_kernel_name", "fa_status_str", "fa_abi_version", "FA_F32", "FA_BF16",
    "fa_fwd_splitkv", "fa_fwd_splitkv_splits", "fa_fwd_splitkv_workspace_size", "fa_fwd_window",
    "fa_fwd_blocksparse", "BLOCK_Q", "BLOCK_K",
]

BLOCK_Q, BLOCK_K = 128, 64   # block-sparse bitmap granularity (query rows, keys)

FA_F32, FA_BF16 = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {fa_status_str(status)} (status {status})")
        self.status = status


def lib_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def load() -> ctypes.CDLL:
    """Load libfa.so once (raises OSError if it is missing: build it first)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise OSError(f"{path} not found: run `python -m exact_io_aware_68_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.fa_fwd.restype = I
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, Z, I, I, I, I, I, F, I, I, P]
    lib.fa_bwd.restype = I
    lib.fa_bwd_prep.argtypes = [P, P, P, P, Z, I, I, I, I, I, P]
    lib.fa_bwd_prep.restype = I
    lib.fa_bwd_dkdv.argtypes = [P, P, P, P, P, P, P, P, Z, I, I, I, I, I, F, I, I, P]
    lib.fa_bwd_dkdv.restype = I
    lib.fa_bwd_dq.argtypes = [P, P, P, P, P, P, P, Z, I, I, I, I, I, F, I, I, P]
    lib.fa_bwd_dq.restype = I
    lib.fa_bwd_workspace_size.argtypes = [I, I, I, I]
    lib.fa_bwd_workspace_size.restype = Z
    lib.fa_fwd_blocksparse.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.fa_fwd_blocksparse.restype = I
    lib.fa_fwd_window.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, I, I, P]
    lib.fa_fwd_window.restype = I
    lib.fa_fwd_splitkv.argtypes = [P, P, P, P, P, P, P, Z, I, I, I, I, I, I, F, I, I, P]
    lib.fa_fwd_splitkv.restype = I
    lib.fa_fwd_splitkv_splits.argtypes = [I, I, I, I, I, I]
    lib.fa_fwd_splitkv_splits.restype = I
    lib.fa_fwd_splitkv_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.fa_fwd_splitkv_workspace_size.restype = Z
    for name in ("fa_fwd_kernel_name", "fa_bwd_dkdv_kernel_name", "fa_bwd_dq_kernel_name"):
        getattr(lib, name).argtypes = [I, I, I, I]
        getattr(lib, name).restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [I]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = I
    _LIB = lib
    return lib


def fa_status_str(status: int) -> str:
    return load().fa_status_str(int(status)).decode()


def fa_abi_version() -> int:
    return load().fa_abi_version()


def fa_bwd_workspace_size(B: int, Hq: int, N: int, d: int) -> int:
    return int(load().fa_bwd_workspace_size(B, Hq, N, d))


def fa_fwd_kernel_name(d: int, causal: bool, has_key_lens: bool, dtype: int) -> str:
    return load().fa_fwd_kernel_name(d, int(causal), int(has_key_lens), dtype).decode()


def fa_bwd_dkdv_kernel_name(d: int, causal: bool, has_key_lens: bool, dtype: int) -> str:
    return load().fa_bwd_dkdv_kernel_name(d, int(causal), int(has_key_lens), dtype).decode()


def fa_bwd_dq_kernel_name(d: int, causal: bool, has_key_lens: bool, dtype: int) -> str:
    return load().fa_bwd_dq_kernel_name(d, int(causal), int(has_key_lens), dtype).decode()


# ------------------------------------------------------------------ marshalling helpers

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    return -1


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _shape(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    return B, Hq, k.shape[1], N, d


def _check(fn: str, status: int):
    if status != 0:
        raise FAError(fn, status)


def _default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def fa_fwd(q, k, v, *, scale: float | None = None, causal: bool = False, key_lens=None,
           o=None, lse=None, want_lse: bool = True, stream=None):
    """Forward attention through libfa.so.  Returns (o, lse); lse is None if not wanted."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if key_lens is not None and key_lens.dtype != torch.int32:
        raise ValueError("key_lens must be int32")
    st = load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(key_lens), B, Hq,
                       Hkv, N, d, ctypes.c_float(_default_scale(d) if scale is None else scale),
                       int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_fwd", st)
    return o, lse


def fa_fwd_window(q, k, v, *, window, scale: float | None = None, key_lens=None, o=None,
                  lse=None, want_lse: bool = True, stream=None):
    """Forward with a local window (left, right): row i sees keys i - left .. i + right (a
    negative side is unbounded).  Returns (o, lse)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if key_lens is not None and key_lens.dtype != torch.int32:
        raise ValueError("key_lens must be int32")
    left, right = window
    st = load().fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(key_lens), B,
                              Hq, Hkv, N, d,
                              ctypes.c_float(_default_scale(d) if scale is None else scale),
                              int(left), int(right), _dtype_code(q), _stream(stream, q.device))
    _check("fa_fwd_window", st)
    return o, lse


def fa_fwd_blocksparse(q, k, v, block_mask, *, scale: float | None = None, causal: bool = False,
                       key_lens=None, o=None, lse=None, want_lse: bool = True, stream=None):
    """Block-sparse forward: block_mask is a uint8 device tensor [ceil(N/128), ceil(N/64)];
    row i sees key j only where block_mask[i // 128, j // 64] != 0.  Returns (o, lse)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    for t in (q, k, v, block_mask):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (
            -(-N // BLOCK_Q), -(-N // BLOCK_K)):
        raise ValueError("block_mask must be uint8 [ceil(N/128), ceil(N/64)]")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if key_lens is not None and key_lens.dtype != torch.int32:
        raise ValueError("key_lens must be int32")
    st = load().fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(key_lens),
                                   _ptr(block_mask), B, Hq, Hkv, N, d,
                                   ctypes.c_float(_default_scale(d) if scale is None else scale),
                                   int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_fwd_blocksparse", st)
    return o, lse


def fa_bwd_prep(o, dO, lse, workspace, *, stream=None):
    B, Hq, N, d = o.shape
    st = load().fa_bwd_prep(_ptr(o), _ptr(dO), _ptr(lse), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), B, Hq, N, d,
                            _dtype_code(o), _stream(stream, o.device))
    _check("fa_bwd_prep", st)


def fa_bwd_dkdv(q, k, v, dO, dk, dv, workspace, *, scale=None, causal=False, key_lens=None,
                stream=None):
    B, Hq, Hkv, N, d = _shape(q, k)
    st = load().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(key_lens), _ptr(dk),
                            _ptr(dv), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), B, Hq, Hkv, N, d,
                            ctypes.c_float(_default_scale(d) if scale is None else scale),
                            int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_bwd_dkdv", st)


def fa_bwd_dq(q, k, v, dO, dq, workspace, *, scale=None, causal=False, key_lens=None,
              stream=None):
    B, Hq, Hkv, N, d = _shape(q, k)
    st = load().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(key_lens), _ptr(dq),
                          _ptr(workspace), workspace.numel() * workspace.element_size(), B, Hq,
                          Hkv, N, d, ctypes.c_float(_default_scale(d) if scale is None else scale),
                          int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_bwd_dq", st)


def fa_bwd(q, k, v, o, dO, lse, *, scale: float | None = None, causal: bool = False,
           key_lens=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward by recomputation through libfa.so.  Returns (dq, dk, dv) in fp32."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(k.shape, **f32) if dk is None else dk
    dv = torch.empty(v.shape, **f32) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(1, fa_bwd_workspace_size(B, Hq, N, d)), dtype=torch.uint8,
                                device=q.device)
    st = load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(key_lens),
                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), B, Hq, Hkv, N, d,
                       ctypes.c_float(_default_scale(d) if scale is None else scale),
                       int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_bwd", st)
    return dq, dk, dv


def fa_fwd_splitkv_splits(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, num_splits: int = 0) -> int:
    return int(load().fa_fwd_splitkv_splits(B, Hq, Hkv, Nq, Nk, num_splits))


def fa_fwd_splitkv_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                                  num_splits: int = 0) -> int:
    return int(load().fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits))


def fa_fwd_splitkv(q, k, v, *, scale: float | None = None, key_lens=None, num_splits: int = 0,
                   o=None, lse=None, want_lse: bool = True, workspace=None, stream=None):
    """Split-KV forward for decode shapes: q [B, Hq, Nq, d] against k, v [B, Hkv, Nk, d]; every
    query row sees keys [0, key_lens[b]).  Returns (o, lse); lse is None if not wanted."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v must be 4-D [B, H, N, d] with k and v of one shape")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    if key_lens is not None and key_lens.dtype != torch.int32:
        raise ValueError("key_lens must be int32")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)
        workspace = torch.empty(max(16, n), dtype=torch.uint8, device=q.device)
    st = load().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(key_lens),
                               _ptr(workspace), workspace.numel() * workspace.element_size(), B,
                               Hq, Hkv, Nq, Nk, d,
                               ctypes.c_float(_default_scale(d) if scale is None else scale),
                               int(num_splits), _dtype_code(q), _stream(stream, q.device))
    _check("fa_fwd_splitkv", st)
    return o, lse
