"""Python binding of libfa.so, the C-ABI exact tiled attention library for MI355X (gfx950).

Argument marshalling only: every step of the attention path runs in the library's HIP kernels.
torch is used for device memory and for the current HIP stream; nothing here computes any part
of the attention.  If libfa.so is missing or cannot be loaded, importing the functions below
raises — there is no fallback implementation.

The functions carry the C names (see include/fa.h for the full contract):

    fa_fwd(q, k, v, *, scale, causal, key_lens, o, lse)              -> (o, lse)
    fa_bwd(q, k, v, o, dO, lse, *, scale, causal, key_lens, ...)     -> (dq, dk, dv)
    fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, *, ...)          (fa_bwd, no allocation)
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
    "fa_fwd_blocksparse", "BLOCK_Q", "BLOCK_K", "fa_bwd_noalloc", "NOALLOC_MAX_ROWS",
]

BLOCK_Q, BLOCK_K = 128, 64   # block-sparse bitmap granularity (query rows, keys)
NOALLOC_MAX_ROWS = 4194304   # FA_NOALLOC_MAX_ROWS: B * Hq * N limit of fa_bwd_noalloc

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
    lib.fa_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.fa_bwd_noalloc.restype = I
    lib.fa_bwd_prep.argtypes = [P, P, P, P, Z, I, I, I, I, I, P]
    lib.fa_bwd_prep.restype = I
    lib.fa_bwd_dkdv.argtypes = [P, P, P, P, P, P, P, P, Z, I, I, I, I, I, F, I, I, P]
    lib.fa_bwd_dkdv.restype = I
    lib.fa_bwd_dq.argtypes = [P, P, P, P, P, P, P, Z, I, I, I, I, I, F, I, I, P]
    lib.fa_bwd_dq.restype = I
    lib.fa_bwd_workspace_size.argtypes = [I, I, I]
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


def fa_bwd_workspace_size(B: int, Hq: int, N: int) -> int:
    return int(load().fa_bwd_workspace_size(B, Hq, N))


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


# Every tensor is checked before the library is called: the C ABI sees raw pointers only, so a
# wrong shape, dtype, stride or device would otherwise be read or written out of bounds on the
# GPU.  Device checks come last, so that the shape rules can be exercised on the CPU.

def _need(cond: bool, fn: str, msg: str):
    if not cond:
        raise ValueError(f"{fn}: {msg}")


def _tensor(fn: str, name: str, t, shape=None, dtype=None):
    """t must be a contiguous tensor, with the given shape and dtype when those are given."""
    _need(hasattr(t, "is_contiguous"), fn, f"{name} must be a torch tensor")
    _need(t.is_contiguous(), fn, f"{name} must be contiguous")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), fn,
              f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None:
        _need(t.dtype == dtype, fn, f"{name} has dtype {t.dtype}, expected {dtype}")


def _qkv(fn: str, q, k, v, key_lens):
    """q [B, Hq, N, d], k and v [B, Hkv, N, d] of q's dtype (bf16 or fp32), key_lens int32 [B]."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _tensor(fn, name, t)
        _need(t.dim() == 4, fn, f"{name} must be 4-D [B, H, N, d]")
    _need(q.dtype in (torch.bfloat16, torch.float32), fn, "q must be bfloat16 or float32")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, fn, "q, k and v must share one dtype")
    _need(tuple(v.shape) == tuple(k.shape), fn, "k and v must have the same shape")
    B, Hq, N, d = q.shape
    _need(k.shape[0] == B and k.shape[2] == N and k.shape[3] == d, fn,
          "k/v shape does not match q ([B, Hkv, N, d])")
    if key_lens is not None:
        _tensor(fn, "key_lens", key_lens, (B,), torch.int32)
    return B, Hq, k.shape[1], N, d


def _on_one_gpu(fn: str, *tensors):
    """Every tensor given (None skipped) lives on one and the same GPU."""
    ts = [t for t in tensors if t is not None]
    for t in ts:
        _need(t.is_cuda, fn, f"every tensor must be on a GPU (found one on {t.device})")
    _need(len({t.device for t in ts}) <= 1, fn, "all tensors must be on the same GPU")


def _check(fn: str, status: int):
    if status != 0:
        raise FAError(fn, status)


def _default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def _fwd_outputs(fn: str, q, o, lse, rows=None):
    """Caller-supplied o must match q; lse must be fp32 [B, Hq, N] (rows = N, or Nq)."""
    torch = _torch()
    B, Hq, N = q.shape[0], q.shape[1], q.shape[2] if rows is None else rows
    if o is not None:
        _tensor(fn, "o", o, q.shape, q.dtype)
    if lse is not None:
        _tensor(fn, "lse", lse, (B, Hq, N), torch.float32)


def fa_fwd(q, k, v, *, scale: float | None = None, causal: bool = False, key_lens=None,
           o=None, lse=None, want_lse: bool = True, stream=None):
    """Forward attention through libfa.so.  Returns (o, lse); lse is None if not wanted."""
    torch = _torch()
    B, Hq, Hkv, N, d = _qkv("fa_fwd", q, k, v, key_lens)
    _fwd_outputs("fa_fwd", q, o, lse)
    _on_one_gpu("fa_fwd", q, k, v, key_lens, o, lse)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
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
    B, Hq, Hkv, N, d = _qkv("fa_fwd_window", q, k, v, key_lens)
    _fwd_outputs("fa_fwd_window", q, o, lse)
    _on_one_gpu("fa_fwd_window", q, k, v, key_lens, o, lse)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
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
    fn = "fa_fwd_blocksparse"
    B, Hq, Hkv, N, d = _qkv(fn, q, k, v, key_lens)
    _tensor(fn, "block_mask", block_mask, (-(-N // BLOCK_Q), -(-N // BLOCK_K)), torch.uint8)
    _fwd_outputs(fn, q, o, lse)
    _on_one_gpu(fn, q, k, v, key_lens, block_mask, o, lse)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    st = load().fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(key_lens),
                                   _ptr(block_mask), B, Hq, Hkv, N, d,
                                   ctypes.c_float(_default_scale(d) if scale is None else scale),
                                   int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_fwd_blocksparse", st)
    return o, lse


def _workspace(fn: str, ws):
    _tensor(fn, "workspace", ws)


def _grad_inputs(fn: str, q, dO, o=None, lse=None):
    """dO (and o) like q; lse fp32 [B, Hq, N]."""
    torch = _torch()
    _tensor(fn, "dO", dO, q.shape, q.dtype)
    if o is not None:
        _tensor(fn, "o", o, q.shape, q.dtype)
    if lse is not None:
        _tensor(fn, "lse", lse, q.shape[:3], torch.float32)


def _grad_outputs(fn: str, q, k, dq=None, dk=None, dv=None):
    """fp32 gradients: dq like q, dk and dv like k."""
    torch = _torch()
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t is not None:
            _tensor(fn, name, t, like.shape, torch.float32)


def fa_bwd_prep(o, dO, lse, workspace, *, stream=None):
    torch = _torch()
    fn = "fa_bwd_prep"
    _tensor(fn, "o", o)
    _need(o.dim() == 4 and o.dtype == torch.bfloat16, fn, "o must be bf16 [B, Hq, N, d]")
    _grad_inputs(fn, o, dO, None, lse)
    _workspace(fn, workspace)
    _on_one_gpu(fn, o, dO, lse, workspace)
    B, Hq, N, d = o.shape
    st = load().fa_bwd_prep(_ptr(o), _ptr(dO), _ptr(lse), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), B, Hq, N, d,
                            _dtype_code(o), _stream(stream, o.device))
    _check("fa_bwd_prep", st)


def fa_bwd_dkdv(q, k, v, dO, dk, dv, workspace, *, scale=None, causal=False, key_lens=None,
                stream=None):
    fn = "fa_bwd_dkdv"
    B, Hq, Hkv, N, d = _qkv(fn, q, k, v, key_lens)
    _grad_inputs(fn, q, dO)
    _need(dk is not None and dv is not None, fn, "dk and dv are required")
    _grad_outputs(fn, q, k, None, dk, dv)
    _workspace(fn, workspace)
    _on_one_gpu(fn, q, k, v, dO, key_lens, dk, dv, workspace)
    st = load().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(key_lens), _ptr(dk),
                            _ptr(dv), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), B, Hq, Hkv, N, d,
                            ctypes.c_float(_default_scale(d) if scale is None else scale),
                            int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_bwd_dkdv", st)


def fa_bwd_dq(q, k, v, dO, dq, workspace, *, scale=None, causal=False, key_lens=None,
              stream=None):
    fn = "fa_bwd_dq"
    B, Hq, Hkv, N, d = _qkv(fn, q, k, v, key_lens)
    _grad_inputs(fn, q, dO)
    _need(dq is not None, fn, "dq is required")
    _grad_outputs(fn, q, k, dq)
    _workspace(fn, workspace)
    _on_one_gpu(fn, q, k, v, dO, key_lens, dq, workspace)
    st = load().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(key_lens), _ptr(dq),
                          _ptr(workspace), workspace.numel() * workspace.element_size(), B, Hq,
                          Hkv, N, d, ctypes.c_float(_default_scale(d) if scale is None else scale),
                          int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_bwd_dq", st)


def fa_bwd(q, k, v, o, dO, lse, *, scale: float | None = None, causal: bool = False,
           key_lens=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward by recomputation through libfa.so.  Returns (dq, dk, dv) in fp32."""
    torch = _torch()
    fn = "fa_bwd"
    B, Hq, Hkv, N, d = _qkv(fn, q, k, v, key_lens)
    _grad_inputs(fn, q, dO, o, lse)
    _grad_outputs(fn, q, k, dq, dk, dv)
    if workspace is not None:
        _workspace(fn, workspace)
    _on_one_gpu(fn, q, k, v, o, dO, lse, key_lens, dq, dk, dv, workspace)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(k.shape, **f32) if dk is None else dk
    dv = torch.empty(v.shape, **f32) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(1, fa_bwd_workspace_size(B, Hq, N)), dtype=torch.uint8,
                                device=q.device)
    st = load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(key_lens),
                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), B, Hq, Hkv, N, d,
                       ctypes.c_float(_default_scale(d) if scale is None else scale),
                       int(causal), _dtype_code(q), _stream(stream, q.device))
    _check("fa_bwd", st)
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, *, scale: float | None = None,
                   causal: bool = False, key_lens=None, stream=None):
    """fa_bwd without a workspace and without any allocation, neither in the library nor here:
    the caller passes every output (fp32 dq like q, dk and dv like k).  The per-row statistics
    live in the library's fixed device scratch (B * Hq * N <= NOALLOC_MAX_ROWS); calls that may
    overlap in time on one GPU race on it."""
    fn = "fa_bwd_noalloc"
    B, Hq, Hkv, N, d = _qkv(fn, q, k, v, key_lens)
    _grad_inputs(fn, q, dO, o, lse)
    _need(dq is not None and dk is not None and dv is not None, fn, "dq, dk and dv are required")
    _grad_outputs(fn, q, k, dq, dk, dv)
    _on_one_gpu(fn, q, k, v, o, dO, lse, key_lens, dq, dk, dv)
    st = load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                               _ptr(key_lens), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d,
                               ctypes.c_float(_default_scale(d) if scale is None else scale),
                               int(causal), _dtype_code(q), _stream(stream, q.device))
    _check(fn, st)


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
    fn = "fa_fwd_splitkv"
    for name, t in (("q", q), ("k", k), ("v", v)):
        _tensor(fn, name, t)
        _need(t.dim() == 4, fn, f"{name} must be 4-D [B, H, N, d]")
    _need(q.dtype in (torch.bfloat16, torch.float32), fn, "q must be bfloat16 or float32")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, fn, "q, k and v must share one dtype")
    _need(tuple(v.shape) == tuple(k.shape), fn, "k and v must have the same shape")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _need(k.shape[0] == B and k.shape[3] == d, fn, "k/v shape does not match q ([B, Hkv, Nk, d])")
    if key_lens is not None:
        _tensor(fn, "key_lens", key_lens, (B,), torch.int32)
    _fwd_outputs(fn, q, o, lse, rows=Nq)
    if workspace is not None:
        _workspace(fn, workspace)
    _on_one_gpu(fn, q, k, v, key_lens, o, lse, workspace)
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
