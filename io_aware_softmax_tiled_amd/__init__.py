"""Exact attention (forward and backward) on MI355X: Python binding of libfa_mi355x.so.

This module only marshals arguments: it allocates outputs with torch on the inputs'
device, passes raw device pointers and the current HIP stream to the C ABI declared in
include/fa.h, and raises on a nonzero status. Every step of the computation runs in
the library's HIP kernels; there is no CPU or PyTorch fallback, and importing a
function here fails loudly when the library has not been built
(python -m io_aware_softmax_tiled_amd.build).

Functions have the C entry points' names (fwd and bwd are short names of fa_fwd and
fa_bwd):
    fa_fwd(q, k, v, *, causal=False, scale=None, kv_len=None) -> (o, lse)
    fa_bwd(q, k, v, o, dout, lse, *, causal=False, scale=None, kv_len=None) -> (dq, dk, dv)
    fa_bwd_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, workspace, *, ...) -> None
    fa_bwd_workspace_size(B, H, N, d) -> int
    fa_split_count(N, split_len) -> int
    fa_split_hint(B, H, N, d, *, causal=False, dtype=torch.bfloat16) -> int (0: unsplit)
    fa_fwd_workspace_size(B, H, N, d, *, causal=False, dtype=torch.bfloat16) -> int
    fa_fwd_auto(q, k, v, *, causal=False, scale=None, kv_len=None, workspace=None)
        -> (o, lse): fa_fwd, or the split fa_split_hint recommends, through a workspace
    fa_fwd_partial(q, k, v, *, split_len, causal=False, scale=None, kv_len=None)
        -> (o_part [P,B,H,N,d], lse_part [P,B,H,N])
    fa_merge(o_part, lse_part) -> (o, lse)
    fa_fwd_sparse(q, k, v, block_mask, *, causal=False, scale=None, kv_len=None) -> (o, lse)
    fa_bwd_sparse(q, k, v, o, dout, lse, block_mask, *, ...) -> (dq, dk, dv)
    fa_status_str(code) -> str, fa_last_error() -> str, fa_version() -> int
Tensors are [B, H, N, d] contiguous (q, k, v, dout: float32, bfloat16 or float16;
o, dq, dk, dv: float32), lse is [B, H, N] float32, kv_len an int32 [B] device tensor
or None. The default scale is 1/sqrt(d). Caller-supplied buffers (out=, lse=, o, lse,
dout, dq/dk/dv, workspace) are checked for shape, dtype, device and contiguity before
any pointer reaches the library.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["fwd", "bwd", "fa_fwd", "fa_bwd", "fa_bwd_noalloc", "FA_NOALLOC_SCRATCH_BYTES", "fa_bwd_stage", "fa_bwd_workspace_size", "fa_split_count", "fa_split_hint", "fa_fwd_workspace_size", "fa_fwd_auto", "fa_fwd_partial",
           "fa_merge", "fa_fwd_sparse", "fa_bwd_sparse", "fa_fwd_dropout", "fa_bwd_dropout",
           "fa_fwd_deferred", "fa_dropout_threshold", "FA_DEFERRED_MAX_N", "FA_SPARSE_BLOCK", "fa_status_str", "fa_last_error", "fa_version", "FaError", "lib_path",
           "load_library",
           "FA_F32", "FA_BF16", "FA_F16"]

FA_F32, FA_BF16, FA_F16 = 0, 1, 2
FA_SPARSE_BLOCK = 128
FA_DEFERRED_MAX_N = 512
FA_NOALLOC_SCRATCH_BYTES = 32 << 20
_DTYPE_CODE = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.float16: FA_F16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "libfa_mi355x.so")


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{fa_status_str(status)}: {detail}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libfa_mi355x.so once and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m io_aware_softmax_tiled_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp, vp]
    lib.fa_fwd.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32,
                           i32, vp, vp, sz, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                   i32, i32, vp, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_bwd_stage.argtypes = [i32] + lib.fa_bwd.argtypes
    lib.fa_bwd_stage.restype = i32
    lib.fa_bwd_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_split_count.argtypes = [i32, i32]
    lib.fa_split_count.restype = i32
    lib.fa_split_hint.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_split_hint.restype = i32
    lib.fa_fwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_fwd_workspace_size.restype = sz
    lib.fa_fwd_auto.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp, vp,
                                sz, vp]
    lib.fa_fwd_auto.restype = i32
    lib.fa_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp,
                                   i32, vp]
    lib.fa_fwd_partial.restype = i32
    lib.fa_merge.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.fa_merge.restype = i32
    lib.fa_fwd_sparse.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp,
                                  vp, vp]
    lib.fa_fwd_sparse.restype = i32
    lib.fa_bwd_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                  i32, i32, vp, vp, vp, sz, vp]
    lib.fa_bwd_sparse.restype = i32
    lib.fa_fwd_deferred.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp,
                                    vp]
    lib.fa_fwd_deferred.restype = i32
    u64 = ctypes.c_uint64
    u32 = ctypes.c_uint32
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp,
                                   f32, u64, u32, vp]
    lib.fa_fwd_dropout.restype = i32
    lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                   i32, i32, vp, f32, u64, u32, vp, sz, vp]
    lib.fa_bwd_dropout.restype = i32
    lib.fa_dropout_threshold.argtypes = [f32]
    lib.fa_dropout_threshold.restype = i32
    lib.fa_status_str.argtypes = [i32]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i32
    _LIB = lib
    return lib


def fa_status_str(code: int) -> str:
    return load_library().fa_status_str(int(code)).decode()


def fa_last_error() -> str:
    return load_library().fa_last_error().decode()


def fa_version() -> int:
    return int(load_library().fa_version())


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d))


def fa_dropout_threshold(p: float) -> int:
    """Byte threshold t of dropout probability p (keep iff byte >= t), -1 if p is not in
    [0, 1)."""
    return int(load_library().fa_dropout_threshold(float(p)))


def fa_split_count(N: int, split_len: int) -> int:
    return int(load_library().fa_split_count(N, split_len))


def fa_split_hint(B: int, H: int, N: int, d: int, *, causal: bool = False,
                  dtype: torch.dtype = torch.bfloat16) -> int:
    if dtype not in _DTYPE_CODE:
        raise TypeError(f"dtype {dtype} is not float32, bfloat16 or float16")
    r = int(load_library().fa_split_hint(B, H, N, d, int(bool(causal)), _DTYPE_CODE[dtype]))
    if r < 0:
        _check(-r)
    return r


def _check(status: int):
    if status != 0:
        raise FaError(status, fa_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _shape(q, k, v):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must share one dtype among float32, bfloat16, float16")
    for t in (q, k, v):
        if not t.is_cuda:
            raise ValueError("inputs must be GPU tensors")
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    return tuple(int(x) for x in q.shape)


def _kv(kv_len, B, device):
    if kv_len is None:
        return None
    if kv_len.dtype != torch.int32 or kv_len.device != device or kv_len.numel() != B:
        raise ValueError("kv_len must be an int32 tensor of B elements on the inputs' device")
    return kv_len.contiguous()


def _expect(t, name, shape, dtype, device):
    """Check a caller-supplied tensor against what the kernels will read or write through
    its pointer: exact shape, dtype, device and a contiguous layout. Every size the C
    layer uses is derived from B, H, N and d, so a buffer that does not match would be
    read or written out of bounds."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(t, name, shape, device):
    """A float32 output buffer: allocated when t is None, else checked."""
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    return _expect(t, name, shape, torch.float32, device)


def _workspace(ws, B, H, N, d, device):
    need = fa_bwd_workspace_size(B, H, N, d)
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes, got {ws.numel() * ws.element_size()}")
    return ws


def _grad_inputs(q, o, dout, lse):
    """o and lse as fa_fwd returned them, dout like q."""
    B, H, N, d = (int(x) for x in q.shape)
    _expect(o, "o", (B, H, N, d), torch.float32, q.device)
    _expect(lse, "lse", (B, H, N), torch.float32, q.device)
    _expect(dout, "dout", (B, H, N, d), q.dtype, q.device)


def _stream(device, stream):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def fa_fwd(q, k, v, *, causal=False, scale=None, kv_len=None, out=None, lse=None,
           stream=None):
    """Forward pass: returns (o float32 [B,H,N,d], lse float32 [B,H,N])."""
    B, H, N, d = _shape(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    o = _out(out, "out", (B, H, N, d), q.device)
    lse_t = _out(lse, "lse", (B, H, N), q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d, scale,
                        int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv),
                        _stream(q.device, stream))
    _check(st)
    return o, lse_t


def fa_fwd_workspace_size(B: int, H: int, N: int, d: int, *, causal: bool = False,
                          dtype: torch.dtype = torch.bfloat16) -> int:
    if dtype not in _DTYPE_CODE:
        raise TypeError(f"dtype {dtype} is not float32, bfloat16 or float16")
    return int(load_library().fa_fwd_workspace_size(B, H, N, d, int(bool(causal)),
                                                    _DTYPE_CODE[dtype]))


def fa_fwd_auto(q, k, v, *, causal=False, scale=None, kv_len=None, out=None, lse=None,
                workspace=None, stream=None):
    """Forward pass with the split fa_split_hint recommends (none: fa_fwd): returns
    (o float32 [B,H,N,d], lse float32 [B,H,N]). The workspace (uint8, at least
    fa_fwd_workspace_size bytes) is allocated when not given."""
    B, H, N, d = _shape(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    o = _out(out, "out", (B, H, N, d), q.device)
    lse_t = _out(lse, "lse", (B, H, N), q.device)
    need = fa_fwd_workspace_size(B, H, N, d, causal=causal, dtype=q.dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    elif (not isinstance(workspace, torch.Tensor) or workspace.device != q.device
          or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_auto(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d, scale,
                             int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv), _ptr(workspace),
                             ws_bytes, _stream(q.device, stream))
    _check(st)
    return o, lse_t


def fa_bwd(q, k, v, o, dout, lse, *, causal=False, scale=None, kv_len=None, workspace=None,
           stream=None):
    """Backward pass of sum(dout * O): returns (dq, dk, dv), float32 [B,H,N,d]."""
    B, H, N, d = _shape(q, k, v)
    _grad_inputs(q, o, dout, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    workspace = _workspace(workspace, B, H, N, d, q.device)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), B, H, N, d, scale, int(bool(causal)),
                        _DTYPE_CODE[q.dtype], _ptr(kv), _ptr(workspace),
                        workspace.numel() * workspace.element_size(),
                        _stream(q.device, stream))
    _check(st)
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, *, causal=False, scale=None,
                   kv_len=None, stream=None):
    """fa_bwd into caller-allocated dq, dk, dv (float32 [B,H,N,d]) with the library's
    static per-GPU scratch instead of a workspace: the call allocates nothing. Calls
    that overlap in time on one GPU race on the scratch."""
    B, H, N, d = _shape(q, k, v)
    _grad_inputs(q, o, dout, lse)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, name, (B, H, N, d), torch.float32, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, scale,
                                int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv),
                                _stream(q.device, stream))
    _check(st)


def fa_bwd_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, workspace, *, causal=False,
                 scale=None, kv_len=None, stream=None):
    """One kernel of the backward pass into caller-allocated outputs: stage 0 writes D
    into the workspace, 1 writes dk and dv (needs D), 2 writes dq (forms its own D),
    3 writes dq and D (fa_bwd is stage 3 then stage 1)."""
    B, H, N, d = _shape(q, k, v)
    _grad_inputs(q, o, dout, lse)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, name, (B, H, N, d), torch.float32, q.device)
    workspace = _workspace(workspace, B, H, N, d, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_bwd_stage(int(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, scale,
                              int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(q.device, stream))
    _check(st)


def fa_fwd_partial(q, k, v, *, split_len, causal=False, scale=None, kv_len=None, out=None,
                   lse=None, stream=None):
    """Partial forward over key ranges of split_len keys (a multiple of 64): returns
    (o_part float32 [P,B,H,N,d], lse_part float32 [P,B,H,N]), P = fa_split_count(N,
    split_len). A row that sees no key of a range gets o_part = 0, lse_part = -inf."""
    B, H, N, d = _shape(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    P = fa_split_count(N, int(split_len))
    if P < 0:
        raise ValueError(f"split_len must be a positive multiple of 64 (got {split_len})")
    o = _out(out, "out", (P, B, H, N, d), q.device)
    lse_t = _out(lse, "lse", (P, B, H, N), q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                                scale, int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv),
                                int(split_len), _stream(q.device, stream))
    _check(st)
    return o, lse_t


def fa_merge(o_part, lse_part, *, out=None, lse=None, stream=None):
    """Merge partials (float32 [P,B,H,N,d] and [P,B,H,N]) into (o [B,H,N,d], lse [B,H,N])."""
    if o_part.dim() != 5 or lse_part.dim() != 4 or tuple(lse_part.shape) != tuple(o_part.shape[:4]):
        raise ValueError("o_part must be [P,B,H,N,d] and lse_part [P,B,H,N]")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise ValueError("partials are float32")
    for t in (o_part, lse_part):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("partials must be contiguous GPU tensors")
    P, B, H, N, d = (int(x) for x in o_part.shape)
    o = _out(out, "out", (B, H, N, d), o_part.device)
    lse_t = _out(lse, "lse", (B, H, N), o_part.device)
    lib = load_library()
    with torch.cuda.device(o_part.device):
        st = lib.fa_merge(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse_t), P, B, H, N, d,
                          _stream(o_part.device, stream))
    _check(st)
    return o, lse_t


def _mask(block_mask, N, device):
    nb = -(-N // FA_SPARSE_BLOCK)
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be a uint8 [{nb}, {nb}] tensor")
    if block_mask.device != device or not block_mask.is_contiguous():
        raise ValueError("block_mask must be contiguous on the inputs' device")
    return block_mask


def fa_fwd_sparse(q, k, v, block_mask, *, causal=False, scale=None, kv_len=None, out=None,
                  lse=None, stream=None):
    """Block-sparse forward: block_mask uint8 [ceil(N/128), ceil(N/128)] (nonzero =
    evaluated); returns (o, lse) with o = 0, lse = -inf on rows that see no key."""
    B, H, N, d = _shape(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    bm = _mask(block_mask, N, q.device)
    o = _out(out, "out", (B, H, N, d), q.device)
    lse_t = _out(lse, "lse", (B, H, N), q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                               scale, int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv),
                               _ptr(bm), _stream(q.device, stream))
    _check(st)
    return o, lse_t


def fa_bwd_sparse(q, k, v, o, dout, lse, block_mask, *, causal=False, scale=None,
                  kv_len=None, workspace=None, stream=None):
    """Block-sparse backward of sum(dout * O): returns (dq, dk, dv), float32 [B,H,N,d]."""
    B, H, N, d = _shape(q, k, v)
    _grad_inputs(q, o, dout, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    bm = _mask(block_mask, N, q.device)
    workspace = _workspace(workspace, B, H, N, d, q.device)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_bwd_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, scale,
                               int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv), _ptr(bm),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(q.device, stream))
    _check(st)
    return dq, dk, dv


def _key(seed, offset):
    seed, offset = int(seed), int(offset)
    if not (0 <= seed < 1 << 64 and 0 <= offset < 1 << 32):
        raise ValueError("seed is an unsigned 64-bit and offset an unsigned 32-bit integer")
    return seed, offset


def fa_fwd_dropout(q, k, v, *, p, seed, offset=0, causal=False, scale=None, kv_len=None,
                   out=None, lse=None, stream=None):
    """Forward with dropout p on the probabilities, mask drawn from Philox4x32-10 keyed by
    seed (64-bit) with offset (32-bit) in its counters: returns (o, lse), lse that of the
    undropped scores."""
    seed, offset = _key(seed, offset)
    B, H, N, d = _shape(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    o = _out(out, "out", (B, H, N, d), q.device)
    lse_t = _out(lse, "lse", (B, H, N), q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                                scale, int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv),
                                float(p), seed, offset, _stream(q.device, stream))
    _check(st)
    return o, lse_t


def fa_bwd_dropout(q, k, v, o, dout, lse, *, p, seed, offset=0, causal=False, scale=None,
                   kv_len=None, workspace=None, stream=None):
    """Backward of sum(dout * O) for O from fa_fwd_dropout with the same p, seed and offset
    (the mask is regenerated, not stored): returns (dq, dk, dv), float32 [B,H,N,d]."""
    seed, offset = _key(seed, offset)
    B, H, N, d = _shape(q, k, v)
    _grad_inputs(q, o, dout, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    workspace = _workspace(workspace, B, H, N, d, q.device)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, scale,
                                int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv), float(p),
                                seed, offset, _ptr(workspace),
                                workspace.numel() * workspace.element_size(),
                                _stream(q.device, stream))
    _check(st)
    return dq, dk, dv


def fa_fwd_deferred(q, k, v, *, causal=False, scale=None, kv_len=None, out=None, lse=None,
                    stream=None):
    """Forward pass with the P V product deferred to the end of each query block's key
    row (N <= FA_DEFERRED_MAX_N): the same (o, lse) as fa_fwd."""
    B, H, N, d = _shape(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kv = _kv(kv_len, B, q.device)
    o = _out(out, "out", (B, H, N, d), q.device)
    lse_t = _out(lse, "lse", (B, H, N), q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_deferred(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                                 scale, int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(kv),
                                 _stream(q.device, stream))
    _check(st)
    return o, lse_t


# The Python surface under the short names: fwd(q, k, v, *, causal, scale=None,
# kv_len=None) -> (o, lse) and bwd(q, k, v, o, dout, lse, *, causal, scale=None,
# kv_len=None) -> (dq, dk, dv), the same functions as fa_fwd and fa_bwd.
fwd = fa_fwd
bwd = fa_bwd
