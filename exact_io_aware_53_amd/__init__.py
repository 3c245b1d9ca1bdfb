"""Exact IO-aware attention for MI355X (gfx950): thin Python binding of libfa.so.

Every computation happens in the HIP kernels behind the C ABI declared in
include/fa.h. This module only marshals arguments: it checks tensor shapes,
allocates outputs with torch (device memory and streams are torch's), and
passes raw pointers and the current HIP stream to the library. There is no
CPU or PyTorch fallback: if libfa.so is missing, every call raises.

    o, lse = fwd(q, k, v, causal=True)             # q, k, v: [B, H, N, d] bf16 or fp32 on the GPU
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)
    o, lse = fwd_decode(q_new, k_cache, v_cache)   # [B, H, Nq, d] against [B, H, Nk, d], bf16
    o, lse = fwd(q.transpose(1, 2), ...)           # any strided [B, H, N, d] view, bf16 or fp16,
                                                   # d in {32, 64, 96, 128, 256}
    o, lse = fwd_varlen(q, k, v, cu_seqlens, max_seqlen)   # packed [total, H, d] sequences
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3

# (name, restype, argtypes) of every symbol in include/fa.h
_P, _I, _F, _U64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, ctypes.c_size_t
_FWD_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _F, _U64, _P]
_BWD_ARGS = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _F, _U64, _P, _SZ, _P]
SIGNATURES = {
    "fa_fwd": (_I, _FWD_ARGS),
    "fa_fwd_f32": (_I, _FWD_ARGS),
    "fa_bwd": (_I, _BWD_ARGS),
    "fa_bwd_f32": (_I, _BWD_ARGS),
    "fa_bwd_deterministic": (_I, _BWD_ARGS),
    "fa_bwd_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "fa_bwd_noalloc": (_I, _BWD_ARGS[:17] + [_P]),
    "fa_fwd_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "fa_fwd_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "fa_fwd_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "fa_fwd_decode_paged_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "fa_dropout_mask": (_I, [_P, _I, _I, _I, _I, _I, _F, _U64, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
}



class Layout(ctypes.Structure):
    """fa_layout: element strides of a [B, H, N, d] view (d contiguous)."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("row", ctypes.c_int64)]


class Problem(ctypes.Structure):
    """fa_problem of include/fa.h."""
    _fields_ = [("B", _I), ("H", _I), ("N", _I), ("d", _I), ("dtype", _I),
                ("cu_seqlens", _P), ("total_tokens", _I),
                ("q", Layout), ("k", Layout), ("v", Layout), ("o", Layout), ("lse", Layout),
                ("dout", Layout), ("dq", Layout), ("dk", Layout), ("dv", Layout)]


_PB = ctypes.POINTER(Problem)
SIGNATURES.update({
    "fa_fwd_ex": (_I, [_PB, _P, _P, _P, _P, _P, _F, _I, _F, _U64, _P]),
    "fa_bwd_ex": (_I, [_PB, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _I, _F, _U64, _I, _P, _SZ, _P]),
    "fa_bwd_ex_workspace_size": (_SZ, [_PB]),
})
FA_DTYPE = {torch.bfloat16: 0, torch.float16: 1}

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().fa_status_string(status).decode()}")


def lib() -> ctypes.CDLL:
    """The loaded libfa.so with typed entry points; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m exact_io_aware_53_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, where: str):
    if status != FA_OK:
        raise FAError(status, where)


def _shape4(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return tuple(t.shape)


def _entry(dtype, stem):
    if dtype == torch.bfloat16:
        return getattr(lib(), stem)
    if dtype == torch.float32:
        return getattr(lib(), stem + "_f32")
    raise ValueError("tensors must be bfloat16 or float32")


def fwd(q, k, v, scale=None, causal=False, dropout_p=0.0, seed=0, out=None, lse=None):
    """Forward pass: returns (O [B,H,N,d] in the input dtype, LSE [B,H,N] fp32)."""
    shp = _shape4(q, "q")
    if _shape4(k, "k") != shp or _shape4(v, "v") != shp or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    B, H, N, d = shp
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = _entry(q.dtype, "fa_fwd")(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, N, d, scale, int(bool(causal)),
                                   float(dropout_p), int(seed) & (2**64 - 1), _stream(q.device))
    _check(st, "fa_fwd")
    return out, lse


def _layout4(t: torch.Tensor, name: str) -> Layout:
    """Strides of a [B, H, N, d] view whose last dimension is contiguous."""
    if t.dim() != 4 or not t.is_cuda:
        raise ValueError(f"{name} must be a [B, H, N, d] GPU tensor")
    if t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError(f"{name}: the d dimension must be contiguous")
    return Layout(t.stride(0), t.stride(1), t.stride(2))


def _layout3(t: torch.Tensor, name: str) -> Layout:
    """Strides of a packed [total, H, d] tensor (d contiguous); no batch stride."""
    if t.dim() != 3 or not t.is_cuda:
        raise ValueError(f"{name} must be a packed [total, H, d] GPU tensor")
    if t.stride(2) != 1 and t.shape[2] > 1:
        raise ValueError(f"{name}: the d dimension must be contiguous")
    return Layout(0, t.stride(1), t.stride(0))


def _problem(B, H, N, d, dtype, cu=None, total=0, **layouts) -> Problem:
    if dtype not in FA_DTYPE:
        raise ValueError("tensors must be bfloat16 or float16")
    pb = Problem(B=B, H=H, N=N, d=d, dtype=FA_DTYPE[dtype],
                 cu_seqlens=cu.data_ptr() if cu is not None else None, total_tokens=total)
    for name, lay in layouts.items():
        setattr(pb, name, lay)
    return pb


def fwd_ex(q, k, v, scale=None, causal=False, dropout_p=0.0, seed=0, out=None, lse=None):
    """Forward pass on strided [B, H, N, d] views (bf16 or fp16, d in {32, 64, 96,
    128, 256}), e.g. q.transpose(1, 2) of [B, N, H, d] storage. O gets q's strides
    unless `out` is given; LSE is [B, H, N] fp32."""
    B, H, N, d = q.shape
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v must share the [B, H, N, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share the dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    if lse.dim() != 3:
        raise ValueError("lse must be [B, H, N]")
    pb = _problem(B, H, N, d, q.dtype, q=_layout4(q, "q"), k=_layout4(k, "k"), v=_layout4(v, "v"),
                  o=_layout4(out, "out"), lse=Layout(lse.stride(0), lse.stride(1), lse.stride(2)))
    st = lib().fa_fwd_ex(ctypes.byref(pb), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), scale, int(bool(causal)), float(dropout_p),
                         int(seed) & (2**64 - 1), _stream(q.device))
    _check(st, "fa_fwd_ex")
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen, scale=None, causal=False, dropout_p=0.0, seed=0,
               out=None, lse=None):
    """Forward pass on packed sequences: q, k, v are [total, H, d] (bf16 or fp16),
    sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (int32 on the GPU, B+1
    entries), max_seqlen >= every length. Returns O [total, H, d] and LSE [H, total]."""
    total, H, d = q.shape
    if tuple(k.shape) != (total, H, d) or tuple(v.shape) != (total, H, d):
        raise ValueError("q, k, v must share the [total, H, d] shape")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor")
    B = cu_seqlens.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, total), dtype=torch.float32, device=q.device) if lse is None else lse
    pb = _problem(B, H, int(max_seqlen), d, q.dtype, cu=cu_seqlens, total=total,
                  q=_layout3(q, "q"), k=_layout3(k, "k"), v=_layout3(v, "v"),
                  o=_layout3(out, "out"), lse=Layout(0, lse.stride(0), lse.stride(1)))
    st = lib().fa_fwd_ex(ctypes.byref(pb), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), scale, int(bool(causal)), float(dropout_p),
                         int(seed) & (2**64 - 1), _stream(q.device))
    _check(st, "fa_fwd_ex")
    return out, lse


def _bwd_ex_call(pb, q, k, v, o, lse, do, dq, dk, dv, scale, causal, dropout_p, seed, deterministic,
                 workspace):
    need = int(lib().fa_bwd_ex_workspace_size(ctypes.byref(pb)))
    if need == 0:
        raise FAError(FA_ERR_INVALID_ARG, "fa_bwd_ex_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().fa_bwd_ex(ctypes.byref(pb), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         scale, int(bool(causal)), float(dropout_p), int(seed) & (2**64 - 1),
                         int(bool(deterministic)), workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st, "fa_bwd_ex")


def bwd_ex(q, k, v, o, lse, do, scale=None, causal=False, dropout_p=0.0, seed=0, dq=None, dk=None,
           dv=None, workspace=None, deterministic=False):
    """Backward of fwd_ex on strided [B, H, N, d] views (bf16 or fp16). Gradients
    take the strides of q, k, v unless given."""
    B, H, N, d = q.shape
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, do must share the [B, H, N, d] shape and dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    pb = _problem(B, H, N, d, q.dtype, q=_layout4(q, "q"), k=_layout4(k, "k"), v=_layout4(v, "v"),
                  o=_layout4(o, "o"), lse=Layout(lse.stride(0), lse.stride(1), lse.stride(2)),
                  dout=_layout4(do, "do"), dq=_layout4(dq, "dq"), dk=_layout4(dk, "dk"),
                  dv=_layout4(dv, "dv"))
    _bwd_ex_call(pb, q, k, v, o, lse, do, dq, dk, dv, scale, causal, dropout_p, seed, deterministic,
                 workspace)
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, scale=None, causal=False, dropout_p=0.0,
               seed=0, dq=None, dk=None, dv=None, workspace=None, deterministic=False):
    """Backward of fwd_varlen: packed [total, H, d] tensors, LSE [H, total]."""
    total, H, d = q.shape
    for t in (k, v, o, do):
        if tuple(t.shape) != (total, H, d) or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, do must share the [total, H, d] shape and dtype")
    B = cu_seqlens.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    pb = _problem(B, H, int(max_seqlen), d, q.dtype, cu=cu_seqlens, total=total,
                  q=_layout3(q, "q"), k=_layout3(k, "k"), v=_layout3(v, "v"), o=_layout3(o, "o"),
                  lse=Layout(0, lse.stride(0), lse.stride(1)), dout=_layout3(do, "do"),
                  dq=_layout3(dq, "dq"), dk=_layout3(dk, "dk"), dv=_layout3(dv, "dv"))
    _bwd_ex_call(pb, q, k, v, o, lse, do, dq, dk, dv, scale, causal, dropout_p, seed, deterministic,
                 workspace)
    return dq, dk, dv


def workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, N, d))


def bwd(q, k, v, o, lse, do, scale=None, causal=False, dropout_p=0.0, seed=0,
        dq=None, dk=None, dv=None, workspace=None, deterministic=False):
    """Backward pass: returns (dQ, dK, dV) in the input dtype. deterministic=True
    (bf16 only) computes dQ in its own pass, without atomics, so that the result
    is bitwise reproducible."""
    shp = _shape4(q, "q")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        if _shape4(t, n) != shp or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, do must share shape and dtype")
    B, H, N, d = shp
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if deterministic and q.dtype != torch.bfloat16:
        raise ValueError("the deterministic backward takes bfloat16 tensors")
    name = "fa_bwd_deterministic" if deterministic else "fa_bwd"
    st = _entry(q.dtype, name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), B, H, N, d, scale, int(bool(causal)),
                                   float(dropout_p), int(seed) & (2**64 - 1),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(q.device))
    _check(st, name)
    return dq, dk, dv


# Bytes of the library's own device scratch behind fa_bwd_noalloc (FA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 128 << 20


def bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale=None, causal=False, dropout_p=0.0, seed=0):
    """fa_bwd_noalloc: the bf16 backward with the library's own scratch, for
    callers that cannot allocate. The output tensors are the caller's; nothing
    is allocated here either."""
    shp = _shape4(q, "q")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        if _shape4(t, n) != shp or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, do, dq, dk, dv must share shape and dtype")
    if q.dtype != torch.bfloat16:
        raise ValueError("fa_bwd_noalloc takes bfloat16 tensors")
    B, H, N, d = shp
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                              scale, int(bool(causal)), float(dropout_p), int(seed) & (2**64 - 1),
                              _stream(q.device))
    _check(st, "fa_bwd_noalloc")
    return dq, dk, dv


def decode_workspace_size(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(lib().fa_fwd_decode_workspace_size(B, H, Nq, Nk, d))


def fwd_decode(q, k, v, scale=None, causal=False, out=None, lse=None, workspace=None):
    """Decode-shaped forward (bf16): q [B,H,Nq,d] against k, v [B,H,Nk,d], Nq <= Nk.
    Returns (O [B,H,Nq,d] bf16, LSE [B,H,Nq] fp32)."""
    B, H, Nq, d = _shape4(q, "q")
    kshp = _shape4(k, "k")
    if _shape4(v, "v") != kshp or kshp[:2] != (B, H) or kshp[3] != d:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H, d")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("fwd_decode takes bfloat16 tensors")
    Nk = kshp[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    need = decode_workspace_size(B, H, Nq, Nk, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             B, H, Nq, Nk, d, scale, int(bool(causal)), ws_ptr, ws_bytes,
                             _stream(q.device))
    _check(st, "fa_fwd_decode")
    return out, lse


def fwd_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale=None, causal=False, out=None,
                     lse=None, workspace=None):
    """Decode-shaped forward over a paged cache (bf16): q [B,H,Nq,d]; k_pages, v_pages
    [num_pages, H, page, d]; block_table [B, max_blocks] int32; seq_lens [B] int32 (GPU)."""
    B, H, Nq, d = _shape4(q, "q")
    num_pages, Hk, page, dk = _shape4(k_pages, "k_pages")
    if _shape4(v_pages, "v_pages") != (num_pages, Hk, page, dk) or Hk != H or dk != d:
        raise ValueError("k_pages and v_pages must be [num_pages, H, page, d] with q's H and d")
    for t, n in ((block_table, "block_table"), (seq_lens, "seq_lens")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    max_blocks = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    need = int(lib().fa_fwd_decode_paged_workspace_size(B, H, Nq, max_blocks, page, d))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fa_fwd_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                   block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, Nq, max_blocks, page, num_pages, d, scale,
                                   int(bool(causal)), ws_ptr, ws_bytes, _stream(q.device))
    _check(st, "fa_fwd_decode_paged")
    return out, lse


def dropout_mask(B, H, N, b, h, dropout_p, seed, device="cuda"):
    """[N, N] uint8 keep mask (1 = kept) of head (b, h), from the device generator."""
    mask = torch.empty((N, N), dtype=torch.uint8, device=device)
    st = lib().fa_dropout_mask(mask.data_ptr(), B, H, N, b, h, float(dropout_p),
                               int(seed) & (2**64 - 1), _stream(mask.device))
    _check(st, "fa_dropout_mask")
    return mask


__all__ = ["fwd", "bwd", "fwd_decode", "fwd_decode_paged", "dropout_mask", "workspace_size", "decode_workspace_size", "lib",
           "FAError", "LIB_PATH", "SIGNATURES"]
