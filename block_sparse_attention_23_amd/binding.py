"""Thin ctypes binding of libsol.so (the C ABI in include/sol.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the stream.  There
is no fallback: a missing library or a non-GPU tensor raises.
"""
import ctypes
import math
import os

import torch

from . import build as _build

SOL_BF16, SOL_F32 = 0, 1
SOL_DROP_APPROX, SOL_TOPK, SOL_FUSED_ROUTE = 1, 2, 4

_FUNCS = {
    "sol_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "sol_pool": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 5
                 + [ctypes.c_void_p] * 4),
    "sol_route": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] * 4
                  + [ctypes.c_float] + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sol_sweep": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 5
                  + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_void_p] * 3),
    "sol_sweep_timed": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 5
                        + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_void_p] * 4),
    "sol_attn_fwd": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4
                     + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "sol_attn_fwd_dbg": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4
                         + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                            ctypes.c_void_p, ctypes.c_void_p]),
    "sol_attn_fwd_variant": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4
                             + [ctypes.c_float, ctypes.c_float, ctypes.c_uint, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "sol_attn_fwd_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4
                             + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]),
    "sol_attn_dense": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4
                       + [ctypes.c_void_p, ctypes.c_void_p]),
    "sol_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_LIB = None


class SolError(RuntimeError):
    def __init__(self, func, status):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} (status {status})")


def library_path():
    return _build.LIB


def lib():
    """The loaded libsol.so; raises if it is missing or was built from other
    sources than those in the tree."""
    global _LIB
    if _LIB is None:
        _build.check_current()  # missing or stale (built from other sources): raise
        L = ctypes.CDLL(_build.LIB)
        for name, (res, args) in _FUNCS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def status_string(status):
    return lib().sol_status_string(int(status)).decode()


def _check(func, status):
    if status != 0:
        raise SolError(func, status)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SOL_BF16
    if t.dtype == torch.float32:
        return SOL_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _tokens(*ts):
    q = ts[0]
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (no CPU path exists)")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError("token tensors must be contiguous [H][L][d]")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share shape, dtype and device")
    return q.shape


def _stream_ptr(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream, device):
    """Context in which tensors the binding creates are allocated: the stream
    the kernels run on.  The caching allocator then hands a freed block
    (a temporary workspace, say) to later work on that same stream only, so
    no other stream can reuse it while those kernels still read or write it."""
    with torch.cuda.device(device):
        s = stream if stream is not None else torch.cuda.current_stream(device)
    return torch.cuda.stream(s)


def nblocks(L, B):
    return (L + B - 1) // B


def workspace_bytes(H, L, d, B):
    return int(lib().sol_workspace_bytes(H, L, d, B))


def alloc_workspace(H, L, d, B, device):
    n = workspace_bytes(H, L, d, B)
    if n == 0:
        raise ValueError(f"unsupported shape H={H} L={L} d={d} B={B}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def pool(q, k, v, B, outs=None, stream=None):
    """Block means of q and k and block sums of v, fp32 [H][N][d]."""
    H, L, d = _tokens(q, k, v)
    N = nblocks(L, B)
    if outs is None:
        with _on(stream, q.device):
            outs = [torch.empty((H, N, d), dtype=torch.float32, device=q.device) for _ in range(3)]
    with torch.cuda.device(q.device):
        _check("sol_pool", lib().sol_pool(q.data_ptr(), k.data_ptr(), v.data_ptr(), H, L, d, B,
                                          _dtype_code(q), outs[0].data_ptr(), outs[1].data_ptr(),
                                          outs[2].data_ptr(), _stream_ptr(stream, q.device)))
    return tuple(outs)


def route(qbar, kbar, L, B, beta, tau=None, kept=None, sel_bits=None, workspace=None, stream=None):
    """Thresholds tau [H][N] and kept counts [H][N] from pooled tensors; with
    sel_bits (int32 [H][N][ceil(N/32)]) also the decisions as bits."""
    H, N, d = qbar.shape
    if not (qbar.is_cuda and kbar.is_cuda):
        raise ValueError("pooled tensors must live on the GPU")
    with _on(stream, qbar.device):
        if tau is None:
            tau = torch.empty((H, N), dtype=torch.float32, device=qbar.device)
        if kept is None:
            kept = torch.empty((H, N), dtype=torch.int32, device=qbar.device)
        if workspace is None:
            workspace = alloc_workspace(H, L, d, B, qbar.device)
    with torch.cuda.device(qbar.device):
        _check("sol_route", lib().sol_route(qbar.data_ptr(), kbar.data_ptr(), H, L, d, B,
                                            float(beta), tau.data_ptr(), kept.data_ptr(),
                                            None if sel_bits is None else sel_bits.data_ptr(),
                                            workspace.data_ptr(), workspace.numel(),
                                            _stream_ptr(stream, qbar.device)))
    return tau, kept


def sel_words(N):
    """uint32 words per selection row."""
    return (N + 31) // 32


def sweep(q, k, v, qbar, kbar, vsum, tau, B, out=None, workspace=None, sel_bits=None,
          sel_mask=None, stream=None):
    """The fused exact/approximate sweep given pooled tensors and thresholds
    (and, optionally, the decisions sol_route wrote for them)."""
    H, L, d = _tokens(q, k, v)
    with _on(stream, q.device):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = alloc_workspace(H, L, d, B, q.device)
    with torch.cuda.device(q.device):
        _check("sol_sweep", lib().sol_sweep(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), qbar.data_ptr(), kbar.data_ptr(),
            vsum.data_ptr(), tau.data_ptr(), H, L, d, B, _dtype_code(q), out.data_ptr(),
            workspace.data_ptr(), workspace.numel(),
            None if sel_bits is None else sel_bits.data_ptr(),
            None if sel_mask is None else sel_mask.data_ptr(), _stream_ptr(stream, q.device)))
    return out


def group_items(H, N, B):
    """Work items of the sweep: H heads x ceil(N / (128 / B)) groups of 128 query rows."""
    return H * -(-N // (128 // B))


def sweep_timed(q, k, v, qbar, kbar, vsum, tau, B, sel_bits, order=None, out=None, workspace=None,
                stream=None):
    """sol_sweep (bf16) recording, per group item, the claim time, end time
    (100 MHz clock) and workgroup; `order` (int32 [items]) claims the items in
    that order instead of from the per-XCD queues.  Returns (out, clock)
    with clock an int64 [items][3] tensor."""
    H, L, d = _tokens(q, k, v)
    n = group_items(H, nblocks(L, B), B)
    with _on(stream, q.device):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = alloc_workspace(H, L, d, B, q.device)
        clock = torch.zeros((n, 3), dtype=torch.int64, device=q.device)
    if order is not None and (order.dtype != torch.int32 or order.numel() != n or not order.is_cuda):
        raise ValueError(f"order must be a device int32 tensor of {n} items")
    with torch.cuda.device(q.device):
        _check("sol_sweep_timed", lib().sol_sweep_timed(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), qbar.data_ptr(), kbar.data_ptr(),
            vsum.data_ptr(), tau.data_ptr(), H, L, d, B, _dtype_code(q), out.data_ptr(),
            workspace.data_ptr(), workspace.numel(), sel_bits.data_ptr(),
            None if order is None else order.data_ptr(), clock.data_ptr(),
            _stream_ptr(stream, q.device)))
    return out, clock


def attn_fwd(q, k, v, B, beta, out=None, kept=None, workspace=None, stream=None, debug=False):
    """Sol-Attn forward.  Returns (out, kept_counts) or, with debug=True,
    (out, kept_counts, sel_mask [H][N][ceil(N/32)] int32 bits, tau [H][N])."""
    H, L, d = _tokens(q, k, v)
    N = nblocks(L, B)
    with _on(stream, q.device):
        if out is None:
            out = torch.empty_like(q)
        if kept is None:
            kept = torch.empty((H, N), dtype=torch.int32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(H, L, d, B, q.device)
        if debug:
            W = (N + 31) // 32
            mask = torch.zeros((H, N, W), dtype=torch.int32, device=q.device)
            tau = torch.empty((H, N), dtype=torch.float32, device=q.device)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), H, L, d, B, float(beta), _dtype_code(q),
            out.data_ptr(), kept.data_ptr(), workspace.data_ptr(), workspace.numel(),
            _stream_ptr(stream, q.device)]
    with torch.cuda.device(q.device):
        if not debug:
            _check("sol_attn_fwd", lib().sol_attn_fwd(*args))
            return out, kept
        _check("sol_attn_fwd_dbg", lib().sol_attn_fwd_dbg(*args, mask.data_ptr(), tau.data_ptr()))
        return out, kept, mask, tau


def attn_fwd_noalloc(q, k, v, B, beta, out=None, kept=None, stream=None):
    """Sol-Attn forward through sol_attn_fwd_noalloc: the library uses its
    static per-GPU scratch instead of a workspace (the C call allocates
    nothing; out and kept are created here when not given).  Returns
    (out, kept_counts)."""
    H, L, d = _tokens(q, k, v)
    N = nblocks(L, B)
    with _on(stream, q.device):
        if out is None:
            out = torch.empty_like(q)
        if kept is None:
            kept = torch.empty((H, N), dtype=torch.int32, device=q.device)
    with torch.cuda.device(q.device):
        _check("sol_attn_fwd_noalloc", lib().sol_attn_fwd_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), H, L, d, B, float(beta), _dtype_code(q),
            out.data_ptr(), kept.data_ptr(), _stream_ptr(stream, q.device)))
    return out, kept


def attn_fwd_variant(q, k, v, B, beta, keep_frac=0.0, drop_approx=False, topk=False, out=None,
                     kept=None, workspace=None, stream=None, fused_route=False, debug=True):
    """The forward pass with the pages' comparators (bf16): drop_approx leaves
    the unselected blocks out (keep-or-drop); topk selects the
    round(keep_frac * N) largest proxies of every query block instead of the
    threshold; fused_route takes the decisions inside the sweep, from the
    Eq. (5) thresholds (SOL_FUSED_ROUTE).  Returns (out, kept_counts,
    sel_mask bits, tau); with debug=False the last two are None and nothing
    records them."""
    H, L, d = _tokens(q, k, v)
    N = nblocks(L, B)
    with _on(stream, q.device):
        if out is None:
            out = torch.empty_like(q)
        if kept is None:
            kept = torch.empty((H, N), dtype=torch.int32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(H, L, d, B, q.device)
        mask = torch.zeros((H, N, (N + 31) // 32), dtype=torch.int32, device=q.device) if debug else None
        tau = torch.empty((H, N), dtype=torch.float32, device=q.device) if debug else None
    flags = ((SOL_DROP_APPROX if drop_approx else 0) | (SOL_TOPK if topk else 0) |
             (SOL_FUSED_ROUTE if fused_route else 0))
    with torch.cuda.device(q.device):
        _check("sol_attn_fwd_variant", lib().sol_attn_fwd_variant(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), H, L, d, B, float(beta), float(keep_frac),
            flags, _dtype_code(q), out.data_ptr(), kept.data_ptr(), workspace.data_ptr(),
            workspace.numel(), _stream_ptr(stream, q.device), mask.data_ptr() if debug else None,
            tau.data_ptr() if debug else None))
    return out, kept, mask, tau


def attn_dense(q, k, v, out=None, stream=None):
    """Dense softmax(q k^T / sqrt(d)) v on the same tile machinery."""
    H, L, d = _tokens(q, k, v)
    if out is None:
        with _on(stream, q.device):
            out = torch.empty_like(q)
    with torch.cuda.device(q.device):
        _check("sol_attn_dense", lib().sol_attn_dense(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                      H, L, d, _dtype_code(q), out.data_ptr(),
                                                      _stream_ptr(stream, q.device)))
    return out


def unpack_mask(mask, N):
    """[H][N][W] int32 bit words -> [H][N][N] uint8 (host numpy)."""
    import numpy as np
    m = mask.cpu().numpy().view(np.uint32)
    bits = np.unpackbits(m.view(np.uint8), axis=-1, bitorder="little")
    return bits[..., :N].astype(np.uint8)
