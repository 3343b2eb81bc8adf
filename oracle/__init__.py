"""fp64 CPU oracle of the Sol-Attn forward pass (ctypes front end).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product (the HIP library and its
binding) never imports this package, and this package never imports the
product.  The arithmetic lives in ``sol_oracle.c``; this module only moves
numpy arrays across the C boundary and composes the steps in the pages'
order: pool -> proxy / threshold / selection -> merge.

Sources: "Sol-Attn" visual paper explainer (mxino.github.io), Eq. (4),
Eq. (5), Eq. (9), Eq. (10), Eq. (11); Sol-Attn abstract.
"""
import contextlib
import ctypes
import math
import os

import numpy as np

from . import build as _build

_LIB = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)


def _load(path):
    L = ctypes.CDLL(path)
    L.sol_oracle_pool.argtypes = [_fp, _fp, _fp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, _dp, _dp, _dp]
    L.sol_oracle_route.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, _dp, _dp, _dp, _dp, _u8p, _i32p]
    L.sol_oracle_moments.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _dp, _dp]
    L.sol_oracle_merge.argtypes = [_fp, _fp, _fp, _dp, _dp, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, _u8p, ctypes.c_int64, _i32p, _dp]
    L.sol_oracle_merge_ex.argtypes = [_fp, _fp, _fp, _dp, _dp, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, _u8p, ctypes.c_int,
                                      ctypes.c_int64, _i32p, _dp]
    L.sol_oracle_route_topk.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, _dp, _dp, _u8p, _i32p]
    L.sol_oracle_dense.argtypes = [_fp, _fp, _fp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int64, _i32p, _dp]
    L.sol_oracle_num_threads.argtypes = []
    for f in ("sol_oracle_pool", "sol_oracle_route", "sol_oracle_moments",
              "sol_oracle_merge", "sol_oracle_merge_ex", "sol_oracle_route_topk",
              "sol_oracle_dense", "sol_oracle_num_threads"):
        getattr(L, f).restype = ctypes.c_int
    return L


def lib():
    """The loaded oracle library, built here if it is missing; raises if the
    library present was built from another version of sol_oracle.c."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        if _build.built_digest() != _build.source_digest():
            raise RuntimeError(f"{_build.LIB} is stale: it was not built from the current "
                               "sol_oracle.c (rebuild with `python -m oracle.build`)")
        _LIB = _load(_build.LIB)
    return _LIB


@contextlib.contextmanager
def using_library(path):
    """Run the oracle from another build of its source (used to check that the
    pins reject deliberately broken copies of the oracle)."""
    global _LIB
    saved = _LIB
    _LIB = _load(path)
    try:
        yield
    finally:
        _LIB = saved


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _f32(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 3:
        raise ValueError("token tensors must be [H][L][d]")
    return x


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def nblocks(L, B):
    return (L + B - 1) // B


def pool(q, k, v, B):
    """Per-block mean of Q and K and per-block sum of V, [H][N][d] float64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    H, L, d = q.shape
    N = nblocks(L, B)
    qbar = np.empty((H, N, d)); kbar = np.empty((H, N, d)); vsum = np.empty((H, N, d))
    _check(lib().sol_oracle_pool(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), H, L, d, B,
                                 _ptr(qbar, _dp), _ptr(kbar, _dp), _ptr(vsum, _dp)), "pool")
    return qbar, kbar, vsum


def route(qbar, kbar, beta, want_shat=False):
    """Proxy row, mu, sigma, tau, selection mask and kept count per (h, i).

    Returns a dict with ``sel`` [H][N][N] uint8, ``kept`` [H][N] int32,
    ``mu``, ``sigma``, ``tau`` [H][N] float64 and optionally ``shat``.
    """
    qbar = np.ascontiguousarray(qbar, dtype=np.float64)
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    H, N, d = qbar.shape
    if math.isnan(beta):
        raise ValueError("beta is NaN")
    out = {
        "mu": np.empty((H, N)), "sigma": np.empty((H, N)), "tau": np.empty((H, N)),
        "sel": np.empty((H, N, N), dtype=np.uint8), "kept": np.empty((H, N), dtype=np.int32),
        "shat": np.empty((H, N, N)) if want_shat else None,
    }
    _check(lib().sol_oracle_route(_ptr(qbar, _dp), _ptr(kbar, _dp), H, N, d, float(beta),
                                  _ptr(out["shat"], _dp), _ptr(out["mu"], _dp),
                                  _ptr(out["sigma"], _dp), _ptr(out["tau"], _dp),
                                  _ptr(out["sel"], _u8p), _ptr(out["kept"], _i32p)), "route")
    return out


def moments(qbar, kbar):
    """Eq. (5) moment form: (mu, sigma^2) per (h, i)."""
    qbar = np.ascontiguousarray(qbar, dtype=np.float64)
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    H, N, d = qbar.shape
    mu = np.empty((H, N)); s2 = np.empty((H, N))
    _check(lib().sol_oracle_moments(_ptr(qbar, _dp), _ptr(kbar, _dp), H, N, d,
                                    _ptr(mu, _dp), _ptr(s2, _dp)), "moments")
    return mu, s2


def _rows_arg(rows):
    if rows is None:
        return None, 0
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
    return rows, rows.shape[0]


def route_topk(qbar, kbar, k, want_shat=False):
    """Fixed-budget comparator: the k largest proxy scores of every query
    block (ties to the lower block index).  Returns a dict with ``sel``,
    ``kept`` (= k), ``kth`` (the k-th largest score) and optionally ``shat``."""
    qbar = np.ascontiguousarray(qbar, dtype=np.float64)
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    H, N, d = qbar.shape
    out = {"kth": np.empty((H, N)), "sel": np.empty((H, N, N), dtype=np.uint8),
           "kept": np.empty((H, N), dtype=np.int32),
           "shat": np.empty((H, N, N)) if want_shat else None}
    _check(lib().sol_oracle_route_topk(_ptr(qbar, _dp), _ptr(kbar, _dp), H, N, d, int(k),
                                       _ptr(out["shat"], _dp), _ptr(out["kth"], _dp),
                                       _ptr(out["sel"], _u8p), _ptr(out["kept"], _i32p)),
           "route_topk")
    return out


def topk_count(keep_frac, N):
    """Blocks a fixed-budget row keeps for a kept fraction: round(keep_frac * N)
    (halves up), clamped to [0, N]."""
    return int(min(N, max(0, math.floor(keep_frac * N + 0.5))))


def merge(q, k, v, kbar, vsum, B, sel, rows=None, drop_approx=False):
    """Eq. (9)/(10) merge for every row ([H][L][d]) or for (h, r) pairs ([n][d]).
    drop_approx: leave the unselected blocks out (keep-or-drop)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    H, L, d = q.shape
    N = nblocks(L, B)
    sel = np.ascontiguousarray(sel, dtype=np.uint8)
    if sel.shape != (H, N, N):
        raise ValueError(f"sel must be [H][N][N] = {(H, N, N)}, got {sel.shape}")
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    vsum = np.ascontiguousarray(vsum, dtype=np.float64)
    rows, n = _rows_arg(rows)
    out = np.empty((H, L, d)) if rows is None else np.empty((n, d))
    _check(lib().sol_oracle_merge_ex(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp),
                                     _ptr(kbar, _dp), _ptr(vsum, _dp), H, L, d, B,
                                     _ptr(sel, _u8p), int(bool(drop_approx)), n,
                                     _ptr(rows, _i32p), _ptr(out, _dp)), "merge")
    return out


def dense(q, k, v, rows=None):
    """Textbook softmax(Q K^T / sqrt(d)) V in fp64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    H, L, d = q.shape
    rows, n = _rows_arg(rows)
    out = np.empty((H, L, d)) if rows is None else np.empty((n, d))
    _check(lib().sol_oracle_dense(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), H, L, d, n,
                                  _ptr(rows, _i32p), _ptr(out, _dp)), "dense")
    return out


def attention(q, k, v, B, beta, sel=None, rows=None):
    """The whole forward pass in the pages' order.

    pool -> route (unless a selection ``sel`` is injected) -> merge.
    Returns (out, route_dict).
    """
    qbar, kbar, vsum = pool(q, k, v, B)
    r = route(qbar, kbar, beta)
    use = r["sel"] if sel is None else sel
    out = merge(q, k, v, kbar, vsum, B, use, rows=rows)
    r.update(qbar=qbar, kbar=kbar, vsum=vsum)
    return out, r


def num_threads():
    return lib().sol_oracle_num_threads()
