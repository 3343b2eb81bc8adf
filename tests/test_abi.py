"""The C ABI without a GPU: libsol.so loads, exports every function that
include/sol.h declares, sizes workspaces, and rejects bad arguments on the
host before anything is enqueued (no kernel runs in these tests)."""
import ctypes
import math
import os
import re

import pytest

from block_sparse_attention_23_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sol.h")

FAKE = 0x10000  # 16-byte-aligned non-null address; validation fails before any use
FAKE_WS = 0x100000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sol_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB):
        build.build()
    return binding.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "sol_attn_dense", "sol_attn_fwd", "sol_attn_fwd_dbg", "sol_attn_fwd_noalloc",
        "sol_attn_fwd_variant", "sol_pool", "sol_route",
        "sol_status_string", "sol_sweep", "sol_sweep_timed", "sol_workspace_bytes"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(build.LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5):
        assert binding.status_string(st)
    assert binding.status_string(7) == "unknown status"


def test_workspace_bytes(lib):
    H, L, d, B = 40, 75600, 128, 64
    N = 1182
    n = binding.workspace_bytes(H, L, d, B)
    assert n >= 3 * H * N * d * 4 + H * N * 4
    assert n % 256 == 0
    assert binding.workspace_bytes(1, 1, 64, 64) > 0
    assert binding.workspace_bytes(1, 8192 * 32, 128, 32) > 0
    for bad in [(0, 10, 64, 64), (1, 0, 64, 64), (1, 10, 96, 64), (1, 10, 64, 16),
                (1, 8192 * 64 + 1, 64, 64), (1, 8192 * 32 + 1, 64, 32)]:
        assert binding.workspace_bytes(*bad) == 0


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, H=2, L=100, d=64, B=64, beta=1.0, dt=0, out=FAKE,
             kept=FAKE, ws=FAKE_WS, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.sol_attn_fwd(a["q"], a["k"], a["v"], a["H"], a["L"], a["d"], a["B"], a["beta"],
                            a["dt"], a["out"], a["kept"], a["ws"], a["ws_bytes"], a["stream"])


def test_forward_rejects_bad_arguments_before_launch(lib):
    assert _fwd(lib, q=None) == -1
    assert _fwd(lib, out=None) == -1
    assert _fwd(lib, kept=None) == -1
    assert _fwd(lib, H=0) == -1
    assert _fwd(lib, L=-5) == -1
    assert _fwd(lib, d=96) == -2
    assert _fwd(lib, B=16) == -2
    assert _fwd(lib, B=96) == -2
    assert _fwd(lib, L=8192 * 64 + 1) == -2
    assert _fwd(lib, beta=math.nan) == -1
    assert _fwd(lib, dt=5) == -1
    assert _fwd(lib, q=FAKE + 2) == -1          # misaligned
    assert _fwd(lib, ws=None) == -3
    assert _fwd(lib, ws=FAKE_WS + 16) == -3     # workspace must be 256-byte aligned
    assert _fwd(lib, ws_bytes=16) == -3


def test_pool_and_dense_reject_bad_arguments(lib):
    assert lib.sol_pool(FAKE, FAKE, None, 1, 10, 64, 64, 0, FAKE, FAKE, FAKE, None) == -1
    assert lib.sol_pool(FAKE, FAKE, FAKE, 1, 10, 64, 48, 0, FAKE, FAKE, FAKE, None) == -2
    assert lib.sol_attn_dense(FAKE, FAKE, FAKE, 1, 10, 80, 0, FAKE, None) == -2
    assert lib.sol_attn_dense(FAKE, None, FAKE, 1, 10, 64, 0, FAKE, None) == -1
    assert lib.sol_attn_dense(FAKE, FAKE, FAKE, 1, 10, 64, 3, FAKE, None) == -1


def test_stage_entry_points_reject_bad_arguments(lib):
    assert lib.sol_route(FAKE, None, 1, 100, 64, 64, 1.0, FAKE, FAKE, None, FAKE_WS, 1 << 30, None) == -1
    assert lib.sol_route(FAKE, FAKE, 1, 100, 64, 64, math.nan, FAKE, FAKE, None, FAKE_WS, 1 << 30, None) == -1
    assert lib.sol_route(FAKE, FAKE, 1, 100, 64, 16, 1.0, FAKE, FAKE, None, FAKE_WS, 1 << 30, None) == -2
    assert lib.sol_route(FAKE, FAKE, 1, 100, 64, 64, 1.0, FAKE, FAKE, FAKE + 2, FAKE_WS, 1 << 30, None) == -1
    assert lib.sol_route(FAKE, FAKE, 1, 100, 64, 64, 1.0, FAKE, FAKE, None, None, 1 << 30, None) == -3
    assert lib.sol_route(FAKE, FAKE, 1, 100, 64, 64, 1.0, FAKE, FAKE, None, FAKE_WS, 16, None) == -3
    args = [FAKE] * 7 + [1, 100, 64, 64, 0, FAKE, FAKE_WS, 1 << 30, None, None, None]
    bad = list(args)
    bad[13] = None  # workspace
    assert lib.sol_sweep(*bad) == -3
    bad = list(args)
    bad[14] = 64  # workspace too small
    assert lib.sol_sweep(*bad) == -3
    bad = list(args)
    bad[6] = None  # tau
    assert lib.sol_sweep(*bad) == -1
    bad = list(args)
    bad[9] = 96  # d
    assert lib.sol_sweep(*bad) == -2
    bad = list(args)
    bad[15] = FAKE + 2  # misaligned selection bits
    assert lib.sol_sweep(*bad) == -1


def test_sweep_timed_rejects_bad_arguments(lib):
    # (q, k, v, qbar, kbar, vsum, tau, H, L, d, B, dt, out, ws, ws_bytes, bits, order, clock, stream)
    ok = [FAKE] * 7 + [1, 100, 64, 64, 0, FAKE, FAKE_WS, 1 << 30, FAKE, None, FAKE, None]
    for i, val, want in [(11, 1, -2),       # fp32 inputs: bf16 sweep only
                         (15, None, -1),    # selection bits required
                         (17, None, -1),    # clock records required
                         (16, FAKE + 2, -1),  # misaligned order
                         (13, None, -3)]:   # workspace
        bad = list(ok)
        bad[i] = val
        assert lib.sol_sweep_timed(*bad) == want, (i, val)


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.attn_fwd(x, x, x, 64, 1.0)
    with pytest.raises(ValueError):
        binding.attn_dense(x, x, x)


def test_unpack_mask_bit_order():
    import numpy as np
    import torch
    m = torch.tensor([[[0b1011, 1 << 31]]], dtype=torch.int64).to(torch.int32)
    bits = binding.unpack_mask(m, 33)
    assert bits.shape == (1, 1, 33)
    assert list(np.nonzero(bits[0, 0])[0]) == [0, 1, 3]
    m2 = torch.tensor([[[0, 1]]], dtype=torch.int32)
    assert list(np.nonzero(binding.unpack_mask(m2, 40)[0, 0])[0]) == [32]


def test_variant_rejects_bad_flags_and_fractions(lib):
    # (q, k, v, H, L, d, B, beta, keep_frac, flags, dt, out, kept, ws, ws_bytes, stream, mask, tau)
    ok = [FAKE, FAKE, FAKE, 1, 100, 64, 64, 1.0, 0.5, 0, 0, FAKE, FAKE, FAKE_WS, 1 << 30, None,
          None, None]
    for i, val, want in [(9, 8, -1), (9, 2 | 8, -1), (9, 2 | 4, -1), (8, math.nan, -1), (8, -0.1, -1),
                         (8, 1.5, -1), (10, 1, -2)]:
        bad = list(ok)
        bad[i] = val
        if i == 10:
            bad[9] = 1  # drop with fp32 inputs
        if i == 8:
            bad[9] = 2  # the fraction matters for the fixed budget only
        assert lib.sol_attn_fwd_variant(*bad) == want, (i, val)


def test_noalloc_rejects_on_the_host(lib):
    """sol_attn_fwd_noalloc checks its arguments, then the scratch its shape
    needs against SOL_NOALLOC_SCRATCH_BYTES, before any HIP call."""
    def call(H=2, L=100, d=64, B=64, beta=1.0, dt=0, q=FAKE, out=FAKE, kept=FAKE):
        return lib.sol_attn_fwd_noalloc(q, FAKE, FAKE, H, L, d, B, beta, dt, out, kept, None)
    assert call(q=None) == -1
    assert call(kept=None) == -1
    assert call(beta=math.nan) == -1
    assert call(d=96) == -2
    assert call(out=FAKE + 2) == -1
    # 24 heads of 131,072 tokens at d = 128: B = 32 needs about 200 MB (too
    # much), B = 64 about 90 MB (fits in the 96 MiB)
    assert call(H=24, L=131072, d=128, B=32) == -5
    assert "scratch" in binding.status_string(-5)


def test_library_built_from_current_sources(lib):
    """build() records the digest of the sources and flags it compiled; the
    library in the tree matches the sources in the tree."""
    assert build.built_digest() == build.source_digest()


def test_digest_does_not_depend_on_the_tree_location():
    """The tree is built in one directory and run from another: no path may
    enter the digest."""
    assert not any(build.ROOT in f or f.startswith("-I") for f in build.digest_flags())


def test_stale_library_is_refused(monkeypatch):
    """A library built from other sources (digest mismatch) is not loaded."""
    monkeypatch.setattr(binding, "_LIB", None)
    monkeypatch.setattr(build, "source_digest", lambda extra=(): "0" * 64)
    with pytest.raises(RuntimeError, match="stale"):
        binding.lib()


def test_stale_oracle_is_refused(monkeypatch):
    import oracle
    from oracle import build as obuild
    monkeypatch.setattr(oracle, "_LIB", None)
    monkeypatch.setattr(obuild, "source_digest", lambda: "0" * 64)
    with pytest.raises(RuntimeError, match="stale"):
        oracle.lib()
