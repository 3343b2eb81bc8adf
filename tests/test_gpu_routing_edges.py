"""Routing edge cases on the GPU against the fp64 oracle ("Sol-Attn" visual
explainer, Eq. (4) and Eq. (5)): proxy rows whose mean is large against their
spread, and constant proxy rows (sigma = 0), on both of the routing kernel's
paths -- rows held on chip (N <= 1280) and thresholds from the centred key
moments (N > 1280).  Selection is compared for every (h, i, j) with the flip
rule; outputs on sampled query blocks (every row for the small cases)."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_23_amd import binding
from block_sparse_attention_23_amd import inputs as gen

from .parity import block_rows, run_and_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


_BASE = {}


def base(B, nblocks, tail):
    """Two heads of the Fourier-feature generator, nblocks blocks of B tokens
    with a last block `tail` tokens short."""
    key = (B, nblocks, tail)
    if key not in _BASE:
        _BASE.clear()
        L = nblocks * B - tail
        X = 64
        T = -(-L // (64 * X))
        _BASE[key] = gen.grid_inputs(2, (T, 64, X), 128, seed=41, dtype="bf16", truncate=L)
    return _BASE[key]


def sampled_rows(L, B, N, heads=(0, 1)):
    blocks = sorted({0, 1, N // 3, N // 2, N - 2, N - 1})
    return block_rows(L, B, [(h, i) for h in heads for i in blocks])


def unit(d, seed=5):
    u = np.random.default_rng(seed).standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


@pytest.mark.parametrize("beta", [0.5, 1.0, 2.0])
def test_large_common_key_component_moment_route(beta):
    """N = 2048 (moment route).  Every key carries 60 u and every query 4 u
    for one unit vector u: the proxy rows' |mu| / sigma is about 100, where
    the uncentred moment form loses several 1e-3 of tau."""
    inp0 = base(64, 2048, 21)
    u = unit(128)
    inp = gen.shifted_inputs(inp0, q_shift=4.0 * u, k_shift=60.0 * u)
    L, N = inp.q.shape[1], 2048
    s = run_and_check(inp, 64, beta, rows=sampled_rows(L, 64, N))
    print(f"offset keys beta={beta}: kept={s['kept_frac']:.4f} flips={s['flips']} "
          f"max_err={s['max_err']:.2e}", flush=True)
    assert 0.0 < s["kept_frac"] < 0.5


@pytest.mark.parametrize("beta", [0.5, 1.0])
def test_large_common_key_component_row_route(beta):
    """The same offsets at N = 1000 (rows held on chip, two-pass statistics)."""
    inp0 = base(64, 1000, 5)
    u = unit(128)
    inp = gen.shifted_inputs(inp0, q_shift=4.0 * u, k_shift=60.0 * u)
    L = inp.q.shape[1]
    s = run_and_check(inp, 64, beta, rows=sampled_rows(L, 64, 1000))
    assert 0.0 < s["kept_frac"] < 0.5


@pytest.mark.parametrize("B,nblocks,tail", [(64, 2048, 21), (64, 1000, 5), (32, 1500, 7),
                                            (128, 1400, 5), (64, 16, 0)])
def test_equal_keys_select_nothing(B, nblocks, tail):
    """Every key token equal: all pooled keys are equal, every proxy row is
    constant (sigma = 0, tau = mu), and no block is strictly above its
    threshold, on either routing path; beta = -inf still selects every
    block.  Outputs against the oracle."""
    inp0 = base(B, nblocks, tail)
    inp = gen.shifted_inputs(inp0, k_const=inp0.k[0, 0])
    L = inp.q.shape[1]
    rows = None if nblocks <= 16 else sampled_rows(L, B, nblocks)
    for beta in (0.0, 1.0, -math.inf):
        s = run_and_check(inp, B, beta, rows=rows)
        assert s["flips"] == 0
        assert s["kept_frac"] == (1.0 if beta == -math.inf else 0.0), (beta, s)
