"""HIP path vs the fp64 oracle at the workloads' full sizes, in the launch
configuration the benchmark times (every head and query block runs on the
GPU).  Selection parity is checked for every (h, i, j); outputs are compared
element by element on sampled query blocks that the oracle computes one by
one, including the first, middle and ragged last block of first, middle and
last heads."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_23_amd import binding
from block_sparse_attention_23_amd import inputs as gen

from .parity import block_rows, run_and_check

pytestmark = pytest.mark.gpu

_CACHE = {}


def workload_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()  # keep one workload in host memory at a time
        _CACHE[name] = gen.generate(gen.WORKLOADS[name])
    return _CACHE[name]


CASES = [(n, b) for n in ("C2", "C3", "C4", "C5", "C5b", "C6", "C6b") for b in gen.WORKLOADS[n].betas]


@pytest.mark.parametrize("name,beta", CASES, ids=[f"{n}-beta{b}" for n, b in CASES])
def test_workload_full_size(name, beta):
    assert torch.cuda.is_available()
    w = gen.WORKLOADS[name]
    inp = workload_inputs(name)
    H, N, L, B = w.H, w.N, w.L, w.B
    heads = sorted({0, H // 2, H - 1})
    blocks = sorted({0, 1, N // 3, N // 2, N - 2, N - 1})
    rows = block_rows(L, B, [(h, i) for h in heads for i in blocks])
    s = run_and_check(inp, B, beta, rows=rows)
    print(f"{name} beta={beta}: kept={s['kept_frac']:.4f} flips={s['flips']} "
          f"max_err={s['max_err']:.3e} mean_err={s['mean_err']:.3e}", flush=True)
    if beta == -math.inf:
        assert s["kept_frac"] == 1.0
