"""HIP path vs the fp64 oracle at the workloads' full sizes, in the launch
configuration the benchmark times (every head and query block runs on the
GPU).  Selection parity is checked for every (h, i, j).  Outputs are
compared element by element: every element where the oracle is cheap (C2 at
both betas; C5 and C5b at beta = 3; one whole head of C3 at beta = 1, of C4
at beta = 1 and of C6 and C6b at beta = 1.25, each with sampled blocks of the
first, middle and last heads), elsewhere on sampled query
blocks that the oracle computes one by one, including the first, middle and
ragged last block of first, middle and last heads.  The dense kernel (the
speedup baseline) is compared with textbook attention on sampled C3 rows."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_23_amd import binding
from block_sparse_attention_23_amd import inputs as gen

from .parity import block_rows, check_output, run_and_check, to_device

pytestmark = pytest.mark.gpu

_CACHE = {}


def workload_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()  # keep one workload in host memory at a time
        _CACHE[name] = gen.generate(gen.WORKLOADS[name])
    return _CACHE[name]


CASES = [(n, b) for n in ("C2", "C3", "C4", "C5", "C5b", "C6", "C6b") for b in gen.WORKLOADS[n].betas]

# (workload, beta) -> heads whose every output element is compared
EVERY_ELEMENT = {("C2", -math.inf): "all", ("C2", 1.0): "all", ("C5", 3.0): "all",
                 ("C5b", 3.0): "all", ("C3", 1.0): [20], ("C4", 1.0): [11], ("C6", 1.25): [7],
                 ("C6b", 1.25): [17]}


def sampled_blocks(N):
    return sorted({0, 1, N // 3, N // 2, N - 2, N - 1})


@pytest.mark.parametrize("name,beta", CASES, ids=[f"{n}-beta{b}" for n, b in CASES])
def test_workload_full_size(name, beta):
    assert torch.cuda.is_available()
    w = gen.WORKLOADS[name]
    inp = workload_inputs(name)
    H, N, L, B = w.H, w.N, w.L, w.B
    full = EVERY_ELEMENT.get((name, beta))
    if full == "all":
        rows = None
    else:
        heads = sorted({0, H // 2, H - 1})
        pairs = [(h, i) for h in heads for i in sampled_blocks(N)]
        if full:
            pairs = [(h, i) for h in heads if h not in full for i in sampled_blocks(N)]
            pairs += [(h, i) for h in full for i in range(N)]
        rows = block_rows(L, B, pairs)
    s = run_and_check(inp, B, beta, rows=rows)
    print(f"{name} beta={beta}: kept={s['kept_frac']:.4f} flips={s['flips']} "
          f"max_err={s['max_err']:.3e} mean_err={s['mean_err']:.3e} over {s['compared']} elements",
          flush=True)
    if full == "all":
        assert s["compared"] == H * L * w.d
    elif full:
        assert s["compared"] >= len(full) * L * w.d
    if beta == -math.inf:
        assert s["kept_frac"] == 1.0


def test_dense_kernel_c3_sampled_rows():
    """sol_attn_dense over the whole C3 layer; sampled query blocks of the
    first, middle and last heads against textbook softmax attention."""
    w = gen.WORKLOADS["C3"]
    inp = workload_inputs("C3")
    q, k, v = to_device(inp)
    out = binding.attn_dense(q, k, v)
    torch.cuda.synchronize()
    heads = sorted({0, w.H // 2, w.H - 1})
    rows = block_rows(w.L, w.B, [(h, i) for h in heads for i in sampled_blocks(w.N)])
    ref = oracle.dense(inp.q, inp.k, inp.v, rows=rows)
    hidx = torch.tensor(rows[:, 0], device=out.device, dtype=torch.long)
    ridx = torch.tensor(rows[:, 1], device=out.device, dtype=torch.long)
    got = out[hidx, ridx].float().cpu().numpy()
    s = check_output(got, ref, "bf16")
    print(f"C3 dense: max_err={s['max_err']:.3e} mean_err={s['mean_err']:.3e} over {got.size} elements",
          flush=True)


def test_full_size_forward_is_bit_reproducible():
    """C3 at beta = 1 (23,640 work items over the persistent workgroups, so
    which workgroup takes which item varies from run to run): three forward
    passes give bit-identical outputs, counts and decisions, because each
    item's tile order is fixed."""
    w = gen.WORKLOADS["C3"]
    q, k, v = to_device(workload_inputs("C3"))
    runs = [binding.attn_fwd(q, k, v, w.B, 1.0, debug=True) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            assert torch.equal(x, y)
