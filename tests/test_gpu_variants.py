"""The comparators the pages contrast Sol-Attn with (keep-or-drop, and a
fixed top-k budget), HIP path vs the fp64 oracle through the C ABI.

Selection: the threshold variant follows the same flip rule as the main
path; the fixed budget must keep exactly k blocks per query block and agree
with the oracle's ranking except for blocks whose oracle score lies within
1e-3 of the oracle's k-th largest score (fp32 vs fp64 ranking at the cut).
Outputs: compared with the oracle's merge (with or without the unselected
blocks) recomputed on the kernel's own selection, to the bf16 tolerance."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_23_amd import binding
from block_sparse_attention_23_amd import inputs as gen

from .parity import FLIP_BAND, TOL, block_rows, check_selection, check_output, to_device

pytestmark = pytest.mark.gpu
INF = math.inf


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def grid_inp(H, L, d, seed=0):
    W = max(1, -(-L // 64))
    return gen.grid_inputs(H, (4, 16, W), d, seed, "bf16", truncate=L)


def run_variant(inp, B, beta, keep_frac, drop, topk, rows=None):
    q, k, v = to_device(inp)
    out, kept, mask, tau = binding.attn_fwd_variant(q, k, v, B, beta, keep_frac=keep_frac,
                                                    drop_approx=drop, topk=topk)
    torch.cuda.synchronize()
    H, L, d = q.shape
    N = (L + B - 1) // B
    gsel = binding.unpack_mask(mask, N)
    gkept = kept.cpu().numpy()
    if topk:
        qbar, kbar, vsum = oracle.pool(inp.q, inp.k, inp.v, B)
        kk = oracle.topk_count(keep_frac, N)
        r = oracle.route_topk(qbar, kbar, kk, want_shat=True)
        assert (gkept == kk).all() and (gsel.sum(-1) == kk).all()
        near_cut = np.abs(r["shat"] - r["kth"][:, :, None]) < FLIP_BAND
        bad = (gsel != r["sel"]) & ~near_cut
        assert not bad.any(), f"{int(bad.sum())} ranking mismatches away from the cut"
        if kk > 0:
            gt = tau.cpu().numpy()
            assert np.all(np.abs(gt - r["kth"]) < FLIP_BAND)
    else:
        _, _, (qbar, kbar, vsum) = check_selection(inp.q, inp.k, inp.v, B, beta, gsel, gkept)
    ref = oracle.merge(inp.q, inp.k, inp.v, kbar, vsum, B, gsel, rows=rows, drop_approx=drop)
    if rows is None:
        got = out.float().cpu().numpy()
    else:
        got = out[torch.tensor(rows[:, 0], device=out.device, dtype=torch.long),
                  torch.tensor(rows[:, 1], device=out.device, dtype=torch.long)].float().cpu().numpy()
    stats = check_output(got, ref, "bf16")
    stats["kept_frac"] = float(gsel.mean())
    return stats, out


@pytest.mark.parametrize("d,B,L", [(128, 64, 1000), (64, 128, 700), (128, 64, 130), (128, 32, 1000)])
@pytest.mark.parametrize("drop,topk", [(True, False), (False, True), (True, True)])
def test_variants_small(d, B, L, drop, topk):
    inp = grid_inp(2, L, d, seed=12)
    s, _ = run_variant(inp, B, 1.0, 0.15, drop, topk)
    assert s["max_err"] <= TOL["bf16"][0]


def test_drop_with_nothing_selected_writes_zeros():
    inp = grid_inp(2, 300, 128, seed=13)
    s, out = run_variant(inp, 64, INF, 0.0, True, False)
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("frac", [0.0, 1.0])
def test_fixed_budget_extremes(frac):
    inp = grid_inp(2, 500, 128, seed=14)
    s, _ = run_variant(inp, 64, 0.0, frac, False, True)
    assert s["kept_frac"] == frac


def test_drop_with_every_block_selected_equals_the_main_path():
    inp = grid_inp(2, 1000, 128, seed=15)
    q, k, v = to_device(inp)
    a, _, _, _ = binding.attn_fwd_variant(q, k, v, 64, -INF, drop_approx=True)
    b, _ = binding.attn_fwd(q, k, v, 64, -INF)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("drop,topk", [(True, False), (False, True), (True, True)])
def test_variants_full_size_c3(drop, topk):
    w = gen.WORKLOADS["C3"]
    inp = gen.generate(w, heads=[0, 21, 39])
    N = w.N
    blocks = sorted({0, 1, N // 2, N - 1})
    rows = block_rows(w.L, w.B, [(h, i) for h in range(3) for i in blocks])
    s, _ = run_variant(inp, w.B, 1.0, 0.147, drop, topk, rows=rows)
    print(f"C3 heads 0/21/39 drop={drop} topk={topk}: kept={s['kept_frac']:.4f} "
          f"max_err={s['max_err']:.3e} mean_err={s['mean_err']:.3e}", flush=True)
