"""Self-tests of the seeded synthetic input generator (CPU only)."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_23_amd import inputs as gen


def test_workload_shapes():
    W = gen.WORKLOADS
    assert (W["C1"].L, W["C1"].N) == (1024, 16)
    assert (W["C2"].L, W["C2"].N) == (8192, 128)
    assert (W["C3"].L, W["C3"].N, W["C3"].L - (W["C3"].N - 1) * 64) == (75600, 1182, 16)
    assert (W["C4"].L, W["C4"].N, W["C4"].L - (W["C4"].N - 1) * 64) == (119056, 1861, 16)
    assert (W["C5"].L, W["C5"].N, W["C5"].L - (W["C5"].N - 1) * 128) == (65520, 512, 112)
    assert (W["C5b"].L, W["C5b"].N, W["C5b"].L - (W["C5b"].N - 1) * 128) == (65500, 512, 92)
    assert (W["C6"].L, W["C6"].N, W["C6"].L - (W["C6"].N - 1) * 64) == (131072, 2048, 64)
    assert (W["C6b"].L, W["C6b"].N, W["C6b"].B) == (131072, 4096, 32)
    assert abs(W["C3"].dense_flops / 1e12 - 117.05) < 0.01


def test_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # ties to even
    bits, vals = gen.round_bf16(x)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(vals, t.float().numpy())


def test_generator_deterministic_and_head_subsets():
    w = gen.WORKLOADS["C2"]
    small = gen.Workload("t", H=3, d=64, B=64, dtype="bf16", betas=(), seed=7, grids=((2, 8, 8),))
    a = gen.generate(small)
    b = gen.generate(small, heads=[2, 0])
    assert np.array_equal(a.q[2], b.q[0]) and np.array_equal(a.v[0], b.v[1])
    assert np.array_equal(a.k_bits[1], gen.generate(small, heads=[1]).k_bits[0])
    assert w.H == 12


def test_zero_offset_logit_is_eight():
    """s^2 (d/2)/sqrt(d) = 8: the mean of q_t . k_t / sqrt(d) over tokens is about 8."""
    for d in (64, 128):
        w = gen.Workload("t", H=4, d=d, B=64, dtype="fp32", betas=(), seed=3, grids=((4, 16, 16),))
        inp = gen.generate(w)
        self_logit = np.einsum("hld,hld->hl", inp.q.astype(np.float64), inp.k) / math.sqrt(d)
        assert abs(self_logit.mean() - 8.0) < 0.3


def test_locality_structure():
    """Neighbouring tokens score higher than distant ones."""
    w = gen.Workload("t", H=2, d=128, B=64, dtype="fp32", betas=(), seed=5, grids=((4, 16, 16),))
    inp = gen.generate(w)
    q, k = inp.q[0].astype(np.float64), inp.k[0].astype(np.float64)
    near = np.mean(np.sum(q[:-1] * k[1:], axis=1)) / math.sqrt(128)
    far = np.mean(np.sum(q[:512] * k[512:], axis=1)) / math.sqrt(128)
    # one step along x on a 16-wide grid: 8 exp(-18 pi^2 / 16^2) = 4.0 in expectation
    assert near > 3.0 and far < near / 2


def test_text_tokens_and_edit_pairs():
    w = gen.Workload("t", H=1, d=64, B=64, dtype="fp32", betas=(), seed=1, grids=((2, 4, 4),),
                     text_tokens=8)
    inp = gen.generate(w)
    assert inp.q.shape == (1, 40, 64)
    w2 = gen.Workload("t", H=1, d=64, B=64, dtype="fp32", betas=(), seed=1,
                      grids=((2, 4, 4), (2, 4, 4)), edit_pair=True, truncate=60)
    inp2 = gen.generate(w2)
    assert inp2.q.shape == (1, 60, 64)
    diff = inp2.q[0, 32:60] - inp2.q[0, 0:28]
    assert 0.1 < diff.std() < 0.3  # target = source + 0.2 N(0,1)
