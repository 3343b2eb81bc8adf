"""Pins of the fp64 CPU oracle to facts fixed by the pages and by mathematics.

None of these re-types an oracle formula: each check comes from a different
route -- a closed form, an invariant, a special case that reduces to textbook
softmax attention (scipy's softmax), brute force over a token-level logit
matrix, an identity printed on the pages (Eq. (5), Eq. (11)), or the pages'
Gaussian density figure (tests/golden/gaussian_density.txt).

Sources: "Sol-Attn" visual paper explainer (mxino.github.io), Eq. (4),
Eq. (5), Eq. (9), Eq. (10), Eq. (11), "Key consequence", "Limits and open
questions"; Sol-Attn explainer (papers.ananclaw.com) attention formula.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import norm

import oracle
from block_sparse_attention_23_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, scale=1.0):
    return (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)


def textbook_dense(q, k, v):
    """softmax(Q K^T / sqrt(d)) V with scipy's softmax, fp64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    d = q.shape[-1]
    s = np.einsum("hrd,htd->hrt", q, k) / math.sqrt(d)
    return np.einsum("hrt,htd->hrd", softmax(s, axis=-1), v)


def blocks(L, B):
    return [(j * B, min(L, (j + 1) * B)) for j in range((L + B - 1) // B)]


# --------------------------------------------------------------------------- pooling


@pytest.mark.parametrize("L,B", [(10, 4), (64, 64), (100, 64), (7, 16)])
def test_pool_constant_blocks_closed_form(L, B):
    """A block of identical tokens pools to that token (mean) and n_j copies (sum)."""
    H, d = 2, 5
    base = rand((H, (L + B - 1) // B, d), 1)
    q = np.empty((H, L, d), np.float32)
    for j, (lo, hi) in enumerate(blocks(L, B)):
        q[:, lo:hi] = base[:, j:j + 1]
    qbar, kbar, vsum = oracle.pool(q, q, q, B)
    for j, (lo, hi) in enumerate(blocks(L, B)):
        np.testing.assert_allclose(qbar[:, j], base[:, j], rtol=1e-7, atol=1e-7)
        np.testing.assert_allclose(kbar[:, j], base[:, j], rtol=1e-7, atol=1e-7)
        np.testing.assert_allclose(vsum[:, j], (hi - lo) * base[:, j].astype(np.float64),
                                   rtol=1e-7, atol=1e-6)


def test_pool_permutation_inside_block_invariant():
    H, L, d, B = 2, 50, 6, 8
    q, k, v = rand((H, L, d), 2), rand((H, L, d), 3), rand((H, L, d), 4)
    perm = np.arange(L)
    rng = np.random.default_rng(0)
    for lo, hi in blocks(L, B):
        perm[lo:hi] = lo + rng.permutation(hi - lo)
    a = oracle.pool(q, k, v, B)
    b = oracle.pool(q[:, perm], k[:, perm], v[:, perm], B)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)
    # a permutation that crosses block boundaries changes the pooled tensors
    c = oracle.pool(q[:, ::-1], k[:, ::-1], v[:, ::-1], B)
    assert not np.allclose(a[1], c[1])


# --------------------------------------------------------------------------- proxy / threshold


@pytest.mark.parametrize("L,B", [(300, 64), (256, 64), (77, 8)])
def test_eq11_column_mean_of_token_tile_is_proxy(L, B):
    """Eq. (11): the column mean of c Q_i Kbar^T over the query block's tokens is s_i."""
    H, d = 2, 16
    q, k, v = rand((H, L, d), 5), rand((H, L, d), 6), rand((H, L, d), 7)
    qbar, kbar, _ = oracle.pool(q, k, v, B)
    r = oracle.route(qbar, kbar, 0.5, want_shat=True)
    c = 1.0 / math.sqrt(d)
    for h in range(H):
        for i, (lo, hi) in enumerate(blocks(L, B)):
            tile = c * q[h, lo:hi].astype(np.float64) @ kbar[h].T  # token-to-block tile
            np.testing.assert_allclose(tile.mean(axis=0), r["shat"][h, i], rtol=1e-11, atol=1e-12)


def test_eq5_moment_form_matches_direct_statistics():
    """Eq. (5): mu and sigma^2 from key moments equal the direct row statistics."""
    H, L, d, B = 3, 700, 32, 16
    q, k, v = rand((H, L, d), 8), rand((H, L, d), 9, 2.0), rand((H, L, d), 10)
    qbar, kbar, _ = oracle.pool(q, k, v, B)
    r = oracle.route(qbar, kbar, 1.0)
    mu, s2 = oracle.moments(qbar, kbar)
    np.testing.assert_allclose(r["mu"], mu, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["sigma"] ** 2, s2, rtol=1e-9, atol=1e-12)


def _gaussian_row_kept(beta, N=4000, d=8, seed=11):
    """Fixed pooled query, i.i.d. Gaussian pooled keys: the proxy row is Gaussian."""
    rng = np.random.default_rng(seed)
    qbar = np.tile(rng.standard_normal(d), (N, 1))[None]
    kbar = rng.standard_normal((1, N, d))
    r = oracle.route(qbar, kbar, beta)
    return r["kept"][0, 0] / N, r


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, -1.0])
def test_gaussian_row_density_is_upper_tail(beta):
    """A Gaussian score row keeps the fraction 1 - Phi(beta) (Eq. (4) with mu, sigma)."""
    frac, _ = _gaussian_row_kept(beta)
    p = 1.0 - norm.cdf(beta)
    tol = 5.0 * math.sqrt(p * (1 - p) / 4000) + 2e-3
    assert abs(frac - p) < tol, (beta, frac, p)


def test_pages_gaussian_density_example():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "gaussian_density.txt"))
            if l.strip() and not l.startswith("#")]
    for beta, expect, tol in ((float(a), float(b), float(c)) for a, b, c in rows):
        fracs = [_gaussian_row_kept(beta, seed=s)[0] for s in range(4)]
        assert abs(np.mean(fracs) - expect) < tol, (beta, fracs, expect)


def test_threshold_is_strict_and_infinite_betas():
    """Eq. (4) uses '>': a constant row (sigma = 0) keeps nothing at finite beta."""
    # small integers and d = 4 (c = 1/2): every score, sum and mean is exact in
    # fp64, so the row is a true tie and the strict comparison decides alone
    H, N, d = 1, 12, 4
    rng = np.random.default_rng(12)
    qbar = rng.integers(-3, 4, size=(H, N, d)).astype(np.float64)
    kbar = np.tile(rng.integers(-3, 4, size=(1, 1, d)).astype(np.float64), (H, N, 1))
    for beta in (-2.0, 0.0, 1.0):
        r = oracle.route(qbar, kbar, beta)
        assert r["kept"].sum() == 0
        assert np.all(r["sigma"] == 0.0)
    assert oracle.route(qbar, kbar, float("-inf"))["kept"].min() == N
    assert oracle.route(qbar, kbar, float("inf"))["kept"].max() == 0
    # a constant row of non-dyadic scores (equal pooled keys, random query):
    # the scores are bitwise equal, so mu is that score, sigma = 0 and no
    # block is strictly above tau, although a sum of 37 equal fp64 terms
    # over 37 need not return the score
    qr = rng.standard_normal((2, 37, 16))
    kr = np.tile(rng.standard_normal((1, 1, 16)), (2, 37, 1))
    for beta in (-2.0, 0.0, 1.0):
        r = oracle.route(qr, kr, beta, want_shat=True)
        assert r["kept"].sum() == 0
        assert np.all(r["sigma"] == 0.0)
        assert np.array_equal(r["mu"], r["shat"][:, :, 0]) and np.array_equal(r["tau"], r["mu"])
    assert oracle.route(qr, kr, float("-inf"))["kept"].min() == 37
    # a non-constant row: beta=-inf keeps all, beta=+inf keeps none
    kb2 = rand((H, N, d), 14).astype(np.float64)
    assert oracle.route(qbar, kb2, float("-inf"))["kept"].min() == N
    assert oracle.route(qbar, kb2, float("inf"))["kept"].max() == 0
    with pytest.raises(ValueError):
        oracle.route(qbar, kb2, float("nan"))


def test_selection_monotone_in_beta():
    H, L, d, B = 2, 640, 16, 32
    q, k, v = rand((H, L, d), 15), rand((H, L, d), 16), rand((H, L, d), 17)
    qbar, kbar, _ = oracle.pool(q, k, v, B)
    prev = None
    for beta in (-1.0, 0.0, 0.5, 1.0, 2.0):
        sel = oracle.route(qbar, kbar, beta)["sel"]
        if prev is not None:
            assert np.all(sel <= prev)  # a larger beta never adds blocks
        prev = sel


# --------------------------------------------------------------------------- merge


@pytest.mark.parametrize("L,B,d", [(100, 16, 8), (64, 64, 4), (33, 8, 16)])
def test_beta_minus_inf_is_dense_attention(L, B, d):
    H = 2
    q, k, v = rand((H, L, d), 20, 1.5), rand((H, L, d), 21, 1.5), rand((H, L, d), 22)
    out, r = oracle.attention(q, k, v, B, float("-inf"))
    assert np.all(r["sel"] == 1)
    ref = textbook_dense(q, k, v)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(oracle.dense(q, k, v), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("beta", [float("-inf"), -0.5, 0.0, 1.0, float("inf")])
def test_block_size_one_is_dense_for_every_beta(beta):
    """B = 1: every pooled key is its token, so both paths are exact."""
    H, L, d = 2, 37, 8
    q, k, v = rand((H, L, d), 23, 1.5), rand((H, L, d), 24, 1.5), rand((H, L, d), 25)
    out, _ = oracle.attention(q, k, v, 1, beta)
    np.testing.assert_allclose(out, textbook_dense(q, k, v), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("beta", [-1.0, 0.0, 0.7, float("inf")])
@pytest.mark.parametrize("L,B", [(96, 16), (90, 16), (64, 8)])
def test_block_constant_keys_give_dense_for_every_beta(beta, L, B):
    """Keys constant inside each block: replacing keys by their block mean is exact."""
    H, d = 2, 8
    q, v = rand((H, L, d), 26, 1.5), rand((H, L, d), 27)
    kb = rand((H, (L + B - 1) // B, d), 28, 1.5)
    k = np.empty_like(q)
    for j, (lo, hi) in enumerate(blocks(L, B)):
        k[:, lo:hi] = kb[:, j:j + 1]
    out, _ = oracle.attention(q, k, v, B, beta)
    np.testing.assert_allclose(out, textbook_dense(q, k, v), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("beta", [-1.0, 0.0, 2.0, float("inf")])
@pytest.mark.parametrize("L,B", [(64, 64), (40, 64)])
def test_single_approximate_block_gives_its_mean_value(beta, L, B):
    """'Key consequence': one approximate block alone yields the block's mean value."""
    H, d = 2, 8
    q, k, v = rand((H, L, d), 29), rand((H, L, d), 30), rand((H, L, d), 31)
    out, r = oracle.attention(q, k, v, B, beta)
    assert r["kept"].sum() == 0  # N = 1 => sigma = 0 => nothing strictly above tau
    mean_v = v.astype(np.float64).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(mean_v, out.shape), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("beta", [float("-inf"), 0.0, 0.8, float("inf")])
def test_weights_sum_to_one(beta):
    """With V = 1 every output is 1: per-row weights (exact and n_j-weighted) sum to 1."""
    H, L, d, B = 2, 203, 8, 16
    q, k = rand((H, L, d), 32, 2.0), rand((H, L, d), 33, 2.0)
    ones = np.ones((H, L, d), np.float32)
    out, _ = oracle.attention(q, k, ones, B, beta)
    np.testing.assert_allclose(out, 1.0, rtol=1e-12, atol=1e-12)


def test_permuting_keys_inside_unselected_block_changes_nothing():
    """Only the pooled key of an unselected block enters the output: permuting the
    keys inside block j leaves every query block with j unselected untouched and
    changes the query blocks that compute j exactly."""
    H, L, d, B = 1, 256, 16, 32
    q, k, v = rand((H, L, d), 34, 1.5), rand((H, L, d), 35, 1.5), rand((H, L, d), 36)
    beta = 0.5
    out, r = oracle.attention(q, k, v, B, beta)
    sel = r["sel"][0]
    mixed = [j for j in range(sel.shape[1]) if 0 < sel[:, j].sum() < sel.shape[0]]
    assert mixed
    j = mixed[0]
    k2 = k.copy()
    k2[0, j * B:(j + 1) * B] = k[0, j * B + np.random.default_rng(1).permutation(B)]
    out2, r2 = oracle.attention(q, k2, v, B, beta)
    assert np.array_equal(r2["sel"], r["sel"])  # pooled keys, hence routing, unchanged
    for i in range(sel.shape[0]):
        rows = slice(i * B, (i + 1) * B)
        if sel[i, j]:
            assert np.abs(out2[0, rows] - out[0, rows]).max() > 1e-6
        else:
            np.testing.assert_allclose(out2[0, rows], out[0, rows], rtol=1e-12, atol=1e-13)


def brute_force_modified_logits(q, k, v, B, sel):
    """Token-level form of Eq. (9)/(10): dense softmax in which each key of an
    unselected block is replaced by its block's mean key."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    H, L, d = q.shape
    out = np.empty((H, L, d))
    for h in range(H):
        for i, (qlo, qhi) in enumerate(blocks(L, B)):
            keff = k[h].copy()
            for j, (lo, hi) in enumerate(blocks(L, B)):
                if not sel[h, i, j]:
                    keff[lo:hi] = k[h, lo:hi].mean(axis=0)
            logits = q[h, qlo:qhi] @ keff.T / math.sqrt(d)
            out[h, qlo:qhi] = softmax(logits, axis=-1) @ v[h]
    return out


@pytest.mark.parametrize("L,B,d,beta", [(130, 16, 8, 0.3), (64, 8, 4, 1.0), (200, 32, 16, -0.2),
                                        (75, 16, 8, 0.0), (9, 4, 3, 1.0)])
def test_merge_equals_brute_force_token_logits(L, B, d, beta):
    H = 2
    q, k, v = rand((H, L, d), 40 + L, 1.5), rand((H, L, d), 41 + L, 1.5), rand((H, L, d), 42 + L)
    out, r = oracle.attention(q, k, v, B, beta)
    assert 0 < r["kept"].sum() < H * r["kept"].shape[1] ** 2 or L < 2 * B
    np.testing.assert_allclose(out, brute_force_modified_logits(q, k, v, B, r["sel"]),
                               rtol=1e-10, atol=1e-12)


def test_injected_selection_is_used_verbatim():
    H, L, d, B = 1, 96, 8, 16
    q, k, v = rand((H, L, d), 50), rand((H, L, d), 51), rand((H, L, d), 52)
    N = 6
    sel = (np.random.default_rng(3).random((H, N, N)) < 0.4).astype(np.uint8)
    out, _ = oracle.attention(q, k, v, B, 0.0, sel=sel)
    np.testing.assert_allclose(out, brute_force_modified_logits(q, k, v, B, sel),
                               rtol=1e-10, atol=1e-12)


def test_beta_plus_inf_is_attention_over_pooled_keys():
    """beta = +inf: softmax over pooled keys with log(n_j) bias, applied to block means."""
    H, L, d, B = 2, 150, 8, 32
    q, k, v = rand((H, L, d), 53, 1.5), rand((H, L, d), 54, 1.5), rand((H, L, d), 55)
    out, _ = oracle.attention(q, k, v, B, float("inf"))
    bl = blocks(L, B)
    n = np.array([hi - lo for lo, hi in bl], dtype=np.float64)
    for h in range(H):
        km = np.stack([k[h, lo:hi].astype(np.float64).mean(0) for lo, hi in bl])
        vm = np.stack([v[h, lo:hi].astype(np.float64).mean(0) for lo, hi in bl])
        logits = q[h].astype(np.float64) @ km.T / math.sqrt(d) + np.log(n)[None]
        np.testing.assert_allclose(out[h], softmax(logits, axis=-1) @ vm, rtol=1e-10, atol=1e-12)


def test_row_subset_matches_full_run():
    H, L, d, B = 2, 150, 8, 32
    q, k, v = rand((H, L, d), 56), rand((H, L, d), 57), rand((H, L, d), 58)
    full, r = oracle.attention(q, k, v, B, 0.5)
    rows = np.array([[0, 0], [1, 149], [0, 77], [1, 31], [1, 32]], dtype=np.int32)
    sub = oracle.merge(q, k, v, r["kbar"], r["vsum"], B, r["sel"], rows=rows)
    np.testing.assert_array_equal(sub, full[rows[:, 0], rows[:, 1]])
    dsub = oracle.dense(q, k, v, rows=rows)
    dfull = oracle.dense(q, k, v)
    np.testing.assert_array_equal(dsub, dfull[rows[:, 0], rows[:, 1]])


def test_locality_inputs_route_sanely():
    """On the synthetic video-grid inputs the proxy keeps near blocks: each query
    block's own key block is selected at beta = 1 far more often than not."""
    inp = gen.grid_inputs(H=2, grid=(4, 16, 16), d=64, seed=0, dtype="fp32")
    B = 64
    qbar, kbar, _ = oracle.pool(inp.q, inp.k, inp.v, B)
    r = oracle.route(qbar, kbar, 1.0)
    diag = np.mean([r["sel"][h, i, i] for h in range(2) for i in range(r["sel"].shape[1])])
    assert diag > 0.8
    kept = r["kept"].sum() / r["sel"].size
    assert 0.02 < kept < 0.5


# ------------------------------------------------- ablations: fixed budget, keep-or-drop
# The abstract contrasts Sol-Attn with fixed top-ranked budgets and with
# keep-or-drop sparsification; the explainer's "Place it among nearby methods"
# says ordinary block sparse attention lets every unselected block contribute
# zero.  The oracle implements both as comparators.


@pytest.mark.parametrize("k", [0, 1, 5, 17, 40])
def test_topk_keeps_k_blocks_and_none_scored_below_a_dropped_one(k):
    qbar = rand((2, 40, 12), 30).astype(np.float64)
    kbar = rand((2, 40, 12), 31).astype(np.float64)
    r = oracle.route_topk(qbar, kbar, k, want_shat=True)
    sel = r["sel"].astype(bool)
    assert (sel.sum(-1) == k).all() and (r["kept"] == k).all()
    s = r["shat"]
    if 0 < k < 40:
        lo_kept = np.where(sel, s, np.inf).min(-1)
        hi_dropped = np.where(sel, -np.inf, s).max(-1)
        assert (lo_kept >= hi_dropped).all()
        np.testing.assert_array_equal(r["kth"], lo_kept)
    # the scores themselves are the threshold route's proxies
    np.testing.assert_array_equal(s, oracle.route(qbar, kbar, 1.0, want_shat=True)["shat"])


def test_topk_ties_go_to_the_lower_block_index():
    qbar = rand((1, 12, 6), 32).astype(np.float64)
    kbar = np.tile(rand((1, 1, 6), 33).astype(np.float64), (1, 12, 1))  # equal scores
    for k in (0, 1, 5, 12):
        sel = oracle.route_topk(qbar, kbar, k)["sel"][0]
        expect = np.zeros(12, np.uint8)
        expect[:k] = 1
        assert (sel == expect[None, :]).all()


def test_topk_at_a_rows_own_count_is_the_threshold_selection():
    """Eq. (4) keeps {j : s_ij > tau_i}; with distinct scores that is the
    kept_i largest, so a fixed budget equal to a row's own count selects the
    same blocks."""
    qbar = rand((2, 48, 16), 34).astype(np.float64)
    kbar = rand((2, 48, 16), 35).astype(np.float64)
    t = oracle.route(qbar, kbar, 0.7)
    checked = 0
    for k in np.unique(t["kept"]):
        rows = t["kept"] == k
        tk = oracle.route_topk(qbar, kbar, int(k))
        assert (tk["sel"][rows] == t["sel"][rows]).all()
        checked += int(rows.sum())
    assert checked == 2 * 48


def test_topk_count_rounds_half_up():
    assert [oracle.topk_count(f, 10) for f in (0.0, 0.04, 0.05, 0.149, 0.15, 1.0, 2.0)] == \
        [0, 0, 1, 1, 2, 10, 10]


def test_drop_with_every_block_selected_is_dense_attention():
    q, k, v = rand((2, 90, 8), 36), rand((2, 90, 8), 37), rand((2, 90, 8), 38)
    qbar, kbar, vsum = oracle.pool(q, k, v, 16)
    sel = np.ones((2, 6, 6), np.uint8)
    out = oracle.merge(q, k, v, kbar, vsum, 16, sel, drop_approx=True)
    np.testing.assert_allclose(out, textbook_dense(q, k, v), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("L,B", [(100, 16), (64, 8)])
def test_drop_is_softmax_over_the_selected_tokens_only(L, B):
    """Brute force: mask the logits of every token outside S_i, softmax, V."""
    H, d = 2, 8
    q, k, v = rand((H, L, d), 39), rand((H, L, d), 40), rand((H, L, d), 41)
    N = (L + B - 1) // B
    sel = (np.random.default_rng(42).random((H, N, N)) < 0.4).astype(np.uint8)
    sel[:, :, 0] = 1  # every row keeps at least block 0
    qbar, kbar, vsum = oracle.pool(q, k, v, B)
    out = oracle.merge(q, k, v, kbar, vsum, B, sel, drop_approx=True)
    logits = np.einsum("hrd,htd->hrt", q.astype(np.float64), k.astype(np.float64)) / math.sqrt(d)
    tok_blk = np.arange(L) // B
    keep = sel[:, tok_blk][:, :, tok_blk]  # [H][r][t]: block of r selects block of t
    logits = np.where(keep.astype(bool), logits, -np.inf)
    ref = np.einsum("hrt,htd->hrd", softmax(logits, axis=-1), v.astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_drop_with_nothing_selected_is_zero():
    q, k, v = rand((1, 50, 8), 43), rand((1, 50, 8), 44), rand((1, 50, 8), 45)
    qbar, kbar, vsum = oracle.pool(q, k, v, 16)
    sel = np.zeros((1, 4, 4), np.uint8)
    sel[0, 1, 2] = 1  # only query block 1 keeps anything
    out = oracle.merge(q, k, v, kbar, vsum, 16, sel, drop_approx=True)
    assert (out[0, :16] == 0).all() and (out[0, 32:] == 0).all()
    assert np.abs(out[0, 16:32]).max() > 0
