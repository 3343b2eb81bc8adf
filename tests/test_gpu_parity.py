"""HIP path vs the fp64 oracle on small and ragged inputs (every output element).

All calls go through the C ABI (libsol.so) via the ctypes binding."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_23_amd import binding
from block_sparse_attention_23_amd import inputs as gen

from .parity import block_rows, check_output, check_result, run_and_check, to_device

pytestmark = pytest.mark.gpu
INF = math.inf


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def grid_inp(H, L, d, dtype, seed=0):
    # a 4-frame grid wide enough for L tokens, truncated to L (ragged tail)
    W = max(1, -(-L // 64))
    return gen.grid_inputs(H, (4, 16, W), d, seed, dtype, truncate=L)


@pytest.mark.parametrize("dtype,d,B,L", [("bf16", 128, 64, 1000), ("bf16", 64, 128, 1000),
                                         ("fp32", 64, 64, 1024), ("bf16", 128, 128, 300),
                                         ("bf16", 64, 64, 1), ("fp32", 128, 64, 77),
                                         ("bf16", 128, 64, 4096), ("bf16", 128, 32, 1000),
                                         ("fp32", 64, 32, 77)])
def test_pool_matches_oracle(dtype, d, B, L):
    inp = grid_inp(3, L, d, dtype, seed=1)
    q, k, v = to_device(inp)
    qb, kb, vs = binding.pool(q, k, v, B)
    torch.cuda.synchronize()
    ref = oracle.pool(inp.q, inp.k, inp.v, B)
    for got, want in zip((qb, kb, vs), ref):
        np.testing.assert_allclose(got.cpu().numpy(), want, rtol=2e-6, atol=2e-5)


@pytest.mark.parametrize("beta", [-INF, 0.0, 1.0, INF])
@pytest.mark.parametrize("d,B", [(128, 64), (64, 64), (128, 128), (64, 128), (128, 32), (64, 32)])
@pytest.mark.parametrize("L", [1000, 1024, 130, 50, 1])
def test_forward_bf16_small(L, d, B, beta):
    inp = grid_inp(2, L, d, "bf16", seed=L + d + B)
    s = run_and_check(inp, B, beta)
    if beta == -INF:
        assert s["kept_frac"] == 1.0
    if beta == INF:
        assert s["kept_frac"] == 0.0


@pytest.mark.parametrize("beta", [0.5, 1.5])
def test_forward_bf16_unstructured(beta):
    inp = gen.random_inputs(3, 700, 128, seed=9, dtype="bf16", scale=1.5)
    run_and_check(inp, 64, beta)


def grouping_cost(bits, QB, st):
    """Host model of the sweep's grouping cost at group stride st: over every
    head, the number of key blocks selected by any query block of a group,
    summed over the groups that stride forms (runs of QB st blocks, group r of
    a run holding blocks r, r + st, ...; consecutive groups after the last
    whole run).  bits: the selection mask [H][N][W] (uint32)."""
    H, N, _ = bits.shape
    span = QB * st
    full = (N // span) * span
    groups = [[a + r + k * st for k in range(QB)] for a in range(0, full, span) for r in range(st)]
    groups += [list(range(i, min(i + QB, N))) for i in range(full, N, QB)]
    assert sorted(b for g in groups for b in g) == list(range(N))
    tot = 0
    for h in range(H):
        for g in groups:
            u = np.bitwise_or.reduce(bits[h, g], axis=0)
            tot += int(np.unpackbits(u.view(np.uint8)).sum())
    return tot


@pytest.mark.parametrize("B,grid,L,d", [(32, (2, 16, 64), 2000, 128), (32, (2, 32, 64), 4000, 64),
                                        (32, (2, 32, 96), 6000, 128), (64, (2, 8, 128), 2000, 128),
                                        (64, (2, 16, 128), 4000, 64)])
def test_forward_strided_groups(B, grid, L, d):
    """Frames whose rows span several query blocks: the selection makes a
    group stride above 1 the cheapest, so the sweep groups blocks of
    neighbouring rows instead of consecutive ones (ragged last block, and
    groups of consecutive blocks after the last whole run).  Every element
    against the oracle."""
    inp = gen.grid_inputs(2, grid, d, 11, "bf16", truncate=L)
    q, k, v = to_device(inp)
    out, kept, mask, tau = binding.attn_fwd(q, k, v, B, 1.0, debug=True)
    torch.cuda.synchronize()
    bits = mask.cpu().numpy().view(np.uint32)
    costs = [grouping_cost(bits, 128 // B, st) for st in range(1, 9)]
    assert int(np.argmin(costs)) + 1 > 1, costs
    s = check_result(inp, B, 1.0, out, kept, mask)
    assert 0.0 < s["kept_frac"] < 1.0


@pytest.mark.parametrize("beta", [-INF, 0.0, 1.0, INF])
@pytest.mark.parametrize("d,B,L", [(64, 64, 1024), (128, 64, 333), (64, 128, 1000), (128, 32, 1000),
                                   (64, 32, 333), (128, 128, 1000), (128, 128, 256)])
def test_forward_fp32(d, B, L, beta):
    inp = grid_inp(2, L, d, "fp32", seed=5)
    run_and_check(inp, B, beta)


@pytest.mark.parametrize("beta", [0.0, 1.0, 2.0])
def test_forward_b32_many_groups(beta):
    """B = 32: four query blocks per workgroup and exact tiles made of aligned
    pairs of key blocks, each half used by its own set of query blocks; 2 heads
    of 8229 tokens (N = 258 blocks, 65 groups, ragged last block of 5 tokens)."""
    inp = grid_inp(2, 8229, 128, "bf16", seed=12)
    s = run_and_check(inp, 32, beta)
    assert 0.0 < s["kept_frac"] < 1.0


def test_forward_c1_full():
    """Workload C1 (1 head, 4x16x16 grid, d=64, B=64, fp32, beta=1) in full."""
    w = gen.WORKLOADS["C1"]
    inp = gen.generate(w)
    for beta in w.betas:
        s = run_and_check(inp, w.B, beta)
        assert s["max_err"] <= 1e-5


@pytest.mark.parametrize("dtype,d,L", [("bf16", 128, 1000), ("bf16", 64, 2048), ("fp32", 64, 1024),
                                       ("fp32", 128, 200), ("bf16", 128, 1)])
def test_dense_matches_textbook_attention(dtype, d, L):
    inp = grid_inp(2, L, d, dtype, seed=3)
    q, k, v = to_device(inp)
    out = binding.attn_dense(q, k, v)
    torch.cuda.synchronize()
    ref = oracle.dense(inp.q, inp.k, inp.v)
    check_output(out.float().cpu().numpy(), ref, dtype)


def test_beta_minus_inf_equals_dense_kernel():
    inp = grid_inp(2, 1000, 128, "bf16", seed=4)
    q, k, v = to_device(inp)
    a, _ = binding.attn_fwd(q, k, v, 64, -INF)
    b = binding.attn_dense(q, k, v)
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 1e-2


@pytest.mark.parametrize("B", [32, 64, 128])
def test_deterministic_across_runs(B):
    inp = grid_inp(4, 4000, 128, "bf16", seed=6)
    q, k, v = to_device(inp)
    r1 = binding.attn_fwd(q, k, v, B, 1.0, debug=True)
    r2 = binding.attn_fwd(q, k, v, B, 1.0, debug=True)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_outputs_stay_inside_their_buffers():
    """Guard bands around out, kept_counts and the decision bits are
    untouched, and the values written inside them pass the parity rule."""
    inp = grid_inp(2, 1000, 128, "bf16", seed=7)
    q, k, v = to_device(inp)
    H, L, d = q.shape
    N = (L + 63) // 64
    W = binding.sel_words(N)
    guard = 4096
    big = torch.full((2 * guard + H * L * d,), 1234.0, dtype=torch.bfloat16, device="cuda")
    out = big[guard:guard + H * L * d].view(H, L, d)
    kbig = torch.full((2 * 256 + H * N,), -77, dtype=torch.int32, device="cuda")
    kept = kbig[256:256 + H * N].view(H, N)
    mbig = torch.full((2 * 256 + H * N * W,), -5, dtype=torch.int32, device="cuda")
    mask = mbig[256:256 + H * N * W].view(H, N, W)
    ws = binding.alloc_workspace(H, L, d, 64, q.device)
    st = binding.lib().sol_attn_fwd_dbg(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), H, L, d, 64, 1.0, binding.SOL_BF16,
        out.data_ptr(), kept.data_ptr(), ws.data_ptr(), ws.numel(),
        binding._stream_ptr(None, q.device), mask.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(big[:guard] == 1234.0) and torch.all(big[guard + H * L * d:] == 1234.0)
    assert torch.all(kbig[:256] == -77) and torch.all(kbig[256 + H * N:] == -77)
    assert torch.all(mbig[:256] == -5) and torch.all(mbig[256 + H * N * W:] == -5)
    s = check_result(inp, 64, 1.0, out, kept, mask)
    assert s["compared"] == H * L * d


def test_workspace_reuse_across_shapes():
    """One workspace sized for the larger call serves a smaller call next
    (its stale contents from the larger call do not leak into the result):
    selection with the flip rule and every output element."""
    big = grid_inp(2, 2000, 128, "bf16", seed=8)
    small = grid_inp(1, 300, 128, "bf16", seed=9)
    ws = binding.alloc_workspace(2, 2000, 128, 64, "cuda")
    qb, kb, vb = to_device(big)
    binding.attn_fwd(qb, kb, vb, 64, 1.0, workspace=ws)
    s = run_and_check(small, 64, 1.0, workspace=ws)
    assert s["compared"] == 300 * 128
    s = run_and_check(big, 64, 1.0, workspace=ws)
    assert s["compared"] == 2 * 2000 * 128


def test_side_stream_without_workspace_survives_default_stream_reuse():
    """attn_fwd on a side stream with no caller workspace: the binding's
    temporary workspace belongs to the side stream, so a same-sized buffer
    that the default stream allocates and clears right after the call does
    not share its memory while the side-stream kernels still use it."""
    inp = grid_inp(8, 16000, 128, "bf16", seed=18)
    q, k, v = to_device(inp)
    H, L, d = q.shape
    ref_out, ref_kept = binding.attn_fwd(q, k, v, 64, 1.0)
    torch.cuda.synchronize()
    n_ws = binding.workspace_bytes(H, L, d, 64)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = torch.empty_like(q)
        kept = torch.empty_like(ref_kept)
    side.synchronize()
    for _ in range(3):
        binding.attn_fwd(q, k, v, 64, 1.0, out=out, kept=kept, stream=side)
        junk = torch.empty(n_ws, dtype=torch.uint8, device=q.device)
        junk.zero_()
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(kept, ref_kept)


@pytest.mark.parametrize("dtype,d,B,L", [("bf16", 128, 64, 1000), ("bf16", 64, 128, 700),
                                         ("fp32", 64, 64, 500), ("bf16", 128, 32, 1000),
                                         ("fp32", 128, 32, 300), ("bf16", 64, 32, 45000)])
def test_stage_entry_points_equal_forward(dtype, d, B, L):
    """sol_pool -> sol_route -> sol_sweep (with the route's selection bits, and
    without them) launches the forward pass's own kernels: identical output,
    thresholds, kept counts and decisions."""
    inp = grid_inp(2, L, d, dtype, seed=11)
    q, k, v = to_device(inp)
    H, N = q.shape[0], -(-L // B)
    out_f, kept_f, sel_f, tau_f = binding.attn_fwd(q, k, v, B, 1.0, debug=True)
    qb, kb, vs = binding.pool(q, k, v, B)
    bits = torch.full((H, N, binding.sel_words(N)), -1, dtype=torch.int32, device="cuda")
    tau, kept = binding.route(qb, kb, L, B, 1.0, sel_bits=bits)
    mask_a = torch.full_like(bits, -1)
    mask_b = torch.full_like(bits, -1)
    out_a = binding.sweep(q, k, v, qb, kb, vs, tau, B, sel_bits=bits, sel_mask=mask_a)
    out_b = binding.sweep(q, k, v, qb, kb, vs, tau, B, sel_mask=mask_b)
    torch.cuda.synchronize()
    assert torch.equal(tau, tau_f) and torch.equal(kept, kept_f)
    for m in (bits, mask_a, mask_b):
        assert torch.equal(m, sel_f)
    assert torch.equal(out_a, out_f) and torch.equal(out_b, out_f)


@pytest.mark.parametrize("B", [64, 32])
def test_largest_supported_block_count(B):
    """N = 8192 key blocks (the library's bound), ragged last block: the
    routing kernel's fewest rows per workgroup and the sweep's largest tile
    list (at B = 32 also its largest LDS footprint).  Selection over every
    (i, j); outputs on sampled query blocks."""
    L = 8192 * B - (37 if B == 64 else 11)  # last block: 27 or 21 tokens
    inp = gen.grid_inputs(1, (8, 64, 1024), 64, 21, "bf16", truncate=L)
    N = -(-L // B)
    assert N == 8192
    blocks = [0, 1, 2, 3, N // 2, N - 1]
    rows = block_rows(L, B, [(0, i) for i in blocks])
    s = run_and_check(inp, B, 1.0, rows=rows)
    print(f"B={B} N=8192: kept={s['kept_frac']:.4f} flips={s['flips']} max_err={s['max_err']:.2e}",
          flush=True)


def test_side_stream_matches_default_stream():
    """Every entry point runs on the stream it is given: the staged calls and
    the fused forward on a second stream (default priority) reproduce the
    default-stream results bit for bit, with only that stream synchronised."""
    inp = grid_inp(2, 1500, 128, "bf16", seed=14)
    q, k, v = to_device(inp)
    torch.cuda.synchronize()
    ref_out, ref_kept = binding.attn_fwd(q, k, v, 64, 1.0)
    ref_dense = binding.attn_dense(q, k, v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = torch.empty_like(q)
        kept = torch.empty_like(ref_kept)
        dense = torch.empty_like(q)
        ws = binding.alloc_workspace(2, 1500, 128, 64, q.device)
    side.synchronize()
    binding.attn_fwd(q, k, v, 64, 1.0, out=out, kept=kept, workspace=ws, stream=side)
    binding.attn_dense(q, k, v, out=dense, stream=side)
    qb, kb, vs = binding.pool(q, k, v, 64, stream=side)
    bits = torch.empty((2, 24, binding.sel_words(24)), dtype=torch.int32, device=q.device)
    tau, kept2 = binding.route(qb, kb, 1500, 64, 1.0, sel_bits=bits, stream=side)
    staged = binding.sweep(q, k, v, qb, kb, vs, tau, 64, sel_bits=bits, stream=side)
    side.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(kept, ref_kept)
    assert torch.equal(dense, ref_dense)
    assert torch.equal(staged, ref_out) and torch.equal(kept2, ref_kept)


@pytest.mark.parametrize("B,L", [(64, 200), (32, 200), (128, 700)])
def test_many_heads_few_groups_per_head(B, L):
    """50 heads with 2 (B = 64, 32) or 6 (B = 128) query groups each: some of
    the eight per-XCD work queues are empty for every head, and (B = 64, 32)
    the last group holds fewer query blocks than a full one; every element
    against the oracle."""
    inp = gen.random_inputs(50, L, 64, seed=15, dtype="bf16", scale=1.5)
    s = run_and_check(inp, B, 0.5)
    assert 0.0 < s["kept_frac"] < 1.0


def test_concurrent_calls_with_distinct_workspaces():
    """Two forward passes in flight at once on two streams, each with its own
    workspace, give the same bits as the same calls run one after another."""
    a_in = grid_inp(2, 3000, 128, "bf16", seed=16)
    b_in = grid_inp(3, 2100, 64, "bf16", seed=17)
    qa, ka, va = to_device(a_in)
    qb, kb, vb = to_device(b_in)
    ref_a = binding.attn_fwd(qa, ka, va, 64, 1.0)
    ref_b = binding.attn_fwd(qb, kb, vb, 128, 0.5)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    wa = binding.alloc_workspace(2, 3000, 128, 64, qa.device)
    wb = binding.alloc_workspace(3, 2100, 64, 128, qb.device)
    oa, ob = torch.empty_like(qa), torch.empty_like(qb)
    kpa, kpb = torch.empty_like(ref_a[1]), torch.empty_like(ref_b[1])
    torch.cuda.synchronize()
    for _ in range(3):
        binding.attn_fwd(qa, ka, va, 64, 1.0, out=oa, kept=kpa, workspace=wa, stream=s1)
        binding.attn_fwd(qb, kb, vb, 128, 0.5, out=ob, kept=kpb, workspace=wb, stream=s2)
    s1.synchronize()
    s2.synchronize()
    assert torch.equal(oa, ref_a[0]) and torch.equal(kpa, ref_a[1])
    assert torch.equal(ob, ref_b[0]) and torch.equal(kpb, ref_b[1])


@pytest.mark.parametrize("B", [64, 32, 128])
def test_sweep_timed_matches_sweep_and_records_every_item(B):
    """sol_sweep_timed runs the sweep kernel itself: with the per-XCD queues
    and with a shuffled claim order it reproduces sol_sweep bit for bit (each
    group item is computed the same way whoever claims it), and it records
    every item once, with its claim before its end."""
    inp = grid_inp(3, 3000, 128, "bf16", seed=19)
    q, k, v = to_device(inp)
    H, L, d = q.shape
    N = -(-L // B)
    qb, kb, vs = binding.pool(q, k, v, B)
    bits = torch.empty((H, N, binding.sel_words(N)), dtype=torch.int32, device="cuda")
    tau, _ = binding.route(qb, kb, L, B, 1.0, sel_bits=bits)
    ref = binding.sweep(q, k, v, qb, kb, vs, tau, B, sel_bits=bits)
    n = binding.group_items(H, N, B)
    out0, c0 = binding.sweep_timed(q, k, v, qb, kb, vs, tau, B, bits)
    order = torch.from_numpy(np.random.default_rng(3).permutation(n).astype(np.int32)).cuda()
    out1, c1 = binding.sweep_timed(q, k, v, qb, kb, vs, tau, B, bits, order=order)
    torch.cuda.synchronize()
    assert torch.equal(out0, ref) and torch.equal(out1, ref)
    for c in (c0.cpu().numpy(), c1.cpu().numpy()):
        assert c.shape == (n, 3)
        assert np.all(c[:, 0] > 0) and np.all(c[:, 1] >= c[:, 0])
        assert np.all(c[:, 2] >= 0) and np.all(c[:, 2] < 4096)
