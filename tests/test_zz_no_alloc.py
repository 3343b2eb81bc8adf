"""sol_attn_fwd_noalloc, the allocation-free forward pass, against
sol_attn_fwd (the same kernels with a caller workspace) through the C ABI:
consecutive calls on one GPU share the library's static scratch, each
smaller than the one before and of another layout (moment route, row-holding
route, fp32 inputs), and each must reproduce the workspace entry point bit
for bit; the workspace entry point itself is checked against the fp64
oracle with the parity rule."""
import pytest
import torch

from block_sparse_attention_23_amd import binding
from block_sparse_attention_23_amd import inputs as gen

from .parity import run_and_check, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


# (heads, grid, d, dtype, truncate, B, beta): largest first
CALLS = [
    (2, (22, 64, 64), 128, "bf16", 1400 * 64 - 9, 64, 1.0),   # N = 1400: key moments in the scratch
    (3, (4, 16, 40), 128, "bf16", 2500, 64, 1.0),             # N = 40: rows held on chip
    (2, (4, 16, 20), 64, "fp32", 700, 128, 0.5),              # fp32 inputs: the other layout
    (1, (2, 16, 16), 64, "bf16", 300, 32, 0.0),               # B = 32
]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    for H, grid, d, dtype, L, B, beta in CALLS:
        inp = gen.grid_inputs(H, grid, d, seed=51 + H + d, dtype=dtype, truncate=L)
        q, k, v = to_device(inp)
        ref_out, ref_kept = binding.attn_fwd(q, k, v, B, beta)
        out, kept = binding.attn_fwd_noalloc(q, k, v, B, beta)
        torch.cuda.synchronize()
        print(f"noalloc H={H} L={L} d={d} B={B} {dtype}: kept={kept.float().mean().item():.2f}", flush=True)
        assert torch.equal(kept, ref_kept)
        assert torch.equal(out, ref_out)
        if L <= 2500:
            run_and_check(inp, B, beta)


def test_noalloc_on_a_side_stream():
    inp = gen.grid_inputs(2, (4, 16, 30), 128, seed=61, dtype="bf16", truncate=1900)
    q, k, v = to_device(inp)
    ref_out, ref_kept = binding.attn_fwd(q, k, v, 64, 1.0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = torch.empty_like(q)
        kept = torch.empty_like(ref_kept)
    side.synchronize()
    for _ in range(2):
        binding.attn_fwd_noalloc(q, k, v, 64, 1.0, out=out, kept=kept, stream=side)
    side.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(kept, ref_kept)


@pytest.mark.parametrize("H,grid,L", [(3, (4, 16, 40), 2500), (2, (22, 64, 64), 1400 * 64 - 9)],
                         ids=["rows-on-chip", "key-moments"])
def test_noalloc_forward_replays_from_a_hip_graph(H, grid, L):
    """The callers the allocation-free entry point is for include HIP graph
    capture: sol_attn_fwd_noalloc captured on torch's capture stream and
    replayed three times, with unrelated eager work and synchronisations
    between the replays, reproduces the eager sol_attn_fwd result bit for
    bit on every replay (nothing inside it allocates, clears memory from
    the host or synchronises)."""
    inp = gen.grid_inputs(H, grid, 128, seed=77 + H, dtype="bf16", truncate=L)
    q, k, v = to_device(inp)
    ref_out, ref_kept = binding.attn_fwd(q, k, v, 64, 1.0)
    out = torch.empty_like(q)
    kept = torch.empty_like(ref_kept)
    binding.attn_fwd_noalloc(q, k, v, 64, 1.0, out=out, kept=kept)  # the scratch is looked up eagerly
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.attn_fwd_noalloc(q, k, v, 64, 1.0, out=out, kept=kept)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(0)
        kept.fill_(-1)
        other = torch.randn(1 << 20, device=q.device)
        other.mul_(2.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(kept, ref_kept), rep
    del graph
    torch.cuda.synchronize()
