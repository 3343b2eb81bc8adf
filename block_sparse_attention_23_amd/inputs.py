"""Seeded synthetic inputs for Sol-Attn workloads.

This module holds the workload definitions and the input generators that both
the HIP path and the CPU oracle are fed from.  It contains none of the
method's arithmetic (no pooling, scoring, thresholding or attention): it only
draws Q, K and V.

The pages measure on video diffusion transformers (Wan 2.1 at 720p / 81
frames, HunyuanVideo at 720p / 129 frames, video editing; "Sol-Attn" visual
explainer, "What the paper measured").  Their activations are not available,
so locality-structured synthetic tokens stand in for them: each token sits on
a (frame, row, column) latent grid in raster order, and Q and K share random
Fourier position features, so nearby tokens attend to each other strongly and
far tokens weakly, as in video latents.

Recipe (per head h, each head with its own PCG64 stream spawned from the
workload seed, so any subset of heads can be generated on its own):
  1. omega (d/2 x 3) ~ N(0, 3^2),  2. phi (d/2) ~ U(0, 2 pi),
  3. Q noise (L_grid x d) ~ N(0,1), 4. K noise (L_grid x d) ~ N(0,1),
  5. V (L_grid x d) ~ N(0,1), 6. workload extras (text tokens, edit targets).
  e(p) = [cos(2 pi omega_r . p + phi_r) for r] ++ [sin(...) for r],
  p = (t/T, y/Y, x/X);  Q = s e + 0.3 N(0,1),  K = s e + 0.3 N(0,1),
  s = sqrt(16/sqrt(d)) so that the zero-offset logit s^2 (d/2) / sqrt(d) is 8.
Values are drawn in float64, rounded to float32, then (for bf16 workloads)
rounded to bf16 with round-to-nearest-even.  Both sides receive exactly the
same bf16/fp32 values.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    d: int
    B: int
    dtype: str                      # "fp32" or "bf16"
    betas: Tuple[float, ...]
    seed: int
    grids: Tuple[Tuple[int, int, int], ...]   # latent grids concatenated in order
    text_tokens: int = 0            # N(0,1) tokens appended after the grids
    headline_beta: float = 1.0      # the beta a benchmark of this workload leads with
    edit_pair: bool = False         # second grid = first grid + 0.2 N(0,1)
    truncate: Optional[int] = None  # keep only the first `truncate` tokens
    desc: str = ""

    @property
    def L(self) -> int:
        n = sum(t * y * x for (t, y, x) in self.grids) + self.text_tokens
        return n if self.truncate is None else min(n, self.truncate)

    @property
    def N(self) -> int:
        return (self.L + self.B - 1) // self.B

    @property
    def dense_flops(self) -> float:
        """Dense-equivalent work 4 H L^2 d (QK^T and PV, 2 flops per MAC)."""
        return 4.0 * self.H * float(self.L) ** 2 * self.d


NEG_INF = float("-inf")

WORKLOADS = {
    "C1": Workload("C1", H=1, d=64, B=64, dtype="fp32", betas=(1.0,), seed=0,
                   grids=((4, 16, 16),),
                   desc="1 head, 4x16x16 grid, L=1024, d=64, B=64, fp32"),
    "C2": Workload("C2", H=12, d=128, B=64, dtype="bf16", betas=(NEG_INF, 1.0), seed=1,
                   grids=((8, 32, 32),),
                   desc="12 heads, 8x32x32 grid, L=8192, d=128, B=64, bf16"),
    "C3": Workload("C3", H=40, d=128, B=64, dtype="bf16", betas=(0.5, 1.0, 1.5, 2.0), seed=2,
                   grids=((21, 45, 80),),
                   desc="Wan-2.1-14B-shaped layer: 40 heads, 21x45x80 grid, L=75600, d=128, B=64, bf16"),
    "C4": Workload("C4", H=24, d=128, B=64, dtype="bf16", betas=(0.5, 1.0, 1.5), seed=3,
                   grids=((33, 45, 80),), text_tokens=256,
                   desc="HunyuanVideo-13B-shaped layer: 24 heads, 33x45x80 grid + 256 text "
                        "tokens, L=119056, d=128, B=64, bf16"),
    "C5": Workload("C5", H=24, d=128, B=128, dtype="bf16", betas=(NEG_INF, 0.0, 1.0, 3.0), seed=4,
                   grids=((21, 30, 52), (21, 30, 52)), edit_pair=True,
                   desc="editing-shaped layer: source+target 2x(21x30x52), L=65520, 24 heads, "
                        "d=128, B=128, bf16"),
    "C5b": Workload("C5b", H=24, d=64, B=128, dtype="bf16", betas=(NEG_INF, 0.0, 1.0, 3.0), seed=4,
                    grids=((21, 30, 52), (21, 30, 52)), edit_pair=True, truncate=65500,
                    desc="editing-shaped layer at L=65500 (ragged), 24 heads, d=64, B=128, bf16"),
    # The pages' kernel-level point: 128K tokens at about 90 % sparsity ("Sol-Attn"
    # visual explainer, "What the paper measured", Figure 5a).  The head count is
    # not given there; 24 heads keep the host-side arrays near 7 GB.
    "C6": Workload("C6", H=24, d=128, B=64, dtype="bf16", betas=(1.0, 1.25, 1.5), seed=5,
                   grids=((32, 64, 64),), headline_beta=1.25,
                   desc="long-sequence kernel point: 24 heads, 32x64x64 grid, L=131072, d=128, "
                        "B=64, bf16"),
    # The same inputs at B = 32, the smallest block size the pages' integration
    # notes suggest sweeping (papers.ananclaw.com explainer, its integration
    # notes: try 32, 64 and 128 on the target hardware).
    "C6b": Workload("C6b", H=24, d=128, B=32, dtype="bf16", betas=(1.0, 1.25, 1.5), seed=5,
                    grids=((32, 64, 64),), headline_beta=1.25,
                    desc="long-sequence kernel point at B=32: 24 heads, 32x64x64 grid, L=131072, "
                         "d=128, B=32, bf16"),
}


def feature_scale(d: int) -> float:
    """s with s^2 (d/2) / sqrt(d) = 8 (zero-offset logit of 8)."""
    return math.sqrt(16.0 / math.sqrt(d))


def round_bf16(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns (bits as uint16, the rounded values as float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    bits = ((u + r) >> 16).astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits, vals


def _grid_positions(T: int, Y: int, X: int) -> np.ndarray:
    t, y, x = np.meshgrid(np.arange(T) / T, np.arange(Y) / Y, np.arange(X) / X, indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)  # raster order, t major


def _fourier(pos: np.ndarray, omega: np.ndarray, phi: np.ndarray) -> np.ndarray:
    ang = 2.0 * np.pi * (pos @ omega.T) + phi[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def _head(w: Workload, rng: np.random.Generator) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    d = w.d
    s = feature_scale(d)
    omega = rng.normal(0.0, 3.0, size=(d // 2, 3))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=d // 2)
    T, Y, X = w.grids[0]
    pos = _grid_positions(T, Y, X)
    Lg = pos.shape[0]
    e = _fourier(pos, omega, phi)
    q = s * e + 0.3 * rng.standard_normal((Lg, d))
    k = s * e + 0.3 * rng.standard_normal((Lg, d))
    del e
    full_L = sum(a * b * c for (a, b, c) in w.grids) + w.text_tokens
    v_len = Lg if w.edit_pair else full_L
    v = rng.standard_normal((v_len, d))
    if w.edit_pair:
        # target latents: source + 0.2 N(0,1), independently for Q, K and V
        q = np.concatenate([q, q + 0.2 * rng.standard_normal((Lg, d))])
        k = np.concatenate([k, k + 0.2 * rng.standard_normal((Lg, d))])
        v = np.concatenate([v, v + 0.2 * rng.standard_normal((Lg, d))])
    if w.text_tokens:
        q = np.concatenate([q, rng.standard_normal((w.text_tokens, d))])
        k = np.concatenate([k, rng.standard_normal((w.text_tokens, d))])
    L = w.L
    return q[:L], k[:L], v[:L]


def head_rngs(seed: int, H: int) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(H)]


class Inputs:
    """Generated Q, K, V of one workload.

    ``q, k, v`` are float32 [H][L][d] holding the exact values the GPU gets;
    ``q_bits`` etc. hold the bf16 bit patterns (uint16) for bf16 workloads."""

    def __init__(self, w: Workload, heads: Sequence[int], q, k, v, bits):
        self.workload = w
        self.heads = list(heads)
        self.q, self.k, self.v = q, k, v
        self.q_bits, self.k_bits, self.v_bits = bits


def generate(w: Workload, heads: Optional[Sequence[int]] = None, threads: int = 8) -> Inputs:
    """Generate the listed heads (default: all) of workload ``w``."""
    heads = list(range(w.H)) if heads is None else list(heads)
    rngs = head_rngs(w.seed, w.H)
    L, d = w.L, w.d
    q = np.empty((len(heads), L, d), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    bf = w.dtype == "bf16"
    bits = tuple(np.empty((len(heads), L, d), dtype=np.uint16) for _ in range(3)) if bf else (None,) * 3

    def one(slot_h):
        slot, h = slot_h
        qh, kh, vh = _head(w, rngs[h])
        for dst, src, b in ((q, qh, bits[0]), (k, kh, bits[1]), (v, vh, bits[2])):
            f32 = src.astype(np.float32)
            if bf:
                bb, vals = round_bf16(f32)
                b[slot] = bb
                dst[slot] = vals
            else:
                dst[slot] = f32

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, enumerate(heads)))
    return Inputs(w, heads, q, k, v, bits)


def random_inputs(H: int, L: int, d: int, seed: int, dtype: str = "bf16",
                  scale: float = 1.0) -> Inputs:
    """Unstructured N(0, scale^2) Q/K/V for small parity and edge cases."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = Workload(f"rand{H}x{L}x{d}", H=H, d=d, B=64, dtype=dtype, betas=(), seed=seed,
                 grids=((1, 1, L),))
    arrs = [(scale * rng.standard_normal((H, L, d))).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        rb = [round_bf16(a) for a in arrs]
        return Inputs(w, range(H), rb[0][1], rb[1][1], rb[2][1], (rb[0][0], rb[1][0], rb[2][0]))
    return Inputs(w, range(H), arrs[0], arrs[1], arrs[2], (None, None, None))


def grid_inputs(H: int, grid: Tuple[int, int, int], d: int, seed: int, dtype: str = "bf16",
                truncate: Optional[int] = None) -> Inputs:
    """Locality-structured inputs on an arbitrary small grid (same recipe as the workloads)."""
    w = Workload(f"grid{grid}", H=H, d=d, B=64, dtype=dtype, betas=(), seed=seed,
                 grids=(grid,), truncate=truncate)
    return generate(w)


def shifted_inputs(inp: Inputs, q_shift: Optional[np.ndarray] = None,
                   k_shift: Optional[np.ndarray] = None,
                   k_const: Optional[np.ndarray] = None) -> Inputs:
    """Edge-case inputs built from ``inp``: ``q_shift`` / ``k_shift`` (length d)
    are added to every query / key token, or every key token is replaced by
    ``k_const``; the result is re-rounded to the workload's dtype.  A common
    key component makes every proxy row's mean large against its spread; equal
    keys make every proxy row constant."""
    w = inp.workload
    q, k = inp.q.copy(), inp.k.copy()
    if q_shift is not None:
        q += np.asarray(q_shift, dtype=np.float32)
    if k_shift is not None:
        k += np.asarray(k_shift, dtype=np.float32)
    if k_const is not None:
        k[...] = np.asarray(k_const, dtype=np.float32)
    if w.dtype == "bf16":
        qb, qv = round_bf16(q)
        kb, kv = round_bf16(k)
        return Inputs(w, inp.heads, qv, kv, inp.v, (qb, kb, inp.v_bits))
    return Inputs(w, inp.heads, q, k, inp.v, (None, None, None))
