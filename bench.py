#!/usr/bin/env python3
"""Sol-Attn benchmark on one MI355X (gfx950).

Workload: the Wan-2.1-14B-shaped attention layer -- 40 heads, a 21x45x80
latent grid (L = 75,600 tokens, ragged last block of 16), d = 128, B = 64,
bf16, synthetic locality-structured Q/K/V (seed 2) -- at beta = 1.0, then the
beta sweep {0.5, 1.5, 2.0}.  One step = one sol_attn_fwd call (pool, route
and the fused sweep) on inputs already resident in HBM.

Prints one JSON line on stdout: dense-equivalent TFLOP/s (4 H L^2 d / step
time) as `value`, the sweep kernel's roofline (algorithmic FLOPs per launch /
its HIP-event-timed duration), kept-block fraction, the in-library dense
baseline, and the fp64 CPU oracle timed on a bounded sample as a baseline.
Progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector ALU (the fp32 path computes on the VALU)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sweep_c3_beta1_pmc.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C3")
    ap.add_argument("--betas", default=None,
                    help="comma-separated betas; the first is the headline (default: the workload's "
                         "headline beta, then the rest of its sweep)")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the benchmark line: error against dense attention and time "
                         "per forward of Sol-Attn, keep-or-drop and a fixed top-k budget at "
                         "equal kept fraction, per beta (one JSON line)")
    ap.add_argument("--schedule", action="store_true",
                    help="instead of the benchmark line: the sweep's per-workgroup finish times under "
                         "the per-XCD locality queues and under a longest-first claim order, per beta "
                         "(one JSON line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--oracle-full-run", default=None, help=argparse.SUPPRESS)
    return ap.parse_args()


SWEEP_SOURCES = ("sol_device.h", "sol_launch.h", "sol_tile.h", "sol_sweep.hip")


def source_digest():
    """Digest of the code the sweep kernel is built from (its source and the
    headers it includes): comments and whitespace are dropped first, so a
    comment edit keeps recorded counters valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_23_amd", "csrc")
    for f in SWEEP_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(f.encode() + b"\0" + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, beta):
    """HBM bytes per sweep launch from the committed PMC summary, if it was
    taken on the current kernel sources, for this workload and beta (else
    None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        if kv.get("workload") != workload or float(kv.get("beta", "nan")) != beta:
            return None
    except ValueError:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_loop(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def cpu_model():
    """The host CPU as /proc/cpuinfo describes it: model name, vendor, family,
    model and stepping of the first processor, and the processor count."""
    info, count = {}, 0
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                continue
            k, v = (x.strip() for x in line.split(":", 1))
            if k == "processor":
                count += 1
            elif count == 1 and k in ("model name", "vendor_id", "cpu family", "model", "stepping"):
                info[k] = v
    except OSError:
        return None
    info["processors"] = count
    return info


def oracle_full_run(name):
    """(Child process) the fp64 oracle over a whole workload at its first
    beta -- pool, route and the merge of every row -- timed by wall clock;
    the thread count comes from OMP_NUM_THREADS.  Prints one JSON line."""
    import numpy as np  # noqa: F401
    import oracle
    from block_sparse_attention_23_amd import inputs as gen
    w = gen.WORKLOADS[name]
    beta = w.headline_beta if w.headline_beta in w.betas else w.betas[-1]
    inp = gen.generate(w)
    oracle.lib()
    t0 = time.perf_counter()
    oracle.attention(inp.q, inp.k, inp.v, w.B, beta)
    sec = time.perf_counter() - t0
    print(json.dumps({"workload": name, "beta": beta, "threads": oracle.num_threads(), "seconds": sec,
                      "dense_equiv_tflops": w.dense_flops / sec / 1e12}))


def oracle_full_runs():
    """Whole-workload oracle times for C1 and C2, on every host thread and on
    one, each in a child process (OMP_NUM_THREADS set there)."""
    import subprocess
    runs = []
    for name in ("C1", "C2"):
        for threads in (None, 1):
            env = dict(os.environ)
            if threads:
                env["OMP_NUM_THREADS"] = str(threads)
            r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-full-run", name],
                               capture_output=True, text=True, env=env, timeout=600)
            if r.returncode != 0:
                raise RuntimeError(f"oracle run {name} failed: {r.stderr[-2000:]}")
            runs.append(json.loads(r.stdout.strip().splitlines()[-1]))
            log(f"[bench] oracle {name} in full: {runs[-1]['seconds']:.2f} s on {runs[-1]['threads']} thread(s)")
    return runs


def cpu_baseline(w, inp, beta, target_s):
    """The fp64 oracle on a bounded sample of about target_s seconds: heads
    0, 1, ... in turn, each with pool + route of the whole head and then the
    merge of its first n query blocks (all of them while time remains)."""
    import numpy as np
    import oracle
    B, L, d = w.B, w.L, w.d
    total, flops, parts = 0.0, 0.0, []
    for h in range(w.H):
        q, k, v = (np.ascontiguousarray(a[h:h + 1]) for a in (inp.q, inp.k, inp.v))
        t0 = time.perf_counter()
        qbar, kbar, vsum = oracle.pool(q, k, v, B)
        r = oracle.route(qbar, kbar, beta)
        total += time.perf_counter() - t0

        def merge_blocks(n):
            rows = np.array([(0, x) for x in range(min(L, n * B))], dtype=np.int32)
            t = time.perf_counter()
            oracle.merge(q, k, v, kbar, vsum, B, r["sel"], rows=rows)
            return time.perf_counter() - t

        if h == 0:
            merge_blocks(1)  # warm the thread pool and caches
        t1 = merge_blocks(8) / 8  # a probe, not counted
        n = max(8, min(w.N, int(max(1.0, target_s - total) / max(t1, 1e-6))))
        total += merge_blocks(n)
        rows_n = min(L, n * B)
        flops += rows_n * 4.0 * L * d
        parts.append((h, n, rows_n))
        if total >= target_s or n < w.N:
            break
    whole = [p for p in parts if p[1] >= w.N]
    desc = f"heads 0-{len(whole) - 1} whole" if whole else ""
    if len(whole) < len(parts):
        h, n, rows_n = parts[-1]
        desc += ("; " if desc else "") + f"head {h}: first {n} query blocks ({rows_n} rows)"
    return {
        "value": flops / total / 1e12, "unit": "dense-equiv TFLOP/s", "cores": oracle.num_threads(),
        "kind": "oracle", "cpu_model": cpu_model(),
        "sample": (f"{w.name} at beta={beta}: per head, pool + route of the whole head and the "
                   f"merge of its query blocks; {desc} = {flops / 1e12:.3f} dense-equiv TFLOP "
                   f"in {total:.1f} s"),
        "seconds": total,
    }


def ablation(args, np, torch, binding, gen):
    """What the approximate correction buys: for each beta, relative L2 error
    against the in-library dense attention and time per forward of
      sol        Sol-Attn (threshold selection, approximate correction),
      fused_route  the same, its decisions taken inside the sweep from the
                 Eq. (5) thresholds (SOL_FUSED_ROUTE),
      drop       the same selection, unselected blocks left out (keep-or-drop),
      topk       a fixed budget of round(rho N) blocks per query block, rho =
                 Sol-Attn's kept fraction at that beta, with the correction,
      topk_drop  the fixed budget without it.
    The dense reference is itself bf16 (a ~0.3 % rounding floor)."""
    w = gen.WORKLOADS[args.workload]
    betas = ([float(b) for b in args.betas.split(",")] if args.betas else list(w.betas))
    log(f"[ablation] generating {w.name}: {w.desc}")
    inp = gen.generate(w)
    q, k, v = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
               for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    del inp
    ws = binding.alloc_workspace(w.H, w.L, w.d, w.B, "cuda")
    ref = binding.attn_dense(q, k, v).float()
    ref_norm = torch.linalg.vector_norm(ref).item()
    out = torch.empty_like(q)

    def err(o):
        return torch.linalg.vector_norm(o.float() - ref).item() / ref_norm

    rows = []
    for beta in betas:
        _, kept = binding.attn_fwd(q, k, v, w.B, beta, out=out, workspace=ws)
        rho = kept.sum().item() / (w.H * w.N * w.N)
        runs = {
            "sol": lambda: binding.attn_fwd(q, k, v, w.B, beta, out=out, workspace=ws),
            "fused_route": lambda: binding.attn_fwd_variant(q, k, v, w.B, beta, fused_route=True,
                                                            out=out, workspace=ws, debug=False),
            "drop": lambda: binding.attn_fwd_variant(q, k, v, w.B, beta, drop_approx=True,
                                                     out=out, workspace=ws, debug=False),
            "topk": lambda: binding.attn_fwd_variant(q, k, v, w.B, beta, keep_frac=rho, topk=True,
                                                     out=out, workspace=ws, debug=False),
            "topk_drop": lambda: binding.attn_fwd_variant(q, k, v, w.B, beta, keep_frac=rho,
                                                          topk=True, drop_approx=True, out=out,
                                                          workspace=ws, debug=False),
        }
        row = {"beta": beta, "kept_frac": rho}
        for name, fn in runs.items():
            ms, _ = time_loop(fn, args.steps, args.warmup, torch)
            fn()
            torch.cuda.synchronize()
            row[name] = {"rel_l2_err": err(out), "ms": ms}
        log(f"[ablation] beta={beta} kept={rho:.4f} " +
            ", ".join(f"{n}: err {row[n]['rel_l2_err']:.4f} {row[n]['ms']:.2f} ms" for n in runs))
        rows.append(row)
    print(json.dumps({"ablation": w.name, "reference": "in-library dense attention (bf16)",
                      "error": "relative L2 over all outputs", "rows": rows}))


def sweep_groups(sel, QB, np):
    """The bf16 sweep's query-block groups of one head (the rule stated at
    sol_attn_fwd in include/sol.h): group stride st in 1..8 with the
    smallest summed union size of the groups' selections, the smaller stride
    on a tie; runs of QB st blocks, group r of a run holding blocks r, r + st,
    ...; consecutive groups after the last whole run.  sel: [N][N] bool.
    Returns (st, list of block-index lists in group order)."""
    N = sel.shape[0]

    def groups(st):
        span = QB * st
        full = (N // span) * span
        gs = [[a + r + k * st for k in range(QB)] for a in range(0, full, span) for r in range(st)]
        return gs + [list(range(i, min(i + QB, N))) for i in range(full, N, QB)]

    best = None
    for st in range(1, 9):
        gs = groups(st)
        c = sum(int(sel[g].any(axis=0).sum()) for g in gs)
        if best is None or c < best[0]:
            best = (c, st, gs)
    return best[1], best[2]


def group_tiles(sel_g, B, TB, np):
    """64-key steps of one group's tile list: approximate chunks of TB pooled
    keys holding an unselected block of a member, then the exact tiles (B >=
    64: one per selected key block of the union, B / 64 steps each; B = 32:
    key blocks chosen by the same members pair up, ceil(count / 2) tiles per
    membership mask).  sel_g: [members][N] bool."""
    N = sel_g.shape[1]
    NC = -(-N // TB)
    unsel = ~np.pad(sel_g, ((0, 0), (0, NC * TB - N)), constant_values=True).reshape(len(sel_g), NC, TB)
    approx = int(unsel.any(axis=2).any(axis=0).sum()) * (TB // 64)
    if B >= 64:
        return approx + int(sel_g.any(axis=0).sum()) * (B // 64)
    masks = (sel_g * (1 << np.arange(len(sel_g)))[:, None]).sum(axis=0)
    counts = np.bincount(masks, minlength=1 << len(sel_g))[1:]
    return approx + int(((counts + 1) // 2).sum())


def schedule(args, np, torch, binding, gen):
    """Load balance of the sweep's persistent workgroups ("dynamic but
    potentially imbalanced budgets"): for each beta, the sweep kernel runs
    with the per-XCD locality queues (the library's order) and with a
    longest-first order (group items by their tile count, descending), each
    recording per item its claim and end times on the GPU's constant clock.
    Reports the kernel time (HIP events), the spread of workgroup finish
    times (first to last) and the mean idle time of a workgroup after its
    last item, in ms."""
    w = gen.WORKLOADS[args.workload]
    betas = [float(b) for b in args.betas.split(",")] if args.betas else [min(w.betas), max(w.betas)]
    if w.dtype != "bf16":
        raise SystemExit("--schedule measures the bf16 sweep")
    H, L, d, B, N = w.H, w.L, w.d, w.B, w.N
    QB = 128 // B
    G = -(-N // QB)
    TB = max(B, 64)
    NC = -(-N // TB)
    log(f"[schedule] generating {w.name}: {w.desc}")
    inp = gen.generate(w)
    q, k, v = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
               for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    del inp
    ws = binding.alloc_workspace(H, L, d, B, "cuda")
    qbar, kbar, vsum = binding.pool(q, k, v, B)
    bits = torch.empty((H, N, binding.sel_words(N)), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    rows = []
    for beta in betas:
        tau, kept = binding.route(qbar, kbar, L, B, beta, sel_bits=bits, workspace=ws)
        sel = binding.unpack_mask(bits, N).astype(bool)  # [H][N][N]
        cost, strides = [], []
        for h in range(H):
            st, gs = sweep_groups(sel[h], QB, np)
            strides.append(st)
            cost += [group_tiles(sel[h][g], B, TB, np) for g in gs]
        cost = np.array(cost)
        lpt = torch.from_numpy(np.argsort(-cost, kind="stable").astype(np.int32)).cuda()
        res = {"beta": beta, "kept_frac": float(sel.mean()), "items": int(H * G),
               "tiles_per_item": {"mean": float(cost.mean()), "min": int(cost.min()), "max": int(cost.max())},
               "group_strides": {str(x): strides.count(x) for x in sorted(set(strides))}}
        for name, order in (("xcd_queues", None), ("longest_first", lpt)):
            fn = lambda: binding.sweep_timed(q, k, v, qbar, kbar, vsum, tau, B, bits, order=order, out=out,
                                             workspace=ws)
            ms, _ = time_loop(fn, args.steps, args.warmup, torch)
            _, clock = fn()
            torch.cuda.synchronize()
            c = clock.cpu().numpy()
            t0 = c[:, 0].min()
            ticks = c[:, 1].max() - t0
            tick_ms = ms / ticks  # the clock's period, from the same launch's HIP-event time
            wg = c[:, 2]
            finish = np.array([c[wg == x, 1].max() for x in np.unique(wg)]) - t0
            end = finish.max()
            res[name] = {"kernel_ms": ms, "finish_spread_ms": float((end - finish.min()) * tick_ms),
                         "mean_idle_after_last_item_ms": float((end - finish).mean() * tick_ms),
                         "mean_item_ms": float(((c[:, 1] - c[:, 0]).mean()) * tick_ms),
                         "workgroups": int(len(finish)), "clock_mhz": 1e-3 / tick_ms}
            log(f"[schedule] beta={beta} {name}: {ms:.3f} ms, finish spread "
                f"{res[name]['finish_spread_ms']:.3f} ms, mean idle at end "
                f"{res[name]['mean_idle_after_last_item_ms']:.3f} ms")
        rows.append(res)
    print(json.dumps({"schedule": w.name, "rows": rows}))


def main():
    args = parse()
    if args.oracle_full_run:
        return oracle_full_run(args.oracle_full_run)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(heads shard across GPUs with no exchange); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_23_amd import binding
    from block_sparse_attention_23_amd import inputs as gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()
    if args.ablation:
        return ablation(args, np, torch, binding, gen)
    if args.schedule:
        return schedule(args, np, torch, binding, gen)
    w = gen.WORKLOADS[args.workload]
    betas = ([float(b) for b in args.betas.split(",")] if args.betas else
             [w.headline_beta] + [b for b in w.betas if b != w.headline_beta])
    H, L, d, B, N = w.H, w.L, w.d, w.B, w.N
    log(f"[bench] generating {w.name}: {w.desc}")
    t = time.perf_counter()
    inp = gen.generate(w)
    log(f"[bench] generated in {time.perf_counter() - t:.1f}s")
    if w.dtype == "bf16":
        dev = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
               for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    else:
        dev = [torch.from_numpy(a).cuda() for a in (inp.q, inp.k, inp.v)]
    q, k, v = dev
    if args.no_cpu_baseline:
        del inp
    else:  # the oracle sample reads the float32 arrays only
        inp.q_bits = inp.k_bits = inp.v_bits = None
    out = torch.empty_like(q)
    kept = torch.empty((H, N), dtype=torch.int32, device="cuda")
    ws = binding.alloc_workspace(H, L, d, B, "cuda")
    torch.cuda.synchronize()

    F_dense = w.dense_flops
    results = []
    for beta in betas:
        fn = lambda: binding.attn_fwd(q, k, v, B, beta, out=out, kept=kept, workspace=ws)
        ms, wall = time_loop(fn, args.steps, args.warmup, torch)
        kc = kept.to(torch.int64)
        n_sel = int(kc.sum().item())
        n_unsel = H * N * N - n_sel
        F_exact = n_sel * 4.0 * B * B * d
        F_approx = n_unsel * 4.0 * B * d
        results.append(dict(beta=beta, ms=ms, wall_s=wall, kept_frac=n_sel / (H * N * N),
                            F_exact=F_exact, F_approx=F_approx,
                            tflops_dense_eq=F_dense / (ms * 1e-3) / 1e12))
        log(f"[bench] beta={beta}: {ms:.3f} ms/step, kept {n_sel / (H * N * N):.4f}, "
            f"{F_dense / (ms * 1e-3) / 1e12:.1f} dense-equiv TFLOP/s")
    head = results[0]

    # Stage breakdown at the headline beta: the same three kernels launched
    # through the stage entry points, with HIP events between them.
    qbar = torch.empty((H, N, d), dtype=torch.float32, device="cuda")
    kbar, vsum = torch.empty_like(qbar), torch.empty_like(qbar)
    tau = torch.empty((H, N), dtype=torch.float32, device="cuda")
    bits = torch.empty((H, N, binding.sel_words(N)), dtype=torch.int32, device="cuda")
    beta0 = head["beta"]
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for it in range(args.warmup + args.steps):
        e = ev[it - args.warmup] if it >= args.warmup else None
        if e: e[0].record(s)
        binding.pool(q, k, v, B, outs=(qbar, kbar, vsum))
        if e: e[1].record(s)
        binding.route(qbar, kbar, L, B, beta0, tau=tau, kept=kept, sel_bits=bits, workspace=ws)
        if e: e[2].record(s)
        binding.sweep(q, k, v, qbar, kbar, vsum, tau, B, out=out, workspace=ws, sel_bits=bits)
        if e: e[3].record(s)
    torch.cuda.synchronize()
    st = {"pool": 0.0, "route": 0.0, "sweep": 0.0}
    for e in ev:
        st["pool"] += e[0].elapsed_time(e[1]) / args.steps
        st["route"] += e[1].elapsed_time(e[2]) / args.steps
        st["sweep"] += e[2].elapsed_time(e[3]) / args.steps
    log(f"[bench] stages at beta={beta0}: " + ", ".join(f"{k} {v:.3f} ms" for k, v in st.items()))
    F_alg = head["F_exact"] + head["F_approx"]
    # token-pair density at the headline beta: selected (i, j) pairs weighted
    # by the valid tokens n_i n_j (only the last block is short)
    nlast = L - (N - 1) * B
    kept_h = kept.to(torch.float64)  # the staged route wrote the headline beta's counts
    last_sel = ((bits[:, :, (N - 1) // 32] >> ((N - 1) % 32)) & 1).to(torch.float64)
    n_i = torch.full((N,), float(B), dtype=torch.float64, device="cuda")
    n_i[N - 1] = nlast
    pair_tokens = (n_i[None, :] * (kept_h * B - (B - nlast) * last_sel)).sum().item()
    kept_token_pair_frac = pair_tokens / (H * float(L) * L)
    achieved = F_alg / (st["sweep"] * 1e-3) / 1e12
    pool_bytes = 3.0 * H * L * d * (2 if w.dtype == "bf16" else 4) + 3.0 * H * N * d * 4
    traffic = measured_traffic(w.name, beta0)
    # bf16 tiles run on the bf16 MFMA; the fp32 path on the fp32 vector ALU
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_VALU_TFLOPS

    dense = None
    if not args.no_dense:
        fn = lambda: binding.attn_dense(q, k, v, out=out)
        dms, _ = time_loop(fn, max(2, args.steps // 2), 1, torch)
        dt = F_dense / (dms * 1e-3) / 1e12
        dense = {"ms": dms, "tflops": dt, "mfma_util": dt / peak}
        log(f"[bench] dense: {dms:.3f} ms, {dt:.1f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, inp, beta0, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['sample']} ({cpu['cores']} threads)")
        cpu["full_runs"] = oracle_full_runs()

    line = {
        "metric": "dense-equiv attn TFLOPS + MFMA util at L=75.6K,d=128 vs beta; kept-block %",
        "value": head["tflops_dense_eq"],
        "unit": "TFLOP/s (dense-equivalent, 4*H*L^2*d / step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded locality-structured Fourier-feature Q/K, N(0,1) V)",
        "config": {"workload": f"{w.name}: {w.desc}", "H": H, "L": L, "d": d, "B": B,
                   "N": N, "beta": head["beta"], "seed": w.seed},
        "kept_block_frac": head["kept_frac"],
        "kept_token_pair_frac": kept_token_pair_frac,
        "exact_tile_mfma_util": head["F_exact"] / (st["sweep"] * 1e-3) / 1e12 / peak,
        "roofline": {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": traffic, "kernel": (f"sweep_bf16_kernel<{d}, {B}, false, false>" if w.dtype == "bf16"
                                                    else f"attn_f32_kernel<{d}, {B}, false>"),
                     "algorithmic_flop_per_launch": F_alg},
        "stage_ms": st,
        "pool_gbs": pool_bytes / (st["pool"] * 1e-3) / 1e9,
        "dense_baseline": dense,
        "speedup_vs_dense": (dense["ms"] / head["ms"]) if dense else None,
        # per beta: exact-tile flops over the whole forward's time (pool and
        # route included) as a fraction of the path's peak, and the speedup
        "beta_sweep": [{"beta": r["beta"], "ms": r["ms"], "kept_frac": r["kept_frac"],
                        "tflops_dense_eq": r["tflops_dense_eq"],
                        "exact_tflop": r["F_exact"] / 1e12,
                        "exact_util_of_forward": r["F_exact"] / (r["ms"] * 1e-3) / 1e12 / peak,
                        "speedup_vs_dense": (dense["ms"] / r["ms"]) if dense else None}
                       for r in results],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
