"""bench.py's command-line contract, checked on the CPU: it runs on one GPU
only and says so for --gpus N > 1, before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_options_parse():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py", "--workload", "C6", "--betas", "1.25,1.5", "--steps", "3",
                    "--warmup", "1", "--no-dense", "--no-cpu-baseline", "--ablation"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert (a.workload, a.betas, a.steps, a.warmup, a.no_dense, a.no_cpu_baseline, a.ablation) == \
        ("C6", "1.25,1.5", 3, 1, True, True, True)


def test_traffic_only_for_the_profiled_workload(tmp_path, monkeypatch):
    """The PMC summary's bytes are reported for its own workload and beta on
    the sources it was taken on, and for nothing else."""
    sys.path.insert(0, ROOT)
    import bench
    f = tmp_path / "pmc.txt"
    f.write_text(f"# comment: ignored\nsource_digest: {bench.source_digest()}\nworkload: C3\n"
                 "beta: 1.0\nhbm_bytes_per_launch: 1.5e+11\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("C3", 1.0) == 1.5e11
    assert bench.measured_traffic("C6", 1.0) is None
    assert bench.measured_traffic("C3", 1.5) is None
    f.write_text("source_digest: 0123456789abcdef\nworkload: C3\nbeta: 1.0\n"
                 "hbm_bytes_per_launch: 1.5e+11\n")
    assert bench.measured_traffic("C3", 1.0) is None



def test_schedule_model_of_the_sweep_groups():
    """--schedule orders items by a host model of each group's tile list; the
    model groups query blocks as the sweep does.  Blocks whose selections
    repeat with period 2 group best at stride 2; every block lands in exactly
    one group; the B = 32 exact tiles pair key blocks of equal membership."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    N, QB = 19, 4
    sel = np.zeros((N, N), bool)
    for i in range(N):
        sel[i, (i % 2) * 8:(i % 2) * 8 + 4] = True   # even blocks pick keys 0-3, odd ones 8-11
    st, gs = bench.sweep_groups(sel, QB, np)
    assert st == 2
    assert sorted(b for g in gs for b in g) == list(range(N))
    assert gs[0] == [0, 2, 4, 6] and gs[1] == [1, 3, 5, 7] and gs[-1] == [16, 17, 18]
    # consecutive blocks when nothing favours a stride (ties go to stride 1)
    st1, gs1 = bench.sweep_groups(np.zeros((N, N), bool), QB, np)
    assert st1 == 1 and gs1[0] == [0, 1, 2, 3]
    # B = 32 tile count of one group: chunk 0 (64 pooled keys) holds unselected
    # blocks -> 1 approximate step; masks {0,1}: 3 key blocks -> 2 tiles,
    # mask {0}: 1 block -> 1 tile
    g = np.zeros((2, 40), bool)
    g[:, [3, 5, 9]] = True
    g[0, 20] = True
    assert bench.group_tiles(g, 32, 64, np) == 1 + 2 + 1
    # B = 64: one step per key block of the union
    assert bench.group_tiles(g, 64, 64, np) == 1 + 4
