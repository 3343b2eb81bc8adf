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

