"""Host-side checks of bench.py's command-line contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_bench_refuses_more_than_one_gpu():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)


def test_bench_help_lists_the_contract_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_cpu_baseline_leg_on_a_small_sample():
    """The benchmark's CPU leg (the oracle on one thread, then on all host
    threads in slices) on a 2 x 512 x 2048 sample of the activations: both
    rates positive, the slices' global scale equal to the whole sample's
    (asserted inside), the host reported."""
    sys.path.insert(0, ROOT)
    import bench
    from precision_numerics_block_amd import synth

    X, Y = synth.make_pair(2, 0, (2, 512, 2048), "cpu")
    r = bench.cpu_baseline(X, Y, X.numel(), 2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    assert r["all_cores"]["cores"] >= 1 and r["all_cores"]["value"] > 0
    assert r["host"]["nproc"] >= 1
