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
    threads in slices) on a small version of the batched MoE workload
    (activations 1 x 64 x 4096 and a KV layer 2 x 256 x 8 x 128): a slice of
    each tensor in proportion to its size, both rates positive, the pieces'
    global scales equal to each slice's own (asserted inside), the host
    reported."""
    sys.path.insert(0, ROOT)
    import torch

    import bench
    from precision_numerics_block_amd import synth

    act = synth.make_pair(5, 0, (1, 64, 4096), "cpu")
    K, Ky = synth.make_pair(5, 1, (256, 8, 128), "cpu")
    V, Vy = synth.make_pair(5, 2, (256, 8, 128), "cpu")
    pairs = [act, (torch.stack([K, V]), torch.stack([Ky, Vy]))]
    r = bench.cpu_baseline(pairs, ["act", "kv"], 3 * 65536, 2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    assert "65536 of act" in r["sample"] and "131072 of kv" in r["sample"], r["sample"]
    assert r["all_cores"]["cores"] >= 1 and r["all_cores"]["value"] > 0
    assert r["host"]["nproc"] >= 1
