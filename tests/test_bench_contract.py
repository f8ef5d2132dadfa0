"""CPU-side checks of the benchmark's command-line contract (no GPU used)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_workload_names_resolve():
    sys.path.insert(0, ROOT)
    from block_scaled_fp4_sigmoid_amd import synth
    assert len(synth.WORKLOAD_ORDER) == 5
    for name in synth.WORKLOAD_ORDER + list(synth.EXTRA_WORKLOADS):
        assert name in synth.WORKLOADS
        assert synth.seed_of(name) >= 1
    assert [synth.seed_of(n) for n in synth.WORKLOAD_ORDER] == [1, 2, 3, 4, 5]
