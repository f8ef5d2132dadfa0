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


def test_headline_is_the_largest_configuration():
    """The bench's headline is the configuration with the most rows (the
    metric covers 1-384 rows), and its byte model matches sizes worked out by
    hand: an MXFP4 expert of hidden 7168 and intermediate 2048 is three
    7168 x 2048 matrices at half a byte per weight plus one E8M0 byte per 32."""
    sys.path.insert(0, ROOT)
    import bench
    from block_scaled_fp4_sigmoid_amd import synth
    assert bench.HEADLINE == max(synth.WORKLOAD_ORDER, key=lambda n: synth.WORKLOADS[n].M)
    s = synth.WORKLOADS[bench.HEADLINE]
    bm = bench.byte_model(s, 256)
    per = 3 * 7168 * 2048 // 2 + 3 * 7168 * 2048 // 32
    assert bm["per_expert"] == per == 23396352
    assert bm["shared"] == per
    assert bm["routed"] == 256 * per
    assert bm["router"] == 4 * 256 * 7168
    assert bm["total"] == 257 * per + 4 * 256 * 7168 + 8 * 384 * 7168
    # gate_up launch: the experts' W13, the token rows of MXFP8 x, h of every pair
    assert bm["gate_up_launch"] == 256 * 2 * per // 3 + 384 * 7168 * 33 // 32 + 384 * 8 * 2048 * 33 // 32
    assert bm["gate_up_flop"] == 2 * 384 * 8 * 2 * 2048 * 7168
