"""Host-side checks of bench.py's contract (no GPU needed): a request for
more than one GPU exits with a message, and the workload table covers the
shapes the benchmark is quoted on."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus_requested"] == 2


def test_workload_shapes():
    sys.path.insert(0, ROOT)
    import torch
    from workloads import WORKLOADS
    expect = {  # name: (B, H, S, d_h, dtype, causal)
        "tiny": (1, 2, 64, 32, torch.float32, False),
        "launch": (1, 8, 128, 16, torch.float16, True),
        "bandwidth": (10000, 8, 128, 16, torch.float16, True),
        "compute": (16, 4, 1024, 256, torch.float16, False),
        "long": (32, 16, 100000, 64, torch.float16, True),
    }
    for name, (B, H, S, D, dt, causal) in expect.items():
        w = WORKLOADS[name]
        assert (w.B, w.H, w.S, w.D, w.dtype, w.causal) == (B, H, S, D, dt, causal), name
    assert WORKLOADS["bandwidth"].key_len == ("uniform", 64, 128)
    assert WORKLOADS["compute"].key_len == ("fixed", 1024)


def test_graph_plan_submits_exactly_the_requested_steps():
    sys.path.insert(0, ROOT)
    import bench
    for steps in (1, 5, 20, 99, 100, 101, 250, 2000):
        for graph in (0, 1, 7, 100):
            g1, n_rep, g2 = bench.graph_plan(steps, graph)
            if graph == 0:
                assert (g1, n_rep, g2) == (0, 0, 0)
                continue
            assert g1 <= graph and g2 < g1
            assert g1 * n_rep + g2 == steps, (steps, graph)


def test_default_line_is_the_long_workload_with_subrecords():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.HEADLINE == "long"
    assert set(bench.SUBRECORDS) == {"bandwidth", "compute", "launch"}
    for name in (bench.HEADLINE,) + tuple(bench.SUBRECORDS):
        assert name in bench.DEFAULT_STEPS and name in bench.BOUND
