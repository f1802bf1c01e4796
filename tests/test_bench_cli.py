"""bench.py's command line on the host: more than one GPU is refused with a
message before anything touches a GPU, and the work-model helpers agree with
the workload shapes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from test_trained_neural_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr


def test_work_model():
    wl = I.WORKLOADS["mlp384"]
    # the layer-1 forward of every key and query row: 2 x 2 x 1024 x 1536 x 384 flops per stream
    assert bench.fwd_flops(wl, 2, 1024) == 2 * 2 * 2 * 1024 * 1536 * 384
    assert bench.bwd_flops(wl, 2, 1024) == 0
    # the per-token read at depth 1: scores, the two chunk-start products, the
    # correction and the output layer's Delta, per chunk and stream
    lin = I.WORKLOADS["linear64"]
    b, d = lin.chunk, lin.dim
    per = 2 * b * b * d + 4 * b * d * d + 2 * b * b * d + 2 * b * d * d
    assert bench.token_read_flops(lin, 1, lin.tokens_per_call) == per * (lin.tokens_per_call // b)
    # the projection kernel: three projections and three gates per token
    assert bench.project_flops(wl, 2, 1024) == 2 * 2 * 1024 * 384 * (3 * 384 + 3)
