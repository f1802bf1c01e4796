"""The launch variants behind the environment switches give the results of
the default launches: grouping a stream's workgroups on one XCD
(TM_XCD_STREAMS=0 turns it off) only renumbers workgroups, so y, the
retrieval and the state are bitwise the same; the small-dim first-layer
workgroups of 4 waves (TM_FIRST4=0 selects 8) sum the waves' partial tiles
in another order, so they agree to rounding, and both agree with the
oracle.  Each variant runs in a process of its own (the switches are read
once per process): 8 streams (2 x 4 heads) of 128 -> 512 -> 128, chunk 64,
256 tokens, bf16."""
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from harness import TOL, compare_state, oracle_forward, relerr, say, yerr
from oracle import tmref
from test_trained_neural_amd import inputs as I

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WL = I.Workload("variants", batch=2, seq=256, heads=4, dim=128, depth=2, expansion=4, chunk=64, dtype="bf16",
                offsets=(-7.0, 2.0, -7.0))

RUN = r"""
import sys
sys.path.insert(0, %(root)r); sys.path.insert(0, %(tests)r)
import numpy as np, torch
from harness import GpuMemory, dev_inputs
from test_trained_neural_amd import inputs as I
wl = I.Workload("variants", batch=2, seq=256, heads=4, dim=128, depth=2, expansion=4, chunk=64, dtype="bf16",
                offsets=(-7.0, 2.0, -7.0))
p = I.make_params(wl)
ci = I.make_call(wl, p)
g = GpuMemory(wl, p)
d = dev_inputs(ci, "bf16")
y = g.forward(d).cpu().numpy()
r = g.retrieve(d["q"]).cpu().numpy()
np.savez(%(out)r, y=y, r=r, st=g.export())
"""


def run_variant(env):
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "out.npz")
        code = RUN % {"root": ROOT, "tests": os.path.join(ROOT, "tests"), "out": out}
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                             env=dict(os.environ, **env))
        assert res.returncode == 0, res.stderr[-2000:]
        z = np.load(out)
        return {k: z[k] for k in ("y", "r", "st")}


def test_launch_variants_agree():
    say("case", WL)
    base = run_variant({})
    noxcd = run_variant({"TM_XCD_STREAMS": "0"})
    for k in ("y", "r", "st"):
        assert np.array_equal(base[k], noxcd[k]), k
    eight = run_variant({"TM_FIRST4": "0"})
    p = I.make_params(WL)
    ci = I.make_call(WL, p)
    ref = I.initial_state(WL, p)
    yr = oracle_forward(WL, ref, ci)
    for name, v in (("4-wave", base), ("8-wave", eight)):
        ey = yerr(v["y"], yr)
        em, es = compare_state(WL, v["st"], ref)
        er = yerr(v["r"], tmref.retrieve(WL.dim, WL.depth, WL.expansion, v["st"].astype(np.float64), ci.q))
        say("  %s first-layer workgroups: y %.2e  M %.2e  S %.2e  retrieval %.2e" % (name, ey, em, es, er))
        assert ey < TOL["bf16"] and em < TOL["bf16"] and es < 2 * TOL["bf16"] and er < TOL["bf16"]
    d = relerr(base["y"], eight["y"])
    say("  4-wave against 8-wave: y %.2e" % d)
    assert d < 5e-3
