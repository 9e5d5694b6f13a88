"""The library's debugging switches (needs an MI355X): with RPA_LOG set a
forward call prints its plan, and with RPA_TRACE set it brackets its
launches with roctx ranges; neither changes a result. The switches are read
once per process, so the calls run in a child process with them set and are
compared bit for bit with the same calls in this one."""

import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as wl
from gpu_util import run_numpy

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import numpy as np
import workloads as wl
from gpu_util import run_numpy
out, lse = run_numpy(wl.named(1))
np.savez({path!r}, out=out, lse=lse)
"""


def test_plan_log_and_trace_ranges_leave_results_unchanged(tmp_path):
    w = wl.named(1)
    ref_out, ref_lse = run_numpy(w)
    path = str(tmp_path / "child.npz")
    env = dict(os.environ, RPA_LOG="1", RPA_TRACE="1")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), path=path)
    print("[debug-env] child run with RPA_LOG=1 RPA_TRACE=1", flush=True)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    got = np.load(path)
    T = w.valid_tokens()
    assert np.array_equal(got["out"][:T], ref_out[:T]) and np.array_equal(got["lse"][:T], ref_lse[:T])
    # the tiny workload: q_lens [1, 5, 16] with G = 2 give 2, 10 and 32 packed
    # rows, so two decode sequences (4 units over 2 kv heads) and one prefill
    # sequence (one 32-row unit per kv head)
    lines = [l for l in r.stderr.splitlines() if l.startswith("rpa plan:")]
    assert lines, r.stderr[-2000:]
    assert "decode 2 seqs, 4 units" in lines[0] and "prefill 2 units" in lines[0], lines[0]
