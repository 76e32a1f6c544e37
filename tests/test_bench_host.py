"""Host-side helpers of bench.py, on the CPU: the closed-form committed
tokens per round against exact enumeration, the reading of the committed
rocprofv3 summary, and the one-GPU contract of the command line."""

import itertools
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _enumerated(p, d, decay):
    """E[a + 1] by summing over every accept/reject pattern of the d drafts:
    a is the number of leading accepts, depth i accepted with p decay^i."""
    total = 0.0
    for pat in itertools.product((0, 1), repeat=d):
        prob = 1.0
        for i, acc in enumerate(pat):
            q = p * decay ** i
            prob *= q if acc else 1.0 - q
        a = 0
        while a < d and pat[a]:
            a += 1
        total += prob * (a + 1)
    return total


@pytest.mark.parametrize("p,d,decay", [(0.74, 2, 1.0), (0.74, 8, 1.0), (0.69, 5, 1.0),
                                       (0.9, 15, 0.98), (0.0, 4, 1.0), (1.0, 6, 1.0)])
def test_closed_form_committed_matches_enumeration(p, d, decay):
    assert abs(bench.closed_form_committed(p, d, decay) - _enumerated(p, d, decay)) < 1e-12
    if decay == 1.0 and p < 1.0:   # the geometric closed form
        assert abs(bench.closed_form_committed(p, d) - (1 - p ** (d + 1)) / (1 - p)) < 1e-12


def test_committed_profile_reads_the_summary_table():
    path = os.path.join(ROOT, "profiles", "verify_q14b_48l_nt3_kernel_stats.md")
    want = None
    for line in open(path):
        if line.startswith("void k_qgemm<2, 4, 3, 3>("):
            want = float(line.rsplit("...", 1)[1].split()[2])
    assert want is not None
    assert bench.committed_profile("k_qgemm<2, 4, 3, 3>") == want
    assert bench.committed_profile("k_not_a_kernel<1>") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
