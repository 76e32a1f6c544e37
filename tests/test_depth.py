"""The adaptive draft-depth policy (host only, sv_depth_*), on the CPU.

Pins:
* the expected committed tokens per round: for a constant conditional
  acceptance c the policy's E(d) equals the DFlash/DSpark page's closed form
  A = (1 - c^(d+1)) / (1 - c) ("Is it worth it?"), and the Beta-smoothed
  estimate equals (a0 + successes) / (a0 + b0 + trials);
* convergence: rounds simulated from a known acceptance process and a known
  cost line T(nt) = w + nt * t_row (the weights-once cost model) drive the
  policy to a depth whose true rate is within a few percent of the best
  depth's, computed by brute force over all depths;
* hysteresis: with two depths within 5% of each other it does not flap;
* the minimum-of-four cost window ignores one slow outlier;
* optimism: with nothing observed the policy explores the deepest depth;
  the depth never exceeds d_max; bad arguments fail closed.
"""

import numpy as np
import pytest

import target_verification_amd as tva


def test_expected_tokens_match_closed_form():
    for c in (0.3, 0.74, 0.9):
        pol = tva.DepthPolicy(d_max=7, d_start=7, prior_a=1.0, prior_b=1.0, hysteresis=0.1)
        # many rounds at depth 7 whose conditional acceptance is exactly c
        # (per depth j: successes and failures in the ratio c : 1 - c)
        n = 20000
        for j in range(1, 8):
            reached = int(round(n * c ** (j - 1)))
            acc_here = int(round(reached * c))
            fail = reached - acc_here
            pol.observe(7, np.full(fail, j - 1, dtype=np.int32))
        pol.observe(7, np.full(int(round(n * c ** 7)), 7, dtype=np.int32))
        acc, cost, rate = pol.estimates()
        E = rate * cost
        for d in range(8):
            A = (1 - c ** (d + 1)) / (1 - c)
            assert abs(E[d] - A) < 2e-3 * A, (c, d, E[d], A)
        pol.close()


def test_beta_smoothing_estimate():
    pol = tva.DepthPolicy(d_max=3, d_start=3, prior_a=2.0, prior_b=3.0)
    pol.observe(3, [3, 3, 1, 0, 2])     # depth 1: 4 successes, 1 failure
    acc, _, _ = pol.estimates()
    assert abs(acc[0] - (2 + 4) / (2 + 3 + 5)) < 1e-12
    # depth 2 reached by 4 rounds: 3 accepted (3, 3, 2), 1 rejected (a = 1)
    assert abs(acc[1] - (2 + 3) / (2 + 3 + 4)) < 1e-12
    # depth 3 reached by 3 rounds: 2 accepted, 1 rejected (a = 2)
    assert abs(acc[2] - (2 + 2) / (2 + 3 + 3)) < 1e-12


def _true_rate(c, w, t_row, t_draft, d):
    E = sum(np.prod(c[:k]) for k in range(d + 1))
    return E / (w + (d + 1) * t_row + d * t_draft)


@pytest.mark.parametrize("c0,decay,t_draft", [(0.8, 1.0, 1.0), (0.9, 0.93, 0.5),
                                              (0.5, 1.0, 2.0)])
def test_policy_converges_to_the_best_depth(c0, decay, t_draft):
    rng = np.random.default_rng(int(c0 * 100) + int(t_draft * 10))
    d_max, w, t_row, S = 7, 10.0, 0.6, 4
    c = np.array([c0 * decay ** j for j in range(d_max)])
    pol = tva.DepthPolicy(d_max=d_max, d_start=2, draft_ms=t_draft)
    d = pol.next()
    for _ in range(600):
        acc = []
        for _s in range(S):
            a = 0
            while a < d and rng.random() < c[a]:
                a += 1
            acc.append(a)
        ms = (w + (d + 1) * t_row) * (1.0 + 0.05 * rng.random())   # measurement noise
        pol.observe(d, acc, ms)
        d = pol.next()
    best = max(_true_rate(c, w, t_row, t_draft, k) for k in range(d_max + 1))
    assert _true_rate(c, w, t_row, t_draft, d) >= 0.95 * best, (d, c0, t_draft)


def test_hysteresis_prevents_flapping():
    pol = tva.DepthPolicy(d_max=4, d_start=2, hysteresis=0.10)
    rng = np.random.default_rng(3)
    seen = []
    for _ in range(400):
        d = pol.next()
        seen.append(d)
        # two depths with rates within a few percent: 2 and 3
        acc = [min(d, int(rng.random() < 0.7) + int(rng.random() < 0.5)) for _ in range(4)]
        pol.observe(d, acc, 10.0 + d * 0.2)
    tail = seen[200:]
    assert sum(1 for x, y in zip(tail, tail[1:]) if x != y) <= 2, tail


def test_cost_window_ignores_one_outlier():
    pol = tva.DepthPolicy(d_max=3, d_start=1)
    for ms in (10.0, 10.2, 30.0, 10.1):
        pol.observe(1, [1], ms)
    _, cost, _ = pol.estimates()
    assert cost[1] == 10.0                     # min of the last four at nt = 2
    for ms in (11.0, 11.0, 11.0, 11.0):        # the window slides
        pol.observe(1, [1], ms)
    _, cost, _ = pol.estimates()
    assert cost[1] == 11.0


def test_optimism_cap_and_arguments():
    pol = tva.DepthPolicy(d_max=5, d_start=1)
    assert pol.next() == 5                     # nothing seen: the deepest depth
    for _ in range(50):                        # nothing is ever accepted
        d = pol.next()
        pol.observe(d, [0, 0, 0], 10.0 + 1.0 * (d + 1))
    assert pol.next() <= 1
    assert all(0 <= pol.next() <= 5 for _ in range(3))
    with pytest.raises(tva.SvError):
        pol.observe(2, [3])                    # a > d
    with pytest.raises(tva.SvError):
        pol.observe(9, [0])                    # d > d_max
    for bad in (dict(d_max=0), dict(d_max=16), dict(d_start=9), dict(prior_a=0.0),
                dict(hysteresis=-1.0), dict(draft_ms=-1.0)):
        with pytest.raises(tva.SvError):
            tva.DepthPolicy(**bad)
