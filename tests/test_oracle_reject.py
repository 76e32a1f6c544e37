"""Strict rejection sampling is lossless: exact rational enumeration.

For a toy bigram target P(.|prev) and drafter Q(.|prev) over a 3-token
vocabulary with dyadic probabilities, every multi-round speculative run is
enumerated exactly: draft ids with their Q weights, and each uniform over the
intervals between the decision's breakpoints (the oracle is evaluated at an
interior point of every interval and weighted by the exact interval length).
The distribution of the first L emitted tokens must equal the autoregressive
distribution prod_i P(t_i | t_{i-1}) exactly, as Fractions, for depths 1..3.
This is the losslessness that the DFlash/DSpark page attributes to rejection
sampling ("Both DFlash and DSpark are lossless under rejection sampling").

Special cases: p = q always accepts; a draft that the target gives zero
probability is always rejected and the residual is p itself; a one-hot p fixes
the emitted token.  Plus the sampler-state rule of the Power page (the
stream position moves once per emitted token, never for a rejected suffix).
"""

import itertools
from fractions import Fraction as Fr

import numpy as np

from oracle.decide import reject_decide_probs, reject_decide, softmax_t, inverse_cdf
from synth.rng import round_uniforms

V = 3
P = {0: [Fr(1, 2), Fr(1, 4), Fr(1, 4)],
     1: [Fr(1, 8), Fr(5, 8), Fr(1, 4)],
     2: [Fr(3, 8), Fr(1, 8), Fr(1, 2)]}
Q = {0: [Fr(1, 4), Fr(1, 4), Fr(1, 2)],
     1: [Fr(1, 2), Fr(1, 4), Fr(1, 4)],
     2: [Fr(3, 8), Fr(3, 8), Fr(1, 4)]}


def _arr(rows):
    return np.array([[float(x) for x in r] for r in rows], dtype=np.float64)


def _cuts(weights):
    c, acc = [], Fr(0)
    tot = sum(weights)
    if tot == 0:
        return []
    for w in weights:
        acc += w
        c.append(acc / tot)
    return c


def _intervals(points):
    pts = sorted(set([Fr(0), Fr(1)] + [p for p in points if 0 < p < 1]))
    return [(a, b) for a, b in zip(pts[:-1], pts[1:])]


def _round_outcomes(prev, d):
    """Exact distribution of the tokens one round emits from context `prev`."""
    out = {}
    for drafts in itertools.product(range(V), repeat=d):
        w = Fr(1)
        ctx = prev
        for x in drafts:
            w *= Q[ctx][x]
            ctx = x
        if w == 0:
            continue
        ctxs = [prev] + list(drafts)
        p_rows = [P[c] for c in ctxs]           # rows 0..d
        q_rows = [Q[c] for c in ctxs[:d]]       # rows 0..d-1
        u_pts = []
        for r in range(d):
            x = drafts[r]
            u_pts.append(_intervals([p_rows[r][x] / q_rows[r][x]] if q_rows[r][x] else []))
        res_pts = []
        for r in range(d):
            res = [max(Fr(0), p_rows[r][i] - q_rows[r][i]) for i in range(V)]
            res_pts += _cuts(res) + _cuts(p_rows[r])
        res_pts += _cuts(p_rows[d])
        u_pts.append(_intervals(res_pts))
        p_f, q_f = _arr(p_rows), _arr(q_rows) if d else np.zeros((0, V))
        ids = np.array([prev] + list(drafts))
        for box in itertools.product(*u_pts):
            vol = Fr(1)
            u = np.empty(d + 1)
            for i, (a, b) in enumerate(box):
                vol *= b - a
                u[i] = float((a + b) / 2)
            acc, em = reject_decide_probs(p_f, q_f, ids, u)
            toks = tuple(drafts[:acc]) + (em,)
            out[toks] = out.get(toks, Fr(0)) + w * vol
    return out


def _stream_dist(anchor, d, L):
    dist = {}

    def rec(prev, prefix, w):
        if len(prefix) >= L:
            key = tuple(prefix[:L])
            dist[key] = dist.get(key, Fr(0)) + w
            return
        for toks, pw in _round_outcomes(prev, d).items():
            rec(toks[-1], prefix + list(toks), w * pw)

    rec(anchor, [], Fr(1))
    return dist


def _ar_dist(anchor, L):
    dist = {}
    for seq in itertools.product(range(V), repeat=L):
        w, prev = Fr(1), anchor
        for t in seq:
            w *= P[prev][t]
            prev = t
        if w:
            dist[seq] = w
    return dist


def test_single_round_first_token_is_p():
    for d in (1, 2, 3):
        for prev in range(V):
            first = {}
            for toks, w in _round_outcomes(prev, d).items():
                first[toks[0]] = first.get(toks[0], Fr(0)) + w
            assert first == {i: P[prev][i] for i in range(V) if P[prev][i]}


def test_multi_round_stream_equals_autoregressive_exactly():
    for d, L in ((1, 3), (2, 3), (3, 4)):
        got = _stream_dist(anchor=1, d=d, L=L)
        want = _ar_dist(1, L)
        assert sum(got.values()) == 1
        assert got == want, (d, L)


def test_special_cases():
    p = np.array([[0.5, 0.25, 0.25], [0.25, 0.5, 0.25]])
    # p == q: always accepted, bonus from p_d
    for u0 in (0.0, 0.5, 0.999999):
        a, e = reject_decide_probs(p, p[:1], np.array([0, 2]), np.array([u0, 0.6]))
        assert a == 1 and e == inverse_cdf(p[1], 0.6)
    # q one-hot on x with p(x) = 0: always rejected, residual is p itself
    p0 = np.array([[0.0, 0.5, 0.5], [1, 0, 0]])
    q0 = np.array([[1.0, 0.0, 0.0]])
    for ur in (0.1, 0.6):
        a, e = reject_decide_probs(p0, q0, np.array([0, 0]), np.array([0.0, ur]))
        assert a == 0 and e == (1 if ur < 0.5 else 2)
    # draft with q(x) = 0 but p(x) > 0 is accepted (u*0 < p)
    a, _ = reject_decide_probs(np.array([[0.5, 0.5, 0], [1, 0, 0]]),
                               np.array([[0.0, 0.0, 1.0]]), np.array([0, 1]),
                               np.array([0.99, 0.3]))
    assert a == 1
    # one-hot target row fixes the emitted token whatever the uniform
    onehot = np.array([[0.0, 0.0, 1.0]])
    for ur in (0.0, 0.3, 0.999):
        assert reject_decide_probs(onehot, np.zeros((0, 3)), np.array([0]),
                                   np.array([ur])) == (0, 2)


def test_inverse_cdf_order_and_edges():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert inverse_cdf(w, 0.0) == 1
    assert inverse_cdf(w, 0.2499) == 1
    assert inverse_cdf(w, 0.25) == 3
    assert inverse_cdf(w, 0.7499) == 3
    assert inverse_cdf(w, 0.75) == 4
    assert inverse_cdf(w, 1 - 2 ** -53) == 4


def test_softmax_temperature_matches_scipy():
    from scipy.special import softmax
    rng = np.random.default_rng(4)
    z = rng.standard_normal((3, 50)) * 4
    np.testing.assert_allclose(softmax_t(z, 0.8), softmax(z / 0.8, axis=-1), rtol=1e-13)


def test_logit_level_decision_uses_temperature():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((4, 30)) * 3
    draft = logits[:3] + rng.standard_normal((3, 30)) * 0.5
    ids = np.array([0, 4, 9, 1])
    u = np.array([0.3, 0.6, 0.2, 0.7])
    for T in (0.5, 0.8, 2.0):
        want = reject_decide_probs(softmax_t(logits, T), softmax_t(draft, T), ids, u)
        assert reject_decide(logits, draft, ids, u, T) == want


def test_sampler_state_moves_once_per_emitted_token():
    """Uniforms are keyed by absolute position: after N emitted tokens the
    stream sits at position len0 + N whatever the depths, a round replayed from
    the same committed length draws identical uniforms, and a round never
    re-reads a position it has already committed."""
    seed = 1234
    len0 = 100
    u1 = round_uniforms(seed, [len0], 4)
    np.testing.assert_array_equal(u1, round_uniforms(seed, [len0], 4))
    # after emitting a+1 = 2 tokens the next round's draws start at len0 + 3
    u2 = round_uniforms(seed, [len0 + 2], 4)
    np.testing.assert_array_equal(u2[0, :1], round_uniforms(seed, [len0 + 2], 2)[0, :1])
    # acceptance draw of row r is the lane-0 draw at position len+r+1, shared by
    # every round that reaches that position as its row r
    np.testing.assert_array_equal(u1[0, 2], round_uniforms(seed, [len0 + 2], 2)[0, 0])
    assert np.all((u1 >= 0) & (u1 < 1))
    # residual lanes differ from acceptance lanes at the same position
    assert u1[0, 3] != u1[0, 0]
