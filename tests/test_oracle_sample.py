"""Pins of the exact-match sampled verify (oracle.decide.sample_verify*).

* The Power page's rule for stochastic decoding ("The exactness
  transaction" and the sampler-state rule after it): with the target
  sampler's draw keyed by absolute position, multi-round speculative output
  equals one-token-at-a-time sampling token for token, whatever the drafter
  proposes.  Checked on a toy target over 7 tokens whose next-token logits
  depend on the last two tokens and the position, for three drafters (the
  sampled stream itself, uniform noise, a 60/40 mix) and several seeds.
  The one-token-at-a-time side is a plain loop over positions; the
  speculative side commits drafts and the emitted token per round.
* First-mismatch structure: a is the first row whose draw differs from the
  next draft; drafts equal to every draw give a = d and the last row's draw.
* The inverse CDF draws exactly p: over an exact grid of N uniforms each
  token is drawn N p_k times, up to one.
"""

import numpy as np

from oracle.decide import inverse_cdf, sample_verify, sample_verify_probs, softmax_t
from synth.rng import sample_uniforms, uniform

V = 7
T = 0.8


def _toy_logits(prefix, tab1, tab2):
    """Next-token logits after `prefix` (a list of ids)."""
    a = prefix[-1]
    b = prefix[-2] if len(prefix) > 1 else 0
    return tab1[a, len(prefix) % 3] + 0.5 * tab2[b]


def _autoregressive(seed, s, start, n, tab1, tab2):
    toks = list(start)
    for _ in range(n):
        pos = len(toks)                       # absolute position of the new token
        p = softmax_t(_toy_logits(toks, tab1, tab2), T)
        toks.append(inverse_cdf(p, float(uniform(seed, s, pos, 2))))
    return toks


def _speculative(seed, s, start, n, d, drafter, tab1, tab2):
    toks = list(start)                        # toks[-1] is the anchor
    rounds = 0
    while len(toks) < len(start) + n:
        ln = len(toks) - 1                    # anchor position
        drafts = [drafter(ln + 1 + j) for j in range(d)]
        ids = np.array([toks[-1]] + drafts)
        rows = [_toy_logits(toks + drafts[:r], tab1, tab2) for r in range(d + 1)]
        u = sample_uniforms(seed, [ln], d + 1)[0]
        a, e, draws = sample_verify(np.array(rows), ids, u, T)
        assert all(draws[r] == ids[r + 1] for r in range(a))
        toks += drafts[:a] + [e]
        rounds += 1
    return toks[:len(start) + n], rounds


def test_speculative_stream_equals_one_token_sampling():
    rng = np.random.default_rng(7)
    for seed in (1, 2, 3):
        tab1 = rng.normal(size=(V, 3, V)) * 1.5
        tab2 = rng.normal(size=(V, V))
        start = [3, 1, 4]
        n = 60
        ar = _autoregressive(seed, 0, start, n, tab1, tab2)
        noise = np.random.default_rng(seed)
        drafters = {
            "stream": lambda pos: ar[pos] if pos < len(ar) else 0,
            "noise": lambda pos: int(noise.integers(0, V)),
            "mixed": lambda pos: (ar[pos] if pos < len(ar) and noise.random() < 0.6
                                  else int(noise.integers(0, V))),
        }
        for name, dr in drafters.items():
            for d in (1, 3, 7):
                spec, rounds = _speculative(seed, 0, start, n, d, dr, tab1, tab2)
                assert spec == ar, (seed, name, d)
                if name == "stream":          # every draft accepted
                    assert rounds == -(-n // (d + 1)), (seed, d, rounds)


def test_first_mismatch_and_all_accepted():
    rng = np.random.default_rng(11)
    nt = 6
    p = softmax_t(rng.normal(size=(nt, 50)) * 2.0, 1.0)
    u = rng.random(nt)
    draws = [inverse_cdf(p[r], u[r]) for r in range(nt)]
    ids = np.array([5] + draws[:-1])            # every draft equals the row's draw
    a, e, dr = sample_verify_probs(p, ids, u)
    assert a == nt - 1 and e == draws[-1] and list(dr) == draws
    for j in range(nt - 1):                     # first mismatch at row j
        bad = ids.copy()
        bad[j + 1] = (draws[j] + 1) % 50
        a, e, _ = sample_verify_probs(p, bad, u)
        assert a == j and e == draws[j]


def test_inverse_cdf_draws_exactly_p():
    rng = np.random.default_rng(5)
    p = softmax_t(rng.normal(size=V) * 1.3, 1.0)
    N = 1 << 14
    counts = np.bincount([inverse_cdf(p, i / N) for i in range(N)], minlength=V)
    assert np.all(np.abs(counts - N * p) <= 1.0), (counts, N * p)


def test_sample_uniforms_are_keyed_by_position():
    u = sample_uniforms(9, [10, 20], 4)
    for s, ln in enumerate((10, 20)):
        for r in range(4):
            assert u[s, r] == uniform(9, s, ln + r + 1, 2)
    # a later round starting at a committed position reuses that position's draw
    assert sample_uniforms(9, [12], 2)[0, 0] == u[0, 2]
