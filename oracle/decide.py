"""The per-round decision: greedy first-mismatch rule and strict rejection
sampling, on fp64.

Greedy (the minfer plan, section 3 "Mechanism -- one round"; the Power page,
"The exactness transaction", steps 4 to 6): take the argmax of every verify
row (lowest id among equal maxima); accept while the argmax of row r equals
the drafted id ids[r+1]; a is the first mismatch index (d if none); emit
argmax_a, the correction or bonus token.  Exactly one token beyond the a
accepted drafts is emitted.

Exact-match sampled verify (the Power page, "The exactness transaction",
step 4, and the sampler-state rule after it): every row r draws its token
x_r from p_r = softmax(logits_r / T) with the target sampler's own uniform
for that position; drafts are accepted while ids[r+1] == x_r, and x_a of the
first mismatching row a (or of the last row) is emitted.  Because the
uniform of a position does not depend on the round, the committed stream is
the one that sampling one token at a time produces.

Strict rejection sampling (named on the DFlash/DSpark page, "How DSpark
Works" and "Notes"; the rule itself is the textbook one): with
p_r = softmax(logits_r / T) and q_r = softmax(draft_logits_r / T), draft row r
with drafted id x = ids[r+1] is accepted iff u_r * q_r(x) < p_r(x) (this is
"accept with probability min(1, p/q)" for u uniform in [0,1), written without
a division).  At the first rejected row a the emitted token is drawn from the
normalised residual max(0, p_a - q_a); if no row is rejected (a = d) it is
drawn from p_d.  Draws use the inverse CDF in token-id order: the smallest k
with cumsum(w)[k] > u * sum(w).  A residual with zero mass (p_a = q_a up to
rounding) falls back to p_a.
"""

import numpy as np


def argmax_lowest(row: np.ndarray) -> int:
    row = np.asarray(row)
    if np.isnan(row).any():
        raise ValueError("NaN in logits row")
    return int(np.argmax(row))  # numpy returns the first (lowest) maximal index


def greedy_decide(logits: np.ndarray, ids: np.ndarray):
    """logits [nt][V], ids [nt] -> (a, emitted, argmax [nt])."""
    nt = logits.shape[0]
    am = np.array([argmax_lowest(logits[r]) for r in range(nt)], dtype=np.int64)
    d = nt - 1
    a = d
    for r in range(d):
        if am[r] != ids[r + 1]:
            a = r
            break
    return a, int(am[a]), am


def softmax_t(logits: np.ndarray, T: float) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64) / T
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def inverse_cdf(w: np.ndarray, u: float) -> int:
    """Smallest k with cumsum(w)[k] > u * total, total = cumsum(w)[-1]."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return int(np.argmax(c > u * c[-1]))


def reject_decide_probs(p: np.ndarray, q: np.ndarray, ids: np.ndarray,
                        u: np.ndarray):
    """p [nt][V] target probs, q [nt-1][V] draft probs, ids [nt] (ids[0] is the
    anchor), u [nt] uniforms (u[r] tests draft row r, u[nt-1] is the residual
    or bonus draw) -> (a, emitted)."""
    nt = p.shape[0]
    d = nt - 1
    for r in range(d):
        x = int(ids[r + 1])
        if not (u[r] * q[r, x] < p[r, x]):
            res = np.maximum(0.0, p[r] - q[r])
            if res.sum() > 0.0:
                return r, inverse_cdf(res, u[d])
            return r, inverse_cdf(p[r], u[d])
    return d, inverse_cdf(p[d], u[d])


def reject_decide(logits: np.ndarray, draft_logits: np.ndarray, ids: np.ndarray,
                  u: np.ndarray, T: float):
    """logits [nt][V], draft_logits [nt-1][V] (fp32 or fp64), T > 0."""
    p = softmax_t(logits, T)
    q = softmax_t(draft_logits, T) if draft_logits.shape[0] else \
        np.zeros((0, logits.shape[1]))
    return reject_decide_probs(p, q, ids, u)


def sample_verify_probs(p: np.ndarray, ids: np.ndarray, u: np.ndarray):
    """p [nt][V] target probs, ids [nt] (ids[0] is the anchor), u [nt] the
    sampler's uniforms for rows 0..nt-1 -> (a, emitted, draws [nt])."""
    nt = p.shape[0]
    draws = np.array([inverse_cdf(p[r], u[r]) for r in range(nt)], dtype=np.int64)
    a = nt - 1
    for r in range(nt - 1):
        if draws[r] != ids[r + 1]:
            a = r
            break
    return a, int(draws[a]), draws


def sample_verify(logits: np.ndarray, ids: np.ndarray, u: np.ndarray, T: float):
    """logits [nt][V] (fp32 or fp64), T > 0."""
    return sample_verify_probs(softmax_t(logits, T), ids, u)
