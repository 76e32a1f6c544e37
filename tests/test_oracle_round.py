"""Invariants of the greedy verify round that the pages fix.

* Greedy speculative output equals plain autoregressive output token for
  token, over many rounds with arbitrary drafts, including depth 0 (the Power
  page, the sentence after "The exactness transaction"; the minfer plan,
  section 7 "Acceptance gates").
* a is the first-mismatch index and exactly one token beyond the accepted
  drafts is emitted (Power page, steps 4 to 6; minfer plan section 3): an
  exhaustive table over a 3-token vocabulary and depths 0..3.
* Rows are causal (later drafts never change earlier rows) and a batched row
  equals the one-row computation bitwise (the oracle's own invariant).
* Commit moves the length by a+1; a dry run leaves it; replay is bitwise.
"""

import itertools

import numpy as np

from oracle.decide import greedy_decide
from oracle.model import OracleModel
from oracle.round import verify_round
from tests.oracle_util import tiny_spec, tiny_tensors, random_kv


def _setup(n_seq=1, ctx=5, cap=48, fmt="b4_32", seed=7):
    spec = tiny_spec(fmt)
    t = tiny_tensors(spec, seed)
    kc, vc = random_kv(spec, n_seq, cap, ctx)
    return spec, OracleModel(spec, t), kc, vc


def test_first_mismatch_table_exhaustive():
    V = 3
    for d in range(0, 4):
        nt = d + 1
        for am in itertools.product(range(V), repeat=nt):
            logits = np.full((nt, V), -1.0)
            for r, a in enumerate(am):
                logits[r, a] = 2.0
            for drafts in itertools.product(range(V), repeat=d):
                ids = np.array((0,) + drafts)
                a, emitted, got_am = greedy_decide(logits, ids)
                want_a = next((r for r in range(d) if am[r] != drafts[r]), d)
                assert a == want_a and emitted == am[want_a]
                assert list(got_am) == list(am)


def test_argmax_ties_lowest_id():
    logits = np.array([[0.0, 3.0, 3.0, 1.0], [5.0, 5.0, 5.0, 5.0]])
    a, e, am = greedy_decide(logits, np.array([9, 1]))
    assert list(am) == [1, 0] and a == 1 and e == 0


def test_greedy_spec_equals_autoregressive():
    spec, model, kc, vc = _setup()
    kc_ar, vc_ar = kc.copy(), vc.copy()
    n_tok = 14
    lens = np.array([5])
    anchor = 17
    ar = []
    tok = anchor
    for _ in range(n_tok):
        out = verify_round(model, np.array([[tok]]), lens, kc_ar, vc_ar)
        tok = int(out["emitted"][0])
        ar.append(tok)
        lens = out["lens"]
    # speculative: drafts are a mix of the true continuation and junk
    rng = np.random.default_rng(11)
    lens = np.array([5])
    stream = []
    tok = anchor
    depths = [0, 3, 1, 2, 4, 2, 3, 1, 4, 2]
    for d in depths:
        pos0 = len(stream)
        truth = ar[pos0: pos0 + d]
        truth = truth + [0] * (d - len(truth))
        drafts = [t if rng.random() < 0.7 else int(rng.integers(0, spec.vocab))
                  for t in truth]
        ids = np.array([[tok] + drafts])
        out = verify_round(model, ids, lens, kc, vc)
        a = int(out["accepted_len"][0])
        stream += drafts[:a] + [int(out["emitted"][0])]
        tok = stream[-1]
        assert out["lens"][0] == lens[0] + a + 1
        lens = out["lens"]
        if len(stream) >= n_tok:
            break
    assert len(stream) >= n_tok
    assert stream[:n_tok] == ar


def test_causal_rows_and_batched_equals_single_row():
    spec, model, kc, vc = _setup(n_seq=2)
    ids = np.array([[3, 8, 1, 44], [90, 2, 2, 7]])
    lens = np.array([5, 3])
    full = model.verify_logits(ids, lens, kc.copy(), vc.copy())
    for r in range(4):
        pert = ids.copy()
        pert[:, r + 1:] = (pert[:, r + 1:] + 13) % spec.vocab
        got = model.verify_logits(pert, lens, kc.copy(), vc.copy())
        np.testing.assert_array_equal(got[:, : r + 1], full[:, : r + 1])
    # teacher-forced one-row rounds reproduce each batched row bitwise
    k2, v2 = kc.copy(), vc.copy()
    for r in range(4):
        one = model.verify_logits(ids[:, r: r + 1], lens + r, k2, v2)
        np.testing.assert_array_equal(one[:, 0], full[:, r])


def test_commit_dry_run_and_replay():
    spec, model, kc, vc = _setup()
    ids = np.array([[3, 8, 1]])
    lens = np.array([5])
    a = verify_round(model, ids, lens, kc.copy(), vc.copy(), commit=False)
    assert a["lens"][0] == 5
    b = verify_round(model, ids, lens, kc.copy(), vc.copy(), commit=True)
    np.testing.assert_array_equal(a["logits"], b["logits"])
    assert b["lens"][0] == 5 + b["accepted_len"][0] + 1
    assert 0 <= b["accepted_len"][0] <= 2


def test_fp64_cache_keeps_in_block_rows_unrounded():
    """With fp64 caches the rows a round writes are the unrounded k and v:
    layer 0's row-0 k and v (computed before any cache read) round to exactly
    the fp16 run's rows, and every row's logits move only by the rounding's
    small effect (each row reads at least its own new row)."""
    spec, model, kc, vc = _setup(n_seq=2)
    ids = np.array([[3, 8, 1, 44], [90, 2, 2, 7]])
    lens = np.array([5, 3])
    k16, v16 = kc.copy(), vc.copy()
    k64, v64 = kc.astype(np.float64), vc.astype(np.float64)
    l16 = model.verify_logits(ids, lens, k16, v16)
    l64 = model.verify_logits(ids, lens, k64, v64)
    for s in range(2):
        p = lens[s]
        # row 0 of layer 0 is computed from identical inputs in both runs
        np.testing.assert_array_equal(k64[0, s, p].astype(np.float16), k16[0, s, p])
        np.testing.assert_array_equal(v64[0, s, p].astype(np.float16), v16[0, s, p])
        assert not np.array_equal(k64[0, s, p], k16[0, s, p].astype(np.float64))
        # untouched positions keep the prefilled fp16 values exactly
        np.testing.assert_array_equal(k64[:, s, :p], kc[:, s, :p].astype(np.float64))
    d = np.abs(l64 - l16).max(axis=-1)
    assert (d > 0).all() and d.max() < 1e-2
