"""One verify round end to end: logits, decision, commit.

Commit follows the minfer plan's one-round mechanism (section 3): the target
wrote nt = d+1 cache rows in place; the accepted prefix keeps rows
len..len+a, and the length moves to len + a + 1; rows past that are dead and
are overwritten by the next round (no rollback copy).  A dry run (commit=0)
leaves the length unchanged, which is also how a cancelled round restores the
last committed state (the Power page, "The exactness transaction", step 7).
"""

import numpy as np

from .decide import greedy_decide, reject_decide


def verify_round(model, ids, lens, kc, vc, mode="greedy", temperature=0.0,
                 draft_logits=None, uniforms=None, commit=True, hidden=None):
    """ids int [S][nt]; lens int [S]; kc/vc fp16 caches (updated in place).

    Returns dict(logits fp64 [S][nt][V], accepted_len [S], emitted [S],
    lens [S] after commit, argmax [S][nt] in greedy mode)."""
    ids = np.asarray(ids)
    lens = np.asarray(lens, dtype=np.int64)
    S, nt = ids.shape
    if hidden is not None:
        logits = model.lm_only_logits(np.asarray(hidden, dtype=np.float64))
    else:
        logits = model.verify_logits(ids, lens, kc, vc)
    acc = np.zeros(S, dtype=np.int64)
    emi = np.zeros(S, dtype=np.int64)
    am = np.zeros((S, nt), dtype=np.int64)
    for s in range(S):
        if mode == "greedy":
            acc[s], emi[s], am[s] = greedy_decide(logits[s], ids[s])
        elif mode == "reject":
            acc[s], emi[s] = reject_decide(logits[s], np.asarray(draft_logits[s]),
                                           ids[s], np.asarray(uniforms[s]),
                                           temperature)
        else:
            raise ValueError(mode)
    new_lens = lens + acc + 1 if commit else lens.copy()
    return dict(logits=logits, accepted_len=acc, emitted=emi, lens=new_lens,
                argmax=am)
