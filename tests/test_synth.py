"""The seeded input generators: published SplitMix64 vectors, workload sizes,
and the synthetic drafter's acceptance law.

The closed form E[a+1] = (1 - p^(K+1)) / (1 - p) for K drafts with
per-position acceptance p is the wiki page's break-even arithmetic ("Is it
worth it?", step 2); the depth-decayed law of the block workload is
E[a+1] = 1 + sum_k prod_{i<k} p_i.
"""

import numpy as np
import pytest

from synth.configs import CONFIGS, weight_bytes, kv_read_bytes
from synth.make import chain_drafts, accept_prob
from synth.rng import splitmix64_stream, round_uniforms, fmix64, GAMMA


def test_splitmix64_published_vectors():
    # state 0 and state 1234567: the reference outputs of the published algorithm
    assert splitmix64_stream(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                       0x06C45D188009454F]
    assert splitmix64_stream(1234567, 2) == [6457827717110365317, 3203168211198807973]
    # the vectorised output function is the same map
    assert int(fmix64(np.uint64(GAMMA))) == 0xE220A8397B1DCDAF


def test_uniform_range_and_independence():
    u = round_uniforms(9, np.arange(0, 4000, 7), 9)
    assert u.shape == (572, 9) and np.all((u >= 0) & (u < 1))
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005


def test_workload_byte_counts():
    """Round bytes (weights once + KV read) of each workload."""
    c = CONFIGS
    assert weight_bytes(c["tiny"].model) == 3_096_576
    assert weight_bytes(c["q7b_4l"].model) == 971_421_696
    assert weight_bytes(c["q14b_48l"].model) == 8_070_451_200
    assert weight_bytes(c["lm248k_reject"].model) == 1_042_944_000
    assert weight_bytes(c["q14b_8l_block16"].model) == 2_281_574_400
    assert kv_read_bytes(c["q14b_48l"], 3) == 805_896_192
    assert kv_read_bytes(c["q14b_48l"], 9) == 807_075_840
    assert kv_read_bytes(c["q14b_8l_block16"], 16) == 207_618_048
    assert kv_read_bytes(c["tiny"], 3) == 137_216
    # logits readback of the pages' example: 3 rows x 152064 x 4 B ~ 1.8 MB
    assert 3 * c["q14b_48l"].model.vocab * 4 == 1_824_768


@pytest.mark.parametrize("name,nt", [("tiny", 3), ("q14b_48l", 3), ("q14b_48l", 9), ("q14b_8l_block16", 16),
                                     ("q7b_4l", 8)])
def test_draft_chain_acceptance_law(name, nt):
    cfg = CONFIGS[name].with_(n_seq=20000)
    V = cfg.model.vocab
    target = lambda prefix, need=None: (prefix[:, -1].astype(np.int64) * 31 + 7) % V
    needed = []

    def target_logged(prefix, need):
        needed.append(need.copy())
        return target(prefix)
    ids = chain_drafts(cfg, np.arange(20000, dtype=np.int32) % V, nt, target_logged)
    d = nt - 1
    a = np.full(cfg.n_seq, d)
    for s_ in range(cfg.n_seq):
        for r in range(d):
            if ids[s_, r + 1] != target(ids[s_:s_ + 1, : r + 1])[0]:
                a[s_] = r
                break
    probs = [accept_prob(cfg, i) for i in range(d)]
    closed = 1 + sum(np.prod(probs[:k + 1]) for k in range(d))
    if cfg.p_decay == 1.0 and d:
        p = probs[0]
        assert abs(closed - (1 - p ** (d + 1)) / (1 - p)) < 1e-12
    se = np.sqrt(np.var(a + 1) / cfg.n_seq)
    assert abs(np.mean(a + 1) - closed) < 5 * se + 1e-9, (np.mean(a + 1), closed)
    if cfg.drafts != "oracle_corrupt":
        # a sequence's argmax is asked for only up to its first miss
        for r, need in enumerate(needed, start=1):
            np.testing.assert_array_equal(need, a >= r - 1)


def test_closed_forms_quoted_for_the_workloads():
    f = lambda p, K: (1 - p ** (K + 1)) / (1 - p)
    assert round(f(0.74, 2), 4) == 2.2876
    assert round(f(0.74, 8), 4) == 3.5902
    assert round(f(0.7, 2), 2) == 2.19
    p = [0.9 * 0.98 ** i for i in range(15)]
    assert round(1 + sum(np.prod(p[:k + 1]) for k in range(15)), 4) == 6.0126
