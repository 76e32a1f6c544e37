"""GPU parity of the exact-match sampled verify (mode SV_SAMPLE).

* lm_head-only rounds against the oracle (vocabulary 8192 at nt = 1, 4, 16,
  and the full 248320-row lm_head with 12 sequences at nt = 8): logits at
  the logits bar; every
  row's draw equal to the oracle's where the draw is clear (u * Z farther
  than max(1e-2 * (the bin's mass), 1e-6 * Z) from both edges of its bin in
  the oracle's cumulative distribution), and a valid draw (its bin within
  1e-4 * Z of u * Z) everywhere; accepted length and emitted token exact
  when every draw up to the oracle's accepted row is clear.  Drafts copy the
  oracle's draws with probability 0.7 so that rounds accept several rows.
* Multi-round generation on a full model (one decoder layer, hidden 512,
  vocabulary 4096): speculative rounds of nt = 5 with a drafter that proposes
  the reference stream's token with probability 0.6 commit exactly the
  stream that nt = 1 rounds (one token at a time) sample, on the same
  uniforms keyed by absolute position.  Both sides run on the GPU, so the
  comparison is bit for bit (the pages' rule that stochastic speculative
  output advances the sampler once per emitted token).
* Argument errors fail closed.
"""

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from oracle.decide import inverse_cdf, sample_verify_probs, softmax_t
from oracle.model import OracleModel
from synth.configs import CONFIGS, Config, ModelSpec
from synth.make import make_hidden, make_weights
from synth.rng import sample_uniforms
from tests.gpu_util import logits_close
from tests.oracle_util import to_numpy_tensors
from tests.test_gpu_round import Case

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = 0.8


def _lm_cfg(nt, n_seq=6, seed=311):
    spec = ModelSpec(n_layer=0, hidden=512, n_head=8, n_kv_head=8, head_dim=64, ffn=1536,
                     vocab=8192, fmt_proj="b4_256", fmt_lm="b6_256", lm_only=True)
    return Config(name="lm8k_sample", seed=seed, model=spec, n_seq=n_seq, nt=(nt,), ctx=0,
                  mode="sample", temperature=T)


@pytest.fixture(scope="module")
def small():
    cfg = _lm_cfg(8)
    w = make_weights(cfg.model, cfg.seed, DEV)
    oracle = OracleModel(cfg.model, to_numpy_tensors(w))
    model = tva.Model(cfg.model, w, max_pos=128)
    return cfg, oracle, model


def _clear(w, k, t):
    c = np.cumsum(w)
    Z = c[-1]
    lo = c[k - 1] if k > 0 else 0.0
    return min(t - lo, c[k] - t) > max(1e-2 * w[k], 1e-6 * Z)


def _valid(w, k, t):
    c = np.cumsum(w)
    Z = c[-1]
    lo = c[k - 1] if k > 0 else 0.0
    return w[k] > 0 and lo - 1e-4 * Z <= t <= c[k] + 1e-4 * Z


def _sample_parity(cfg, oracle, model, nt, seed_drafts):
    """One SV_SAMPLE round of the lm_head-only workload against the oracle;
    returns the number of sequences compared exactly."""
    S = cfg.n_seq
    hidden = make_hidden(cfg, nt, DEV)
    o_logits = oracle.lm_only_logits(hidden.cpu().numpy().astype(np.float64))
    u = sample_uniforms(cfg.seed, np.zeros(S, np.int64), nt)        # lm-only: len 0
    rng = np.random.default_rng(seed_drafts)
    ids = np.zeros((S, nt), dtype=np.int32)
    ids[:, 0] = rng.integers(0, cfg.model.vocab, S)
    p = [softmax_t(o_logits[s], cfg.temperature) for s in range(S)]
    for s in range(S):
        for r in range(nt - 1):
            ids[s, r + 1] = (inverse_cdf(p[s][r], u[s, r]) if rng.random() < 0.7
                             else rng.integers(0, cfg.model.vocab))
    t_ids = torch.from_numpy(ids).to(DEV)
    t_u = torch.from_numpy(u).to(DEV)
    out = tva.verify_round(model, None, t_ids, mode=tva.SV_SAMPLE, temperature=cfg.temperature,
                           hidden=hidden, uniforms=t_u, want_logits=True)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items() if v is not None}
    ok, nbad, worst = logits_close(g["logits"], o_logits)
    assert ok, f"logits: {nbad} outside the bar, worst |g - o| {worst}"
    exact = 0
    for s in range(S):
        a, e, dr = sample_verify_probs(p[s], ids[s], u[s])
        clear = []
        for r in range(nt):
            t = u[s, r] * np.cumsum(p[s][r])[-1]
            assert _valid(p[s][r], int(g["argmax"][s, r]), t), (s, r)
            clear.append(_clear(p[s][r], int(dr[r]), t))
            if clear[-1]:
                assert g["argmax"][s, r] == dr[r], (s, r)
        if all(clear[: a + 1]):
            assert (g["accepted_len"][s], g["emitted"][s]) == (a, e), (s, a, e)
            exact += 1
    return exact, g


@pytest.mark.parametrize("nt", [1, 4, 16])
def test_sample_lm_parity(small, nt):
    cfg, oracle, model = small
    exact, _ = _sample_parity(cfg.with_(nt=(nt,)), oracle, model, nt, nt)
    assert exact >= cfg.n_seq // 2, exact


@pytest.mark.timeout(600)
def test_sample_full_lm248k():
    """Exact-match sampled verify at the full stochastic workload's size:
    6-bit 248320 x 5120 lm_head, 12 sequences, nt = 8, T = 0.8 (each of the
    32 vocabulary slices of a row then holds 7760 tokens, several per thread
    of the inverse-CDF kernel)."""
    cfg = CONFIGS["lm248k_reject"].with_(mode="sample")
    nt = cfg.nt[0]
    w = make_weights(cfg.model, cfg.seed, DEV)
    oracle = OracleModel(cfg.model, to_numpy_tensors(w), cache_weights=False)
    model = tva.Model(cfg.model, w, max_pos=128)
    exact, g = _sample_parity(cfg, oracle, model, nt, 248)
    print(f"lm248k sample: {exact}/{cfg.n_seq} sequences compared exactly; "
          f"a = {g['accepted_len'].tolist()}", flush=True)
    assert exact >= cfg.n_seq // 2, exact


def test_sample_multi_round_equals_one_token_sampling():
    cfg = CONFIGS["tiny"]
    S, n_tok, nt = 2, 40, 5
    case = Case(cfg.model, S, cfg.ctx, 256, cfg.seed)
    seed = 77
    start = np.array([11, 2024], dtype=np.int32)

    def run(kv, ids, lens):
        u = sample_uniforms(seed, lens, ids.shape[1])
        out = tva.verify_round(case.model, kv, torch.from_numpy(ids).to(DEV),
                               mode=tva.SV_SAMPLE, temperature=0.9,
                               uniforms=torch.from_numpy(u).to(DEV), want_logits=False)
        torch.cuda.synchronize()
        return out["accepted_len"].cpu().numpy(), out["emitted"].cpu().numpy()

    # one token at a time
    kv = case.kv()
    lens = case.lens.astype(np.int64).copy()
    anchor = start.copy()
    ref = [[] for _ in range(S)]
    for _ in range(n_tok):
        a, e = run(kv, anchor[:, None].copy(), lens)
        assert (a == 0).all()
        for s in range(S):
            ref[s].append(int(e[s]))
        lens += 1
        anchor = e.astype(np.int32)
    np.testing.assert_array_equal(kv.len.cpu().numpy(), case.lens + n_tok)

    # speculative rounds from the same cache contents
    kv = case.kv()
    lens = case.lens.astype(np.int64).copy()
    anchor = start.copy()
    got = [[] for _ in range(S)]
    rng = np.random.default_rng(3)
    rounds = 0
    while min(len(x) for x in got) < n_tok:
        ids = np.zeros((S, nt), dtype=np.int32)
        ids[:, 0] = anchor
        for s in range(S):
            for j in range(nt - 1):
                k = len(got[s]) + j              # index into the stream of this draft
                ids[s, j + 1] = (ref[s][k] if k < n_tok and rng.random() < 0.6
                                 else rng.integers(0, cfg.model.vocab))
        a, e = run(kv, ids, lens)
        for s in range(S):
            got[s] += [int(x) for x in ids[s, 1:1 + a[s]]] + [int(e[s])]
        lens += a + 1
        anchor = e.astype(np.int32)
        rounds += 1
    for s in range(S):
        assert got[s][:n_tok] == ref[s], (s, rounds)
    assert rounds < n_tok                     # some drafts were accepted


def test_sample_invalid_arguments(small):
    cfg, oracle, model = small
    nt = 3
    cfg = cfg.with_(nt=(nt,))
    hidden = make_hidden(cfg, nt, DEV)
    ids = torch.zeros((cfg.n_seq, nt), dtype=torch.int32, device=DEV)
    u = torch.from_numpy(sample_uniforms(1, np.zeros(cfg.n_seq, np.int64), nt)).to(DEV)
    dl = torch.zeros((cfg.n_seq, nt - 1, cfg.model.vocab), dtype=torch.float32, device=DEV)
    for kw in (dict(temperature=0.0, uniforms=u), dict(temperature=T, uniforms=None),
               dict(temperature=T, uniforms=u, draft_logits=dl)):
        with pytest.raises(tva.SvError) as e:
            tva.verify_round(model, None, ids, mode=tva.SV_SAMPLE, hidden=hidden, **kw)
        assert e.value.status == tva.SV_E_INVALID
