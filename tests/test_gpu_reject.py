"""GPU parity of the stochastic verify decision (strict rejection sampling).

The round's lm_head logits are compared with the fp64 oracle at the logits
bar (|g - o| <= 1e-4 + 1e-3 |o|).  The decision is compared under the same
pre-generated uniforms:

* an acceptance test r is clear when |u_r - min(1, p_r(x)/q_r(x))| > 1e-2
  (p, q from the oracle's fp64 softmax at temperature T);
* the residual / bonus draw t = u_res * Z is clear when it lies farther than
  max(1e-2 * (its bin's mass), 1e-6 * Z) from both edges of its bin in the
  oracle's cumulative distribution (the second term covers the CDF's rounding
  from fp32 logits, about 5e-7 Z at vocabulary 248320);
* when every test up to the oracle's accepted length and the draw are clear,
  accepted length and emitted token must be identical;
* whether or not they are clear, the GPU's emitted token must be a valid
  draw: its bin in the oracle's distribution (the residual at the GPU's own
  accepted length, or p when nothing was rejected) must lie within 1e-4 * Z
  of the oracle's t, and the GPU's accepted length may differ from the
  oracle's only at a test that is not clear.

Inputs follow the lm_head-only stochastic workload: hidden states N(0,1),
draft logits = oracle target logits + N(0, 0.5^2), drafts sampled from
q = softmax(draft logits / T), uniforms keyed by (seed, sequence, position,
lane).
"""

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from oracle.decide import reject_decide_probs, softmax_t
from oracle.model import OracleModel
from synth.configs import CONFIGS, Config, ModelSpec
from synth.make import (draft_logits_from_target, make_anchors, make_hidden, make_weights,
                        sample_drafts_from_q)
from synth.rng import round_uniforms
from tests.gpu_util import logits_close
from tests.oracle_util import to_numpy_tensors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _small_cfg(nt, n_seq=6, seed=211):
    spec = ModelSpec(n_layer=0, hidden=512, n_head=8, n_kv_head=8, head_dim=64, ffn=1536,
                     vocab=8192, fmt_proj="b4_256", fmt_lm="b6_256", lm_only=True)
    return Config(name="lm8k_reject", seed=seed, model=spec, n_seq=n_seq, nt=(nt,), ctx=0,
                  mode="reject", temperature=0.8, drafts="sample_q", draft_noise=0.5)


def _inputs(cfg, nt, oracle):
    hidden = make_hidden(cfg, nt, DEV)
    o_logits = oracle.lm_only_logits(hidden.cpu().numpy().astype(np.float64))
    dl = draft_logits_from_target(cfg, o_logits)                    # [S][nt-1][V] fp32
    ids = sample_drafts_from_q(cfg, make_anchors(cfg), dl)          # [S][nt]
    u = round_uniforms(cfg.seed, np.zeros(cfg.n_seq, np.int64), nt)  # lm-only: len 0
    return hidden, o_logits, dl, ids, u


def _gpu(model, hidden, dl, ids, u, T):
    t_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
    t_dl = (torch.from_numpy(np.ascontiguousarray(dl)).to(DEV) if dl.shape[1] > 0 else None)
    t_u = torch.from_numpy(np.ascontiguousarray(u, dtype=np.float64)).to(DEV)
    out = tva.verify_round(model, None, t_ids, mode=tva.SV_REJECT, temperature=T,
                           hidden=hidden, draft_logits=t_dl, uniforms=t_u, want_logits=True)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def _residual(p, q, a, d):
    if a < d:
        w = np.maximum(p[a] - q[a], 0.0)
        if w.sum() == 0.0:
            w = p[a]
        return w
    return p[d]


def check_reject(o_logits, dl, ids, u, T, g):
    """Returns (sequences compared exactly, acceptance tests not clear)."""
    S, nt, V = o_logits.shape
    d = nt - 1
    exact = unclear_tests = 0
    for s in range(S):
        p = softmax_t(o_logits[s], T)
        q = softmax_t(dl[s].astype(np.float64), T) if d > 0 else np.zeros((0, V))
        a_o, e_o = reject_decide_probs(p, q, ids[s], u[s])
        a_g, e_g = int(g["accepted_len"][s]), int(g["emitted"][s])
        assert 0 <= a_g <= d and 0 <= e_g < V, (s, a_g, e_g)
        clear_tests = True
        first_unclear = None
        for r in range(min(a_o + 1, d)):
            x = ids[s, r + 1]
            ratio = p[r, x] / q[r, x] if q[r, x] > 0 else np.inf
            if abs(u[s, r] - min(1.0, ratio)) <= 1e-2:
                clear_tests = False
                unclear_tests += 1
                if first_unclear is None:
                    first_unclear = r
        # accepted length: equal, or differing only past an unclear test
        if a_g != a_o:
            assert first_unclear is not None and min(a_g, a_o) >= first_unclear, \
                (s, a_g, a_o, first_unclear)
        # the GPU's token is a valid draw from the distribution of its own a
        w = _residual(p, q, a_g, d)
        c = np.cumsum(w)
        Z = c[-1]
        t = u[s, d] * Z
        lo = c[e_g - 1] if e_g > 0 else 0.0
        assert w[e_g] > 0 and lo - 1e-4 * Z <= t <= c[e_g] + 1e-4 * Z, \
            (s, a_g, e_g, t, lo, c[e_g], Z)
        # exact match where everything is clear
        w = _residual(p, q, a_o, d)
        c = np.cumsum(w)
        Z = c[-1]
        t = u[s, d] * Z
        lo = c[e_o - 1] if e_o > 0 else 0.0
        margin = max(1e-2 * w[e_o], 1e-6 * Z)
        if clear_tests and min(t - lo, c[e_o] - t) > margin:
            assert (a_g, e_g) == (a_o, e_o), (s, a_g, e_g, a_o, e_o)
            exact += 1
    return exact, unclear_tests


@pytest.fixture(scope="module")
def small():
    cfg = _small_cfg(8)
    w = make_weights(cfg.model, cfg.seed, DEV)
    oracle = OracleModel(cfg.model, to_numpy_tensors(w))
    model = tva.Model(cfg.model, w, max_pos=128)
    return cfg, w, oracle, model


@pytest.mark.parametrize("nt", [1, 2, 8, 16])
def test_reject_small_parity(small, nt):
    cfg, _, oracle, model = small
    cfg = cfg.with_(nt=(nt,))
    hidden, o_logits, dl, ids, u = _inputs(cfg, nt, oracle)
    g = _gpu(model, hidden, dl, ids, u, cfg.temperature)
    ok, nbad, worst = logits_close(g["logits"], o_logits)
    assert ok, f"logits: {nbad} outside the bar, worst |g - o| {worst}"
    exact, unclear = check_reject(o_logits, dl, ids, u, cfg.temperature, g)
    assert exact >= cfg.n_seq // 2, (exact, unclear)


def test_reject_uniform_dependence(small):
    """Moving only the residual draw moves the emitted token the way the
    oracle's inverse CDF does (same accepted length)."""
    cfg, _, oracle, model = small
    nt = 4
    cfg = cfg.with_(nt=(nt,))
    hidden, o_logits, dl, ids, u = _inputs(cfg, nt, oracle)
    for ures in (0.0, 0.25, 0.5, 0.999):
        u2 = u.copy()
        u2[:, nt - 1] = ures
        g = _gpu(model, hidden, dl, ids, u2, cfg.temperature)
        check_reject(o_logits, dl, ids, u2, cfg.temperature, g)


def test_reject_all_accept_and_all_reject(small):
    """u = 0 accepts every test with p(x) > 0 (bonus from p_d); u just below
    1 rejects wherever p(x) < q(x)."""
    cfg, _, oracle, model = small
    nt = 6
    cfg = cfg.with_(nt=(nt,))
    hidden, o_logits, dl, ids, u = _inputs(cfg, nt, oracle)
    u0 = u.copy()
    u0[:, : nt - 1] = 0.0
    g = _gpu(model, hidden, dl, ids, u0, cfg.temperature)
    check_reject(o_logits, dl, ids, u0, cfg.temperature, g)
    assert (g["accepted_len"] == nt - 1).all()
    u1 = u.copy()
    u1[:, : nt - 1] = np.nextafter(1.0, 0.0)
    g = _gpu(model, hidden, dl, ids, u1, cfg.temperature)
    check_reject(o_logits, dl, ids, u1, cfg.temperature, g)


def test_reject_invalid_arguments(small):
    cfg, _, oracle, model = small
    nt = 3
    cfg = cfg.with_(nt=(nt,))
    hidden, o_logits, dl, ids, u = _inputs(cfg, nt, oracle)
    t_ids = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    t_dl = torch.from_numpy(dl).to(DEV)
    t_u = torch.from_numpy(u).to(DEV)
    with pytest.raises(tva.SvError) as e:   # T must be > 0
        tva.verify_round(model, None, t_ids, mode=tva.SV_REJECT, temperature=0.0,
                         hidden=hidden, draft_logits=t_dl, uniforms=t_u)
    assert e.value.status == tva.SV_E_INVALID
    with pytest.raises(tva.SvError) as e:   # uniforms are required
        tva.verify_round(model, None, t_ids, mode=tva.SV_REJECT, temperature=0.8,
                         hidden=hidden, draft_logits=t_dl, uniforms=None)
    assert e.value.status == tva.SV_E_INVALID


def test_reject_full_lm248k():
    """The full-size stochastic workload: 6-bit 248320 x 5120 lm_head, 12
    sequences, nt = 8, T = 0.8."""
    cfg = CONFIGS["lm248k_reject"]
    nt = cfg.nt[0]
    w = make_weights(cfg.model, cfg.seed, DEV)
    oracle = OracleModel(cfg.model, to_numpy_tensors(w), cache_weights=False)
    model = tva.Model(cfg.model, w, max_pos=128)
    hidden, o_logits, dl, ids, u = _inputs(cfg, nt, oracle)
    g = _gpu(model, hidden, dl, ids, u, cfg.temperature)
    ok, nbad, worst = logits_close(g["logits"], o_logits)
    assert ok, f"logits: {nbad} outside the bar, worst |g - o| {worst}"
    exact, unclear = check_reject(o_logits, dl, ids, u, cfg.temperature, g)
    print(f"lm248k_reject: {exact}/{cfg.n_seq} sequences compared exactly, "
          f"{unclear} acceptance tests within the margin; a = {g['accepted_len'].tolist()}")
    assert exact >= cfg.n_seq // 2
