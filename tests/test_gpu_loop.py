"""The device-resident multi-round loop (sv_advance) on the GPU.

A full model (one decoder layer, hidden 512, vocabulary 4096, two
sequences) first produces its own stream one token per round (nt = 1,
commit).  That stream is the stub drafter's reference: at depth j the
drafter proposes it with probability 0.7 * 0.9^j, else a noise id.  Then
rounds of nt = 4 run back to back with no host read in between, each
followed by sv_advance (emitted token -> next anchor, drafts for the next
positions, committed tokens logged by absolute position):

* greedy, eagerly and replayed from one captured HIP graph: the log equals
  the one-token stream (greedy speculative output equals autoregressive
  output, the Power page's exactness rule), the committed count equals the
  length moved, and drafts were accepted;
* sampled (SV_SAMPLE), with the next round's uniforms gathered on the device
  from a table of draws by absolute position: the log equals one-token
  sampling on the same table.

The one-token stream itself is checked against the oracle's: the oracle
decodes the same model one token at a time from the same anchors (greedy
argmax, or the inverse-CDF draw with the same table of uniforms), and the
two streams must agree token for token up to the first position whose
oracle decision is not clear (top-2 logit gap within 1e-2, or u * Z within
1e-2 of the drawn token's mass from an edge of its bin), after which a
correct kernel may legitimately take the other branch.
"""

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from synth.configs import CONFIGS
from oracle.decide import argmax_lowest, inverse_cdf, softmax_t
from oracle.model import OracleModel, rmsnorm
from synth.rng import uniform
from tests.gpu_util import top2_gap
from tests.test_gpu_round import Case

pytestmark = pytest.mark.gpu
DEV = "cuda"
S, N_REF, NT, ROUNDS, CAP = 2, 100, 4, 24, 256
P_ACCEPT, P_DECAY, TEMP, SEED = 0.7, 0.9, 0.9, 55


@pytest.fixture(scope="module")
def case():
    cfg = CONFIGS["tiny"]
    return Case(cfg.model, S, cfg.ctx, CAP, cfg.seed)


def _utab():
    s = np.arange(S, dtype=np.uint64)[:, None]
    pos = np.arange(CAP, dtype=np.uint64)[None, :]
    return uniform(SEED, s, pos, 2)


def _one_token_stream(case, mode):
    """[S][CAP] int32: the token at each position produced one per round."""
    kv = case.kv()
    lens = case.lens.astype(np.int64).copy()
    anchor = np.array([7, 3001], dtype=np.int32)
    ref = np.zeros((S, CAP), dtype=np.int32)
    ut = _utab()
    for _ in range(N_REF):
        kw = {}
        if mode == tva.SV_SAMPLE:
            kw = dict(temperature=TEMP,
                      uniforms=torch.from_numpy(ut[np.arange(S), lens + 1][:, None].copy()).to(DEV))
        out = tva.verify_round(case.model, kv, torch.from_numpy(anchor[:, None].copy()).to(DEV),
                               mode=mode, commit=1, want_logits=False, **kw)
        e = out["emitted"].cpu().numpy()
        for s in range(S):
            ref[s, lens[s] + 1] = e[s]
        lens += 1
        anchor = e.astype(np.int32)
    return ref, np.array([7, 3001], dtype=np.int32)


def _oracle_stream_prefix(case, mode, ref, start):
    """Positions (per sequence) over which the GPU's one-token stream equals
    the oracle's; every compared position is one where the oracle's
    decision is clear.  Returns the compared count per sequence."""
    om = OracleModel(case.spec, case.wnp)
    kc, vc = case.np_kv()
    ut = _utab()
    counts = []
    for s in range(S):
        tok, pos, n = int(start[s]), int(case.lens[s]), 0
        for _ in range(N_REF):
            x = om.forward_rows([(s, pos, tok)], kc, vc)[0]
            lg = om.logits_rows(rmsnorm(x, case.wnp["out_norm"], case.spec.rms_eps)[None])[0]
            if mode == tva.SV_GREEDY:
                nxt = argmax_lowest(lg)
                clear = top2_gap(lg) > 1e-2
            else:
                p = softmax_t(lg, TEMP)
                c = np.cumsum(p)
                t = ut[s, pos + 1] * c[-1]
                nxt = inverse_cdf(p, ut[s, pos + 1])
                lo = c[nxt - 1] if nxt > 0 else 0.0
                clear = min(t - lo, c[nxt] - t) > max(1e-2 * p[nxt], 1e-6 * c[-1])
            if not clear:
                break
            assert ref[s, pos + 1] == nxt, (s, pos + 1, int(ref[s, pos + 1]), nxt)
            n += 1
            tok, pos = nxt, pos + 1
        counts.append(n)
    return counts


def _run_loop(case, mode, ref, start, graph):
    rng = np.random.default_rng(9)
    draw = torch.from_numpy(rng.random((S, CAP)).astype(np.float32)).to(DEV)
    noise = torch.from_numpy(rng.integers(0, 4096, (S, CAP)).astype(np.int32)).to(DEV)
    ref_t = torch.from_numpy(ref).to(DEV)
    ut = torch.from_numpy(_utab()).to(DEV)
    kv = case.kv()
    len0 = case.lens.astype(np.int64)
    # first round's ids: the anchor and the drafter's proposals (same rule)
    ids_np = np.zeros((S, NT), dtype=np.int32)
    ids_np[:, 0] = start
    dr, no = draw.cpu().numpy(), noise.cpu().numpy()
    for s in range(S):
        p = P_ACCEPT
        for j in range(NT - 1):
            P = len0[s] + 1 + j
            ids_np[s, 1 + j] = ref[s, P] if dr[s, P] < p else no[s, P]
            p *= P_DECAY
    ids = torch.from_numpy(ids_np).to(DEV)
    uni = torch.from_numpy(_utab()[np.arange(S)[:, None],
                                   len0[:, None] + 1 + np.arange(NT)[None, :]].copy()).to(DEV)
    tokens = torch.full((S, CAP), -1, dtype=torch.int32, device=DEV)
    committed = torch.zeros(S, dtype=torch.int32, device=DEV)
    outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device=DEV),
                emitted=torch.empty(S, dtype=torch.int32, device=DEV),
                argmax=torch.empty((S, NT), dtype=torch.int32, device=DEV), logits=None)
    ws = case.model.workspace(S, NT, mode, DEV)
    kw = dict(temperature=TEMP, uniforms=uni) if mode == tva.SV_SAMPLE else {}
    adv = dict(utab=ut, uniforms=uni) if mode == tva.SV_SAMPLE else {}

    def step():
        tva.verify_round(case.model, kv, ids, mode=mode, commit=1, workspace=ws, outs=outs,
                         **kw)
        tva.sv_advance(ids, outs["accepted_len"], outs["emitted"], kv.len, tokens=tokens,
                       committed=committed, ref=ref_t, draw=draw, noise=noise,
                       p_accept=P_ACCEPT, p_decay=P_DECAY, **adv)

    if graph:
        step()                                 # the first round eagerly
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s_ = torch.cuda.Stream()
        s_.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s_):
            step()                             # captured, not run
        torch.cuda.current_stream().wait_stream(s_)
        for _ in range(ROUNDS - 1):
            g.replay()
    else:
        for _ in range(ROUNDS):
            step()
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), committed.cpu().numpy(), kv.len.cpu().numpy() - len0


def _check(case, ref, tokens, committed, moved):
    len0 = case.lens.astype(np.int64)
    np.testing.assert_array_equal(committed, moved)
    assert (committed > ROUNDS).all(), committed          # drafts were accepted
    assert (committed <= N_REF).all(), committed          # stayed inside the reference
    for s in range(S):
        span = slice(len0[s] + 1, len0[s] + 1 + committed[s])
        np.testing.assert_array_equal(tokens[s, span], ref[s, span])


@pytest.mark.parametrize("mode", [tva.SV_GREEDY, tva.SV_SAMPLE])
def test_one_token_stream_matches_oracle(case, mode):
    ref, start = _one_token_stream(case, mode)
    counts = _oracle_stream_prefix(case, mode, ref, start)
    print(f"[loop] mode {mode}: one-token stream equals the oracle's over {counts} clear positions",
          flush=True)
    assert sum(counts) >= 4, counts


@pytest.mark.parametrize("graph", [False, True])
def test_greedy_loop_equals_one_token_stream(case, graph):
    ref, start = _one_token_stream(case, tva.SV_GREEDY)
    tokens, committed, moved = _run_loop(case, tva.SV_GREEDY, ref, start, graph)
    _check(case, ref, tokens, committed, moved)


def test_sampled_loop_equals_one_token_sampling(case):
    ref, start = _one_token_stream(case, tva.SV_SAMPLE)
    tokens, committed, moved = _run_loop(case, tva.SV_SAMPLE, ref, start, graph=True)
    _check(case, ref, tokens, committed, moved)
