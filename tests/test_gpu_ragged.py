"""Ragged (per-sequence nt) verify rounds on the GPU (sv_round.nts).

A ragged round must give every sequence exactly what a uniform round with
that sequence's own nt gives it:

* full model (one decoder layer, hidden 512, vocabulary 4096), greedy,
  nts = (1, 3, 8, 5) under nt = 8: the logits of each sequence's real rows,
  its accepted length and emitted token, and the cache rows it writes equal
  (bit for bit) those of a uniform round with nt = nts[s]; padding rows
  write no cache row (every other position is unchanged); the commit moves
  each length by a + 1; and each sequence's real rows also meet the oracle's
  verify round of that sequence alone (logits at the 1e-3 / 1e-4 bar, the
  decision on clear rows, the cache rows written);
* capacity is checked against nts[s]: a sequence one position short of the
  capacity verifies with nts[s] = 1 where nt = 8 fails closed; nts[s] out of
  range fails that sequence alone with SV_E_INVALID;
* lm_head-only rounds in SV_SAMPLE and SV_REJECT (vocabulary 8192, six
  sequences): logits rows and decisions equal the uniform rounds', and the
  real rows' logits meet the oracle's at the bar.
"""

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from oracle.model import OracleModel
from synth.configs import CONFIGS, Config, ModelSpec
from synth.make import make_hidden, make_weights
from synth.rng import round_uniforms, sample_uniforms
from oracle.round import verify_round as oracle_round
from tests.gpu_util import logits_close
from tests.oracle_util import to_numpy_tensors
from tests.test_gpu_round import Case, _check_greedy

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(out):
    return {k: v.cpu().numpy() for k, v in out.items() if v is not None}


def _round(model, kv, ids, commit, nts=None, **kw):
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
    n = torch.from_numpy(np.asarray(nts, dtype=np.int32)).to(DEV) if nts is not None else None
    out = tva.verify_round(model, kv, t, commit=commit, nts=n, **kw)
    torch.cuda.synchronize()
    return _np(out)


def test_ragged_greedy_equals_uniform_rounds():
    cfg = CONFIGS["tiny"]
    S, nt = 4, 8
    nts = np.array([1, 3, 8, 5], dtype=np.int32)
    case = Case(cfg.model, S, cfg.ctx, 256, cfg.seed)
    rng = np.random.default_rng(21)
    ids = rng.integers(0, cfg.model.vocab, (S, nt)).astype(np.int32)
    # make the first drafts of two sequences the target's own argmax
    dry = _round(case.model, case.kv(), ids, 0)
    ids[1, 1], ids[2, 1] = dry["argmax"][1, 0], dry["argmax"][2, 0]
    ids_pad = ids.copy()
    for s in range(S):
        ids_pad[s, nts[s]:] = -5                     # padding ids are never read
    kv_r = case.kv()
    K0, V0 = [t.cpu().numpy() for t in tva.kv_from_library_layout(kv_r.k, kv_r.v)]
    g = _round(case.model, kv_r, ids_pad, 1, nts=nts)
    Kr, Vr = [t.cpu().numpy() for t in tva.kv_from_library_layout(kv_r.k, kv_r.v)]
    lens = case.lens
    for s in range(S):
        n = int(nts[s])
        kv_u = case.kv()
        u = _round(case.model, kv_u, ids[:, :n], 0)
        Ku, Vu = [t.cpu().numpy() for t in tva.kv_from_library_layout(kv_u.k, kv_u.v)]
        np.testing.assert_array_equal(g["logits"][s, :n], u["logits"][s])
        np.testing.assert_array_equal(g["argmax"][s, :n], u["argmax"][s])
        assert (g["accepted_len"][s], g["emitted"][s]) == (u["accepted_len"][s], u["emitted"][s])
        w = slice(lens[s], lens[s] + n)
        np.testing.assert_array_equal(Kr[:, s, w], Ku[:, s, w])
        np.testing.assert_array_equal(Vr[:, s, w], Vu[:, s, w])
        rest = np.ones(Kr.shape[2], dtype=bool)
        rest[w] = False
        np.testing.assert_array_equal(Kr[:, s, rest], K0[:, s, rest])
        np.testing.assert_array_equal(Vr[:, s, rest], V0[:, s, rest])
    assert (g["accepted_len"][1:3] >= 1).all()
    np.testing.assert_array_equal(kv_r.len.cpu().numpy(), lens + g["accepted_len"] + 1)
    # each sequence's real rows against the oracle's round of that sequence alone
    om = OracleModel(case.spec, case.wnp)
    for s in range(S):
        n = int(nts[s])
        kc, vc = (a[:, s:s + 1].copy() for a in case.np_kv())
        o = oracle_round(om, ids[s:s + 1, :n], lens[s:s + 1], kc, vc, commit=False)
        ok, nbad, mx = logits_close(g["logits"][s:s + 1, :n], o["logits"])
        assert ok, (s, nbad, mx)
        sub = {"argmax": g["argmax"][s:s + 1, :n], "accepted_len": g["accepted_len"][s:s + 1],
               "emitted": g["emitted"][s:s + 1]}
        _check_greedy(o["logits"], ids[s:s + 1, :n], sub)
        w = slice(lens[s], lens[s] + n)
        for g_, o_ in ((Kr, kc), (Vr, vc)):
            a = g_[:, s, w].astype(np.float64)
            b = o_[:, 0, w].astype(np.float64)
            rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
            assert (np.abs(a - b) <= np.abs(b) * 2 ** -10 + 1e-4 * rms + 1e-7).all(), s


def test_ragged_capacity_and_bad_row_counts():
    cfg = CONFIGS["tiny"]
    S, nt, cap = 4, 8, 128
    lens = np.array([cap - 1, 64, 64, 64], dtype=np.int32)
    case = Case(cfg.model, S, cfg.ctx, cap, cfg.seed, lens=lens)
    ids = np.full((S, nt), 17, dtype=np.int32)
    g = _round(case.model, case.kv(), ids, 0)                 # uniform nt = 8
    assert g["accepted_len"][0] == tva.SV_E_CAPACITY and (g["accepted_len"][1:] >= 0).all()
    kv = case.kv()
    g = _round(case.model, kv, ids, 1, nts=[1, 8, 0, 9])
    assert g["accepted_len"][0] == 0 and g["accepted_len"][1] >= 0
    assert g["accepted_len"][2] == tva.SV_E_INVALID and g["accepted_len"][3] == tva.SV_E_INVALID
    got = kv.len.cpu().numpy()
    assert got[0] == cap and got[1] == 64 + g["accepted_len"][1] + 1
    assert got[2] == 64 and got[3] == 64                       # failed sequences: no commit


@pytest.mark.parametrize("mode", [tva.SV_SAMPLE, tva.SV_REJECT])
def test_ragged_lm_decisions_equal_uniform_rounds(mode):
    spec = ModelSpec(n_layer=0, hidden=512, n_head=8, n_kv_head=8, head_dim=64, ffn=1536,
                     vocab=8192, fmt_proj="b4_256", fmt_lm="b6_256", lm_only=True)
    S, nt, T = 6, 8, 0.8
    cfg = Config(name="lm8k_ragged", seed=404, model=spec, n_seq=S, nt=(nt,), ctx=0,
                 mode="sample", temperature=T)
    w = make_weights(spec, cfg.seed, DEV)
    model = tva.Model(spec, w, max_pos=128)
    nts = np.array([1, 2, 8, 4, 3, 6], dtype=np.int32)
    hidden = make_hidden(cfg, nt, DEV)
    rng = np.random.default_rng(8)
    ids = rng.integers(0, spec.vocab, (S, nt)).astype(np.int32)
    dl = torch.from_numpy(rng.normal(size=(S, nt - 1, spec.vocab)).astype(np.float32)).to(DEV)
    # each sequence's uniforms for its own nt, laid out in the nt-wide array
    U = np.zeros((S, nt))
    for s in range(S):
        n = int(nts[s])
        u = (sample_uniforms if mode == tva.SV_SAMPLE else round_uniforms)(
            cfg.seed, np.zeros(S, np.int64), n)
        U[s, :n] = u[s]
    kw = dict(mode=mode, temperature=T, hidden=hidden, want_logits=True)
    if mode == tva.SV_REJECT:
        kw["draft_logits"] = dl
    g = _round(model, None, ids, 0, nts=nts,
               uniforms=torch.from_numpy(U).to(DEV), **kw)
    for s in range(S):
        n = int(nts[s])
        Un = np.zeros((S, n))
        Un[s] = U[s, :n]
        kwn = dict(kw, hidden=hidden[:, :n].contiguous())
        if mode == tva.SV_REJECT:
            kwn["draft_logits"] = dl[:, : n - 1].contiguous() if n > 1 else None
        u = _round(model, None, ids[:, :n], 0, uniforms=torch.from_numpy(Un).to(DEV), **kwn)
        np.testing.assert_array_equal(g["logits"][s, :n], u["logits"][s])
        assert (g["accepted_len"][s], g["emitted"][s]) == (u["accepted_len"][s], u["emitted"][s])
    o = OracleModel(spec, to_numpy_tensors(w)).lm_only_logits(
        hidden.cpu().numpy().astype(np.float64))
    for s in range(S):
        n = int(nts[s])
        ok, nbad, mx = logits_close(g["logits"][s, :n], o[s, :n])
        assert ok, (s, nbad, mx)
