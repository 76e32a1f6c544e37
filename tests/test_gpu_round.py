"""GPU parity of whole verify rounds against the fp64 oracle.

Bars (stated for the workloads): logits |g - o| <= 1e-4 + 1e-3 |o|; a row's
argmax must match wherever the oracle's top-2 gap exceeds 1e-2, and the
accepted length and emitted token must match whenever every row up to the
oracle's accepted length is that clear; the GPU's own row bits must not
depend on nt.  Cache rows written by the round must match the oracle's fp16
rows to one fp16 rounding (the GPU rounds an fp32 value, the oracle an fp64
one) plus 1e-4 of the cache row's RMS for the fp32 rounding that deeper
layers accumulate in near-cancelling values (the logits' 1e-4 absolute bar,
carried to the row's own scale).
"""

import os

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from oracle.decide import greedy_decide
from oracle.model import OracleModel
from oracle.round import verify_round as oracle_round
from synth.configs import CONFIGS, ModelSpec
from synth.make import make_weights, make_kv, make_anchors, chain_drafts, kv_capacity
from tests.gpu_util import logits_close, top2_gap
from tests.oracle_util import to_numpy_tensors

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Case:
    def __init__(self, spec, n_seq, ctx, cap, seed, lens=None):
        self.spec = spec
        self.w = make_weights(spec, seed, DEV)
        self.wnp = to_numpy_tensors(self.w)
        from synth.configs import Config
        cfg = Config(name="t", seed=seed, model=spec, n_seq=n_seq, nt=(1,), ctx=ctx,
                     mode="greedy")
        self.K, self.V, l0 = make_kv(cfg, cap, DEV)
        self.lens = np.asarray(lens if lens is not None else l0, dtype=np.int32)
        self.cap = cap
        self.oracle = OracleModel(spec, self.wnp)
        self.model = tva.Model(spec, self.w, max_pos=cap)

    def kv(self):
        return tva.KVCache.from_logical(self.K, self.V, self.lens)

    def np_kv(self):
        return self.K.cpu().numpy().copy(), self.V.cpu().numpy().copy()

    def oracle_argmax_fn(self):
        def fn(prefix, need=None):
            kc, vc = self.np_kv()
            lg = self.oracle.verify_logits(prefix, self.lens, kc, vc)
            return np.argmax(lg[:, -1], axis=-1)
        return fn


def _gpu_round(case, ids, kv=None, commit=1, **kw):
    kv = kv or case.kv()
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
    out = tva.verify_round(case.model, kv, t, commit=commit, **kw)
    torch.cuda.synchronize()
    return kv, {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def _check_greedy(o_logits, ids, g):
    S, nt, _ = o_logits.shape
    excluded = 0
    for s in range(S):
        a, e, am = greedy_decide(o_logits[s], ids[s])
        gaps = [top2_gap(o_logits[s, r]) for r in range(nt)]
        for r in range(nt):
            if gaps[r] > 1e-2:
                assert g["argmax"][s, r] == am[r], (s, r)
            else:
                excluded += 1
        if all(gp > 1e-2 for gp in gaps[: a + 1]):
            assert g["accepted_len"][s] == a and g["emitted"][s] == e, (s, a, e)
    return excluded


def _check_cache_rows(case, kv, o_kc, o_vc, lens, nt):
    gk, gv = tva.kv_from_library_layout(kv.k, kv.v)
    gk, gv = gk.cpu().numpy(), gv.cpu().numpy()
    K0, V0 = case.np_kv()
    for s in range(len(lens)):
        new = slice(lens[s], lens[s] + nt)
        for nm, g_, o_ in (("k", gk, o_kc), ("v", gv, o_vc)):
            a = g_[:, s, new].astype(np.float64)
            b = o_[:, s, new].astype(np.float64)
            rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))   # per (layer, pos, head)
            r = np.abs(a - b) / (np.abs(b) * 2 ** -10 + 1e-4 * rms + 1e-7)
            i = np.unravel_index(int(np.argmax(r)), r.shape)
            assert r.max() <= 1.0, f"{nm} seq {s}: worst {r.max():.3g} at {i}: gpu {a[i]!r} oracle {b[i]!r}" 
        keep = np.ones(case.cap, bool)
        keep[new] = False
        np.testing.assert_array_equal(gk[:, s, keep], K0[:, s, keep])
        np.testing.assert_array_equal(gv[:, s, keep], V0[:, s, keep])


def test_tiny_round_matches_oracle():
    cfg = CONFIGS["tiny"]
    case = Case(cfg.model, cfg.n_seq, cfg.ctx, kv_capacity(cfg), cfg.seed)
    ids = chain_drafts(cfg, make_anchors(cfg), 3, case.oracle_argmax_fn())
    kc, vc = case.np_kv()
    o = oracle_round(case.oracle, ids, case.lens, kc, vc)
    kv, g = _gpu_round(case, ids)
    ok, nbad, mx = logits_close(g["logits"], o["logits"])
    assert ok, (nbad, mx)
    # rows whose oracle top-2 gap is within 1e-2 are excluded by the margin rule
    assert _check_greedy(o["logits"], ids, g) < 3
    if g["accepted_len"][0] == o["accepted_len"][0]:
        np.testing.assert_array_equal(kv.len.cpu().numpy(), o["lens"])
    _check_cache_rows(case, kv, kc, vc, case.lens, 3)


MINI = {
    "gqa64": ModelSpec(n_layer=2, hidden=512, n_head=8, n_kv_head=2, head_dim=64, ffn=1024,
                       vocab=2048, fmt_proj="b4_256", fmt_lm="b6_256"),
    "gqa128": ModelSpec(n_layer=2, hidden=512, n_head=4, n_kv_head=1, head_dim=128, ffn=768,
                        vocab=1024, fmt_proj="b4_256", fmt_lm="b6_256"),
}


@pytest.fixture(scope="module", params=sorted(MINI))
def mini(request):
    return Case(MINI[request.param], 2, 300, 384, seed=77, lens=[300, 171])


def test_mini_round_matches_oracle_and_nt_invariance(mini):
    rng = np.random.default_rng(3)
    V = mini.spec.vocab
    nt_max = 16
    ids = rng.integers(0, V, size=(2, nt_max)).astype(np.int32)
    kc, vc = mini.np_kv()
    o = oracle_round(mini.oracle, ids, mini.lens, kc, vc)
    kv, g = _gpu_round(mini, ids)
    ok, nbad, mx = logits_close(g["logits"], o["logits"])
    assert ok, (nbad, mx)
    excl = _check_greedy(o["logits"], ids, g)
    assert excl <= 8
    np.testing.assert_array_equal(kv.len.cpu().numpy(),
                                  mini.lens + g["accepted_len"] + 1)
    _check_cache_rows(mini, kv, kc, vc, mini.lens, nt_max)
    # nt-invariance: dry runs at smaller nt reproduce the first rows bitwise
    for nt in (1, 2, 5, 9):
        _, gn = _gpu_round(mini, ids[:, :nt], commit=0)
        np.testing.assert_array_equal(gn["logits"], g["logits"][:, :nt])


@pytest.mark.parametrize("ctx,lens,cap", [(1020, [1020, 1015], 1152),
                                          (8188, [8188, 8183], 8320)])
def test_merge_order_agrees_across_chunk_boundaries(ctx, lens, cap):
    """The attention merge deals 128-key chunks to eight lanes by chunk
    index (lane q: chunks q, q + 8, ...), eight chunks per lane and batch.
    At 1020 keys (8 chunks) every lane holds one chunk up to nt = 4 and lane
    0 takes a ninth chunk from nt = 5; at 8188 keys (64 chunks) lane 0
    starts a second batch from nt = 5.  The new chunk lies past every key
    that rows 0..3 see, so the nt = 1 and 4 rows must equal the first rows
    of the nt = 9 and 16 rounds bit for bit; the nt = 16 round matches the
    oracle."""
    spec = MINI["gqa128"]
    case = Case(spec, 2, ctx, cap, seed=91, lens=lens)
    rng = np.random.default_rng(4)
    ids = rng.integers(0, spec.vocab, size=(2, 16)).astype(np.int32)
    kc, vc = case.np_kv()
    o = oracle_round(case.oracle, ids, case.lens, kc, vc)
    _, g = _gpu_round(case, ids, commit=0)
    ok, nbad, mx = logits_close(g["logits"], o["logits"])
    assert ok, (nbad, mx)
    for nt in (1, 4, 9):
        _, gn = _gpu_round(case, ids[:, :nt], commit=0)
        np.testing.assert_array_equal(gn["logits"], g["logits"][:, :nt])


def test_mini_greedy_spec_equals_autoregressive(mini):
    """GPU greedy speculation emits exactly the GPU autoregressive stream."""
    n_tok = 24
    kv = mini.kv()
    tok = np.array([5, 9], dtype=np.int32)
    ar = [[], []]
    for _ in range(n_tok):
        kv, g = _gpu_round(mini, tok[:, None], kv=kv)
        tok = g["emitted"].astype(np.int32)
        for s in range(2):
            ar[s].append(int(tok[s]))
    kv = mini.kv()
    rng = np.random.default_rng(9)
    stream = [[], []]
    cur = np.array([5, 9], dtype=np.int32)
    while min(len(x) for x in stream) < n_tok:
        d = int(rng.integers(0, 8))
        ids = np.zeros((2, d + 1), dtype=np.int32)
        ids[:, 0] = cur
        for s in range(2):
            p = len(stream[s])
            truth = ar[s][p: p + d]
            truth = truth + [0] * (d - len(truth))
            ids[s, 1:] = [t if rng.random() < 0.75 else int(rng.integers(0, mini.spec.vocab))
                          for t in truth]
        kv, g = _gpu_round(mini, ids, kv=kv)
        for s in range(2):
            a = int(g["accepted_len"][s])
            stream[s] += [int(t) for t in ids[s, 1: a + 1]] + [int(g["emitted"][s])]
            cur[s] = stream[s][-1]
    for s in range(2):
        assert stream[s][:n_tok] == ar[s]


def test_capacity_overflow_is_flagged_without_side_effects():
    spec = MINI["gqa64"]
    case = Case(spec, 2, 300, 384, seed=5, lens=[300, 380])
    kv = case.kv()
    ids = np.zeros((2, 8), dtype=np.int32)
    k0, v0 = kv.k.clone(), kv.v.clone()
    kv, g = _gpu_round(case, ids, kv=kv)
    assert g["accepted_len"][1] == tva.SV_E_CAPACITY
    assert 0 <= g["accepted_len"][0] <= 7
    lens = kv.len.cpu().numpy()
    assert lens[1] == 380 and lens[0] == 300 + g["accepted_len"][0] + 1
    # sequence 1's cache is untouched
    assert torch.equal(kv.k[:, 1], k0[:, 1]) and torch.equal(kv.v[:, 1], v0[:, 1])


def test_invalid_and_unsupported_arguments_fail_closed():
    spec = MINI["gqa64"]
    case = Case(spec, 1, 64, 128, seed=6)
    kv = case.kv()
    ids = torch.zeros((1, 17), dtype=torch.int32, device=DEV)
    with pytest.raises(tva.SvError) as e:
        tva.verify_round(case.model, kv, ids)
    assert e.value.status == tva.SV_E_UNSUPPORTED
    ids = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(tva.SvError) as e:
        tva.verify_round(case.model, kv, ids, mode=tva.SV_REJECT, temperature=0.0)
    assert e.value.status == tva.SV_E_INVALID
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(tva.SvError) as e:
        tva.verify_round(case.model, kv, ids, workspace=ws)
    assert e.value.status == tva.SV_E_INVALID
    # empty rounds: no sequence, or no row per sequence
    for shape in ((0, 4), (1, 0)):
        for static in (False, True):
            with pytest.raises(tva.SvError) as e:
                tva.verify_round(case.model, kv, torch.zeros(shape, dtype=torch.int32, device=DEV),
                                 static_scratch=static)
            assert e.value.status == tva.SV_E_INVALID, (shape, static)
    torch.cuda.synchronize()
    assert int(kv.len[0]) == 64


def test_fault_after_verify_leaves_length(monkeypatch):
    spec = MINI["gqa64"]
    case = Case(spec, 1, 64, 128, seed=8)
    kv = case.kv()
    monkeypatch.setenv("SV_FAULT", "after_verify")
    with pytest.raises(tva.SvError) as e:
        tva.verify_round(case.model, kv, torch.zeros((1, 4), dtype=torch.int32, device=DEV))
    assert e.value.status == tva.SV_E_FAULT_INJECTED
    torch.cuda.synchronize()
    assert int(kv.len[0]) == 64


def test_poisoned_rejected_rows_are_never_read(monkeypatch):
    """NaN in every rejected cache row must not reach the next round."""
    spec = MINI["gqa64"]
    case = Case(spec, 2, 200, 256, seed=10)
    rng = np.random.default_rng(1)
    ids = rng.integers(0, spec.vocab, size=(2, 6)).astype(np.int32)
    kv_a = case.kv()
    monkeypatch.setenv("SV_DEBUG_POISON", "1")
    kv_a, ga = _gpu_round(case, ids, kv=kv_a)
    kv_b = case.kv()
    monkeypatch.delenv("SV_DEBUG_POISON")
    kv_b, gb = _gpu_round(case, ids, kv=kv_b)
    nxt = np.stack([ga["emitted"], ga["emitted"]], 1).astype(np.int32)
    nxt[:, 1] = (nxt[:, 1] + 1) % spec.vocab
    _, ra = _gpu_round(case, nxt, kv=kv_a)
    _, rb = _gpu_round(case, nxt, kv=kv_b)
    assert np.isfinite(ra["logits"]).all()
    np.testing.assert_array_equal(ra["logits"], rb["logits"])


def _garbage_past_lengths(case):
    """Cache positions at or past each sequence's length hold large values,
    so a key read past L would change the logits."""
    for s, l in enumerate(case.lens):
        K = case.K.clone()
        K[:, s, int(l):] = 7.0
        V = case.V.clone()
        V[:, s, int(l):] = -7.0
        case.K, case.V = K, V
    return case.kv()


@pytest.mark.parametrize("static", [False, True])
def test_max_len_narrows_attention_with_the_same_bits(static):
    """A length bound (sv_round.max_len) makes attention visit only the
    chunks below max_len + nt of a cache whose capacity is 16 chunks; the
    logits, decisions, committed lengths and cache rows are those of the
    unbounded round, bit for bit."""
    spec = MINI["gqa64"]
    lens = [300, 517, 129]
    case = Case(spec, 3, 520, 2048, seed=11, lens=lens)
    rng = np.random.default_rng(3)
    ids = rng.integers(0, spec.vocab, size=(3, 5)).astype(np.int32)
    base = None
    for ml in (0, max(lens), max(lens) + 200, 2048, 2**31 - 1):
        kv = _garbage_past_lengths(case)
        kv, g = _gpu_round(case, ids, kv=kv, max_len=ml, static_scratch=static)
        res = dict(g, len=kv.len.cpu().numpy(), k=kv.k.cpu().numpy(), v=kv.v.cpu().numpy())
        assert (res["accepted_len"] >= 0).all(), (ml, res["accepted_len"])
        if base is None:
            base = res
            continue
        for key in ("logits", "argmax", "accepted_len", "emitted", "len", "k", "v"):
            assert np.array_equal(res[key], base[key]), (ml, key)


def test_length_above_max_len_fails_that_sequence_alone():
    spec = MINI["gqa64"]
    lens = [300, 517, 129]
    case = Case(spec, 3, 520, 2048, seed=12, lens=lens)
    rng = np.random.default_rng(4)
    ids = rng.integers(0, spec.vocab, size=(3, 4)).astype(np.int32)
    kv0, ref = _gpu_round(case, ids, kv=case.kv())
    kv = case.kv()
    k0, v0 = kv.k.clone(), kv.v.clone()
    kv, g = _gpu_round(case, ids, kv=kv, max_len=516)
    assert g["accepted_len"][1] == tva.SV_E_INVALID and g["emitted"][1] == -1
    got_len = kv.len.cpu().numpy()
    assert got_len[1] == 517
    assert torch.equal(kv.k[:, 1], k0[:, 1]) and torch.equal(kv.v[:, 1], v0[:, 1])
    for s in (0, 2):
        assert g["accepted_len"][s] == ref["accepted_len"][s]
        assert g["emitted"][s] == ref["emitted"][s]
        assert np.array_equal(g["logits"][s], ref["logits"][s])
        assert got_len[s] == int(kv0.len[s])
    with pytest.raises(tva.SvError) as e:
        tva.verify_round(case.model, case.kv(), torch.from_numpy(ids).to(DEV), max_len=-1)
    assert e.value.status == tva.SV_E_INVALID


def test_max_len_sizes_the_static_scratch():
    """The no-allocation entry point lays its workspace out for the chunks
    the round visits: a cache of 65536 positions needs more than the scratch
    array holds, a length bound of 200 does not, and the bounded round's
    results equal the allocating entry point's unbounded ones."""
    spec = MINI["gqa64"]
    case = Case(spec, 5, 200, 65536, seed=13)
    rng = np.random.default_rng(5)
    ids = torch.from_numpy(rng.integers(0, spec.vocab, size=(5, 16)).astype(np.int32)).to(DEV)
    with pytest.raises(tva.SvError) as e:
        tva.verify_round(case.model, case.kv(), ids, commit=0, static_scratch=True)
    assert e.value.status == tva.SV_E_UNSUPPORTED
    ref = tva.verify_round(case.model, case.kv(), ids, commit=0)
    got = tva.verify_round(case.model, case.kv(), ids, commit=0, static_scratch=True, max_len=200)
    torch.cuda.synchronize()
    for key in ("logits", "argmax", "accepted_len", "emitted"):
        assert torch.equal(got[key], ref[key]), key
