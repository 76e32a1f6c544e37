"""Greedy verify rounds at the workloads' full shapes on the GPU, against the
fp64 oracle at full depth.

* q7b_4l (4 layers of the 7B shape, vocabulary 152064, context 2048): the
  oracle builds the draft chain (acceptance 0.69, uniform after the first
  miss) and supplies every row's logits; the GPU runs nt = 1..8 with
  commit = 0.  Logits at the 1e-3 / 1e-4 bar, greedy decision on clear
  rows, cache rows written, and the GPU's own row bits identical at every nt.
* q14b_48l (the whole 48-layer 14B-shaped stack, context 4096, vocabulary
  152064): the oracle builds the nt = 9 draft chain (acceptance 0.74, uniform
  after the first miss) and computes all nine rows through all 48 layers;
  every logit of the GPU's nt = 1, 3 and 9 rounds is held to the bar, the
  argmax, accepted length and emitted token on clear rows, and the cache rows
  written in all 48 layers.  The same stack also runs the GPU-only property
  checks (row bits across nt, decision rule, commit, untouched cache rows)
  on drafts that follow the GPU's own argmax chain.
* q14b_8l_block16 (8 layers, vocabulary 248320, context 512, 12 sequences):
  the GPU runs all 12 sequences at nt = 16 (the wide-row kernels, M = 192)
  and nt = 1; two sequences follow the oracle's draft chain (acceptance
  0.9 * 0.98^depth, uniform after the first miss) and are compared with the
  oracle at full depth, the other ten carry uniform random drafts.  A one-
  layer variant with random ids on every sequence does the same for three
  sequences.

Logits bar: 1e-4 + 1e-3 |o| per logit, widened per row by twice the
oracle's own effect of rounding the in-block cache rows to fp16 (the oracle
run again with an unrounded fp64 cache): where an in-block k or v value lies
within the kernel's fp32 error of an fp16 rounding boundary, the GPU and the
oracle may store neighbouring codes, both correct, and later rows and layers
carry the difference.  Each test prints how many logits lie outside the
plain bar and how large the widening is next to the base bar.

The oracle's rows are computed layer by layer for each batch of rows whose
ids are known (one pass over the layers per step of the draft chain); no
oracle input comes from the GPU.
"""

import time

import numpy as np
import pytest
import torch
from dataclasses import replace

import target_verification_amd as tva
from oracle.decide import argmax_lowest
from oracle.model import OracleModel, rmsnorm
from synth.configs import CONFIGS
from synth.make import chain_drafts, kv_capacity, make_anchors, make_kv, make_weights
from tests.gpu_util import logits_close
from tests.oracle_util import to_numpy_tensors
from tests.test_gpu_round import Case, _check_cache_rows, _check_greedy, _gpu_round

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[full] {msg}", flush=True)


class OracleChain:
    """Oracle logits of the rows of a growing id prefix.  Each row is
    computed once, in batches: every call evaluates the rows whose ids it
    has not seen yet, for the sequences asked for, in one layer-by-layer
    pass (their cache rows are written into the oracle's own copy of the
    cache, where later rows read them)."""

    def __init__(self, spec, wnp, K, V, lens):
        self.spec, self.lens = spec, np.asarray(lens, dtype=np.int64)
        self.om = OracleModel(spec, wnp, cache_weights=False)
        self.out_norm = wnp["out_norm"]
        self.kc, self.vc = K.copy(), V.copy()
        self.rows = {}

    def _extend(self, ids, seqs):
        todo = []
        for s in seqs:
            have = self.rows.setdefault(int(s), [])
            for r in range(len(have), ids.shape[1]):
                todo.append((int(s), int(self.lens[s]) + r, int(ids[s, r])))
        if not todo:
            return
        t0 = time.time()

        def prog(l, n_layer):
            if (l + 1) % 8 == 0 or l + 1 == n_layer:
                say(f"oracle: {len(todo)} rows through layer {l + 1}/{n_layer} "
                    f"({time.time() - t0:.0f} s)")
        x = self.om.forward_rows(todo, self.kc, self.vc, progress=prog)
        fin = np.stack([rmsnorm(xi, self.out_norm, self.spec.rms_eps) for xi in x])
        lg = self.om.logits_rows(fin)
        for (s, _, _), row in zip(todo, lg):
            self.rows[s].append(row)

    def argmax_fn(self, seqs):
        """argmax_fn for chain_drafts restricted to the sequences `seqs`."""
        def fn(prefix, need=None):
            want = [s for s in seqs if need is None or need[s]]
            self._extend(prefix, want)
            r = prefix.shape[1]
            am = np.zeros(prefix.shape[0], dtype=np.int64)
            for s in want:
                am[s] = argmax_lowest(self.rows[s][r - 1])
            return am
        return fn

    def logits(self, ids, seqs):
        self._extend(ids, seqs)
        return np.stack([np.stack(self.rows[s][: ids.shape[1]]) for s in seqs])


def _sweep(case, ids, nts, o_logits=None, o_kc=None, o_vc=None):
    """GPU rounds (commit = 0) at each nt; returns {nt: (kv, out)} and checks
    row bits and written cache rows against the largest nt."""
    res = {}
    for nt in nts:
        kv, g = _gpu_round(case, ids[:, :nt], commit=0)
        if o_logits is not None:
            ok, nbad, mx = logits_close(g["logits"], o_logits[:, :nt])
            assert ok, (nt, nbad, mx)
        res[nt] = (kv, g)
    top = max(nts)
    gk_top, gv_top = [t.cpu().numpy() for t in tva.kv_from_library_layout(res[top][0].k,
                                                                           res[top][0].v)]
    for nt in nts:
        kv, g = res[nt]
        np.testing.assert_array_equal(g["logits"], res[top][1]["logits"][:, :nt])
        np.testing.assert_array_equal(g["argmax"], res[top][1]["argmax"][:, :nt])
        gk, gv = [t.cpu().numpy() for t in tva.kv_from_library_layout(kv.k, kv.v)]
        for s, l0 in enumerate(case.lens):
            np.testing.assert_array_equal(gk[:, s, l0:l0 + nt], gk_top[:, s, l0:l0 + nt])
            np.testing.assert_array_equal(gv[:, s, l0:l0 + nt], gv_top[:, s, l0:l0 + nt])
        np.testing.assert_array_equal(kv.len.cpu().numpy(), case.lens)   # commit = 0
    return res


def _decision_properties(ids, g):
    """accepted_len = first r with argmax_r != ids[r+1] (else d); emitted =
    argmax at that row."""
    S, nt = ids.shape
    for s in range(S):
        am = g["argmax"][s]
        a = 0
        while a < nt - 1 and am[a] == ids[s, a + 1]:
            a += 1
        assert g["accepted_len"][s] == a and g["emitted"][s] == am[a], (s, a)


def test_q7b_4l_sweep_nt_1_to_8():
    cfg = CONFIGS["q7b_4l"]
    case = Case(cfg.model, cfg.n_seq, cfg.ctx, kv_capacity(cfg, 8), cfg.seed)
    K, V = case.np_kv()
    ch = OracleChain(case.spec, case.wnp, K, V, case.lens)
    ids = chain_drafts(cfg, make_anchors(cfg), 8, ch.argmax_fn(range(cfg.n_seq)))
    o = ch.logits(ids, range(cfg.n_seq))
    res = _sweep(case, ids, list(range(1, 9)), o)
    kv, g = res[8]
    assert _check_greedy(o, ids, g) <= 2
    _check_cache_rows(case, kv, ch.kc, ch.vc, case.lens, 8)
    _decision_properties(ids, g)


class FullStack:
    """A whole workload on the GPU, with host copies of its canonical tensors
    and prefilled cache for the oracle."""

    def __init__(self, cfg, nt_max):
        self.cfg, self.spec = cfg, cfg.model
        say(f"{cfg.name}: generating weights")
        w = make_weights(cfg.model, cfg.seed, DEV)
        self.wnp = to_numpy_tensors(w)
        self.cap = kv_capacity(cfg, nt_max)
        self.model = tva.Model(cfg.model, w, max_pos=self.cap)
        del w
        torch.cuda.empty_cache()
        self.K, self.V, l0 = make_kv(cfg, self.cap, DEV)
        self.lens = np.asarray(l0, dtype=np.int32)
        say(f"{cfg.name}: model and cache ready")

    def kv(self):
        return tva.KVCache.from_logical(self.K, self.V, self.lens)

    def np_kv(self):
        return self.K.cpu().numpy(), self.V.cpu().numpy()

    def round(self, ids, commit=0):
        kv = self.kv()
        t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
        out = tva.verify_round(self.model, kv, t, commit=commit)
        torch.cuda.synchronize()
        return kv, {k: v.cpu().numpy() for k, v in out.items() if v is not None}


def _gpu_only_checks(wl, ids, nts):
    res = {}
    for nt in nts:
        res[nt] = wl.round(ids[:, :nt])
    top = max(nts)
    for nt in nts:
        g = res[nt][1]
        assert np.isfinite(g["logits"]).all()
        np.testing.assert_array_equal(g["logits"], res[top][1]["logits"][:, :nt])
        _decision_properties(ids[:, :nt], g)
    # commit moves len by a + 1 and leaves every other cache row untouched
    kv, out = wl.round(ids[:, :top], commit=1)
    np.testing.assert_array_equal(kv.len.cpu().numpy(), wl.lens + out["accepted_len"] + 1)
    gk, gv = tva.kv_from_library_layout(kv.k, kv.v)
    for s, l0 in enumerate(wl.lens):
        keep = torch.ones(wl.cap, dtype=torch.bool, device=DEV)
        keep[l0:l0 + top] = False
        assert torch.equal(gk[:, s][:, keep], wl.K[:, s][:, keep])
        assert torch.equal(gv[:, s][:, keep], wl.V[:, s][:, keep])
    return res


def _argmax_chain_gpu(wl, nt):
    """Drafts following the GPU's own argmax chain (input construction for
    the property checks only; no oracle value depends on them)."""
    def fn(prefix, need=None):
        t = torch.from_numpy(np.ascontiguousarray(prefix, dtype=np.int32)).to(DEV)
        out = tva.verify_round(wl.model, wl.kv(), t, commit=0, want_logits=False)
        return out["argmax"][:, -1].cpu().numpy()
    return chain_drafts(wl.cfg, make_anchors(wl.cfg), nt, fn)


def _in_block_rounding_widening(wl, K, V, ids, seqs, o):
    """Twice the oracle's own effect of rounding the in-block cache rows to
    fp16, per row: max over the row of |L(fp16 cache) - L(unrounded fp64
    cache)|, both computed by the oracle on the same inputs.  The fp16 code of
    an in-block k or v value is a rounding decision that the GPU takes on its
    fp32 value and the oracle on its fp64 value; where the exact value lies
    within the kernel's rounding error of a boundary both neighbouring codes
    are correct, and the rows that read such a code move by at most the
    effect of the rounding itself.  No GPU value enters this bound."""
    ch64 = OracleChain(wl.spec, wl.wnp, K.astype(np.float64), V.astype(np.float64), wl.lens)
    o64 = ch64.logits(ids, seqs)
    return 2.0 * np.abs(o - o64).max(axis=-1, keepdims=True), ch64


def _full_depth_parity(wl, ids, o, ch, seqs, nts, widen, ch64):
    """Every logit of the sequences `seqs` at each nt against the oracle at
    the bar 1e-4 + 1e-3 |o|, widened per row by the in-block rounding bound
    (both the plain and the widened counts are reported); row bits across
    nt; decisions on clear rows; the cache rows written in every layer, at
    one fp16 rounding plus 1e-4 of the row's RMS, widened per (layer,
    position, head) row by twice the largest difference between the
    oracle's own rounded and unrounded runs over that row (layer 0, which
    no in-block rounding reaches, keeps the plain bar)."""
    res = {}
    base = 1e-4 + 1e-3 * np.abs(o)
    say(f"{wl.cfg.name}: in-block rounding widening per row: median {np.median(widen):.3g}, "
        f"max {widen.max():.3g} (base bar median {np.median(base):.3g}, min {base.min():.3g})")
    for nt in nts:
        kv, g = wl.round(ids[:, :nt])
        gl = g["logits"][seqs].astype(np.float64)
        err = np.abs(gl - o[:, :nt])
        plain = err > base[:, :nt]
        bad = err > base[:, :nt] + widen[:, :nt]
        say(f"{wl.cfg.name} nt={nt}: worst |g - o| {err.max():.3g}, worst fraction of the "
            f"plain bar {(err / base[:, :nt]).max():.3f}; {int(plain.sum())} of {err.size} logits "
            f"outside the plain bar, {int(bad.sum())} outside the widened bar")
        assert not bad.any(), (nt, int(bad.sum()), float(err.max()))
        res[nt] = (kv, g)
    top = max(nts)
    for nt in nts:
        np.testing.assert_array_equal(res[nt][1]["logits"], res[top][1]["logits"][:, :nt])
    kv, g = res[top]
    sub = {k: v[seqs] for k, v in g.items() if k in ("argmax", "accepted_len", "emitted")}
    excluded = _check_greedy(o, ids[seqs, :top], sub)
    say(f"{wl.cfg.name}: {excluded} rows within the 1e-2 top-2 margin (excluded); "
        f"accepted_len {sub['accepted_len'].tolist()}, emitted {sub['emitted'].tolist()}")
    gk, gv = [t.cpu().numpy() for t in tva.kv_from_library_layout(kv.k, kv.v)]
    for i, s in enumerate(seqs):
        new = slice(int(wl.lens[s]), int(wl.lens[s]) + top)
        for nm, g_, o_, u_ in (("k", gk, ch.kc, ch64.kc), ("v", gv, ch.vc, ch64.vc)):
            a = g_[:, s, new].astype(np.float64)
            b = o_[:, s, new].astype(np.float64)
            w = 2.0 * np.abs(b - u_[:, s, new]).max(axis=-1, keepdims=True)
            w[0] = 0.0
            rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
            plain = np.abs(b) * 2 ** -10 + 1e-4 * rms + 1e-7
            r = np.abs(a - b) / (plain + w)
            say(f"{wl.cfg.name} seq {s} {nm} rows: {int((np.abs(a - b) > plain).sum())} of "
                f"{a.size} values outside the plain bar (layer 0: "
                f"{int((np.abs(a - b) > plain)[0].sum())}), worst fraction of the widened "
                f"bar {r.max():.3f}")
            assert r.max() <= 1.0, f"{nm} seq {s}: worst {r.max():.3g}"
    return res


@pytest.fixture(scope="module")
def q14b_48l():
    cfg = CONFIGS["q14b_48l"]
    return FullStack(cfg, 9)


@pytest.mark.timeout(1500)
def test_q14b_48l_nt9_against_oracle_at_full_depth(q14b_48l):
    wl = q14b_48l
    K, V = wl.np_kv()
    ch = OracleChain(wl.spec, wl.wnp, K, V, wl.lens)
    say("q14b_48l: oracle draft chain")
    ids = chain_drafts(wl.cfg, make_anchors(wl.cfg), 9, ch.argmax_fn([0]))
    say(f"q14b_48l: ids {ids.tolist()}; oracle rows through 48 layers")
    o = ch.logits(ids, [0])
    say("q14b_48l: oracle rows with unrounded in-block cache rows")
    widen, ch64 = _in_block_rounding_widening(wl, K, V, ids, [0], o)
    _full_depth_parity(wl, ids, o, ch, [0], [1, 3, 9], widen, ch64)


@pytest.mark.timeout(900)
def test_q14b_48l_full_depth_properties(q14b_48l):
    ids = _argmax_chain_gpu(q14b_48l, 9)
    _gpu_only_checks(q14b_48l, ids, [1, 3, 9])


@pytest.mark.timeout(900)
def test_block16_shapes_1_layer_against_oracle():
    """Random ids make every in-block key matter.  The fp16 code of an
    in-block k or v value is a rounding decision: the GPU rounds its fp32
    value, the oracle its fp64 value, and where the two straddle a rounding
    boundary both neighbouring codes are correct to the kernel's precision.
    Rows reading such codes move by up to the effect of in-block rounding
    itself, so each row's logits bar is widened by twice the oracle's own
    measured effect of rounding the in-block rows (fp16 cache against an
    unrounded fp64 cache), a quantity that involves no GPU value.  The GPU
    runs all 12 sequences; three of them are compared with the oracle."""
    cfg = CONFIGS["q14b_8l_block16"]
    spec = replace(cfg.model, n_layer=1)
    case = Case(spec, cfg.n_seq, cfg.ctx, kv_capacity(cfg, 16), cfg.seed)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, spec.vocab, size=(cfg.n_seq, 16)).astype(np.int32)
    seqs = [0, 5, 11]
    om = OracleModel(spec, case.wnp, cache_weights=False)
    kc, vc = (a[:, seqs].copy() for a in case.np_kv())
    o = om.verify_logits(ids[seqs], case.lens[seqs], kc, vc)
    k64, v64 = (a[:, seqs].astype(np.float64) for a in case.np_kv())
    o64 = om.verify_logits(ids[seqs], case.lens[seqs], k64, v64)
    widen = 2.0 * np.abs(o - o64).max(axis=-1, keepdims=True)       # per row
    base = 1e-4 + 1e-3 * np.abs(o)
    say(f"block16 1 layer: widening per row median {np.median(widen):.3g}, max "
        f"{widen.max():.3g}; base bar median {np.median(base):.3g}, min {base.min():.3g}")
    res = _sweep(case, ids, [1, 16])
    kv, g = res[16]
    for nt in (1, 16):
        gl = res[nt][1]["logits"][seqs].astype(np.float64)
        err = np.abs(gl - o[:, :nt])
        plain = int((err > base[:, :nt]).sum())
        bad = err > base[:, :nt] + widen[:, :nt]
        say(f"block16 1 layer nt={nt}: {plain} of {err.size} logits outside the plain bar, "
            f"{int(bad.sum())} outside the widened bar")
        assert not bad.any(), (nt, int(bad.sum()), float(err.max()), float(widen.max()))
    sub = {k: g[k][seqs] for k in ("argmax", "accepted_len", "emitted")}
    assert _check_greedy(o, ids[seqs], sub) <= len(seqs) * 2
    gk, gv = [t.cpu().numpy() for t in tva.kv_from_library_layout(kv.k, kv.v)]
    for i, s in enumerate(seqs):
        new = slice(int(case.lens[s]), int(case.lens[s]) + 16)
        for g_, o_ in ((gk, kc), (gv, vc)):
            a = g_[:, s, new].astype(np.float64)
            b = o_[:, i, new].astype(np.float64)
            rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
            assert (np.abs(a - b) <= np.abs(b) * 2 ** -10 + 1e-4 * rms + 1e-7).all(), s


@pytest.fixture(scope="module")
def block16():
    return FullStack(CONFIGS["q14b_8l_block16"], 16)


# the two sequences compared with the oracle (their seeded chains miss at
# depths 0 and 1, so the chain needs two passes before the last)
BLOCK16_ORACLE_SEQS = [8, 9]


@pytest.mark.timeout(900)
def test_q14b_8l_block16_nt16_against_oracle_at_full_depth(block16):
    wl = block16
    K, V = wl.np_kv()
    ch = OracleChain(wl.spec, wl.wnp, K, V, wl.lens)
    seqs = BLOCK16_ORACLE_SEQS
    say("block16: oracle draft chain for sequences %s" % seqs)
    ids = chain_drafts(wl.cfg, make_anchors(wl.cfg), 16, ch.argmax_fn(seqs))
    rng = np.random.default_rng(16)
    for s in range(wl.cfg.n_seq):
        if s not in seqs:
            ids[s, 1:] = rng.integers(0, wl.spec.vocab, 15)
    say("block16: oracle rows through 8 layers")
    o = ch.logits(ids, seqs)
    say("block16: oracle rows with unrounded in-block cache rows")
    widen, ch64 = _in_block_rounding_widening(wl, K, V, ids, seqs, o)
    _full_depth_parity(wl, ids, o, ch, seqs, [1, 16], widen, ch64)


@pytest.mark.timeout(900)
def test_q14b_8l_block16_full_depth_properties(block16):
    ids = _argmax_chain_gpu(block16, 16)
    _gpu_only_checks(block16, ids, [1, 16])
