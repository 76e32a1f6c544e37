"""Greedy verify rounds at the workloads' full shapes on the GPU.

* q7b_4l (4 layers of the 7B shape, vocabulary 152064, context 2048): the
  oracle builds the draft chain row by row (acceptance 0.69, uniform after
  the first miss) and supplies every row's logits; the GPU runs nt = 1..8
  with commit = 0.  Logits at the 1e-3 / 1e-4 bar, greedy decision on clear
  rows, cache rows written, and the GPU's own row bits identical at every nt.
* The 14B layer shapes (hidden 5120, 40q/8kv x 128, FFN 13824) at context
  4096 and vocabulary 152064, 2 layers, nt = 9 against the oracle; and the
  full 48-layer stack at nt = 1, 3, 9 through properties that hold at any
  depth: identical row bits across nt, the decision equal to the first
  mismatch of the GPU's own argmax, the commit, untouched cache rows.
* The batch-12 block verify shapes (vocabulary 248320, context 512, nt = 16):
  1 layer against the oracle, and the full 8 layers through the same
  properties at nt = 16 against nt = 1.
"""

import numpy as np
import pytest
import torch
from dataclasses import replace

import target_verification_amd as tva
from oracle.model import rmsnorm
from synth.configs import CONFIGS
from synth.make import chain_drafts, kv_capacity, make_anchors, make_kv, make_weights
from tests.gpu_util import logits_close
from tests.test_gpu_round import Case, _check_cache_rows, _check_greedy, _gpu_round

pytestmark = pytest.mark.gpu
DEV = "cuda"


class OracleChain:
    """Oracle logits of rows 0..r-1 for a growing id prefix; each row is
    computed once (its cache rows are written into the oracle's copy)."""

    def __init__(self, case):
        self.case = case
        self.kc, self.vc = case.np_kv()
        self.case.oracle.weight("lm_head")       # decode the lm_head once
        self.rows = None

    def _extend(self, ids):
        c = self.case
        S, r = ids.shape
        if self.rows is None:
            self.rows = [[] for _ in range(S)]
        for s in range(S):
            while len(self.rows[s]) < r:
                k = len(self.rows[s])
                x = c.oracle.hidden_row(int(ids[s, k]), int(c.lens[s]) + k, s, self.kc, self.vc)
                fin = rmsnorm(x, c.wnp["out_norm"], c.spec.rms_eps)
                self.rows[s].append(c.oracle.logits_rows(fin[None])[0])

    def argmax_fn(self, prefix):
        self._extend(prefix)
        r = prefix.shape[1]
        return np.array([int(np.argmax(self.rows[s][r - 1])) for s in range(prefix.shape[0])])

    def logits(self, ids):
        self._extend(ids)
        return np.stack([np.stack(self.rows[s][: ids.shape[1]]) for s in range(ids.shape[0])])


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
    ch = OracleChain(case)
    ids = chain_drafts(cfg, make_anchors(cfg), 8, ch.argmax_fn)
    o = ch.logits(ids)
    res = _sweep(case, ids, list(range(1, 9)), o)
    kv, g = res[8]
    assert _check_greedy(o, ids, g) <= 2
    _check_cache_rows(case, kv, ch.kc, ch.vc, case.lens, 8)
    _decision_properties(ids, g)


def test_q14b_shapes_2_layers_against_oracle():
    cfg = CONFIGS["q14b_48l"]
    spec = replace(cfg.model, n_layer=2)
    case = Case(spec, 1, cfg.ctx, kv_capacity(cfg, 9), cfg.seed)
    ch = OracleChain(case)
    ids = chain_drafts(cfg, make_anchors(cfg), 9, ch.argmax_fn)
    o = ch.logits(ids)
    res = _sweep(case, ids, [1, 3, 9], o)
    kv, g = res[9]
    assert _check_greedy(o, ids, g) <= 2
    _check_cache_rows(case, kv, ch.kc, ch.vc, case.lens, 9)


class GpuOnly:
    """A workload on the GPU without the oracle (full depth)."""

    def __init__(self, cfg, nt_max):
        self.spec = cfg.model
        w = make_weights(cfg.model, cfg.seed, DEV)
        self.cap = kv_capacity(cfg, nt_max)
        self.model = tva.Model(cfg.model, w, max_pos=self.cap)
        del w
        self.K, self.V, l0 = make_kv(cfg, self.cap, DEV)
        self.lens = np.asarray(l0, dtype=np.int32)

    def kv(self):
        return tva.KVCache.from_logical(self.K, self.V, self.lens)


def _gpu_only_checks(wl, ids, nts):
    res = {}
    for nt in nts:
        kv = wl.kv()
        t = torch.from_numpy(np.ascontiguousarray(ids[:, :nt], dtype=np.int32)).to(DEV)
        out = tva.verify_round(wl.model, kv, t, commit=0)
        torch.cuda.synchronize()
        res[nt] = (kv, {k: v.cpu().numpy() for k, v in out.items() if v is not None})
    top = max(nts)
    for nt in nts:
        g = res[nt][1]
        assert np.isfinite(g["logits"]).all()
        np.testing.assert_array_equal(g["logits"], res[top][1]["logits"][:, :nt])
        _decision_properties(ids[:, :nt], g)
    # commit moves len by a + 1 and leaves every other cache row untouched
    kv = wl.kv()
    t = torch.from_numpy(np.ascontiguousarray(ids[:, :top], dtype=np.int32)).to(DEV)
    out = tva.verify_round(wl.model, kv, t, commit=1)
    torch.cuda.synchronize()
    a = out["accepted_len"].cpu().numpy()
    np.testing.assert_array_equal(kv.len.cpu().numpy(), wl.lens + a + 1)
    gk, gv = tva.kv_from_library_layout(kv.k, kv.v)
    for s, l0 in enumerate(wl.lens):
        keep = torch.ones(wl.cap, dtype=torch.bool, device=DEV)
        keep[l0:l0 + top] = False
        assert torch.equal(gk[:, s][:, keep], wl.K[:, s][:, keep])
        assert torch.equal(gv[:, s][:, keep], wl.V[:, s][:, keep])
    return res


def _argmax_chain_gpu(wl, cfg, nt):
    """Drafts following the GPU's own argmax chain (input construction for
    the property checks only; no oracle value depends on them)."""
    def fn(prefix):
        t = torch.from_numpy(np.ascontiguousarray(prefix, dtype=np.int32)).to(DEV)
        out = tva.verify_round(wl.model, wl.kv(), t, commit=0, want_logits=False)
        return out["argmax"][:, -1].cpu().numpy()
    return chain_drafts(cfg, make_anchors(cfg), nt, fn)


def test_q14b_48l_full_depth_properties():
    cfg = CONFIGS["q14b_48l"]
    wl = GpuOnly(cfg, 9)
    ids = _argmax_chain_gpu(wl, cfg, 9)
    _gpu_only_checks(wl, ids, [1, 3, 9])


def test_block16_shapes_1_layer_against_oracle():
    """Random ids make every in-block key matter.  The fp16 code of an
    in-block k or v value is a rounding decision: the GPU rounds its fp32
    value, the oracle its fp64 value, and where the two straddle a rounding
    boundary both neighbouring codes are correct to the kernel's precision.
    Rows reading such codes move by up to the effect of in-block rounding
    itself, so each row's logits bar is widened by twice the oracle's own
    measured effect of rounding the in-block rows (fp16 cache against an
    unrounded fp64 cache), a quantity that involves no GPU value."""
    cfg = CONFIGS["q14b_8l_block16"]
    spec = replace(cfg.model, n_layer=1)
    case = Case(spec, cfg.n_seq, cfg.ctx, kv_capacity(cfg, 16), cfg.seed)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, spec.vocab, size=(cfg.n_seq, 16)).astype(np.int32)
    case.oracle.weight("lm_head")
    kc, vc = case.np_kv()
    o = case.oracle.verify_logits(ids, case.lens, kc, vc)
    k64, v64 = (a.astype(np.float64) for a in case.np_kv())
    o64 = case.oracle.verify_logits(ids, case.lens, k64, v64)
    widen = 2.0 * np.abs(o - o64).max(axis=-1, keepdims=True)       # per row
    res = _sweep(case, ids, [1, 16])
    kv, g = res[16]
    for nt in (1, 16):
        gl = res[nt][1]["logits"].astype(np.float64)
        err = np.abs(gl - o[:, :nt])
        bad = err > 1e-4 + 1e-3 * np.abs(o[:, :nt]) + widen[:, :nt]
        assert not bad.any(), (nt, int(bad.sum()), float(err.max()), float(widen.max()))
    assert _check_greedy(o, ids, g) <= cfg.n_seq * 2
    _check_cache_rows(case, kv, kc, vc, case.lens, 16)


def test_q14b_8l_block16_full_depth_properties():
    cfg = CONFIGS["q14b_8l_block16"]
    wl = GpuOnly(cfg, 16)
    ids = _argmax_chain_gpu(wl, cfg, 16)
    _gpu_only_checks(wl, ids, [1, 16])
