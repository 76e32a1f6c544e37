"""The fused layer kernel (one launch per decoder layer for rounds of at most
16 rows) against the separate kernels, on the GPU.

The fused launch runs the same device functions with the same work
decomposition as the separate kernels, so every output must be identical
bit for bit: logits, row argmaxes, accepted lengths, emitted tokens, every
cache row and the committed lengths.  SV_FUSED_LAYER=1 selects the fused
launch (off by default), SV_FUSED_LAYER=0 the separate kernels.  Cases:
two-layer GQA models with 128-dim heads over several row counts (packed
rows up to 8, two-part rows up to 16, one to four query tiles per kv head),
two sequences at different lengths, ragged rounds, a capacity overflow and
a NaN token row failing one sequence, the 14B layer shapes at nt = 3 and 9,
and several committed rounds in a row.
"""

import os
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from dataclasses import replace
from synth.configs import CONFIGS, ModelSpec
from synth.make import kv_capacity
from tests.test_gpu_round import Case

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(out):
    return {k: v.cpu().numpy() for k, v in out.items() if v is not None}


def _pair(case, ids, commit=0, lens=None, nts=None, model=None, rounds=1, max_len=0):
    """The same round(s) through the fused and the separate kernels."""
    model = model or case.model
    res = []
    for fused in (True, False):
        os.environ["SV_FUSED_LAYER"] = "1" if fused else "0"
        try:
            kv = tva.KVCache.from_logical(case.K, case.V, case.lens if lens is None else lens)
            outs = []
            cur = np.ascontiguousarray(ids, dtype=np.int32)
            for _ in range(rounds):
                t = torch.from_numpy(cur).to(DEV)
                n = torch.from_numpy(np.asarray(nts, dtype=np.int32)).to(DEV) if nts is not None else None
                o = _np(tva.verify_round(model, kv, t, commit=commit, nts=n, max_len=max_len))
                outs.append(o)
                cur = np.roll(cur, 1, axis=1)
                cur[:, 0] = np.maximum(o["emitted"], 0)
            torch.cuda.synchronize()
            gk, gv = tva.kv_from_library_layout(kv.k, kv.v)
            res.append((outs, gk.cpu().numpy(), gv.cpu().numpy(), kv.len.cpu().numpy()))
        finally:
            os.environ.pop("SV_FUSED_LAYER", None)
    (fo, fk, fv, fl), (so, sk, sv, sl) = res
    for a, b in zip(fo, so):
        assert a.keys() == b.keys()
        np.testing.assert_array_equal(a["accepted_len"], b["accepted_len"])
        np.testing.assert_array_equal(a["emitted"], b["emitted"])
        # a failed sequence's rows are not computed: its logits are undefined
        live = a["accepted_len"] >= 0
        for k in ("logits", "argmax"):
            np.testing.assert_array_equal(a[k][live], b[k][live], err_msg=k)
    np.testing.assert_array_equal(fk, sk)
    np.testing.assert_array_equal(fv, sv)
    np.testing.assert_array_equal(fl, sl)
    return fo


MINI = ModelSpec(n_layer=2, hidden=512, n_head=8, n_kv_head=2, head_dim=128, ffn=1024,
                 vocab=2048, fmt_proj="b4_256", fmt_lm="b6_256")


@pytest.fixture(scope="module")
def mini():
    return Case(MINI, 2, 300, 512, seed=78, lens=[300, 171])


@pytest.mark.parametrize("S,nt", [(1, 1), (1, 3), (1, 8), (2, 4), (1, 9), (1, 16), (2, 8)])
def test_fused_layer_equals_separate_kernels(mini, S, nt):
    print(f"[fused] mini S={S} nt={nt}", flush=True)
    rng = np.random.default_rng(100 + 16 * S + nt)
    ids = rng.integers(0, MINI.vocab, size=(2, nt)).astype(np.int32)
    if S == 1:
        one = SimpleNamespace(K=mini.K[:, :1].contiguous(), V=mini.V[:, :1].contiguous(),
                              lens=mini.lens[:1], model=mini.model)
        out = _pair(one, ids[:1])
    else:
        out = _pair(mini, ids)
    assert all((o["accepted_len"] >= 0).all() for o in out)


def test_fused_layer_ragged_and_committed_rounds(mini):
    print("[fused] mini ragged, three committed rounds", flush=True)
    rng = np.random.default_rng(7)
    ids = rng.integers(0, MINI.vocab, size=(2, 6)).astype(np.int32)
    _pair(mini, ids, commit=1, nts=[6, 2], rounds=3)


def test_fused_layer_with_a_length_bound(mini):
    """The fused launch visits the chunks below max_len + nt like the
    separate kernels (three committed rounds, the bound covering them)."""
    print("[fused] mini with max_len", flush=True)
    rng = np.random.default_rng(9)
    ids = rng.integers(0, MINI.vocab, size=(2, 5)).astype(np.int32)
    _pair(mini, ids, commit=1, rounds=3, max_len=300 + 2 * 5)


def test_fused_layer_failed_sequences(mini):
    print("[fused] mini capacity overflow and NaN row", flush=True)
    rng = np.random.default_rng(8)
    ids = rng.integers(0, MINI.vocab, size=(2, 5)).astype(np.int32)
    out = _pair(mini, ids, commit=1, lens=np.array([300, 510], dtype=np.int32))
    assert out[0]["accepted_len"][1] == tva.SV_E_CAPACITY and out[0]["accepted_len"][0] >= 0
    tok = mini.w["tok_embd"].clone()
    tok[int(ids[0, 2]), 3] = float("nan")
    model = tva.Model(MINI, dict(mini.w, tok_embd=tok), max_pos=512)
    out = _pair(mini, ids, commit=1, model=model)
    assert out[0]["accepted_len"][0] == tva.SV_E_NUMERIC and out[0]["accepted_len"][1] >= 0


@pytest.mark.parametrize("nt", [3, 9])
def test_fused_layer_14b_shapes(nt):
    print(f"[fused] 14B shapes, 2 layers, nt={nt}", flush=True)
    cfg = CONFIGS["q14b_48l"]
    spec = replace(cfg.model, n_layer=2)
    case = Case(spec, 1, cfg.ctx, kv_capacity(cfg, 9), cfg.seed)
    rng = np.random.default_rng(nt)
    ids = rng.integers(0, spec.vocab, size=(1, nt)).astype(np.int32)
    _pair(case, ids)
