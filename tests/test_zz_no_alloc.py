"""spec_verify_round_static (the entry point for callers that cannot
allocate) against spec_verify_round on the GPU.

Both run the same kernels, so every output must be identical bit for bit:
logits, row argmaxes or draws, accepted lengths, emitted tokens, the
committed lengths and every cache row.  Each case makes two calls in a row
on the library's scratch array, the second with a smaller input, so the
second reads nothing the first left behind:

* greedy rounds of a full model (one decoder layer, hidden 512, vocabulary
  4096): 3 sequences x 8 rows, committed, then 1 sequence x 3 rows;
* exact-match sampled rounds of an lm_head-only model (vocabulary 8192):
  6 sequences x 8 rows with the logits kept in the scratch, then 2 x 3
  rows with caller-provided logits;
* a round whose workspace exceeds the scratch (vocabulary 131072, 12 x 16
  rows, logits in the scratch) fails closed with SV_E_UNSUPPORTED, and the
  same round with caller-provided logits fits and matches.
"""

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from synth.configs import CONFIGS, Config, ModelSpec
from synth.make import make_hidden, make_weights
from synth.rng import sample_uniforms
from tests.test_gpu_round import Case

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(out):
    return {k: v.cpu().numpy() for k, v in out.items() if v is not None}


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_static_greedy_rounds_equal_workspace_rounds():
    cfg = CONFIGS["tiny"]
    S = 3
    case = Case(cfg.model, S, cfg.ctx, 256, cfg.seed, lens=[64, 100, 17])
    rng = np.random.default_rng(70)
    for n_seq, nt in ((3, 8), (1, 3)):
        ids = torch.from_numpy(rng.integers(0, cfg.model.vocab, (n_seq, nt))
                               .astype(np.int32)).to(DEV)
        K, V = case.K[:, :n_seq].contiguous(), case.V[:, :n_seq].contiguous()
        lens = case.lens[:n_seq]
        kv_s = tva.KVCache.from_logical(K, V, lens)
        kv_r = tva.KVCache.from_logical(K, V, lens)
        got = _np(tva.verify_round(case.model, kv_s, ids, commit=1, static_scratch=True))
        want = _np(tva.verify_round(case.model, kv_r, ids, commit=1))
        torch.cuda.synchronize()
        _same(got, want)
        assert torch.equal(kv_s.len, kv_r.len)
        assert torch.equal(kv_s.k, kv_r.k) and torch.equal(kv_s.v, kv_r.v)
        np.testing.assert_array_equal(kv_s.len.cpu().numpy(), lens + got["accepted_len"] + 1)


def _lm(vocab, hidden, seed):
    spec = ModelSpec(n_layer=0, hidden=hidden, n_head=8, n_kv_head=8, head_dim=64, ffn=1536,
                     vocab=vocab, fmt_proj="b4_256", fmt_lm="b6_256", lm_only=True)
    w = make_weights(spec, seed, DEV)
    return spec, tva.Model(spec, w, max_pos=128)


def _sample_round(spec, model, S, nt, seed, static, want_logits):
    cfg = Config(name="lm_static", seed=seed, model=spec, n_seq=S, nt=(nt,), ctx=0,
                 mode="sample", temperature=0.8)
    hidden = make_hidden(cfg, nt, DEV)
    u = torch.from_numpy(sample_uniforms(seed, np.zeros(S, np.int64), nt)).to(DEV)
    rng = np.random.default_rng(seed)
    ids = torch.from_numpy(rng.integers(0, spec.vocab, (S, nt)).astype(np.int32)).to(DEV)
    out = tva.verify_round(model, None, ids, mode=tva.SV_SAMPLE, temperature=0.8, hidden=hidden,
                           uniforms=u, want_logits=want_logits, commit=0,
                           static_scratch=static)
    return _np(out)


def test_static_sampled_rounds_equal_workspace_rounds():
    spec, model = _lm(8192, 512, 808)
    for S, nt, want_logits in ((6, 8, False), (2, 3, True)):
        got = _sample_round(spec, model, S, nt, 90 + S, True, want_logits)
        want = _sample_round(spec, model, S, nt, 90 + S, False, want_logits)
        torch.cuda.synchronize()
        _same(got, want)


def test_static_scratch_limit_fails_closed():
    spec, model = _lm(131072, 256, 909)
    S, nt = 12, 16
    with pytest.raises(tva.SvError) as e:
        _sample_round(spec, model, S, nt, 5, True, False)
    assert e.value.status == tva.SV_E_UNSUPPORTED
    got = _sample_round(spec, model, S, nt, 5, True, True)
    want = _sample_round(spec, model, S, nt, 5, False, True)
    torch.cuda.synchronize()
    _same(got, want)
