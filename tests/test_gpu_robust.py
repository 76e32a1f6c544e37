"""Fail-closed numerics, exact greedy ties and replay determinism on the GPU.

* Non-finite logits fail the sequence closed (the Power page, "Capabilities
  fail closed"; the oracle refuses a NaN row): a NaN hidden row in an
  lm_head-only round, NaN draft logits in SV_REJECT, and a NaN row of the
  token table in a full model each give that sequence SV_E_NUMERIC with no
  emitted token and no commit, in all three modes, while the other
  sequences of the batch get exactly the results of a round without the
  NaN.
* Greedy ties are broken toward the lowest id: an integer-exact lm_head
  (d = 1, scale 1, so every weight is an integer and every logit of an
  integer hidden row is an exact integer) with several identical maximal
  rows, inside one 32-column group and across groups, through both GEMM
  kernels (4 rows, and 192 rows on the wide-row kernel).
* A round captured in a HIP graph and replayed several times, with eager
  rounds and host synchronizations in between, gives the eager round's
  bits on every replay.
"""

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from synth.configs import CONFIGS, Config, ModelSpec
from synth.make import make_hidden, make_weights
from synth.rng import round_uniforms, sample_uniforms
from tests.gpu_util import pack_b6_256
from tests.test_gpu_round import Case

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = 0.8


def _np(out):
    return {k: v.cpu().numpy() for k, v in out.items() if v is not None}


def _lm_model(vocab=8192, hidden=512, seed=505):
    spec = ModelSpec(n_layer=0, hidden=hidden, n_head=8, n_kv_head=8, head_dim=64, ffn=1536,
                     vocab=vocab, fmt_proj="b4_256", fmt_lm="b6_256", lm_only=True)
    cfg = Config(name="lm_robust", seed=seed, model=spec, n_seq=3, nt=(4,), ctx=0,
                 mode="sample", temperature=T)
    w = make_weights(spec, seed, DEV)
    return cfg, tva.Model(spec, w, max_pos=128)


@pytest.mark.parametrize("mode", [tva.SV_GREEDY, tva.SV_REJECT, tva.SV_SAMPLE])
def test_nan_hidden_row_fails_closed(mode):
    cfg, model = _lm_model()
    S, nt, V = 3, 4, cfg.model.vocab
    hidden = make_hidden(cfg, nt, DEV)
    bad = hidden.clone()
    bad[1, 2, 17] = float("nan")                 # one value of one row of sequence 1
    rng = np.random.default_rng(4)
    ids = torch.from_numpy(rng.integers(0, V, (S, nt)).astype(np.int32)).to(DEV)
    kw = dict(mode=mode, want_logits=True, commit=0)
    if mode != tva.SV_GREEDY:
        kw["temperature"] = T
        u = (round_uniforms if mode == tva.SV_REJECT else sample_uniforms)(
            cfg.seed, np.zeros(S, np.int64), nt)
        kw["uniforms"] = torch.from_numpy(u).to(DEV)
    if mode == tva.SV_REJECT:
        kw["draft_logits"] = torch.from_numpy(
            rng.normal(size=(S, nt - 1, V)).astype(np.float32)).to(DEV)
    ref = _np(tva.verify_round(model, None, ids, hidden=hidden, **kw))
    got = _np(tva.verify_round(model, None, ids, hidden=bad, **kw))
    torch.cuda.synchronize()
    assert got["accepted_len"][1] == tva.SV_E_NUMERIC and got["emitted"][1] == -1
    for s in (0, 2):
        assert got["accepted_len"][s] == ref["accepted_len"][s] >= 0
        assert got["emitted"][s] == ref["emitted"][s]
        np.testing.assert_array_equal(got["logits"][s], ref["logits"][s])
    if mode == tva.SV_REJECT:
        dl = kw["draft_logits"].clone()
        dl[2, 0, 5] = float("inf")
        got = _np(tva.verify_round(model, None, ids, hidden=hidden, **dict(kw, draft_logits=dl)))
        assert got["accepted_len"][2] == tva.SV_E_NUMERIC and got["emitted"][2] == -1
        assert got["accepted_len"][0] == ref["accepted_len"][0]


def test_nan_token_row_fails_closed_without_commit():
    cfg = CONFIGS["tiny"]
    case = Case(cfg.model, 2, cfg.ctx, 128, cfg.seed)
    tok = case.w["tok_embd"].clone()
    tok[123, 5] = float("nan")
    w = dict(case.w, tok_embd=tok)
    model = tva.Model(cfg.model, w, max_pos=128)
    ids = np.array([[7, 8, 9], [10, 123, 11]], dtype=np.int32)    # sequence 1 reads row 123
    kv = case.kv()
    out = _np(tva.verify_round(model, kv, torch.from_numpy(ids).to(DEV), commit=1))
    torch.cuda.synchronize()
    assert out["accepted_len"][1] == tva.SV_E_NUMERIC and out["emitted"][1] == -1
    lens = kv.len.cpu().numpy()
    assert lens[1] == case.lens[1]                                 # not committed
    assert out["accepted_len"][0] >= 0
    assert lens[0] == case.lens[0] + out["accepted_len"][0] + 1
    kv1 = tva.KVCache.from_logical(case.K[:, :1], case.V[:, :1], case.lens[:1])
    ref = _np(tva.verify_round(case.model, kv1, torch.from_numpy(ids[:1].copy()).to(DEV),
                               commit=0))
    np.testing.assert_array_equal(out["logits"][0], ref["logits"][0])


def _tie_head(H, V, rng):
    """Integer-exact 6-bit lm_head (d = 1, every sub-block scale 1, codes
    16..47: weights -16..15) with two integer hidden rows h0, h1 and rows
    whose weights are sign(h) * 31 / -32 (the maximal dot product with h):
    rows 100, 101, 4000 and V - 1 for h0; rows 200 and 5000 for h1."""
    nsb = H // 256
    q = rng.integers(16, 48, size=(V, nsb, 256))
    h = rng.integers(-3, 4, size=(2, H)).astype(np.float32)
    h[h == 0] = 1.0
    for row_h, rows in ((h[0], (100, 101, 4000, V - 1)), (h[1], (200, 5000))):
        codes = np.where(row_h > 0, 63, 0).reshape(nsb, 256)      # weights +31 / -32
        for r in rows:
            q[r] = codes
    d = np.ones((V, nsb))
    sc = np.ones((V, nsb, 16), dtype=np.int8)
    return pack_b6_256(d, sc, q), h


@pytest.mark.parametrize("S,nt", [(1, 4), (12, 16)])
def test_greedy_exact_ties_take_the_lowest_id(S, nt):
    H, V = 512, 8192
    rng = np.random.default_rng(31)
    raw, h = _tie_head(H, V, rng)
    spec = ModelSpec(n_layer=0, hidden=H, n_head=8, n_kv_head=8, head_dim=64, ffn=1536,
                     vocab=V, fmt_proj="b4_256", fmt_lm="b6_256", lm_only=True)
    model = tva.Model(spec, {"lm_head": torch.from_numpy(raw).to(DEV)}, max_pos=128)
    hid = np.stack([h[(s * nt + r) % 2] for s in range(S) for r in range(nt)]).reshape(S, nt, H)
    ids = np.zeros((S, nt), dtype=np.int32)
    for s in range(S):
        for r in range(1, nt):
            ids[s, r] = 100 if (s * nt + r - 1) % 2 == 0 else 200   # the tied argmaxes
        if s % 3 == 1:
            ids[s, nt // 2] = 101                                    # a tied id, not the lowest
    out = _np(tva.verify_round(model, None, torch.from_numpy(ids).to(DEV),
                               hidden=torch.from_numpy(hid).to(DEV), want_logits=True,
                               commit=0))
    torch.cuda.synchronize()
    lg = out["logits"]
    for s in range(S):
        for r in range(nt):
            want = 100 if (s * nt + r) % 2 == 0 else 200
            ties = (100, 101, 4000, V - 1) if want == 100 else (200, 5000)
            assert len({float(lg[s, r, t]) for t in ties}) == 1       # exact ties
            assert lg[s, r].max() == lg[s, r, want]
            assert out["argmax"][s, r] == want, (s, r, out["argmax"][s, r])
        a = nt - 1 if s % 3 != 1 else nt // 2 - 1
        assert out["accepted_len"][s] == a, (s, out["accepted_len"][s])
        assert out["emitted"][s] == (100 if (s * nt + a) % 2 == 0 else 200)


def test_graph_replays_are_bit_identical():
    cfg = CONFIGS["tiny"]
    S, nt = 2, 4
    case = Case(cfg.model, S, cfg.ctx, 128, cfg.seed)
    rng = np.random.default_rng(12)
    ids = torch.from_numpy(rng.integers(0, cfg.model.vocab, (S, nt)).astype(np.int32)).to(DEV)
    kv = case.kv()
    ws = case.model.workspace(S, nt, tva.SV_GREEDY)
    outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device=DEV),
                emitted=torch.empty(S, dtype=torch.int32, device=DEV),
                argmax=torch.empty((S, nt), dtype=torch.int32, device=DEV),
                logits=torch.empty((S, nt, cfg.model.vocab), device=DEV))

    def step():
        tva.verify_round(case.model, kv, ids, commit=0, workspace=ws, outs=outs)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    other = torch.from_numpy(rng.integers(0, cfg.model.vocab, (S, nt)).astype(np.int32)).to(DEV)
    for i in range(5):
        for v in outs.values():
            v.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], eager[k]), (i, k)
        # eager work between replays: a different round on its own buffers
        tva.verify_round(case.model, case.kv(), other, commit=0)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(kv.len.cpu().numpy(), case.lens)


def test_attention_slot_region_bound():
    """The chunk results of one (sequence, kv head) are addressed with 32-bit
    offsets from their own base, so a round whose region would reach 2^31
    bytes fails closed with SV_E_UNSUPPORTED before anything is enqueued,
    and one just under the bound runs.  Region bytes = capacity / 128 * 16 *
    ceil(nt * G / 16) * head_dim * 4; here G = 8, head_dim = 128 and the
    capacity 4793600 (region 448 B per position at nt = 13..14, 384 B at
    nt = 12).  The caches are allocated at the full capacity."""
    cap = 4793600
    assert cap % 128 == 0 and cap * 448 >= 2 ** 31 > cap * 384
    spec = ModelSpec(n_layer=1, hidden=256, n_head=8, n_kv_head=1, head_dim=128, ffn=256,
                     vocab=256, fmt_proj="b4_256", fmt_lm="b6_256")
    w = make_weights(spec, 606, DEV)
    model = tva.Model(spec, w, max_pos=cap)
    k = torch.zeros((1, 1, 1, cap, 128), dtype=torch.float16, device=DEV)
    v = torch.zeros((1, 1, 1, 128, cap), dtype=torch.float16, device=DEV)
    lens = torch.tensor([40], dtype=torch.int32, device=DEV)
    kv = tva.KVCache(k, v, lens)
    for nt in (14, 13):
        ids = torch.zeros((1, nt), dtype=torch.int32, device=DEV)
        with pytest.raises(tva.SvError) as e:
            tva.verify_round(model, kv, ids, commit=0)
        assert e.value.status == tva.SV_E_UNSUPPORTED, nt
    ids = torch.arange(12, dtype=torch.int32, device=DEV)[None]
    out = _np(tva.verify_round(model, kv, ids, commit=0))
    torch.cuda.synchronize()
    assert 0 <= out["accepted_len"][0] <= 11 and np.isfinite(out["logits"]).all()
