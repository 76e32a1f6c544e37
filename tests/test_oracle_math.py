"""Pins of the oracle's dense math and of how the forward composes it.

Library routines (torch fp64 on CPU, independent of the oracle's numpy code):
RMSNorm, SiLU, scaled-dot-product attention.  Closed forms: RoPE on unit
vectors, RoPE identities (position 0, norm, relative position).  Structural
special cases of the whole forward, each reducing the model to a formula with
one term switched on (zeroed weights decode to exact zeros):
  * W_o = W_down = 0: logits = W_lm RMSNorm(E[id]; g_out);
  * W_down = 0 at position 0 (one key): attention returns v, so
    x = e + W_o [v_{j // G}]_j;
  * W_k = 0 (all keys 0, uniform weights): attention returns the mean of the
    cached values over keys 0..pos inclusive;
  * W_o = 0: x = e + W_d (silu(W_g h2) * (W_u h2));
  * the cache rows the forward writes equal fp16(RoPE(W_k h)) and fp16(W_v h).
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.formats import decode
from oracle.model import OracleModel, rmsnorm, rope, silu, attend, rope_angles
from tests.oracle_util import tiny_spec, tiny_tensors, random_kv, zero_tensor_like


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(300) * 3
    g = 1 + 0.1 * rng.standard_normal(300)
    want = F.rms_norm(torch.tensor(x), (300,), torch.tensor(g), eps=1e-6).numpy()
    np.testing.assert_allclose(rmsnorm(x, g, 1e-6), want, rtol=1e-14, atol=0)


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(silu(z), F.silu(torch.tensor(z)).numpy(), rtol=1e-14,
                               atol=1e-300)


def test_attend_matches_sdpa():
    rng = np.random.default_rng(1)
    for n in (1, 2, 17, 300):
        q = rng.standard_normal(64)
        K = rng.standard_normal((n, 64))
        V = rng.standard_normal((n, 64))
        want = F.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None], torch.tensor(K)[None, None],
            torch.tensor(V)[None, None])[0, 0, 0].numpy()
        np.testing.assert_allclose(attend(q, K, V), want, rtol=1e-12, atol=1e-14)


def test_attend_special_cases():
    rng = np.random.default_rng(2)
    V = rng.standard_normal((9, 8))
    q = rng.standard_normal(8)
    np.testing.assert_allclose(attend(q, np.ones((9, 8)), V), V.mean(0), rtol=1e-13)
    np.testing.assert_allclose(attend(q, V[:1], V[:1]), V[0], rtol=1e-15)


def test_rope_closed_form_and_pairing():
    base = 1.0e6
    for pos in (0, 1, 7, 4100):
        # hd = 4: pairs (0, 2) at theta_0 = pos and (1, 3) at pos * base^-1/2
        a0, a1 = float(pos), pos * base ** -0.5
        np.testing.assert_allclose(rope(np.array([[1.0, 0, 0, 0]]), pos, base)[0],
                                   [np.cos(a0), 0, np.sin(a0), 0], atol=1e-15)
        np.testing.assert_allclose(rope(np.array([[0, 1.0, 0, 0]]), pos, base)[0],
                                   [0, np.cos(a1), 0, np.sin(a1)], atol=1e-15)
        np.testing.assert_allclose(rope(np.array([[0, 0, 1.0, 0]]), pos, base)[0],
                                   [-np.sin(a0), 0, np.cos(a0), 0], atol=1e-15)
    np.testing.assert_allclose(rope_angles(3, 8, 1e6), 3 * 1e6 ** (-np.arange(4) / 4))


def test_rope_identities():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 128))
    k = rng.standard_normal((3, 128))
    np.testing.assert_array_equal(rope(q, 0, 1e6), q)
    r = rope(q, 1234, 1e6)
    np.testing.assert_allclose(np.hypot(r[:, :64], r[:, 64:]),
                               np.hypot(q[:, :64], q[:, 64:]), rtol=1e-13)
    d1 = np.sum(rope(q, 100, 1e6) * rope(k, 40, 1e6), -1)
    d2 = np.sum(rope(q, 3060, 1e6) * rope(k, 3000, 1e6), -1)
    np.testing.assert_allclose(d1, d2, rtol=1e-9)


# ---- structural special cases of the forward --------------------------------

def _model(spec, t):
    return OracleModel(spec, t)


def _dec(spec, t, name, l=0):
    m = OracleModel(spec, t)
    return m.weight(name, l)


@pytest.mark.parametrize("fmt", ["b4_32", "b4_256"])
def test_forward_residual_off(fmt):
    spec = tiny_spec(fmt)
    t = tiny_tensors(spec)
    t["wo"] = [zero_tensor_like(t["wo"][0])]
    t["w_down"] = [zero_tensor_like(t["w_down"][0])]
    kc, vc = random_kv(spec, 1, 16, 5)
    ids = np.array([[11, 3, 50]])
    got = _model(spec, t).verify_logits(ids, np.array([5]), kc, vc)[0]
    Wlm = _dec(spec, t, "lm_head")
    for r in range(3):
        e = t["tok_embd"][ids[0, r]].astype(np.float64)
        want = Wlm @ rmsnorm(e, t["out_norm"], spec.rms_eps)
        np.testing.assert_allclose(got[r], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("fmt", ["b4_32", "b4_256"])
def test_forward_single_key_attention(fmt):
    spec = tiny_spec(fmt)
    t = tiny_tensors(spec)
    t["w_down"] = [zero_tensor_like(t["w_down"][0])]
    kc, vc = random_kv(spec, 1, 16, 0)
    tok = 21
    got = _model(spec, t).verify_logits(np.array([[tok]]), np.array([0]), kc, vc)[0, 0]
    e = t["tok_embd"][tok].astype(np.float64)
    h = rmsnorm(e, t["attn_norm"][0], spec.rms_eps)
    v = (_dec(spec, t, "wv") @ h).reshape(spec.n_kv_head, spec.head_dim)
    v = v.astype(np.float16).astype(np.float64)
    G = spec.n_head // spec.n_kv_head
    o = np.concatenate([v[j // G] for j in range(spec.n_head)])
    x = e + _dec(spec, t, "wo") @ o
    want = _dec(spec, t, "lm_head") @ rmsnorm(x, t["out_norm"], spec.rms_eps)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_forward_uniform_attention_range():
    spec = tiny_spec("b4_32")
    t = tiny_tensors(spec)
    t["w_down"] = [zero_tensor_like(t["w_down"][0])]
    t["wk"] = [zero_tensor_like(t["wk"][0])]
    ctx = 6
    kc, vc = random_kv(spec, 1, 16, ctx)
    kc[:] = 0
    kc0, vc0 = kc.copy(), vc.copy()
    ids = np.array([[5, 9]])
    got = _model(spec, t).verify_logits(ids, np.array([ctx]), kc, vc)[0]
    Wv, Wo, Wlm = (_dec(spec, t, n) for n in ("wv", "wo", "lm_head"))
    G = spec.n_head // spec.n_kv_head
    vcache = vc0.astype(np.float64)
    for r in range(2):
        e = t["tok_embd"][ids[0, r]].astype(np.float64)
        h = rmsnorm(e, t["attn_norm"][0], spec.rms_eps)
        vnew = (Wv @ h).reshape(spec.n_kv_head, spec.head_dim)
        vcache[0, 0, ctx + r] = vnew.astype(np.float16).astype(np.float64)
        mean = vcache[0, 0, : ctx + r + 1].mean(axis=0)          # keys 0..pos
        o = np.concatenate([mean[j // G] for j in range(spec.n_head)])
        want = Wlm @ rmsnorm(e + Wo @ o, t["out_norm"], spec.rms_eps)
        np.testing.assert_allclose(got[r], want, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("fmt", ["b4_32", "b4_256"])
def test_forward_ffn_only(fmt):
    spec = tiny_spec(fmt)
    t = tiny_tensors(spec)
    t["wo"] = [zero_tensor_like(t["wo"][0])]
    kc, vc = random_kv(spec, 1, 16, 3)
    tok = 40
    got = _model(spec, t).verify_logits(np.array([[tok]]), np.array([3]), kc, vc)[0, 0]
    e = t["tok_embd"][tok].astype(np.float64)
    h2 = torch.tensor(rmsnorm(e, t["ffn_norm"][0], spec.rms_eps))
    Wg, Wu, Wd = (torch.tensor(_dec(spec, t, n)) for n in ("w_gate", "w_up", "w_down"))
    a = F.silu(F.linear(h2, Wg)) * F.linear(h2, Wu)
    x = e + F.linear(a, Wd).numpy()
    want = _dec(spec, t, "lm_head") @ rmsnorm(x, t["out_norm"], spec.rms_eps)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_forward_writes_rotated_fp16_cache_rows():
    spec = tiny_spec("b4_32", n_layer=2)
    t = tiny_tensors(spec)
    ctx = 4
    kc, vc = random_kv(spec, 2, 16, ctx)
    before_k, before_v = kc.copy(), vc.copy()
    ids = np.array([[1, 2, 3], [4, 5, 6]])
    lens = np.array([ctx, ctx - 1])
    _model(spec, t).verify_logits(ids, lens, kc, vc)
    # layer 0 rows: computable from the embedding alone
    Wk, Wv = _dec(spec, t, "wk"), _dec(spec, t, "wv")
    for s in range(2):
        for r in range(3):
            pos = lens[s] + r
            h = rmsnorm(t["tok_embd"][ids[s, r]].astype(np.float64), t["attn_norm"][0],
                        spec.rms_eps)
            k = rope((Wk @ h).reshape(spec.n_kv_head, -1), pos, spec.rope_base)
            np.testing.assert_array_equal(kc[0, s, pos], k.astype(np.float16))
            np.testing.assert_array_equal(
                vc[0, s, pos], (Wv @ h).reshape(spec.n_kv_head, -1).astype(np.float16))
        # rows outside [len, len+nt) untouched, in every layer
        keep = np.ones(16, bool)
        keep[lens[s]: lens[s] + 3] = False
        np.testing.assert_array_equal(kc[:, s, keep], before_k[:, s, keep])
        np.testing.assert_array_equal(vc[:, s, keep], before_v[:, s, keep])
