"""Seeded construction of weights, KV caches, ids, hidden states and drafts.

Every stream is keyed by (config seed, purpose, layer, tensor) through the
SplitMix64 hash chain in synth.rng, so a tensor does not depend on the order
in which tensors are generated.  Weights are drawn on the requested torch
device; the bytes therefore depend on that device's generator, and every test
or benchmark hands the *same bytes* to the oracle and to the library.

Distributions (the workloads' stated ones, plus the readings kept in DESIGN):
  projection and lm_head weights  N(0, 0.02^2), then quantized;
  token embedding                 fp16 N(0, 0.02^2);
  RMSNorm gains                   fp32 1 + 0.1 N(0,1);
  prefilled KV                    fp16 N(0,1) at positions 0..ctx-1;
  lm_head-only hidden states      fp32 N(0,1).
"""

import numpy as np
import torch

from .configs import Config, ModelSpec, layer_shapes
from .quant import quantize
from .rng import keyed_u64

P_WEIGHT, P_NORM, P_EMBED, P_KV, P_IDS, P_DRAFT, P_HIDDEN, P_NOISE = range(1, 9)
_TENSOR_ID = {"wq": 1, "wk": 2, "wv": 3, "wo": 4, "w_gate": 5, "w_up": 6,
              "w_down": 7, "lm_head": 8, "attn_norm": 9, "ffn_norm": 10,
              "out_norm": 11, "tok_embd": 12, "k": 13, "v": 14}


def _torch_gen(device, seed, purpose, layer, tensor) -> torch.Generator:
    s = int(keyed_u64(seed, purpose, layer, tensor)) & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _np_rng(seed, purpose, *key) -> np.random.Generator:
    return np.random.default_rng([seed, purpose, *key])


def _randn(shape, gen, device, chunk_rows=8192):
    """N(0,1) fp32, drawn in row chunks to bound peak memory on large tensors."""
    rows = shape[0]
    out = torch.empty(shape, dtype=torch.float32, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen,
                                 device=device, dtype=torch.float32)
    return out


def make_quant_tensor(fmt, rows, cols, seed, layer, name, device, std=0.02,
                      chunk_rows=4096):
    g = _torch_gen(device, seed, P_WEIGHT, layer, _TENSOR_ID[name])
    out = None
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        w = torch.randn((r1 - r0, cols), generator=g, device=device,
                        dtype=torch.float32) * std
        q = quantize(fmt, w)
        del w
        if out is None:
            out = torch.empty((rows, q.shape[1]), dtype=torch.uint8, device=device)
        out[r0:r1] = q
    return out


def make_weights(spec: ModelSpec, seed: int, device="cpu") -> dict:
    """Canonical model tensors.  Quantized tensors are uint8 [rows][bytes]."""
    H = spec.hidden
    w = {}
    if not spec.lm_only:
        g = _torch_gen(device, seed, P_EMBED, 0, _TENSOR_ID["tok_embd"])
        w["tok_embd"] = (_randn((spec.vocab, H), g, device) * 0.02).to(torch.float16)
        for nm in ("attn_norm", "ffn_norm"):
            g = _torch_gen(device, seed, P_NORM, 0, _TENSOR_ID[nm])
            w[nm] = 1.0 + 0.1 * torch.randn((spec.n_layer, H), generator=g,
                                            device=device, dtype=torch.float32)
        g = _torch_gen(device, seed, P_NORM, 0, _TENSOR_ID["out_norm"])
        w["out_norm"] = 1.0 + 0.1 * torch.randn((H,), generator=g, device=device,
                                                dtype=torch.float32)
        for name, rows, cols in layer_shapes(spec):
            w[name] = [make_quant_tensor(spec.fmt_proj, rows, cols, seed, l, name,
                                         device) for l in range(spec.n_layer)]
    w["lm_head"] = make_quant_tensor(spec.fmt_lm, spec.vocab, H, seed, 0, "lm_head",
                                     device)
    return w


def kv_capacity(cfg: Config, nt_max: int = None) -> int:
    nt_max = max(cfg.nt) if nt_max is None else nt_max
    cap = cfg.ctx + nt_max
    return (cap + 127) // 128 * 128


def make_kv(cfg: Config, capacity: int, device="cpu"):
    """fp16 K and V in the logical layout [layer][seq][pos][kv_head][head_dim];
    positions < ctx hold N(0,1), the rest zeros.  Returns (K, V, lens)."""
    m = cfg.model
    shape = (m.n_layer, cfg.n_seq, capacity, m.n_kv_head, m.head_dim)
    K = torch.zeros(shape, dtype=torch.float16, device=device)
    V = torch.zeros(shape, dtype=torch.float16, device=device)
    for l in range(m.n_layer):
        for s in range(cfg.n_seq):
            for nm, buf in (("k", K), ("v", V)):
                g = _torch_gen(device, cfg.seed, P_KV, l * 4096 + s, _TENSOR_ID[nm])
                buf[l, s, : cfg.ctx] = torch.randn(
                    (cfg.ctx, m.n_kv_head, m.head_dim), generator=g, device=device,
                    dtype=torch.float32).to(torch.float16)
    lens = np.full((cfg.n_seq,), cfg.ctx, dtype=np.int32)
    return K, V, lens


def make_anchors(cfg: Config, round_idx: int = 0) -> np.ndarray:
    rng = _np_rng(cfg.seed, P_IDS, round_idx)
    return rng.integers(0, cfg.model.vocab, size=cfg.n_seq).astype(np.int32)


def make_hidden(cfg: Config, nt: int, device="cpu") -> torch.Tensor:
    """lm_head-only workload: fp32 [n_seq][nt][hidden] N(0,1)."""
    g = _torch_gen(device, cfg.seed, P_HIDDEN, nt, 0)
    return torch.randn((cfg.n_seq, nt, cfg.model.hidden), generator=g, device=device,
                       dtype=torch.float32)


def accept_prob(cfg: Config, depth: int) -> float:
    """Per-position probability that the synthetic draft at 0-based depth
    equals the target's argmax."""
    return cfg.p_accept * (cfg.p_decay ** depth)


def chain_drafts(cfg: Config, anchors: np.ndarray, nt: int, argmax_fn,
                 round_idx: int = 0, follow_after_miss: bool = None) -> np.ndarray:
    """ids [n_seq][nt] with ids[:,0] = anchors and synthetic drafts.

    argmax_fn(ids_prefix [n_seq][r], need [n_seq] bool) must return, per
    sequence, the target's argmax on row r-1 given that prefix (the caller
    runs a model for it); only the entries where `need` is set are used.
    Depth i keeps the argmax with probability accept_prob(cfg, i); otherwise
    it takes a uniform id different from the argmax (a miss).  With
    follow_after_miss False (the q7b_4l/q14b_48l/q14b_8l_block16 recipe:
    "uniform random after the first miss") every position after a sequence's
    first miss is a uniform id over the whole vocabulary, and that
    sequence's argmax is no longer needed; with True (the tiny recipe) each
    position is corrupted independently and later positions keep following
    the argmax chain.  The random draws per depth do not depend on which
    argmaxes were needed.
    """
    if follow_after_miss is None:
        follow_after_miss = cfg.drafts == "oracle_corrupt"
    V = cfg.model.vocab
    S = len(anchors)
    rng = _np_rng(cfg.seed, P_DRAFT, round_idx, nt)
    ids = np.zeros((S, nt), dtype=np.int32)
    ids[:, 0] = anchors
    missed = np.zeros(S, dtype=bool)
    for r in range(1, nt):
        keep = rng.random(S) < accept_prob(cfg, r - 1)
        other = rng.integers(0, V - 1, size=S)
        anyid = rng.integers(0, V, size=S)
        need = np.ones(S, dtype=bool) if follow_after_miss else ~missed
        am = np.zeros(S, dtype=np.int64)
        if need.any():
            am = np.where(need, np.asarray(argmax_fn(ids[:, :r], need), dtype=np.int64), 0)
        miss_id = other + (other >= am)          # uniform over ids != argmax
        if follow_after_miss:
            new = np.where(keep, am, miss_id)
        else:
            new = np.where(missed, anyid, np.where(keep, am, miss_id))
            missed |= ~keep
        ids[:, r] = new.astype(np.int32)
    return ids


def draft_logits_from_target(cfg: Config, target_logits: np.ndarray) -> np.ndarray:
    """lm248k_reject drafter: fp32 (target logits + N(0, noise^2)), rows 0..nt-2."""
    S, nt, V = target_logits.shape
    rng = _np_rng(cfg.seed, P_NOISE, nt)
    noise = rng.standard_normal((S, nt - 1, V)) * cfg.draft_noise
    return (target_logits[:, : nt - 1].astype(np.float64) + noise).astype(np.float32)


def sample_drafts_from_q(cfg: Config, anchors, draft_logits: np.ndarray) -> np.ndarray:
    """lm248k_reject drafts: x_{r+1} ~ softmax(draft_logits_r / T) (input construction)."""
    S, d, V = draft_logits.shape
    rng = _np_rng(cfg.seed, P_DRAFT, 99, d)
    ids = np.zeros((S, d + 1), dtype=np.int32)
    ids[:, 0] = anchors
    T = cfg.temperature
    for s in range(S):
        for r in range(d):
            z = draft_logits[s, r].astype(np.float64) / T
            z = np.exp(z - z.max())
            c = np.cumsum(z)
            ids[s, r + 1] = int(np.searchsorted(c, rng.random() * c[-1], side="right"))
    return ids
