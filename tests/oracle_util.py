"""Small helpers shared by the oracle and GPU tests (input plumbing only)."""

import numpy as np
import torch

from synth.configs import ModelSpec
from synth.make import make_weights


def tiny_spec(fmt="b4_32", **kw) -> ModelSpec:
    if fmt == "b4_32":
        base = dict(n_layer=1, hidden=64, n_head=4, n_kv_head=2, head_dim=16, ffn=128,
                    vocab=96, fmt_proj="b4_32", fmt_lm="b4_32")
    else:
        base = dict(n_layer=1, hidden=256, n_head=4, n_kv_head=2, head_dim=64, ffn=512,
                    vocab=200, fmt_proj="b4_256", fmt_lm="b6_256")
    base.update(kw)
    return ModelSpec(**base)


def to_numpy_tensors(w: dict) -> dict:
    out = {}
    for k, v in w.items():
        if isinstance(v, list):
            out[k] = [t.cpu().numpy() for t in v]
        else:
            out[k] = v.cpu().numpy()
    return out


def tiny_tensors(spec: ModelSpec, seed=7) -> dict:
    return to_numpy_tensors(make_weights(spec, seed, "cpu"))


def random_kv(spec: ModelSpec, n_seq: int, cap: int, ctx: int, seed=3):
    rng = np.random.default_rng(seed)
    shape = (spec.n_layer, n_seq, cap, spec.n_kv_head, spec.head_dim)
    kc = np.zeros(shape, dtype=np.float16)
    vc = np.zeros(shape, dtype=np.float16)
    kc[:, :, :ctx] = rng.standard_normal(shape[:2] + (ctx,) + shape[3:]).astype(np.float16)
    vc[:, :, :ctx] = rng.standard_normal(shape[:2] + (ctx,) + shape[3:]).astype(np.float16)
    return kc, vc


def zero_tensor_like(raw: np.ndarray) -> np.ndarray:
    """All-zero bytes: every scale is 0, so every decoded weight is 0 in all
    three formats."""
    return np.zeros_like(raw)
