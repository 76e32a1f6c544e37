"""The five verify workloads (model shapes, formats, batch, depth, context).

tiny  tiny single-layer greedy round, 4-bit/32 blocks everywhere (oracle-fast).
q7b_4l  Qwen2.5-7B-shaped 4-layer stack, nt swept 1..8 (bitwise nt-invariance).
q14b_48l  Qwen2.5-14B-shaped 48-layer stack, ctx 4096, nt = 3 and 9 (bandwidth gate).
lm248k_reject  lm_head only (6-bit, 248320 x 5120), 12 sequences, nt = 8, T = 0.8,
    strict rejection sampling.
q14b_8l_block16  14B layer dims with 8 layers, vocab 248320, 12 sequences, ctx 512,
    nt = 16 (and nt = 1), greedy block verify.

Format names: "b4_32" (4-bit codes in blocks of 32 with an fp16 scale),
"b4_256" (super-blocks of 256 = 8 sub-blocks of 32, 6-bit scale and min per
sub-block, fp16 super scale and super min), "b6_256" (super-blocks of 256 =
16 sub-blocks of 16, signed 8-bit scale per sub-block, fp16 super scale).
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class ModelSpec:
    n_layer: int
    hidden: int
    n_head: int
    n_kv_head: int
    head_dim: int
    ffn: int
    vocab: int
    fmt_proj: str
    fmt_lm: str
    rms_eps: float = 1e-6
    rope_base: float = 1.0e6
    lm_only: bool = False  # lm248k_reject: random hidden states straight into the lm_head


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    model: ModelSpec
    n_seq: int
    nt: Tuple[int, ...]
    ctx: int
    mode: str  # "greedy" | "reject" | "sample"
    temperature: float = 0.0
    # synthetic drafts: "oracle_corrupt" (tiny), "chain" (q7b_4l, q14b_48l), "block" (q14b_8l_block16),
    # "sample_q" (lm248k_reject)
    drafts: str = "chain"
    p_accept: float = 0.0
    p_decay: float = 1.0
    draft_noise: float = 0.0
    description: str = ""

    def with_(self, **kw):
        return replace(self, **kw)


TINY = Config(
    name="tiny", seed=101,
    model=ModelSpec(n_layer=1, hidden=512, n_head=8, n_kv_head=8, head_dim=64,
                    ffn=1536, vocab=4096, fmt_proj="b4_32", fmt_lm="b4_32"),
    n_seq=1, nt=(3,), ctx=64, mode="greedy", drafts="oracle_corrupt",
    p_accept=0.7,
    description="tiny single-round greedy verify, 4-bit/32 everywhere")

Q7B_4L = Config(
    name="q7b_4l", seed=102,
    model=ModelSpec(n_layer=4, hidden=3584, n_head=28, n_kv_head=4, head_dim=128,
                    ffn=18944, vocab=152064, fmt_proj="b4_256", fmt_lm="b6_256"),
    n_seq=1, nt=(1, 2, 3, 4, 5, 6, 7, 8), ctx=2048, mode="greedy",
    drafts="chain", p_accept=0.69,
    description="Qwen2.5-7B-shaped 4-layer stack, nt 1..8 bitwise sweep")

Q14B_48L = Config(
    name="q14b_48l", seed=103,
    model=ModelSpec(n_layer=48, hidden=5120, n_head=40, n_kv_head=8, head_dim=128,
                    ffn=13824, vocab=152064, fmt_proj="b4_256", fmt_lm="b6_256"),
    n_seq=1, nt=(3, 9), ctx=4096, mode="greedy", drafts="chain", p_accept=0.74,
    description="Qwen2.5-14B-shaped 48-layer stack, ctx 4096, nt 3 and 9")

LM248K_REJECT = Config(
    name="lm248k_reject", seed=104,
    model=ModelSpec(n_layer=0, hidden=5120, n_head=40, n_kv_head=8, head_dim=128,
                    ffn=13824, vocab=248320, fmt_proj="b4_256", fmt_lm="b6_256",
                    lm_only=True),
    n_seq=12, nt=(8,), ctx=0, mode="reject", temperature=0.8,
    drafts="sample_q", draft_noise=0.5,
    description="strict rejection sampling over a 6-bit 248320x5120 lm_head")

Q14B_8L_BLOCK16 = Config(
    name="q14b_8l_block16", seed=105,
    model=ModelSpec(n_layer=8, hidden=5120, n_head=40, n_kv_head=8, head_dim=128,
                    ffn=13824, vocab=248320, fmt_proj="b4_256", fmt_lm="b6_256"),
    n_seq=12, nt=(16, 1), ctx=512, mode="greedy", drafts="block",
    p_accept=0.9, p_decay=0.98,
    description="wide block verify, 12 sequences x 16 rows, 8 layers at 14B dims")

CONFIGS = {c.name: c for c in (TINY, Q7B_4L, Q14B_48L, LM248K_REJECT, Q14B_8L_BLOCK16)}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def block_bytes(fmt: str) -> Tuple[int, int]:
    """(weights per block, bytes per block) of a canonical format."""
    return {"b4_32": (32, 18), "b4_256": (256, 144), "b6_256": (256, 210)}[fmt]


def tensor_bytes(fmt: str, rows: int, cols: int) -> int:
    n, b = block_bytes(fmt)
    assert cols % n == 0
    return rows * (cols // n) * b


def layer_shapes(m: ModelSpec):
    """(name, rows, cols) of each projection of one layer, rows = out features."""
    q = m.n_head * m.head_dim
    kv = m.n_kv_head * m.head_dim
    return [("wq", q, m.hidden), ("wk", kv, m.hidden), ("wv", kv, m.hidden),
            ("wo", m.hidden, q), ("w_gate", m.ffn, m.hidden),
            ("w_up", m.ffn, m.hidden), ("w_down", m.hidden, m.ffn)]


def weight_bytes(m: ModelSpec) -> int:
    total = 0
    if not m.lm_only:
        for _, r, c in layer_shapes(m):
            total += m.n_layer * tensor_bytes(m.fmt_proj, r, c)
    total += tensor_bytes(m.fmt_lm, m.vocab, m.hidden)
    return total


def kv_read_bytes(cfg: Config, nt: int) -> int:
    """KV bytes one round reads: (len+nt) positions x layers x 2 x nkv x hd x 2 B."""
    m = cfg.model
    if m.lm_only:
        return 0
    return cfg.n_seq * (cfg.ctx + nt) * m.n_layer * 2 * m.n_kv_head * m.head_dim * 2
