"""CPU fp64 oracle of the batched target-verify round.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or run this package; the library's
product path never does, and this package imports nothing from the library.

What it computes (one verify round, written as plainly as possible):
  formats.py  decode of the three canonical block formats to fp64;
  model.py    embed -> per layer [RMSNorm, q/k/v, RoPE, fp16 KV append,
              causal attention over the fp16 cache, o + residual, RMSNorm,
              SwiGLU FFN + residual] -> final RMSNorm -> lm_head logits,
              one row at a time in fp64;
  decide.py   greedy first-mismatch rule and strict rejection sampling;
  round.py    one whole round: logits, decision, commit of the length.

Sources: the exactness transaction and the sampler-state rule of the Power
page ("Model-neutral Speculative Decoding", sections "The exactness
transaction" and the paragraph after it); the one-round mechanism of the
minfer plan ("Speculative Decoding (D5-R) -- Plan", section 3 "Mechanism --
one round"); the strict rejection sampler named on the DFlash/DSpark wiki
page ("DFlash and DSpark Speculative Decoding", sections "How DSpark Works"
and "Notes"), with the textbook rule accept with min(1, p/q), else sample
the normalised max(0, p - q).

Parity status: every function here is pinned by tests/test_oracle_*.py
against closed forms, library routines, exact enumeration or invariants;
GGUF byte compatibility of the formats is not claimed (parity unpinned for
that, as no GGUF artifact exists here).
"""

from .formats import decode  # noqa: F401
from .model import OracleModel  # noqa: F401
from .decide import greedy_decide, reject_decide, reject_decide_probs  # noqa: F401
from .round import verify_round  # noqa: F401
