"""Seeded synthetic inputs for the batched target-verify round.

This package only *makes inputs*: random weights quantized into the three
canonical block formats, fp16 KV caches, token ids, draft logits and the
pre-generated uniforms of the stochastic sampler.  It holds none of the
verify round's arithmetic (no decode, no forward pass, no decision); both the
CPU oracle (``oracle/``) and the HIP library consume what it produces.

Shapes and distributions follow the workloads the pages describe (a 7B- and
a 14B-shaped Qwen2.5 stack with vocab 152064, vocab 248320 at context 512 and
batch 12, draft depths 2/8/15) with random weights, because no checkpoint or
prompt suite is part of this repository.
"""

from .configs import CONFIGS, ModelSpec, get_config  # noqa: F401
