"""CPU oracle for per-token adapter routing (MoLoRA).  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The GPU library never calls it and shares no code
with it.  See ``oracle/molora_oracle.py`` for the functions and their sources, and
``oracle/transformer.py`` for the synthetic decoder with per-token LoRA.
"""
from .molora_oracle import (  # noqa: F401
    bf16_to_f64,
    route_vocab,
    router_logits,
    route_topk,
    dispatch,
    apply,
    apply_masked_passes,
    pairs_of,
    apply_backward,
    route_topk_backward,
    router_backward,
)
from . import transformer  # noqa: F401,E402
