"""CPU oracle for the AcceptMoE verify-block MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code, tables or constants with the HIP
library under ``moe_speculative_decoding_gemm_amd/`` and it never loads that
library.

Sources (the pages this oracle is written from):

* [AcceptMoE news] -- news article on AcceptMoE (Imperial College London and
  Tile-AI), sections 01-04.
* [AcceptMoE abstract] -- arXiv 2608.02989 abstract page, English abstract.
* [MoE-SD blog] -- blog post "MoE 与推测解码：计算、通信和接受率的联合优化"
  (charlestar.github.io), sections on the single MoE layer, dense versus MoE
  verification, chain versus tree drafts, and the experiment metrics.
* [EcoSpec] -- "Cost-aware speculative decoding for MoE" (arXiv 2607.12696),
  Figure 1.
* [MoESD] -- MoESD summary page (papers.chlience.com), section 5.3.

Modules:

* :mod:`oracle.acceptmoe` -- selection (router, demand, anchor, self-size,
  residency-aware pruning, restricted top-k, gates), permute, grouped SwiGLU
  experts, combine.
* :mod:`oracle.fp8` -- OCP E4M3FN decoding for the fp8 expert weights.
* :mod:`oracle.cache` -- the expert cache under physical expert offload
  (least-recently-used slots; a reading, the pages give no policy).

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
page examples, closed forms, library routines or brute force, except where a
docstring says "parity unpinned".
"""

from . import acceptmoe, fp8  # noqa: F401
from .acceptmoe import (  # noqa: F401
    ERR_BAD_TREE,
    ERR_DEPTH,
    ERR_NONFINITE,
    ERR_COMMIT,
    F_NATURAL,
    F_NO_RENORM,
    F_LOGITS_IN,
    F_DEMAND_FULL,
    F_NO_ANCHOR,
    F_UNIT_COMMIT,
    OracleInputError,
    router_logits,
    softmax64,
    natural_topk,
    validate_tree,
    demand,
    root_anchor,
    effective_rank,
    self_size,
    fill_eligible,
    residency_prune,
    restricted_topk,
    gates,
    permute,
    swiglu,
    grouped_swiglu,
    combine,
    token_outputs,
    select,
    verify_block,
)
