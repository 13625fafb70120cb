"""Seeded synthetic verification blocks shared by the tests, the bench and the
smoke check.  Input generation only: nothing here computes any step of the
method (no routing, no selection, no expert math)."""

from .gen import (  # noqa: F401
    CONFIGS,
    Config,
    Block,
    make_block,
    make_tree,
    expert_weights,
    shared_weights,
    to_exact_f64,
)
