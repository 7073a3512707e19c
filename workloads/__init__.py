"""Seeded synthetic inputs for tree-verify attention (shared by tests and bench).

This package only draws random numbers and lays them out in the metadata
format the verify call consumes; it holds none of the attention arithmetic.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    build,
    chain_parents,
    config,
    random_parents,
    tree_mask,
)
