"""CPU oracle for building the verify visibility mask from draft-tree parents.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module; the product path never does,
and this module imports nothing from the product package.

A DDTree drafter proposes a tree of draft tokens that the target model
verifies in one pass; the verify attention then needs a mask saying which
draft token sees which key ("The Architecture of Capture Safety: Designing a
CUDA Graph-Compatible Verify Kernel for SGLang", section "Input Knowledge
Required", DDTree paragraph), passed raw as custom_mask + mask_indptr
(same page, section "The Design Emerges", third insight). Building it on the
device removes host marshaling around the verify call (the directive quoted
in the same page's introduction).

Definition (a reading of the pages, which give no formula): request b has P_b prefix keys and
T draft nodes; node 0 is the root (parent -1) and parent[i] < i. Row i of the
request's [T][P_b + T] byte block is
    1 at every prefix column p < P_b,
    1 at draft column P_b + j  iff  j == i or j is an ancestor of i,
    0 elsewhere;
blocks are concatenated, mask_indptr[b] = sum over b' < b of T * (P_b' + T).
"""
from __future__ import annotations

import numpy as np


def ancestors_or_self(parents, i: int) -> set:
    """Node i and every node on its path to the root."""
    out = set()
    j = int(i)
    while j >= 0:
        out.add(j)
        j = int(parents[j])
    return out


def build(parents_per_request, prefix_lens):
    """Return (custom_mask uint8 flat, mask_indptr int64 [batch+1])."""
    blocks, indptr = [], [0]
    for parents, P in zip(parents_per_request, prefix_lens):
        T = len(parents)
        m = np.zeros((T, int(P) + T), dtype=np.uint8)
        for i in range(T):
            m[i, :int(P)] = 1
            for j in ancestors_or_self(parents, i):
                m[i, int(P) + j] = 1
        blocks.append(m.reshape(-1))
        indptr.append(indptr[-1] + m.size)
    flat = np.concatenate(blocks) if blocks else np.zeros(0, np.uint8)
    return flat, np.asarray(indptr, dtype=np.int64)
