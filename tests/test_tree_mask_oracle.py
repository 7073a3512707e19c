"""Pins for the tree-mask oracle (oracle/tree_mask.py), CPU only: worked
examples (a chain gives a lower-triangular draft block, a star gives the
identity plus the root column), invariants (row i holds depth(i) + 1 ones in
its draft part, the root column is all ones, the prefix part is all ones),
and agreement with the transitive closure of the parent relation computed by
boolean matrix powers (a different algorithm), on random trees."""
import numpy as np
import pytest

from oracle import tree_mask as otm


def _block(mask, indptr, b, T, P):
    return mask[indptr[b]:indptr[b + 1]].reshape(T, P + T)


def test_chain_is_lower_triangular():
    T, P = 5, 3
    mask, indptr = otm.build([np.arange(-1, T - 1)], [P])
    blk = _block(mask, indptr, 0, T, P)
    assert (blk[:, :P] == 1).all()
    assert np.array_equal(blk[:, P:], np.tril(np.ones((T, T), np.uint8)))


def test_star_is_identity_plus_root():
    T = 6
    mask, indptr = otm.build([np.array([-1] + [0] * (T - 1))], [0])
    blk = _block(mask, indptr, 0, T, 0)
    want = np.eye(T, dtype=np.uint8)
    want[:, 0] = 1
    assert np.array_equal(blk, want)


def test_worked_two_requests():
    # request 0: P=2, tree 0 <- 1 <- 3, 0 <- 2 ; request 1: P=0, single node
    mask, indptr = otm.build([np.array([-1, 0, 0, 1]), np.array([-1])], [2, 0])
    assert indptr.tolist() == [0, 24, 25]
    want0 = np.array([[1, 1, 1, 0, 0, 0],
                      [1, 1, 1, 1, 0, 0],
                      [1, 1, 1, 0, 1, 0],
                      [1, 1, 1, 1, 0, 1]], np.uint8)
    assert np.array_equal(_block(mask, indptr, 0, 4, 2), want0)
    assert mask[24] == 1


def _closure(parents):
    T = len(parents)
    A = np.zeros((T, T), dtype=bool)  # A[i, j]: j is the parent of i
    for i, p in enumerate(parents):
        if p >= 0:
            A[i, p] = True
    R = np.eye(T, dtype=bool)
    step = np.eye(T, dtype=bool)
    for _ in range(T):
        step = (step.astype(np.int64) @ A.astype(np.int64)) > 0
        R |= step
    return R.astype(np.uint8)


@pytest.mark.parametrize("seed", range(6))
def test_random_trees_match_transitive_closure(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 40))
    parents = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)])
    P = int(rng.integers(0, 9))
    mask, indptr = otm.build([parents], [P])
    blk = _block(mask, indptr, 0, T, P)
    assert np.array_equal(blk[:, P:], _closure(parents))
    assert (blk[:, :P] == 1).all() and (blk[:, P] == 1).all()
    depth = np.array([len(otm.ancestors_or_self(parents, i)) for i in range(T)])
    assert np.array_equal(blk[:, P:].sum(1), depth)


def test_planted_mistake_is_caught():
    parents = np.array([-1, 0, 1, 1, 3])
    mask, indptr = otm.build([parents], [1])
    blk = _block(mask, indptr, 0, 5, 1).copy()
    blk[4, 1 + 1] = 0  # drop an ancestor
    assert not np.array_equal(blk[:, 1:], _closure(parents))
