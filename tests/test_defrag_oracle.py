"""Pins for the KV defragmentation oracle (oracle/defrag.py), CPU only.

The pages name the step (the plan's KV defragmentation phase, "The Plan
Document: A Pivot Point in Custom CUDA Kernel Development", section "Output
Knowledge Created") but not its interface; the reading is: prefix position p
of request b moves to slot dst_base[b] + p and its index is rewritten. The
pins: a hand-worked example, and the property that motivates the step --
verify attention over the compacted cache with the rewritten indices equals
verify attention over the original, exactly (checked with the attention
oracle, which shares nothing with the defrag oracle), which a planted
off-by-one breaks.
"""
import numpy as np
import pytest

from oracle import defrag as od
from oracle import verify_fp64 as vo
from workloads import gen


def test_hand_worked_example():
    # 2 requests: prefixes [5, 2, 7] and [3]; rows carry their slot number
    src = np.zeros((8, 576))
    for s in range(8):
        src[s, :] = s + 0.25
    dst = np.full((12, 576), -1.0)
    out, idx = od.defrag(src, dst, [0, 3, 4], [5, 2, 7, 3], [8, 1])
    assert idx.tolist() == [8, 9, 10, 1]
    assert out[8, 0] == 5.25 and out[9, 0] == 2.25 and out[10, 0] == 7.25 and out[1, 0] == 3.25
    assert (out[[0, 2, 3, 4, 5, 6, 7, 11]] == -1.0).all()  # nothing else written


def test_only_576_entries_move():
    src = np.arange(2 * 640, dtype=np.float64).reshape(2, 640)
    dst = np.full((2, 640), -1.0)
    out, _ = od.defrag(src, dst, [0, 1], [1], [0])
    assert (out[0, :576] == src[1, :576]).all() and (out[0, 576:] == -1.0).all()


def test_empty_prefix_and_in_place():
    src = np.arange(6 * 576, dtype=np.float64).reshape(6, 576)
    out, idx = od.defrag(src, src, [0, 0, 2], [4, 5], [7, 0])  # request 0 empty; same array as source
    assert idx.tolist() == [0, 1]
    assert (out[0] == src[4]).all() and (out[1] == src[5]).all()
    assert (src[0] == np.arange(576)).all()  # the input array is not modified


def _attention(w, pool, indices):
    return vo.verify(w.q_nope, w.q_rope, pool, w.kv_indptr, indices, w.out_cache_loc, w.custom_mask,
                     w.mask_indptr, w.sm_scale, w.num_draft)


@pytest.mark.parametrize("name", ["tiny", "ragged_small"])
def test_attention_unchanged_by_defrag(name):
    if name == "tiny":
        w = gen.build("tiny")
    else:
        w = gen.build(gen.small("ragged_small", batch=3, prefix=(0, 40), num_draft=3, num_heads=2, dtype="fp32",
                                tree="random", pool_slots=512, layout="scattered", nsplit=4, seed=77))
    pool = w.host_pool(fill=0.0).double().numpy()
    # destination runs after every used slot: free, disjoint, contiguous
    P = np.diff(w.kv_indptr.numpy())
    base = pool.shape[0] + np.concatenate([[0], np.cumsum(P)[:-1]]).astype(np.int64)
    big = np.vstack([pool, np.full((int(P.sum()) + 1, pool.shape[1]), np.nan)])
    new_pool, new_idx = od.defrag(big, big, w.kv_indptr.numpy(), w.kv_indices.numpy(), base)
    o0, l0 = _attention(w, big, w.kv_indices.numpy())
    o1, l1 = _attention(w, new_pool, new_idx)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # a planted off-by-one in the destination breaks the property
    if P.max() > 1:
        bad = new_idx.copy()
        j = int(np.argmax(P > 1))
        bad[w.kv_indptr.numpy()[j]] += 1
        o2, _ = _attention(w, new_pool, bad)
        assert not np.array_equal(o0, o2)
