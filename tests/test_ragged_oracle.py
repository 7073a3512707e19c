"""Pins for the ragged-tree oracle (oracle.verify_fp64.verify_ragged), CPU
only: with every T_b = T it agrees with the fixed-T oracle; request by
request it agrees with the fixed-T oracle run on that request alone with
T = T_b (an independent indexing path); empty trees produce no rows."""
import numpy as np
import pytest
import torch

from oracle import verify_fp64 as vo
from workloads import gen


def _small(T=6, batch=4, seed=31):
    return gen.build(gen.small("rag", batch=batch, prefix=(0, 50), num_draft=T, num_heads=3, dtype="fp32",
                               tree="random", pool_slots=1024, layout="scattered", nsplit=4, seed=seed))


def _ragged(w, tokens):
    r = gen.ragged_trees(w, tokens)
    pool = w.host_pool(fill=0.0)
    out, lse = vo.verify_ragged(r.q_nope, r.q_rope, pool, w.kv_indptr, w.kv_indices, r.out_cache_loc,
                                r.custom_mask, r.mask_indptr, r.qo_indptr, w.sm_scale)
    return r, pool, out, lse


def test_uniform_tokens_equal_fixed_oracle():
    w = _small()
    _, pool, out, lse = _ragged(w, [w.num_draft] * w.batch)
    ref_o, ref_l = vo.verify(w.q_nope, w.q_rope, pool, w.kv_indptr, w.kv_indices, w.out_cache_loc, w.custom_mask,
                             w.mask_indptr, w.sm_scale, w.num_draft)
    assert np.allclose(out, ref_o, rtol=1e-12, atol=1e-12) and np.allclose(lse, ref_l, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tokens", [[6, 1, 3, 5], [0, 6, 0, 2], [1, 1, 1, 1]])
def test_each_request_equals_its_own_fixed_oracle(tokens):
    w = _small()
    r, pool, out, lse = _ragged(w, tokens)
    qo = r.qo_indptr.numpy()
    assert out.shape[0] == sum(tokens)
    for b, Tb in enumerate(tokens):
        if Tb == 0:
            continue
        P = int(w.prefix_lens[b])
        ip = w.kv_indptr.numpy()
        sl = slice(int(qo[b]), int(qo[b + 1]))
        ref_o, ref_l = vo.verify(r.q_nope[sl], r.q_rope[sl], pool, torch.tensor([0, P], dtype=torch.int32),
                                 w.kv_indices[int(ip[b]):int(ip[b + 1])], r.out_cache_loc[sl],
                                 r.custom_mask[int(r.mask_indptr[b]):int(r.mask_indptr[b + 1])],
                                 torch.tensor([0, Tb * (P + Tb)], dtype=torch.int32), w.sm_scale, Tb)
        assert np.allclose(out[sl], ref_o, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[sl], ref_l, rtol=1e-12, atol=1e-12)


def test_truncated_tree_keeps_its_mask_block():
    w = _small()
    r = gen.ragged_trees(w, [3, 0, 6, 1])
    assert r.qo_indptr.tolist() == [0, 3, 3, 9, 10]
    P0 = int(w.prefix_lens[0])
    full0 = w.custom_mask[:w.num_draft * (P0 + w.num_draft)].reshape(w.num_draft, -1)
    assert torch.equal(r.custom_mask[:3 * (P0 + 3)].reshape(3, -1), full0[:3, :P0 + 3])
