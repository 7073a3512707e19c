"""Reference moves at the default fold threshold, forced by planted keys.

A key whose cache row is a multiple a of one query row's (q_nope, q_rope)
scores a |q|^2 for that row. With 576 standard-normal query entries and
sm_scale = 1/sqrt(192) that is about 60 a in log2 units, against a spread of
~2.5 for the row's other keys. So a = 0.5 moves the row's reference at the
default threshold (2^16), and a = 3 (~180 units) makes the probabilities
overflow fp32 unless the kernel moves the reference before using them; a
negative multiple underflows to a zero weight.

The plants put such keys in key block 0 and key block 1 of a tile (both in
one tile for one row: a move in each block), in the first tile, in later
tiles of a long split, in the ragged last tile, and on a draft key that the
tree mask may hide from the row. `test_planted_oracle` pins the oracle on
this workload to the closed form of a dominating key; the GPU test compares
the 128-row and the 64-row MFMA kernels with the oracle at one and two
splits.
"""
import numpy as np
import pytest
import torch

from oracle import verify_fp64 as vo
from workloads import gen

PREFIX, T, H = 690, 4, 40  # 694 keys: ten whole tiles and a ragged one of 54


# (logical key, token, head, multiple)
PLANTS = [
    (3, 3, 39, 3.0),                              # first tile, block 0: the first reference comes from it
    (64 * 2 + 45, 2, 33, 3.0),                    # block 1 only, after earlier tiles accumulated
    (64 * 3 + 10, 0, 0, 3.0),                     # block 0 of a later tile
    (64 * 4 + 12, 1, 5, 0.5), (64 * 4 + 50, 1, 5, 3.0),  # one tile: a move in block 0, then in block 1
    (64 * 6 + 20, 3, 20, -3.0),                   # a weight that underflows
    (680, 0, 7, 3.0),                             # ragged last tile, block 1
    (PREFIX + 0, 3, 1, 3.0),                      # a draft key: visible to token 3 only through the tree
]


def planted_workload():
    w = gen.build(gen.small("planted", 1, [PREFIX], T, H, tree="random", nsplit=1, seed=4242))
    for key, t, h, a in PLANTS:
        q = torch.cat([w.q_nope[t, h].float(), w.q_rope[t, h].float()])
        w.rows[key] = (a * q).to(w.rows.dtype)
    return w


def _oracle(w):
    return vo.verify(w.q_nope, w.q_rope, w.host_pool(), w.kv_indptr, w.kv_indices, w.out_cache_loc,
                     w.custom_mask, w.mask_indptr, w.sm_scale, w.num_draft)


def test_planted_oracle():
    """A visible planted key with a >= 3 outweighs the row's other keys by
    e^-120 or less: the row's output is that key's latent part and its lse the
    key's scaled score, to fp64 rounding. A negative plant leaves the row as
    it is without the key."""
    w = planted_workload()
    out, lse = _oracle(w)
    vis = w.custom_mask.numpy().reshape(T, PREFIX + T)
    rows = w.rows.double().numpy()
    checked = 0
    for key, t, h, a in PLANTS:
        if a < 3.0 or not vis[t, key]:
            continue
        if any(k2 != key and t2 == t and h2 == h and vis[t, k2] and a2 > a for k2, t2, h2, a2 in PLANTS):
            continue
        q = np.concatenate([w.q_nope[t, h].double().numpy(), w.q_rope[t, h].double().numpy()])
        np.testing.assert_allclose(out[t, h], rows[key, :512], rtol=1e-12, atol=1e-12)
        assert abs(lse[t, h] - float(q @ rows[key]) * w.sm_scale) < 1e-9
        checked += 1
    assert checked >= 5
    # the row with the negative plant: the same result as with the key masked out for it
    key, t, h, a = PLANTS[5]
    assert a < 0
    m2 = w.custom_mask.clone().reshape(T, PREFIX + T)
    m2[t, key] = 0
    out2, lse2 = vo.verify(w.q_nope, w.q_rope, w.host_pool(), w.kv_indptr, w.kv_indices, w.out_cache_loc,
                           m2.reshape(-1), w.mask_indptr, w.sm_scale, w.num_draft)
    np.testing.assert_allclose(out[t, h], out2[t, h], rtol=1e-12, atol=1e-15)
    # the block-0 plant of the pair is outweighed by the block-1 plant of the same row
    key0, t0, h0, _ = PLANTS[3]
    key1, _, _, _ = PLANTS[4]
    np.testing.assert_allclose(out[t0, h0], rows[key1, :512], rtol=1e-12, atol=1e-12)


@pytest.mark.gpu
@pytest.mark.parametrize("nsplit", [1, 2])
def test_planted_gpu(nsplit):
    from speculative_decoding_verify_mla_amd import binding
    from tests.gpu_util import Device, compare, log
    w = planted_workload()
    ref_out, ref_lse = _oracle(w)
    d = Device(w, nsplit=nsplit)
    for algo in (binding.ALGO_ROWS, binding.ALGO_MFMA):
        log(f"[planted] nsplit {nsplit} algo {algo}: default fold threshold")
        out, lse = d.result(algo=algo, nsplit=nsplit)
        compare(w, out, lse, ref_out, ref_lse, f"planted/nsplit{nsplit}/algo{algo}")


@pytest.mark.gpu
def test_planted_gpu_large_threshold():
    """fold_log2 above 64 is taken as 64: with a threshold of 1000 taken
    literally the 180-unit plants would overflow fp32 probabilities."""
    from speculative_decoding_verify_mla_amd import binding
    from tests.gpu_util import Device, compare, log
    w = planted_workload()
    ref_out, ref_lse = _oracle(w)
    d = Device(w, nsplit=1)
    for fold in (64.0, 1000.0):
        log(f"[planted] nsplit 1 row-owner kernel, fold threshold {fold}")
        out, lse = d.result(algo=binding.ALGO_ROWS, nsplit=1, fold_log2=fold)
        compare(w, out, lse, ref_out, ref_lse, f"planted/fold{fold}")
