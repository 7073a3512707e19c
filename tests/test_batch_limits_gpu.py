"""GPU parity at the batch limits of the request order and of the API.

Batches of 2 to 64 requests are served longest request first, larger ones
in index order (one wavefront ranks at most 64 lengths). A batch of 65
ragged requests runs the index-order path on lengths that the longest-first
order would have permuted. The largest batch the API takes (65,535
requests of one draft token and one head, prefixes of 0 to 3 keys) runs the
grid decode and the combine at their largest request count: sampled whole
requests (among them the first and the last) are compared with the oracle,
and every row with the bounds any softmax-weighted mean obeys.
"""
import numpy as np
import pytest
import torch

from oracle import verify_fp64 as vo
from speculative_decoding_verify_mla_amd import binding
from tests.gpu_util import Device, compare, log
from workloads import gen

pytestmark = pytest.mark.gpu

ROWS, MFMA = binding.ALGO_ROWS, binding.ALGO_MFMA


def _oracle_request(w, b, pool):
    """The oracle on request b alone: its query rows and draft slots, the
    two offsets of kv_indptr and mask_indptr (absolute, so they still index
    the whole arrays)."""
    T = w.num_draft
    rows = slice(b * T, (b + 1) * T)
    return vo.verify(w.q_nope[rows], w.q_rope[rows], pool, w.kv_indptr[b:b + 2], w.kv_indices,
                     w.out_cache_loc[rows], w.custom_mask, w.mask_indptr[b:b + 2], w.sm_scale, T)


def test_batch_65_index_order():
    w = gen.build(gen.small("b65_ragged", 65, (0, 400), 2, 8, pool_slots=1 << 15, nsplit=4, seed=78))
    ref_out, ref_lse = vo.verify(w.q_nope, w.q_rope, w.host_pool(), w.kv_indptr, w.kv_indices, w.out_cache_loc,
                                 w.custom_mask, w.mask_indptr, w.sm_scale, w.num_draft)
    d = Device(w)
    for algo, flags in ((ROWS, 0), (ROWS, binding.TUNE_NSPLIT), (MFMA, 0)):
        log(f"[b65_ragged] algo {algo} flags {flags}")
        out, lse = d.result(algo=algo, flags=flags)
        compare(w, out, lse, ref_out, ref_lse, f"b65_ragged/algo{algo}/flags{flags}")


def test_batch_maximum():
    w = gen.build(gen.small("b65535", 65535, (0, 3), 1, 1, pool_slots=1 << 18, nsplit=2, seed=77))
    log(f"[b65535] built: batch {w.batch}, keys {w.total_keys}")
    pool = w.host_pool()
    rng = np.random.default_rng(5)
    picks = sorted({0, 1, 63, 64, 65, w.batch - 2, w.batch - 1} | set(int(x) for x in rng.integers(0, w.batch, 200)))
    refs = {b: _oracle_request(w, b, pool) for b in picks}
    # per-row bounds: the output lies between the smallest and largest latent
    # entry over the row's visible keys (here: its prefix and its own draft key)
    rows_all = w.rows.float().numpy()
    off = w.row_offsets
    lo = np.stack([rows_all[off[b]:off[b + 1], :512].min(0) for b in range(w.batch)])
    hi = np.stack([rows_all[off[b]:off[b + 1], :512].max(0) for b in range(w.batch)])
    d = Device(w)
    for algo, flags in ((ROWS, 0), (ROWS, binding.TUNE_NSPLIT), (MFMA, 0)):
        log(f"[b65535] algo {algo} flags {flags}")
        out, lse = d.result(algo=algo, flags=flags)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), "non-finite output"
        o = out[:, 0, :]
        slack = 2e-2 + 2e-2 * np.maximum(np.abs(lo), np.abs(hi))
        assert np.all(o >= lo - slack) and np.all(o <= hi + slack), "a row outside its values' bounds"
        idx = np.array(picks)
        compare(w, out[idx], lse[idx], np.concatenate([refs[b][0] for b in picks]),
                np.concatenate([refs[b][1] for b in picks]), f"b65535/algo{algo}/flags{flags}, {len(picks)} requests")
