"""tvmla_check_metadata: the host-side check of the metadata a verify call
reads raw (CPU only; no GPU, no HIP call). Well-formed workloads pass; each
kind of bad offset or slot is reported with its array and position."""
import numpy as np
import pytest

from speculative_decoding_verify_mla_amd import binding
from workloads import gen


@pytest.fixture(scope="module")
def lib():
    import os

    if not os.path.exists(binding.LIB_PATH):
        from speculative_decoding_verify_mla_amd import build

        build.build()
    return binding.load()


def _meta(w):
    return dict(kv_indptr=w.kv_indptr.numpy().copy(), kv_indices=w.kv_indices.numpy().copy(),
                out_cache_loc=w.out_cache_loc.numpy().copy(), mask_indptr=w.mask_indptr.numpy().copy(),
                mask_len=int(w.custom_mask.numel()), num_draft=w.num_draft, num_slots=w.spec.pool_slots)


def _check(m, qo=None):
    return binding.check_metadata(m["kv_indptr"], m["kv_indices"], m["out_cache_loc"], m["mask_indptr"],
                                  m["mask_len"], m["num_draft"], m["num_slots"], qo_indptr=qo)


@pytest.mark.parametrize("name", ["tiny", "p4096"])
def test_named_workloads_pass(lib, name):
    assert _check(_meta(gen.build(name))) == (0, "none", -1)


def _small():
    # requests with prefixes 0, 37 and 300 (an empty prefix included), 5 draft tokens, 8 heads
    return gen.build(gen.small("meta", 3, [0, 37, 300], 5, 8, pool_slots=4096, seed=11))


def test_small_workload_passes(lib):
    assert _check(_meta(_small())) == (0, "none", -1)


def test_bad_kv_indices_slot(lib):
    m = _meta(_small())
    m["kv_indices"][20] = m["num_slots"]  # one past the last slot
    assert _check(m) == (9, "kv_indices", 20)
    m["kv_indices"][20] = -1
    assert _check(m)[1:] == ("kv_indices", 20)


def test_bad_out_cache_loc_slot(lib):
    m = _meta(_small())
    m["out_cache_loc"][7] = m["num_slots"] + 5
    assert _check(m) == (9, "out_cache_loc", 7)


def test_kv_indptr_decreasing(lib):
    m = _meta(_small())
    ip = m["kv_indptr"]
    ip[2] = ip[1] - 1  # request 1 would have a negative prefix length
    assert _check(m) == (9, "kv_indptr", 2)


def test_kv_indptr_past_indices(lib):
    m = _meta(_small())
    m["kv_indices"] = m["kv_indices"][:-1]  # the last request's last prefix index is missing
    assert _check(m) == (9, "kv_indptr", 3)


def test_kv_indptr_negative_start(lib):
    m = _meta(_small())
    m["kv_indptr"][0] = -4
    assert _check(m) == (9, "kv_indptr", 0)


def test_mask_block_past_end(lib):
    m = _meta(_small())
    m["mask_len"] -= 1  # the last request's [T][N] block overruns the mask by one byte
    assert _check(m) == (9, "mask_indptr", 2)
    m = _meta(_small())
    m["mask_indptr"][1] = -1
    assert _check(m) == (9, "mask_indptr", 1)


def test_out_cache_loc_too_short(lib):
    m = _meta(_small())
    m["out_cache_loc"] = m["out_cache_loc"][:-1]
    assert _check(m) == (9, "out_cache_loc", 14)


def test_ragged_qo_indptr(lib):
    w = _small()
    m = _meta(w)
    # three requests with 5, 2 and 0 draft tokens: 7 token rows; mask blocks [T_b][P_b + T_b]
    P = np.diff(m["kv_indptr"])
    Tb = np.array([5, 2, 0])
    qo = np.concatenate([[0], np.cumsum(Tb)]).astype(np.int64)
    blocks = Tb * (P + Tb)
    m["mask_indptr"] = np.concatenate([[0], np.cumsum(blocks)]).astype(np.int32)
    m["mask_len"] = int(blocks.sum())
    m["out_cache_loc"] = m["out_cache_loc"][:7]
    assert _check(m, qo) == (0, "none", -1)
    bad = qo.copy()
    bad[2] = bad[1] - 1
    assert _check(m, bad) == (9, "qo_indptr", 2)
    bad = qo.copy()
    bad[3] = 9  # two tokens past out_cache_loc's end
    assert _check(m, bad) == (9, "out_cache_loc", 7)


def test_argument_errors(lib):
    m = _meta(_small())
    assert _check(dict(m, num_slots=0))[0] == 2
    assert _check(dict(m, num_draft=65))[0] == 2
    assert _check(dict(m, mask_len=-1))[0] == 2
