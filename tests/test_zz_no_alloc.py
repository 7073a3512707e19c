"""tvmla_verify_noalloc: the verify call for callers that cannot allocate,
with the split partials in the library's per-device scratch array. Checked
through the C ABI against tvmla_verify_ex (same kernels: bit-identical) and
the fp64 oracle, on two calls in a row, the second with a smaller input,
and its size limit (rejected on the host, nothing enqueued)."""
import numpy as np
import pytest
import torch

from oracle import verify_fp64 as vo
from speculative_decoding_verify_mla_amd import binding
from tests.gpu_util import Device, compare, log
from workloads import gen

pytestmark = pytest.mark.gpu


def _noalloc(d, w, flags, nsplit=None):
    d.out.fill_(float("nan"))
    d.lse.fill_(float("nan"))
    binding.verify_noalloc(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc, d.custom_mask,
                           d.mask_indptr, w.sm_scale, nsplit or d.nsplit, d.out, d.lse, w.num_draft, flags=flags)
    torch.cuda.synchronize()
    return d.out.float().cpu().numpy().astype(np.float64), d.lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("flags", [0, binding.TUNE_NSPLIT])
def test_noalloc_matches_verify_ex_twice(flags):
    """A large call, then a smaller one: each equals tvmla_verify_ex bit for
    bit and matches the oracle (the second call reads none of the first's
    leftovers in the shared scratch)."""
    big = gen.build("p4096")
    small = gen.build(gen.small("noalloc_small", 3, [0, 37, 300], 5, 8, seed=11))
    for w in (big, small):
        log(f"noalloc flags={flags} {w.spec.name}: batch={w.batch} T={w.num_draft} H={w.num_heads}")
        ref_out, ref_lse = vo.verify(w.q_nope, w.q_rope, w.host_pool(), w.kv_indptr, w.kv_indices, w.out_cache_loc,
                                     w.custom_mask, w.mask_indptr, w.sm_scale, w.num_draft)
        d = Device(w)
        o_na, l_na = _noalloc(d, w, flags)
        compare(w, o_na, l_na, ref_out, ref_lse, f"{w.spec.name}/noalloc/flags{flags}")
        o_ex, l_ex = d.result(flags=flags)
        assert np.array_equal(o_na, o_ex) and np.array_equal(l_na, l_ex)


def test_noalloc_scratch_limit():
    """A call whose partials exceed the scratch is rejected before anything
    is enqueued (outputs untouched); at the largest split count that fits it
    runs and matches tvmla_verify_ex."""
    w = gen.build(gen.small("noalloc_limit", 1, [600], 16, 64, seed=12))
    d = Device(w, nsplit=256)
    rows = w.num_draft * w.num_heads  # 1024 rows x 2 KB per split: 128 splits would need 256 MiB + lse
    fits = max(ns for ns in range(1, 257) if rows * ns * 2048 + ((rows * ns * 4 + 255) // 256) * 256
               <= binding.NOALLOC_SCRATCH_BYTES)
    assert fits == 127
    d.out.fill_(7.0)
    with pytest.raises(binding.TvmlaError) as e:
        binding.verify_noalloc(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc,
                               d.custom_mask, d.mask_indptr, w.sm_scale, fits + 1, d.out, d.lse, w.num_draft)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((d.out.float() == 7.0).all())
    o_na, l_na = _noalloc(d, w, 0, nsplit=fits)
    o_ex, l_ex = d.result(nsplit=fits)
    assert np.array_equal(o_na, o_ex) and np.array_equal(l_na, l_ex)
