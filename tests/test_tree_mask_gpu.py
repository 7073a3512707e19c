"""GPU parity of tvmla_tree_mask against the CPU oracle (byte-exact), and
verify with the device-built mask is bit-identical to verify with the
host-built one."""
import numpy as np
import pytest
import torch

from gpu_util import Device, log
from oracle import tree_mask as otm
from speculative_decoding_verify_mla_amd import binding
from workloads import gen

pytestmark = pytest.mark.gpu


def _run(parents_list, prefix_lens, T):
    indptr = np.concatenate([[0], np.cumsum(prefix_lens)]).astype(np.int32)
    exp_mask, exp_indptr = otm.build(parents_list, prefix_lens)
    parents = torch.from_numpy(np.concatenate(parents_list).astype(np.int32)).cuda()
    # poison: every byte the kernel should write starts at 7, plus 64 guard bytes after the end
    mask = torch.full((exp_mask.size + 64,), 7, dtype=torch.uint8, device="cuda")
    mindptr = torch.full((len(prefix_lens) + 1,), -5, dtype=torch.int32, device="cuda")
    binding.tree_mask(parents, torch.from_numpy(indptr).cuda(), T, mask, mindptr)
    torch.cuda.synchronize()
    got = mask.cpu().numpy()
    assert np.array_equal(got[:exp_mask.size], exp_mask), "mask bytes differ from the oracle"
    assert (got[exp_mask.size:] == 7).all(), "wrote past the end"
    assert np.array_equal(mindptr.cpu().numpy(), exp_indptr.astype(np.int32))


@pytest.mark.parametrize("seed", range(4))
def test_random_trees(seed):
    rng = np.random.default_rng(100 + seed)
    batch = int(rng.integers(1, 9))
    T = int(rng.integers(1, 65))
    prefix = [int(rng.integers(0, 3000)) for _ in range(batch)]
    parents = [np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)]) for _ in range(batch)]
    log(f"tree mask case seed {seed}: batch {batch} T {T} prefixes {prefix}")
    _run(parents, prefix, T)


@pytest.mark.parametrize("shape", ["chain", "star"])
def test_chain_and_star(shape):
    T, prefix = 64, [0, 1, 15, 16, 17, 1000]
    par = np.arange(-1, T - 1) if shape == "chain" else np.array([-1] + [0] * (T - 1))
    log(f"tree mask case {shape}: T {T}, prefixes {prefix}")
    _run([par] * len(prefix), prefix, T)


def test_bad_parent_order_terminates():
    # node 2 names a later node as parent: the walk stops there instead of looping
    T = 4
    parents = torch.tensor([-1, 0, 3, 2], dtype=torch.int32, device="cuda")
    indptr = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    mask = torch.zeros(T * T, dtype=torch.uint8, device="cuda")
    mindptr = torch.zeros(2, dtype=torch.int32, device="cuda")
    log("tree mask case: parent after child")
    binding.tree_mask(parents, indptr, T, mask, mindptr)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().reshape(T, T)
    assert m[2].tolist() == [0, 0, 1, 0] and m[3].tolist() == [0, 0, 1, 1]


@pytest.mark.parametrize("name", ["p4096", "ragged32", "long185k"])
def test_device_mask_equals_host_mask_and_verify(name):
    w = gen.build(name)
    log(f"tree mask full size {name}")
    T = w.num_draft
    parents = torch.from_numpy(np.concatenate(w.parents).astype(np.int32)).cuda()
    d = Device(w, fill=0.0)
    out0, lse0 = d.result()
    mask = torch.empty_like(d.custom_mask)
    mindptr = torch.empty_like(d.mask_indptr)
    binding.tree_mask(parents, d.kv_indptr, T, mask, mindptr)
    torch.cuda.synchronize()
    assert torch.equal(mask, d.custom_mask) and torch.equal(mindptr, d.mask_indptr)
    d.custom_mask, d.mask_indptr = mask, mindptr
    out1, lse1 = d.result()
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)
