"""Graph capture of the device-side metadata path: tvmla_tree_mask followed by
tvmla_verify, and tvmla_verify_ragged, each captured once and replayed with
new prefix lengths, trees and token counts written into the same buffers.
Every replay matches the oracle and the eager call (capture safety: the
launches depend only on scalars; "The Architecture of Capture Safety", "The Design Emerges")."""
import numpy as np
import pytest
import torch

from gpu_util import compare, log
from oracle import verify_fp64 as vo
from speculative_decoding_verify_mla_amd import binding
from workloads import gen

pytestmark = pytest.mark.gpu

B, T, H, NS = 2, 8, 16, 16


class Buffers:
    def __init__(self, cap_prefix, cap_mask, pool_slots):
        c = "cuda"
        self.pool = torch.zeros((pool_slots, 576), dtype=torch.bfloat16, device=c)
        self.q_nope = torch.zeros((B * T, H, 512), dtype=torch.bfloat16, device=c)
        self.q_rope = torch.zeros((B * T, H, 64), dtype=torch.bfloat16, device=c)
        self.kv_indptr = torch.zeros(B + 1, dtype=torch.int32, device=c)
        self.kv_indices = torch.zeros(cap_prefix, dtype=torch.int32, device=c)
        self.ocl = torch.zeros(B * T, dtype=torch.int32, device=c)
        self.parents = torch.zeros(B * T, dtype=torch.int32, device=c)
        self.mask = torch.zeros(cap_mask, dtype=torch.uint8, device=c)
        self.mask_indptr = torch.zeros(B + 1, dtype=torch.int32, device=c)
        self.qo_indptr = torch.zeros(B + 1, dtype=torch.int64, device=c)
        self.out = torch.zeros((B * T, H, 512), dtype=torch.bfloat16, device=c)
        self.lse = torch.zeros((B * T, H), dtype=torch.float32, device=c)
        self.ws = torch.zeros(binding.workspace_bytes(B, T, H, NS), dtype=torch.uint8, device=c)


def _specs():
    return [gen.small("cap2", B, [300, 700], T, H, seed=61), gen.small("cap2", B, [1, 950], T, H, seed=62),
            gen.small("cap2", B, [512, 0], T, H, tree="chain", seed=63)]


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_capture_tree_mask_then_verify():
    ws_list = [gen.build(s) for s in _specs()]
    buf = Buffers(max(w.kv_indices.numel() for w in ws_list), max(w.custom_mask.numel() for w in ws_list), 1 << 16)

    def load(w):
        buf.pool[torch.from_numpy(w.slots).cuda()] = w.rows.cuda()
        buf.q_nope.copy_(w.q_nope.cuda())
        buf.q_rope.copy_(w.q_rope.cuda())
        buf.kv_indptr.copy_(w.kv_indptr.cuda())
        buf.kv_indices[:w.kv_indices.numel()].copy_(w.kv_indices.cuda())
        buf.ocl.copy_(w.out_cache_loc.cuda())
        buf.parents.copy_(torch.from_numpy(np.concatenate(w.parents).astype(np.int32)).cuda())

    def step():
        binding.tree_mask(buf.parents, buf.kv_indptr, T, buf.mask, buf.mask_indptr)
        binding.verify(buf.q_nope, buf.q_rope, buf.pool, buf.kv_indptr, buf.kv_indices, buf.ocl, buf.mask,
                       buf.mask_indptr, ws_list[0].sm_scale, NS, buf.out, buf.lse, buf.ws, T)

    load(ws_list[0])
    graph = _capture(step)
    for rep in range(2):
        for w in ws_list:
            log(f"capture tree_mask+verify replay {rep}, prefixes {list(w.prefix_lens)}")
            load(w)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(buf.mask[:w.custom_mask.numel()].cpu(), w.custom_mask)
            assert torch.equal(buf.mask_indptr.cpu(), w.mask_indptr)
            go, gl = buf.out.float().cpu().numpy().astype(np.float64), buf.lse.cpu().numpy().astype(np.float64)
            ro, rl = vo.verify(w.q_nope, w.q_rope, buf.pool.cpu(), w.kv_indptr, w.kv_indices, w.out_cache_loc,
                               w.custom_mask, w.mask_indptr, w.sm_scale, T)
            compare(w, go, gl, ro, rl, f"tree_mask+verify replay{rep}")
            step()  # eager, same buffers
            torch.cuda.synchronize()
            assert np.array_equal(go, buf.out.float().cpu().numpy()) and np.array_equal(gl, buf.lse.cpu().numpy())


def test_capture_ragged_verify():
    ws_list = [gen.build(s) for s in _specs()]
    tokens = [[8, 3], [1, 8], [5, 0]]
    rs = [gen.ragged_trees(w, t) for w, t in zip(ws_list, tokens)]
    buf = Buffers(max(w.kv_indices.numel() for w in ws_list), max(r.custom_mask.numel() for r in rs), 1 << 16)

    def load(w, r):
        n = r.q_nope.shape[0]
        buf.pool[torch.from_numpy(w.slots).cuda()] = w.rows.cuda()
        buf.q_nope[:n].copy_(r.q_nope.cuda())
        buf.q_rope[:n].copy_(r.q_rope.cuda())
        buf.kv_indptr.copy_(w.kv_indptr.cuda())
        buf.kv_indices[:w.kv_indices.numel()].copy_(w.kv_indices.cuda())
        buf.ocl[:n].copy_(r.out_cache_loc.cuda())
        buf.mask[:r.custom_mask.numel()].copy_(r.custom_mask.cuda())
        buf.mask_indptr.copy_(r.mask_indptr.cuda())
        buf.qo_indptr.copy_(r.qo_indptr.cuda())

    def step():
        # the tuned split count: a function of the sizes only, so the captured grid stays valid
        binding.verify_ragged(buf.q_nope, buf.q_rope, buf.pool, buf.kv_indptr, buf.kv_indices, buf.ocl, buf.mask,
                              buf.mask_indptr, buf.qo_indptr, ws_list[0].sm_scale, NS, buf.out, buf.lse, buf.ws, T,
                              flags=binding.TUNE_NSPLIT)

    load(ws_list[0], rs[0])
    graph = _capture(step)
    for rep in range(2):
        for w, r, t in zip(ws_list, rs, tokens):
            log(f"capture ragged replay {rep}, prefixes {list(w.prefix_lens)}, tokens {t}")
            load(w, r)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            n = r.q_nope.shape[0]
            go = buf.out[:n].float().cpu().numpy().astype(np.float64)
            gl = buf.lse[:n].cpu().numpy().astype(np.float64)
            ro, rl = vo.verify_ragged(r.q_nope, r.q_rope, buf.pool.cpu(), w.kv_indptr, w.kv_indices,
                                      r.out_cache_loc, r.custom_mask, r.mask_indptr, r.qo_indptr, w.sm_scale)
            compare(w, go, gl, ro, rl, f"ragged replay{rep}")
            step()
            torch.cuda.synchronize()
            assert np.array_equal(go, buf.out[:n].float().cpu().numpy())
            assert np.array_equal(gl, buf.lse[:n].cpu().numpy())
