"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every output is compared element by element (and by relative L2 error) with
the oracle: the small and medium workloads, the full-size long-context,
8-head and ragged workloads whole, and two whole requests of the heavy one
(its other rows by properties that hold at any size: convex bounds and
bitwise equality of the scattered and contiguous layouts).
"""
import numpy as np
import pytest
import torch

from oracle import verify_fp64 as vo
from speculative_decoding_verify_mla_amd import binding
from tests.gpu_util import Device, compare, log
from workloads import gen

pytestmark = pytest.mark.gpu

MFMA, SCALAR, ROWS = binding.ALGO_MFMA, binding.ALGO_SCALAR, binding.ALGO_ROWS


def _oracle(w, pool=None):
    pool = w.host_pool() if pool is None else pool
    return vo.verify(w.q_nope, w.q_rope, pool, w.kv_indptr, w.kv_indices, w.out_cache_loc, w.custom_mask,
                     w.mask_indptr, w.sm_scale, w.num_draft)


def _explicit(d, w, ns, algo, fold_log2=binding.FOLD_DEFAULT):
    """Split step + combine at exactly `ns` splits, through the two separate
    entry points."""
    binding.verify_partials(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc, d.custom_mask,
                            d.mask_indptr, w.sm_scale, ns, d.ws, w.num_draft, algo=algo, fold_log2=fold_log2)
    binding.combine(d.ws, d.kv_indptr, w.batch, w.num_draft, w.num_heads, ns, d.out, d.lse)
    torch.cuda.synchronize()
    return d.out.float().cpu().numpy().astype(np.float64), d.lse.cpu().numpy().astype(np.float64)


def _algos(w):
    return [SCALAR] if w.spec.dtype == "fp32" else [ROWS, MFMA, SCALAR]


SMALL = {
    # multiple tiles, ragged tails, a partial 128-row group (8 heads x 5 tokens)
    "ragged_h8": gen.small("ragged_h8", 3, [0, 37, 300], 5, 8, seed=11),
    # eight full row groups per request, many splits of a few keys
    "groups_h64": gen.small("groups_h64", 2, [200, 1000], 16, 64, seed=12),
    # degenerate: one token, one head; the second request has no prefix at all
    "t1_h1": gen.small("t1_h1", 2, [5, 0], 1, 1, seed=13),
    # largest tree, two heads
    "t64_h2": gen.small("t64_h2", 1, [100], 64, 2, seed=14),
    # largest head count
    "t2_h128": gen.small("t2_h128", 1, [50], 2, 128, seed=15),
    # largest tree at the largest head count: 8192 rows, 64 row groups of 128
    "t64_h128": gen.small("t64_h128", 1, [100], 64, 128, seed=18),
    # chain tree over a longer prefix
    "chain_h16": gen.small("chain_h16", 2, [700, 65], 8, 16, tree="chain", seed=16),
    # fp32 through the scalar kernel, ragged
    "fp32_ragged": gen.small("fp32_ragged", 3, [0, 9, 130], 4, 8, dtype="fp32", seed=17),
    # many short requests: 19,200 (request, split) pairs, 7,200 output rows (one combine wavefront each)
    "many_requests": gen.small("many_requests", 300, (0, 64), 3, 8, pool_slots=1 << 15, seed=18),
    # 64 requests of random lengths (the largest batch the split kernels order longest first)
    "b64_ragged": gen.small("b64_ragged", 64, (0, 400), 2, 8, pool_slots=1 << 15, seed=19),
    # equal lengths in one batch: the longest-first order breaks ties by request index
    "ties": gen.small("ties", 5, [60, 300, 60, 300, 60], 3, 16, seed=20),
}


@pytest.mark.parametrize("name", ["tiny", "p4096"])
def test_named_configs_full(name):
    w = gen.build(name)
    ref_out, ref_lse = _oracle(w)
    d = Device(w)
    for algo in _algos(w):
        log(f"[{name}] algo={algo} batch={w.batch} T={w.num_draft} H={w.num_heads} P={list(w.prefix_lens)}")
        out, lse = d.result(algo=algo)
        compare(w, out, lse, ref_out, ref_lse, f"{name}/algo{algo}")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_cases_full(name):
    w = gen.build(SMALL[name])
    ref_out, ref_lse = _oracle(w)
    d = Device(w)
    for algo in _algos(w):
        log(f"[{name}] algo={algo}")
        out, lse = d.result(algo=algo)
        compare(w, out, lse, ref_out, ref_lse, f"{name}/algo{algo}")


@pytest.mark.parametrize("batch,prefix,T,H", [
    (1, [300], 16, 64),             # 1024 rows: the combine runs 4 wavefronts per row
    (4, [50, 0, 130, 7], 16, 64),   # 4096 rows: one wavefront per row, four rows per workgroup
])
def test_fp32_combine_widths(batch, prefix, T, H):
    """fp32 queries (scalar split kernel, fp32 partial rows) at row counts that
    take the combine's 4- and 1-wavefront-per-row forms."""
    w = gen.build(gen.small("fp32_wide", batch, prefix, T, H, dtype="fp32", seed=23))
    ref_out, ref_lse = _oracle(w)
    d = Device(w)
    out, lse = d.result(algo=SCALAR)
    compare(w, out, lse, ref_out, ref_lse, f"fp32_wide/{batch}x{T}x{H}")


@pytest.mark.parametrize("algo", [ROWS, MFMA, SCALAR])
def test_packed_query_views(algo):
    """A packed [tokens, heads, 576] query passed as two strided views (latent
    part and rope part of each row) gives the same bits as two contiguous
    tensors."""
    w = gen.build(SMALL["groups_h64"])
    d = Device(w)
    o1, l1 = d.result(algo=algo)
    packed = torch.cat([d.q_nope, d.q_rope], dim=-1).contiguous()  # [tokens, heads, 576]
    d.q_nope, d.q_rope = packed[..., :512], packed[..., 512:]
    assert d.q_nope.stride() == (w.num_heads * 576, 576, 1)
    o2, l2 = d.result(algo=algo)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("nsplit", [1, 3, 64, 200, 256])
def test_nsplit_invariance(nsplit):
    w = gen.build("p4096")
    ref_out, ref_lse = _oracle(w)
    d = Device(w, nsplit=nsplit)
    for algo in (ROWS, MFMA):
        log(f"[p4096] nsplit={nsplit} algo={algo}")
        out, lse = _explicit(d, w, nsplit, algo)
        compare(w, out, lse, ref_out, ref_lse, f"nsplit{nsplit}/algo{algo}")


@pytest.mark.parametrize("fold", [0.0, 0.5, 3.0])
@pytest.mark.parametrize("name", ["ragged_h8", "groups_h64", "t64_h2", "chain_h16", "t2_h128"])
def test_rows_fold_path(fold, name):
    """The row-owner kernel folds its accumulator into the workspace when a
    row's max outgrows its reference by more than 2^fold_log2 (16 by
    default, rare on these inputs). Thresholds of 0..3 make folds frequent,
    including repeated folds into the same slot; the result must not
    change."""
    w = gen.build(SMALL[name])
    ref_out, ref_lse = _oracle(w)
    for ns in (1, 2):  # long splits: folds need tiles after a row's first
        d = Device(w, nsplit=ns)
        base_out, base_lse = _explicit(d, w, ns, ROWS)
        log(f"[{name}] nsplit {ns} fold threshold {fold}")
        out, lse = _explicit(d, w, ns, ROWS, fold_log2=fold)
        compare(w, out, lse, ref_out, ref_lse, f"{name}/nsplit{ns}/fold{fold}")
        if fold == 0.0 and max(w.prefix_lens) + w.num_draft > 2 * 64 * ns:
            # several tiles per split: the folds changed the rounding
            assert not np.array_equal(out, base_out), "no fold happened"
        # the full call passes the threshold to the same kernel
        o2, l2 = d.result(algo=ROWS, nsplit=ns, fold_log2=fold)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_rows_fold_one_split_long():
    """One split over 4,112 keys (65 tiles) with a fold on every growth of a
    row max: many folds per slot."""
    w = gen.build("p4096")
    ref_out, ref_lse = _oracle(w)
    d = Device(w, nsplit=1)
    out, lse = _explicit(d, w, 1, ROWS, fold_log2=0.0)
    compare(w, out, lse, ref_out, ref_lse, "p4096/nsplit1/fold0")


@pytest.mark.parametrize("min_chunk", [16, 256, 100000])
def test_min_chunk(min_chunk):
    w = gen.build(SMALL["groups_h64"])
    ref_out, ref_lse = _oracle(w)
    d = Device(w)
    for algo in (ROWS, MFMA, SCALAR):
        out, lse = d.result(algo=algo, min_chunk=min_chunk)
        compare(w, out, lse, ref_out, ref_lse, f"min_chunk{min_chunk}/algo{algo}")


def test_partials_match_oracle_splits():
    """The workspace after a call holds each split's (normalised output, lse),
    matching the oracle's per-split attention on the pages' schedule."""
    w = gen.build(SMALL["ragged_h8"])
    ns = 7
    pool = w.host_pool()
    o_ref, l_ref, nonempty = vo.verify_partials(w.q_nope, w.q_rope, pool, w.kv_indptr, w.kv_indices,
                                                w.out_cache_loc, w.custom_mask, w.mask_indptr, w.sm_scale,
                                                w.num_draft, ns)
    d = Device(w, nsplit=ns)
    T, H = w.num_draft, w.num_heads
    for algo in (ROWS, MFMA, SCALAR):
        d.ws.fill_(float("nan"))
        binding.verify_partials(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc,
                                d.custom_mask, d.mask_indptr, w.sm_scale, ns, d.ws, w.num_draft, algo=algo)
        torch.cuda.synchronize()
        o_ws, l_ws = binding.workspace_views(d.ws, w.batch, T, H, ns, binding.BF16)
        o_ws, l_ws = o_ws.float().cpu().numpy().astype(np.float64), l_ws.cpu().numpy().astype(np.float64)
        for b in range(w.batch):
            for s in range(ns):
                got_o = o_ws[b, s].reshape(T, H, 512)
                got_l = l_ws[b, s].reshape(T, H)
                if not nonempty[b, s]:
                    assert np.isnan(got_l).all(), "an empty split wrote to the workspace"
                    continue
                ro = o_ref[b * T:(b + 1) * T, :, s]
                rl = l_ref[b * T:(b + 1) * T, :, s]
                assert (np.isneginf(got_l) == np.isneginf(rl)).all()
                fin = np.isfinite(rl)
                assert np.all(np.abs(got_l[fin] - rl[fin]) <= 1e-3)
                assert np.all(np.abs(got_o - ro) <= 2e-2 + 2e-2 * np.abs(ro)), (b, s)


def test_combine_entry_point():
    """tvmla_combine on synthetic partials (some splits at -inf, one row all -inf),
    fp32 partials for an fp32 output and bf16 partials for a bf16 output."""
    batch, T, H, ns = 2, 3, 4, 5
    g = torch.Generator().manual_seed(3)
    nbytes = binding.workspace_bytes(batch, T, H, ns)
    o_src = torch.randn((batch, ns, T * H, 512), generator=g)
    l_src = torch.randn((batch, ns, T * H), generator=g) * 3
    l_src[0, 1] = float("-inf")
    l_src[1, :, 5] = float("-inf")
    for dt, code, tol in ((torch.float32, binding.FP32, 1e-5), (torch.bfloat16, binding.BF16, 1e-2)):
        ws = torch.zeros(nbytes // 4, dtype=torch.float32)
        o_v, l_v = binding.workspace_views(ws, batch, T, H, ns, code)
        o_v.copy_(o_src.to(o_v.dtype))
        l_v.copy_(l_src)
        o_ref = o_v.float().permute(0, 2, 1, 3).reshape(batch * T, H, ns, 512).numpy()
        l_ref = l_v.permute(0, 2, 1).reshape(batch * T, H, ns).numpy()
        ref_out, ref_lse = vo.combine(o_ref, l_ref)
        wsd = ws.cuda()
        out = torch.full((batch * T, H, 512), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((batch * T, H), float("nan"), device="cuda")
        binding.combine(wsd, None, batch, T, H, ns, out, lse)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        assert np.all(np.abs(o - ref_out) <= tol + tol * np.abs(ref_out))
        lg = lse.cpu().numpy()
        assert (np.isneginf(lg) == np.isneginf(ref_lse)).all()
        fin = np.isfinite(ref_lse)
        assert np.all(np.abs(lg[fin] - ref_lse[fin]) <= 1e-5)
        assert np.all(o[~fin] == 0)


def test_deterministic_and_poison_free():
    w = gen.build(SMALL["groups_h64"])
    d = Device(w)
    for algo in (ROWS, MFMA, SCALAR):
        o1, l1 = d.result(algo=algo)
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        d.ws.fill_(float("nan"))
        for _ in range(5):
            o2, l2 = d.result(algo=algo)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_slot_layout_bitwise():
    """Scattered vs contiguous slots (and a padded cache row stride): same bits."""
    a = gen.build(gen.small("lay", 2, [333, 70], 8, 16, seed=21))
    b = gen.build(gen.small("lay", 2, [333, 70], 8, 16, seed=21, layout="contiguous"))
    assert not np.array_equal(a.slots, b.slots)
    da, db, dp = Device(a), Device(b), Device(a, row_stride=640)
    for algo in (ROWS, MFMA, SCALAR):
        oa, la = da.result(algo=algo)
        ob, lb = db.result(algo=algo)
        op, lp = dp.result(algo=algo)
        assert np.array_equal(oa, ob) and np.array_equal(la, lb)
        assert np.array_equal(oa, op) and np.array_equal(la, lp)


def test_masked_content_independence():
    w = gen.build(gen.small("mask", 1, [150], 12, 8, seed=31))
    d = Device(w)
    T, P, H = w.num_draft, int(w.prefix_lens[0]), w.num_heads
    N = P + T
    vis = w.custom_mask.reshape(T, N).numpy() != 0
    leaf = max(range(T), key=lambda j: -vis[:, P + j].sum())  # seen by the fewest tokens
    for algo in (ROWS, MFMA, SCALAR):
        o1, l1 = d.result(algo=algo)
        saved = d.pool[int(w.out_cache_loc[leaf])].clone()
        d.pool[int(w.out_cache_loc[leaf])] = 37.0
        o2, l2 = d.result(algo=algo)
        d.pool[int(w.out_cache_loc[leaf])] = saved
        for i in range(T):
            rows = slice(i, i + 1)
            if not vis[i, P + leaf]:
                assert np.array_equal(o1[rows], o2[rows]) and np.array_equal(l1[rows], l2[rows])
            else:
                assert not np.array_equal(o1[rows], o2[rows])


def _convex_bounds(w, out):
    """Each output entry is a convex combination of the visible values, so it
    lies within [min, max] of the request's 512 latent entries (any size)."""
    for b in range(w.batch):
        sl = slice(int(w.row_offsets[b]), int(w.row_offsets[b + 1]))
        rows = w.rows[sl][:, :512].cuda().float()
        lo, hi = rows.min(0).values, rows.max(0).values
        o = out[b * w.num_draft:(b + 1) * w.num_draft].float()
        slack = 2e-2 + 2e-2 * torch.maximum(lo.abs(), hi.abs())
        assert torch.all(o >= lo - slack) and torch.all(o <= hi + slack), b


def _oracle_request(w, b, pool):
    """The oracle on request b alone: the batch's arrays restricted to its
    query rows, draft slots and its two offsets (kv_indptr and mask_indptr
    keep their absolute values, so they still index the whole arrays)."""
    T = w.num_draft
    rows = slice(b * T, (b + 1) * T)
    return vo.verify(w.q_nope[rows], w.q_rope[rows], pool, w.kv_indptr[b:b + 2], w.kv_indices,
                     w.out_cache_loc[rows], w.custom_mask, w.mask_indptr[b:b + 2], w.sm_scale, T)


def _both_calls(d, w):
    """The pages' call (tvmla_verify: exactly the workload's NSPLIT, kernel
    chosen automatically) and the tuned call (tvmla_verify_ex with
    TVMLA_FLAG_TUNE_NSPLIT, the one bench.py times); yields (label, out, lse)
    on the device."""
    binding.verify_plain(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc, d.custom_mask,
                         d.mask_indptr, w.sm_scale, d.nsplit, d.out, d.lse, d.ws, w.num_draft)
    torch.cuda.synchronize()
    yield f"tvmla_verify nsplit {d.nsplit}", d.out, d.lse
    eff = binding.effective_nsplit(w.batch, w.num_draft, w.num_heads, d.nsplit)
    d.out.fill_(float("nan"))
    d.lse.fill_(float("nan"))
    out, lse = d.run(flags=binding.TUNE_NSPLIT)
    torch.cuda.synchronize()
    yield f"tuned nsplit {d.nsplit}->{eff}", out, lse


@pytest.mark.parametrize("name", ["long185k", "long185k_h8", "ragged32"])
def test_full_size_whole(name):
    """The full-size workloads, every output row against the oracle, through
    both the pages' call and the tuned one."""
    w = gen.build(name)
    log(f"[{name}] built: batch={w.batch} keys={w.total_keys} rows={w.batch * w.num_draft * w.num_heads}")
    d = Device(w)
    ref_out, ref_lse = _oracle(w)
    log(f"[{name}] oracle done")
    for label, out, lse in _both_calls(d, w):
        _convex_bounds(w, out)
        got_o = out.float().cpu().numpy().astype(np.float64)
        got_l = lse.cpu().numpy().astype(np.float64)
        compare(w, got_o, got_l, ref_out, ref_lse, f"{name} {label}, all rows")


def test_full_size_heavy():
    """heavy200k (8 requests x 200,000 prefix keys x 32 draft tokens x 64
    heads): requests 0 and 7 whole against the oracle; every row within the
    convex bounds; scattered and contiguous slots bit-identical."""
    w = gen.build("heavy200k")
    log(f"[heavy200k] built: batch={w.batch} keys={w.total_keys}")
    d = Device(w)
    pool = w.host_pool()
    refs = {b: _oracle_request(w, b, pool) for b in (0, w.batch - 1)}
    log("[heavy200k] oracle done for requests " + ", ".join(map(str, refs)))
    T = w.num_draft
    results = []
    for label, out, lse in _both_calls(d, w):
        _convex_bounds(w, out)
        for b, (ro, rl) in refs.items():
            go = out[b * T:(b + 1) * T].float().cpu().numpy().astype(np.float64)
            gl = lse[b * T:(b + 1) * T].cpu().numpy().astype(np.float64)
            compare(w, go, gl, ro, rl, f"heavy200k {label}, request {b} whole")
        results.append((out.clone(), lse.clone()))
    del d
    c = gen.build("heavy200k_contig")
    dc = Device(c)
    for (o_s, l_s), (label, o_c, l_c) in zip(results, _both_calls(dc, c)):
        assert torch.equal(o_s, o_c) and torch.equal(l_s, l_c), f"{label}: scattered and contiguous slots differ"


@pytest.mark.parametrize("name", ["ragged_h8", "groups_h64", "t1_h1", "t64_h128", "fp32_ragged"])
def test_plain_verify_entry_point(name):
    """tvmla_verify itself (the pages' call, through ctypes): matches the
    oracle and is bit-identical to tvmla_verify_ex with AUTO, no flags and
    the default fold threshold."""
    w = gen.build(SMALL[name])
    ref_out, ref_lse = _oracle(w)
    d = Device(w)
    binding.verify_plain(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc, d.custom_mask,
                         d.mask_indptr, w.sm_scale, d.nsplit, d.out, d.lse, d.ws, w.num_draft)
    torch.cuda.synchronize()
    o1 = d.out.float().cpu().numpy().astype(np.float64)
    l1 = d.lse.cpu().numpy().astype(np.float64)
    compare(w, o1, l1, ref_out, ref_lse, f"{name}/tvmla_verify")
    o2, l2 = d.result()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_graph_capture_replay():
    """Capture one call, then change prefix lengths, trees and masks in place
    (same buffers, same capacity) and replay: every replay matches the oracle
    and the eager call."""
    T, H, ns = 8, 16, 64
    specs = [gen.small("cap", 2, [300, 500], T, H, seed=41), gen.small("cap", 2, [450, 120], T, H, seed=42),
             gen.small("cap", 2, [1, 799], T, H, tree="chain", seed=43)]
    ws_list = [gen.build(s) for s in specs]
    cap_idx = max(x.kv_indices.numel() for x in ws_list)
    cap_mask = max(x.custom_mask.numel() for x in ws_list)
    base = ws_list[0]
    d = Device(base)
    kv_indices = torch.zeros(cap_idx, dtype=torch.int32, device="cuda")
    mask = torch.zeros(cap_mask, dtype=torch.uint8, device="cuda")

    def load(x):
        kv_indices[:x.kv_indices.numel()].copy_(x.kv_indices.cuda())
        mask[:x.custom_mask.numel()].copy_(x.custom_mask.cuda())
        d.kv_indptr.copy_(x.kv_indptr.cuda())
        d.mask_indptr.copy_(x.mask_indptr.cuda())
        d.out_cache_loc.copy_(x.out_cache_loc.cuda())
        d.q_nope.copy_(x.q_nope.cuda())
        d.q_rope.copy_(x.q_rope.cuda())
        d.pool[torch.from_numpy(x.slots).cuda()] = x.rows.cuda()

    d.kv_indices, d.custom_mask = kv_indices, mask
    load(base)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        d.run()
    for rep in range(2):
        for x in ws_list:
            load(x)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            go, gl = d.out.float().cpu().numpy().astype(np.float64), d.lse.cpu().numpy().astype(np.float64)
            ro, rl = _oracle(x, d.pool.cpu())
            compare(x, go, gl, ro, rl, f"replay{rep}/P={list(x.prefix_lens)}")
            eo, el = d.result()  # eager, same buffers
            assert np.array_equal(go, eo) and np.array_equal(gl, el)


def _tuned_chunk(n, ns):
    """Keys per split of the tuned call: ceil(n / ns) rounded up to whole 64-key tiles."""
    return -(-(-(-n // ns)) // 64) * 64


@pytest.mark.parametrize("name,ns,eff_expected", [
    ("ragged_h8", 7, 112),   # 3 requests x 40 rows: 21 workgroups, raised to 336
    ("groups_h64", 32, 16),  # 2 requests x 8 row groups: 512 workgroups, lowered to one round of 256
    ("groups4_h64", 64, 16),  # 4 requests x 8 row groups: 2048 workgroups, halved to 512 (two rounds)
])
def test_effective_nsplit_matches_explicit(name, ns, eff_expected):
    """With TVMLA_FLAG_TUNE_NSPLIT the call runs the effective split count
    with chunks rounded up to whole 64-key tiles; it matches the oracle and
    is bit-identical to the split step and the combine at that count with
    TVMLA_FLAG_TILE_CHUNKS."""
    spec = SMALL[name] if name in SMALL else gen.small(name, 4, [40, 300, 0, 129], 16, 64, seed=19)
    w = gen.build(spec)
    eff = binding.effective_nsplit(w.batch, w.num_draft, w.num_heads, ns)
    assert eff == eff_expected
    ref_out, ref_lse = _oracle(w)
    d = Device(w, nsplit=ns)
    for algo in (binding.ALGO_AUTO, ROWS, MFMA):
        o1, l1 = d.result(algo=algo, flags=binding.TUNE_NSPLIT)
        compare(w, o1, l1, ref_out, ref_lse, f"{name}/nsplit{ns}->{eff}/algo{algo}")
        binding.verify_partials(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc,
                                d.custom_mask, d.mask_indptr, w.sm_scale, eff, d.ws, w.num_draft, algo=algo,
                                flags=binding.TILE_CHUNKS)
        binding.combine(d.ws, d.kv_indptr, w.batch, w.num_draft, w.num_heads, eff, d.out, d.lse,
                        flags=binding.TILE_CHUNKS)
        torch.cuda.synchronize()
        o2 = d.out.float().cpu().numpy().astype(np.float64)
        l2 = d.lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("algo", [ROWS, MFMA, SCALAR])
def test_tile_chunks_flag(algo):
    """TVMLA_FLAG_TILE_CHUNKS at the caller's split count (no tuning):
    matches the oracle and the split step + combine with the same flag."""
    w = gen.build(SMALL["ragged_h8"])
    ref_out, ref_lse = _oracle(w)
    d = Device(w, nsplit=7)
    o1, l1 = d.result(algo=algo, flags=binding.TILE_CHUNKS)
    compare(w, o1, l1, ref_out, ref_lse, f"ragged_h8/tile_chunks/algo{algo}")
    binding.verify_partials(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc, d.custom_mask,
                            d.mask_indptr, w.sm_scale, 7, d.ws, w.num_draft, algo=algo, flags=binding.TILE_CHUNKS)
    binding.combine(d.ws, d.kv_indptr, w.batch, w.num_draft, w.num_heads, 7, d.out, d.lse, flags=binding.TILE_CHUNKS)
    torch.cuda.synchronize()
    assert np.array_equal(o1, d.out.float().cpu().numpy().astype(np.float64))
    assert np.array_equal(l1, d.lse.cpu().numpy().astype(np.float64))


def test_tuned_call_writes_whole_tile_splits():
    """p4096 (4,112 keys) tuned to 32 splits: chunks of 192 keys (129 rounded
    up to three 64-key tiles), so splits 0..21 hold keys and 22..31 are empty
    and never written."""
    w = gen.build("p4096")
    d = Device(w)
    eff = binding.effective_nsplit(1, 16, 64, 64)
    assert eff == 32 and _tuned_chunk(4112, eff) == 192
    d.ws.fill_(float("nan"))
    d.run(flags=binding.TUNE_NSPLIT)
    torch.cuda.synchronize()
    _, l_ws = binding.workspace_views(d.ws, 1, 16, 64, eff, binding.BF16)
    l_ws = l_ws.cpu().numpy()
    assert np.isfinite(l_ws[0, :22]).all()
    assert np.isnan(l_ws[0, 22:]).all()


def test_partials_then_combine_equals_verify():
    w = gen.build(SMALL["groups_h64"])
    d = Device(w)
    # the full call runs exactly nsplit splits; the two steps take it as given
    ns = d.nsplit
    for algo in (ROWS, MFMA, SCALAR):
        o1, l1 = d.result(algo=algo)
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        d.ws.fill_(float("nan"))
        binding.verify_partials(d.q_nope, d.q_rope, d.pool, d.kv_indptr, d.kv_indices, d.out_cache_loc,
                                d.custom_mask, d.mask_indptr, w.sm_scale, ns, d.ws, w.num_draft, algo=algo)
        binding.combine(d.ws, d.kv_indptr, w.batch, w.num_draft, w.num_heads, ns, d.out, d.lse)
        torch.cuda.synchronize()
        o2 = d.out.float().cpu().numpy().astype(np.float64)
        l2 = d.lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
