"""Pins for the fp64 oracle (CPU only).

The pages print no numeric example of the attention itself, so the oracle is
pinned by: the pages' own split-schedule figures (tests/golden), an
independently written brute-force version, a library routine
(torch scaled_dot_product_attention in fp64), the textbook causal case, closed
forms (single visible key, zero query, constant values) and exact invariances
(split/combine identity, slot permutation, masked-content independence).
The sensitivity tests at the end plant mistakes in the oracle and check that
some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import verify_fp64 as vo
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _args(w, pool=None):
    pool = w.host_pool() if pool is None else pool
    return (w.q_nope, w.q_rope, pool, w.kv_indptr, w.kv_indices, w.out_cache_loc, w.custom_mask,
            w.mask_indptr, w.sm_scale, w.num_draft)


def _tiny(seed=3, batch=2, prefix=(5, 0), T=4, H=2, dtype="fp32", tree="random"):
    spec = gen.small("t", batch, list(prefix), T, H, dtype=dtype, tree=tree, pool_slots=256, seed=seed)
    return gen.build(spec)


# ---------------------------------------------------------------- schedule


def test_split_schedule_golden():
    with open(os.path.join(GOLDEN, "split_schedule.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        n, ns = c["kv_len"], c["nsplit"]
        ranges = [vo.split_range(n, ns, s) for s in range(ns)]
        assert ranges[0][1] - ranges[0][0] == c["chunk"]
        nonempty = [s for s, (a, b) in enumerate(ranges) if b > a]
        assert len(nonempty) == c["nonempty"]
        if c["first_empty"] is not None:
            assert nonempty == list(range(c["first_empty"]))
        # the splits tile [0, n) exactly, in order
        covered = [p for a, b in ranges for p in range(a, b)]
        assert covered == list(range(n))


def test_workspace_size_golden():
    with open(os.path.join(GOLDEN, "split_schedule.json")) as f:
        w = json.load(f)["workspace"]
    got = vo.workspace_bytes_fp32(w["batch"], w["num_draft"], w["num_heads"], w["nsplit"])
    assert abs(got - w["approx_bytes"]) <= w["rel_tol"] * w["approx_bytes"]
    # with 8 heads (one tensor-parallel share) it would be 8x smaller: the
    # page's figure fixes 64 heads
    got8 = vo.workspace_bytes_fp32(w["batch"], w["num_draft"], 8, w["nsplit"])
    assert abs(got8 - w["approx_bytes"]) > w["rel_tol"] * w["approx_bytes"]


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("seed,prefix,T,H,dtype,tree", [
    (1, (5, 0), 4, 2, "fp32", "random"),
    (2, (3, 7), 3, 1, "bf16", "random"),
    (3, (6,), 5, 2, "bf16", "chain"),
    (4, (0, 2, 4), 1, 3, "fp32", "random"),
])
def test_brute_matches_vectorised(seed, prefix, T, H, dtype, tree):
    w = _tiny(seed=seed, batch=len(prefix), prefix=prefix, T=T, H=H, dtype=dtype, tree=tree)
    args = _args(w)
    out, lse = vo.verify(*args)
    bo, bl = brute.verify_brute(*args)
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- library routine


def _sdpa_reference(w, pool):
    """torch SDPA (math path, fp64, CPU) with an explicit boolean mask; value
    width 512 differs from key width 576."""
    T, H = w.num_draft, w.num_heads
    outs, lses = [], []
    for b in range(w.batch):
        slots = torch.from_numpy(vo.key_slots(w.kv_indptr, w.kv_indices, w.out_cache_loc, b, T))
        k = pool[slots][:, :576].to(torch.float64)
        N = k.shape[0]
        st = int(w.mask_indptr[b])
        vis = w.custom_mask[st:st + T * N].reshape(T, N).bool()
        q = torch.cat([w.q_nope[b * T:(b + 1) * T], w.q_rope[b * T:(b + 1) * T]], dim=-1).to(torch.float64)
        q = q.permute(1, 0, 2)  # [H, T, 576]
        kk = k.unsqueeze(0).expand(H, N, 576)
        vv = k[:, :512].unsqueeze(0).expand(H, N, 512)
        mask = vis.unsqueeze(0).expand(H, T, N)
        o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=w.sm_scale)
        s = (q @ kk.transpose(1, 2)) * w.sm_scale
        s = s.masked_fill(~mask, float("-inf"))
        outs.append(o.permute(1, 0, 2))
        lses.append(torch.logsumexp(s, dim=-1).permute(1, 0))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


@pytest.mark.parametrize("seed,prefix,T,H,tree", [
    (11, (37, 5), 6, 4, "random"),
    (12, (64,), 16, 3, "random"),
    (13, (9, 0, 30), 8, 2, "chain"),
])
def test_sdpa_library(seed, prefix, T, H, tree):
    w = _tiny(seed=seed, batch=len(prefix), prefix=prefix, T=T, H=H, dtype="bf16", tree=tree)
    pool = w.host_pool()
    out, lse = vo.verify(*_args(w, pool))
    ro, rl = _sdpa_reference(w, pool)
    np.testing.assert_allclose(out, ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- textbook causal


def test_chain_equals_causal():
    """A chain tree is ordinary causal attention over [prefix; drafts]: draft i
    sits at sequence position P + i and sees positions 0..P+i."""
    P, T, H = 23, 6, 3
    w = _tiny(seed=21, batch=1, prefix=(P,), T=T, H=H, dtype="bf16", tree="chain")
    pool = w.host_pool()
    out, lse = vo.verify(*_args(w, pool))
    keys = w.request_rows(0).to(torch.float64)  # [N, 576] in logical order
    N = keys.shape[0]
    g = torch.Generator().manual_seed(5)
    qseq = torch.randn(H, N, 576, generator=g, dtype=torch.float64)
    qd = torch.cat([w.q_nope, w.q_rope], dim=-1).to(torch.float64)  # [T, H, 576]
    qseq[:, P:] = qd.permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qseq, keys.expand(H, N, 576), keys[:, :512].expand(H, N, 512), is_causal=True, scale=w.sm_scale)
    np.testing.assert_allclose(out, ref[:, P:].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    # lse from an explicit causal sum over the first P+i+1 positions
    for i in range(T):
        for h in range(H):
            s = (keys[:P + i + 1] @ qseq[h, P + i]).numpy() * w.sm_scale
            assert lse[i, h] == pytest.approx(vo.lse_natural(s), rel=1e-12, abs=1e-12)


# ---------------------------------------------------------------- closed forms


def test_single_visible_key():
    w = _tiny(seed=31, batch=2, prefix=(7, 4), T=3, H=2, dtype="fp32")
    # rewrite the mask: row i of request b sees only key (3*b + 2*i) % N_b
    cm = w.custom_mask.clone()
    picks = {}
    for b in range(w.batch):
        N = int(w.prefix_lens[b]) + w.num_draft
        st = int(w.mask_indptr[b])
        for i in range(w.num_draft):
            k = (3 * b + 2 * i) % N
            cm[st + i * N: st + (i + 1) * N] = 0
            cm[st + i * N + k] = 1
            picks[(b, i)] = k
    w.custom_mask = cm
    pool = w.host_pool()
    out, lse = vo.verify(*_args(w, pool))
    for (b, i), k in picks.items():
        row = w.request_rows(b)[k].to(torch.float64).numpy()
        t = b * w.num_draft + i
        for h in range(w.num_heads):
            np.testing.assert_array_equal(out[t, h], row[:512])
            s = w.sm_scale * (float(np.dot(w.q_nope[t, h].double().numpy(), row[:512]))
                              + float(np.dot(w.q_rope[t, h].double().numpy(), row[512:])))
            assert lse[t, h] == pytest.approx(s, rel=1e-13, abs=1e-13)


def test_zero_query_is_mean_of_visible():
    w = _tiny(seed=41, batch=2, prefix=(10, 3), T=5, H=2, dtype="bf16")
    w.q_nope = torch.zeros_like(w.q_nope)
    w.q_rope = torch.zeros_like(w.q_rope)
    pool = w.host_pool()
    out, lse = vo.verify(*_args(w, pool))
    for b in range(w.batch):
        N = int(w.prefix_lens[b]) + w.num_draft
        st = int(w.mask_indptr[b])
        vals = w.request_rows(b)[:, :512].to(torch.float64).numpy()
        for i in range(w.num_draft):
            vis = w.custom_mask[st + i * N: st + (i + 1) * N].numpy() != 0
            t = b * w.num_draft + i
            np.testing.assert_allclose(out[t], np.broadcast_to(vals[vis].mean(axis=0), out[t].shape),
                                       rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[t], math.log(vis.sum()), rtol=1e-14)


def test_constant_values():
    w = _tiny(seed=51, batch=1, prefix=(12,), T=4, H=3, dtype="fp32")
    c = torch.randn(512, generator=torch.Generator().manual_seed(1))
    w.rows[:, :512] = c
    out, _ = vo.verify(*_args(w))
    np.testing.assert_allclose(out, np.broadcast_to(c.double().numpy(), out.shape), rtol=1e-12, atol=1e-12)


def test_empty_row_reading():
    """A row that sees no key: out = 0, lse = -inf (reading of an unreachable case)."""
    w = _tiny(seed=61, batch=1, prefix=(4,), T=2, H=1, dtype="fp32")
    N = 4 + 2
    cm = w.custom_mask.clone()
    cm[:N] = 0  # token 0 sees nothing
    w.custom_mask = cm
    out, lse = vo.verify(*_args(w))
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------- invariances


@pytest.mark.parametrize("nsplit", [1, 3, 7, 64, 200])
def test_split_combine_identity(nsplit):
    w = _tiny(seed=71, batch=3, prefix=(40, 0, 17), T=5, H=2, dtype="bf16")
    args = _args(w)
    out, lse = vo.verify(*args)
    op, lp, ne = vo.verify_partials(*args, nsplit=nsplit)
    co, cl = vo.combine(op, lp)
    np.testing.assert_allclose(co, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cl, lse, rtol=1e-13, atol=1e-13)
    for b in range(w.batch):
        n = int(w.prefix_lens[b]) + w.num_draft
        chunk = -(-n // nsplit)
        assert ne[b].sum() == -(-n // chunk)  # ceil(n / chunk) splits hold keys


def test_slot_permutation_is_exact():
    w = _tiny(seed=81, batch=2, prefix=(30, 11), T=4, H=2, dtype="bf16")
    out1, lse1 = vo.verify(*_args(w))
    w2 = gen.build(gen.small("t", 2, [30, 11], 4, 2, dtype="bf16", pool_slots=256, layout="contiguous", seed=81))
    out2, lse2 = vo.verify(*_args(w2))
    assert not np.array_equal(w.slots, w2.slots)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_prefix_permutation_invariant():
    w = _tiny(seed=91, batch=1, prefix=(33,), T=4, H=2, dtype="bf16")
    out1, lse1 = vo.verify(*_args(w))
    P, T = 33, 4
    N = P + T
    perm = np.random.default_rng(0).permutation(P)
    w.kv_indices = w.kv_indices[torch.from_numpy(perm)]
    m = w.custom_mask.reshape(T, N).clone()
    m[:, :P] = m[:, torch.from_numpy(perm)]
    w.custom_mask = m.reshape(-1)
    out2, lse2 = vo.verify(*_args(w))
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-13, atol=1e-13)


def test_masked_content_independence():
    w = _tiny(seed=101, batch=1, prefix=(9,), T=6, H=2, dtype="fp32")
    pool = w.host_pool()
    out1, lse1 = vo.verify(*_args(w, pool))
    P, T = 9, 6
    N = P + T
    vis = w.custom_mask.reshape(T, N).numpy() != 0
    j = T - 1  # last draft node: a leaf, seen only by itself
    assert vis[:, P + j].sum() >= 1
    pool2 = pool.clone()
    pool2[int(w.out_cache_loc[j])] = 1000.0
    out2, lse2 = vo.verify(*_args(w, pool2))
    for i in range(T):
        if not vis[i, P + j]:
            np.testing.assert_array_equal(out1[i], out2[i])
            np.testing.assert_array_equal(lse1[i], lse2[i])
        else:
            assert not np.array_equal(out1[i], out2[i])


# ---------------------------------------------------------------- sensitivity


def _pins_fail(monkeypatch, attr, fn):
    """Plant a mistake in the oracle and report which pins still hold."""
    monkeypatch.setattr(vo, attr, fn)
    fails = []
    for name, check in [("brute", _check_brute), ("sdpa", _check_sdpa), ("causal", _check_causal),
                        ("split", _check_split)]:
        try:
            check()
        except AssertionError:
            fails.append(name)
    return fails


def _check_brute():
    w = _tiny(seed=2, batch=2, prefix=(3, 7), T=3, H=1, dtype="bf16")
    args = _args(w)
    out, lse = vo.verify(*args)
    bo, bl = brute.verify_brute(*args)
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-9, atol=1e-9)


def _check_sdpa():
    w = _tiny(seed=11, batch=2, prefix=(37, 5), T=6, H=2, dtype="bf16")
    pool = w.host_pool()
    out, lse = vo.verify(*_args(w, pool))
    ro, rl = _sdpa_reference(w, pool)
    np.testing.assert_allclose(out, ro, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(lse, rl, rtol=1e-9, atol=1e-9)


def _check_causal():
    test_chain_equals_causal()


def _check_split():
    w = _tiny(seed=71, batch=2, prefix=(40, 0), T=5, H=1, dtype="bf16")
    args = _args(w)
    out, lse = vo.verify(*args)
    op, lp, _ = vo.verify_partials(*args, nsplit=7)
    co, cl = vo.combine(op, lp)
    np.testing.assert_allclose(co, out, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(cl, lse, rtol=1e-9, atol=1e-9)


_real_attend = vo.attend
_real_slots = vo.key_slots
_real_vis = vo.visibility
_real_split = vo.split_range


def _attend_no_rope(qn, qr, keys, vis, sm):
    return _real_attend(qn, qr * 0.0, keys, vis, sm)


def _attend_no_mask(qn, qr, keys, vis, sm):
    return _real_attend(qn, qr, keys, np.ones_like(vis), sm)


def _attend_wrong_scale(qn, qr, keys, vis, sm):
    return _real_attend(qn, qr, keys, vis, sm * 1.01)


def _attend_value_includes_rope_shift(qn, qr, keys, vis, sm):
    k2 = keys.copy()
    k2[:, :512] = np.roll(keys[:, :512], 1, axis=1)  # transposed/shifted value columns
    o, l = _real_attend(qn, qr, keys, vis, sm)
    o2, _ = _real_attend(qn, qr, k2, vis, sm)
    return o2, l


def _slots_drafts_from_prefix(ip, idx, ocl, b, T):
    s = _real_slots(ip, idx, ocl, b, T)
    P = len(s) - T
    if P > 0:
        s[P:] = s[np.arange(T) % P]
    return s


def _vis_transposed(cm, mi, b, T, N):
    st = int(vo._i64(mi)[b])
    flat = cm.detach().cpu().numpy() if hasattr(cm, "detach") else np.asarray(cm)
    return flat[st:st + T * N].reshape(N, T).T != 0


def _split_drops_last(n, ns, s):
    a, b = _real_split(n, ns, s)
    return (a, max(a, b - 1)) if b - a > 1 else (a, b)


@pytest.mark.parametrize("attr,fn", [
    ("attend", _attend_no_rope),
    ("attend", _attend_no_mask),
    ("attend", _attend_wrong_scale),
    ("attend", _attend_value_includes_rope_shift),
    ("key_slots", _slots_drafts_from_prefix),
    ("visibility", _vis_transposed),
    ("split_range", _split_drops_last),
])
def test_planted_mistakes_are_caught(monkeypatch, attr, fn):
    fails = _pins_fail(monkeypatch, attr, fn)
    assert fails, f"planted mistake in {attr} ({fn.__name__}) passed every pin"


# ---------------------------------------------------------------- row picks and request slices
#
# verify_rows (the oracle of chosen (token, head) rows) has its own indexing:
# it groups the picks by request (t // T), takes token t's query and the mask
# row t - b*T. It is pinned against the brute-force oracle directly, over
# several requests (b > 0), the first and last token and head, picks in
# scrambled order with repeats; planted indexing mistakes must fail that pin.


def _row_picks(w):
    T, H = w.num_draft, w.num_heads
    picks = []
    for b in range(w.batch):
        picks += [(b * T, 0), (b * T + T - 1, H - 1), (b * T + T // 2, H // 2), (b * T, H - 1)]
    rng = np.random.default_rng(0)
    picks += [picks[i] for i in rng.permutation(len(picks))[:3]]  # repeats
    return [picks[i] for i in rng.permutation(len(picks))]


def _check_rows_against_brute(rows_fn):
    w = _tiny(seed=51, batch=3, prefix=(6, 0, 11), T=4, H=3, dtype="bf16")
    args = _args(w)
    picks = _row_picks(w)
    out, lse = rows_fn(*args, picks)
    bo, bl = brute.verify_brute(*args)
    for k, (t, h) in enumerate(picks):
        np.testing.assert_allclose(out[k], np.array(bo[t][h]), rtol=1e-12, atol=1e-12)
        assert lse[k] == pytest.approx(bl[t][h], rel=1e-12, abs=1e-12)


def test_verify_rows_matches_brute():
    _check_rows_against_brute(vo.verify_rows)


def test_verify_rows_matches_verify_medium():
    """A medium bf16 case (ragged prefixes, 16 heads): every pick equals the
    whole-batch oracle's row."""
    w = gen.build(gen.small("rows", 3, [300, 17, 1000], 8, 16, pool_slots=4096, seed=52))
    args = _args(w)
    out, lse = vo.verify(*args)
    picks = _row_picks(w)
    ro, rl = vo.verify_rows(*args, picks)
    for k, (t, h) in enumerate(picks):
        np.testing.assert_allclose(ro[k], out[t, h], rtol=1e-12, atol=1e-12)
        assert rl[k] == pytest.approx(lse[t, h], rel=1e-12, abs=1e-12)


def _rows_variant(mistake):
    """verify_rows with one plausible indexing mistake planted."""

    def rows(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr, sm_scale,
             num_draft, picks):
        T = num_draft
        out = np.zeros((len(picks), vo.D_LATENT))
        lse = np.zeros(len(picks))
        for k, (t, h) in enumerate(picks):
            b = t // T
            kb = (b + 1) % (len(vo._i64(kv_indptr)) - 1) if mistake == "keys_of_next_request" else b
            slots = vo.key_slots(kv_indptr, kv_indices, out_cache_loc, kb, T)
            keys = vo.request_keys(kv_cache, slots)
            vis = vo.visibility(custom_mask, mask_indptr, kb, T, len(slots))
            i = {"mask_row_first": 0, "mask_row_global": t % vis.shape[0] if b == 0 else (t + 1) % T}.get(
                mistake, t - b * T)
            hq = 0 if mistake == "head_zero" else h
            qn = vo._f64(q_nope[t, hq])[None]
            qr = vo._f64(q_rope[t, hq])[None]
            o, ls = vo.attend(qn, qr, keys, vis[i][None], sm_scale)
            out[k], lse[k] = o[0], ls[0]
        return out, lse

    return rows


def test_rows_variant_without_mistake_passes():
    _check_rows_against_brute(_rows_variant("none"))


@pytest.mark.parametrize("mistake", ["keys_of_next_request", "mask_row_first", "mask_row_global", "head_zero"])
def test_rows_planted_mistakes_are_caught(mistake):
    with pytest.raises(AssertionError):
        _check_rows_against_brute(_rows_variant(mistake))


def test_request_slice_equals_whole_batch():
    """The oracle run on one request's slice of the batch arrays (its query
    rows and draft slots, kv_indptr[b:b+2] and mask_indptr[b:b+2] keeping
    their absolute offsets) equals that request's rows of the whole-batch
    oracle: the GPU tests check whole requests of the largest workload this
    way."""
    w = _tiny(seed=53, batch=3, prefix=(40, 0, 75), T=5, H=4, dtype="bf16")
    pool = w.host_pool()
    out, lse = vo.verify(*_args(w, pool))
    T = w.num_draft
    for b in range(w.batch):
        rows = slice(b * T, (b + 1) * T)
        o, l = vo.verify(w.q_nope[rows], w.q_rope[rows], pool, w.kv_indptr[b:b + 2], w.kv_indices,
                         w.out_cache_loc[rows], w.custom_mask, w.mask_indptr[b:b + 2], w.sm_scale, T)
        np.testing.assert_array_equal(o, out[rows])
        np.testing.assert_array_equal(l, lse[rows])
