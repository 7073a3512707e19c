"""fp64 CPU oracle for tree-verify attention over an MLA latent KV cache.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module; the product path never does,
and this module imports nothing from the product package.

What it computes is the plain definition of masked softmax attention, in
fp64, per (request, draft token, head):

  keys of request b      prefix tokens through kv_indices[kv_indptr[b] :
                         kv_indptr[b+1]], then the request's draft tokens
                         through out_cache_loc ("The Architecture of Capture
                         Safety", "The Design Emerges", second and fourth
                         insights);
  key vector             the full 576-wide cache row (512-wide latent, shared
                         by every head, then the 64-wide rope part); value
                         vector = the 512-wide latent ("The Plan Document",
                         "The Design Reasoning": one latent vector per token
                         serves all heads);
  visibility             custom_mask bytes at mask_indptr[b], one row of
                         (prefix + draft) columns per draft token ("The
                         Architecture of Capture Safety", "The Design
                         Emerges", third insight; which draft token sees
                         which key: same page, "Input Knowledge Required",
                         DDTree paragraph);
  score                  sm_scale * (q_nope . latent + q_rope . rope);
  result                 out = softmax-weighted mean of the visible values,
                         lse = natural log of the sum of exp(score) over the
                         visible keys.

The split-K form (partials per key range, then a log-sum-exp merge; "The
Architecture of Capture Safety", "The Design Emerges", first insight, and
"The NSPLIT Calculation") reaches the same result exactly up to rounding;
`split_range`, `verify_partials` and `combine` write that schedule out so
tests can check the identity.

Readings of points the pages leave open:
  * kv_indptr spans the prefix only; the T draft tokens follow it, so a
    request has N_b = P_b + T keys in the order prefix, then draft nodes.
  * The mask row for draft token i of request b starts at
    mask_indptr[b] + i * N_b and has N_b bytes; nonzero means visible.
  * sm_scale multiplies the whole 576-wide dot product; inputs are post-rope.
  * A row that sees no key has out = 0 and lse = -inf.
  * chunk = ceil(N_b / nsplit) over prefix plus draft keys; split s covers
    [s*chunk, min((s+1)*chunk, N_b)) and is empty when that range is.
"""
from __future__ import annotations

import math

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_KEY = D_LATENT + D_ROPE


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16/fp32/fp64) or array to float64."""
    if hasattr(x, "detach"):
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def key_slots(kv_indptr, kv_indices, out_cache_loc, b: int, num_draft: int) -> np.ndarray:
    """Pool slot of each of request b's N_b keys: prefix via kv_indices, then
    drafts via out_cache_loc ("The Architecture of Capture Safety", "The Design Emerges", second insight)."""
    ip = _i64(kv_indptr)
    prefix = _i64(kv_indices)[ip[b]:ip[b + 1]]
    drafts = _i64(out_cache_loc)[b * num_draft:(b + 1) * num_draft]
    return np.concatenate([prefix, drafts])


def visibility(custom_mask, mask_indptr, b: int, num_draft: int, n_keys: int) -> np.ndarray:
    """Bool [T, N_b]: row i = draft token i, column p = key p of request b
    ("The Architecture of Capture Safety", "The Design Emerges", third insight)."""
    mi = _i64(mask_indptr)
    flat = _i64(custom_mask) if not hasattr(custom_mask, "detach") else custom_mask.detach().cpu().numpy()
    start = int(mi[b])
    return np.asarray(flat[start:start + num_draft * n_keys]).reshape(num_draft, n_keys) != 0


def attend(qn: np.ndarray, qr: np.ndarray, keys: np.ndarray, vis: np.ndarray, sm_scale: float):
    """Masked softmax attention for a set of query rows against one request's keys.

    qn [R, 512], qr [R, 64], keys [N, 576], vis [R, N] bool, all fp64.
    Returns out [R, 512] and lse [R] (natural log).
    """
    s = sm_scale * (qn @ keys[:, :D_LATENT].T + qr @ keys[:, D_LATENT:].T)
    s = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
    w = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = w.sum(axis=1)
    safe_l = np.where(any_vis, l, 1.0)
    out = (w @ keys[:, :D_LATENT]) / safe_l[:, None]
    lse = np.where(any_vis, m + np.log(safe_l), -np.inf)
    out[~any_vis] = 0.0
    return out, lse


def request_keys(kv_cache, slots: np.ndarray) -> np.ndarray:
    """Gather the 576-wide key rows of the given slots from the cache, as fp64."""
    import torch

    if isinstance(kv_cache, torch.Tensor):
        rows = kv_cache[torch.from_numpy(slots)][:, :D_KEY]
        return _f64(rows)
    return np.asarray(kv_cache[slots][:, :D_KEY], dtype=np.float64)


def verify(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask,
           mask_indptr, sm_scale: float, num_draft: int, row_block: int = 256):
    """Whole-batch oracle. q_* are [batch*T, H, d]; returns out [batch*T, H, 512]
    and lse [batch*T, H], both fp64."""
    qn_all = _f64(q_nope)
    qr_all = _f64(q_rope)
    ntok, H, _ = qn_all.shape
    T = num_draft
    bs = ntok // T
    out = np.zeros((ntok, H, D_LATENT))
    lse = np.zeros((ntok, H))
    for b in range(bs):
        slots = key_slots(kv_indptr, kv_indices, out_cache_loc, b, T)
        keys = request_keys(kv_cache, slots)
        vis = visibility(custom_mask, mask_indptr, b, T, len(slots))
        qn = qn_all[b * T:(b + 1) * T].reshape(T * H, D_LATENT)
        qr = qr_all[b * T:(b + 1) * T].reshape(T * H, D_ROPE)
        row_vis = np.repeat(vis, H, axis=0)  # row r = i*H + h sees what token i sees
        o = np.empty((T * H, D_LATENT))
        ls = np.empty(T * H)
        for r0 in range(0, T * H, row_block):
            r1 = min(r0 + row_block, T * H)
            o[r0:r1], ls[r0:r1] = attend(qn[r0:r1], qr[r0:r1], keys, row_vis[r0:r1], sm_scale)
        out[b * T:(b + 1) * T] = o.reshape(T, H, D_LATENT)
        lse[b * T:(b + 1) * T] = ls.reshape(T, H)
    return out, lse


def verify_ragged(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                  mask_indptr, qo_indptr, sm_scale: float):
    """Oracle for draft trees of different sizes: request b owns query tokens
    qo_indptr[b] .. qo_indptr[b+1]-1 (T_b of them; the int64 token offsets of
    "The Architecture of Capture Safety", "Input Knowledge Required"), its draft keys are out_cache_loc at
    the same positions, its mask block is [T_b][P_b + T_b] at mask_indptr[b].
    Returns out [qo_indptr[-1], H, 512] and lse [qo_indptr[-1], H], fp64."""
    qn_all = _f64(q_nope)
    qr_all = _f64(q_rope)
    qo = _i64(qo_indptr)
    ip = _i64(kv_indptr)
    ocl = _i64(out_cache_loc)
    H = qn_all.shape[1]
    ntok = int(qo[-1])
    out = np.zeros((ntok, H, D_LATENT))
    lse = np.zeros((ntok, H))
    for b in range(len(qo) - 1):
        t0, t1 = int(qo[b]), int(qo[b + 1])
        Tb = t1 - t0
        if Tb == 0:
            continue
        slots = np.concatenate([_i64(kv_indices)[ip[b]:ip[b + 1]], ocl[t0:t1]])
        keys = request_keys(kv_cache, slots)
        vis = visibility(custom_mask, mask_indptr, b, Tb, len(slots))
        qn = qn_all[t0:t1].reshape(Tb * H, D_LATENT)
        qr = qr_all[t0:t1].reshape(Tb * H, D_ROPE)
        o, ls = attend(qn, qr, keys, np.repeat(vis, H, axis=0), sm_scale)
        out[t0:t1] = o.reshape(Tb, H, D_LATENT)
        lse[t0:t1] = ls.reshape(Tb, H)
    return out, lse


def verify_rows(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                mask_indptr, sm_scale: float, num_draft: int, picks):
    """Oracle for selected (token, head) pairs only, for spot checks at full size.

    picks: iterable of (t, h) with t the flat draft-token index (b*T + i).
    Returns out [len(picks), 512] and lse [len(picks)].
    """
    picks = list(picks)
    T = num_draft
    out = np.zeros((len(picks), D_LATENT))
    lse = np.zeros(len(picks))
    by_req = {}
    for k, (t, h) in enumerate(picks):
        by_req.setdefault(t // T, []).append((k, t, h))
    for b, items in sorted(by_req.items()):
        slots = key_slots(kv_indptr, kv_indices, out_cache_loc, b, T)
        keys = request_keys(kv_cache, slots)
        vis = visibility(custom_mask, mask_indptr, b, T, len(slots))
        qn = np.stack([_f64(q_nope[t, h]) for _, t, h in items])
        qr = np.stack([_f64(q_rope[t, h]) for _, t, h in items])
        rv = np.stack([vis[t - b * T] for _, t, _ in items])
        o, ls = attend(qn, qr, keys, rv, sm_scale)
        for j, (k, _, _) in enumerate(items):
            out[k] = o[j]
            lse[k] = ls[j]
    return out, lse


def split_range(n_keys: int, nsplit: int, s: int):
    """Key range [start, end) of split s: chunk = ceil(N / nsplit), split s
    starts at s*chunk; it is empty when start >= end ("The Architecture of Capture Safety", "The Design
    Emerges", first insight, and "The NSPLIT Calculation")."""
    chunk = -(-n_keys // nsplit) if n_keys > 0 else 0
    start = s * chunk
    end = min(start + chunk, n_keys)
    return start, max(start, end)


def verify_partials(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                    mask_indptr, sm_scale: float, num_draft: int, nsplit: int):
    """Per-split partial results: attention restricted to each split's key range.

    Returns o [batch*T, H, nsplit, 512] (normalised within the split),
    lse [batch*T, H, nsplit] (-inf where the split sees no key) and
    nonempty [batch, nsplit] bool.
    """
    qn_all = _f64(q_nope)
    qr_all = _f64(q_rope)
    ntok, H, _ = qn_all.shape
    T = num_draft
    bs = ntok // T
    o_parts = np.zeros((ntok, H, nsplit, D_LATENT))
    lse_parts = np.full((ntok, H, nsplit), -np.inf)
    nonempty = np.zeros((bs, nsplit), dtype=bool)
    for b in range(bs):
        slots = key_slots(kv_indptr, kv_indices, out_cache_loc, b, T)
        keys = request_keys(kv_cache, slots)
        n = len(slots)
        vis = visibility(custom_mask, mask_indptr, b, T, n)
        qn = qn_all[b * T:(b + 1) * T].reshape(T * H, D_LATENT)
        qr = qr_all[b * T:(b + 1) * T].reshape(T * H, D_ROPE)
        row_vis = np.repeat(vis, H, axis=0)
        for s in range(nsplit):
            lo, hi = split_range(n, nsplit, s)
            if lo >= hi:
                continue
            nonempty[b, s] = True
            o, ls = attend(qn, qr, keys[lo:hi], row_vis[:, lo:hi], sm_scale)
            o_parts[b * T:(b + 1) * T, :, s] = o.reshape(T, H, D_LATENT)
            lse_parts[b * T:(b + 1) * T, :, s] = ls.reshape(T, H)
    return o_parts, lse_parts, nonempty


def combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Log-sum-exp merge of per-split partials along the split axis (axis -2 of
    o_parts, axis -1 of lse_parts): weights exp(lse_s - max lse), out = weighted
    mean of the normalised partials, lse = max + log(sum of weights). Splits
    with lse_s = -inf weigh nothing; if every split is -inf the row is empty
    (out = 0, lse = -inf). This is the reduce step of "The Architecture of Capture Safety", "The Design
    Emerges", first insight."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=-1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[..., None]), 0.0)
    wsum = w.sum(axis=-1)
    wsum_safe = np.where(finite, wsum, 1.0)
    out = (w[..., None] * o_parts).sum(axis=-2) / wsum_safe[..., None]
    out = np.where(finite[..., None], out, 0.0)
    lse = np.where(finite, m_safe + np.log(wsum_safe), -np.inf)
    return out, lse


def workspace_bytes_fp32(batch: int, num_draft: int, num_heads: int, nsplit: int) -> int:
    """Bytes of fp32 split partials: a 512-wide output plus one lse per
    (token, head, split). Page 1, "Assumptions and Their Validity", puts this
    workspace at about 600 MB for batch 8 with 9 draft tokens and NSPLIT 64."""
    return batch * num_draft * num_heads * nsplit * (D_LATENT + 1) * 4


def lse_natural(x) -> float:
    """Natural log-sum-exp of a 1-D array (helper for tests)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return float(m + math.log(np.exp(x - m).sum()))
