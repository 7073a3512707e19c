"""Brute-force scalar oracle for tree-verify attention (tiny inputs only).

TEST INFRASTRUCTURE. Only tests/ may call this; it exists to pin the
vectorised fp64 oracle in verify_fp64.py with an independently written
pure-Python version: explicit loops over (request, draft token, head, key),
dot products and sums accumulated with math.fsum (exactly rounded), and the
same definition ("The Architecture of Capture Safety", "The Design Emerges": prefix keys through
kv_indices/kv_indptr, draft keys through out_cache_loc, mask through
custom_mask/mask_indptr; "The Plan Document", "The Design Reasoning": the 512-wide latent
is both the value and the first 512 key entries, shared by all heads).
It shares no code with verify_fp64.py.
"""
from __future__ import annotations

import math


def _tolist(x):
    if hasattr(x, "detach"):
        import torch

        x = x.detach().cpu()
        if x.dtype in (torch.bfloat16, torch.float16, torch.float32):
            x = x.to(torch.float64)
        return x.tolist()
    if hasattr(x, "tolist"):
        return x.tolist()
    return list(x)


def verify_brute(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                 mask_indptr, sm_scale, num_draft):
    """Returns (out, lse) as nested Python lists: out[t][h][d], lse[t][h]."""
    qn = _tolist(q_nope)
    qr = _tolist(q_rope)
    ip = [int(v) for v in _tolist(kv_indptr)]
    idx = [int(v) for v in _tolist(kv_indices)]
    ocl = [int(v) for v in _tolist(out_cache_loc)]
    mask = [int(v) for v in _tolist(custom_mask)]
    mip = [int(v) for v in _tolist(mask_indptr)]
    T = int(num_draft)
    bs = len(ip) - 1
    H = len(qn[0])
    dl = len(qn[0][0])
    dr = len(qr[0][0])

    cache_rows = {}

    def row(slot):
        if slot not in cache_rows:
            r = kv_cache[slot]
            cache_rows[slot] = [float(v) for v in _tolist(r)][: dl + dr]
        return cache_rows[slot]

    out = []
    lse = []
    for b in range(bs):
        P = ip[b + 1] - ip[b]
        N = P + T
        slots = [idx[ip[b] + p] if p < P else ocl[b * T + (p - P)] for p in range(N)]
        for i in range(T):
            t = b * T + i
            vis = [mask[mip[b] + i * N + p] != 0 for p in range(N)]
            out_t = []
            lse_t = []
            for h in range(H):
                scores = []
                for p in range(N):
                    if not vis[p]:
                        continue
                    k = row(slots[p])
                    terms = [qn[t][h][d] * k[d] for d in range(dl)]
                    terms += [qr[t][h][r] * k[dl + r] for r in range(dr)]
                    scores.append((p, sm_scale * math.fsum(terms)))
                if not scores:
                    out_t.append([0.0] * dl)
                    lse_t.append(-math.inf)
                    continue
                mx = max(s for _, s in scores)
                ws = [(p, math.exp(s - mx)) for p, s in scores]
                total = math.fsum(w for _, w in ws)
                o = [math.fsum(w * row(slots[p])[d] for p, w in ws) / total for d in range(dl)]
                out_t.append(o)
                lse_t.append(mx + math.log(total))
            out.append(out_t)
            lse.append(lse_t)
    return out, lse
