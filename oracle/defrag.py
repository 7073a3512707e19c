"""CPU oracle for KV-cache defragmentation (compaction of a request's prefix rows).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module; the product path never does,
and this module imports nothing from the product package.

The pages name the step and its reason, not its interface: page_size = 1
paging scatters a request's cache rows over the pool, so reading them is a
gather of isolated rows ("The Plan Document: A Pivot Point in Custom CUDA
Kernel Development", section "Context: The Bottleneck That Demanded a Custom
Kernel"), and the plan's last phase is KV defragmentation (same page, section
"Output Knowledge Created"). The reading taken here, since they give no interface:

  for each request b, prefix position p in [0, P_b), P_b = kv_indptr[b+1] -
  kv_indptr[b]:
      dst_slot          = dst_base[b] + p
      kv_dst[dst_slot]  = kv_src[kv_indices[kv_indptr[b] + p]]   (576 entries)
      new_indices[kv_indptr[b] + p] = dst_slot

Draft rows (out_cache_loc) are not moved. Destination runs of different
requests must not overlap each other or any source row of the same call;
the caller picks them.
"""
from __future__ import annotations

import numpy as np

D_KEY = 576


def defrag(kv_src: np.ndarray, kv_dst: np.ndarray, kv_indptr, kv_indices, dst_base):
    """Return (kv_dst with the compacted rows written, new kv_indices).

    kv_src, kv_dst: [slots, >=576] arrays (kv_dst is copied, not modified);
    only the first 576 entries of a row move. kv_indptr [batch+1],
    kv_indices [kv_indptr[batch]], dst_base [batch]: integer arrays.
    """
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    idx = np.asarray(kv_indices, dtype=np.int64)
    base = np.asarray(dst_base, dtype=np.int64)
    out = np.array(kv_dst, copy=True)
    new_idx = idx.copy()
    for b in range(len(indptr) - 1):
        for p in range(int(indptr[b + 1] - indptr[b])):
            j = int(indptr[b]) + p
            d = int(base[b]) + p
            out[d, :D_KEY] = kv_src[int(idx[j]), :D_KEY]
            new_idx[j] = d
    return out, new_idx.astype(np.int32)
