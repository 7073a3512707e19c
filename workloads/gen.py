"""Seeded synthetic workloads for tree-verify attention over an MLA latent cache.

Every input the verify call consumes is drawn here: query vectors, latent
cache rows, draft-tree shapes, page_size=1 slot choices, and the metadata
arrays (kv_indptr / kv_indices / out_cache_loc / custom_mask / mask_indptr)
in the layout the serving engine hands to its attention backend ("The Architecture of Capture Safety",
"The Design Emerges": the prefix is addressed through kv_indices and
kv_indptr, the draft tokens through out_cache_loc, and the visibility mask
through custom_mask plus mask_indptr).

Nothing here computes attention. Tree visibility ("a draft token sees the
whole prefix, its ancestors and itself", "The Architecture of Capture Safety", "Input Knowledge Required")
is input construction: it turns a parent array into mask bytes.

Draw order per workload (one numpy PCG64 stream, fixed seed):
  prefix lengths (ragged specs only) -> tree parents -> q_nope -> q_rope ->
  cache rows (logical order) -> slot choice.
Slots are drawn last so the scattered and contiguous variants of one spec
share every other value bit for bit.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Sequence, Union

import numpy as np
import torch

D_LATENT = 512  # MLA latent width: the value, and the first part of the key
D_ROPE = 64  # decoupled rope part of the key
D_KEY = D_LATENT + D_ROPE  # 576

_TORCH_DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}


@dataclass(frozen=True)
class Spec:
    """Shape and seed of one synthetic verify workload."""

    name: str
    batch: int
    prefix: Union[int, tuple, Sequence[int]]  # int, (lo, hi) uniform inclusive, or explicit list
    num_draft: int
    tree: str  # "random" (parent of i uniform in [0, i-1]) or "chain" (parent i-1)
    num_heads: int
    dtype: str  # "bf16" or "fp32"
    pool_slots: int
    layout: str  # "scattered", "contiguous" or "permutation"
    nsplit: int
    seed: int
    sm_scale: float = 1.0 / math.sqrt(192.0)


CONFIGS = {
    # tiny: one request, 21 prefix tokens, 4-node random tree, fp32, slots
    # from a random permutation of a 4096-slot pool
    "tiny": Spec("tiny", 1, 21, 4, "random", 64, "fp32", 4096, "permutation", 64, 1001),
    # one request, 4096-token prefix, 16-node random tree, 1M-slot pool
    "p4096": Spec("p4096", 1, 4096, 16, "random", 64, "bf16", 1 << 20, "scattered", 64, 1002),
    # long context: 185,000-token prefix, 16-node random tree, 2M-slot pool
    "long185k": Spec("long185k", 1, 185000, 16, "random", 64, "bf16", 1 << 21, "scattered", 64, 1003),
    # ragged batch: 32 requests, prefixes uniform in [1024, 32768], 8-token chain
    "ragged32": Spec("ragged32", 32, (1024, 32768), 8, "chain", 64, "bf16", 1 << 21, "scattered", 64, 1004),
    # heavy: 8 requests x 200,000 prefix, 32-node random tree; scattered vs contiguous
    "heavy200k": Spec("heavy200k", 8, 200000, 32, "random", 64, "bf16", 1 << 21, "scattered", 64, 1005),
    "heavy200k_contig": Spec("heavy200k_contig", 8, 200000, 32, "random", 64, "bf16", 1 << 21,
                             "contiguous", 64, 1005),
    # one tensor-parallel share of the long-context case: 8 heads per GPU
    "long185k_h8": Spec("long185k_h8", 1, 185000, 16, "random", 8, "bf16", 1 << 21, "scattered", 64, 1003),
}


def config(name: str, **overrides) -> Spec:
    """A named spec, optionally with fields replaced (e.g. a smaller pool)."""
    spec = CONFIGS[name]
    return dataclasses.replace(spec, **overrides) if overrides else spec


def random_parents(rng: np.random.Generator, num_draft: int) -> np.ndarray:
    """Node 0 is the root; node i > 0 takes a parent uniform in [0, i-1]."""
    parents = np.full(num_draft, -1, dtype=np.int64)
    for i in range(1, num_draft):
        parents[i] = rng.integers(0, i)
    return parents


def chain_parents(num_draft: int) -> np.ndarray:
    """A linear chain: node i's parent is i-1."""
    return np.arange(-1, num_draft - 1, dtype=np.int64)


def tree_mask(parents: np.ndarray, prefix_len: int) -> np.ndarray:
    """Visibility bytes [T, prefix_len + T] for one request.

    Row i (draft node i) sees every prefix column, itself, and each ancestor.
    """
    T = len(parents)
    m = np.zeros((T, prefix_len + T), dtype=np.uint8)
    m[:, :prefix_len] = 1
    for i in range(T):
        j = i
        while j >= 0:
            m[i, prefix_len + j] = 1
            j = int(parents[j])
    return m


@dataclass
class Workload:
    spec: Spec
    prefix_lens: np.ndarray  # int64 [batch]
    parents: list  # per request int64 [T]
    q_nope: torch.Tensor  # [batch*T, H, 512] dtype, CPU
    q_rope: torch.Tensor  # [batch*T, H, 64] dtype, CPU
    rows: torch.Tensor  # [sum N_b, 576] dtype, CPU: cache rows in logical key order
    slots: np.ndarray  # int64 [sum N_b]: pool slot of each logical row
    kv_indptr: torch.Tensor  # int32 [batch+1]
    kv_indices: torch.Tensor  # int32 [sum P_b]
    out_cache_loc: torch.Tensor  # int32 [batch*T]
    custom_mask: torch.Tensor  # uint8 [sum T*N_b]
    mask_indptr: torch.Tensor  # int32 [batch+1]
    row_offsets: np.ndarray = field(default=None)  # int64 [batch+1]: start of request b in `rows`

    @property
    def batch(self) -> int:
        return self.spec.batch

    @property
    def num_draft(self) -> int:
        return self.spec.num_draft

    @property
    def num_heads(self) -> int:
        return self.spec.num_heads

    @property
    def sm_scale(self) -> float:
        return self.spec.sm_scale

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.spec.dtype]

    @property
    def total_keys(self) -> int:
        return int(self.prefix_lens.sum()) + self.batch * self.num_draft

    def host_pool(self, fill: float = float("nan")) -> torch.Tensor:
        """The whole [pool_slots, 576] cache on the host; unreferenced rows = fill."""
        pool = torch.full((self.spec.pool_slots, D_KEY), fill, dtype=self.torch_dtype)
        pool[torch.from_numpy(self.slots)] = self.rows
        return pool

    def device_pool(self, device, fill: Optional[float] = float("nan"), row_stride: int = D_KEY) -> torch.Tensor:
        """The cache on `device`, [pool_slots, row_stride] (a view of width 576 is
        what the kernel reads). fill=None leaves unreferenced rows uninitialised."""
        if fill is None:
            pool = torch.empty((self.spec.pool_slots, row_stride), dtype=self.torch_dtype, device=device)
        else:
            pool = torch.full((self.spec.pool_slots, row_stride), fill, dtype=self.torch_dtype, device=device)
        idx = torch.from_numpy(self.slots).to(device)
        pool[idx, :D_KEY] = self.rows.to(device)
        return pool

    def request_rows(self, b: int) -> torch.Tensor:
        """Logical rows (prefix then drafts) of request b, [N_b, 576]."""
        return self.rows[self.row_offsets[b]:self.row_offsets[b + 1]]


def _prefix_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    p = spec.prefix
    if isinstance(p, int):
        return np.full(spec.batch, p, dtype=np.int64)
    if isinstance(p, tuple) and len(p) == 2:
        return rng.integers(p[0], p[1] + 1, size=spec.batch).astype(np.int64)
    arr = np.asarray(list(p), dtype=np.int64)
    if arr.shape != (spec.batch,):
        raise ValueError("explicit prefix list must have one length per request")
    return arr


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = rng.standard_normal(shape, dtype=np.float32)
    t = torch.from_numpy(x)
    return t.to(dtype) if dtype != torch.float32 else t


def build(spec: Union[Spec, str], **overrides) -> Workload:
    """Draw a workload from its spec (deterministic in spec.seed)."""
    if isinstance(spec, str):
        spec = config(spec, **overrides)
    elif overrides:
        spec = dataclasses.replace(spec, **overrides)
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    bs, T, H = spec.batch, spec.num_draft, spec.num_heads
    dtype = _TORCH_DTYPES[spec.dtype]

    prefix = _prefix_lengths(spec, rng)
    if spec.tree == "random":
        parents = [random_parents(rng, T) for _ in range(bs)]
    elif spec.tree == "chain":
        parents = [chain_parents(T) for _ in range(bs)]
    else:
        raise ValueError(f"unknown tree kind {spec.tree!r}")

    q_nope = _normal(rng, (bs * T, H, D_LATENT), dtype)
    q_rope = _normal(rng, (bs * T, H, D_ROPE), dtype)
    n_keys = prefix + T
    total = int(n_keys.sum())
    rows = _normal(rng, (total, D_KEY), dtype)

    if total > spec.pool_slots:
        raise ValueError("pool too small for the referenced rows")
    if spec.layout == "scattered":
        slots = rng.choice(spec.pool_slots, size=total, replace=False).astype(np.int64)
    elif spec.layout == "permutation":
        slots = rng.permutation(spec.pool_slots)[:total].astype(np.int64)
    elif spec.layout == "contiguous":
        slots = np.arange(total, dtype=np.int64)
    else:
        raise ValueError(f"unknown layout {spec.layout!r}")

    row_off = np.zeros(bs + 1, dtype=np.int64)
    row_off[1:] = np.cumsum(n_keys)
    kv_indptr = np.zeros(bs + 1, dtype=np.int64)
    kv_indptr[1:] = np.cumsum(prefix)
    kv_indices = np.empty(int(prefix.sum()), dtype=np.int64)
    out_cache_loc = np.empty(bs * T, dtype=np.int64)
    masks = []
    mask_indptr = np.zeros(bs + 1, dtype=np.int64)
    for b in range(bs):
        s = slots[row_off[b]:row_off[b + 1]]
        kv_indices[kv_indptr[b]:kv_indptr[b + 1]] = s[:prefix[b]]
        out_cache_loc[b * T:(b + 1) * T] = s[prefix[b]:]
        m = tree_mask(parents[b], int(prefix[b]))
        masks.append(m.reshape(-1))
        mask_indptr[b + 1] = mask_indptr[b] + m.size
    if mask_indptr[-1] >= 2**31 or total >= 2**31:
        raise ValueError("metadata exceeds int32 offsets")

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))  # noqa: E731
    return Workload(
        spec=spec,
        prefix_lens=prefix,
        parents=parents,
        q_nope=q_nope,
        q_rope=q_rope,
        rows=rows,
        slots=slots,
        kv_indptr=i32(kv_indptr),
        kv_indices=i32(kv_indices),
        out_cache_loc=i32(out_cache_loc),
        custom_mask=torch.from_numpy(np.concatenate(masks) if masks else np.zeros(0, np.uint8)),
        mask_indptr=i32(mask_indptr),
        row_offsets=row_off,
    )


def small(name: str, batch: int, prefix, num_draft: int, num_heads: int, dtype: str = "bf16",
          tree: str = "random", pool_slots: int = 1 << 16, layout: str = "scattered",
          nsplit: int = 64, seed: int = 7) -> Spec:
    """A custom spec for tests (ragged tails, tiny heads, empty prefixes, ...)."""
    return Spec(name, batch, prefix, num_draft, tree, num_heads, dtype, pool_slots, layout, nsplit, seed)


@dataclass
class RaggedTrees:
    """A workload whose request b keeps only the first T_b of its draft nodes
    (a valid subtree: parents precede children). Arrays in the layout of the
    ragged verify call: token offsets qo_indptr, draft slots, mask blocks
    [T_b][P_b + T_b] and queries for the kept tokens only."""
    base: Workload
    tokens: np.ndarray  # int64 [batch]: T_b
    qo_indptr: torch.Tensor  # int64 [batch+1]
    q_nope: torch.Tensor  # [sum T_b, H, 512]
    q_rope: torch.Tensor  # [sum T_b, H, 64]
    out_cache_loc: torch.Tensor  # int32 [sum T_b]
    custom_mask: torch.Tensor  # uint8 [sum T_b * (P_b + T_b)]
    mask_indptr: torch.Tensor  # int32 [batch+1]


def ragged_trees(w: Workload, tokens) -> RaggedTrees:
    """Cut request b's tree of w to its first tokens[b] nodes (0 <= T_b <= T)."""
    T = w.num_draft
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.shape != (w.batch,) or (tokens < 0).any() or (tokens > T).any():
        raise ValueError("need one token count in [0, num_draft] per request")
    qo = np.zeros(w.batch + 1, dtype=np.int64)
    qo[1:] = np.cumsum(tokens)
    keep = np.concatenate([np.arange(b * T, b * T + tokens[b]) for b in range(w.batch)]).astype(np.int64)
    ocl = w.out_cache_loc.numpy()[keep]
    masks, mind = [], np.zeros(w.batch + 1, dtype=np.int64)
    full = w.custom_mask.numpy()
    for b in range(w.batch):
        P, Tb = int(w.prefix_lens[b]), int(tokens[b])
        blk = full[int(w.mask_indptr[b]):int(w.mask_indptr[b + 1])].reshape(T, P + T)
        m = np.ascontiguousarray(blk[:Tb, :P + Tb])
        masks.append(m.reshape(-1))
        mind[b + 1] = mind[b] + m.size
    idx = torch.from_numpy(keep)
    return RaggedTrees(
        base=w, tokens=tokens, qo_indptr=torch.from_numpy(qo),
        q_nope=w.q_nope[idx].contiguous(), q_rope=w.q_rope[idx].contiguous(),
        out_cache_loc=torch.from_numpy(ocl.astype(np.int32)),
        custom_mask=torch.from_numpy(np.concatenate(masks) if masks else np.zeros(0, np.uint8)),
        mask_indptr=torch.from_numpy(mind.astype(np.int32)),
    )
