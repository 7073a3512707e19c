"""fp64 CPU oracle for tree-verify attention over an MLA latent KV cache.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports, links or calls it, and this package
imports nothing from the product.

verify_fp64  vectorised fp64 definition (NumPy), split partials and the
             log-sum-exp combine
brute        pure-Python scalar loops with math.fsum, used to pin verify_fp64
defrag       compaction of a request's prefix rows into a contiguous run
tree_mask    the visibility mask built from draft-tree parent arrays
"""
from . import brute, defrag, tree_mask, verify_fp64  # noqa: F401
