"""Tree-verify attention over an MLA latent KV cache, for AMD MI355X (gfx950).

The computation lives in libtvmla.so (HIP kernels behind a C ABI, declared
in include/tvmla.h); `binding` marshals torch tensors into it.
"""
from .binding import (  # noqa: F401
    ALGO_AUTO,
    ALGO_MFMA,
    ALGO_SCALAR,
    BF16,
    FP32,
    TvmlaError,
    combine,
    load,
    status_str,
    verify,
    verify_partials,
    version,
    workspace_bytes,
    workspace_views,
)
