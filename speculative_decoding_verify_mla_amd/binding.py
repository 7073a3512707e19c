"""ctypes binding for libtvmla.so: the same entry points as include/tvmla.h.

Argument marshalling only. Tensors are torch tensors on the GPU (device
memory and streams are PyTorch's job here); every step of the computation
runs in the library's HIP kernels. If the library is missing the binding
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtvmla.so")

BF16, FP32 = 0, 1
ALGO_AUTO, ALGO_SCALAR, ALGO_MFMA, ALGO_ROWS = 0, 1, 2, 3
TUNE_NSPLIT = 1  # TVMLA_FLAG_TUNE_NSPLIT
TILE_CHUNKS = 2  # TVMLA_FLAG_TILE_CHUNKS
FOLD_DEFAULT = -1.0  # fold_log2 < 0: the library's default threshold
META_ARRAYS = {0: "none", 1: "kv_indptr", 2: "kv_indices", 3: "out_cache_loc", 4: "mask_indptr", 5: "qo_indptr"}
D_LATENT, D_ROPE, D_KEY = 512, 64, 576

STATUS = {
    0: "TVMLA_OK",
    1: "TVMLA_E_NULLPTR",
    2: "TVMLA_E_SHAPE",
    3: "TVMLA_E_DTYPE",
    4: "TVMLA_E_WORKSPACE",
    5: "TVMLA_E_ALIGN",
    6: "TVMLA_E_LAUNCH",
    7: "TVMLA_E_ALGO",
    8: "TVMLA_E_VALUE",
    9: "TVMLA_E_INDEX",
}

# every symbol include/tvmla.h declares
EXPORTS = ("tvmla_workspace_bytes", "tvmla_verify", "tvmla_verify_ex", "tvmla_verify_ragged", "tvmla_verify_partials",
           "tvmla_combine", "tvmla_defrag", "tvmla_tree_mask", "tvmla_status_str", "tvmla_version",
           "tvmla_auto_algo", "tvmla_effective_nsplit", "tvmla_check_metadata", "tvmla_verify_noalloc")
NOALLOC_SCRATCH_BYTES = 256 << 20  # TVMLA_NOALLOC_SCRATCH_BYTES


class TvmlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None

_P, _I32, _U32, _I64, _F32, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_size_t)
_VERIFY_ARGS = [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _I32, _I32, _I32, _F32, _I32, _I32,
                _P, _P, _P, _SZ, _P]


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m speculative_decoding_verify_mla_amd.build`")
    lib = ctypes.CDLL(path)
    lib.tvmla_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
    lib.tvmla_workspace_bytes.restype = _SZ
    lib.tvmla_verify.argtypes = _VERIFY_ARGS
    lib.tvmla_verify.restype = ctypes.c_int
    lib.tvmla_verify_ex.argtypes = _VERIFY_ARGS + [_I32, _I32, _U32, _F32]
    lib.tvmla_verify_ex.restype = ctypes.c_int
    lib.tvmla_verify_noalloc.argtypes = _VERIFY_ARGS[:21] + [_P, _I32, _I32, _U32, _F32]
    lib.tvmla_verify_noalloc.restype = ctypes.c_int
    lib.tvmla_verify_ragged.argtypes = _VERIFY_ARGS[:13] + [_P] + _VERIFY_ARGS[13:] + [_I32, _I32, _U32, _F32]
    lib.tvmla_verify_ragged.restype = ctypes.c_int
    lib.tvmla_verify_partials.argtypes = _VERIFY_ARGS[:19] + _VERIFY_ARGS[21:] + [_I32, _I32, _U32, _F32]
    lib.tvmla_verify_partials.restype = ctypes.c_int
    lib.tvmla_combine.argtypes = [_P, _SZ, _P, _I32, _I32, _I32, _I32, _I32, _U32, _I32, _P, _P, _P]
    lib.tvmla_combine.restype = ctypes.c_int
    lib.tvmla_defrag.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _P, _I32, _I32, _P]
    lib.tvmla_defrag.restype = ctypes.c_int
    lib.tvmla_tree_mask.argtypes = [_P, _P, _I32, _I32, _P, _P, _P]
    lib.tvmla_tree_mask.restype = ctypes.c_int
    lib.tvmla_status_str.argtypes = [_I32]
    lib.tvmla_status_str.restype = ctypes.c_char_p
    lib.tvmla_version.argtypes = []
    lib.tvmla_version.restype = _I32
    lib.tvmla_auto_algo.argtypes = [_I32] * 5
    lib.tvmla_auto_algo.restype = _I32
    lib.tvmla_effective_nsplit.argtypes = [_I32] * 4
    lib.tvmla_effective_nsplit.restype = _I32
    lib.tvmla_check_metadata.argtypes = [_P, _P, _I64, _P, _I64, _P, _I64, _P, _I32, _I32, _I64, _P, _P]
    lib.tvmla_check_metadata.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().tvmla_status_str(status).decode()


def version() -> int:
    return load().tvmla_version()


def effective_nsplit(batch: int, num_draft: int, num_heads: int, nsplit: int) -> int:
    """Splits verify() really uses for these sizes (negative status if out of range)."""
    return load().tvmla_effective_nsplit(batch, num_draft, num_heads, nsplit)


def auto_algo(batch: int, num_draft: int, num_heads: int, nsplit: int, dtype: int = 0) -> int:
    """The algorithm ALGO_AUTO resolves to for these sizes (negative status if out of range)."""
    return load().tvmla_auto_algo(batch, num_draft, num_heads, nsplit, dtype)


def workspace_bytes(batch: int, num_draft: int, num_heads: int, nsplit: int) -> int:
    return load().tvmla_workspace_bytes(batch, num_draft, num_heads, nsplit)


def _check(status: int):
    if status != 0:
        raise TvmlaError(status, status_str(status))


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TvmlaError(3, f"unsupported dtype {t.dtype}")


def _stream_ptr(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _verify_args(q_nope, q_rope, kv_cache, num_draft):
    ntok, H, dl = q_nope.shape
    if dl != D_LATENT or tuple(q_rope.shape) != (ntok, H, D_ROPE):
        raise TvmlaError(2, "q_nope must be [tok, H, 512] and q_rope [tok, H, 64]")
    if q_nope.stride(2) != 1 or q_rope.stride(2) != 1 or kv_cache.stride(1) != 1:
        raise TvmlaError(5, "last dimensions must be contiguous")
    if ntok % num_draft:
        raise TvmlaError(2, "token count must be batch * num_draft")
    dt = _dtype_code(q_nope)
    if q_rope.dtype != q_nope.dtype or kv_cache.dtype != q_nope.dtype:
        raise TvmlaError(3, "q_nope, q_rope and kv_cache must share one dtype")
    return ntok // num_draft, H, dt


def _out_args(q_nope, out, lse):
    if not (out.is_contiguous() and lse.is_contiguous()):
        raise TvmlaError(5, "out and lse must be contiguous")
    if out.dtype != q_nope.dtype:
        raise TvmlaError(3, "out must have q's dtype")


def verify(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
           sm_scale: float, nsplit: int, out, lse, workspace, num_draft: int,
           algo: int = ALGO_AUTO, min_chunk: int = 0, flags: int = 0, fold_log2: float = FOLD_DEFAULT,
           stream=None) -> None:
    """Enqueue tvmla_verify_ex on `stream` (default: torch's current stream).

    q_nope [batch*T, H, 512], q_rope [batch*T, H, 64] (last dim contiguous),
    kv_cache [slots, >=576] (row-contiguous), int32 metadata, uint8 mask,
    out [batch*T, H, 512] (q's dtype), lse [batch*T, H] fp32, workspace a
    tensor of at least workspace_bytes(...) bytes. flags = TUNE_NSPLIT runs
    effective_nsplit(...) splits instead of exactly nsplit.
    """
    batch, H, dt = _verify_args(q_nope, q_rope, kv_cache, num_draft)
    _out_args(q_nope, out, lse)
    st = load().tvmla_verify_ex(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_cache), kv_cache.stride(0),
        _ptr(kv_indptr), _ptr(kv_indices), _ptr(out_cache_loc), _ptr(custom_mask), _ptr(mask_indptr),
        batch, num_draft, H, float(sm_scale), nsplit, dt,
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream), algo, min_chunk, flags, float(fold_log2))
    _check(st)


def verify_plain(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                 sm_scale: float, nsplit: int, out, lse, workspace, num_draft: int, stream=None) -> None:
    """Enqueue tvmla_verify itself (the pages' call: exactly nsplit splits,
    automatic kernel choice); same tensors as verify()."""
    batch, H, dt = _verify_args(q_nope, q_rope, kv_cache, num_draft)
    _out_args(q_nope, out, lse)
    st = load().tvmla_verify(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_cache), kv_cache.stride(0),
        _ptr(kv_indptr), _ptr(kv_indices), _ptr(out_cache_loc), _ptr(custom_mask), _ptr(mask_indptr),
        batch, num_draft, H, float(sm_scale), nsplit, dt,
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream))
    _check(st)


def verify_noalloc(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                   sm_scale: float, nsplit: int, out, lse, num_draft: int, algo: int = ALGO_AUTO,
                   min_chunk: int = 0, flags: int = 0, fold_log2: float = FOLD_DEFAULT, stream=None) -> None:
    """Enqueue tvmla_verify_noalloc: verify() without a workspace (the split
    partials go to the library's per-device scratch array; calls on one
    device must not overlap)."""
    batch, H, dt = _verify_args(q_nope, q_rope, kv_cache, num_draft)
    _out_args(q_nope, out, lse)
    st = load().tvmla_verify_noalloc(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_cache), kv_cache.stride(0),
        _ptr(kv_indptr), _ptr(kv_indices), _ptr(out_cache_loc), _ptr(custom_mask), _ptr(mask_indptr),
        batch, num_draft, H, float(sm_scale), nsplit, dt,
        _ptr(out), _ptr(lse), _stream_ptr(stream), algo, min_chunk, flags, float(fold_log2))
    _check(st)


def verify_ragged(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                  qo_indptr, sm_scale: float, nsplit: int, out, lse, workspace, max_draft: int,
                  algo: int = ALGO_AUTO, min_chunk: int = 0, flags: int = 0, fold_log2: float = FOLD_DEFAULT,
                  stream=None) -> None:
    """Enqueue tvmla_verify_ragged: request b has qo_indptr[b+1] - qo_indptr[b]
    draft tokens (at most max_draft); q/out/lse hold qo_indptr[batch] token rows."""
    ntok, H, dl = q_nope.shape
    if dl != D_LATENT or tuple(q_rope.shape) != (ntok, H, D_ROPE):
        raise TvmlaError(2, "q_nope must be [tok, H, 512] and q_rope [tok, H, 64]")
    if q_nope.stride(2) != 1 or q_rope.stride(2) != 1 or kv_cache.stride(1) != 1:
        raise TvmlaError(5, "last dimensions must be contiguous")
    if not (out.is_contiguous() and lse.is_contiguous()):
        raise TvmlaError(5, "out and lse must be contiguous")
    dt = _dtype_code(q_nope)
    if q_rope.dtype != q_nope.dtype or kv_cache.dtype != q_nope.dtype or out.dtype != q_nope.dtype:
        raise TvmlaError(3, "q_nope, q_rope, kv_cache and out must share one dtype")
    batch = kv_indptr.numel() - 1
    st = load().tvmla_verify_ragged(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_cache), kv_cache.stride(0),
        _ptr(kv_indptr), _ptr(kv_indices), _ptr(out_cache_loc), _ptr(custom_mask), _ptr(mask_indptr),
        _ptr(qo_indptr), batch, max_draft, H, float(sm_scale), nsplit, dt,
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream), algo, min_chunk, flags, float(fold_log2))
    _check(st)


def verify_partials(q_nope, q_rope, kv_cache, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                    sm_scale: float, nsplit: int, workspace, num_draft: int, algo: int = ALGO_AUTO,
                    min_chunk: int = 0, fold_log2: float = FOLD_DEFAULT, flags: int = 0, stream=None) -> None:
    """Enqueue tvmla_verify_partials: the split step only (partials land in workspace)."""
    batch, H, dt = _verify_args(q_nope, q_rope, kv_cache, num_draft)
    st = load().tvmla_verify_partials(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_cache), kv_cache.stride(0),
        _ptr(kv_indptr), _ptr(kv_indices), _ptr(out_cache_loc), _ptr(custom_mask), _ptr(mask_indptr),
        batch, num_draft, H, float(sm_scale), nsplit, dt,
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream), algo, min_chunk, flags, float(fold_log2))
    _check(st)


def combine(workspace, kv_indptr, batch: int, num_draft: int, num_heads: int, nsplit: int, out, lse,
            min_chunk: int = 0, flags: int = 0, stream=None) -> None:
    """Enqueue tvmla_combine: merge the workspace's split partials into out/lse."""
    st = load().tvmla_combine(_ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(kv_indptr),
                              batch, num_draft, num_heads, nsplit, min_chunk, flags, _dtype_code(out),
                              _ptr(out), _ptr(lse), _stream_ptr(stream))
    _check(st)


def workspace_views(workspace, batch: int, num_draft: int, num_heads: int, nsplit: int, dtype: int = FP32):
    """The partial-result regions of a workspace as tensors: o_part [batch,
    nsplit, R, 512] (bf16 for dtype BF16: the first half of each 2 KB slot;
    fp32 for FP32) and lse_part [batch, nsplit, R] (fp32)."""
    import torch

    R = num_draft * num_heads
    rows = batch * nsplit * R
    o_bytes = rows * D_LATENT * 4
    lse_off = (o_bytes + 255) // 256 * 256
    raw = workspace.view(torch.uint8)
    if dtype == BF16:
        o = raw[:o_bytes].view(torch.bfloat16).view(batch, nsplit, R, 2 * D_LATENT)[..., :D_LATENT]
    else:
        o = raw[:o_bytes].view(torch.float32).view(batch, nsplit, R, D_LATENT)
    lse = raw[lse_off:lse_off + rows * 4].view(torch.float32).view(batch, nsplit, R)
    return o, lse


def defrag(kv_src, kv_dst, kv_indptr, kv_indices, dst_base, kv_indices_out, stream=None) -> None:
    """Enqueue tvmla_defrag: move each request's prefix rows of kv_src to slots
    dst_base[b] + p of kv_dst and write the new indices to kv_indices_out
    (which may be kv_indices itself)."""
    if kv_src.dtype != kv_dst.dtype:
        raise TvmlaError(3, "kv_src and kv_dst must share one dtype")
    if kv_src.stride(1) != 1 or kv_dst.stride(1) != 1:
        raise TvmlaError(5, "cache rows must be contiguous")
    batch = kv_indptr.numel() - 1
    st = load().tvmla_defrag(_ptr(kv_src), kv_src.stride(0), _ptr(kv_dst), kv_dst.stride(0), _ptr(kv_indptr),
                             _ptr(kv_indices), _ptr(dst_base), _ptr(kv_indices_out), batch,
                             _dtype_code(kv_src), _stream_ptr(stream))
    _check(st)


def tree_mask(parents, kv_indptr, num_draft: int, custom_mask, mask_indptr, stream=None) -> None:
    """Enqueue tvmla_tree_mask: build custom_mask / mask_indptr on the device
    from int32 parents [batch*num_draft] (-1 for each root)."""
    batch = kv_indptr.numel() - 1
    st = load().tvmla_tree_mask(_ptr(parents), _ptr(kv_indptr), batch, num_draft, _ptr(custom_mask),
                                _ptr(mask_indptr), _stream_ptr(stream))
    _check(st)


def check_metadata(kv_indptr, kv_indices, out_cache_loc, mask_indptr, mask_len: int, num_draft: int,
                   num_slots: int, qo_indptr=None):
    """Run tvmla_check_metadata on host copies of the metadata (numpy arrays
    or CPU tensors; int32, qo_indptr int64). Returns (status, array name,
    position): status 0 when every offset and slot is in range."""
    import numpy as np

    def host(a, dt):
        if a is None:
            return None
        if hasattr(a, "detach"):
            a = a.detach().cpu().numpy()
        return np.ascontiguousarray(np.asarray(a), dtype=dt)

    ip, idx, ocl, mi = host(kv_indptr, np.int32), host(kv_indices, np.int32), host(out_cache_loc, np.int32), \
        host(mask_indptr, np.int32)
    qo = host(qo_indptr, np.int64)
    bad_array, bad_pos = ctypes.c_int32(-7), ctypes.c_int64(-7)
    st = load().tvmla_check_metadata(ip.ctypes.data, idx.ctypes.data if idx.size else None, idx.size,
                                     ocl.ctypes.data, ocl.size, mi.ctypes.data, int(mask_len),
                                     None if qo is None else qo.ctypes.data, ip.size - 1, num_draft, int(num_slots),
                                     ctypes.byref(bad_array), ctypes.byref(bad_pos))
    return st, META_ARRAYS.get(bad_array.value, bad_array.value), bad_pos.value
