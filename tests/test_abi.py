"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/tvmla.h declares, sizes its workspace as documented, and rejects bad
arguments on the host before any HIP call (so these run on a GPU-less box)."""
import ctypes
import os
import re

import pytest

from speculative_decoding_verify_mla_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tvmla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from speculative_decoding_verify_mla_amd import build

        build.build()
    return binding.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tvmla_[a-z_]+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert _declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_version_and_status_strings(lib):
    assert binding.version() >= 100
    for code in range(10):
        s = binding.status_str(code)
        assert isinstance(s, str) and s
    assert binding.status_str(99) == "unknown status"


def test_auto_algo(lib):
    # nsplit is the count the call runs. 64 splits x 8 row groups of 128 (16 tokens x 64 heads): 512
    # workgroups -> the 128-row kernel; so at the 32 splits TVMLA_FLAG_TUNE_NSPLIT runs (256 workgroups)
    assert binding.auto_algo(1, 16, 64, 64) == binding.ALGO_ROWS
    assert binding.auto_algo(1, 16, 64, 32) == binding.ALGO_ROWS
    # 16 tokens x 8 heads: one row group; 64 splits leave 192 CUs idle -> the 64-row kernel (128 workgroups)
    assert binding.auto_algo(1, 16, 8, 64) == binding.ALGO_MFMA
    # ... the 256 splits the tuned call runs fill them -> the 128-row kernel
    assert binding.auto_algo(1, 16, 8, 256) == binding.ALGO_ROWS
    assert binding.auto_algo(4, 16, 8, 64) == binding.ALGO_ROWS
    assert binding.auto_algo(1, 16, 8, 200) == binding.ALGO_MFMA
    assert binding.auto_algo(1, 4, 64, 64, binding.FP32) == binding.ALGO_SCALAR
    assert binding.auto_algo(0, 4, 64, 64) == -2
    assert binding.auto_algo(1, 4, 64, 64, 7) == -3


def test_effective_nsplit(lib):
    ens = binding.effective_nsplit
    assert ens(1, 16, 64, 64) == 32          # 8 row groups x 64 splits = 512 workgroups: one round of 256 instead
    assert ens(1, 16, 64, 63) == 63          # 504 workgroups, odd count: kept
    assert ens(1, 16, 64, 48) == 48          # 384 workgroups: halving would leave CUs idle
    assert ens(1, 16, 64, 32) == 32          # exactly one round
    assert ens(2, 16, 64, 64) == 32          # 1024 workgroups: halved to two rounds
    assert ens(2, 16, 64, 128) == 32         # 2048 workgroups: halved twice
    assert ens(32, 8, 64, 64) == 4           # 32 requests x 4 row groups: 8192 workgroups, halved down to 512
    assert ens(8, 32, 64, 64) == 4           # 8 requests x 16 row groups: likewise
    assert ens(96, 8, 64, 64) == 4           # 96 requests (index order): halved while four rounds remain
    assert ens(64, 8, 64, 64) == 2           # 64 requests (longest first): two rounds
    assert ens(3, 16, 64, 32) == 32          # 768 workgroups: halving would leave fewer than two rounds
    assert ens(8, 32, 64, 63) == 63          # odd: kept
    assert ens(1, 16, 8, 64) == 256          # one row group: doubled twice
    assert ens(3, 5, 8, 7) == 112            # 3 x 56 = 168 < 256, 3 x 112 = 336
    assert ens(1, 1, 1, 64) == 256
    assert ens(1, 16, 8, 200) == 200         # doubling would pass 256
    assert ens(0, 1, 1, 1) == -2 and ens(1, 1, 1, 257) == -2
    # the workspace covers the splits the call uses
    assert binding.workspace_bytes(1, 16, 8, 64) == binding.workspace_bytes(1, 16, 8, 256)
    # ... and the caller's count, which the split step alone and the combine take as given
    assert binding.workspace_bytes(1, 16, 64, 64) == binding.workspace_bytes(2, 16, 64, 32)


def test_workspace_bytes(lib):
    # fp32 partials: 512-wide output + lse per (token, head, split), 256-byte aligned regions
    bs, T, H, ns = 8, 9, 64, 64
    rows = bs * T * H * ns
    o = rows * 512 * 4
    expect = o + ((rows * 4 + 255) // 256) * 256
    assert binding.workspace_bytes(bs, T, H, ns) == expect
    # the pages' figure: about 600 MB at batch 8, 9 draft tokens, NSPLIT 64 (64 heads)
    assert abs(expect - 600e6) < 0.05 * 600e6
    # a pure function of its arguments; rejects out-of-range ones
    assert binding.workspace_bytes(1, 16, 64, 64) == binding.workspace_bytes(1, 16, 64, 64)
    for bad in [(0, 1, 1, 1), (1, 0, 1, 1), (1, 65, 1, 1), (1, 1, 0, 1), (1, 1, 129, 1), (1, 1, 1, 0),
                (1, 1, 1, 257)]:
        assert binding.workspace_bytes(*bad) == 0


# ---------------------------------------------------------------- error paths

_FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case fails a host check first


@pytest.fixture(autouse=True)
def _fake_pointers_only_without_gpu(request):
    """The error-path tests pass fake device pointers and rely on a host
    check rejecting each call; where a GPU is visible a wrong expectation
    would launch kernels on them, so these tests run on GPU-less hosts only
    (device_count does not initialise the runtime)."""
    if "lib" in request.fixturenames and request.node.name.split("[")[0] in _FAKE_POINTER_TESTS:
        import torch

        if torch.cuda.device_count() > 0:
            pytest.skip("fake-pointer error-path test: GPU-less hosts only")


_FAKE_POINTER_TESTS = {"test_null_pointer", "test_null_workspace", "test_bad_shape", "test_bad_dtype", "test_bad_algo",
                       "test_bad_scale", "test_bad_flags_and_fold", "test_misaligned", "test_small_workspace",
                       "test_combine_errors", "test_plain_verify_errors", "test_partials_errors",
                       "test_noalloc_host_checks", "test_defrag_null_pointer", "test_defrag_bad_shape",
                       "test_defrag_bad_dtype", "test_defrag_misaligned", "test_tree_mask_null_pointer",
                       "test_tree_mask_bad_shape"}


def _call(lib, **kw):
    a = dict(q_nope=_FAKE, qn_st=64 * 512, qn_sh=512, q_rope=_FAKE, qr_st=64 * 64, qr_sh=64, kv=_FAKE,
             kv_stride=576, kv_indptr=_FAKE, kv_indices=_FAKE, ocl=_FAKE, mask=_FAKE, mask_indptr=_FAKE,
             batch=1, T=4, H=64, scale=0.07, nsplit=64, dtype=binding.BF16, out=_FAKE, lse=_FAKE,
             ws=_FAKE, ws_bytes=None, stream=None, algo=0, min_chunk=0, flags=0, fold=-1.0)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = binding.workspace_bytes(max(a["batch"], 1), max(min(a["T"], 64), 1),
                                                max(min(a["H"], 128), 1), max(min(a["nsplit"], 256), 1))
    return lib.tvmla_verify_ex(a["q_nope"], a["qn_st"], a["qn_sh"], a["q_rope"], a["qr_st"], a["qr_sh"], a["kv"],
                               a["kv_stride"], a["kv_indptr"], a["kv_indices"], a["ocl"], a["mask"],
                               a["mask_indptr"], a["batch"], a["T"], a["H"], a["scale"], a["nsplit"], a["dtype"],
                               a["out"], a["lse"], a["ws"], a["ws_bytes"], a["stream"], a["algo"],
                               a["min_chunk"], a["flags"], a["fold"])


@pytest.mark.parametrize("field", ["q_nope", "q_rope", "kv", "kv_indptr", "kv_indices", "ocl", "mask",
                                   "mask_indptr", "out", "lse"])
def test_null_pointer(lib, field):
    assert _call(lib, **{field: None}) == 1


def test_null_workspace(lib):
    assert _call(lib, ws=None) == 4


@pytest.mark.parametrize("kw", [dict(batch=0), dict(batch=70000), dict(T=0), dict(T=65), dict(H=0), dict(H=129),
                                dict(nsplit=0), dict(nsplit=257), dict(min_chunk=-1), dict(kv_stride=575),
                                dict(qn_st=-512)])
def test_bad_shape(lib, kw):
    assert _call(lib, **kw) == 2


@pytest.mark.parametrize("kw", [dict(dtype=2), dict(dtype=-1), dict(dtype=binding.FP32, algo=binding.ALGO_MFMA),
                                dict(dtype=binding.FP32, algo=binding.ALGO_ROWS)])
def test_bad_dtype(lib, kw):
    assert _call(lib, **kw) == 3


def test_bad_algo(lib):
    assert _call(lib, algo=4) == 7


@pytest.mark.parametrize("scale", [0.0, -0.07, float("inf"), float("nan")])
def test_bad_scale(lib, scale):
    assert _call(lib, scale=scale) == 8


@pytest.mark.parametrize("kw", [dict(flags=4), dict(flags=0xFFFFFFFF), dict(flags=7), dict(fold=float("nan"))])
def test_bad_flags_and_fold(lib, kw):
    assert _call(lib, **kw) == 8


@pytest.mark.parametrize("kw", [dict(q_nope=_FAKE + 8), dict(kv=_FAKE + 2), dict(out=_FAKE + 4), dict(ws=_FAKE + 8),
                                dict(kv_stride=580), dict(qn_sh=516), dict(qr_st=64 * 64 + 4)])
def test_misaligned(lib, kw):
    assert _call(lib, **kw) == 5


def test_effective_nsplit_properties(lib):
    """Over a grid of sizes, the tuned split count has the properties it
    exists for (host-only call, no GPU needed): it stays in 1..256 and is the
    caller's count times or divided by a power of two; a raised count is the
    smallest doubling whose 128-row grid covers the 256 compute units (or
    the largest within 256); a lowered one keeps at least one round of 256
    workgroups, and at least two rounds (batches up to 64, served longest
    request first) or four (larger batches) unless the caller's grid had at
    most two rounds; an unchanged count could not be halved under those
    rules."""

    def grid(batch, T, H, n):
        return batch * n * -(-(T * H) // 128)

    n = 0
    for batch in (1, 2, 3, 7, 32, 64, 65, 300):
        for T, H in ((1, 1), (4, 8), (5, 8), (16, 8), (16, 64), (8, 64), (32, 64), (64, 128)):
            for ns in (1, 3, 7, 8, 32, 48, 63, 64, 128, 200, 256):
                e = binding.effective_nsplit(batch, T, H, ns)
                g = lambda k: grid(batch, T, H, k)
                case = (batch, T, H, ns, e)
                assert 1 <= e <= 256, case
                ratio = e / ns if e >= ns else ns / e
                assert ratio == int(ratio) and int(ratio) & (int(ratio) - 1) == 0, case
                keep = 512 if batch <= 64 else 1024
                if g(ns) < 256:
                    # too few workgroups: doubled until the grid covers the CUs or 256 splits would be passed
                    assert e >= ns and (g(e) >= 256 or 2 * e > 256), case
                    assert e == ns or g(e // 2) < 256, case
                elif e < ns:
                    assert g(e) >= 256, case  # never leaves compute units idle
                    if g(ns) <= 512:
                        assert e * 2 == ns, case  # one round instead of two
                    else:
                        assert g(e) >= keep, case
                        assert e % 2 == 1 or g(e // 2) < keep, case  # halved as far as allowed
                else:
                    assert e == ns, case
                    if 256 < g(ns) <= 512:
                        assert ns % 2 == 1 or g(ns // 2) < 256, case
                    elif g(ns) > 512:
                        assert ns % 2 == 1 or g(ns // 2) < keep, case
                n += 1
    assert n == 8 * 8 * 11


def _layout_bytes(batch, T, H, ns):
    rows = batch * T * H * ns
    o = (rows * 512 * 4 + 255) // 256 * 256
    return o + (rows * 4 + 255) // 256 * 256


def test_small_workspace(lib):
    # exactly nsplit splits: the workspace of 64 splits
    need = _layout_bytes(1, 4, 64, 64)
    assert binding.workspace_bytes(1, 4, 64, 64) >= need
    assert _call(lib, ws_bytes=need - 1) == 4
    # tuned: 2 row groups x 64 splits = 128 workgroups, raised to 128 splits
    assert binding.effective_nsplit(1, 4, 64, 64) == 128
    assert binding.workspace_bytes(1, 4, 64, 64) == _layout_bytes(1, 4, 64, 128)
    assert _call(lib, ws_bytes=_layout_bytes(1, 4, 64, 128) - 1, flags=binding.TUNE_NSPLIT) == 4


def test_combine_errors(lib):
    f = lib.tvmla_combine
    # 2 requests x 16 tokens x 64 heads x 64 splits (args: ws, bytes, kv_indptr, batch, T, H, nsplit,
    # min_chunk, flags, dtype, out, lse, stream)
    ws = binding.workspace_bytes(2, 16, 64, 64)
    assert f(_FAKE, ws, _FAKE, 2, 16, 64, 64, 0, 0, 5, _FAKE, _FAKE, None) == 3
    assert f(_FAKE, ws, _FAKE, 2, 16, 64, 64, 0, 0, 0, None, _FAKE, None) == 1
    assert f(None, ws, _FAKE, 2, 16, 64, 64, 0, 0, 0, _FAKE, _FAKE, None) == 4
    assert f(_FAKE, ws - 1, _FAKE, 2, 16, 64, 64, 0, 0, 0, _FAKE, _FAKE, None) == 4
    assert f(_FAKE, ws, _FAKE, 0, 16, 64, 64, 0, 0, 0, _FAKE, _FAKE, None) == 2
    assert f(_FAKE + 4, ws, _FAKE, 2, 16, 64, 64, 0, 0, 0, _FAKE, _FAKE, None) == 5
    # the combine takes nsplit as given: only TVMLA_FLAG_TILE_CHUNKS is accepted
    assert f(_FAKE, ws, _FAKE, 2, 16, 64, 64, 0, binding.TUNE_NSPLIT, 0, _FAKE, _FAKE, None) == 8
    assert f(_FAKE, ws, _FAKE, 2, 16, 64, 64, 0, 4, 0, _FAKE, _FAKE, None) == 8


def test_plain_verify_errors(lib):
    """tvmla_verify (no algo, flags or fold arguments) runs the same host checks."""
    f = lib.tvmla_verify
    ws = _layout_bytes(1, 4, 64, 64)  # exactly the 64 splits the call runs
    good = [_FAKE, 64 * 512, 512, _FAKE, 64 * 64, 64, _FAKE, 576, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, 1, 4, 64, 0.07,
            64, binding.BF16, _FAKE, _FAKE, _FAKE, ws, None]
    for idx, val, code in [(0, None, 1), (19, None, 1), (21, None, 4), (22, ws - 1, 4), (17, 257, 2), (18, 3, 3),
                           (16, -1.0, 8), (6, _FAKE + 2, 5)]:
        a = list(good)
        a[idx] = val
        assert f(*a) == code, (idx, val)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(FileNotFoundError):
        binding.load(str(tmp_path / "missing.so"))


def test_partials_errors(lib):
    f = lib.tvmla_verify_partials
    ws = binding.workspace_bytes(2, 16, 64, 64)
    good = [_FAKE, 64 * 512, 512, _FAKE, 64 * 64, 64, _FAKE, 576, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, 2, 16, 64, 0.07,
            64, binding.BF16, _FAKE, ws, None, 0, 0, 0, -1.0]
    for idx, val, code in [(0, None, 1), (6, None, 1), (19, None, 4), (20, ws - 1, 4), (13, 0, 2), (18, 7, 3),
                           (22, 9, 7), (7, 580, 5), (23, -1, 2), (25, float("nan"), 8),
                           (24, binding.TUNE_NSPLIT, 8), (24, 4, 8)]:
        a = list(good)
        a[idx] = val
        assert f(*a) == code, (idx, val)


def _defrag(lib, **kw):
    a = dict(src=_FAKE, src_stride=576, dst=_FAKE, dst_stride=576, indptr=_FAKE, indices=_FAKE, base=_FAKE,
             out=_FAKE, batch=2, dtype=binding.BF16, stream=None)
    a.update(kw)
    return lib.tvmla_defrag(a["src"], a["src_stride"], a["dst"], a["dst_stride"], a["indptr"], a["indices"],
                            a["base"], a["out"], a["batch"], a["dtype"], a["stream"])


@pytest.mark.parametrize("field", ["src", "dst", "indptr", "indices", "base", "out"])
def test_defrag_null_pointer(lib, field):
    assert _defrag(lib, **{field: None}) == 1


@pytest.mark.parametrize("kw", [dict(batch=0), dict(batch=65536), dict(src_stride=575), dict(dst_stride=100)])
def test_defrag_bad_shape(lib, kw):
    assert _defrag(lib, **kw) == 2


@pytest.mark.parametrize("kw", [dict(dtype=2), dict(dtype=-1)])
def test_defrag_bad_dtype(lib, kw):
    assert _defrag(lib, **kw) == 3


@pytest.mark.parametrize("kw", [dict(src=_FAKE + 8), dict(dst=_FAKE + 4), dict(src_stride=580),
                                dict(dst_stride=578, dtype=binding.FP32)])
def test_defrag_misaligned(lib, kw):
    assert _defrag(lib, **kw) == 5


def _tree_mask(lib, **kw):
    a = dict(parents=_FAKE, indptr=_FAKE, batch=2, T=9, mask=_FAKE, mask_indptr=_FAKE, stream=None)
    a.update(kw)
    return lib.tvmla_tree_mask(a["parents"], a["indptr"], a["batch"], a["T"], a["mask"], a["mask_indptr"],
                               a["stream"])


@pytest.mark.parametrize("field", ["parents", "indptr", "mask", "mask_indptr"])
def test_tree_mask_null_pointer(lib, field):
    assert _tree_mask(lib, **{field: None}) == 1


@pytest.mark.parametrize("kw", [dict(batch=0), dict(batch=65536), dict(T=0), dict(T=65)])
def test_tree_mask_bad_shape(lib, kw):
    assert _tree_mask(lib, **kw) == 2


def test_noalloc_host_checks(lib):
    """tvmla_verify_noalloc rejects on the host, before any HIP call: a
    workspace beyond its scratch, bad flags, a NULL pointer, a bad shape."""
    f = lib.tvmla_verify_noalloc
    good = [_FAKE, 64 * 512, 512, _FAKE, 64 * 64, 64, _FAKE, 576, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, 1, 16, 64, 0.07,
            64, binding.BF16, _FAKE, _FAKE, None, 0, 0, 0, -1.0]
    # 1024 rows x 128 splits x 2 KB = 256 MiB, plus the lse region: one step past the scratch
    assert _layout_bytes(1, 16, 64, 128) > binding.NOALLOC_SCRATCH_BYTES >= _layout_bytes(1, 16, 64, 127)
    for idx, val, code in [(17, 128, 4), (24, 4, 8), (0, None, 1), (19, None, 1), (13, 0, 2), (17, 0, 2),
                           (18, 5, 3), (16, 0.0, 8), (6, _FAKE + 2, 5)]:
        a = list(good)
        a[idx] = val
        assert f(*a) == code, (idx, val)
