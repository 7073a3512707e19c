"""Host-side pieces of bench.py that decide what the bench line reports.

The bench line's `roofline.traffic` comes from the committed rocprofv3
summary of the split kernel, and only while the kernel's code is the code
those counters were taken on. The check compares a digest of the source
with comments and blank space removed, so these tests pin what it must and
must not react to.
"""
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = """// a kernel
__global__ void k(float* p) {  // one thread
  /* scale
     by two */
  p[threadIdx.x] *= 2.f;
}
"""


def _digest(tmp_path, text, name="k.hip"):
    f = tmp_path / name
    f.write_text(text)
    return bench.code_digest(str(f))


def test_digest_ignores_comments_and_blank_space(tmp_path):
    base = _digest(tmp_path, SRC)
    edited = SRC.replace("// a kernel", "// a kernel that doubles").replace("/* scale\n     by two */", "/* x2 */")
    assert _digest(tmp_path, edited) == base
    reindented = "\n\n" + SRC.replace("  p[", "      p[").replace("{  //", "{    //") + "\n"
    assert _digest(tmp_path, reindented) == base


def test_digest_sees_code_changes(tmp_path):
    base = _digest(tmp_path, SRC)
    assert _digest(tmp_path, SRC.replace("2.f", "3.f")) != base
    assert _digest(tmp_path, SRC.replace("threadIdx.x", "threadIdx.y")) != base
    # a cache-policy immediate is code too
    a = "__builtin_amdgcn_global_load_lds(a, l, 16, 0, 0);\n"
    assert _digest(tmp_path, a) != _digest(tmp_path, a.replace("0, 0)", "0, 2)"))


def test_committed_profile_matches_current_kernel():
    """The headline profile names the digest of the split kernel in the
    tree, so the bench line carries its traffic figure."""
    t = bench.profiled_traffic("split_rows")
    assert t is not None, "profiles/split_rows_long185k.md is stale against csrc/split_rows.hip"
    assert 2e8 < t < 4e8  # 213 MB of cache rows read plus the partial rows, at long185k
