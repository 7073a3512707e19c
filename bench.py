"""Benchmark: tree-verify attention over an MLA latent cache at 185k context.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long185k]

One step = one verify call (split kernel + combine kernel) over the whole
synthetic batch, inputs resident in HBM: tvmla_verify_ex with
TVMLA_FLAG_TUNE_NSPLIT (the workload's NSPLIT adapted to the 256 compute
units). Prints ONE JSON line: value = effective KV-read GB/s (cache-row bytes
the call must read / time per call), plus us per call, the split kernel's
MFMA roofline fraction (timed live with HIP events through
tvmla_verify_partials on the same stream), and the fp64 CPU oracle timed on
the same workload (whole, or a bounded sample). The line also carries the
pages' own call -- tvmla_verify at exactly the workload's NSPLIT -- timed
the same way, the call captured in a HIP graph and replayed warm and cold
(L2 and MALL flushed before each replay), the HBM copy bandwidth and bf16
MFMA rate measured on the same GPU, and what the part sustains cold for the
call's bytes (a streaming read and a gather of the cache rows, with the
non-temporal loads the kernels use).

    python bench.py --op defrag|tree_mask [--workload W]

times the compaction kernel (cold copy rate as the value, warm beside it)
or the device-side tree mask instead.

    python bench.py --report

instead prints one diagnostic line per synthetic configuration (us per call
eager and graph-replayed warm/cold, KV-read GB/s and share of HBM peak, MFMA
share, roofline fraction max(t_HBM, t_MFMA) / t).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "us per verify call + effective KV-read GB/s (% HBM peak) at 185k ctx"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector ALU, TFLOP/s
FLOP_PER_ROW_KEY = 2 * 576 + 2 * 512  # QK over the 576-wide key + PV over the 512-wide latent


def algorithmic(w):
    """Algorithmic bytes and flops of one verify call on workload w."""
    keys = w.total_keys
    T, H = w.num_draft, w.num_heads
    esz = 2 if w.spec.dtype == "bf16" else 4
    kv_bytes = keys * 576 * esz
    meta_bytes = int(w.kv_indices.numel()) * 4 + w.batch * T * 4 + int(w.custom_mask.numel())
    q_bytes = w.batch * T * H * 576 * esz
    out_bytes = w.batch * T * H * (512 * esz + 4)
    flops = FLOP_PER_ROW_KEY * T * H * keys
    return dict(kv_bytes=kv_bytes, all_bytes=kv_bytes + meta_bytes + q_bytes + out_bytes, flops=flops)


KERNEL_OF_ALGO = {1: "split_scalar", 2: "split_mfma", 3: "split_rows"}
REPORT_WORKLOADS = ["tiny", "p4096", "long185k", "ragged32", "heavy200k", "heavy200k_contig", "long185k_h8"]
GRAPH_REPLAYS = 200
FLUSH_BYTES = 1 << 30  # a 1 GiB write evicts the 4 MB L2s and the 256 MB MALL


def _stats_us(ms_list):
    import numpy as np

    a = np.asarray(ms_list) * 1e3
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def graph_timing(torch, call_on, replays=GRAPH_REPLAYS):
    """Capture one call (call_on(stream) launches it on `stream`) in a HIP
    graph, then time `replays` replays, each bracketed by its own events:
    warm (back to back, the working set partly cached) and cold (an untimed
    1 GiB write before each replay). Returns µs statistics of both."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            call_on(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call_on(side)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    res = {}
    for mode in ("warm", "cold"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
        for i, (e0, e1) in enumerate(evs):
            if mode == "cold":
                scratch.fill_(i & 0xFF)
            e0.record(cur)
            g.replay()
            e1.record(cur)
        torch.cuda.synchronize()
        res[mode] = _stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    res["replays"] = replays
    del g, scratch
    return res


PROBE_SRC = os.path.join(ROOT, "bench_probes.hip")
PROBE_LIB = os.path.join(ROOT, "libtvmla_probe.so")


def build_probe(verbose=False):
    """Compile the matrix-core throughput probe (bench infrastructure, not
    part of libtvmla.so) into libtvmla_probe.so beside this file:
    python bench.py --build-probe (on the build machine, before a GPU run)."""
    from speculative_decoding_verify_mla_amd import build as tvbuild

    tmp = PROBE_LIB + ".tmp"
    tvbuild._run([tvbuild.HIPCC, *tvbuild.CFLAGS, "-shared", "-o", tmp, PROBE_SRC], verbose)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def measured_peaks(torch):
    """HBM bandwidth of a plain 1 GiB device copy (read + write bytes) and
    the bf16 MFMA rate of the throughput probe, on this GPU."""
    import ctypes

    dev = "cuda"
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del src, dst
    out = {"hbm_copy_GBps": round(copy_gbs, 1)}
    if not os.path.exists(PROBE_LIB):
        out["mfma_bf16_TFLOPs"] = None
        return out
    probe = ctypes.CDLL(PROBE_LIB)
    probe.tvmla_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    probe.tvmla_probe_mfma_flops.restype = ctypes.c_double
    probe.tvmla_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    blocks, iters = 512, 2000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        assert probe.tvmla_probe_mfma_bf16(sink.data_ptr(), blocks, iters, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        probe.tvmla_probe_mfma_bf16(sink.data_ptr(), blocks, iters, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    out["mfma_bf16_TFLOPs"] = round(probe.tvmla_probe_mfma_flops(blocks, iters) / (ms * 1e-3) / 1e12, 1)
    return out


def read_ceilings(torch, pool, kv_indices, kv_bytes):
    """What this GPU sustains, cold (L2 and MALL flushed before each of 10
    launches, median), for the bytes the verify call must read: a plain
    streaming read of kv_bytes (the pool's first rows) and a gather of
    exactly the workload's prefix rows through its kv_indices (the verify
    path's access pattern without its arithmetic). Both from
    bench_probes.hip; None if the probe library is not built."""
    import ctypes

    import numpy as np

    if not os.path.exists(PROBE_LIB):
        return None
    probe = ctypes.CDLL(PROBE_LIB)
    probe.tvmla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p]
    probe.tvmla_probe_gather_rows.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    row_bytes = pool.stride(0) * pool.element_size()
    nrows = int(kv_indices.numel())
    gather_bytes = nrows * 576 * pool.element_size()
    stream_bytes = min(kv_bytes, pool.numel() * pool.element_size()) // 16 * 16

    def cold(launch):
        for _ in range(3):
            assert launch() == 0
        ts = []
        for i in range(10):
            flush.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    t_stream = cold(lambda: probe.tvmla_probe_stream_read(pool.data_ptr(), stream_bytes, sink.data_ptr(), 2048,
                                                          stream.cuda_stream))
    # rows of 576 entries at the pool's row stride (1152 bytes for a bf16 pool of 576-wide rows)
    t_gather = cold(lambda: probe.tvmla_probe_gather_rows(pool.data_ptr(), row_bytes, kv_indices.data_ptr(), nrows,
                                                          sink.data_ptr(), 1024, stream.cuda_stream))
    del flush
    return {"stream_read_us": round(t_stream, 2), "stream_read_GBps": round(stream_bytes / (t_stream * 1e-6) / 1e9, 1),
            "gather_rows_us": round(t_gather, 2), "gather_rows_GBps": round(gather_bytes / (t_gather * 1e-6) / 1e9, 1),
            "bytes": stream_bytes, "rows": nrows, "row_bytes": int(row_bytes), "cache": "cold (1 GiB flushed)"}


def code_digest(path):
    """sha256 of a HIP source file's code: comments and blank space dropped,
    so that editing a comment does not mark a profile of the file stale."""
    import hashlib
    import re

    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = "\n".join(" ".join(line.split()) for line in text.split("\n") if line.strip())
    return hashlib.sha256(text.encode()).hexdigest()


def profiled_traffic(kernel):
    """HBM bytes per split launch of `kernel` (a csrc file stem) from the
    committed rocprofv3 summary, or None if there is none or the kernel's
    code has changed since those counters were taken."""
    import re

    prof = os.path.join(ROOT, "profiles", f"{kernel}_long185k.md")
    src = os.path.join(ROOT, "speculative_decoding_verify_mla_amd", "csrc", f"{kernel}.hip")
    try:
        text = open(prof).read()
        m = re.search(r"traffic_bytes_per_launch: fetch=(\d+) write=(\d+) code_sha256_prefix=([0-9a-f]+)", text)
        cur = code_digest(src)
    except OSError:
        return None
    if not m or not cur.startswith(m.group(3)):
        return None
    return int(m.group(1)) + int(m.group(2))


def cpu_baseline(w, pool_host):
    """Time the fp64 oracle on the same workload on the host cores. The whole
    job is the sample when it fits in about half a minute of CPU time;
    otherwise the rows of the first draft tokens (all heads), scaled."""
    from oracle import verify_fp64 as vo

    threads = blas_threads()
    T, H = w.num_draft, w.num_heads
    rows = w.batch * T * H
    kv = algorithmic(w)["kv_bytes"]
    whole = algorithmic(w)["flops"] <= 2e12  # ~0.5-2 TFLOP of fp64 BLAS: seconds to tens of seconds
    t0 = time.perf_counter()
    if whole:
        vo.verify(w.q_nope, w.q_rope, pool_host, w.kv_indptr, w.kv_indices, w.out_cache_loc, w.custom_mask,
                  w.mask_indptr, w.sm_scale, T)
        frac, what = 1.0, f"the whole job ({rows} query rows x {w.total_keys} keys), oracle.verify"
    else:
        tokens = min(2, T)
        picks = [(i, h) for i in range(tokens) for h in range(H)]
        vo.verify_rows(w.q_nope, w.q_rope, pool_host, w.kv_indptr, w.kv_indices, w.out_cache_loc, w.custom_mask,
                       w.mask_indptr, w.sm_scale, T, picks)
        frac = len(picks) / float(rows)
        what = f"oracle.verify_rows on {len(picks)} of {rows} query rows (draft tokens 0-{tokens - 1} of request 0)"
    dt = time.perf_counter() - t0
    return {
        "value": round(kv * frac / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what} in {dt:.2f} s; value = cache-row bytes x {frac:.4f} / time",
        "seconds": round(dt, 3),
        "cpu_model": cpu_model(),
        "cpu_count": os.cpu_count(),
    }


def blas_threads():
    """Threads the fp64 oracle's BLAS runs with (its matrix products are
    where the oracle spends its time)."""
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the OMP setting
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_defrag(args, w, torch, binding):
    """tvmla_defrag on the workload: every prefix moves to a fresh contiguous
    run appended to the cache (indices written to a separate array, so each
    timed call does the same work). HBM-bound: per moved row 2 x 576 x
    elem_size bytes plus 8 bytes of indices. Timed cold (the median of single
    calls, each after an untimed 1 GiB write that evicts the L2s and the
    MALL: the value and the roofline) and warm (back to back: a destination
    that fits the 256 MB MALL is then partly absorbed there, so warm can run
    above what HBM delivers). Also times the verify step on the scattered and
    on the compacted layout (the read-side gain)."""
    import numpy as np

    dev = "cuda"
    pool = w.device_pool(dev, fill=0.0)
    P = np.diff(w.kv_indptr.numpy())
    n = int(P.sum())
    first = pool.shape[0]
    pool = torch.cat([pool, torch.zeros((n, pool.shape[1]), dtype=pool.dtype, device=dev)], 0)
    bases = torch.from_numpy((first + np.concatenate([[0], np.cumsum(P)[:-1]])).astype(np.int32)).to(dev)
    indptr, idx = w.kv_indptr.to(dev), w.kv_indices.to(dev)
    new_idx = torch.empty_like(idx)
    stream = torch.cuda.current_stream()

    def timed(fn, k):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    def defrag():
        binding.defrag(pool, pool, indptr, idx, bases, new_idx, stream=stream)

    T, H, ns = w.num_draft, w.num_heads, w.spec.nsplit
    q_nope, q_rope = w.q_nope.to(dev), w.q_rope.to(dev)
    ocl, mask, mask_indptr = w.out_cache_loc.to(dev), w.custom_mask.to(dev), w.mask_indptr.to(dev)
    out = torch.empty((w.batch * T, H, 512), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((w.batch * T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.workspace_bytes(w.batch, T, H, ns), dtype=torch.uint8, device=dev)

    def verify_with(indices):
        return lambda: binding.verify(q_nope, q_rope, pool, indptr, indices, ocl, mask, mask_indptr, w.sm_scale,
                                      ns, out, lse, ws, T, stream=stream)

    def cold_ms(fn, k):
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        ts = []
        for i in range(k):
            flush.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        del flush
        return float(np.median(ts))

    for _ in range(max(args.warmup, 20)):
        defrag()
    ms_warm = timed(defrag, args.steps)
    ms_defrag = cold_ms(defrag, max(args.steps, 10))
    for _ in range(max(args.warmup, 20)):
        verify_with(idx)()
    ms_scattered = timed(verify_with(idx), args.steps)
    ms_compact = timed(verify_with(new_idx), args.steps)
    esz = pool.element_size()
    moved = n * (2 * 576 * esz + 8)
    gbs = moved / (ms_defrag * 1e-3) / 1e9
    gbs_warm = moved / (ms_warm * 1e-3) / 1e9
    print(json.dumps({
        "metric": "tvmla_defrag GB/s moved, cold caches (HBM roofline), and verify step before/after compaction",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "us_per_defrag": round(ms_defrag * 1e3, 2), "rows_moved": n, "bytes_moved": moved,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "warm": {"us_per_defrag": round(ms_warm * 1e3, 2), "GBps": round(gbs_warm, 2),
                 "frac": round(gbs_warm / HBM_PEAK_GBS, 4)},
        "verify_us": {"scattered": round(ms_scattered * 1e3, 2), "compacted": round(ms_compact * 1e3, 2)},
        "config": {"workload": args.workload, "batch": w.batch, "num_draft": T, "num_heads": H, "nsplit": ns},
        "dtype": w.spec.dtype, "data": "synthetic",
    }), flush=True)
    return 0


def bench_tree_mask(args, w, torch, binding):
    """tvmla_tree_mask on the workload's trees: T * N_b mask bytes written per
    request (HBM-bound when large, launch-bound when small)."""
    import numpy as np

    dev = "cuda"
    T = w.num_draft
    parents = torch.from_numpy(np.concatenate(w.parents).astype(np.int32)).to(dev)
    indptr = w.kv_indptr.to(dev)
    mask = torch.empty_like(w.custom_mask, device=dev)
    mindptr = torch.empty_like(w.mask_indptr, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        binding.tree_mask(parents, indptr, T, mask, mindptr, stream=stream)

    for _ in range(max(args.warmup, 20)):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = mask.numel() + 4 * (mindptr.numel() + indptr.numel() + parents.numel())
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "tvmla_tree_mask us per call (mask bytes written, HBM roofline)",
        "value": round(ms * 1e3, 2), "unit": "us", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
        "mask_bytes": mask.numel(),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "config": {"workload": args.workload, "batch": w.batch, "num_draft": T}, "data": "synthetic",
    }), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="long185k")
    ap.add_argument("--algo", type=int, default=0, help="0 auto, 1 scalar, 2 mfma (64 rows), 3 mfma (128 rows)")
    ap.add_argument("--min-chunk", type=int, default=0)
    ap.add_argument("--nsplit", type=int, default=0, help="override the workload's split count (diagnostics)")
    ap.add_argument("--op", default="verify", choices=["verify", "defrag", "tree_mask"],
                    help="defrag: time tvmla_defrag on the workload (a separate diagnostic line, not the "
                         "verify bench line) and the verify step before and after compaction")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="run only the settle phase, the warm-up and the K timed steps of the bench call (no "
                         "split-only, combine-only or exact-NSPLIT timings, graph replays, peaks or CPU baseline), "
                         "so that a profiler run sees one dispatch shape per kernel")
    ap.add_argument("--build-probe", action="store_true",
                    help="compile the MFMA throughput probe (libtvmla_probe.so) and exit; no GPU needed")
    ap.add_argument("--report", action="store_true",
                    help="one diagnostic line per synthetic configuration instead of the bench line")
    ap.add_argument("--report-workloads", default=",".join(REPORT_WORKLOADS),
                    help="comma-separated configurations for --report")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the verify step, time a plain device copy of this many MiB "
                         "(reference kernel for scaling HBM traffic counters)")
    args = ap.parse_args(argv)

    if args.build_probe:
        print(build_probe(verbose=True))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify path shards by heads or requests with no exchange)", file=sys.stderr)
        return 2

    import torch

    from speculative_decoding_verify_mla_amd import binding
    from workloads import gen

    binding.load()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda"
    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"copy_bytes": n, "ms": ms, "read_write_GBps": 2 * n / (ms * 1e-3) / 1e9}), flush=True)
        return 0
    if args.report:
        return report(args, torch, binding)
    w = gen.build(args.workload, **({"nsplit": args.nsplit} if args.nsplit else {}))
    if args.op == "defrag":
        return bench_defrag(args, w, torch, binding)
    if args.op == "tree_mask":
        return bench_tree_mask(args, w, torch, binding)
    if args.step_only:
        return step_only(args, w, torch, binding)
    res = measure(args, w, args.workload, torch, binding)
    res["measured_peaks"] = measured_peaks(torch)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        host_pool = w.host_pool(fill=0.0)
        res["cpu_baseline"] = cpu_baseline(w, host_pool)
    print(json.dumps(res), flush=True)
    return 0


def step_only(args, w, torch, binding):
    """The bench call alone (tuned split count), for profiler runs: settle,
    warm-up, then K timed steps; prints us per call."""
    dev = "cuda"
    T, H, ns = w.num_draft, w.num_heads, w.spec.nsplit
    pool = w.device_pool(dev, fill=0.0)
    q_nope, q_rope = w.q_nope.to(dev), w.q_rope.to(dev)
    kv_indptr, kv_indices = w.kv_indptr.to(dev), w.kv_indices.to(dev)
    ocl, mask, mask_indptr = w.out_cache_loc.to(dev), w.custom_mask.to(dev), w.mask_indptr.to(dev)
    out = torch.empty((w.batch * T, H, 512), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((w.batch * T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.workspace_bytes(w.batch, T, H, ns), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        binding.verify(q_nope, q_rope, pool, kv_indptr, kv_indices, ocl, mask, mask_indptr, w.sm_scale, ns, out, lse,
                       ws, T, algo=args.algo, min_chunk=args.min_chunk, flags=binding.TUNE_NSPLIT, stream=stream)

    t0 = time.perf_counter()
    settle = 0
    while time.perf_counter() - t0 < 0.15:
        for _ in range(10):
            step()
        settle += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"workload": args.workload, "us_per_call": round(ms * 1e3, 2), "settle_calls": settle,
                      "warmup": args.warmup, "steps": args.steps,
                      "nsplit_effective": binding.effective_nsplit(w.batch, T, H, ns)}), flush=True)
    return 0


def measure(args, w, name, torch, binding, graph=True):
    """The verify call on workload w: eager step, split-only and combine-only
    times, the roofline of the split kernel, and (graph=True) the call
    replayed from a HIP graph, warm and cold. Returns the bench line."""
    dev = "cuda"
    T, H, ns = w.num_draft, w.num_heads, w.spec.nsplit
    dcode = 0 if w.spec.dtype == "bf16" else 1
    # the split count the tuned call runs (tvmla_effective_nsplit); the
    # split-only and combine-only timings use it too, so they time the same
    # launches as the step
    ns_eff = binding.effective_nsplit(w.batch, T, H, ns)
    algo_used = args.algo or binding.auto_algo(w.batch, T, H, ns_eff, dcode)
    algo_exact = args.algo or binding.auto_algo(w.batch, T, H, ns, dcode)
    kernel = KERNEL_OF_ALGO.get(algo_used, "split")
    pool = w.device_pool(dev, fill=0.0)
    kv = pool
    q_nope, q_rope = w.q_nope.to(dev), w.q_rope.to(dev)
    kv_indptr, kv_indices = w.kv_indptr.to(dev), w.kv_indices.to(dev)
    ocl, mask, mask_indptr = w.out_cache_loc.to(dev), w.custom_mask.to(dev), w.mask_indptr.to(dev)
    ntok = w.batch * T
    out = torch.empty((ntok, H, 512), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((ntok, H), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.workspace_bytes(w.batch, T, H, ns), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step_on(st):
        binding.verify(q_nope, q_rope, kv, kv_indptr, kv_indices, ocl, mask, mask_indptr, w.sm_scale, ns, out, lse,
                       ws, T, algo=args.algo, min_chunk=args.min_chunk, flags=binding.TUNE_NSPLIT, stream=st)

    def step():
        step_on(stream)

    def exact_step():
        # the pages' call: exactly the workload's NSPLIT
        if args.algo == 0 and args.min_chunk == 0:
            binding.verify_plain(q_nope, q_rope, kv, kv_indptr, kv_indices, ocl, mask, mask_indptr, w.sm_scale, ns,
                                 out, lse, ws, T, stream=stream)
        else:
            binding.verify(q_nope, q_rope, kv, kv_indptr, kv_indices, ocl, mask, mask_indptr, w.sm_scale, ns, out,
                           lse, ws, T, algo=args.algo, min_chunk=args.min_chunk, stream=stream)

    # the two steps apart, launched exactly as the tuned call launches them
    def split_only():
        binding.verify_partials(q_nope, q_rope, kv, kv_indptr, kv_indices, ocl, mask, mask_indptr, w.sm_scale,
                                ns_eff, ws, T, algo=args.algo, min_chunk=args.min_chunk, flags=binding.TILE_CHUNKS,
                                stream=stream)

    def combine_only():
        binding.combine(ws, kv_indptr, w.batch, T, H, ns_eff, out, lse, min_chunk=args.min_chunk,
                        flags=binding.TILE_CHUNKS, stream=stream)

    def timed(fn, k):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k  # ms

    # Power-state settle (untimed): the GPU reaches steady clocks only after
    # some tens of milliseconds of load, and calls made before that run up to
    # ~15% slower. Serving runs at steady clocks, so before the warm-up steps
    # the step runs in batches of 10 until 150 ms of load have passed.
    settle_calls, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < 0.15:
        for _ in range(10):
            step()
        settle_calls += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {name}: warmup done", file=sys.stderr, flush=True)
    ms_step = timed(step, args.steps)
    ms_split = timed(split_only, args.steps)
    ms_combine = timed(combine_only, args.steps)
    assert torch.isfinite(lse).all(), "non-finite lse"
    for _ in range(args.warmup):
        exact_step()
    ms_exact = timed(exact_step, args.steps)
    assert torch.isfinite(lse).all(), "non-finite lse"
    print(f"[bench] {name}: step {ms_step * 1e3:.1f} us, split {ms_split * 1e3:.1f} us, combine "
          f"{ms_combine * 1e3:.1f} us; tvmla_verify at nsplit {ns}: {ms_exact * 1e3:.1f} us", file=sys.stderr,
          flush=True)
    graph_us = graph_timing(torch, step_on) if graph else None
    ceilings = read_ceilings(torch, pool, kv_indices, algorithmic(w)["kv_bytes"]) if graph else None

    alg = algorithmic(w)
    kv_gbs = alg["kv_bytes"] / (ms_step * 1e-3) / 1e9
    split_tflops = alg["flops"] / (ms_split * 1e-3) / 1e12
    # the split kernel is MFMA-bound when its flops per KV byte exceed the
    # ridge point (peak flops / peak bandwidth), HBM-bound otherwise
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if alg["flops"] / alg["kv_bytes"] >= ridge:
        roof = dict(bound="mfma", achieved=round(split_tflops, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(split_tflops / MFMA_BF16_PEAK_TFLOPS, 4))
    else:
        split_gbs = alg["all_bytes"] / (ms_split * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(split_gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(split_gbs / HBM_PEAK_GBS, 4))
    res = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_calls": settle_calls,
        "ms_per_step": round(ms_step, 5),
        "us_per_call": round(ms_step * 1e3, 2),
        "hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.spec.dtype,
        "data": "synthetic",
        "config": {
            "workload": name,
            "batch": w.batch,
            "prefix": int(w.prefix_lens[0]) if len(set(w.prefix_lens.tolist())) == 1 else "ragged",
            "num_draft": T,
            "num_heads": H,
            "nsplit": ns,
            "nsplit_effective": ns_eff,
            "min_chunk": args.min_chunk,
            "algo": algo_used,
            "pool_slots": w.spec.pool_slots,
            "layout": w.spec.layout,
            "kv_bytes": alg["kv_bytes"],
            "flops": alg["flops"],
        },
        "kernels_us": {"split": round(ms_split * 1e3, 2), "combine": round(ms_combine * 1e3, 2)},
        "nsplit_exact_call": {"api": "tvmla_verify", "nsplit": ns, "algo": algo_exact,
                              "us_per_call": round(ms_exact * 1e3, 2),
                              "kv_GBps": round(alg["kv_bytes"] / (ms_exact * 1e-3) / 1e9, 2)},
        "roofline": dict(roof, kernel=kernel,
                         traffic=profiled_traffic(kernel) if name == "long185k" and args.min_chunk == 0 else None),
    }
    if graph_us is not None:
        res["graph_us"] = graph_us
    if ceilings is not None:
        res["read_ceilings"] = ceilings
    del pool, kv, ws
    return res


def report(args, torch, binding):
    """One diagnostic line per synthetic configuration (not the bench line):
    the whole call against both roofs, t_HBM = all algorithmic bytes / 8 TB/s
    and t_compute = flops / the dtype's peak (bf16 MFMA 2.5 PFLOP/s; fp32
    vector 157.3 TFLOP/s for the fp32 configuration), and the fp64 oracle
    timed once per configuration on the host cores (thread count and CPU
    model recorded)."""
    from workloads import gen

    for name in args.report_workloads.split(","):
        w = gen.build(name)
        r = measure(args, w, name, torch, binding)
        alg = algorithmic(w)
        t = r["us_per_call"] * 1e-6
        peak = MFMA_BF16_PEAK_TFLOPS if w.spec.dtype == "bf16" else FP32_VECTOR_PEAK_TFLOPS
        t_hbm = alg["all_bytes"] / (HBM_PEAK_GBS * 1e9)
        t_cmp = alg["flops"] / (peak * 1e12)
        line = {
            "metric": "verify call per configuration: us, KV-read GB/s, roofline fractions",
            "workload": name, "dtype": w.spec.dtype, "us_per_call": r["us_per_call"], "graph_us": r["graph_us"],
            "kv_GBps": r["value"], "hbm_frac": r["hbm_frac"],
            "compute_frac": round(t_cmp / t, 4), "compute_peak_TFLOPs": peak,
            "bound": "hbm" if t_hbm >= t_cmp else ("mfma" if w.spec.dtype == "bf16" else "valu"),
            "roofline_frac": round(max(t_hbm, t_cmp) / t, 4),
            "t_hbm_us": round(t_hbm * 1e6, 2), "t_compute_us": round(t_cmp * 1e6, 2),
            "kernels_us": r["kernels_us"], "split_roofline": r["roofline"],
            "nsplit_exact_call": r["nsplit_exact_call"], "read_ceilings": r.get("read_ceilings"),
            "config": r["config"],
        }
        if not args.no_cpu_baseline:
            print(f"[bench] {name}: timing the CPU oracle", file=sys.stderr, flush=True)
            line["cpu_baseline"] = cpu_baseline(w, w.host_pool(fill=0.0))
        print(json.dumps(line), flush=True)
        del w
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
