#!/usr/bin/env python3
"""Throughput of the compressed sparse attention hot path on one MI355X.

A step is one pass of the whole hot path (fp4 round trip of the step's new
latent and indexer-k rows, ring write, window columns, indexer scores + top-k,
sparse attention with the sink) over one batch: B independent sequences of a
workload, every input resident in HBM before the timed region.

Default workload: decode, m = 1 at start_pos = 32767, 64 heads x 512, window
128, ratio 4 (8192 compressed rows), indexer 64 x 128 with top-512, batched
over B = 2048 independent sequences (eight attention workgroups per compute
unit and call, two at a time, so that the launch, dispatch and
per-workgroup start-up cost is spread over more queries); one step streams
~2.8 GB, far past the 256 MB last-level cache.

Prints ONE JSON line (stdout): metric tokens/s, roofline of the dominant
kernel (HIP-event time on the library's stream), and the oracle timed on the
host cores as a CPU baseline.  Everything else goes to stderr.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, datasheet
FP4_PEAK_TFLOPS = 10100.0   # MI355X dense fp4 (MXFP4) MFMA, datasheet

DEFAULT_B = {"tiny_decode": 1, "decode": 2048, "long_decode": 512, "causal_prefill": 1, "chunked_prefill": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def describe(w):
    s = (f"{w.name}: m={w.m} start_pos={w.start_pos} H={w.H} D={w.D} win={w.win} ratio={w.ratio} "
         f"n_c={w.n_c}")
    if w.Hi:
        s += f" indexer {w.Hi}x{w.Di} top-{w.K}"
    else:
        s += f" all visible compressed rows (<= {w.K})"
    return s


def counts(w, B, call, kcache="bf16", latent="bf16"):
    """Algorithmic bytes and flops of one library call for one step of B
    sequences: what the method must read and write (each needed row once,
    valid (query, row) pairs only) in the storage the step uses: bf16 rows as
    on the pages, or, for the packed caches, codes + scale bytes (an indexer k
    row 68 B at Di = 128, a latent row 288 B at D = 512).  The
    implementation's workspace traffic is not counted.  bound: the roofline
    the call is judged against."""
    m, win, D = w.m, w.win, w.D
    V = [min(w.n_c, (w.start_pos + t + 1) // w.ratio) for t in range(m)]
    Wv = [min(win, w.start_pos + t + 1) for t in range(m)]
    C = [min(w.K, v) for v in V]
    pairs = sum(Wv) + sum(C)
    n_new = w.n_c - w.first_new_row
    dense = m > 1
    lrow = D // 2 + D // 16 if latent == "fp4" else D * 2  # stored bytes of a latent row
    if call == "quant_latent":
        return {"bytes": B * n_new * (D * 2 + lrow), "flops": 0, "bound": "hbm"}
    krow = w.Di // 2 + w.Di // 32 if kcache == "fp4" else w.Di * 2  # stored bytes of an indexer k row
    if call == "quant_index_k":
        return {"bytes": B * n_new * (w.Di * 2 + krow), "flops": 0, "bound": "hbm"}
    if call == "ring_write":
        return {"bytes": B * min(m, win) * D * 4, "flops": 0, "bound": "hbm"}
    if call == "window_idx":
        return {"bytes": B * m * win * 4, "flops": 0, "bound": "hbm"}
    if call == "decode_step":  # a whole small-batch decode step in one launch
        parts = [counts(w, B, c, kcache, latent) for c in ("decode_prepare", "index_scores_topk", "sparse_attn_sink")]
        return {"bytes": sum(c["bytes"] for c in parts), "flops": sum(c["flops"] for c in parts), "bound": "hbm"}
    if call == "decode_prepare":  # the four set-up calls of a decode step in one launch
        return {"bytes": sum(counts(w, B, c, kcache, latent)["bytes"]
                             for c in ("quant_latent", "quant_index_k", "ring_write", "window_idx")),
                "flops": 0, "bound": "hbm"}
    if call == "visible_idx":
        return {"bytes": B * m * w.K * 4, "flops": 0, "bound": "hbm"}
    if call == "prefill_prepare":  # the set-up calls of a step that is not a decode step, in one launch
        parts = ["quant_latent"] + (["quant_index_k", "window_idx"] if w.Hi else ["window_idx", "visible_idx"])
        parts += ["ring_write"] if w.start_pos == 0 else []
        return {"bytes": sum(counts(w, B, c, kcache, latent)["bytes"] for c in parts), "flops": 0, "bound": "hbm"}
    if call == "index_scores_topk":
        # flops: only queries that see more than K rows need scores (a query
        # seeing V <= K rows selects all of them); the all-visible-pairs count
        # is reported beside it
        by = B * (max(V) * krow + m * w.Hi * w.Di * 2 + m * w.Hi * 4 + m * w.K * 4)
        fl = B * sum(v for v in V if v > w.K) * w.Hi * w.Di * 2
        return {"bytes": by, "flops": fl, "bound": "mfma" if dense else "hbm",
                "flops_all_visible": B * sum(V) * w.Hi * w.Di * 2}
    if call == "sparse_attn_sink":
        rows = (w.m if w.start_pos == 0 else (win + m if m > 1 else None))
        row_bytes = (rows * D * 2 + w.n_c * lrow) if rows is not None else (sum(Wv) * D * 2 + sum(C) * lrow)
        by = B * (row_bytes + 2 * m * w.H * D * 2 + m * w.T * 4 + w.H * 4)
        fl = B * pairs * w.H * D * 4
        return {"bytes": by, "flops": fl, "bound": "mfma" if dense else "hbm"}
    raise KeyError(call)


def kernel_source_hash():
    """Hash of the kernel sources with comments and blank space removed, so that
    only code changes invalidate counters taken earlier."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_compressed_kv_e2m1_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f == "peak.hip":  # measurement kernels, not the hot path
            continue
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_for(workload, B, call, kcache, latent="bf16"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    lat = "" if latent == "bf16" else f"/latent_{latent}"
    entry = rec.get("entries", {}).get(f"{workload}/B{B}/{kcache}{lat}/{call}")
    return None if entry is None else entry.get("hbm_bytes_per_launch")


# Library call -> the kernels it launches (demangled-name prefixes).
CALL_KERNELS = {
    "quant_latent": ["quant_rows_kernel<0,", "quant_pack_kernel<0,"],
    "quant_index_k": ["quant_rows_kernel<1,", "quant_pack_kernel<1,"],
    "ring_write": ["ring_write_kernel"],
    "decode_prepare": ["decode_prepare_kernel"],
    "prefill_prepare": ["prefill_prepare_kernel"],
    "decode_step": ["decode_step_kernel"],
    "window_idx": ["window_idx_kernel"],
    "visible_idx": ["visible_idx_kernel"],
    "index_scores_topk": ["index_score_kernel", "topk_kernel"],
    "sparse_attn_sink": ["sparse_attn_kernel", "combine_kernel"],
}


def _kernel_short(name):
    name = re.sub(r"^void ", "", name)
    name = name.replace("sckv::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name).replace(" ", "")


def _steady_groups(rows, key):
    """Per kernel: the dispatches of its most frequent grid size (the step's
    launches; one-off set-up launches of other sizes drop out)."""
    groups = {}
    for r in rows:
        if "sckv::" not in r["Kernel_Name"]:
            continue
        groups.setdefault(_kernel_short(r["Kernel_Name"]), {}).setdefault(key(r), []).append(r)
    return {k: max(v.values(), key=len) for k, v in groups.items()}


def _csv_rows(folder, suffix):
    import csv  # noqa: PLC0415
    import glob  # noqa: PLC0415

    paths = glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)
    if len(paths) != 1:
        raise SystemExit(f"expected one *{suffix} under {folder}, found {paths}")
    return list(csv.DictReader(open(paths[0])))


# Matrix-core and LDS counters of one --pmc pass (6 SQ counters + 1 GRBM),
# and the MI355X unit counts the ratios divide by.
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F6F4",
               "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"]
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8  # GRBM_GUI_ACTIVE comes summed over the 8 XCDs


def _sq_counters(folder):
    """Per kernel (steady-state dispatches): the average per dispatch of each
    counter of the SQ/ pass under folder, or {} without one."""
    d = os.path.join(folder, "SQ")
    if not os.path.isdir(d):
        return {}
    g = _steady_groups(_csv_rows(d, "counter_collection.csv"), lambda r: r["Grid_Size"])
    out = {}
    for k, rows in g.items():
        nd = len({r["Dispatch_Id"] for r in rows})
        acc, span = {}, {}
        for r in rows:
            acc[r["Counter_Name"]] = acc.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            span[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        out[k] = {c: v / nd for c, v in acc.items()}
        out[k]["duration_ns"] = sum(span.values()) / len(span)
    return out


def summarize_profiles(w, B, folder, commands, kcache="bf16", latent="bf16"):
    """Turn rocprofv3 output under `folder` (trace/, FETCH_SIZE/, WRITE_SIZE/,
    SQ/, copy_FETCH_SIZE/, copy_WRITE_SIZE/) into the text summary
    profiles/hot_path_kernels_<workload>_B<B>.txt and the HBM-traffic entries
    of profiles/traffic.json (counter KiB per dispatch, scaled so that a plain
    1 GiB device copy reads and writes 1 GiB)."""
    tr = _steady_groups(_csv_rows(os.path.join(folder, "trace"), "kernel_trace.csv"),
                        lambda r: (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"]))
    # durations after the warm-up launches (the first 40% of a kernel's
    # dispatches: the GPU's clocks are still settling there)
    tr = {k: sorted(v, key=lambda r: int(r["Start_Timestamp"]))[(len(v) * 2) // 5:] for k, v in tr.items()}
    dur = {k: sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in v) / len(v) / 1e3
           for k, v in tr.items()}
    calls = {k: len(v) for k, v in tr.items()}
    res = {"FETCH_SIZE": None, "WRITE_SIZE": None}
    scale = {}
    for c in res:
        d = os.path.join(folder, c)
        if not os.path.isdir(d):
            continue
        g = _steady_groups(_csv_rows(d, "counter_collection.csv"), lambda r: r["Grid_Size"])
        res[c] = {k: sum(float(r["Counter_Value"]) for r in v) / len(v) * 1024 for k, v in g.items()}
        cdir = os.path.join(folder, "copy_" + c)
        if not os.path.isdir(cdir):  # one calibration next to several workloads' folders
            cdir = os.path.join(os.path.dirname(os.path.normpath(folder)), "copy_" + c)
        cp = _csv_rows(cdir, "counter_collection.csv")
        # the 1 GiB copy: the largest per-dispatch value of the copy kernel
        copy_bytes = max(float(r["Counter_Value"]) * 1024 for r in cp if "copyBuffer" in r["Kernel_Name"]
                         or "copy" in r["Kernel_Name"].lower())
        scale[c] = (1 << 30) / copy_bytes
    lines = [f"# rocprofv3 summary: compressed sparse attention hot path, {describe(w)}, B={B}"
             + (f", indexer k cache {kcache}" if w.Hi else "") + f", latent cache {latent}", "#"]
    lines += ["# commands (repo root as working directory):"] + [f"#   {c}" for c in commands]
    lines += [f"# counter scale (1 GiB device copy): FETCH_SIZE x{scale.get('FETCH_SIZE', float('nan')):.3f}, "
              f"WRITE_SIZE x{scale.get('WRITE_SIZE', float('nan')):.3f}",
              "# steady-state dispatches only (most frequent grid size per kernel; durations after the first 40%"
              " of its dispatches, the warm-up)", "#",
              f"{'kernel':<44} {'calls':>5} {'avg_us':>9} {'read_MB':>9} {'write_MB':>9}"]
    # only the kernels of the step's own calls (set-up launches are left out)
    from sparse_compressed_kv_e2m1_amd.step import step_call_names  # noqa: PLC0415
    names = step_call_names(w, kcache, latent, B)
    mine = lambda k: any(k.startswith(p.replace(" ", "")) for c in names for p in CALL_KERNELS[c])  # noqa: E731
    dur = {k: v for k, v in dur.items() if mine(k)}
    for k in sorted(dur, key=lambda k: -dur[k]):
        rd = res["FETCH_SIZE"].get(k) if res["FETCH_SIZE"] else None
        wr = res["WRITE_SIZE"].get(k) if res["WRITE_SIZE"] else None
        rd = "-" if rd is None else f"{rd * scale['FETCH_SIZE'] / 1e6:.2f}"
        wr = "-" if wr is None else f"{wr * scale['WRITE_SIZE'] / 1e6:.2f}"
        lines.append(f"{k[:44]:<44} {calls[k]:>5} {dur[k]:>9.2f} {rd:>9} {wr:>9}")
    sq = _sq_counters(folder)
    if sq:
        lines += ["#", "# matrix-core and LDS counters (one rocprofv3 --pmc pass: " + " ".join(SQ_COUNTERS) + ")",
                  f"#   gui        = GRBM_GUI_ACTIVE / {XCD_NUM} (the counter is summed over the XCDs): active cycles",
                  f"#   mfma_busy  = SQ_VALU_MFMA_BUSY_CYCLES / (gui x {SIMD_NUM} SIMDs)",
                  "#   mfma_GFLOP = (SQ_INSTS_VALU_MFMA_MOPS_BF16 + SQ_INSTS_VALU_MFMA_MOPS_F6F4) x 512",
                  f"#   lds_active = SQ_LDS_IDX_ACTIVE / (gui x {CU_NUM} CUs); "
                  "bank_conf = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
                  "#   gui_GHz    = gui / the dispatch's duration in this pass (the clock the kernel ran at)",
                  f"{'kernel':<44} {'mfma_busy':>9} {'mfma_GFLOP':>10} {'lds_active':>10} {'bank_conf':>9} "
                  f"{'lds_instr':>10} {'gui_GHz':>7}"]
        for k in sorted(dur, key=lambda k: -dur[k]):
            c = sq.get(k)
            if not c or not c.get("GRBM_GUI_ACTIVE"):
                continue
            gui = c["GRBM_GUI_ACTIVE"] / XCD_NUM
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (gui * SIMD_NUM)
            fl = (c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0)) * 512 / 1e9
            act = c.get("SQ_LDS_IDX_ACTIVE", 0) / (gui * CU_NUM)
            bc = c.get("SQ_LDS_BANK_CONFLICT", 0) / max(1.0, c.get("SQ_LDS_IDX_ACTIVE", 0))
            ghz = gui / c["duration_ns"] if c.get("duration_ns") else float("nan")
            lines.append(f"{k[:44]:<44} {busy:>9.1%} {fl:>10.2f} {act:>10.1%} {bc:>9.1%} "
                         f"{c.get('SQ_INSTS_LDS', 0):>10.3g} {ghz:>7.2f}")
    lines += ["#", f"{'library call':<20} {'avg_us':>9} {'alg_MB':>9} {'hbm_MB':>9}"]
    entries = {}
    for call in dict.fromkeys(names):
        pre = CALL_KERNELS[call]
        ks = [k for k in dur if any(k.startswith(p.replace(" ", "")) for p in pre)]
        if not ks:
            continue
        us = sum(dur[k] for k in ks)
        hbm = None
        if res["FETCH_SIZE"] and res["WRITE_SIZE"] and all(k in res[c] for c in res for k in ks):
            hbm = sum(res["FETCH_SIZE"].get(k, 0) * scale["FETCH_SIZE"] + res["WRITE_SIZE"].get(k, 0)
                      * scale["WRITE_SIZE"] for k in ks)
        alg = counts(w, B, call, kcache, latent)["bytes"]
        lines.append(f"{call:<20} {us:>9.2f} {alg / 1e6:>9.2f} {'-' if hbm is None else f'{hbm / 1e6:.2f}':>9}")
        lat = "" if latent == "bf16" else f"/latent_{latent}"
        entries[f"{w.name}/B{B}/{kcache if w.Hi else 'none'}{lat}/{call}"] = {"kernels": ks, "avg_us": round(us, 3),
                                            "hbm_bytes_per_launch": None if hbm is None else int(hbm)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    kc = (f"_kcache_{kcache}" if w.Hi else "") + ("" if latent == "bf16" else f"_latent_{latent}")
    out = os.path.join(ROOT, "profiles", f"hot_path_kernels_{w.name}_B{B}{kc}.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    tj = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(tj)) if os.path.exists(tj) else {}
    if rec.get("kernel_source_hash") != kernel_source_hash():
        rec = {"kernel_source_hash": kernel_source_hash(), "entries": {}}
    rec["note"] = ("HBM bytes per library call (all its kernels), rocprofv3 FETCH_SIZE + WRITE_SIZE scaled by a "
                   "1 GiB copy; valid only for the kernel sources whose hash is kernel_source_hash")
    if res["FETCH_SIZE"] and res["WRITE_SIZE"]:
        rec["entries"].update(entries)
    json.dump(rec, open(tj, "w"), indent=1, sort_keys=True)
    log(f"wrote {out} and {tj}")


def cpu_info():
    """Host CPU model and the CPUs this process may run on."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_available": avail}


def cpu_baseline(w, seconds, threads):
    """The oracle as it stands on a bounded sample of the same workload, on one
    thread and on `threads` threads (the oracle's C calls release the GIL;
    work is split over independent sequences for decode, over the queries of
    one step for prefill, which changes no result).  Decode: whole steps of one
    sequence each; prefill: sampled query tokens of one step (index list +
    attention per query)."""
    import numpy as np  # noqa: PLC0415
    from concurrent.futures import ThreadPoolExecutor  # noqa: PLC0415

    import sckv_synth as synth  # noqa: PLC0415
    from tests.helpers import oracle_step, sample_queries  # noqa: PLC0415

    x = synth.make_inputs(w, 1)
    qs = None if w.m == 1 else np.concatenate([sample_queries(w, extra=64, seed=1),
                                               np.random.default_rng(2).integers(0, w.m, size=4096)])

    def unit(i):
        if w.m == 1:
            oracle_step(w, x, 0)
        else:
            oracle_step(w, x, 0, np.array([qs[i % qs.size]]))
        return 1

    def timed(nthreads):
        tokens, i, t0 = 0, 0, time.perf_counter()
        with ThreadPoolExecutor(nthreads) as ex:
            while time.perf_counter() - t0 < seconds:
                tokens += sum(ex.map(unit, range(i, i + nthreads)))
                i += nthreads
        return tokens, time.perf_counter() - t0

    t1, e1 = timed(1)
    tn, en = timed(threads)
    what = "whole decode step(s) of one sequence" if w.m == 1 else \
        f"query token(s) of one {w.m}-token step (index list + attention per query)"
    out = {"value": tn / en, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{tn} {what} on {threads} threads in {en:.1f} s",
           "single_thread": {"value": t1 / e1, "cores": 1, "sample": f"{t1} {what} in {e1:.1f} s"}}
    out.update(cpu_info())
    return out


def peak_lib():
    import ctypes  # noqa: PLC0415

    path = os.path.join(ROOT, "sparse_compressed_kv_e2m1_amd", "libsckv_peak.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.sckv_peak_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    L.sckv_peak_read.argtypes = [vp, i64, vp, i32, i32, vp]
    L.sckv_peak_gather.argtypes = [vp, i64, vp, i64, vp, i32, i32, vp]
    L.sckv_peak_mfma.argtypes = [i32, i64, i32, vp, vp]
    L.sckv_peak_mfma_flops.argtypes = [i32, i64, i32]
    L.sckv_peak_mfma_flops.restype = ctypes.c_double
    L.sckv_peak_last_error.restype = ctypes.c_char_p
    return L


def measure_peaks():
    """The roofline denominators re-measured on this GPU (libsckv_peak.so):
    a 2 GiB copy and a 4 GiB read (past the 256 MB last-level cache), and
    dense matrix-core loops for bf16 and for e2m1 x e2m1 with block scales.
    Each figure is the best over a small sweep of launch shapes (workgroups,
    loads in flight) of a few launches each, timed with HIP events."""
    import torch  # noqa: PLC0415

    L = peak_lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ncu = torch.cuda.get_device_properties(0).multi_processor_count

    def best(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = fn()
            b.record(stream)
            if rc:
                raise RuntimeError(L.sckv_peak_last_error().decode())
            ts.append((a, b))
        torch.cuda.synchronize()
        return min(a.elapsed_time(b) for a, b in ts) / 1e3

    n = 2 << 30
    src = torch.empty(2 * n, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty(ncu * 32 * 256, dtype=torch.int32, device="cuda")
    shapes = [(ncu * wpc, depth) for wpc in (4, 8, 16, 32) for depth in (4, 8, 16)]
    t_copy = min(best(lambda: L.sckv_peak_copy(src.data_ptr(), dst.data_ptr(), n, g, d, sp), 3) for g, d in shapes)
    t_read = min(best(lambda: L.sckv_peak_read(src.data_ptr(), 2 * n, out.data_ptr(), g, d, sp), 3) for g, d in shapes)
    # 1 KiB rows of the 4 GiB buffer named by a seeded uniform index list of
    # one decode step's size (2048 queries x 640 rows)
    n_rows = 2 * n // 1024
    n_idx = 2048 * 640
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    gidx = torch.randint(0, n_rows, (n_idx,), generator=gen, dtype=torch.int32, device="cuda")
    t_gather = min(best(lambda: L.sckv_peak_gather(src.data_ptr(), n_rows, gidx.data_ptr(), n_idx, out.data_ptr(),
                                                   g, d, sp), 3) for g, d in shapes)
    del src, dst, gidx
    res = {"hbm_copy_GBs": round(2 * n / t_copy / 1e9, 1), "hbm_read_GBs": round(2 * n / t_read / 1e9, 1),
           "hbm_gather_1KiB_GBs": round(n_idx * 1024 / t_gather / 1e9, 1),
           "copy_bytes": n, "read_bytes": 2 * n, "gather_rows": n_idx}
    fo = torch.empty(ncu * 4 * 256, dtype=torch.float32, device="cuda")
    iters = 512
    for kind, name in ((0, "bf16_mfma_TFLOPs"), (1, "fp4_mfma_TFLOPs")):
        res[name] = round(max(L.sckv_peak_mfma_flops(kind, iters, ncu * wpc)
                              / best(lambda: L.sckv_peak_mfma(kind, iters, ncu * wpc, fo.data_ptr(), sp), reps=3)
                              / 1e12 for wpc in (1, 2, 4)), 1)
    torch.cuda.empty_cache()
    return res


def roofline_of(cnt, ms, peaks=None, dtype=None, gather=False):
    """Achieved rate of a call against the datasheet peak (and the measured
    one when given) of its bound: HBM bytes, or matrix-core flops of its
    contraction's dtype (bf16, or fp4 for the packed indexer).  gather: the
    call reads its rows through an index list, so it is also put against the
    measured rate of 1 KiB row gathers."""
    if cnt["bound"] == "hbm":
        achieved = cnt["bytes"] / (ms / 1e3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(achieved / HBM_PEAK_GBS, 4)}
        if peaks:
            r["measured_peak"] = peaks["hbm_read_GBs"]
            r["frac_measured"] = round(achieved / peaks["hbm_read_GBs"], 4)
            if gather and "hbm_gather_1KiB_GBs" in peaks:
                r["measured_gather_peak"] = peaks["hbm_gather_1KiB_GBs"]
                r["frac_of_gather_peak"] = round(achieved / peaks["hbm_gather_1KiB_GBs"], 4)
        return r
    achieved = cnt["flops"] / (ms / 1e3) / 1e12
    pk = FP4_PEAK_TFLOPS if dtype == "fp4" else BF16_PEAK_TFLOPS
    r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": pk, "unit": "TFLOP/s", "frac": round(achieved / pk, 4),
         "contraction": dtype or "bf16"}
    if dtype == "fp4":
        r["frac_of_bf16_peak"] = round(achieved / BF16_PEAK_TFLOPS, 4)
    if peaks:
        mp = peaks["fp4_mfma_TFLOPs" if dtype == "fp4" else "bf16_mfma_TFLOPs"]
        r["measured_peak"] = mp
        r["frac_measured"] = round(achieved / mp, 4)
    return r


def run_leg(w, B, kcache, steps, warmup, single=True, graph=False, peaks=None, latent="bf16",
            decode_launch="separate", prepare="one"):
    """Time whole steps of workload w over B sequences (inputs drawn on the
    device, resident before the timed region), then each library call with
    events around it on the same stream; optionally the B = 1 latency."""
    import torch  # noqa: PLC0415

    import sckv_synth as synth  # noqa: PLC0415
    from sparse_compressed_kv_e2m1_amd.step import PathState  # noqa: PLC0415

    # the B = 1 latency first, on a fresh allocator (measured: after the large
    # batch's buffers are freed the same step runs up to 20% slower)
    sing = None
    stream = torch.cuda.current_stream()
    if single and B > 1:
        x1 = synth.make_inputs(w, 1, device="cuda")
        s1 = PathState(w, x1, 1, kcache=kcache, latent=latent, decode_launch=decode_launch, prepare=prepare)
        s1.setup()
        for _ in range(warmup):
            s1.step()
        torch.cuda.synchronize()

        def time_steps(fn):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps

        # one sequence's step is shorter than the host work of its calls
        # through the Python binding, so its GPU latency is taken from replays
        # of a HIP graph of the step (the same calls, no per-call host work);
        # the call-by-call figure is reported beside it
        ms_eager = time_steps(s1.step)
        g1 = s1.capture_graph()
        for _ in range(warmup):
            g1.replay()
        torch.cuda.synchronize()
        ms1 = time_steps(g1.replay)
        sing = {"instances": 1, "ms_per_step": round(ms1, 5), "tokens_per_s": round(w.m / (ms1 / 1e3), 1),
                "launch": "hip graph", "eager_ms_per_step": round(ms_eager, 5)}
        del g1, s1, x1
        torch.cuda.empty_cache()

    log(f"bench: workload {w.name} B={B}: generating inputs on the device")
    x = synth.make_inputs(w, B, device="cuda")
    st = PathState(w, x, B, kcache=kcache, latent=latent, decode_launch=decode_launch, prepare=prepare)
    del x
    st.setup()
    calls = st.calls()
    st._calls = calls
    torch.cuda.synchronize()
    log(f"bench: {w.name}: warmup {warmup}")
    for _ in range(warmup):
        st.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    run_step, launch = st.step, "eager"
    if graph:
        g = st.capture_graph()
        run_step, launch = g.replay, "hip graph"
        for _ in range(warmup):
            run_step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        run_step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / steps
    log(f"bench: {w.name}: {steps} steps, {ms:.4f} ms/step (events), wall {wall * 1e3 / steps:.4f} ms/step")
    per = {name: [] for name, _ in calls}
    for _ in range(steps):
        for name, f in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            per[name].append((a, b))
    torch.cuda.synchronize()
    per_ms = {n: sum(a.elapsed_time(b) for a, b in v) / len(v) for n, v in per.items()}
    log(f"bench: {w.name}: per call ms " + json.dumps({k: round(v, 5) for k, v in per_ms.items()}))
    del st, calls
    torch.cuda.empty_cache()

    kc = kcache if w.Hi else "none"
    dtypes = {"index_scores_topk": "fp4" if kcache == "fp4" else "bf16"}
    call_info = {}
    for name, t in per_ms.items():
        cnt = counts(w, B, name, kcache, latent)
        r = roofline_of(cnt, t, peaks, dtypes.get(name), gather=name.startswith("sparse_attn"))
        r.update({"ms_per_launch": round(t, 5), "algorithmic_bytes": cnt["bytes"], "algorithmic_flops": cnt["flops"],
                  "traffic": traffic_for(w.name, B, name, kc, latent)})
        if "flops_all_visible" in cnt:
            r["flops_all_visible_pairs"] = cnt["flops_all_visible"]
        call_info[name] = r
    dom = max(per_ms, key=per_ms.get)
    roof = dict(call_info[dom])
    roof["kernel"] = dom
    tokens = B * w.m
    return {"workload": describe(w), "instances": B, "tokens_per_step": tokens, "value": round(tokens / (ms / 1e3), 1),
            "ms_per_step": round(ms, 5), "indexer_k_cache": kcache if w.Hi else None, "latent_cache": latent,
            "step_launch": launch,
            "roofline": roof, "calls": call_info, "single_instance": sing}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # (the GPU's clocks settle over ~50-80 decode steps after idle time: a
    # decode step measured 1.8 ms in its first 20 steps, 567 us in steps 20-40
    # and 542 us from step 80 on; 60 warm-up steps reach that steady state)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--instances", type=int, default=None, help="B independent sequences per step")
    ap.add_argument("--kcache", choices=["fp4", "bf16"], default="fp4",
                    help="indexer k cache storage: packed fp4 codes + E8M0 bytes (default) or bf16 rows")
    ap.add_argument("--latent", choices=["fp4", "bf16"], default="bf16",
                    help="latent cache storage: packed fp4 codes + e4m3 bytes, or bf16 rows (the pages' layout)")
    ap.add_argument("--decode-launch", choices=["separate", "one"], default="separate",
                    help="decode steps: the separate calls (default), or the one cooperative launch "
                         "sckv_decode_step for small batches")
    ap.add_argument("--prepare", choices=["one", "separate"], default="one",
                    help="set-up of steps that are not decode steps: the one launch sckv_prefill_prepare "
                         "(default) or its separate calls")
    ap.add_argument("--legs", default="long_decode,causal_prefill,chunked_prefill",
                    help="other workloads timed in the same run and reported under 'legs' (comma list; '' = none)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="oracle time per thread count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip re-measuring the HBM and matrix-core peaks")
    ap.add_argument("--no-single", action="store_true", help="skip the B = 1 latency run (for profiling)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of one step (measured: within noise of the call-by-call "
                         "launches for prefill, ~1.5%% slower for decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scale for HBM byte counters)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="only write the profiles/ summary of the rocprofv3 output under DIR (no GPU)")
    ap.add_argument("--command", action="append", default=[], help="profiling command to record (--summarize)")
    args = ap.parse_args()
    if args.summarize:
        import sckv_synth as synth  # noqa: PLC0415

        w = synth.WORKLOADS[args.workload]
        summarize_profiles(w, args.instances or DEFAULT_B[args.workload], args.summarize, args.command, args.kcache,
                           args.latent)
        return
    if args.copy_calibration:
        import torch  # noqa: PLC0415

        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 5}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the multi-GPU "
              "sharding of this path is a design note, not an implementation.", file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: PLC0415

    import sckv_synth as synth  # noqa: PLC0415

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    peaks = None
    if not args.no_peaks:
        log("bench: re-measuring the HBM and matrix-core peaks")
        peaks = measure_peaks()
        log("bench: measured peaks " + json.dumps(peaks))
    w = synth.WORKLOADS[args.workload]
    B = args.instances or DEFAULT_B[args.workload]
    head = run_leg(w, B, args.kcache, args.steps, args.warmup, single=not args.no_single, graph=args.graph,
                   peaks=peaks, latent=args.latent, decode_launch=args.decode_launch, prepare=args.prepare)
    legs = {}
    for name in [n for n in args.legs.split(",") if n and n != w.name]:
        lw = synth.WORKLOADS[name]
        legs[name] = run_leg(lw, DEFAULT_B[name], args.kcache, args.steps, args.warmup, single=False,
                             graph=args.graph, peaks=peaks, latent=args.latent, decode_launch=args.decode_launch,
                             prepare=args.prepare)

    line = {
        "metric": "sparse-attn tokens/s (decode & prefill) + % of HBM/MFMA roofline, 1 MI355X",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_note": ("attention: bf16 operands, f32 accumulation; indexer contraction: e2m1 x e2m1 with "
                       "power-of-two block scales on the fp4 matrix cores (products and sums exact), bf16 scores"
                       if args.kcache == "fp4" else "bf16 operands, f32 accumulation"),
        "data": "synthetic (seeded N(0,1), device generator)",
        "config": {"workload": head["workload"], "instances": B, "tokens_per_step": head["tokens_per_step"],
                   "indexer_k_cache": head["indexer_k_cache"], "latent_cache": head["latent_cache"],
                   "step_launch": head["step_launch"]},
        "roofline": head["roofline"],
        "per_call_ms": {k: v["ms_per_launch"] for k, v in head["calls"].items()},
        "calls": head["calls"],
        "single_instance": head["single_instance"],
        "legs": legs,
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"bench: timing the oracle on the host (~{args.cpu_seconds:.0f} s on 1 and on {threads} threads)")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
